// The two weight absorptions around absorbed-MLA attention, as bf16 MFMA
// GEMMs, one 16 x 64 output tile per workgroup:
//   before: q = [ q_nope . W_UK[h] | q_rope ]   (576-wide query per head)
//   after:  o = o_latent . W_UV[h]              (per-head value projection)
// The latent width is 512; the per-head widths (128 nope, 128 value) follow
// the common MLA configuration.
//
// Weights are stored transposed (one row per output column, its inputs
// contiguous), so every MFMA operand is one 16-byte load per lane:
// A = weight rows (output columns), B = token rows, D[column][token]. A lane
// then holds four consecutive output columns of one token and writes them
// with one store.
#include "device_common.h"
#include "mla_internal.h"
#include "mla_verify.h"

namespace mla {
namespace {

constexpr int kNope = 128;  // per-head q_nope width (input of W_UK)
constexpr int kVh = 128;    // per-head value width (output of W_UV)

// grid (heads, 512 / 64), one wavefront: its 64 x 128 slice of W_UK[h]
// stays in registers while the token blocks of 16 stream past.
__global__ __launch_bounds__(64) void absorb_q_kernel(const __bf16* q_nope, const __bf16* q_rope, const __bf16* w_uk,
                                                      int tokens, int heads, __bf16* q_out) {
  constexpr int kSteps = kNope / 32;
  const int h = blockIdx.x, c0 = blockIdx.y * 64;
  const int lane = threadIdx.x, g = lane >> 4, li = lane & 15;
  bf16x8 a[kSteps][4];
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      a[ks][cb] = *reinterpret_cast<const bf16x8*>(w_uk + ((size_t)h * kDv + c0 + 16 * cb + li) * kNope + 32 * ks +
                                                  8 * g);
  // the next token block's query loads are issued before this block's MFMAs
  auto load_q = [&](int t0, bf16x8* b) {
    const int t = t0 + li;
    const __bf16* qrow = q_nope + ((size_t)(t < tokens ? t : 0) * heads + h) * kNope + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) b[ks] = t < tokens ? *reinterpret_cast<const bf16x8*>(qrow + 32 * ks) : bf16x8{};
  };
  bf16x8 b[kSteps], bn[kSteps];
  load_q(0, b);
  for (int t0 = 0; t0 < tokens; t0 += 16) {
    const int t = t0 + li;
    const bool tok_ok = t < tokens;
    if (t0 + 16 < tokens) load_q(t0 + 16, bn);
    f32x4 acc[4] = {};
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[cb] = mfma_16x16x32(a[ks][cb], b[ks], acc[cb]);
    // lane (g, li) holds columns c0 + 16 cb + 4 g + r of token t0 + li
    if (tok_ok) {
      __bf16* orow = q_out + ((size_t)t * heads + h) * kDk;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        *reinterpret_cast<bf16x4*>(orow + c0 + 16 * cb + 4 * g) = __builtin_convertvector(acc[cb], bf16x4);
      if (blockIdx.y == 0) {  // the rope part passes through unchanged
        const __bf16* rrow = q_rope + ((size_t)t * heads + h) * kDrope;
        *reinterpret_cast<bf16x8*>(orow + kDv + 16 * g) = *reinterpret_cast<const bf16x8*>(rrow + 16 * g);
        *reinterpret_cast<bf16x8*>(orow + kDv + 16 * g + 8) = *reinterpret_cast<const bf16x8*>(rrow + 16 * g + 8);
      }
    }
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) b[ks] = bn[ks];
  }
}

// grid (heads, 128 / 64), four wavefronts that split the 512 inputs (128
// each); every wavefront keeps its 64 x 128 slice of W_UV[h] in registers
// while the token blocks of 16 stream past, and the four partial tiles of a
// block are added in LDS in a fixed order. o_latent is rounded to bf16 as it
// is read.
__global__ __launch_bounds__(256) void project_o_kernel(const float* o_latent, const __bf16* w_uv, int tokens,
                                                        int heads, float* o_out) {
  constexpr int kSteps = kDv / 32 / 4;  // k-steps per wavefront
  __shared__ f32x4 part[3][4][64];      // wavefronts 1..3: [cb][lane]
  const int h = blockIdx.x, c0 = blockIdx.y * 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  const int k0 = wave * (kDv / 4);
  bf16x8 a[kSteps][4];
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      a[ks][cb] = *reinterpret_cast<const bf16x8*>(w_uv + ((size_t)h * kVh + c0 + 16 * cb + li) * kDv + k0 +
                                                  32 * ks + 8 * g);
  // the next token block's loads are issued before this block's MFMAs
  auto load_o = [&](int t0, f32x4* lo, f32x4* hi) {
    const int t = t0 + li;
    const float* orow_in = o_latent + ((size_t)(t < tokens ? t : 0) * heads + h) * kDv + k0 + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      lo[ks] = t < tokens ? *reinterpret_cast<const f32x4*>(orow_in + 32 * ks) : f32x4{};
      hi[ks] = t < tokens ? *reinterpret_cast<const f32x4*>(orow_in + 32 * ks + 4) : f32x4{};
    }
  };
  f32x4 lo[kSteps], hi[kSteps], lo_n[kSteps], hi_n[kSteps];
  load_o(0, lo, hi);
  for (int t0 = 0; t0 < tokens; t0 += 16) {
    const int t = t0 + li;
    const bool tok_ok = t < tokens;
    bf16x8 b[kSteps];
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks)
      b[ks] = __builtin_convertvector(__builtin_shufflevector(lo[ks], hi[ks], 0, 1, 2, 3, 4, 5, 6, 7), bf16x8);
    if (t0 + 16 < tokens) load_o(t0 + 16, lo_n, hi_n);
    f32x4 acc[4] = {};
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[cb] = mfma_16x16x32(a[ks][cb], b[ks], acc[cb]);
    if (wave > 0) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) part[wave - 1][cb][lane] = acc[cb];
    }
    __syncthreads();
    if (wave == 0 && tok_ok) {
      float* orow = o_out + ((size_t)t * heads + h) * kVh;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const f32x4 v = ((acc[cb] + part[0][cb][lane]) + part[1][cb][lane]) + part[2][cb][lane];
        *reinterpret_cast<f32x4*>(orow + c0 + 16 * cb + 4 * g) = v;
      }
    }
    __syncthreads();  // part is rewritten by the next token block
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      lo[ks] = lo_n[ks];
      hi[ks] = hi_n[ks];
    }
  }
}

}  // namespace

hipError_t launch_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int tokens, int heads,
                           void* q_out, hipStream_t stream) {
  hipLaunchKernelGGL(absorb_q_kernel, dim3(heads, kDv / 64), dim3(64), 0, stream,
                     static_cast<const __bf16*>(q_nope), static_cast<const __bf16*>(q_rope),
                     static_cast<const __bf16*>(w_uk), tokens, heads, static_cast<__bf16*>(q_out));
  return hipGetLastError();
}

hipError_t launch_project_o(const float* o_latent, const void* w_uv, int tokens, int heads, float* o_out,
                            hipStream_t stream) {
  hipLaunchKernelGGL(project_o_kernel, dim3(heads, kVh / 64), dim3(256), 0, stream, o_latent,
                     static_cast<const __bf16*>(w_uv), tokens, heads, o_out);
  return hipGetLastError();
}

}  // namespace mla
