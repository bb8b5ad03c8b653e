// Log-sum-exp merge of split partials, and the draft-tree mask builder.
//
// Merge: for each (sequence, query row) with split results (O_s, lse_s),
//   lse = M + ln sum_s exp(lse_s - M),  M = max_s lse_s,
//   out = sum_s exp(lse_s - lse) * O_s.
// Splits whose lse is -inf (no visible key) carry zero weight, so an empty
// split never turns the result into NaN. The pages only say the KV axis is
// split into partial reductions ("How One Environment Variable Unlocked 3x
// Throughput", section "Input Knowledge Required"); this is the standard
// flash-decoding merge that makes the split exact in real arithmetic.
#include "device_common.h"
#include "mla_internal.h"
#include "mla_verify.h"

namespace mla {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

// One wavefront per row; each lane owns 8 of the 512 output columns.
__global__ __launch_bounds__(256) void combine_kernel(Args a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  const int b = blockIdx.y;
  const int S = a.nsplit, R = a.rows;
  if (row >= R) return;
  const float* pl = a.part_lse + (size_t)b * S * R + row;  // stride R between splits
  float mx = -INFINITY;
  for (int s = lane; s < S; s += 64) mx = fmaxf(mx, pl[(size_t)s * R]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  float wsum = 0.f;
  if (mx != -INFINITY) {
    const float* po = a.part_o + ((size_t)b * S * R + row) * kDv + lane * 8;
    const size_t sstride = (size_t)R * kDv;
    int s = 0;
    for (; s + 2 <= S; s += 2) {
      const float l0 = pl[(size_t)s * R], l1 = pl[(size_t)(s + 1) * R];
      const float w0 = fast_exp2((l0 - mx) * kLog2e);  // -inf -> 0
      const float w1 = fast_exp2((l1 - mx) * kLog2e);
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(po + s * sstride);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(po + s * sstride + 4);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(po + (s + 1) * sstride);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(po + (s + 1) * sstride + 4);
      wsum += w0 + w1;
      acc0 += w0 * a0 + w1 * b0;
      acc1 += w0 * a1 + w1 * b1;
    }
    if (s < S) {
      const float l0 = pl[(size_t)s * R];
      const float w0 = fast_exp2((l0 - mx) * kLog2e);
      wsum += w0;
      acc0 += w0 * *reinterpret_cast<const f32x4*>(po + s * sstride);
      acc1 += w0 * *reinterpret_cast<const f32x4*>(po + s * sstride + 4);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float* dst = a.out + ((size_t)b * R + row) * kDv + lane * 8;
  *reinterpret_cast<f32x4*>(dst) = acc0 * inv;
  *reinterpret_cast<f32x4*>(dst + 4) = acc1 * inv;
  if (lane == 0 && a.lse) a.lse[(size_t)b * R + row] = wsum > 0.f ? mx + fast_log2(wsum) * kLn2 : -INFINITY;
}

// One thread per (sequence, draft): walk the parent chain to the root.
// Parents strictly decrease along a valid chain, so the walk ends.
__global__ void tree_mask_kernel(const int32_t* parents, int batch, int q_len, uint64_t* anc, unsigned* err) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= batch * q_len) return;
  const int b = idx / q_len, i = idx - b * q_len;
  const int32_t* par = parents + (size_t)b * q_len;
  uint64_t bits = 1ull << i;
  int node = i;
  bool bad = false;
  while (true) {
    const int p = par[node];
    if (p == -1) break;
    if (p < -1 || p >= node) {
      bad = true;
      break;
    }
    bits |= 1ull << p;
    node = p;
  }
  if (bad) {
    bits = 1ull << i;
    flag_error(err, MLA_DEVERR_TREE_PARENT);
  }
  anc[idx] = bits;
}

}  // namespace

hipError_t launch_combine(const Args& a, hipStream_t stream) {
  dim3 grid((a.rows + 3) / 4, a.batch);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_tree_mask(const int32_t* parents, int batch, int q_len, uint64_t* anc, unsigned* err,
                            hipStream_t stream) {
  const int n = batch * q_len;
  hipLaunchKernelGGL(tree_mask_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, parents, batch, q_len, anc,
                     err);
  return hipGetLastError();
}

}  // namespace mla
