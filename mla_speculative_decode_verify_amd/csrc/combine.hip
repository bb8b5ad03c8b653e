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
#include "split_epilogue.h"

namespace mla {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kCombThreads = 256;

// Partials are fp16 rows of 512 columns with a power-of-two multiplier per
// 256-column half (stored by the split kernels), plus an fp32 LSE.
//
// One workgroup per (sequence, query row, kCols-column slice); kCols / 8
// lanes cover one split's slice with one 16-byte load each, so a pass of the
// workgroup covers kGroups = 256 * 8 / kCols splits. Every lane first issues
// the loads of its splits' slices (up to kMaxPer of them, kept in
// registers) together with their LSEs and multipliers; the max LSE is found
// while those loads are in flight, so the whole merge costs about one
// memory round trip. Splits beyond kMaxPer per lane are handled by further
// rounds of the same loop. kCols = 64 suits many splits (8 splits per
// wavefront load), kCols = 512 up to 32 (a wavefront per split).
template <int kCols>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(Args a) {
  constexpr int kLanes = kCols / 8;                 // lanes per split slice
  constexpr int kGroups = kCombThreads / kLanes;    // splits per pass
  constexpr int kMaxPer = 8;                        // splits per lane per round
  __shared__ float red[kCombThreads / 64];
  __shared__ float acc_lds[kGroups][kCols + 4];
  __shared__ float den_lds[kGroups];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slice = blockIdx.x, row = blockIdx.y, b = blockIdx.z;
  const int S = a.nsplit, R = a.rows;
  const int grp = tid / kLanes, cl = tid % kLanes;
  const int half = (slice * kCols + cl * 8) / 256;
  const size_t p0 = (size_t)b * S * R + row;  // partial output of split s: row p0 + s * R
  const size_t q0 = ((size_t)b * R + row) * S;  // its LSE / scales: q0 + s (splits contiguous)
  const _Float16* po = a.part_o + p0 * kDv + slice * kCols + cl * 8;
  const size_t sstride = (size_t)R * kDv;

  // ---- max LSE over all splits (a separate, small pass: S floats)
  float mx = -INFINITY;
  for (int s = tid; s < S; s += kCombThreads) mx = fmaxf(mx, a.part_lse[q0 + s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;

  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  float den = 0.f;  // this lane's share of sum_s w_s (counted once per split: by lane cl == 0)
  f16x8 v[kMaxPer];
  float ls[kMaxPer], sc[kMaxPer];
  auto load_round = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
      const int s = s0 + u * kGroups;
      const bool ok = s < S;
      const size_t q = q0 + (ok ? s : 0);
      v[u] = ok ? *reinterpret_cast<const f16x8*>(po + (size_t)s * sstride) : f16x8{};
      ls[u] = ok ? a.part_lse[q] : -INFINITY;
      sc[u] = ok ? a.part_scale[q * 2 + half] : 0.f;
    }
  };
  auto accumulate = [&]() {
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
      const float w = ls[u] == -INFINITY ? 0.f : fast_exp2((ls[u] - mx) * kLog2e);  // mx > -inf whenever ls is
      if (cl == 0) den += w;
      const float ws = w * sc[u];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(ws, (float)v[u][j], acc[j]);
    }
  };
  // first round's loads are issued before the barrier that publishes the
  // max, so they fly while it is reduced; every thread reaches the barrier
  load_round(grp);
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < kCombThreads / 64; ++w) mx = fmaxf(mx, red[w]);
  accumulate();
  for (int s0 = grp + kMaxPer * kGroups; s0 < S; s0 += kMaxPer * kGroups) {
    load_round(s0);
    accumulate();
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) acc_lds[grp][cl * 8 + j] = acc[j];
  if (cl == 0) den_lds[grp] = den;
  __syncthreads();
  float tot = 0.f;
#pragma unroll 8
  for (int gi = 0; gi < kGroups; ++gi) tot += den_lds[gi];
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  for (int c = tid; c < kCols; c += kCombThreads) {
    float t = 0.f;
#pragma unroll 8
    for (int gi = 0; gi < kGroups; ++gi) t += acc_lds[gi][c];
    a.out[((size_t)b * R + row) * kDv + slice * kCols + c] = t * inv;
  }
  if (slice == 0 && tid == 0 && a.lse)
    a.lse[(size_t)b * R + row] = tot > 0.f ? mx + fast_log2(tot) * kLn2 : -INFINITY;
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
  if (a.nsplit <= 32) {
    hipLaunchKernelGGL(combine_kernel<kDv>, dim3(1, a.rows, a.batch), dim3(kCombThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(combine_kernel<64>, dim3(kDv / 64, a.rows, a.batch), dim3(kCombThreads), 0, stream, a);
  }
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
