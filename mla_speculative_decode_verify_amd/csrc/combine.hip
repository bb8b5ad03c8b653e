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
// One workgroup per (sequence, query row, kCols-column slice). Phase 1 takes
// M = max_s lse_s and the weights w_s = exp(lse_s - M): their sum is the
// denominator, and w_s times each half's multiplier goes to LDS for the
// numerator.
// Phase 2 streams the partial slices: kCols / 8 lanes cover one split's
// slice with one 16-byte load each, so a pass over the workgroup covers
// 256 * 8 / kCols splits, and four passes are issued before any is used.
// The per-lane sums meet in LDS. kCols = 64 suits many splits (8 splits per
// wavefront load); kCols = 512 suits a few (a wavefront per split).
template <int kCols>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(Args a) {
  constexpr int kLanes = kCols / 8;                     // lanes per split slice
  constexpr int kGroups = kCombThreads / kLanes;        // splits per pass
  constexpr int kUnroll = 4;
  __shared__ float wnum[2][MLA_MAX_NSPLIT];  // numerator weights per 256-column half
  __shared__ float red[kCombThreads / 64];
  __shared__ float acc_lds[kGroups][kCols + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slice = blockIdx.x, row = blockIdx.y, b = blockIdx.z;
  const int S = a.nsplit, R = a.rows;
  const size_t p0 = (size_t)b * S * R + row;  // partial index of split s: p0 + s * R

  // ---- phase 1: max LSE, then weights and their sum
  float mx = -INFINITY;
  for (int s = tid; s < S; s += kCombThreads) mx = fmaxf(mx, a.part_lse[p0 + (size_t)s * R]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < kCombThreads / 64; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();  // red is reused below
  float den = 0.f;
  for (int s = tid; s < S; s += kCombThreads) {
    const size_t p = p0 + (size_t)s * R;
    const float ls = a.part_lse[p];
    const float w = ls == -INFINITY ? 0.f : fast_exp2((ls - mx) * kLog2e);  // mx > -inf whenever ls is
    den += w;
    wnum[0][s] = w * a.part_scale[p * 2];
    wnum[1][s] = w * a.part_scale[p * 2 + 1];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  if (lane == 0) red[wave] = den;
  __syncthreads();
  den = red[0];
#pragma unroll
  for (int w = 1; w < kCombThreads / 64; ++w) den += red[w];

  // ---- phase 2: weighted sum of the partial slices
  const int grp = tid / kLanes, cl = tid % kLanes;
  const int half = (slice * kCols + cl * 8) / 256;
  const _Float16* po = a.part_o + p0 * kDv + slice * kCols + cl * 8;
  const size_t sstride = (size_t)R * kDv;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int s0 = grp; s0 < S; s0 += kUnroll * kGroups) {
    f16x8 v[kUnroll];
    float w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int s = s0 + u * kGroups;
      const bool ok = s < S;
      v[u] = ok ? *reinterpret_cast<const f16x8*>(po + (size_t)s * sstride) : f16x8{};
      w[u] = ok ? wnum[half][s] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(w[u], (float)v[u][j], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) acc_lds[grp][cl * 8 + j] = acc[j];
  __syncthreads();
  const float inv = den > 0.f ? 1.f / den : 0.f;
  for (int c = tid; c < kCols; c += kCombThreads) {
    float t = 0.f;
#pragma unroll 8
    for (int gi = 0; gi < kGroups; ++gi) t += acc_lds[gi][c];
    a.out[((size_t)b * R + row) * kDv + slice * kCols + c] = t * inv;
  }
  if (slice == 0 && tid == 0 && a.lse)
    a.lse[(size_t)b * R + row] = den > 0.f ? mx + fast_log2(den) * kLn2 : -INFINITY;
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
  if (a.nsplit <= 16) {
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
