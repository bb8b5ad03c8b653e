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

// One workgroup per (sequence, query row, 128-column quarter). The four
// wavefronts take every fourth split; each lane owns 2 of the 128 columns
// (512 contiguous bytes per wavefront and split). Partial sums meet in LDS.
constexpr int kCombCols = 128;
constexpr int kCombWaves = 4;

__global__ __launch_bounds__(256) void combine_kernel(Args a) {
  __shared__ float red_max[kCombWaves];
  __shared__ float red_sum[kCombWaves];
  __shared__ float2 red_acc[kCombWaves - 1][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int quarter = blockIdx.x, row = blockIdx.y, b = blockIdx.z;
  const int S = a.nsplit, R = a.rows;
  const float* pl = a.part_lse + (size_t)b * S * R + row;  // split s at pl[s * R]

  float mx = -INFINITY;
  for (int s = tid; s < S; s += 256) mx = fmaxf(mx, pl[(size_t)s * R]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red_max[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red_max[0], red_max[1]), fmaxf(red_max[2], red_max[3]));

  float2 acc = {0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {
    const size_t sstride = (size_t)R * kDv;
    const float* po = a.part_o + ((size_t)b * S * R + row) * kDv + quarter * kCombCols + lane * 2;
    int s = wave;
    for (; s + 3 * kCombWaves < S; s += 4 * kCombWaves) {
      float w[4];
      float2 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int su = s + u * kCombWaves;
        w[u] = fast_exp2((pl[(size_t)su * R] - mx) * kLog2e);  // -inf -> 0
        v[u] = *reinterpret_cast<const float2*>(po + su * sstride);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wsum += w[u];
        acc.x += w[u] * v[u].x;
        acc.y += w[u] * v[u].y;
      }
    }
    for (; s < S; s += kCombWaves) {
      const float w = fast_exp2((pl[(size_t)s * R] - mx) * kLog2e);
      const float2 v = *reinterpret_cast<const float2*>(po + s * sstride);
      wsum += w;
      acc.x += w * v.x;
      acc.y += w * v.y;
    }
  }
  if (lane == 0) red_sum[wave] = wsum;
  if (wave > 0) red_acc[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  const float tot = red_sum[0] + red_sum[1] + red_sum[2] + red_sum[3];
#pragma unroll
  for (int k = 0; k < kCombWaves - 1; ++k) {
    acc.x += red_acc[k][lane].x;
    acc.y += red_acc[k][lane].y;
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  float* dst = a.out + ((size_t)b * R + row) * kDv + quarter * kCombCols + lane * 2;
  *reinterpret_cast<float2*>(dst) = float2{acc.x * inv, acc.y * inv};
  if (quarter == 0 && lane == 0 && a.lse) a.lse[(size_t)b * R + row] = tot > 0.f ? mx + fast_log2(tot) * kLn2 : -INFINITY;
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
  dim3 grid(kDv / kCombCols, a.rows, a.batch);
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
