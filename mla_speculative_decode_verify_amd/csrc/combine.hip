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

// Splits holding sequence b's partials: the stride S, or, when the counts
// follow the lengths, the count the split kernel recorded (kept in [0, S]).
__device__ __forceinline__ int split_count(const Args& a, int b) {
  if (a.balance_units <= 0) return a.nsplit;
  return __builtin_amdgcn_readfirstlane(min(max(a.part_count[b], 0), a.nsplit));
}

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
// rounds of the same loop. kCols = 128 suits many splits (4 splits per
// wavefront load), kCols = 512 up to 32 (a wavefront per split); rows with
// only a few splits take combine_rows_kernel below.
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
  const int S = a.nsplit, R = a.rows;  // S: the partials' split stride
  // splits that hold this sequence's partials: all S, or its own count when
  // the counts follow the lengths (recorded by the split kernel)
  const int Sb = split_count(a, b);
  const int grp = tid / kLanes, cl = tid % kLanes;
  const int half = (slice * kCols + cl * 8) / 256;
  const size_t p0 = (size_t)b * S * R + row;  // partial output of split s: row p0 + s * R
  const size_t q0 = ((size_t)b * R + row) * S;  // its LSE / scales: q0 + s (splits contiguous)
  const _Float16* po = a.part_o + p0 * kDv + slice * kCols + cl * 8;
  const size_t sstride = (size_t)R * kDv;

  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  float den = 0.f;  // this lane's share of sum_s w_s (counted once per split: by lane cl == 0)
  float mx = -INFINITY;  // max LSE over the splits
  f16x8 v[kMaxPer];
  float ls[kMaxPer], sc[kMaxPer];
  auto load_round = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
      const int s = s0 + u * kGroups;
      const bool ok = s < Sb;
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
  // The first round's loads are issued first. When one round covers every
  // split, its LSEs are all the max needs, so the max costs no extra memory
  // round trip; otherwise a separate pass reads all S LSEs while the first
  // round's loads are in flight. Every thread reaches the barrier.
  load_round(grp);
  if (Sb <= kMaxPer * kGroups) {
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) mx = fmaxf(mx, ls[u]);
  } else {
    for (int s = tid; s < Sb; s += kCombThreads) mx = fmaxf(mx, a.part_lse[q0 + s]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < kCombThreads / 64; ++w) mx = fmaxf(mx, red[w]);
  accumulate();
  for (int s0 = grp + kMaxPer * kGroups; s0 < Sb; s0 += kMaxPer * kGroups) {
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

// Merge with one wavefront per (sequence, query row), for rows with few
// splits: lane l owns output columns 8 l .. 8 l + 7 (one 16-byte fp16 load
// per split) and the wavefront walks the splits in rounds of kPer, all of a
// round's loads in flight together. The base of the exponentials is the
// running max of the LSEs seen so far; when a round raises it, the sums so
// far are rescaled once (exact in real arithmetic: every weight is
// exp(lse_s - M) for the final M). With at most kPer splits, as with the
// library's split counts for most shapes, there is a single round and no
// rescale. Four wavefronts per workgroup take four rows; the wavefronts
// never synchronise, so those past the last row leave at once.
__global__ __launch_bounds__(256) void combine_rows_kernel(Args a) {
  constexpr int kPer = 8;
  const int lane = (int)__lane_id();
  const int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6), b = blockIdx.y;
  const int S = a.nsplit, R = a.rows;  // S: the partials' split stride
  if (row >= R) return;
  const int Sb = split_count(a, b);
  const int half = lane >> 5;
  const _Float16* po = a.part_o + ((size_t)b * S * R + row) * kDv + 8 * lane;
  const size_t sstride = (size_t)R * kDv;
  const size_t q0 = ((size_t)b * R + row) * S;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  float m = -INFINITY, den = 0.f;
  for (int s0 = 0; s0 < Sb; s0 += kPer) {
    f16x8 v[kPer];
    float ls[kPer], sc[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int s = s0 + u;
      const bool ok = s < Sb;
      v[u] = ok ? *reinterpret_cast<const f16x8*>(po + (size_t)s * sstride) : f16x8{};
      ls[u] = ok ? a.part_lse[q0 + s] : -INFINITY;
      sc[u] = ok ? a.part_scale[(q0 + s) * 2 + half] : 0.f;
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < kPer; ++u) mx = fmaxf(mx, ls[u]);
    if (mx != m && m != -INFINITY) {  // uniform: every lane holds the same LSEs
      const float alpha = fast_exp2((m - mx) * kLog2e);
      den *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= alpha;
    }
    m = mx;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const float w = ls[u] == -INFINITY ? 0.f : fast_exp2((ls[u] - m) * kLog2e);  // m > -inf whenever ls is
      den += w;
      const float ws = w * sc[u];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(ws, (float)v[u][j], acc[j]);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float* dst = a.out + ((size_t)b * R + row) * kDv + 8 * lane;
  reinterpret_cast<f32x4*>(dst)[0] = f32x4{acc[0], acc[1], acc[2], acc[3]} * inv;
  reinterpret_cast<f32x4*>(dst)[1] = f32x4{acc[4], acc[5], acc[6], acc[7]} * inv;
  if (lane == 0 && a.lse) a.lse[(size_t)b * R + row] = den > 0.f ? m + fast_log2(den) * kLn2 : -INFINITY;
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
  // one wavefront per row while its splits fit a few rounds of loads
  // (length-following counts stay far below their stride, and a workgroup
  // per row and slice would mostly idle); a workgroup per row up to 32
  // splits, per 128-column slice beyond
  if (a.nsplit <= 8 || (a.balance_units > 0 && a.nsplit <= 64)) {
    hipLaunchKernelGGL(combine_rows_kernel, dim3((a.rows + 3) / 4, a.batch), dim3(256), 0, stream, a);
  } else if (a.nsplit <= 32) {
    hipLaunchKernelGGL(combine_kernel<kDv>, dim3(1, a.rows, a.batch), dim3(kCombThreads), 0, stream, a);
  } else {
    // 128-column slices: half the workgroups of 64-column ones, and at H=64
    // (576 rows) a 42-split merge in 6.6 us instead of 10.1 (equal at H=8)
    hipLaunchKernelGGL(combine_kernel<128>, dim3(kDv / 128, a.rows, a.batch), dim3(kCombThreads), 0, stream, a);
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
