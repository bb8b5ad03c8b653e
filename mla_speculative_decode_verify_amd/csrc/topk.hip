// Top-k selection feeding the sparse decode: for each (sequence b, query i)
// row of scores, the `topk` positions below seq_lens[b] with the largest
// scores, ties going to the lower position, written in ascending position
// order (so the result is unique).
//
// Order: scores compare as floats, with -0.0 below +0.0 and NaN below every
// number. Each score maps to a 32-bit key with the same order (sign bit
// flipped for non-negatives, all bits flipped for negatives, NaN -> 0).
//
// One workgroup of 1024 threads per row:
//   1. radix select of the topk-th largest key in three passes (11, 11 and
//      10 bits, most significant first); each pass builds an LDS histogram
//      of the keys that still match the bits found so far, and one
//      wavefront finds the bin where the count from the top reaches topk;
//   2. every thread takes a contiguous run of positions and counts the keys
//      above the threshold and those equal to it; block scans give each run
//      its output offset and its share of the ties (the first ones in
//      position order);
//   3. every thread writes its selected positions.
// The row is read five times; after the first pass it comes from the L2.
#include "device_common.h"
#include "mla_internal.h"
#include "mla_verify.h"

namespace mla {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  if (x != x) return 0u;  // NaN: below every number
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup (thread order); `tot` gets the total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_sums, uint32_t& tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  if (lane == 63) wave_sums[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t s = wave_sums[w];
    before += w < wave ? s : 0u;
    tot += s;
  }
  __syncthreads();  // wave_sums is reused by the next scan
  return before + inc - v;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* scores, int q_len, int score_stride,
                                                        const int32_t* seq_lens, int topk, int32_t* out,
                                                        unsigned* err) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wave_sums[kWaves];
  __shared__ uint32_t sel[3];  // key prefix, its mask, keys equal to the threshold still to take
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int b = (int)(row / q_len);
  const float* s = scores + row * score_stride;
  int32_t* o = out + row * topk;
  int n = seq_lens[b];
  if (n < 0 || n > score_stride || n < topk) {
    if (tid == 0) flag_error(err, MLA_DEVERR_SEQ_LEN);
    n = min(max(n, 0), score_stride);
  }
  if (n <= topk) {  // every position is selected; the rest of the row is -1
    for (int j = tid; j < topk; j += kThreads) o[j] = j < n ? j : -1;
    return;
  }

  // ---- 1. radix select of the topk-th largest key
  uint32_t prefix = 0, mask = 0, rem = (uint32_t)topk;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    const int nbins = pass == 2 ? 1024 : 2048;
    for (int j = tid; j < nbins; j += kThreads) hist[j] = 0;
    __syncthreads();
    for (int p = tid; p < n; p += kThreads) {
      const uint32_t k = order_key(s[p]);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & (nbins - 1)], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns bins [lane * per, lane * per + per); count from the top
      const int per = nbins / 64;
      uint32_t mine = 0;
      for (int j = 0; j < per; ++j) mine += hist[lane * per + j];
      uint32_t from_top = mine;  // sum over lanes >= this one
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_down(from_top, off);
        if (lane + off < 64) from_top += t;
      }
      const uint32_t above = from_top - mine;
      if (above < rem && rem <= from_top) {  // exactly one lane
        uint32_t cum = above;
        for (int j = per - 1; j >= 0; --j) {
          const uint32_t c = hist[lane * per + j];
          if (cum + c >= rem) {
            sel[0] = prefix | ((uint32_t)(lane * per + j) << shift);
            sel[1] = mask | ((uint32_t)(nbins - 1) << shift);
            sel[2] = rem - cum;
            break;
          }
          cum += c;
        }
      }
    }
    __syncthreads();
    prefix = sel[0];
    mask = sel[1];
    rem = sel[2];
    __syncthreads();  // sel is rewritten by the next pass
  }
  const uint32_t thr = prefix;  // the topk-th largest key; take `rem` of the keys equal to it

  // ---- 2. per-run counts, offsets and tie shares
  const int run = (n + kThreads - 1) / kThreads;
  const int p0 = min(n, tid * run), p1 = min(n, p0 + run);
  uint32_t n_above = 0, n_eq = 0;
  for (int p = p0; p < p1; ++p) {
    const uint32_t k = order_key(s[p]);
    n_above += k > thr;
    n_eq += k == thr;
  }
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan(n_eq, wave_sums, tot);
  const uint32_t ties = eq_before >= rem ? 0u : min(n_eq, rem - eq_before);
  const uint32_t off = block_exclusive_scan(n_above + ties, wave_sums, tot);

  // ---- 3. write the selected positions in order
  uint32_t w = off, t_seen = 0;
  for (int p = p0; p < p1; ++p) {
    const uint32_t k = order_key(s[p]);
    bool take = k > thr;
    if (k == thr) {
      take = t_seen < ties;
      ++t_seen;
    }
    if (take) o[w++] = p;
  }
}

}  // namespace

hipError_t launch_topk(const float* scores, int batch, int q_len, int score_stride, const int32_t* seq_lens,
                       int topk, int32_t* out, unsigned* err, hipStream_t stream) {
  const long rows = (long)batch * q_len;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, scores, q_len, score_stride,
                     seq_lens, topk, out, err);
  return hipGetLastError();
}

}  // namespace mla
