// Top-k selection feeding the sparse decode: for each (sequence b, query i)
// row of scores, the `topk` positions below seq_lens[b] with the largest
// scores, ties going to the lower position, written in ascending position
// order (so the result is unique).
//
// Order: scores compare as floats, with -0.0 below +0.0 and NaN below every
// number. Each score maps to a 32-bit key with the same order (sign bit
// flipped for non-negatives, all bits flipped for negatives, NaN -> 1); key 0
// marks a position past the row's length, which is never counted.
//
// One workgroup of 768 threads (12 wavefronts) per row, rows of up to 67584
// positions. Wavefront w owns positions w*5632 .. w*5632+5631, as 22 blocks
// of 256 read with one 16-byte load per lane (lane l holds positions
// 4l .. 4l+3 of a block); the row is read once and kept in registers as
// order keys.
//   1. radix select of the topk-th largest key in three passes (11, 11 and
//      10 bits, most significant first); each pass builds a histogram of the
//      keys that still match the bits found so far, one copy per wavefront
//      in LDS (few bins are hot, so shared bins would serialise the
//      atomics), sums the copies, and one wavefront finds the bin where the
//      count from the top reaches topk;
//   2. every wavefront counts the keys above the threshold and those equal
//      to it; the counts in position order give each wavefront its output
//      offset and its share of the ties (the first ones in position order);
//   3. every wavefront writes its selected positions, ordered within each
//      block by a prefix sum over lanes of their 0..4 selected keys.
#include "device_common.h"
#include "mla_internal.h"
#include "mla_verify.h"

namespace mla {
namespace {

constexpr int kThreads = 768;  // 12 wavefronts: three per SIMD, 168 registers each
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  if (x != x) return 1u;  // NaN: below every number (-inf maps to 0x007FFFFF)
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Sum of a 0..4 count over the lanes below this one (three bit-plane ballots).
__device__ __forceinline__ uint32_t prefix_below(uint32_t c) {
  return lanes_below(__ballot(c & 1u)) + 2u * lanes_below(__ballot(c & 2u)) + 4u * lanes_below(__ballot(c & 4u));
}

constexpr int kBlocks = 22;                   // blocks of 256 positions per wavefront
constexpr int kRowMax = kWaves * kBlocks * 256;  // 67584 positions

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* scores, int q_len, int score_stride,
                                                        const int32_t* seq_lens, int topk, int32_t* out,
                                                        unsigned* err) {
  __shared__ uint32_t hist[kWaves][2048];  // one histogram per wavefront
  __shared__ uint32_t total[2048];
  __shared__ uint32_t cnt[kWaves][2];  // keys above / equal to the threshold, per wavefront
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
  // keys of this lane: block j, element e is position wave*5632 + j*256 +
  // 4*lane + e; positions >= n get no key
  uint32_t key[kBlocks][4];
#pragma unroll
  for (int j = 0; j < kBlocks; ++j) {
    const int p = wave * (kBlocks * 256) + j * 256 + 4 * lane;
    // score_stride is a multiple of 4, so a 16-byte load at p < n stays in the row
    const float4 v = p < n ? *reinterpret_cast<const float4*>(s + p) : float4{0.f, 0.f, 0.f, 0.f};
    key[j][0] = p + 0 < n ? order_key(v.x) : 0u;
    key[j][1] = p + 1 < n ? order_key(v.y) : 0u;
    key[j][2] = p + 2 < n ? order_key(v.z) : 0u;
    key[j][3] = p + 3 < n ? order_key(v.w) : 0u;
  }
  const int lane_p0 = wave * (kBlocks * 256) + 4 * lane;  // position of key[0][0]

  // ---- 1. radix select of the topk-th largest key
  uint32_t prefix = 0, mask = 0, rem = (uint32_t)topk;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    const int nbins = pass == 2 ? 1024 : 2048;
    for (int j = lane; j < nbins; j += 64) hist[wave][j] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kBlocks; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (key[j][e] != 0u && (key[j][e] & mask) == prefix)
          atomicAdd(&hist[wave][(key[j][e] >> shift) & (nbins - 1)], 1u);
    __syncthreads();
    for (int j = tid; j < nbins; j += kThreads) {
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) t += hist[w][j];
      total[j] = t;
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns bins [lane * per, lane * per + per); count from the top
      const int per = nbins / 64;
      uint32_t mine = 0;
      for (int j = 0; j < per; ++j) mine += total[lane * per + j];
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
          const uint32_t c = total[lane * per + j];
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
    __syncthreads();  // sel and the histograms are rewritten by the next pass
  }
  const uint32_t thr = prefix;  // the topk-th largest key (never 0); take `rem` of the keys equal to it

  // ---- 2. counts per wavefront, in position order
  uint32_t above = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kBlocks; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      above += key[j][e] > thr;
      eq += key[j][e] == thr;
    }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    above += __shfl_xor(above, off);
    eq += __shfl_xor(eq, off);
  }
  if (lane == 0) {
    cnt[wave][0] = above;
    cnt[wave][1] = eq;
  }
  __syncthreads();
  uint32_t off = 0, eq_before = 0;  // over the wavefronts before this one
  for (int w = 0; w < wave; ++w) {
    const uint32_t e_w = cnt[w][1];
    off += cnt[w][0] + (eq_before >= rem ? 0u : min(e_w, rem - eq_before));
    eq_before += e_w;
  }
  const uint32_t ties = eq_before >= rem ? 0u : min(eq, rem - eq_before);

  // ---- 3. write the selected positions in order
  uint32_t t_seen = 0;
#pragma unroll
  for (int j = 0; j < kBlocks; ++j) {
    uint32_t n_eq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) n_eq += key[j][e] == thr;
    const uint32_t eq_pre = prefix_below(n_eq);
    uint32_t tie_rank = t_seen + eq_pre;  // ties in this wavefront before this lane's first
    uint32_t n_take = 0;
    uint32_t take_bits = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool is_eq = key[j][e] == thr;
      const bool t = key[j][e] > thr || (is_eq && tie_rank < ties);
      tie_rank += is_eq;
      take_bits |= (uint32_t)t << e;
      n_take += t;
    }
    const uint32_t take_pre = prefix_below(n_take);
    uint32_t w_pos = off + take_pre;
    const int p0 = lane_p0 + j * 256;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (take_bits & (1u << e)) o[w_pos++] = p0 + e;
    // block totals: the last lane's prefix plus its own count
    t_seen += __shfl(eq_pre + n_eq, 63);
    off += __shfl(take_pre + n_take, 63);
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
