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
// A row is cut into parts of 8192 positions, one 256-thread workgroup each,
// so every CU takes part even with few rows. Three kernels:
//   1. hist:  per part, the histogram of the keys' top 11 bits;
//   2. cands: per part, the bin B0 where the row's count from the top
//             reaches topk (from all parts' histograms); the part counts its
//             keys above B0 and appends those inside B0 (key, position) to
//             the row's candidate list;
//   3. write: per part, first the selection (every part of a row computes
//             the same): a radix select over the candidates' remaining 21
//             bits (11 + 10) finds the topk-th largest key and how many of
//             the keys equal to it are kept, and, in part order, this part's
//             output offset and its share of those ties; then the selected
//             positions in ascending order, each wavefront taking a
//             contiguous quarter of the part and every 16-byte-load block
//             ordered by a prefix sum over lanes.
#include "device_common.h"
#include "mla_internal.h"
#include "mla_verify.h"

namespace mla {

namespace {

constexpr int kPartThreads = 256;
constexpr int kPartWaves = kPartThreads / 64;
constexpr int kPart = 8192;                          // positions per part
constexpr int kPartBlocks = kPart / kPartWaves / 256;  // 256-position blocks per wavefront (8)

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

// Workspace views of one call.
struct TopkWs {
  uint32_t* hist;       // [rows][parts][2048]
  uint32_t* cand;       // [rows][parts * kPart][2]: key, position
  uint32_t* row_info;   // [rows][4]: candidate count, B0, rem after B0, above-B0 total
  uint32_t* part_cnt;   // [rows][parts][3]: keys above B0, then output offset and tie share
  int parts;
};

__device__ __forceinline__ int row_len(const int32_t* seq_lens, int b, int stride) {
  return min(max(seq_lens[b], 0), stride);
}

// This part's keys: wavefront w, block j, element e is position
// part*8192 + w*2048 + j*256 + 4*lane + e (score_stride is a multiple of 4,
// so a 16-byte load at a position below n stays in the row).
__device__ __forceinline__ void load_part(const float* s, int part, int n, uint32_t (&key)[kPartBlocks][4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kPartBlocks; ++j) {
    const int p = part * kPart + wave * (kPartBlocks * 256) + j * 256 + 4 * lane;
    const float4 v = p < n ? *reinterpret_cast<const float4*>(s + p) : float4{0.f, 0.f, 0.f, 0.f};
    key[j][0] = p + 0 < n ? order_key(v.x) : 0u;
    key[j][1] = p + 1 < n ? order_key(v.y) : 0u;
    key[j][2] = p + 2 < n ? order_key(v.z) : 0u;
    key[j][3] = p + 3 < n ? order_key(v.w) : 0u;
  }
}

// ---- 1. per-part histogram of the top 11 key bits
__global__ __launch_bounds__(kPartThreads) void topk_hist_kernel(const float* scores, int score_stride,
                                                                 const int32_t* seq_lens, int q_len, int topk,
                                                                 TopkWs ws) {
  __shared__ uint32_t hist[kPartWaves][2048];
  const int part = blockIdx.x, row = blockIdx.y, b = row / q_len;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = row_len(seq_lens, b, score_stride);
  if (n <= topk) return;  // the write kernel lists every position
  if (part == 0 && threadIdx.x == 0) ws.row_info[row * 4 + 0] = 0u;  // candidate count, appended to later
  uint32_t key[kPartBlocks][4];
  load_part(scores + (size_t)row * score_stride, part, n, key);
  for (int j = lane; j < 2048; j += 64) hist[wave][j] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPartBlocks; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (key[j][e] != 0u) atomicAdd(&hist[wave][key[j][e] >> 21], 1u);
  __syncthreads();
  uint32_t* out = ws.hist + ((size_t)row * ws.parts + part) * 2048;
  for (int j = threadIdx.x; j < 2048; j += kPartThreads) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kPartWaves; ++w) t += hist[w][j];
    out[j] = t;
  }
}

// One wavefront finds, in totals[0..2048), the bin where the count from the
// top reaches `rem`; returns (bin, rem within the bin, count above the bin)
// through `res` (lane 0 of the crossing writes it).
__device__ __forceinline__ void find_bin(const uint32_t* totals, uint32_t rem, uint32_t* res) {
  const int lane = threadIdx.x & 63;
  uint32_t mine = 0;
  for (int j = 0; j < 32; ++j) mine += totals[lane * 32 + j];
  uint32_t from_top = mine;  // sum over lanes >= this one
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_down(from_top, off);
    if (lane + off < 64) from_top += t;
  }
  const uint32_t above = from_top - mine;
  if (above < rem && rem <= from_top) {  // exactly one lane
    uint32_t cum = above;
    for (int j = 31; j >= 0; --j) {
      const uint32_t c = totals[lane * 32 + j];
      if (cum + c >= rem) {
        res[0] = (uint32_t)(lane * 32 + j);
        res[1] = rem - cum;
        res[2] = cum;
        break;
      }
      cum += c;
    }
  }
}

// ---- 2. bin B0 of the row; keys above it counted, keys inside it listed
__global__ __launch_bounds__(kPartThreads) void topk_cands_kernel(const float* scores, int score_stride,
                                                                  const int32_t* seq_lens, int q_len, int topk,
                                                                  TopkWs ws) {
  __shared__ uint32_t total[2048];
  __shared__ uint32_t res[3];
  __shared__ uint32_t wave_above[kPartWaves];
  __shared__ uint32_t wave_in[kPartWaves];
  __shared__ uint32_t base_lds;
  const int part = blockIdx.x, row = blockIdx.y, b = row / q_len;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = row_len(seq_lens, b, score_stride);
  if (n <= topk) return;
  const uint32_t* h = ws.hist + (size_t)row * ws.parts * 2048;
  const int parts_used = (n + kPart - 1) / kPart;
  {
    // 8 bins per thread; the parts' counts are loaded 8 parts at a time, 64
    // loads in flight per thread
    constexpr int kBinsPer = 2048 / kPartThreads;
    uint32_t t[kBinsPer] = {};
    for (int q0 = 0; q0 < parts_used; q0 += 8) {
      uint32_t v[8][kBinsPer];
#pragma unroll
      for (int qq = 0; qq < 8; ++qq)
#pragma unroll
        for (int i = 0; i < kBinsPer; ++i)
          v[qq][i] = q0 + qq < parts_used ? h[(size_t)(q0 + qq) * 2048 + threadIdx.x + i * kPartThreads] : 0u;
#pragma unroll
      for (int qq = 0; qq < 8; ++qq)
#pragma unroll
        for (int i = 0; i < kBinsPer; ++i) t[i] += v[qq][i];
    }
#pragma unroll
    for (int i = 0; i < kBinsPer; ++i) total[threadIdx.x + i * kPartThreads] = t[i];
  }
  __syncthreads();
  if (wave == 0) find_bin(total, (uint32_t)topk, res);
  __syncthreads();
  const uint32_t b0 = res[0];
  if (part == 0 && threadIdx.x == 0) {
    ws.row_info[row * 4 + 1] = b0;
    ws.row_info[row * 4 + 2] = res[1];
    ws.row_info[row * 4 + 3] = res[2];
  }
  uint32_t key[kPartBlocks][4];
  load_part(scores + (size_t)row * score_stride, part, n, key);
  // count first, reserve the workgroup's range of the row's list with one
  // atomic, then write (the list's order does not matter)
  uint32_t above = 0, in_b0 = 0;
#pragma unroll
  for (int j = 0; j < kPartBlocks; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = key[j][e];
      above += k != 0u && (k >> 21) > b0;
      in_b0 += k != 0u && (k >> 21) == b0;
    }
  uint32_t lane_pre = in_b0;  // inclusive prefix over lanes, then exclusive
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(lane_pre, off);
    if (lane >= off) lane_pre += t;
  }
  const uint32_t wave_total = __shfl(lane_pre, 63);
  lane_pre -= in_b0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) above += __shfl_xor(above, off);
  if (lane == 0) {
    wave_above[wave] = above;
    wave_in[wave] = wave_total;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0, c = 0;
    for (int w = 0; w < kPartWaves; ++w) {
      t += wave_above[w];
      c += wave_in[w];
    }
    ws.part_cnt[((size_t)row * ws.parts + part) * 3 + 0] = t;
    base_lds = c ? atomicAdd(&ws.row_info[row * 4 + 0], c) : 0u;
  }
  __syncthreads();
  uint32_t slot = base_lds + lane_pre;
  for (int w = 0; w < wave; ++w) slot += wave_in[w];
  uint32_t* cand = ws.cand + (size_t)row * ws.parts * kPart * 2;
#pragma unroll
  for (int j = 0; j < kPartBlocks; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = key[j][e];
      if (k != 0u && (k >> 21) == b0) {
        cand[2 * slot] = k;
        cand[2 * slot + 1] = (uint32_t)(part * kPart + wave * (kPartBlocks * 256) + j * 256 + 4 * lane + e);
        ++slot;
      }
    }
}

// ---- 3. exact threshold from the candidates, then this part's output offset
// and tie share. Every part's workgroup of the write kernel computes it from
// the row's candidates (all get the same values), which costs each a few
// microseconds of LDS work but saves a kernel launch and its round trips.
struct RowSelect {
  uint32_t thr, off, ties;
};
__device__ RowSelect row_select(int row, int n, int part, const TopkWs& ws, uint32_t* total, uint32_t* res,
                                uint32_t* gt, uint32_t* eq, uint32_t* out3) {
  constexpr int NT = kPartThreads;
  const int tid = threadIdx.x, wave = tid >> 6;
  const uint32_t m = ws.row_info[row * 4 + 0];
  const uint32_t b0 = ws.row_info[row * 4 + 1];
  uint32_t rem = ws.row_info[row * 4 + 2];
  const uint32_t* cand = ws.cand + (size_t)row * ws.parts * kPart * 2;
  uint32_t prefix = b0 << 21;
  // two passes over the candidates: bits 20..10, then 9..0
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const uint32_t known = pass == 0 ? 0xFFE00000u : 0xFFFFFC00u;  // bits fixed so far
    const int nbins = pass == 0 ? 2048 : 1024;
    for (int j = tid; j < 2048; j += NT) total[j] = 0;
    __syncthreads();
    for (uint32_t c = tid; c < m; c += NT) {
      const uint32_t k = cand[2 * c];
      if ((k & known) == prefix) atomicAdd(&total[(k >> shift) & (nbins - 1)], 1u);
    }
    __syncthreads();
    if (wave == 0) find_bin(total, rem, res);
    __syncthreads();
    prefix |= res[0] << shift;
    rem = res[1];
    __syncthreads();  // res and the histogram are rewritten by the next pass
  }
  const uint32_t thr = prefix;  // the topk-th largest key; keep `rem` of the keys equal to it
  const int parts_used = (n + kPart - 1) / kPart;
  for (int q = tid; q < 128; q += NT) {
    gt[q] = 0;
    eq[q] = 0;
  }
  __syncthreads();
  for (uint32_t c = tid; c < m; c += NT) {
    const uint32_t k = cand[2 * c], q = cand[2 * c + 1] / kPart;
    if (k > thr) atomicAdd(&gt[q], 1u);
    if (k == thr) atomicAdd(&eq[q], 1u);
  }
  // keys above B0 per part (counted by the cands kernel)
  const uint32_t* pc_row = ws.part_cnt + (size_t)row * ws.parts * 3;
  for (int q = tid; q < parts_used; q += NT) atomicAdd(&gt[q], pc_row[q * 3 + 0]);
  __syncthreads();
  if (tid == 0) {
    uint32_t off = 0, eq_before = 0;
    for (int q = 0; q < part; ++q) {
      off += gt[q] + (eq_before >= rem ? 0u : min(eq[q], rem - eq_before));
      eq_before += eq[q];
    }
    out3[0] = off;
    out3[1] = eq_before >= rem ? 0u : min(eq[part], rem - eq_before);
  }
  __syncthreads();
  return RowSelect{thr, out3[0], out3[1]};
}

// ---- 4. selected positions of a part, in ascending order
__global__ __launch_bounds__(kPartThreads) void topk_write_kernel(const float* scores, int score_stride,
                                                                  const int32_t* seq_lens, int q_len, int topk,
                                                                  int32_t* out, unsigned* err, TopkWs ws) {
  __shared__ uint32_t wcnt[kPartWaves][2];
  __shared__ uint32_t total[2048];
  __shared__ uint32_t res[3], out3[2];
  __shared__ uint32_t gt[128], eq[128];  // per part: keys above / candidates equal to the threshold
  const int part = blockIdx.x, row = blockIdx.y, b = row / q_len;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t* o = out + (size_t)row * topk;
  const int n_raw = seq_lens[b];
  const int n = row_len(seq_lens, b, score_stride);
  if (n <= topk) {  // every position is selected; the rest of the row is -1
    if (part == 0) {
      if (threadIdx.x == 0 && (n_raw < topk || n_raw > score_stride)) flag_error(err, MLA_DEVERR_SEQ_LEN);
      for (int j = threadIdx.x; j < topk; j += kPartThreads) o[j] = j < n ? j : -1;
    }
    return;
  }
  if (part * kPart >= n) return;
  if (part == 0 && threadIdx.x == 0 && n_raw > score_stride) flag_error(err, MLA_DEVERR_SEQ_LEN);
  uint32_t key[kPartBlocks][4];
  load_part(scores + (size_t)row * score_stride, part, n, key);  // in flight during the selection
  const RowSelect sel = row_select(row, n, part, ws, total, res, gt, eq, out3);
  const uint32_t thr = sel.thr, part_off = sel.off, part_ties = sel.ties;
  uint32_t above = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < kPartBlocks; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      above += key[j][e] > thr;
      n_eq += key[j][e] == thr;
    }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    above += __shfl_xor(above, off);
    n_eq += __shfl_xor(n_eq, off);
  }
  if (lane == 0) {
    wcnt[wave][0] = above;
    wcnt[wave][1] = n_eq;
  }
  __syncthreads();
  uint32_t off = part_off, eq_before = 0;  // over the wavefronts before this one
  for (int w = 0; w < wave; ++w) {
    const uint32_t e_w = wcnt[w][1];
    off += wcnt[w][0] + (eq_before >= part_ties ? 0u : min(e_w, part_ties - eq_before));
    eq_before += e_w;
  }
  const uint32_t ties = eq_before >= part_ties ? 0u : min(n_eq, part_ties - eq_before);
  uint32_t t_seen = 0;
  const int lane_p0 = part * kPart + wave * (kPartBlocks * 256) + 4 * lane;
#pragma unroll
  for (int j = 0; j < kPartBlocks; ++j) {
    uint32_t c_eq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c_eq += key[j][e] == thr;
    const uint32_t eq_pre = prefix_below(c_eq);
    uint32_t tie_rank = t_seen + eq_pre;  // ties in this wavefront before this lane's first
    uint32_t n_take = 0, take_bits = 0;
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
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (take_bits & (1u << e)) o[w_pos++] = lane_p0 + j * 256 + e;
    t_seen += __shfl(eq_pre + c_eq, 63);
    off += __shfl(take_pre + n_take, 63);
  }
}

}  // namespace

size_t topk_workspace_bytes(int rows, int score_stride) {
  const size_t parts = (size_t)(score_stride + kPart - 1) / kPart;
  return (size_t)rows * (parts * 2048 * 4 + parts * kPart * 8 + 16 + parts * 12);
}

hipError_t launch_topk(const float* scores, int batch, int q_len, int score_stride, const int32_t* seq_lens,
                       int topk, int32_t* out, unsigned* err, void* workspace, hipStream_t stream) {
  const int rows = batch * q_len;
  TopkWs ws;
  ws.parts = (score_stride + kPart - 1) / kPart;
  char* p = static_cast<char*>(workspace);
  ws.hist = reinterpret_cast<uint32_t*>(p);
  p += (size_t)rows * ws.parts * 2048 * 4;
  ws.cand = reinterpret_cast<uint32_t*>(p);
  p += (size_t)rows * ws.parts * kPart * 8;
  ws.row_info = reinterpret_cast<uint32_t*>(p);
  p += (size_t)rows * 16;
  ws.part_cnt = reinterpret_cast<uint32_t*>(p);
  const dim3 parts_grid(ws.parts, rows);
  hipLaunchKernelGGL(topk_hist_kernel, parts_grid, dim3(kPartThreads), 0, stream, scores, score_stride, seq_lens,
                     q_len, topk, ws);
  hipLaunchKernelGGL(topk_cands_kernel, parts_grid, dim3(kPartThreads), 0, stream, scores, score_stride, seq_lens,
                     q_len, topk, ws);
  hipLaunchKernelGGL(topk_write_kernel, parts_grid, dim3(kPartThreads), 0, stream, scores, score_stride, seq_lens,
                     q_len, topk, out, err, ws);
  return hipGetLastError();
}

}  // namespace mla
