// Split-KV verify attention over a bf16 latent cache (page_size = 1), gfx950.
//
// One workgroup handles one (sequence, KV split, row group). A row group is
// NW blocks of 16 query rows (row = draft * heads + head); each wavefront owns
// one block: its 16 absorbed query rows stay in VGPRs for the whole split and
// its 16 x 512 fp32 output accumulator lives in registers.
//
// Per tile of 32 cache positions:
//   1. gather: every thread loads 16-byte pieces of the 32 latent rows through
//      the slot table (coalesced 16 B loads; each 1152 B row is 72 pieces)
//      into registers one tile ahead, then stores them to an LDS tile
//      [32][576 + 8 pad] that all wavefronts share. The rows are read from
//      HBM once per row group, not once per head ("The Occupancy Epiphany",
//      section "The Per-Head Design": head-tile amortisation of the KV loads).
//   2. S^T = K Q^T on MFMA 16x16x32 bf16: 2 key blocks x 18 k-steps.
//   3. draft mask (only in tiles that reach the drafts or the split end),
//      online softmax in the log2 domain, probabilities rounded to bf16.
//   4. O^T += V^T P^T on MFMA: V is the first 512 columns of the same LDS tile,
//      read with the gfx950 transposing LDS load, so no second copy exists.
// The epilogue writes the normalised partial output and its natural-log LSE
// (or the final output when the call has one split).
#include "device_common.h"
#include "mla_internal.h"
#include "mla_verify.h"

namespace mla {
namespace {

constexpr int kTile = 32;                          // cache positions per tile (2 MFMA key blocks)
constexpr int kPieces = kDk / 8;                   // 16-byte pieces per latent row (72)
constexpr int kRowPieces = kPieces + 1;            // + one pad piece: LDS row = 1168 B (spreads banks)
constexpr int kLdsStride = kRowPieces * 8;         // bf16 elements per LDS row
constexpr int kTilePieces = kTile * kRowPieces;    // 2336
constexpr int kSegments = (kTilePieces + 63) / 64; // 64-piece wave loads per tile (37)
constexpr int kBufElems = kSegments * 64 * 8;      // one tile buffer incl. the tail segment

// Issue this wave's share of one tile's gather straight into LDS. Piece p of
// the padded tile is row p / 73, column piece p % 73; each wave instruction
// moves 64 consecutive pieces (1 KiB) from 64 independent 16-byte addresses.
// Rows outside [lo, hi) or with a bad slot read the zero row instead, so the
// tile never holds stale or poisoned data.
__device__ __forceinline__ void gather_tile(__bf16* buf, int wave, int nw, int lane, int slot_vec,
                                            const __bf16* pool, const __bf16* zero_row) {
  for (int sg = wave; sg < kSegments; sg += nw) {
    const int p = sg * 64 + lane;
    const int row = p / kRowPieces;
    const int part = min(p - row * kRowPieces, kPieces - 1);
    const int slot = __shfl(slot_vec, row & 31);
    const __bf16* src = slot >= 0 ? pool + (size_t)slot * kDk + part * 8 : zero_row + part * 8;
    if (p < kTilePieces) {
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(buf + sg * 512), 16, 0, 0);
    }
  }
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void split_bf16_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) __bf16 kv[2 * kBufElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int split = blockIdx.x, grp = blockIdx.y, b = blockIdx.z;
  const int S = a.nsplit, R = a.rows;
  const bool leader = (tid == 0) && (split == 0) && (grp == 0);

  // ---- sequence bounds and this split's key range
  int n = a.seq_lens[b];
  if (n < 0 || n > a.slot_stride) {
    if (leader) flag_error(a.err, MLA_DEVERR_SEQ_LEN);
    n = n < 0 ? 0 : a.slot_stride;
  }
  int prefix = n;
  if (a.mask_kind != MLA_MASK_NONE) {
    prefix = n - a.q_len;
    if (prefix < 0) {
      if (leader) flag_error(a.err, MLA_DEVERR_SEQ_LEN);
      prefix = 0;
    }
  }
  const int chunk = (n + S - 1) / S;
  const int lo = min(n, split * chunk);
  const int hi = min(n, lo + chunk);

  const int32_t* slot_row = a.slots + (size_t)b * a.slot_stride;
  const __bf16* pool = static_cast<const __bf16*>(a.latent);
  const __bf16* zero_row = static_cast<const __bf16*>(a.zero_row);
  // lane k < 32 of every wave holds the slot of key t0 + k (-1: read zeros)
  auto load_slots = [&](int t0) {
    const int j = t0 + (lane & 31);
    int s = -1;
    if (j < hi) {
      s = slot_row[j];
      if (s < 0 || (int64_t)s >= a.pool_rows) {
        flag_error(a.err, MLA_DEVERR_SLOT_RANGE);
        s = -1;
      }
    }
    return s;
  };

  // ---- start the first tile's gather before anything else
  int slots_next = -1;
  if (lo < hi) {
    const int s0 = load_slots(lo);
    gather_tile(kv, wave, NW, lane, s0, pool, zero_row);
    if (lo + kTile < hi) slots_next = load_slots(lo + kTile);
  }

  // ---- this wavefront's 16 query rows
  const int row0 = (grp * NW + wave) * 16;
  const bool wave_active = row0 < R;
  const int row = row0 + li;
  const int rowc = row < R ? row : R - 1;
  const int qi = rowc / a.heads;
  uint64_t anc_bits = ~0ull;
  if (a.mask_kind == MLA_MASK_CAUSAL) anc_bits = (2ull << qi) - 1ull;  // drafts 0..qi
  else if (a.mask_kind == MLA_MASK_TREE) anc_bits = a.anc[(size_t)b * a.q_len + qi];
  const uint32_t anc_lo = (uint32_t)anc_bits, anc_hi = (uint32_t)(anc_bits >> 32);

  bf16x8 qr[18];
  {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) +
                                                       ((size_t)b * R + rowc) * kDk) + g;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qr[ks] = qp[ks * 4];
  }

  f32x4 o[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // running max, log2 domain
  float l = 0.f;        // this lane's share of the running sum of exp (gives the LSE)
  float lr = 0.f;       // same sum over the bf16-rounded weights fed to the MFMA (normalises O)

  // lane coordinates for the transposing V reads: row 4g + tb, column 4tc
  const int tb = li >> 2, tc = li & 3;
  const int offA = li * kLdsStride + 8 * g;
  const int offV = (4 * g + tb) * kLdsStride + 4 * tc;

  int buf = 0;
  for (int t0 = lo; t0 < hi; t0 += kTile, buf ^= 1) {
    wait_vm_all();     // this wave's pieces of tile t0 have landed
    __syncthreads();   // ... and every other wave's; the other buffer is free
    if (t0 + kTile < hi) {
      const int s_cur = slots_next;
      if (t0 + 2 * kTile < hi) slots_next = load_slots(t0 + 2 * kTile);
      gather_tile(kv + (buf ^ 1) * kBufElems, wave, NW, lane, s_cur, pool, zero_row);
    }
    if (!wave_active) continue;
    const __bf16* tile = kv + buf * kBufElems;
    const __bf16* kA0 = tile + offA;
    const __bf16* kA1 = kA0 + 16 * kLdsStride;
    const __bf16* vT0 = tile + offV;
    const __bf16* vT1 = vT0 + 16 * kLdsStride;

    // ---- S^T[key][row] = K Q^T
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kA0 + 32 * ks);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kA1 + 32 * ks);
      s0 = mfma_16x16x32(k0, qr[ks], s0);
      s1 = mfma_16x16x32(k1, qr[ks], s1);
    }
    // lane holds row li, keys t0 + 16*kb + 4g + r
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = s0[r] * a.scale_log2;
      x[4 + r] = s1[r] * a.scale_log2;
    }
    if (t0 + kTile > hi || t0 + kTile > prefix) {
      // branch-free: key j is visible iff j < hi and (j is in the prefix or
      // its draft bit is set for this row's query)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int j = t0 + (r >> 2) * 16 + 4 * g + (r & 3);
        const int d = j - prefix;
        const uint32_t word = d < 32 ? anc_lo : anc_hi;
        const uint32_t bit = (word >> (d & 31)) & 1u;
        const bool vis = (j < hi) & ((d < 0) | (bit != 0u));
        x[r] = vis ? x[r] : -INFINITY;
      }
    }
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmaxf(mx, x[r]);
    mx = group4_max(mx);
    const float m_new = fmaxf(m, mx);
    const float base = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - base);
    bf16x8 pv;
    float psum = 0.f, psum_r = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float pf = fast_exp2(x[r] - base);
      const __bf16 pb = static_cast<__bf16>(pf);
      pv[r] = pb;
      psum += pf;
      psum_r += static_cast<float>(pb);
    }
    l = l * alpha + psum;
    lr = lr * alpha + psum_r;
    m = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int d = 0; d < 32; ++d) o[d] *= alpha;
    }

    // ---- O^T[dim][row] += V^T P^T
#pragma unroll
    for (int d = 0; d < 32; ++d) {
      const bf16x4 lo4 = lds_read_tr16(vT0 + 16 * d);
      const bf16x4 hi4 = lds_read_tr16(vT1 + 16 * d);
      const bf16x8 va = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
      o[d] = mfma_16x16x32(va, pv, o[d]);
    }
  }

  if (!wave_active) return;
  // ---- epilogue: normalise and store this split's result
  const float lt = group4_sum(l);
  const float ltr = group4_sum(lr);
  const float inv = ltr > 0.f ? 1.f / ltr : 0.f;
  const float lse_v = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
  if (row < R) {
    float* dst;
    float* lse_dst;
    if (S == 1) {
      dst = a.out + ((size_t)b * R + row) * kDv;
      lse_dst = a.lse ? a.lse + (size_t)b * R + row : nullptr;
    } else {
      const size_t pr = ((size_t)b * S + split) * R + row;
      dst = a.part_o + pr * kDv;
      lse_dst = a.part_lse + pr;
    }
#pragma unroll
    for (int d = 0; d < 32; ++d) *reinterpret_cast<f32x4*>(dst + 16 * d + 4 * g) = o[d] * inv;
    if (g == 0 && lse_dst) *lse_dst = lse_v;
  }
}

template <int NW>
hipError_t launch_nw(const Args& a, int row_groups, hipStream_t stream) {
  dim3 grid(a.nsplit, row_groups, a.batch);
  hipLaunchKernelGGL(split_bf16_kernel<NW>, grid, dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split_bf16(const Args& a, int waves, int row_groups, hipStream_t stream) {
  switch (waves) {
    case 1: return launch_nw<1>(a, row_groups, stream);
    case 2: return launch_nw<2>(a, row_groups, stream);
    case 3: return launch_nw<3>(a, row_groups, stream);
    case 4: return launch_nw<4>(a, row_groups, stream);
    case 5: return launch_nw<5>(a, row_groups, stream);
    case 6: return launch_nw<6>(a, row_groups, stream);
    case 7: return launch_nw<7>(a, row_groups, stream);
    case 8: return launch_nw<8>(a, row_groups, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mla
