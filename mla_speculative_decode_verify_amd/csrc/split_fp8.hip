// Split-KV top-k sparse decode over an fp8 E4M3FN latent cache, gfx950.
//
// Cache row of token t: 512 E4M3FN latent bytes (scaled by the fp32 per-token
// scale[t]), plus 64 bf16 rope elements; the value is the scaled latent.
// Every (sequence, query) attends to exactly its list of top-k prefix
// positions ("The Occupancy Probe", section "The Scene": sparse decode of
// DeepSeek-V4 against an fp8 cache with per-token scales). The list is
// shared by all heads of that query, so a workgroup serves one (sequence,
// query, KV split, row group of heads) and reads each listed row once.
//
// The compute follows the bf16 verify kernel (pairs of wavefronts per 16-row
// block, each half owning 9 k-steps of the score and 256 output columns),
// with three differences:
//   * Tiles are built by four load-only wavefronts (one per SIMD), so the
//     pairs only compute: 8-byte fp8 pieces are loaded into registers one
//     tile ahead, converted exactly to bf16 (every E4M3FN value is a bf16
//     value) and written to a padded LDS tile of the same [32][576 + 16]
//     layout; rope pieces are copied as they are.
//   * The per-token scale stays in fp32: the score is
//       s_j = scale_j * <q_lat, lat_j> + <q_rope, rope_j>
//     from separate latent and rope MFMA accumulators, and the weight that
//     multiplies the raw latent in the PV product is bf16(p_j * scale_j).
//     The output is normalised by sum_j bf16(p_j * scale_j) / scale_j, the
//     weights actually applied, so a single key reproduces scale * latent
//     exactly; the LSE uses the exact fp32 sum of p_j.
//   * Keys that are past the split end, or whose position or slot is out of
//     range, get an additive score bias of -inf (and read the zero row), so
//     they carry no weight; no draft mask exists on this path.
#include <type_traits>

#include "device_common.h"
#include "mla_internal.h"
#include "mla_verify.h"
#include "split_epilogue.h"

namespace mla {
namespace {

constexpr int kTile = 32;                           // listed positions per tile
constexpr int kLdsStride = kDk + 16;                // bf16 elements per padded LDS row (1184 B)
constexpr int kTileElems = kTile * kLdsStride;
constexpr int kHalfSteps = kDk / 32 / 2;            // 9 MFMA k-steps per half
constexpr int kLatHalf1 = kDv / 32 - kHalfSteps;    // latent k-steps owned by half 1 (7)
constexpr int kHalfBlocks = kDv / 16 / 2;           // 16 output column blocks per half
constexpr int kLatPieces = kDv / 8;                 // 8-byte fp8 pieces per latent row (64)
constexpr int kRopePieces = kDrope / 8;             // 16-byte bf16 pieces per rope row (8)
constexpr int kChunk = 4096;                        // top-k entries staged in LDS at a time
constexpr float kRescaleSlack = 8.f;
constexpr int kAhead = 2;                           // LDS fragments read ahead of their MFMAs
// Bound on the polls of the pair-exchange wait (each poll sleeps about 64
// cycles; the partner publishes within a tile). Past it the wave records
// MLA_DEVERR_SYNC and continues, so a protocol fault can never hang the GPU.
constexpr int kSpinCap = 1 << 20;

__device__ __forceinline__ bf16x8 lds_read_b128(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ bf16x8 v_operand(const __bf16* vT0, int d) {
  const bf16x4 lo4 = lds_read_tr16(vT0 + 16 * d);
  const bf16x4 hi4 = lds_read_tr16(vT0 + 16 * d + 16 * kLdsStride);
  return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Eight E4M3FN bytes -> eight bf16 values (exact; NaN stays NaN).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint2 w) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_convertvector(__builtin_amdgcn_cvt_pk_f32_fp8(w.x, false), bf16x2);
  const bf16x2 b = __builtin_convertvector(__builtin_amdgcn_cvt_pk_f32_fp8(w.x, true), bf16x2);
  const bf16x2 c = __builtin_convertvector(__builtin_amdgcn_cvt_pk_f32_fp8(w.y, false), bf16x2);
  const bf16x2 d = __builtin_convertvector(__builtin_amdgcn_cvt_pk_f32_fp8(w.y, true), bf16x2);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One tile's worth of raw cache data held in registers by one lane: its
// share of the 32 x 64 latent pieces, of the 32 x 8 rope pieces and (lanes
// 0..31) one key's scale and validity.
template <int NW>
struct TileRegs {
  static constexpr int kNT = NW * 64;
  static constexpr int kL = (kTile * kLatPieces + kNT - 1) / kNT;
  static constexpr int kR = (kTile * kRopePieces + kNT - 1) / kNT;
  uint2 lat[kL];
  u32x4 rope[kR];
  float scale;
  bool valid;
};

// Issue the loads of tile [t0, t0 + 32) of the staged chunk (slots_lds holds
// the pool row of entry cb + i, or -1 for an invalid entry). Keys at or past
// `ce` and invalid keys read the zero row.
template <int NW>
__device__ __forceinline__ void load_tile(TileRegs<NW>& R, int tid, const int* slots_lds, int cb, int t0, int ce,
                                          const uint8_t* lat, const __bf16* rope, const float* scale,
                                          const uint8_t* zero_row) {
  constexpr int kNT = TileRegs<NW>::kNT;
  auto slot_of = [&](int k) { return t0 + k < ce ? slots_lds[t0 + k - cb] : -1; };
#pragma unroll
  for (int u = 0; u < TileRegs<NW>::kL; ++u) {
    const int it = tid + u * kNT;
    const int k = min(it / kLatPieces, kTile - 1), c = it % kLatPieces;
    const int s = slot_of(k);
    const uint8_t* src = s >= 0 ? lat + (size_t)s * kDv : zero_row;
    R.lat[u] = (kTile * kLatPieces % kNT == 0 || it < kTile * kLatPieces)
                   ? *reinterpret_cast<const uint2*>(src + 8 * c)
                   : uint2{0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < TileRegs<NW>::kR; ++u) {
    const int it = tid + u * kNT;
    const int k = min(it / kRopePieces, kTile - 1), c = it % kRopePieces;
    const int s = slot_of(k);
    const __bf16* src = s >= 0 ? rope + (size_t)s * kDrope : reinterpret_cast<const __bf16*>(zero_row);
    R.rope[u] = (kTile * kRopePieces % kNT == 0 || it < kTile * kRopePieces)
                    ? *reinterpret_cast<const u32x4*>(src + 8 * c)
                    : u32x4{0u, 0u, 0u, 0u};
  }
  R.valid = false;
  R.scale = 0.f;
  if (tid < kTile) {
    const int s = slot_of(tid);
    R.valid = s >= 0;
    R.scale = s >= 0 ? scale[s] : 0.f;
  }
}

// Convert and write a loaded tile into LDS buffer `buf` and its per-key
// scale, reciprocal scale (0 where the scale is 0 or the key is invalid) and
// score bias (0 or -inf).
template <int NW>
__device__ __forceinline__ void store_tile(const TileRegs<NW>& R, int tid, __bf16* buf, float* sc, float* isc,
                                           float* bias, int* plain) {
  constexpr int kNT = TileRegs<NW>::kNT;
#pragma unroll
  for (int u = 0; u < TileRegs<NW>::kL; ++u) {
    const int it = tid + u * kNT;
    if (kTile * kLatPieces % kNT == 0 || it < kTile * kLatPieces) {
      const int k = it / kLatPieces, c = it % kLatPieces;
      *reinterpret_cast<bf16x8*>(buf + k * kLdsStride + 8 * c) = e4m3x8_to_bf16(R.lat[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < TileRegs<NW>::kR; ++u) {
    const int it = tid + u * kNT;
    if (kTile * kRopePieces % kNT == 0 || it < kTile * kRopePieces) {
      const int k = it / kRopePieces, c = it % kRopePieces;
      *reinterpret_cast<u32x4*>(buf + k * kLdsStride + kDv + 8 * c) = R.rope[u];
    }
  }
  if (tid < kTile) {
    sc[tid] = R.scale;
    isc[tid] = (R.valid && R.scale != 0.f) ? 1.f / R.scale : 0.f;
    bias[tid] = R.valid ? 0.f : -INFINITY;
    // plain tile: every key valid with a nonzero scale, so its bias is 0 and
    // its reciprocal scale never needs the zero-scale fallback
    const uint64_t ok = __ballot(R.valid && R.scale != 0.f);
    if (tid == 0) *plain = (uint32_t)ok == 0xFFFFFFFFu ? 1 : 0;
  }
}

template <int NB>
constexpr int kThreads8 = (2 * NB + fp8_load_waves(NB)) * 64;

template <int NB>
__global__ __launch_bounds__(kThreads8<NB>, 1) void split_fp8_topk_kernel(Args a) {
  constexpr int NW = 2 * NB;                 // compute wavefronts (a pair per block)
  constexpr int NL = fp8_load_waves(NB);     // load-only wavefronts after them
  constexpr int NLW = NL > 0 ? NL : NW;      // wavefronts that load the tiles
  constexpr int kNT = (NW + NL) * 64;        // threads that stage the chunk
  __shared__ __attribute__((aligned(16))) __bf16 kv[2 * kTileElems];   // double-buffered tile
  __shared__ __attribute__((aligned(16))) float sc_lds[2][3][kTile];   // scale, 1/scale, bias per key
  __shared__ int plain_lds[2];                                         // the tile's keys all plain (see store_tile)
  __shared__ __attribute__((aligned(16))) f32x4 spart[NW][2][64];      // partial scores per wave
  __shared__ int slots_lds[kChunk];                                    // pool row per entry, -1 = invalid
  __shared__ int pair_seq[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const bool loader = NL > 0 && wave >= NW;  // wave-uniform
  const int half = wave & 1, blk = wave >> 1;
  // unit = (z * nsplit + split) * row_groups + grp with z = b * q_len + qi,
  // in XCD-aware order
  const int G = a.row_groups;
  const int unit = xcd_unit(a.batch * a.q_len * a.nsplit * G);
  if (unit < 0) return;  // padding workgroup: uniform exit before any barrier
  const int grp = unit % G, split = (unit / G) % a.nsplit, z = unit / (G * a.nsplit);
  const int b = z / a.q_len, qi = z - b * a.q_len;
  const int S = a.nsplit, H = a.heads, R = a.rows;

  int n = a.seq_lens[b];
  if (n < 0 || n > a.slot_stride) {
    if (tid == 0 && split == 0 && grp == 0 && qi == 0) flag_error(a.err, MLA_DEVERR_SEQ_LEN);
    n = n < 0 ? 0 : a.slot_stride;
  }
  const int K = a.topk;
  const int chunk = (K + S - 1) / S;
  const int lo = min(K, split * chunk);
  const int hi = min(K, lo + chunk);

  const int32_t* slot_row = a.slots + (size_t)b * a.slot_stride;
  const int32_t* topk_row = a.topk_idx + ((size_t)b * a.q_len + qi) * K;
  const uint8_t* lat = static_cast<const uint8_t*>(a.latent);
  const __bf16* rope = static_cast<const __bf16*>(a.rope);
  const uint8_t* zero_row = static_cast<const uint8_t*>(a.zero_row);
  const uint32_t pool_lim = (uint32_t)min<int64_t>(a.pool_rows, (int64_t)1 << 31);

  // ---- this wavefront's rows (heads) and query k-steps
  const int row0 = (grp * NB + blk) * 16;
  const bool active = row0 < H;  // uniform per wavefront pair
  const int h = row0 + li;
  const int r_glob = qi * H + min(h, H - 1);  // row within the sequence: query * heads + head

  bf16x8 qr[kHalfSteps];
  if (!loader) {
    const __bf16* qp =
        static_cast<const __bf16*>(a.q) + ((size_t)b * R + r_glob) * kDk + 32 * kHalfSteps * half + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kHalfSteps; ++ks) qr[ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks);
  }
  // queries in registers before the tile loads start, so no wait inside the
  // tile loop has to cover them
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  f32x4 o[kHalfBlocks];
#pragma unroll
  for (int d = 0; d < kHalfBlocks; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // exponent base, log2 domain
  float l = 0.f;        // lane share of sum p_j (gives the LSE)
  float lr = 0.f;       // lane share of the applied weights sum bf16(p_j scale_j) / scale_j (normalises O)
  bool bad_pos = false, bad_slot = false;

  const int offA = li * kLdsStride + 32 * kHalfSteps * half + 8 * g;
  const int offV = (4 * g + (li >> 2)) * kLdsStride + 256 * half + 4 * (li & 3);

  if (lane == 0 && !loader) __hip_atomic_store(&pair_seq[wave], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  int seq = 0;

  auto compute_tile = [&](const __bf16* cur, const float* sc, const float* isc, const float* bias, bool plain_in) {
    if (!active) return;
    const bool plain = __builtin_amdgcn_readfirstlane(plain_in ? 1 : 0) != 0;  // wave-uniform
    // ---- partial scores over this half's k-steps: latent and rope kept
    // apart. K fragments are read kAhead steps ahead of their MFMAs; the
    // scheduling barrier keeps the reads from sinking next to their use.
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, r0 = s0, r1 = s0;
    const __bf16* kA0 = cur + offA;
    bf16x8 kf0[kAhead + 1], kf1[kAhead + 1];
#pragma unroll
    for (int ks = 0; ks < kAhead; ++ks) {
      kf0[ks] = lds_read_b128(kA0 + 32 * ks);
      kf1[ks] = lds_read_b128(kA0 + 16 * kLdsStride + 32 * ks);
    }
    const bool rope_steps = half == 1;  // half 1's last two k-steps are the rope
#pragma unroll
    for (int ks = 0; ks < kHalfSteps; ++ks) {
      if (ks + kAhead < kHalfSteps) {
        kf0[(ks + kAhead) % (kAhead + 1)] = lds_read_b128(kA0 + 32 * (ks + kAhead));
        kf1[(ks + kAhead) % (kAhead + 1)] = lds_read_b128(kA0 + 16 * kLdsStride + 32 * (ks + kAhead));
      }
      const bf16x8 k0 = kf0[ks % (kAhead + 1)], k1 = kf1[ks % (kAhead + 1)];
      if (ks >= kLatHalf1 && rope_steps) {
        r0 = mfma_16x16x32(k0, qr[ks], r0);
        r1 = mfma_16x16x32(k1, qr[ks], r1);
      } else {
        s0 = mfma_16x16x32(k0, qr[ks], s0);
        s1 = mfma_16x16x32(k1, qr[ks], s1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane holds keys 16 kb + 4 g + r (r = 0..3) of row li
    const f32x4 sc0 = *reinterpret_cast<const f32x4*>(sc + 4 * g);
    const f32x4 sc1 = *reinterpret_cast<const f32x4*>(sc + 16 + 4 * g);
    const f32x4 own0 = sc0 * s0 + r0, own1 = sc1 * s1 + r1;
    spart[wave][0][lane] = own0;
    spart[wave][1][lane] = own1;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): partial stored before the flag
    if (lane == 0) __hip_atomic_store(&pair_seq[wave], seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    {
      int spins = 0;
      while (__hip_atomic_load(&pair_seq[wave ^ 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != seq) {
        if (++spins > kSpinCap) {  // a protocol fault: leave (results invalid) rather than hang
          flag_error(a.err, MLA_DEVERR_SYNC);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    asm volatile("" ::: "memory");
    // own + partner: addition commutes exactly, so both halves hold bitwise
    // the same sums
    f32x4 x0 = own0 + spart[wave ^ 1][0][lane];
    f32x4 x1 = own1 + spart[wave ^ 1][1][lane];
    if (!plain) {  // some key of the tile is masked: add its -inf bias
      x0 += *reinterpret_cast<const f32x4*>(bias + 4 * g);
      x1 += *reinterpret_cast<const f32x4*>(bias + 16 + 4 * g);
    }
    const f32x4 is0 = *reinterpret_cast<const f32x4*>(isc + 4 * g);
    const f32x4 is1 = *reinterpret_cast<const f32x4*>(isc + 16 + 4 * g);
    float x[8], s[8], is[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = x0[r];
      x[4 + r] = x1[r];
      s[r] = sc0[r];
      s[4 + r] = sc1[r];
      is[r] = is0[r];
      is[4 + r] = is1[r];
    }

    // ---- online softmax (log2 domain, lazy rescale)
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmaxf(mx, x[r]);
    mx = group4_max(mx) * a.scale_log2;
    if (__any(mx > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
      lr *= alpha;
#pragma unroll
      for (int d = 0; d < kHalfBlocks; ++d) o[d] *= alpha;
    }
    const float base = (m == -INFINITY) ? 0.f : m;
    bf16x8 pv;
    if (plain) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float pf = fast_exp2(fmaf(x[r], a.scale_log2, -base));
        const __bf16 wb = static_cast<__bf16>(pf * s[r]);
        pv[r] = wb;
        l += pf;
        lr += static_cast<float>(wb) * is[r];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float pf = fast_exp2(fmaf(x[r], a.scale_log2, -base));
        const __bf16 wb = static_cast<__bf16>(pf * s[r]);
        pv[r] = wb;
        l += pf;
        lr += is[r] != 0.f ? static_cast<float>(wb) * is[r] : pf;
      }
    }

    // ---- O^T[dim][row] += V^T P^T over this half's 16 column blocks
    const __bf16* vT0 = cur + offV;
    bf16x8 vf[kAhead + 1];
#pragma unroll
    for (int d = 0; d < kAhead; ++d) vf[d] = v_operand(vT0, d);
#pragma unroll
    for (int d = 0; d < kHalfBlocks; ++d) {
      if (d + kAhead < kHalfBlocks) vf[(d + kAhead) % (kAhead + 1)] = v_operand(vT0, d + kAhead);
      o[d] = mfma_16x16x32(vf[d % (kAhead + 1)], pv, o[d]);
    }
  };

  // ---- main loop. kLoad / kCompute select a wavefront's roles: with
  // load-only wavefronts (NL > 0) those stage nothing more than the others but
  // load, convert and store every tile, and the pairs only compute;
  // otherwise every wavefront does both. Both roles meet at the same
  // barriers: two per chunk before its first tile, one per tile.
  auto main_loop = [&](auto load_role, auto compute_role) {
    constexpr bool kLoad = decltype(load_role)::value;
    constexpr bool kCompute = decltype(compute_role)::value;
    const int ltid = NL > 0 ? tid - NW * 64 : tid;  // thread index among the loading wavefronts
    TileRegs<NLW> regs;
    for (int cb = lo; cb < hi; cb += kChunk) {
      const int ce = min(hi, cb + kChunk);
      // ---- stage the chunk: top-k position -> checked position -> checked pool row
      for (int i0 = 0; i0 < ce - cb; i0 += 8 * kNT) {
        int p[8], sl[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * kNT + tid;
          p[u] = i < ce - cb ? topk_row[cb + i] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * kNT + tid;
          const bool pos_ok = (uint32_t)p[u] < (uint32_t)n;
          bad_pos |= (i < ce - cb) && !pos_ok;
          sl[u] = (i < ce - cb && pos_ok) ? slot_row[p[u]] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * kNT + tid;
          const bool slot_ok = (uint32_t)sl[u] < pool_lim;
          bad_slot |= sl[u] != -1 && !slot_ok;
          if (i < ce - cb) slots_lds[i] = slot_ok ? sl[u] : -1;
        }
      }
      lds_barrier();  // staged rows visible to every wave
      if constexpr (kLoad) {
        load_tile<NLW>(regs, ltid, slots_lds, cb, cb, ce, lat, rope, a.kscale, zero_row);
        store_tile<NLW>(regs, ltid, kv, sc_lds[0][0], sc_lds[0][1], sc_lds[0][2], &plain_lds[0]);
        if (cb + kTile < ce) load_tile<NLW>(regs, ltid, slots_lds, cb, cb + kTile, ce, lat, rope, a.kscale, zero_row);
      }
      lds_barrier();
      int buf = 0;
      for (int t0 = cb; t0 < ce; t0 += kTile) {
        if constexpr (kCompute) {
          compute_tile(kv + buf * kTileElems, sc_lds[buf][0], sc_lds[buf][1], sc_lds[buf][2], plain_lds[buf] != 0);
          ++seq;
        }
        if constexpr (kLoad) {
          if (t0 + kTile < ce) {
            // The other buffer was last read in the previous tile, which every
            // wave finished before the barrier that ended it.
            store_tile<NLW>(regs, ltid, kv + (buf ^ 1) * kTileElems, sc_lds[buf ^ 1][0], sc_lds[buf ^ 1][1],
                            sc_lds[buf ^ 1][2], &plain_lds[buf ^ 1]);
            if (t0 + 2 * kTile < ce)
              load_tile<NLW>(regs, ltid, slots_lds, cb, t0 + 2 * kTile, ce, lat, rope, a.kscale, zero_row);
          }
        }
        lds_barrier();  // next tile in LDS; this tile's buffer and the partial scores are free
        buf ^= 1;
      }
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  if constexpr (NL == 0) {
    main_loop(yes{}, yes{});
  } else {
    if (loader) {
      // (returning here keeps the pairs' query registers and accumulators
      // out of this path's live ranges)
      main_loop(yes{}, no{});
      if (__any(bad_pos) && lane == 0) flag_error(a.err, MLA_DEVERR_TOPK_RANGE);
      if (__any(bad_slot) && lane == 0) flag_error(a.err, MLA_DEVERR_SLOT_RANGE);
      return;
    }
    main_loop(no{}, yes{});
  }
  if (__any(bad_pos) && lane == 0) flag_error(a.err, MLA_DEVERR_TOPK_RANGE);
  if (__any(bad_slot) && lane == 0) flag_error(a.err, MLA_DEVERR_SLOT_RANGE);

  // ---- epilogue
  if (!active) return;
  const float lt = group4_sum(l);
  const float ltr = group4_sum(lr);
  const float inv = ltr > 0.f ? 1.f / ltr : 0.f;
  const float lse_v = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
  // the tile buffers are free now: 8 KiB of them per wavefront stage the stores
  static_assert(NW * kStageHalves * 2 <= (int)sizeof(kv), "staging areas fit the tile buffers");
  store_block_half(a, o, inv, lse_v, b, split, qi * H + row0, min(16, H - row0), half, g, half == 0 && g == 0,
                   reinterpret_cast<_Float16*>(kv) + wave * kStageHalves);
}

template <int NB>
hipError_t launch_nb(const Args& a, int row_groups, hipStream_t stream) {
  Args b = a;
  b.row_groups = row_groups;
  const long units = (long)a.batch * a.q_len * a.nsplit * row_groups;
  hipLaunchKernelGGL(split_fp8_topk_kernel<NB>, dim3(xcd_grid(units, b.xcd_chunk)), dim3(kThreads8<NB>), 0, stream,
                     b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split_fp8_topk(const Args& a, int blocks, int row_groups, hipStream_t stream) {
  switch (blocks) {
    case 1: return launch_nb<1>(a, row_groups, stream);
    case 2: return launch_nb<2>(a, row_groups, stream);
    case 3: return launch_nb<3>(a, row_groups, stream);
    case 4: return launch_nb<4>(a, row_groups, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mla
