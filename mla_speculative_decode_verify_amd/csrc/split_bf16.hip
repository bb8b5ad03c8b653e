// Split-KV verify attention over a bf16 latent cache (page_size = 1), gfx950.
//
// One workgroup handles one (sequence, KV split, row group). Query rows are
// row = draft * heads + head, cut into blocks of 16 (one MFMA tile); a row
// group is NB blocks. Every block is served by a PAIR of wavefronts: half 0
// owns k-steps 0..8 of the 576-wide score dot product and output columns
// 0..255, half 1 owns k-steps 9..17 and columns 256..511. Each half computes
// a partial S over its k-steps, the two partials meet in LDS (summed in a
// fixed order so both halves hold bitwise the same scores; the two waves
// synchronise through a per-wave sequence flag, not a workgroup barrier), both run the
// same online softmax, and each accumulates its own 256 output columns. A
// wavefront therefore keeps only 36 query registers and a 16 x 256 fp32
// accumulator, which leaves room for two or three wavefronts per SIMD: the
// hardware hides LDS and MFMA latency by switching between them.
//
// Up to 4 blocks, and with 5, extra wavefronts do nothing but issue the
// gathers and L2 prefetches of step 1: two on SIMDs 2 and 3 (the SIMDs the
// pairs leave one wavefront short) for an odd number of blocks, one per SIMD
// for 2 and 4. With 6 blocks the pairs issue them.
//
// Per tile of 32 cache positions:
//   1. gather: 16-byte pieces of the 32 latent rows (each 1152 B row is 72
//      pieces) are loaded through the slot table straight into an LDS tile
//      [32][576 + 16 pad] shared by all wavefronts, two tiles ahead of the
//      one being consumed. The rows are read from HBM once per row group,
//      not once per head ("The Occupancy Epiphany", section "The Per-Head
//      Design": head-tile amortisation of the KV loads).
//   2. partial S^T = K Q^T on MFMA 16x16x32 bf16 (2 key blocks x 9 k-steps).
//   3. exchange partials, draft mask (only in tiles that reach the drafts or
//      the split end), online softmax in the log2 domain, bf16 weights.
//   4. O^T += V^T P^T on MFMA: V is the first 512 columns of the same LDS tile,
//      read with the gfx950 transposing LDS load, so no second copy exists.
// The epilogue writes the normalised partial output and its natural-log LSE
// (or the final output when the call has one split).
//
// The gathers are issued as inline assembly and counted by hand: the compiler
// would otherwise drain the whole load queue before every LDS read of a tile
// (it cannot tell which buffer an in-flight global-to-LDS load writes). The
// slot table of each chunk of up to 2048 positions is staged in LDS first, so
// the only vector-memory operations inside the tile loop are the gathers.
//
// The running max is updated lazily: the exponent base only moves (and the
// accumulators are only rescaled) when some row's max grows by more than
// kRescaleSlack in log2 units, so weights stay below 2^kRescaleSlack.
#include <type_traits>

#include "device_common.h"
#include "mla_internal.h"
#include "mla_verify.h"
#include "split_common.h"
#include "split_epilogue.h"

namespace mla {
namespace {

using namespace tile;

constexpr int kHalfSteps = kDk / 32 / 2;           // 9 MFMA k-steps per half
constexpr int kHalfBlocks = kDv / 16 / 2;          // 16 output column blocks per half
constexpr int kSlotChunk = 2048;                   // cache positions whose row addresses are staged in LDS at a time
#ifndef MLA_KAHEAD
#define MLA_KAHEAD 2
#endif
constexpr int kAhead = MLA_KAHEAD;                 // LDS fragments read ahead of their MFMAs
#ifndef MLA_V_EARLY
#define MLA_V_EARLY 0
#endif
#ifndef MLA_VAHEAD
#define MLA_VAHEAD MLA_KAHEAD
#endif
constexpr int kVAhead = MLA_VAHEAD;                // V fragments read ahead of their MFMAs

template <int NB>
constexpr int kGatherWaves = bf16_gather_waves(NB);
template <int NB>
constexpr int kThreads = (2 * NB + kGatherWaves<NB>) * 64;

// Bound on the polls of the pair-exchange wait (each poll sleeps about 64
// cycles; the partner publishes within a tile, well under a thousand polls).
// Past it the wave records MLA_DEVERR_SYNC and continues, so a protocol fault
// can never hang the GPU.
constexpr int kSpinCap = 1 << 20;

template <int NB, bool kBalanced, bool kPf>
__global__ __launch_bounds__(kThreads<NB>, 1) void split_bf16_kernel(Args a) {
  constexpr int NW = 2 * NB;             // compute wavefronts (a pair per block)
  constexpr int NG = kGatherWaves<NB>;   // gather-only wavefronts after them
  constexpr int NGW = NG > 0 ? NG : NW;  // wavefronts that issue the gathers
  constexpr int NT = NW + NG;
  // Fewest gather instructions any gathering wave issues per tile: waiting
  // until at most that many are outstanding proves tile t has landed
  // whenever tile t+1 was issued after it (loads retire in order).
  constexpr int kWaitAhead = (kSegments / NGW) < 63 ? (kSegments / NGW) : 63;
  __shared__ __attribute__((aligned(16))) __bf16 kv[kStages * kBufElems];  // tile ring
  __shared__ __attribute__((aligned(16))) f32x4 spart[NW][2][64];          // partial scores per wave
  __shared__ const char* rows_lds[kSlotChunk + kTile];                     // cache-row addresses of the chunk
  __shared__ int pair_seq[NW];  // last tile whose partial scores each wave has published
  __shared__ uint32_t pf_sink[kPfAhead > 0 ? kPfOps * 64 : 1];  // landing words of the L2 prefetches (never read)

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar wave index
  const int g = lane >> 4, li = lane & 15;
  const int half = wave & 1, blk = wave >> 1;
  // unit = (k * row_groups + grp) in XCD-aware order, where k = b * nsplit +
  // split (uniform counts) or the running split index over the batch
  // (length-following counts, kBalanced)
  const int G = a.row_groups;
  const int unit = xcd_unit((kBalanced ? a.balance_units : a.batch * a.nsplit) * G);
  if (unit < 0) return;  // padding workgroup: uniform exit before any barrier
  const int grp = unit % G, k = unit / G;
  int b, split, S, len = 0;  // S = splits of sequence b
  if (kBalanced) {
    // every wavefront derives the same schedule, so the exit is uniform
    const BalancedSplit bs = balanced_split(a.seq_lens, a.batch, a.slot_stride, a.nsplit, a.balance_units);
    if (k >= bs.total) return;
    // wave-uniform values, kept in scalar registers
    b = __builtin_amdgcn_readfirstlane(__popcll(__ballot(lane < a.batch && bs.first + bs.count <= k)));
    split = __builtin_amdgcn_readfirstlane(k - __shfl(bs.first, b));
    S = __builtin_amdgcn_readfirstlane(__shfl(bs.count, b));
    len = __builtin_amdgcn_readfirstlane(__shfl(bs.len, b));
  } else {
    split = k % a.nsplit;
    b = k / a.nsplit;
    S = a.nsplit;
  }
  const int R = a.rows;
  const bool leader = (tid == 0) && (split == 0) && (grp == 0);
  // the merge reads each sequence's split count from the workspace instead
  // of deriving the schedule again in every one of its workgroups
  if (kBalanced && leader) a.part_count[b] = S;
  const int32_t* slot_row = a.slots + (size_t)b * a.slot_stride;

  // ---- first batch of slot loads, issued before the sequence length is
  // known: they assume the split range that the host's length bound implies
  // and are used only if the true range turns out the same, so the slot
  // loads no longer wait behind the length load (uniform counts only: with
  // length-following counts the length is already known)
  constexpr int kBatch = NT * 64;  // slot loads per staging pass and unroll step
  int lo_h = 0, hi_h = 0;
  if (!kBalanced) split_range(a.len_hint, S, split, lo_h, hi_h);
  int v_h[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = u * kBatch + tid;
    v_h[u] = (i < min(hi_h - lo_h, kSlotChunk) && lo_h + i < a.slot_stride) ? slot_row[lo_h + i] : -1;
  }

  // ---- sequence bounds and this split's key range
  int n = kBalanced ? len : a.seq_lens[b];
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
  int lo, hi;
  split_range(n, S, split, lo, hi);
  const bool hint_ok = lo == lo_h && hi <= hi_h;  // the early loads hold this split's first slots
  const char* pool = static_cast<const char*>(a.latent);
  const char* zero_row = static_cast<const char*>(a.zero_row);
  const uint32_t pool_lim = (uint32_t)min<int64_t>(a.pool_rows, (int64_t)1 << 31);
  // uniform; the instantiation without prefetch keeps the registers its
  // plan would take (short splits, where the prefetch does not pay)
  const bool pf_on = kPf && kPfAhead > 2 && hi - lo >= kPfMinKeys;
  const bool gather_only = NG > 0 && wave >= NW;  // wave-uniform

  // ---- this wavefront's rows, draft-mask words and query k-steps
  const int row0 = (grp * NB + blk) * 16;
  const bool active = row0 < R;  // uniform per wavefront pair
  const int row = row0 + li;
  const int qi = min(row, R - 1) / a.heads;
  uint64_t bits = ~0ull;
  if (a.mask_kind == MLA_MASK_CAUSAL) bits = (2ull << qi) - 1ull;  // drafts 0..qi
  else if (a.mask_kind == MLA_MASK_TREE) bits = a.anc[(size_t)b * a.q_len + qi];
  const uint32_t anc_lo = (uint32_t)bits, anc_hi = (uint32_t)(bits >> 32);

  bf16x8 qr[kHalfSteps];
  if (!gather_only) {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + ((size_t)b * R + min(row, R - 1)) * kDk +
                       32 * kHalfSteps * half + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kHalfSteps; ++ks) qr[ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks);
  }
  // (the query loads retire while the slot chunk is staged; the drain before
  // the first gathers makes sure of it)

  f32x4 o[kHalfBlocks];
#pragma unroll
  for (int d = 0; d < kHalfBlocks; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // exponent base, log2 domain (a lower bound of the running max)
  float l = 0.f;        // lane share of the running sum of exp (gives the LSE)
  float lr = 0.f;       // same over the bf16-rounded weights fed to the MFMA (normalises O)
  bool bad_slot = false;

  // lane offsets: K operand row li, columns 8g of this half's k-range;
  // V operand row 4g + li / 4, columns 4 (li % 4) of this half's columns
  const int offA = li * kLdsStride + 32 * kHalfSteps * half + 8 * g;
  const int offV = (4 * g + (li >> 2)) * kLdsStride + 256 * half + 4 * (li & 3);

  if (lane == 0 && !gather_only) __hip_atomic_store(&pair_seq[wave], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  int seq = 0;                         // tiles processed by this workgroup

  // chunk_bad: the staged chunk holds an invalid slot, so every tile of it
  // takes the masked path, which also drops keys staged with the zero row.
  auto compute_tile = [&](const __bf16* cur, int t0, int cb, int ce, bool chunk_bad) {
    // ---- partial S^T[key][row] over this half's 9 k-steps; K fragments are
    // read kAhead steps ahead of the MFMAs that use them
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
    const __bf16* vT0 = cur + offV;
    bf16x8 vf[kVAhead + 1];
    if (active) {
      const __bf16* kA0 = cur + offA;
      bf16x8 kf0[kAhead + 1], kf1[kAhead + 1];
#pragma unroll
      for (int ks = 0; ks < kAhead; ++ks) {
        kf0[ks] = lds_read_b128(kA0 + 32 * ks);
        kf1[ks] = lds_read_b128(kA0 + 16 * kLdsStride + 32 * ks);
      }
#pragma unroll
      for (int ks = 0; ks < kHalfSteps; ++ks) {
        if (ks + kAhead < kHalfSteps) {
          kf0[(ks + kAhead) % (kAhead + 1)] = lds_read_b128(kA0 + 32 * (ks + kAhead));
          kf1[(ks + kAhead) % (kAhead + 1)] = lds_read_b128(kA0 + 16 * kLdsStride + 32 * (ks + kAhead));
        }
        s0 = mfma_16x16x32(kf0[ks % (kAhead + 1)], qr[ks], s0);
        s1 = mfma_16x16x32(kf1[ks % (kAhead + 1)], qr[ks], s1);
        // keep the reads where they are: left alone, the scheduler sinks
        // them next to their MFMAs to save registers and serialises the loop
        __builtin_amdgcn_sched_barrier(0);
      }
      spart[wave][0][lane] = s0;
      spart[wave][1][lane] = s1;
      if (MLA_V_EARLY) {
        // the first V fragments do not depend on the scores: their LDS
        // latency overlaps the score exchange and the softmax
#pragma unroll
        for (int d = 0; d < kVAhead; ++d) vf[d] = v_operand(vT0, d);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!active) return;
    // Publish this wave's partial, then wait for the partner wave's: only the
    // pair synchronises here, not the workgroup. The partner publishes every
    // tile too, so the wait ends; it cannot run a tile ahead because both
    // must pass the next tile barrier first.
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
    // Both halves form half 0 + half 1 (addition commutes exactly), so the
    // pair holds bitwise the same scores.
    s0 += spart[wave ^ 1][0][lane];
    s1 += spart[wave ^ 1][1][lane];

    // ---- mask + online softmax (lane holds row li, keys t0 + 16 kb + 4g + r)
    float x[8];  // raw scores; the softmax scale (> 0) is applied inside the exponent
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = s0[r];
      x[4 + r] = s1[r];
    }
    if (chunk_bad || t0 + kTile > hi || t0 + kTile > prefix) {
      // branch-free: key j is visible iff j < hi, its slot is valid and (j is
      // in the prefix or its draft bit is set for this row's query)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int j = t0 + (r >> 2) * 16 + 4 * g + (r & 3);
        const int d = j - prefix;
        const uint32_t word = d < 32 ? anc_lo : anc_hi;
        const uint32_t bit = (word >> (d & 31)) & 1u;
        const bool slot_ok = rows_lds[j - cb] != zero_row;
        const bool vis = (j < hi) & slot_ok & ((d < 0) | (bit != 0u));
        x[r] = vis ? x[r] : -INFINITY;
      }
    }
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmaxf(mx, x[r]);
    mx = group4_max(mx) * a.scale_log2;
    // move the base only when some row's max outgrew it by more than the slack
    if (__any(mx > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mx);
      // 0 when the old base was -inf; rows still without a visible key keep alpha = 1
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
      lr *= alpha;
#pragma unroll
      for (int d = 0; d < kHalfBlocks; ++d) o[d] *= alpha;
    }
    const float base = (m == -INFINITY) ? 0.f : m;
    bf16x8 pv;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float pf = fast_exp2(fmaf(x[r], a.scale_log2, -base));
      pv[r] = static_cast<__bf16>(pf);
      l += pf;
    }
    lr = sum_bf16x8(pv, lr);

    // ---- O^T[dim][row] += V^T P^T over this half's 16 column blocks
    if (!MLA_V_EARLY) {
#pragma unroll
      for (int d = 0; d < kVAhead; ++d) vf[d] = v_operand(vT0, d);
    }
#pragma unroll
    for (int d = 0; d < kHalfBlocks; ++d) {
      if (d + kVAhead < kHalfBlocks) vf[(d + kVAhead) % (kVAhead + 1)] = v_operand(vT0, d + kVAhead);
      o[d] = mfma_16x16x32(vf[d % (kVAhead + 1)], pv, o[d]);
    }
  };

  // ---- main loop: chunks of up to kSlotChunk positions, tiles pipelined two
  // ahead. kGather / kCompute select a wavefront's roles: with gather-only
  // wavefronts (NG > 0) those issue every gather and prefetch and the pairs
  // only compute; otherwise every wavefront does both. Both roles meet at the
  // same barriers: one per chunk after the staging, one per tile, one at the
  // chunk's end.
  auto main_loop = [&](auto gather_role, auto compute_role) {
    constexpr bool kGather = decltype(gather_role)::value;
    constexpr bool kCompute = decltype(compute_role)::value;
    const int gw = NG > 0 ? wave - NW : wave;  // index among the gathering wavefronts
    GatherPlan<NGW> gp(kGather ? gw : 0, lane);
    // prefetch ops of one tile this wavefront issues: gw, gw + NGW, ...
    constexpr int kPfPer = (kPfOps + NGW - 1) / NGW;
    uint32_t pf_plan[kPfPer];
#pragma unroll
    for (int k = 0; k < kPfPer; ++k) pf_plan[k] = prefetch_plan(min(gw + k * NGW, kPfOps - 1), lane);
    auto prefetch = [&](uint32_t sink, int t_rel) {
#pragma unroll
      for (int k = 0; k < kPfPer; ++k)
        if (gw + k * NGW < kPfOps) prefetch_tile(sink, gw + k * NGW, pf_plan[k], rows_lds, t_rel);
    };
    for (int cb = lo; cb < hi; cb += kSlotChunk) {
      const int ce = min(hi, cb + kSlotChunk);
      // stage the chunk's row addresses (batches of 8 slot loads per thread in
      // flight at once), plus kTile zero-row entries past its end
      bool lane_bad = false;
      for (int i0 = 0; i0 < ce - cb + kTile; i0 += 8 * kBatch) {
        int v[8];
        const bool early = hint_ok && cb == lo && i0 == 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * kBatch + tid;
          v[u] = i < ce - cb ? (early ? v_h[u] : slot_row[cb + i]) : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * kBatch + tid;
          const bool ok = (uint32_t)v[u] < pool_lim;
          lane_bad |= (i < ce - cb) && !ok;
          if (i < ce - cb + kTile) rows_lds[i] = ok ? pool + (size_t)(uint32_t)v[u] * (kDk * 2) : zero_row;
        }
      }
      bad_slot |= lane_bad;
      // Drain every load the compiler issued (the query loads too): it cannot
      // see the gathers below, and with any of its own loads still pending it
      // puts vmcnt waits before the score MFMAs of every tile, which then also
      // wait for the gathers of the next tiles and undo the lookahead.
      wait_vmcnt<0>();
      // Row addresses visible to every wave, and whether any slot was invalid.
      // No gather is in flight here (the previous chunk ended with a full
      // drain), so the full barrier costs nothing.
      const bool chunk_bad = __syncthreads_or(lane_bad) != 0;
      const uint32_t kv_lds = lds_addr_of(kv);
      const uint32_t sink_lds = lds_addr_of(pf_sink);
      if constexpr (kGather) {
        gather_tile<NGW>(kv_lds, gw, gp, rows_lds, 0);
        if (cb + kTile < ce) gather_tile<NGW>(kv_lds + kBufElems * 2, gw, gp, rows_lds, kTile);
        // tiles 2 .. kPfAhead - 1 of the chunk, before the loop prefetches the rest
        if (pf_on) {
#pragma unroll
          for (int k = 2; k < kPfAhead; ++k)
            if (cb + k * kTile < ce) prefetch(sink_lds, k * kTile);
        }
      }
      int buf = 0;
      for (int t0 = cb; t0 < ce; t0 += kTile) {
        // Waiting for this wave's gathers of tile t0: the prefetches issued
        // after them only add to the loads still allowed in flight.
        if constexpr (kGather) {
          if (t0 + kTile < ce) wait_vmcnt<kWaitAhead>();
          else wait_vmcnt<0>();
        }
        lds_barrier();  // tile t0 is in LDS for every wave; the buffer of tile t0 - 32 is free
        if constexpr (kGather) {
          if (t0 + 2 * kTile < ce) {
            const int nb = buf == 0 ? kStages - 1 : buf - 1;
            gather_tile<NGW>(kv_lds + nb * kBufElems * 2, gw, gp, rows_lds, t0 + 2 * kTile - cb);
          }
          // (the staged rows of the chunk reach kTile entries past its end, so a
          // prefetched tile that starts inside the chunk stays in range)
          if (pf_on && t0 + kPfAhead * kTile < ce) prefetch(sink_lds, t0 + kPfAhead * kTile - cb);
        }
        if constexpr (kCompute) {
          compute_tile(kv + buf * kBufElems, t0, cb, ce, chunk_bad);
          ++seq;
        }
        buf = buf + 1 == kStages ? 0 : buf + 1;
      }
      lds_barrier();  // every wave is done with the tiles and the slot chunk
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  if constexpr (NG == 0) {
    main_loop(yes{}, yes{});
  } else {
    if (gather_only) {
      // (returning here keeps the pairs' query registers and accumulators
      // out of this path's live ranges)
      main_loop(yes{}, no{});
      if (bad_slot) flag_error(a.err, MLA_DEVERR_SLOT_RANGE);
      return;
    }
    main_loop(no{}, yes{});
  }
  if (bad_slot) flag_error(a.err, MLA_DEVERR_SLOT_RANGE);

  // ---- epilogue: normalise and store this split's result
  if (!active) return;
  const float lt = group4_sum(l);
  const float ltr = group4_sum(lr);
  const float inv = ltr > 0.f ? 1.f / ltr : 0.f;
  const float lse_v = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
  // the tile ring is free now: kStageHalves of it per wavefront stage the stores
  static_assert(NW * kStageHalves * 2 <= (int)sizeof(kv), "staging areas fit the tile ring");
  store_block_half(a, o, inv, lse_v, b, split, row0, min(16, R - row0), half, g, half == 0 && g == 0,
                   reinterpret_cast<_Float16*>(kv) + wave * kStageHalves);
}

template <int NB, bool kPf>
hipError_t launch_nb_pf(const Args& b, long units, hipStream_t stream) {
  if (b.balance_units > 0)
    hipLaunchKernelGGL((split_bf16_kernel<NB, true, kPf>), dim3(xcd_grid(units, b.xcd_chunk)), dim3(kThreads<NB>), 0, stream, b);
  else
    hipLaunchKernelGGL((split_bf16_kernel<NB, false, kPf>), dim3(xcd_grid(units, b.xcd_chunk)), dim3(kThreads<NB>), 0, stream, b);
  return hipGetLastError();
}

template <int NB>
hipError_t launch_nb(const Args& a, int row_groups, hipStream_t stream) {
  Args b = a;
  b.row_groups = row_groups;
  const long units = (long)(a.balance_units > 0 ? a.balance_units : a.batch * a.nsplit) * row_groups;
  return a.l2_prefetch ? launch_nb_pf<NB, true>(b, units, stream) : launch_nb_pf<NB, false>(b, units, stream);
}

}  // namespace

hipError_t launch_split_bf16(const Args& a, int blocks, int row_groups, hipStream_t stream) {
  switch (blocks) {
    case 1: return launch_nb<1>(a, row_groups, stream);
    case 2: return launch_nb<2>(a, row_groups, stream);
    case 3: return launch_nb<3>(a, row_groups, stream);
    case 4: return launch_nb<4>(a, row_groups, stream);
    case 5: return launch_nb<5>(a, row_groups, stream);
    case 6: return launch_nb<6>(a, row_groups, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mla
