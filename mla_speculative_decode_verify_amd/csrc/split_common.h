// Tile geometry and gather machinery of the bf16 split kernel
// (split_bf16.hip). A tile is 32 cache positions whose
// 576-element bf16 rows are gathered through the page_size = 1 slot table
// straight into a padded LDS buffer, 16 bytes per lane, by
// global_load_lds_dwordx4 ("How a CUDA Kernel Designer Discovered That GPU
// Utilization Trumps Memory Bandwidth", section "Context: The Problem and
// the Stakes": scattered single-token pages are the path's central cost;
// section "Potential Mistakes": 128-bit loads need 16-byte alignment).
#pragma once

#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace tile {

constexpr int kTile = 32;                          // cache positions per tile (2 MFMA key blocks)
constexpr int kPieces = kDk / 8;                   // 16-byte pieces per latent row (72)
constexpr int kRowPieces = kPieces + 2;            // 16-byte pad pieces per LDS row spread the banks
constexpr int kLdsStride = kRowPieces * 8;         // bf16 elements per LDS row (1184 bytes)
constexpr int kTilePieces = kTile * kRowPieces;    // 2368
constexpr int kSegments = (kTilePieces + 63) / 64; // 64-piece wave loads per tile (37)
constexpr int kBufElems = kSegments * 64 * 8;      // one tile buffer incl. the tail segment
constexpr int kStages = 3;                         // LDS tile buffers (two tiles in flight)
constexpr float kRescaleSlack = 8.f;               // lazy online-softmax rescale threshold (log2 units)
// Tiles ahead of the one being consumed whose cache lines are pulled into
// L2 by one 4-byte load per 128-byte line. The LDS ring only holds the tile
// in use and two in flight, so the gathers alone would wait on HBM latency;
// with the lines already in L2 they wait on L2.
constexpr int kPfAhead = 4;
// Splits shorter than this many positions skip the prefetch: every split
// starts at once, so their first tiles already arrive in one burst that
// saturates HBM, and extra requests only delay them (measured: 9-tile
// splits slower by 3 us, 100-tile splits of random slots faster by 25%).
constexpr int kPfMinKeys = kPfMinTiles * kTile;
constexpr int kRowLines = kDk * 2 / 128;                  // 128-byte lines per cache row (9)
constexpr int kPfOps = (kTile * kRowLines + 63) / 64;     // wave loads per prefetched tile (5)

// Per-lane geometry of one wave's share of a tile gather. Piece p of the
// padded tile is row p / kRowPieces, column piece p % kRowPieces; each wave
// instruction moves 64 consecutive pieces (1 KiB) from 64 independent 16-byte
// addresses. Computed once per kernel, per piece, as (byte offset of the
// piece in its cache row << 16) | (8 * tile row): the tile row indexes the
// staged row addresses. Pieces past the tile (the tail of the last segment
// lands in the buffer's padding, never read) use row kTile, an in-bounds
// staged entry, so no lane needs a test.
template <int NW>
struct GatherPlan {
  static constexpr int kPer = (kSegments + NW - 1) / NW;
  uint32_t packed[kPer];
  __device__ __forceinline__ GatherPlan(int wave, int lane) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int sg = wave + k * NW;
      const int p = sg * 64 + lane;
      const bool live = sg < kSegments && p < kTilePieces;
      const int row = live ? p / kRowPieces : kTile;
      const int col = live ? min(p - row * kRowPieces, kPieces - 1) : 0;
      packed[k] = ((uint32_t)(16 * col) << 16) | (uint32_t)(8 * row);
    }
  }
};

// Issue this wave's share of one tile's gather straight into LDS. rows_lds
// holds, for every position of the staged chunk and for 32 entries past its
// end, the byte address of the cache row to read: the pool row of its slot,
// or the zero row for positions past the split or with an invalid slot. So
// a tile never holds stale or poisoned data, and a piece costs one LDS read
// and one 64-bit add. `lds_base` and `wave` are wave-uniform (scalar).
// All of the wave's row-address reads are issued before the first load: each
// load is an asm statement that clobbers memory, so a read placed after one
// could not be moved ahead of it and every piece would wait out its own LDS
// round trip.
template <int NW>
__device__ __forceinline__ void gather_tile(uint32_t lds_base, int wave, const GatherPlan<NW>& gp,
                                            const char* const* rows_lds, int t_rel) {
  constexpr int kPer = GatherPlan<NW>::kPer;
  const char* const* rows = rows_lds + t_rel;
  // Piece k exists for every wave when (k + 1) * NW <= kSegments (wave <
  // NW), a compile-time fact; only the last one needs the run-time test.
  // With a test (a branch) between two pieces, the compiler consumes each
  // address read before the next one and every piece waits on LDS alone.
  auto live = [&](int k) { return (k + 1) * NW <= kSegments || wave + k * NW < kSegments; };
  uint32_t v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    v[k] = gp.packed[k];
    // Opaque per tile, so the compiler recomputes the source address instead
    // of holding one 64-bit address per piece across the tile loop.
    asm volatile("" : "+v"(v[k]));
  }
  // (pieces past the tile point at an in-bounds staged entry, so reading the
  // address of a piece that is not issued is harmless)
  const char* src[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    src[k] = *reinterpret_cast<const char* const*>(reinterpret_cast<const char*>(rows) + (v[k] & 0xFFFFu)) +
             (v[k] >> 16);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (!live(k)) continue;  // wave-uniform
    lds_dma_b128(src[k], lds_base + (wave + k * NW) * 1024);
  }
}

// Pull the cache lines of the staged tile at t_rel into L2: wave loads
// ("ops") 0 .. kPfOps - 1 each touch 64 of its 32 x 9 lines with one 4-byte
// load per lane (the last op's spare lanes repeat the final line). Rows
// staged as the zero row touch that row. `op` is wave-uniform; `plan` is the
// lane's (line byte offset << 16) | (8 * tile row) for that op, from
// prefetch_plan.
__device__ __forceinline__ uint32_t prefetch_plan(int op, int lane) {
  const int idx = min(op * 64 + lane, kTile * kRowLines - 1);
  const int r = idx / kRowLines, line = idx - r * kRowLines;
  return ((uint32_t)(128 * line) << 16) | (uint32_t)(8 * r);
}
__device__ __forceinline__ void prefetch_tile(uint32_t sink_lds, int op, uint32_t plan,
                                              const char* const* rows_lds, int t_rel) {
  if (op >= kPfOps) return;
  asm volatile("" : "+v"(plan));  // recomputed per use rather than held as a 64-bit address
  const char* row =
      *reinterpret_cast<const char* const*>(reinterpret_cast<const char*>(rows_lds + t_rel) + (plan & 0xFFFFu));
  lds_dma_b32(row + (plan >> 16), sink_lds + op * 256);
}

// Positions [lo, hi) of split `split` of S over n positions: the ceil(n / 32)
// tiles are dealt out as evenly as possible, the extra ones to the last
// splits (which also hold the sequence's final, possibly partial tile), so
// no split pays a full tile for a few leftover positions and the splits
// that finish first are the many with fewer tiles.
__device__ __forceinline__ void split_range(int n, int S, int split, int& lo, int& hi) {
  const int tiles = (n + kTile - 1) / kTile;
  const int base = tiles / S, first_big = S - (tiles - base * S);
  const int t0 = split * base + max(0, split - first_big);
  const int nt = base + (split >= first_big ? 1 : 0);
  lo = min(n, t0 * kTile);
  hi = min(n, (t0 + nt) * kTile);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// V operand of the 16x16x32 MFMA for output columns [16 d, 16 d + 16): keys
// 4g..4g+3 and 16+4g..16+4g+3 in k-slots 0..7 (matching the P operand).
__device__ __forceinline__ bf16x8 v_operand(const __bf16* vT0, int d) {
  const bf16x4 lo4 = lds_read_tr16(vT0 + 16 * d);
  const bf16x4 hi4 = lds_read_tr16(vT0 + 16 * d + 16 * kLdsStride);
  return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace tile
}  // namespace mla
