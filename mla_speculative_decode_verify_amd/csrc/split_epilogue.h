// Epilogue shared by the split kernels: one wavefront's half of a finished
// 16-row block goes either to the final output (single split) or to the
// split-partial workspace.
//
// Partials are stored compactly: the normalised output O_s of each (split,
// row) as fp16, with one power-of-two multiplier per 256-column half chosen
// so the half's largest magnitude lands in [2^14, 2^15). The stored values
// therefore never overflow fp16 and keep its full 11-bit precision whatever
// the cache's value range (a relative error of at most 2^-12 per element,
// well below the bf16 rounding of the weights), at half the bytes of fp32.
// The LSE stays fp32.
#pragma once

#include "device_common.h"
#include "mla_internal.h"

namespace mla {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Staging rows are padded by 16 halves (32 bytes): with a bare 512-byte
// stride the 16 rows of one 8-byte write instruction all hit the same LDS
// banks (a 16-way conflict on every staging write); with a stride of 136
// words each group of rows covers every bank once.
constexpr int kStageRow = 256 + 16;              // halves per staged row
constexpr int kStageHalves = 16 * kStageRow;     // one wavefront's staging area (8.5 KiB)

// Lane (g, li) holds o[d][r] (d < 16) = unnormalised output column
// 256 half + 16 d + 4 g + r of block row li; `inv` normalises it.
// All 64 lanes must call this (it reduces across lanes). The block's rows
// are r_first .. r_first + n_valid - 1 within the sequence (n_valid <= 16),
// so lane li's row exists iff li < n_valid.
// `stage` is kStageHalves halves of LDS owned by this wavefront alone (free
// after the tile loop): fp16 partials are transposed through it so that
// every store instruction writes two whole 512-byte row halves instead of
// 32-byte pieces of 16 rows.
__device__ __forceinline__ void store_block_half(const Args& a, const f32x4* o, float inv, float lse_v,
                                                 int b, int split, int r_first, int n_valid, int half, int g,
                                                 bool write_lse, _Float16* stage) {
  constexpr int kBlocks = kDv / 32;  // 16 column blocks of 16 per half
  const int S = a.nsplit, R = a.rows;
  const int lane = (int)__lane_id(), li = lane & 15;
  const bool row_ok = li < n_valid;
  const int r_out = r_first + li;
  if (S == 1) {
    if (!row_ok) return;
    float* dst = a.out + ((size_t)b * R + r_out) * kDv + 256 * half + 4 * g;
#pragma unroll
    for (int d = 0; d < kBlocks; ++d) *reinterpret_cast<f32x4*>(dst + 16 * d) = o[d] * inv;
    if (write_lse && a.lse) a.lse[(size_t)b * R + r_out] = lse_v;
    return;
  }
  float mx = 0.f;
#pragma unroll
  for (int d = 0; d < kBlocks; ++d)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(o[d][r] * inv));
  mx = group4_max(mx);
  // exponent of the half's largest magnitude (NaN / inf propagate unchanged)
  const int ex = (int)((__float_as_uint(mx) >> 23) & 0xFF) - 127;
  const int e = min(max(ex - 14, -126), 113);
  const float down = __builtin_amdgcn_ldexpf(inv, -e);
  // stage[row li][256 columns (row stride kStageRow)] in fp16, then 16-byte pieces row-major
#pragma unroll
  for (int d = 0; d < kBlocks; ++d) {
    const f32x4 v = o[d] * down;
    *reinterpret_cast<f16x4*>(stage + li * kStageRow + 16 * d + 4 * g) = __builtin_convertvector(v, f16x4);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = lane + 64 * i;       // 16-byte piece: row q / 32, column piece q % 32
    const int rr = q >> 5, cp = q & 31;
    const f32x4 piece = *reinterpret_cast<const f32x4*>(stage + rr * kStageRow + 8 * cp);
    if (rr < n_valid) {
      const size_t pr = ((size_t)b * S + split) * R + r_first + rr;
      // streaming store: the partials are read once, by the merge kernel
      __builtin_nontemporal_store(piece, reinterpret_cast<f32x4*>(a.part_o + pr * kDv + 256 * half + 8 * cp));
    }
  }
  __builtin_amdgcn_wave_barrier();  // the stage is reused by the next call
  if (!row_ok) return;
  const size_t pl = ((size_t)b * R + r_out) * S + split;  // LSE / scale: splits contiguous per row
  if (g == 0) a.part_scale[pl * 2 + half] = __builtin_amdgcn_ldexpf(1.f, e);
  if (write_lse) a.part_lse[pl] = lse_v;
}

}  // namespace mla
