// Internal interface between the C-ABI host layer (api.cpp) and the kernel
// translation units. Not installed; the public ABI is include/mla_verify.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kDk = 576;    // absorbed query / key width (512 latent ++ 64 rope)
constexpr int kDv = 512;    // value width: the latent part of the same row
constexpr int kDrope = 64;
// Splits of at least this many 32-position tiles take the bf16 split
// kernel's L2 prefetch (the plan picks the instantiation; the kernel checks
// each split's own length).
constexpr int kPfMinTiles = 24;

// Gather-only wavefronts of a bf16 split workgroup with `nb` 16-row blocks.
// They issue every gather and L2 prefetch (and read the row addresses from
// LDS) in place of the pairs, which then run no global-memory instruction
// in the tile loop. With an odd number of blocks the pairs leave SIMDs 2 and
// 3 one wavefront short of SIMDs 0 and 1 (wavefront w runs on SIMD w % 4),
// and a SIMD's LDS reads and MFMAs barely overlap, so two extra wavefronts
// land on SIMDs 2 and 3 and also even out the SIMDs. With 2 or 4 blocks four
// extra wavefronts take one SIMD each. With 6 blocks three pair halves per
// SIMD leave no registers for a fourth wavefront. MLA_GATHER_WAVES=0 (or
// MLA_GATHER_WAVES_EVEN=0 for the even counts) builds the kernel without
// them.
#ifndef MLA_GATHER_WAVES
#define MLA_GATHER_WAVES 1
#endif
#ifndef MLA_GATHER_WAVES_EVEN
#define MLA_GATHER_WAVES_EVEN 1
#endif
constexpr int bf16_gather_waves(int nb) {
  return !MLA_GATHER_WAVES ? 0 : nb % 2 == 1 ? 2 : (MLA_GATHER_WAVES_EVEN && (nb == 2 || nb == 4)) ? 4 : 0;
}

// Load-only wavefronts of an fp8 split workgroup: they stage the positions
// and slots, load each tile's fp8 rows, convert them to bf16 and write the
// LDS tile, one wavefront per SIMD, so the pairs only compute.
// MLA_FP8_LOAD_WAVES=0 builds the kernel with the pairs loading the tiles.
#ifndef MLA_FP8_LOAD_WAVES
#define MLA_FP8_LOAD_WAVES 4
#endif
constexpr int fp8_load_waves(int) { return MLA_FP8_LOAD_WAVES; }

// Everything a kernel needs, with pointers already validated by the host.
struct Args {
  const void* q;            // bf16 [batch, rows, 576]
  const void* latent;       // bf16 [pool, 576] or e4m3 [pool, 512]
  const void* rope;         // bf16 [pool, 64] (fp8 cache only)
  const float* kscale;      // fp32 [pool] (fp8 cache only)
  const int32_t* slots;     // [batch, slot_stride]
  const int32_t* seq_lens;  // [batch]
  const uint64_t* anc;      // [batch, q_len] (tree)
  const int32_t* topk_idx;  // [batch, q_len, topk] (sparse)
  float* out;               // [batch, rows, 512]
  float* lse;               // [batch, rows] or nullptr
  _Float16* part_o;         // [batch, nsplit, rows, 512] fp16, times part_scale per 256-column half
  float* part_lse;          // [batch, rows, nsplit]
  float* part_scale;        // [batch, rows, nsplit, 2] power-of-two multipliers of part_o
  int32_t* part_count;      // [batch] splits holding partials, written by the split kernel
                            // when the counts follow the lengths (balance_units > 0)
  unsigned* err;            // device error flag word
  const void* zero_row;     // >= 1152 zero bytes, read in place of masked / invalid cache rows
  int64_t pool_rows;
  int slot_stride;
  int len_hint;             // host-side bound of seq_lens (max_seq_len, else slot_stride): the
                            // split kernels start loading the slots of the split this implies
                            // before the true length arrives, and keep them if it matches
  int batch, q_len, heads, rows;  // rows = q_len * heads
  int nsplit;               // splits per sequence; with balance_units, their upper bound and
                            // the partials' stride
  int balance_units;        // > 0: per-sequence split counts follow the lengths
                            // (balanced_split), with at most this many splits in all
  int row_groups;           // workgroups along the row axis (set at launch)
  int xcd_chunk;            // work units per XCD (grid = 8 * xcd_chunk, at least ceil(units / 8)):
                            // a multiple of row_groups when that still gives every XCD no more
                            // workgroups than CUs, so all row groups of a split share one L2
  int l2_prefetch;          // bf16 split kernel: pull cache lines into L2 a few tiles ahead of
                            // the gathers (long splits only; set by the plan)
  int mask_kind;
  int topk;
  float scale_log2;         // sm_scale * log2(e)
};

// Split kernels. `blocks` = 16-row query blocks per workgroup (two wavefronts
// each), `row_groups` = workgroups along the row axis. Grid = nsplit *
// row_groups * batch.
hipError_t launch_split_bf16(const Args& a, int blocks, int row_groups, hipStream_t stream);
hipError_t launch_split_fp8_topk(const Args& a, int blocks, int row_groups, hipStream_t stream);
// Log-sum-exp merge of the partials into out / lse.
hipError_t launch_combine(const Args& a, hipStream_t stream);
// Draft-KV append: row i of sequence b of new_rows (bf16 [batch, q_len, 576])
// to pool row slots[b, seq_lens[b] - q_len + i].
hipError_t launch_append(void* latent, int64_t pool_rows, int slot_stride, const void* new_rows, int batch,
                         int q_len, const int32_t* slots, const int32_t* seq_lens, unsigned* err,
                         hipStream_t stream);
// Top-k selection: per (sequence, query) row of scores, the topk best
// positions below seq_lens[b], in ascending order.
hipError_t launch_topk(const float* scores, int batch, int q_len, int score_stride, const int32_t* seq_lens,
                       int topk, int32_t* out, unsigned* err, void* workspace, hipStream_t stream);
size_t topk_workspace_bytes(int rows, int score_stride);
// Weight absorption around the attention (per-head widths 128 / 128).
hipError_t launch_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int tokens, int heads,
                           void* q_out, hipStream_t stream);
hipError_t launch_project_o(const float* o_latent, const void* w_uv, int tokens, int heads, float* o_out,
                            hipStream_t stream);
// Ancestor-or-self masks from parent arrays.
hipError_t launch_tree_mask(const int32_t* parents, int batch, int q_len, uint64_t* anc, unsigned* err,
                            hipStream_t stream);

}  // namespace mla
