/*
 * mla_verify.h - C ABI of libmla_verify.so: absorbed-MLA verify / sparse-decode
 * attention for speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * What it computes. A block of q_len draft-token queries per sequence, H heads
 * each, every query a 576-element absorbed vector (512 latent + 64 rope),
 * attends over the sequence's latent KV cache: one 576-element row per cached
 * token, shared by all heads, whose first 512 elements are also the value.
 * ("How a CUDA Kernel Designer Discovered That GPU Utilization Trumps Memory
 * Bandwidth": sections "Context: The Problem and the Stakes" for verify
 * attention and "The Warp-Per-Key Dot Product" for the 576-element score;
 * "The Occupancy Probe", section "The Scene", for the 512-wide latent
 * accumulator and the fp8 sparse decode.) For sequence b, query i, head h:
 *
 *   s_j   = sm_scale * <q[b,i,h,0:576], k_j[0:576]>      for visible j
 *   lse   = ln sum_j exp(s_j)                           (natural log)
 *   out[c]= sum_j exp(s_j - lse) * k_j[c]               for c < 512
 *
 * Visible positions (N = seq_lens[b]):
 *   MLA_MASK_NONE   all N positions.
 *   MLA_MASK_CAUSAL prefix P = N - q_len positions, plus drafts 0..i
 *                   (draft d sits at position P + d).
 *   MLA_MASK_TREE   prefix, plus draft d iff bit d of tree_anc[b,i] is set
 *                   (ancestor-or-self mask, built by mla_build_tree_mask).
 *   MLA_MASK_TOPK   exactly the positions topk_idx[b,i,0:topk] (prefix
 *                   positions, distinct), fp8 cache only.
 * An empty visible set yields out = 0 and lse = -inf.
 *
 * The KV axis of each sequence is cut into nsplit contiguous chunks of
 * ceil(N / nsplit) positions ("How One Environment Variable Unlocked 3x
 * Throughput", section "The Occupancy Revelation": the split count NSPLIT
 * multiplies the grid); the bf16 kernel instead deals the ceil(N / 32)
 * 32-position tiles out as evenly as possible, the extra ones to the last
 * chunks (leading chunks are empty when nsplit exceeds the tile count). Each chunk
 * produces a normalised partial output and
 * its LSE, and a second kernel merges them by log-sum-exp weights. The merge
 * is exact in real arithmetic, so results do not depend on nsplit beyond
 * floating-point rounding.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller (e.g. torch
 *    tensors). The library never copies them, never frees them and never
 *    keeps them after the call returns.
 *  - Tensors are dense and row-major in the shapes given below.
 *  - 16-byte alignment is required for q, the cache arrays and out (the
 *    kernels use 16-byte vector loads and stores); 8 bytes for tree_anc;
 *    4 bytes for the int32 arrays, lse and scale. Misalignment returns
 *    MLA_ERR_ALIGN.
 *  - Work is enqueued on `stream` and the call returns without waiting. All
 *    argument checks happen on the host before any HIP call, so a bad
 *    argument never launches anything.
 *  - Errors are returned as negative MLA_ERR_* codes; nothing throws across
 *    the ABI. Conditions only the GPU can see (a slot outside the pool, a
 *    seq_len outside [q_len, slot_stride], a bad tree parent) set a sticky
 *    per-device flag read by mla_get_device_error(); the offending key is
 *    treated as masked and the kernels never read outside the pool.
 */
#ifndef MLA_VERIFY_H
#define MLA_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_VERIFY_ABI_VERSION 4

/* Status codes. */
#define MLA_OK 0
#define MLA_ERR_INVALID_ARG (-1)  /* null pointer, bad size, bad enum, bad parent */
#define MLA_ERR_ALIGN (-2)        /* pointer not aligned as required */
#define MLA_ERR_UNSUPPORTED (-3)  /* shape or combination outside what the kernels cover */
#define MLA_ERR_WORKSPACE (-4)    /* workspace must grow while the stream is being captured */
#define MLA_ERR_LAUNCH (-5)       /* a HIP call or kernel launch failed */
#define MLA_ERR_SCRATCH (-6)      /* mla_verify_attn_noalloc: partials exceed its static scratch */

/* Device-side error flag bits (mla_get_device_error). */
#define MLA_DEVERR_SLOT_RANGE 0x1u   /* slot_table entry outside [0, pool_rows) */
#define MLA_DEVERR_SEQ_LEN 0x2u      /* seq_len < q_len (masked kinds) or > slot_stride */
#define MLA_DEVERR_TREE_PARENT 0x4u  /* parent outside [-1, i-1] in mla_build_tree_mask */
#define MLA_DEVERR_TOPK_RANGE 0x8u   /* top-k position outside [0, seq_len) */
#define MLA_DEVERR_SYNC 0x10u        /* a wait between the wavefronts of a workgroup exceeded
                                        its bound (a library fault: the call's results are
                                        invalid; raised instead of hanging the GPU) */

/* Cache element types. */
#define MLA_KV_BF16 0      /* latent: bf16 [pool_rows, 576] (512 latent ++ 64 rope) */
#define MLA_KV_FP8_E4M3 1  /* latent: OCP E4M3FN [pool_rows, 512]; rope: bf16 [pool_rows, 64];
                              scale: fp32 [pool_rows] multiplying the latent part */

/* Mask kinds (see the header comment for the visible sets). */
#define MLA_MASK_NONE 0
#define MLA_MASK_CAUSAL 1
#define MLA_MASK_TREE 2
#define MLA_MASK_TOPK 3

/* Limits. */
#define MLA_MAX_Q_LEN 64     /* draft masks are 64-bit */
#define MLA_MAX_HEADS 128
#define MLA_MAX_NSPLIT 1024
#define MLA_MAX_TOPK 65536
/* Static scratch of mla_verify_attn_noalloc per device (32 MiB). */
#define MLA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Queries: bf16 [batch, q_len, heads, 576], absorbed (512 latent ++ 64 rope). */
typedef struct mla_q_t {
  const void* data;
  int batch;
  int q_len;
  int heads;
  float sm_scale; /* multiplies the full 576-element dot product; > 0 and finite */
} mla_q_t;

/* Latent KV cache with page_size = 1: one pool row per cached token. */
typedef struct mla_kv_t {
  int dtype;            /* MLA_KV_BF16 or MLA_KV_FP8_E4M3 */
  const void* latent;   /* see MLA_KV_* */
  const void* rope;     /* NULL for bf16; bf16 [pool_rows, 64] for fp8 */
  const float* scale;   /* NULL for bf16; fp32 [pool_rows] for fp8 */
  int64_t pool_rows;    /* number of rows in the pool */
  int slot_stride;      /* row length of slot_table (max tokens per sequence) */
  int max_seq_len;      /* host-side upper bound of seq_lens used to size the
                           split grid; 0 means slot_stride */
} mla_kv_t;

typedef struct mla_mask_t {
  int kind;                  /* MLA_MASK_* */
  const uint64_t* tree_anc;  /* MLA_MASK_TREE: device uint64 [batch, q_len] */
  const int32_t* topk_idx;   /* MLA_MASK_TOPK: device int32 [batch, q_len, topk] */
  int topk;                  /* MLA_MASK_TOPK: entries per (sequence, query) */
} mla_mask_t;

/* Plan of one call, as chosen by the library (for tests and measurement). */
typedef struct mla_plan_t {
  int nsplit;            /* KV splits per sequence actually used */
  int waves_per_group;   /* wavefronts per workgroup: two per 16-row query block,
                            plus the bf16 kernel's gather-only ones (two with
                            1, 3 or 5 blocks, four with 2 or 4) */
  int row_groups;        /* workgroups along the query-row axis per split */
  int grid;              /* split-kernel workgroups with work (the launch adds
                            idle ones up to a multiple of 8, and up to whole
                            splits per XCD when that still fits the CUs) */
  size_t workspace_bytes;/* partial storage needed (0 when nsplit == 1) */
  int kernel;            /* 0 = bf16 verify, 1 = fp8 top-k sparse */
  int row_blocks;        /* 16-row query blocks per workgroup */
  int balanced;          /* 1: split counts follow the sequence lengths (see
                            mla_verify_attn); nsplit is then their upper bound */
  int l2_prefetch;       /* 1: the bf16 split kernel pulls cache lines into L2
                            four tiles ahead of its gathers (splits of at
                            least 24 tiles of 32 positions) */
} mla_plan_t;

/*
 * Verify / sparse-decode attention.
 *   slot_table: int32 [batch, slot_stride]; position j of sequence b lives in
 *               pool row slot_table[b, j] (page_size = 1).
 *   seq_lens:   int32 [batch]; N_b. For CAUSAL/TREE this counts the prefix
 *               plus the q_len drafts, whose rows are already in the cache
 *               at positions N_b - q_len .. N_b - 1. For TOPK it is the
 *               prefix length bounding the top-k positions.
 *   out:        fp32 [batch, q_len, heads, 512].
 *   lse:        fp32 [batch, q_len, heads] or NULL.
 *   nsplit:     KV splits per sequence; <= 0 lets the library choose
 *               from the CU count: one count for every sequence
 *               (mla_choose_nsplit) when batch == 1, an fp8 cache or
 *               batch > 64; otherwise (bf16 cache, 2..64 sequences) counts
 *               that follow each sequence's length, derived on the device
 *               from seq_lens, so that every split holds about the same
 *               number of 32-position tiles and the grid (one workgroup per
 *               CU at most) is not held up by the longest sequence. A
 *               sequence of t tiles then gets ceil(t / T) splits, at most
 *               ceil(t / 4) and at least 1, for the smallest T that keeps
 *               the total within the grid. Capped at MLA_MAX_NSPLIT.
 * When nsplit > 1 the call keeps its split partials in the library's
 * workspace for (device, stream): it grows on demand (synchronising `stream`
 * first), or returns MLA_ERR_WORKSPACE if the stream is capturing and the
 * reserve is too small. Calls on the same stream are ordered; calls on
 * different streams have separate workspaces. A graph captured on a stream
 * keeps using that stream's workspace when it is replayed, whatever stream
 * it is replayed on: the caller must order replays against eager calls made
 * on the capture stream (e.g. replay on that stream), or they race on the
 * partials. See mla_reserve_workspace / mla_release_workspace.
 */
int mla_verify_attn(const mla_q_t* q, const mla_kv_t* kv_cache, const int32_t* slot_table,
                    const int32_t* seq_lens, const mla_mask_t* mask_desc, float* out, float* lse,
                    int nsplit, hipStream_t stream);

/* The two halves of mla_verify_attn with identical arguments: the split
 * kernel alone (writes partials to the workspace, or out/lse directly when
 * the plan has nsplit == 1), then the merge alone (no-op when nsplit == 1).
 * Calling mla_verify_split then mla_verify_combine on one stream equals one
 * mla_verify_attn. Exposed so a caller can time or schedule the kernels
 * separately. */
int mla_verify_split(const mla_q_t* q, const mla_kv_t* kv_cache, const int32_t* slot_table,
                     const int32_t* seq_lens, const mla_mask_t* mask_desc, float* out, float* lse,
                     int nsplit, hipStream_t stream);
int mla_verify_combine(const mla_q_t* q, const mla_kv_t* kv_cache, const int32_t* slot_table,
                       const int32_t* seq_lens, const mla_mask_t* mask_desc, float* out, float* lse,
                       int nsplit, hipStream_t stream);

/* Fill *plan for a call with these arguments (host only, no HIP call except
 * reading the current device's CU count once). Returns a status code. */
int mla_plan(const mla_q_t* q, const mla_kv_t* kv_cache, const mla_mask_t* mask_desc, int nsplit,
             mla_plan_t* plan);

/* Split count the library picks when nsplit <= 0 (one count for every
 * sequence): a pure function of the shape and the CU count, so it is
 * deterministic and safe under graph capture. At most one split-kernel
 * workgroup per CU. For a bf16 cache the library picks the query rows per
 * workgroup (up to six 16-row blocks; more rows are dealt to several
 * workgroups of two to six blocks that gather the same keys) together with
 * the count s, by a cost model fitted to cold-cache calls on MI355X: per
 * 32-position tile of the slowest split about 1.21, 1.52, 1.60, 1.86 and
 * 2.21 us with two, three, four, five and six blocks per workgroup (1.86 us
 * with one), 7.2 to 8.1 us fixed (11.4 us with six blocks), and, when
 * s > 1, 4 us for the merge plus 0.49 us per MB of partials (1036 bytes per
 * split and query row, written and read back); the cheapest wins, the
 * fewest splits on ties. A single sequence whose rows fill exactly five blocks (e.g. 8 heads,
 * q_len 9) may instead be dealt to two groups of three blocks or three of
 * two, chosen with the count by split + merge times fitted per layout (the
 * smaller groups win below about 32k positions: fewer wavefronts per SIMD
 * make a tile cheaper, fewer splits make fewer partials). mla_plan reports
 * the layout taken. For an fp8 cache, as many as fit, with at least 128 list entries
 * per split. max_seq_len is the longest sequence for a bf16 cache and the
 * top-k list length for an fp8 cache (each query's list is split). ("How
 * One Environment Variable Unlocked 3x Throughput", section "The Occupancy
 * Revelation": a small per-rank head count shrinks the grid until the
 * machine starves, and more splits refill it.) */
int mla_choose_nsplit(int batch, int q_len, int heads, int max_seq_len, int kv_dtype, int num_cus);

/* Bytes of split partials one call needs: batch * nsplit * q_len * heads *
 * (512 * 2 + 12) (fp16 partial output, its two power-of-two scales and the
 * fp32 LSE per split and row) plus batch * 4 (each sequence's split count
 * when the counts follow the lengths), or 0 for nsplit <= 1. For a ragged
 * batch whose split counts follow the lengths, nsplit here must be the
 * partials' stride, which can exceed mla_choose_nsplit's uniform count:
 * the size to reserve for a given call is mla_plan(...).workspace_bytes.
 * ("How One Environment Variable Unlocked 3x Throughput", section "The
 * Occupancy Revelation": the partial buffers grow with NSPLIT and are
 * sized ahead of graph capture; section "Assumptions Underlying the
 * Reasoning", item 5: the kernel runs inside captured graphs and must not
 * allocate there.) */
size_t mla_workspace_bytes(int batch, int q_len, int heads, int nsplit);

/* Make the workspace of (current device, stream) at least `bytes` long
 * (take mla_plan(...).workspace_bytes of the largest call to be captured),
 * so later calls on `stream`, e.g. under graph capture, do not allocate.
 * Same passages as mla_workspace_bytes. A workspace that a call made under
 * capture has used is never freed implicitly: if a later eager call on the
 * stream needs more, the library allocates a larger buffer and parks the
 * old one (graphs keep replaying with it) until mla_release_workspace. A
 * buffer no captured call has used is freed on growth, after synchronising
 * `stream`. Returns a status code. */
int mla_reserve_workspace(size_t bytes, hipStream_t stream);

/* Free the workspace of (current device, stream) and every buffer parked
 * for it, after synchronising `stream`. Call it when no graph captured on
 * `stream` will be replayed again (e.g. before destroying the stream); the
 * next call on `stream` allocates afresh. Returns a status code. */
int mla_release_workspace(hipStream_t stream);

/* No-allocation variant of mla_verify_attn, for callers that cannot call
 * hipMalloc: code under graph capture with no reserve made, tight serving
 * loops, harnesses that forbid allocation. Same arguments, same plan, same
 * kernels and bitwise the same results as mla_verify_attn, but the split
 * partials live in a static device array of MLA_NOALLOC_SCRATCH_BYTES that
 * every device the library runs on holds from its first use until the
 * process ends. Returns MLA_ERR_SCRATCH, launching nothing, when the plan's
 * workspace_bytes exceed it (e.g. batch 8 x 64 heads x 40 splits); a
 * smaller nsplit can bring a call under the limit. The call allocates
 * nothing; the scratch keeps the last call's contents (nothing in it needs
 * clearing: every call writes the partials it reads). All calls of this
 * entry point on one device share the one array: calls that overlap on a
 * device (different streams, or graphs replayed concurrently) race and
 * give wrong results; order them on one stream. */
int mla_verify_attn_noalloc(const mla_q_t* q, const mla_kv_t* kv_cache, const int32_t* slot_table,
                            const int32_t* seq_lens, const mla_mask_t* mask_desc, float* out, float* lse,
                            int nsplit, hipStream_t stream);

/* Draft tree -> ancestor-or-self masks. parents: int32 [batch, q_len] with
 * parents[b,i] in [-1, i-1] (-1 = child of the prefix tail). Bit d of
 * anc_out[b,i] is set iff draft d is node i or one of its ancestors.
 * ("How One Environment Variable Unlocked 3x Throughput", sections "The
 * Broader Context" and "Input Knowledge Required": the draft tree is built
 * per step and turned into the verify mask.)
 * Device variant: pointers are device memory, enqueued on `stream`; a bad
 * parent sets MLA_DEVERR_TREE_PARENT and yields mask 1<<i for that node.
 * Host variant: pointers are host memory; a bad parent returns
 * MLA_ERR_INVALID_ARG. q_len must be in [1, 64]. */
int mla_build_tree_mask(const int32_t* parents, int batch, int q_len, uint64_t* anc_out,
                        hipStream_t stream);
int mla_build_tree_mask_host(const int32_t* parents, int batch, int q_len, uint64_t* anc_out);

/* Draft-KV append: write the q_len new tokens of every sequence into a bf16
 * latent pool (page_size = 1) before a verify call. Row i of sequence b,
 * new_rows[b, i, :] (bf16 [batch, q_len, 576], contiguous), goes to pool row
 * slot_table[b, seq_lens[b] - q_len + i], i.e. the draft positions that
 * mla_verify_attn reads. ("How One Environment Variable Unlocked 3x
 * Throughput", sections "The Central Dilemma" and "Potential Mistakes":
 * each request's KV lives in pool slots handed out by the allocator, and
 * whether they are contiguous decides how the gather behaves.)
 *   latent:     device bf16 [pool_rows, 576], written in place (16-byte
 *               aligned, like new_rows).
 *   slot_table: device int32 [batch, slot_stride]; seq_lens: device int32
 *               [batch] with q_len <= seq_lens[b] <= slot_stride.
 * The target slots must be distinct (two writes to one pool row race).
 * A sequence with an out-of-range length writes nothing and sets
 * MLA_DEVERR_SEQ_LEN; a row whose slot is outside [0, pool_rows) is skipped
 * and sets MLA_DEVERR_SLOT_RANGE. Enqueued on `stream`; allocates
 * nothing. q_len must be in [1, 64]. */
int mla_append_kv(void* latent, int64_t pool_rows, int slot_stride, const void* new_rows, int batch, int q_len,
                  const int32_t* slot_table, const int32_t* seq_lens, hipStream_t stream);

/* Top-k selection feeding the sparse decode: for each (sequence b, query i)
 * row of scores, the topk positions p < seq_lens[b] with the largest
 * scores[b, i, p], written to topk_idx[b, i, 0..topk) in ascending position
 * order. Ties go to the lower position, so the result is unique. Scores
 * compare as floats with -0.0 below +0.0 and NaN below every number.
 * ("The Occupancy Probe: A Methodical Approach to GPU Kernel
 * Optimization", sections "The Thinking Process: Risk Assessment and
 * Safety" and "Assumptions and Potential Pitfalls": a sparse indexer kernel
 * picks the top-k positions each query of the sparse decode attends to; the
 * pages give no scoring formula, so the scores are an input here.)
 *   scores:   device fp32 [batch, q_len, score_stride], 16-byte aligned,
 *             score_stride a multiple of 4 (else MLA_ERR_ALIGN) and at
 *             most 2^20, with batch * q_len at most 65535 (else
 *             MLA_ERR_UNSUPPORTED).
 *   seq_lens: device int32 [batch]: positions [0, seq_lens[b]) are eligible.
 *   topk_idx: device int32 [batch, q_len, topk], written.
 * A row with seq_lens[b] < topk (or outside [0, score_stride]) sets
 * MLA_DEVERR_SEQ_LEN and gets its positions 0 .. n-1 followed by -1.
 * Enqueued on `stream` (four kernels, each row cut into parts of 8192
 * positions); uses the library's workspace for (device, stream) like
 * mla_verify_attn, mla_topk_workspace_bytes(batch, q_len, score_stride)
 * bytes (reserve it with mla_reserve_workspace before graph capture). */
int mla_topk_select(const float* scores, int batch, int q_len, int score_stride, const int32_t* seq_lens,
                    int topk, int32_t* topk_idx, hipStream_t stream);
size_t mla_topk_workspace_bytes(int batch, int q_len, int score_stride);

/* Weight absorption around the attention, as bf16 MFMA GEMMs with fp32
 * accumulation. ("How a CUDA Kernel Designer Discovered That GPU Utilization
 * Trumps Memory Bandwidth", section "The Warp-Per-Key Dot Product": scores
 * are 576-element dot products; "The Occupancy Probe", section "The Scene":
 * the latent accumulator is 512 wide per head.) The pages fix only the
 * 576 / 512 widths;
 * the per-head widths here, 128 for q_nope and 128 for the value, are the
 * common MLA configuration (an assumption). tokens = rows of the call
 * (batch * q_len); every pointer is device memory, 16-byte aligned.
 *
 * mla_absorb_q: q_out[t, h, 0:512] = q_nope[t, h, :] . W_UK[h] (rounded to
 *   bf16) and q_out[t, h, 512:576] = q_rope[t, h, :], i.e. the absorbed
 *   query mla_verify_attn takes.
 *     q_nope bf16 [tokens, heads, 128]; q_rope bf16 [tokens, heads, 64];
 *     w_uk bf16 [heads, 512, 128] (W_UK[h] transposed: row c holds the 128
 *     weights of latent column c); q_out bf16 [tokens, heads, 576].
 * mla_project_o: o_out[t, h, :] = o_latent[t, h, :] . W_UV[h], with o_latent
 *   rounded to bf16 on the way in.
 *     o_latent fp32 [tokens, heads, 512] (mla_verify_attn's out);
 *     w_uv bf16 [heads, 128, 512] (W_UV[h] transposed: row c holds the 512
 *     weights of value column c); o_out fp32 [tokens, heads, 128].
 * Enqueued on `stream`; nothing is allocated. */
int mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int tokens, int heads, void* q_out,
                 hipStream_t stream);
int mla_project_o(const float* o_latent, const void* w_uv, int tokens, int heads, float* o_out,
                  hipStream_t stream);

/* Read (and optionally clear) the current device's sticky error flags.
 * Synchronises the device. Returns the MLA_DEVERR_* bits, or a negative
 * status code. */
int mla_get_device_error(int clear);

/* Text for a status code (static storage). */
const char* mla_status_string(int status);

/* MLA_VERIFY_ABI_VERSION of the built library. */
int mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_H */
