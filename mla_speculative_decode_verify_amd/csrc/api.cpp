// C-ABI host layer of libmla_verify.so: argument validation, planning
// (row grouping and split count), per-(device, stream) workspace, static
// per-device memory (error flag, zero row, no-allocation scratch), and
// kernel launches. Validation runs before any HIP call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "mla_internal.h"
#include "mla_verify.h"

namespace {

using mla::kDk;
using mla::kDv;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ----------------------------------------------------------------- per-device state
// Static device memory. The GPU runtime gives every device the library runs
// on its own copy of these arrays, from the first use on that device until
// the process ends; host code reaches a device's copy only through the
// address hipGetSymbolAddress returns with that device current (the array
// names below are host-side stand-ins, not device addresses).
//   dev_block: the sticky error word at offset 0 and a zero cache row at
//              kZeroRowOffset (read in place of masked or invalid rows).
//   scratch:   split partials of mla_verify_attn_noalloc, for callers that
//              cannot allocate.
constexpr size_t kDevBlockBytes = 4096;
constexpr size_t kZeroRowOffset = 256;
static __device__ __align__(256) unsigned char dev_block[kDevBlockBytes];
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

struct WsKey {
  int device;
  hipStream_t stream;
  bool operator<(const WsKey& o) const {
    return device != o.device ? device < o.device : reinterpret_cast<uintptr_t>(stream) < reinterpret_cast<uintptr_t>(o.stream);
  }
};
struct WsBuf {
  void* ptr = nullptr;
  size_t bytes = 0;
  bool captured = false;  // handed to a call made while its stream was capturing
};
struct DevPtrs {
  unsigned* block = nullptr;  // this device's dev_block
  void* scratch = nullptr;    // this device's scratch
};

std::mutex g_mu;
std::map<WsKey, WsBuf> g_ws;
// Buffers replaced by a larger one after a captured call used them: a graph
// may still replay with them, so only mla_release_workspace frees them.
std::map<WsKey, std::vector<void*>> g_retired;
std::map<int, DevPtrs> g_dev;
std::map<int, int> g_cus;

int current_device(int* dev) {
  return hipGetDevice(dev) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int device_cus(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_cus.find(dev);
  if (it != g_cus.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  g_cus[dev] = cus;
  return cus;
}

bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) return false;
  return st != hipStreamCaptureStatusNone;
}

// Largest batch whose split counts may follow the sequence lengths: the
// kernels derive them with one sequence per lane of a wavefront.
constexpr int kBalanceMaxBatch = 64;

// Device addresses of this device's static arrays, looked up once per device
// (`dev` must be the current device). Allocates nothing.
int dev_ptrs(int dev, DevPtrs* out) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_dev.find(dev);
  if (it != g_dev.end()) {
    *out = it->second;
    return MLA_OK;
  }
  DevPtrs d;
  if (hipGetSymbolAddress(reinterpret_cast<void**>(&d.block), HIP_SYMBOL(dev_block)) != hipSuccess || !d.block)
    return MLA_ERR_LAUNCH;
  if (hipGetSymbolAddress(&d.scratch, HIP_SYMBOL(scratch)) != hipSuccess || !d.scratch) return MLA_ERR_LAUNCH;
  g_dev[dev] = d;
  *out = d;
  return MLA_OK;
}

int error_word(int dev, unsigned** out) {
  DevPtrs d;
  const int st = dev_ptrs(dev, &d);
  if (st == MLA_OK) *out = d.block;
  return st;
}

// The workspace of (dev, stream), grown to at least `bytes`. A buffer that a
// call made under capture has used is never freed implicitly: when a later
// eager call needs more, it is parked until mla_release_workspace.
int workspace(int dev, hipStream_t stream, size_t bytes, void** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  const WsKey key{dev, stream};
  WsBuf& w = g_ws[key];
  const bool capturing = stream_capturing(stream);
  if (w.bytes >= bytes) {
    w.captured |= capturing;
    *out = w.ptr;
    return MLA_OK;
  }
  if (capturing) return MLA_ERR_WORKSPACE;
  if (w.ptr) {
    if (w.captured) {
      g_retired[key].push_back(w.ptr);
    } else {
      // only earlier eager calls on this stream can still use it
      if (hipStreamSynchronize(stream) != hipSuccess) return MLA_ERR_LAUNCH;
      if (hipFree(w.ptr) != hipSuccess) return MLA_ERR_LAUNCH;
    }
    w = WsBuf{};
  }
  // round up to 2 MiB so small growth steps do not reallocate every call
  const size_t want = (bytes + (2u << 20) - 1) & ~((size_t)(2u << 20) - 1);
  if (hipMalloc(&w.ptr, want) != hipSuccess) {
    w.ptr = nullptr;
    return MLA_ERR_LAUNCH;
  }
  w.bytes = want;
  *out = w.ptr;
  return MLA_OK;
}

int release_workspace(int dev, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  const WsKey key{dev, stream};
  auto it = g_ws.find(key);
  auto rt = g_retired.find(key);
  if (it == g_ws.end() && rt == g_retired.end()) return MLA_OK;
  if (hipStreamSynchronize(stream) != hipSuccess) return MLA_ERR_LAUNCH;
  int st = MLA_OK;
  if (it != g_ws.end()) {
    if (it->second.ptr && hipFree(it->second.ptr) != hipSuccess) st = MLA_ERR_LAUNCH;
    g_ws.erase(it);
  }
  if (rt != g_retired.end()) {
    for (void* p : rt->second)
      if (hipFree(p) != hipSuccess) st = MLA_ERR_LAUNCH;
    g_retired.erase(rt);
  }
  return st;
}

// ----------------------------------------------------------------- planning
// Query rows are cut into 16-row blocks; a bf16 split workgroup serves `nb`
// blocks with two wavefronts each (split_bf16.hip), at most 6 blocks (12
// wavefronts, three per SIMD). Rows of one sequence that do not fit one
// workgroup are dealt to `groups` workgroups, each gathering the same keys.
//
// Cost model of one bf16 call (microseconds; a least-squares fit to 23
// cold-cache call times on MI355X at H=8 and H=64 with 4, 5 and 6 blocks per
// workgroup and 1 to 74 tiles per split, residuals within 2 us): a
// 32-position tile of the slowest split costs about 1.86 us with up to 5
// blocks per workgroup and 2.21 us with 6 (three wavefronts per SIMD share
// its MFMA and LDS instead of two), a call has about 8 us of fixed cost
// (11.4 us with 6 blocks: more query rows to load and partial rows to
// store per workgroup); with several splits the merge kernel adds about
// 4 us, and every split's partials (1036 bytes per query row, written and
// read back) about 0.49 us per MB. With 4 blocks the workgroup carries four
// gather-only wavefronts (one per SIMD), which made its tile cheaper: 1.60 us
// here. (Least squares over its H=64 calls at full occupancy, the other
// constants kept, gives 1.52 us, but then 64k prefixes would take 4 blocks,
// which measured 2-3% slower there than 6; 1.60 keeps the measured order at
// 16k and 32k, where 4 blocks are fastest, and at 64k.)
// Groups of 2 and 3 blocks (balanced by their gather-only wavefronts) were
// fitted on a sweep of H=64 calls (prefixes 256 to 32k, every group size
// from 2 to 6 at three split counts each): relative to 4 blocks their tile
// costs 0.76x and 0.95x and their call about 0.9 and 0.2 us less fixed time,
// scaled onto the constants above. With them, 18 groups of 2 blocks (fewer
// splits, so fewer partials) win up to 4k positions, as measured.
constexpr double kTileUs[7] = {0.0, 1.86, 1.21, 1.52, 1.60, 1.86, 2.21};  // by blocks per workgroup
constexpr double kFixedUs[7] = {0.0, 8.1, 7.2, 7.94, 8.1, 8.1, 11.4};
constexpr double kPartUsPerByte = 0.49e-6;
constexpr double kMergeUs = 4.0;
constexpr int kMaxBlocks = 6;

double bf16_cost_us(int nb, long wgs_per_split, long tiles, long s, long rows_total, int num_cus) {
  const long passes = (wgs_per_split * s + num_cus - 1) / num_cus;
  double t = kFixedUs[nb] + (double)(passes * ((tiles + s - 1) / s)) * kTileUs[nb];
  if (s > 1) t += kMergeUs + kPartUsPerByte * 1036.0 * (double)rows_total * (double)s;
  return t;
}

// Best split count for `nb` blocks per workgroup and `wgs_per_split`
// workgroups per split (key sets times row groups): one workgroup per CU at
// most (a split workgroup fills a CU), so the grid runs in a single pass;
// the cheapest count wins, the fewest on ties.
long bf16_best_split(int nb, long wgs_per_split, long tiles, long rows_total, int num_cus, double* cost) {
  const long one_pass = std::max<long>(1, num_cus / wgs_per_split);
  long s = 1;
  double best = 0.0;
  for (long c = 1; c <= std::min(one_pass, tiles); ++c) {
    const double t = bf16_cost_us(nb, wgs_per_split, tiles, c, rows_total, num_cus);
    if (c == 1 || t < best) {
      best = t;
      s = c;
    }
  }
  *cost = best;
  return s;
}

struct Layout {
  int nb = 1, groups = 1;
  int nsplit = 1;
  long key_sets = 1;
};

// One sequence whose rows fill exactly five 16-row blocks (H=8 with q_len 9
// or 10, one tensor-parallel rank's share): its rows may go to one
// workgroup of 5 blocks, 2 of 3 (3 + 2) or 3 of 2 (2 + 2 + 1), the smaller
// groups gathering every key once each (the second read mostly from L2).
// Each layout's split + merge kernel time was fitted to batch-1 calls at
// prefixes 256 to 64k (least squares over 16 to 23 points each, rms error
// 0.25-0.7 us) as
//   f + t * T + p * R * S / 1000 + q * G * S * T / 1000
// with T the tiles of the longest split, R the rows, S the splits and G the
// groups (the last term: HBM traffic growing with the workgroups in
// flight; with one group S * T is about the tile count, so that fit leaves
// it out). The 5- and 3-block workgroups carry two gather-only wavefronts.
// Smaller groups win up to about 32k positions (fewer wavefronts per SIMD
// make a tile cheaper, and fewer splits mean fewer partials), one group of
// 5 beyond (measured: 35.5 us of kernel time at 64k against 37.0 for
// 2 x 3 blocks).
struct FiveBlockFit {
  int nb;
  double f, t, p, q;
};
constexpr FiveBlockFit kFiveBlockFits[3] = {
    {5, 14.025, 1.379, 0.516, 0.0}, {3, 12.831, 1.222, 0.282, 0.183}, {2, 11.968, 1.454, 0.097, 0.771}};
constexpr double kMergeKernelUs = 4.5;  // what a single split saves: no merge kernel

double five_block_cost_us(const FiveBlockFit& fit, int groups, long tiles, long s, long rows) {
  const long t = (tiles + s - 1) / s;
  double c = fit.f + fit.t * (double)t + fit.p * (double)(rows * s) / 1000.0 +
             fit.q * (double)((long)groups * s * t) / 1000.0;
  if (s == 1) c -= kMergeKernelUs;
  return c;
}

Layout plan_five_blocks(int rows, long tiles, int num_cus, int nsplit) {
  Layout L;
  double best = 0.0;
  bool have = false;
  for (const FiveBlockFit& fit : kFiveBlockFits) {
#ifdef MLA_FIVE_BLOCK_NB
    if (fit.nb != MLA_FIVE_BLOCK_NB) continue;  // tuning builds that time one layout
#endif
    const int groups = (5 + fit.nb - 1) / fit.nb;
    const long one_pass = std::max<long>(1, num_cus / groups);
    long lo = 1, hi = std::min(one_pass, tiles);
    if (nsplit > 0) {
      if (fit.nb != 5 && (long)nsplit > one_pass) continue;  // the fits hold for one pass of the grid
      lo = hi = nsplit;
    }
    for (long s = lo; s <= hi; ++s) {
      const double c = five_block_cost_us(fit, groups, tiles, s, rows);
      if (!have || c < best) {  // the first layout and the fewest splits win ties
        have = true;
        best = c;
        L.nb = fit.nb;
        L.groups = groups;
        L.nsplit = (int)std::max<long>(1, std::min<long>(s, MLA_MAX_NSPLIT));
      }
    }
  }
  return L;
}

// Row grouping and split count. bf16 verify: all q_len * heads rows of a
// sequence share its keys, so they form the key set; up to 6 blocks fit one
// workgroup, else the blocks-per-workgroup and split count come jointly from
// the cost model. fp8 top-k: the heads of one query share its list, so the
// key sets are batch * q_len; that kernel converts tiles in registers and
// spills with 5 blocks, so its groups hold at most 4 blocks and its splits
// never hold fewer than 128 list entries. `keys` = positions per key set
// (the longest sequence, or the top-k list length); `nsplit` > 0 is kept.
Layout plan_layout(int batch, int q_len, int heads, int keys, int kv_dtype, int num_cus, int nsplit) {
  Layout L;
  num_cus = std::max(1, num_cus);
  if (kv_dtype == MLA_KV_FP8_E4M3) {
    const int blocks = (heads + 15) / 16;
    L.nb = std::min(blocks, 4);
    L.groups = (blocks + L.nb - 1) / L.nb;
    L.key_sets = (long)batch * q_len;
    long s = nsplit;
    if (s <= 0) {
      s = std::max<long>(1, num_cus / (L.key_sets * L.groups));
      s = std::min(s, std::max<long>(1, ((long)keys + 127) / 128));
    }
    L.nsplit = (int)std::max<long>(1, std::min<long>(s, MLA_MAX_NSPLIT));
    return L;
  }
  const int rows = q_len * heads;
  const int blocks = (rows + 15) / 16;
  const long tiles = std::max<long>(1, ((long)keys + 31) / 32);
  const long rows_total = (long)batch * rows;
  L.key_sets = batch;
  if (batch == 1 && blocks == 5) {
    Layout F = plan_five_blocks(rows, tiles, num_cus, nsplit);
    F.key_sets = batch;
    return F;
  }
  double best = 0.0;
  bool have = false;
  for (int nb = 1; nb <= kMaxBlocks; ++nb) {
    // one workgroup when the blocks fit; otherwise 2 to 6 blocks per group
    if (blocks <= kMaxBlocks ? nb != blocks : nb < 2) continue;
#ifdef MLA_ONLY_NB
    if (blocks > kMaxBlocks && nb != MLA_ONLY_NB) continue;  // tuning builds that time one group size
#endif
    const int groups = (blocks + nb - 1) / nb;
    const long wgs = (long)batch * groups;
    double cost = 0.0;
    long s = nsplit;
    if (s > 0) cost = bf16_cost_us(nb, wgs, tiles, s, rows_total, num_cus);
    else s = bf16_best_split(nb, wgs, tiles, rows_total, num_cus, &cost);
    if (!have || cost < best) {
      have = true;
      best = cost;
      L.nb = nb;
      L.groups = groups;
      L.nsplit = (int)std::max<long>(1, std::min<long>(s, MLA_MAX_NSPLIT));
    }
  }
  return L;
}

int choose_nsplit_impl(int batch, int q_len, int heads, int keys, int kv_dtype, int num_cus) {
  if (batch < 1 || q_len < 1 || heads < 1 || num_cus < 1) return 1;
  return plan_layout(batch, q_len, heads, keys, kv_dtype, num_cus, 0).nsplit;
}

struct Call {
  mla::Args a;
  int nb = 1, groups = 1;
  int kernel = 0;
  size_t ws_bytes = 0;
};

int validate(const mla_q_t* q, const mla_kv_t* kv, const int32_t* slot_table, const int32_t* seq_lens,
             const mla_mask_t* m, const float* out, const float* lse, int nsplit, bool need_data) {
  if (!q || !kv || !m) return MLA_ERR_INVALID_ARG;
  if (need_data && (!q->data || !slot_table || !seq_lens || !out || !kv->latent)) return MLA_ERR_INVALID_ARG;
  if (q->batch < 1 || q->q_len < 1 || q->heads < 1) return MLA_ERR_INVALID_ARG;
  if (q->q_len > MLA_MAX_Q_LEN || q->heads > MLA_MAX_HEADS) return MLA_ERR_UNSUPPORTED;
  if (q->batch > 65535) return MLA_ERR_UNSUPPORTED;
  if (!(q->sm_scale > 0.f) || !std::isfinite(q->sm_scale)) return MLA_ERR_INVALID_ARG;
  if (kv->pool_rows < 1 || kv->slot_stride < 1) return MLA_ERR_INVALID_ARG;
  if (kv->max_seq_len < 0 || kv->max_seq_len > kv->slot_stride) return MLA_ERR_INVALID_ARG;
  if (nsplit > MLA_MAX_NSPLIT) return MLA_ERR_INVALID_ARG;
  if (kv->dtype == MLA_KV_BF16) {
    if (m->kind != MLA_MASK_NONE && m->kind != MLA_MASK_CAUSAL && m->kind != MLA_MASK_TREE) {
      return m->kind == MLA_MASK_TOPK ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
    }
    if (m->kind == MLA_MASK_TREE) {
      if (need_data && !m->tree_anc) return MLA_ERR_INVALID_ARG;
      if (!aligned(m->tree_anc, 8)) return MLA_ERR_ALIGN;
    }
  } else if (kv->dtype == MLA_KV_FP8_E4M3) {
    if (m->kind != MLA_MASK_TOPK) {
      return (m->kind >= MLA_MASK_NONE && m->kind <= MLA_MASK_TREE) ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
    }
    if (need_data && (!kv->rope || !kv->scale || !m->topk_idx)) return MLA_ERR_INVALID_ARG;
    if (m->topk < 1) return MLA_ERR_INVALID_ARG;
    if (m->topk > MLA_MAX_TOPK) return MLA_ERR_UNSUPPORTED;
    if (!aligned(kv->rope, 16) || !aligned(kv->scale, 4) || !aligned(m->topk_idx, 4)) return MLA_ERR_ALIGN;
  } else {
    return MLA_ERR_INVALID_ARG;
  }
  if (!aligned(q->data, 16) || !aligned(kv->latent, 16) || !aligned(out, 16)) return MLA_ERR_ALIGN;
  if (!aligned(lse, 4) || !aligned(slot_table, 4) || !aligned(seq_lens, 4)) return MLA_ERR_ALIGN;
  return MLA_OK;
}

int make_plan(const mla_q_t* q, const mla_kv_t* kv, const mla_mask_t* m, int nsplit, int num_cus, Call* c) {
  c->kernel = kv->dtype == MLA_KV_FP8_E4M3 ? 1 : 0;
  const int maxlen = kv->max_seq_len > 0 ? kv->max_seq_len : kv->slot_stride;
  const int seqlen_for_split = c->kernel == 1 ? std::min(maxlen, m->topk) : maxlen;
  const Layout L = plan_layout(q->batch, q->q_len, q->heads, seqlen_for_split, kv->dtype, num_cus, nsplit);
  const long key_sets = L.key_sets;
  if (key_sets > 65535) return MLA_ERR_UNSUPPORTED;
  c->nb = L.nb;
  c->groups = L.groups;
  int s = L.nsplit;
  if (s > MLA_MAX_NSPLIT) return MLA_ERR_INVALID_ARG;
  c->a.balance_units = 0;
  if (nsplit <= 0 && c->kernel == 0 && q->batch >= 2 && q->batch <= kBalanceMaxBatch) {
    // Ragged batch, library-chosen splits: per-sequence split counts that
    // follow the lengths (balanced_split in the kernels), `units` splits in
    // all so the grid runs in one pass. s becomes the partials' stride: the
    // most one sequence can take (all others get one), at least 4 tiles each.
    const long units = num_cus / c->groups;
    const long tiles = ((long)maxlen + 31) / 32;
    const long smax = std::min<long>({(long)MLA_MAX_NSPLIT, units - q->batch + 1, std::max<long>(1, (tiles + 3) / 4)});
    // (the kernels sum the tile counts in 32-bit integers)
    const long stride_tiles = ((long)kv->slot_stride + 31) / 32;
    if (units > q->batch && smax >= 2 && (long)q->batch * stride_tiles < (1L << 30)) {
      // no more units than the splits the caps allow
      c->a.balance_units = (int)std::min<long>(units, (long)q->batch * smax);
      s = (int)smax;
    }
  }
  // workgroup units of the 1-D split grid, indexed with int on the device
  const long units = (c->a.balance_units > 0 ? c->a.balance_units : key_sets * s) * c->groups;
  if (units > 0x7fffffffL - 8) return MLA_ERR_UNSUPPORTED;
  // Units k * groups + g go to the XCDs in contiguous runs of xcd_chunk (the
  // kernels' xcd_unit). A run that is a multiple of the row groups keeps all
  // groups of a split, which gather the same cache rows, on one XCD and its
  // L2. That is used when the padded grid still fits the XCDs' CUs in one
  // pass and still spreads the work over all 8 XCDs (idle padding units
  // return at once).
  long chunk = (units + 7) / 8;
  if (c->groups > 1) {
    const long aligned = (chunk + c->groups - 1) / c->groups * c->groups;
    if (aligned * 8 <= num_cus && units > 7 * aligned) chunk = aligned;
  }
  c->a.xcd_chunk = (int)chunk;
  c->a.nsplit = s;
  c->ws_bytes = mla_workspace_bytes(q->batch, q->q_len, q->heads, s);
  // L2 prefetch ahead of the gathers pays only for long splits (the kernel
  // also checks each split's own length): at least kPfMinTiles tiles in the
  // longest split of a uniform count, or of the stride of length-following
  // counts (a lower bound of the longest sequence's tiles per split).
  const long max_tiles = ((long)maxlen + 31) / 32;
  c->a.l2_prefetch = c->kernel == 0 && (max_tiles + s - 1) / s >= mla::kPfMinTiles ? 1 : 0;
  return MLA_OK;
}

void fill_args(const mla_q_t* q, const mla_kv_t* kv, const int32_t* slot_table, const int32_t* seq_lens,
               const mla_mask_t* m, float* out, float* lse, Call* c) {
  mla::Args& a = c->a;
  a.q = q->data;
  a.latent = kv->latent;
  a.rope = kv->rope;
  a.kscale = kv->scale;
  a.slots = slot_table;
  a.seq_lens = seq_lens;
  a.anc = m->kind == MLA_MASK_TREE ? m->tree_anc : nullptr;
  a.topk_idx = m->kind == MLA_MASK_TOPK ? m->topk_idx : nullptr;
  a.out = out;
  a.lse = lse;
  a.part_o = nullptr;
  a.part_lse = nullptr;
  a.part_scale = nullptr;
  a.part_count = nullptr;
  a.err = nullptr;
  a.zero_row = nullptr;
  a.pool_rows = kv->pool_rows;
  a.slot_stride = kv->slot_stride;
  a.len_hint = kv->max_seq_len > 0 ? kv->max_seq_len : kv->slot_stride;
  a.batch = q->batch;
  a.q_len = q->q_len;
  a.heads = q->heads;
  a.rows = q->q_len * q->heads;
  a.row_groups = 1;
  a.mask_kind = m->kind;
  a.topk = m->kind == MLA_MASK_TOPK ? m->topk : 0;
  a.scale_log2 = (float)((double)q->sm_scale * 1.4426950408889634);
}

enum Stage { kSplit = 1, kCombine = 2, kBoth = 3 };

// Where a call's split partials live: the per-(device, stream) workspace,
// or this device's static scratch (mla_verify_attn_noalloc).
enum class Parts { kWorkspace, kScratch };

int run(const mla_q_t* q, const mla_kv_t* kv, const int32_t* slot_table, const int32_t* seq_lens,
        const mla_mask_t* m, float* out, float* lse, int nsplit, hipStream_t stream, int stages,
        Parts parts = Parts::kWorkspace) {
  int st = validate(q, kv, slot_table, seq_lens, m, out, lse, nsplit, true);
  if (st != MLA_OK) return st;
  int dev = 0;
  if ((st = current_device(&dev)) != MLA_OK) return st;
  Call c;
  fill_args(q, kv, slot_table, seq_lens, m, out, lse, &c);
  if ((st = make_plan(q, kv, m, nsplit, device_cus(dev), &c)) != MLA_OK) return st;
  if (parts == Parts::kScratch && c.ws_bytes > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_SCRATCH;
  DevPtrs dp;
  if ((st = dev_ptrs(dev, &dp)) != MLA_OK) return st;
  c.a.err = dp.block;
  c.a.zero_row = reinterpret_cast<const char*>(dp.block) + kZeroRowOffset;
  if (c.a.nsplit > 1) {
    void* ws = dp.scratch;
    if (parts == Parts::kWorkspace && (st = workspace(dev, stream, c.ws_bytes, &ws)) != MLA_OK) return st;
    // [fp16 O: P x 512][fp32 LSE: P][fp32 scale: P x 2], P = batch * nsplit * rows;
    // O is split-major per sequence, LSE and scales row-major (splits contiguous)
    const size_t P = (size_t)q->batch * c.a.nsplit * c.a.rows;
    char* base = static_cast<char*>(ws);
    c.a.part_o = reinterpret_cast<_Float16*>(base);
    c.a.part_lse = reinterpret_cast<float*>(base + P * kDv * sizeof(_Float16));
    c.a.part_scale = c.a.part_lse + P;
    c.a.part_count = reinterpret_cast<int32_t*>(c.a.part_scale + 2 * P);
  }
  if (stages & kSplit) {
    hipError_t e = c.kernel == 0 ? mla::launch_split_bf16(c.a, c.nb, c.groups, stream)
                                 : mla::launch_split_fp8_topk(c.a, c.nb, c.groups, stream);
    if (e != hipSuccess) return MLA_ERR_LAUNCH;
  }
  if ((stages & kCombine) && c.a.nsplit > 1) {
    if (mla::launch_combine(c.a, stream) != hipSuccess) return MLA_ERR_LAUNCH;
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_verify_attn(const mla_q_t* q, const mla_kv_t* kv_cache, const int32_t* slot_table, const int32_t* seq_lens,
                    const mla_mask_t* mask_desc, float* out, float* lse, int nsplit, hipStream_t stream) {
  return run(q, kv_cache, slot_table, seq_lens, mask_desc, out, lse, nsplit, stream, kBoth);
}

int mla_verify_attn_noalloc(const mla_q_t* q, const mla_kv_t* kv_cache, const int32_t* slot_table,
                            const int32_t* seq_lens, const mla_mask_t* mask_desc, float* out, float* lse,
                            int nsplit, hipStream_t stream) {
  return run(q, kv_cache, slot_table, seq_lens, mask_desc, out, lse, nsplit, stream, kBoth, Parts::kScratch);
}

int mla_verify_split(const mla_q_t* q, const mla_kv_t* kv_cache, const int32_t* slot_table, const int32_t* seq_lens,
                     const mla_mask_t* mask_desc, float* out, float* lse, int nsplit, hipStream_t stream) {
  return run(q, kv_cache, slot_table, seq_lens, mask_desc, out, lse, nsplit, stream, kSplit);
}

int mla_verify_combine(const mla_q_t* q, const mla_kv_t* kv_cache, const int32_t* slot_table,
                       const int32_t* seq_lens, const mla_mask_t* mask_desc, float* out, float* lse, int nsplit,
                       hipStream_t stream) {
  return run(q, kv_cache, slot_table, seq_lens, mask_desc, out, lse, nsplit, stream, kCombine);
}

int mla_plan(const mla_q_t* q, const mla_kv_t* kv_cache, const mla_mask_t* mask_desc, int nsplit, mla_plan_t* plan) {
  if (!plan) return MLA_ERR_INVALID_ARG;
  int st = validate(q, kv_cache, nullptr, nullptr, mask_desc, nullptr, nullptr, nsplit, false);
  if (st != MLA_OK) return st;
  // the current device's CU count, as the call itself would use (256 when no
  // device is visible)
  int cus = 256;
  int dev = 0;
  if (current_device(&dev) == MLA_OK) cus = device_cus(dev);
  Call c;
  if ((st = make_plan(q, kv_cache, mask_desc, nsplit, cus, &c)) != MLA_OK) return st;
  plan->nsplit = c.a.nsplit;
  plan->waves_per_group = 2 * c.nb + (c.kernel == 0 ? mla::bf16_gather_waves(c.nb) : mla::fp8_load_waves(c.nb));
  plan->row_groups = c.groups;
  plan->grid = c.a.balance_units > 0 ? c.a.balance_units * c.groups
                                      : c.a.nsplit * c.groups * q->batch * (c.kernel == 1 ? q->q_len : 1);
  plan->workspace_bytes = c.ws_bytes;
  plan->kernel = c.kernel;
  plan->row_blocks = c.nb;
  plan->balanced = c.a.balance_units > 0 ? 1 : 0;
  plan->l2_prefetch = c.a.l2_prefetch;
  return MLA_OK;
}

int mla_choose_nsplit(int batch, int q_len, int heads, int max_seq_len, int kv_dtype, int num_cus) {
  if (batch < 1 || q_len < 1 || heads < 1 || max_seq_len < 0 || num_cus < 1) return MLA_ERR_INVALID_ARG;
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_INVALID_ARG;
  return choose_nsplit_impl(batch, q_len, heads, max_seq_len, kv_dtype, num_cus);
}

size_t mla_workspace_bytes(int batch, int q_len, int heads, int nsplit) {
  if (batch < 1 || q_len < 1 || heads < 1 || nsplit <= 1) return 0;
  return (size_t)batch * nsplit * q_len * heads * (kDv * sizeof(_Float16) + 3 * sizeof(float)) +
         (size_t)batch * sizeof(int32_t);
}

int mla_reserve_workspace(size_t bytes, hipStream_t stream) {
  int dev = 0;
  int st = current_device(&dev);
  if (st != MLA_OK) return st;
  DevPtrs dp;
  if ((st = dev_ptrs(dev, &dp)) != MLA_OK) return st;
  if (bytes == 0) return MLA_OK;
  void* p = nullptr;
  return workspace(dev, stream, bytes, &p);
}

int mla_release_workspace(hipStream_t stream) {
  int dev = 0;
  int st = current_device(&dev);
  if (st != MLA_OK) return st;
  return release_workspace(dev, stream);
}

int mla_build_tree_mask_host(const int32_t* parents, int batch, int q_len, uint64_t* anc_out) {
  if (!parents || !anc_out || batch < 1 || q_len < 1) return MLA_ERR_INVALID_ARG;
  if (q_len > MLA_MAX_Q_LEN) return MLA_ERR_UNSUPPORTED;
  for (int b = 0; b < batch; ++b) {
    const int32_t* par = parents + (size_t)b * q_len;
    for (int i = 0; i < q_len; ++i) {
      if (par[i] < -1 || par[i] >= i) return MLA_ERR_INVALID_ARG;
    }
    for (int i = 0; i < q_len; ++i) {
      uint64_t bits = 1ull << i;
      for (int p = par[i]; p != -1; p = par[p]) bits |= 1ull << p;
      anc_out[(size_t)b * q_len + i] = bits;
    }
  }
  return MLA_OK;
}

int mla_build_tree_mask(const int32_t* parents, int batch, int q_len, uint64_t* anc_out, hipStream_t stream) {
  if (!parents || !anc_out || batch < 1 || q_len < 1) return MLA_ERR_INVALID_ARG;
  if (q_len > MLA_MAX_Q_LEN) return MLA_ERR_UNSUPPORTED;
  if (!aligned(parents, 4) || !aligned(anc_out, 8)) return MLA_ERR_ALIGN;
  int dev = 0;
  int st = current_device(&dev);
  if (st != MLA_OK) return st;
  unsigned* err = nullptr;
  if ((st = error_word(dev, &err)) != MLA_OK) return st;
  return mla::launch_tree_mask(parents, batch, q_len, anc_out, err, stream) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int mla_append_kv(void* latent, int64_t pool_rows, int slot_stride, const void* new_rows, int batch, int q_len,
                  const int32_t* slot_table, const int32_t* seq_lens, hipStream_t stream) {
  if (!latent || !new_rows || !slot_table || !seq_lens) return MLA_ERR_INVALID_ARG;
  if (batch < 1 || q_len < 1 || pool_rows < 1 || slot_stride < q_len) return MLA_ERR_INVALID_ARG;
  if (q_len > MLA_MAX_Q_LEN) return MLA_ERR_UNSUPPORTED;
  if (!aligned(latent, 16) || !aligned(new_rows, 16) || !aligned(slot_table, 4) || !aligned(seq_lens, 4))
    return MLA_ERR_ALIGN;
  int dev = 0;
  int st = current_device(&dev);
  if (st != MLA_OK) return st;
  unsigned* err = nullptr;
  if ((st = error_word(dev, &err)) != MLA_OK) return st;
  return mla::launch_append(latent, pool_rows, slot_stride, new_rows, batch, q_len, slot_table, seq_lens, err,
                            stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_LAUNCH;
}

int mla_topk_select(const float* scores, int batch, int q_len, int score_stride, const int32_t* seq_lens,
                    int topk, int32_t* topk_idx, hipStream_t stream) {
  if (!scores || !seq_lens || !topk_idx) return MLA_ERR_INVALID_ARG;
  if (batch < 1 || q_len < 1 || score_stride < 1 || topk < 1) return MLA_ERR_INVALID_ARG;
  if ((long)batch * q_len > 65535 || score_stride > (1 << 20)) return MLA_ERR_UNSUPPORTED;
  if (!aligned(scores, 16) || score_stride % 4 != 0 || !aligned(seq_lens, 4) || !aligned(topk_idx, 4))
    return MLA_ERR_ALIGN;
  int dev = 0;
  int st = current_device(&dev);
  if (st != MLA_OK) return st;
  unsigned* err = nullptr;
  if ((st = error_word(dev, &err)) != MLA_OK) return st;
  void* ws = nullptr;
  if ((st = workspace(dev, stream, mla::topk_workspace_bytes(batch * q_len, score_stride), &ws)) != MLA_OK) return st;
  return mla::launch_topk(scores, batch, q_len, score_stride, seq_lens, topk, topk_idx, err, ws, stream) ==
                 hipSuccess
             ? MLA_OK
             : MLA_ERR_LAUNCH;
}

size_t mla_topk_workspace_bytes(int batch, int q_len, int score_stride) {
  if (batch < 1 || q_len < 1 || score_stride < 1) return 0;
  return mla::topk_workspace_bytes(batch * q_len, score_stride);
}

int mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk, int tokens, int heads, void* q_out,
                 hipStream_t stream) {
  if (!q_nope || !q_rope || !w_uk || !q_out || tokens < 1 || heads < 1) return MLA_ERR_INVALID_ARG;
  if (heads > 65535) return MLA_ERR_UNSUPPORTED;
  if (!aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(w_uk, 16) || !aligned(q_out, 16)) return MLA_ERR_ALIGN;
  return mla::launch_absorb_q(q_nope, q_rope, w_uk, tokens, heads, q_out, stream) == hipSuccess ? MLA_OK
                                                                                                : MLA_ERR_LAUNCH;
}

int mla_project_o(const float* o_latent, const void* w_uv, int tokens, int heads, float* o_out,
                  hipStream_t stream) {
  if (!o_latent || !w_uv || !o_out || tokens < 1 || heads < 1) return MLA_ERR_INVALID_ARG;
  if (heads > 65535) return MLA_ERR_UNSUPPORTED;
  if (!aligned(o_latent, 16) || !aligned(w_uv, 16) || !aligned(o_out, 16)) return MLA_ERR_ALIGN;
  return mla::launch_project_o(o_latent, w_uv, tokens, heads, o_out, stream) == hipSuccess ? MLA_OK
                                                                                          : MLA_ERR_LAUNCH;
}

int mla_get_device_error(int clear) {
  int dev = 0;
  int st = current_device(&dev);
  if (st != MLA_OK) return st;
  unsigned* err = nullptr;
  if ((st = error_word(dev, &err)) != MLA_OK) return st;
  if (hipDeviceSynchronize() != hipSuccess) return MLA_ERR_LAUNCH;
  unsigned v = 0;
  if (hipMemcpy(&v, err, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return MLA_ERR_LAUNCH;
  if (clear && hipMemset(err, 0, sizeof(unsigned)) != hipSuccess) return MLA_ERR_LAUNCH;
  return (int)(v & 0x7fffffffu);
}

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_ALIGN: return "pointer misaligned";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or combination";
    case MLA_ERR_WORKSPACE: return "workspace too small while the stream is capturing";
    case MLA_ERR_LAUNCH: return "HIP call or kernel launch failed";
    case MLA_ERR_SCRATCH: return "split partials exceed the static scratch of mla_verify_attn_noalloc";
    default: return "unknown status";
  }
}

int mla_abi_version(void) { return MLA_VERIFY_ABI_VERSION; }

}  // extern "C"
