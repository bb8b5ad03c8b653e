// Device-side building blocks for gfx950 (CDNA4): MFMA wrappers, the LDS
// transposing read, fast exp2/log2 and wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// D = A * B + C for A 16x32, B 32x16 (bf16), C/D 16x16 fp32.
// Lane l holds A[l % 16][8*(l/16) .. +7], B[8*(l/16) .. +7][l % 16] and
// C[4*(l/16) + r][l % 16] for r = 0..3 (checked on gfx950).
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read. Within each 16-lane group, lane 4*b + c supplies the
// address of 4 consecutive 16-bit elements of "row" b (b, c in 0..3); lane i
// of the group receives element i of the 16-element span, taken from rows
// 0..3 in order. The address must be 8-byte aligned.
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + sum of the 8 bf16 values, two at a time with the bf16 dot product
// against (1, 1) (products are exact; each step rounds once in fp32).
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2 * i], v[2 * i + 1]}, one, acc, false);
  return acc;
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Max / sum across the four 16-lane groups (lanes l, l^16, l^32, l^48),
// with the gfx950 lane swaps: permlane16_swap(v, v) yields, in lane l, the
// values of lanes l and l^16 (the even 16-lane row's first), and
// permlane32_swap(v, v) those of lanes l and l^32 (lower half first). Each
// step combines the same two operands in the same order in every lane, so
// all four lanes end with bitwise the same result.
__device__ __forceinline__ float group4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations (lgkmcnt) and meets the other waves, but unlike __syncthreads()
// does not drain the vector-memory queue, so global loads and global-to-LDS
// gathers stay in flight across it. Callers wait for any global-to-LDS data
// they need with an explicit vmcnt wait first. The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Global-to-LDS load of 16 bytes per lane (gfx950 global_load_lds_dwordx4):
// lane i's 16 bytes land at LDS byte address lds_addr + 16 i, where lds_addr
// is wave-uniform (it goes through M0). Written as inline assembly so the
// compiler neither tracks these loads nor inserts its own waits for them:
// callers count them and wait with an explicit vmcnt before reading the data,
// and must drain them (vmcnt(0)) before the workgroup ends.
__device__ __forceinline__ void lds_dma_b128(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds_addr) : "memory", "m0");
}

// Global-to-LDS load of 4 bytes per lane (global_load_lds_dword): lane i's
// word lands at LDS byte address lds_addr + 4 i. Counted and drained by the
// caller like lds_dma_b128; used to pull cache lines into L2 ahead of the
// 16-byte gathers that will read them (the landed words are never read).
__device__ __forceinline__ void lds_dma_b32(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(src), "s"(lds_addr) : "memory", "m0");
}

// 32-bit LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

__device__ __forceinline__ void flag_error(unsigned* err, unsigned bits) {
  if (err) atomicOr(err, bits);
}

constexpr float kLn2 = 0.69314718055994530942f;

// XCD-aware work order for a 1-D grid of 8 * C workgroups (C = ceil(units /
// 8)). The hardware hands consecutive workgroup ids to the 8 XCDs in turn,
// so id L runs on XCD L % 8. Unit j = (L % 8) * C + L / 8 gives every XCD a
// contiguous range of units: the row groups of one KV split (numbered
// consecutively by the caller) then run on the same XCD at about the same
// time and share its L2 for the cache rows they all read. Ids whose unit is
// >= `units` have no work. Only locality depends on the dispatch order;
// every unit is covered exactly once whatever it is.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_unit(int units) {
  const int L = blockIdx.x;
  const int C = gridDim.x / kXcds;
  const int j = (L % kXcds) * C + L / kXcds;
  return j < units ? j : -1;
}
// Grid for `units` work units: 8 * C workgroups, C = max(ceil(units / 8), chunk).
inline unsigned xcd_grid(long units, long chunk = 0) {
  const long c = (units + kXcds - 1) / kXcds;
  return (unsigned)((c > chunk ? c : chunk) * kXcds);
}

// Sum / max over the 64 lanes, every lane getting the result, in VALU
// cross-lane moves only (no LDS permute): DPP swaps within quads, then
// mirrors within 8- and 16-lane rows (each pairs every lane with one of the
// other half, which is all a symmetric reduction needs), then the gfx950
// 16- and 32-lane swaps.
template <typename Op>
__device__ __forceinline__ int wave_reduce_i32(int v, Op op) {
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false));  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
  v = op((int)a[0], (int)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  return op((int)b[0], (int)b[1]);
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  return wave_reduce_i32(v, [](int x, int y) { return x + y; });
}
__device__ __forceinline__ int wave_max_i32(int v) {
  return wave_reduce_i32(v, [](int x, int y) { return max(x, y); });
}

// Split counts that follow the sequence lengths of a ragged batch (at most
// 64 sequences, one per lane). Sequence b, with n_b positions clamped to
// [0, slot_stride] and t_b = ceil(n_b / 32) tiles, gets
//   S_b = min(ceil(t_b / T), cap_b), at least 1,  cap_b = min(smax, ceil(t_b / 4)),
// where T is the smallest tile budget for which sum_b S_b <= units. Every
// split then holds about T tiles whichever sequence it belongs to, so the
// splits of a one-pass grid finish together instead of all waiting for the
// longest sequence; cap_b keeps at least 4 tiles per split, as the uniform
// rule does. sum_b S_b is non-increasing in T, and at most units already at
// T = ceil(sum_b t_b / (units - batch)) (each S_b <= t_b / T + 1) when
// units > batch, and at T = max_b t_b, where it equals the batch size; so a
// binary search below the smaller bound finds T whenever units >= batch
// (the host guarantees it). Computed from seq_lens alone, so the split and merge
// kernels agree without a table in memory. All 64 lanes must call it; lane b
// (< batch) gets S_b, the splits of sequences 0..b-1 in `first`, and its raw
// seq_lens entry in `len`; every lane gets the sum in `total`.
struct BalancedSplit {
  int count, first, total, len;
};
__device__ __forceinline__ BalancedSplit balanced_split(const int32_t* seq_lens, int batch, int slot_stride,
                                                        int smax, int units) {
  const int lane = (int)__lane_id();
  const bool live = lane < batch;
  const int len = live ? seq_lens[lane] : 0;
  const int n = min(max(len, 0), slot_stride);
  const int t = (n + 31) / 32;
  const int cap = live ? min(smax, max(1, (t + 3) / 4)) : 0;
  auto count = [&](int T) { return live ? min(cap, max(1, (t + T - 1) / T)) : 0; };
  const int tot = wave_sum_i32(t);
  int lo = 1, hi = max(1, wave_max_i32(t));
  if (units > batch) hi = min(hi, max(1, (tot + (units - batch) - 1) / (units - batch)));
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (wave_sum_i32(count(mid)) <= units) hi = mid;
    else lo = mid + 1;
  }
  const int c = count(lo);
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  return BalancedSplit{c, incl - c, __shfl(incl, 63), len};
}

}  // namespace mla
