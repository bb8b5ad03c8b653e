// Draft-KV append: the q_len new tokens of every sequence are written into
// the page_size = 1 latent pool through the slot table, the step that
// precedes a verify call (the verify reads the drafts' rows from the cache
// at positions seq_len - q_len .. seq_len - 1).
//
// A pure copy, bound by HBM: each row is 1152 bytes = 72 pieces of 16 bytes;
// consecutive threads take consecutive pieces of a row, so every wavefront
// moves whole contiguous runs of a source row and of its pool row.
#include "device_common.h"
#include "mla_internal.h"
#include "mla_verify.h"

namespace mla {
namespace {

constexpr int kRowPieces16 = kDk * 2 / 16;  // 72

__global__ __launch_bounds__(256) void append_kernel(char* latent, int64_t pool_rows, int slot_stride,
                                                     const char* new_rows, int batch, int q_len,
                                                     const int32_t* slots, const int32_t* seq_lens, unsigned* err) {
  const int64_t total = (int64_t)batch * q_len * kRowPieces16;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / kRowPieces16;  // source row = b * q_len + i
    const int p = (int)(t - r * kRowPieces16);
    const int b = (int)(r / q_len), i = (int)(r - (int64_t)b * q_len);
    const int n = seq_lens[b];
    if (n < q_len || n > slot_stride) {
      if (i == 0 && p == 0) flag_error(err, MLA_DEVERR_SEQ_LEN);
      continue;
    }
    const int32_t s = slots[(size_t)b * slot_stride + (n - q_len + i)];
    if (s < 0 || (int64_t)s >= pool_rows) {
      if (p == 0) flag_error(err, MLA_DEVERR_SLOT_RANGE);
      continue;
    }
    const f32x4 v = *reinterpret_cast<const f32x4*>(new_rows + r * (kDk * 2) + 16 * p);
    *reinterpret_cast<f32x4*>(latent + (int64_t)s * (kDk * 2) + 16 * p) = v;
  }
}

}  // namespace

hipError_t launch_append(void* latent, int64_t pool_rows, int slot_stride, const void* new_rows, int batch,
                         int q_len, const int32_t* slots, const int32_t* seq_lens, unsigned* err,
                         hipStream_t stream) {
  const int64_t total = (int64_t)batch * q_len * kRowPieces16;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream,
                     static_cast<char*>(latent), pool_rows, slot_stride, static_cast<const char*>(new_rows), batch,
                     q_len, slots, seq_lens, err);
  return hipGetLastError();
}

}  // namespace mla
