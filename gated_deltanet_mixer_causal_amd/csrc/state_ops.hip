// State maintenance: an indirect row copy driven by device-resident row
// indices (Flare core-design, the prepared state operations: initialize,
// restore, snapshot and reset, each an indirect copy kernel over slot-index
// buffers; state maintenance installs a snapshot or a checkpoint column in a
// live slot or freezes a live slot into a snapshot).
//
// Rows are opaque byte blocks of row_bytes (a multiple of 16): a per-request
// recurrent state, one checkpoint column, a conv history.  The copy is exact
// (plain 16-byte moves).
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

constexpr int kCopyThreads = 256;
constexpr int kCopyVecPerThread = 4;
constexpr int64_t kCopyChunk = int64_t(kCopyThreads) * kCopyVecPerThread;   // 16-byte vectors per block

// Block b copies chunk b % chunks of entry b / chunks: dst row dst_rows[e] <-
// src row src_rows[e], or <- zeros when src is null.  An index outside
// [0, rows) of its buffer skips the entry, so no access leaves the buffers.
__global__ __launch_bounds__(kCopyThreads) void k_rows_copy(uint4* __restrict__ dst, int64_t n_dst,
                                                            const int32_t* __restrict__ dst_rows,
                                                            const uint4* __restrict__ src, int64_t n_src,
                                                            const int32_t* __restrict__ src_rows, int64_t row_vec,
                                                            int64_t chunks) {
  const int64_t b = blockIdx.x;
  const int64_t e = b / chunks, c = b % chunks;
  const int64_t dr = dst_rows[e];
  if (dr < 0 || dr >= n_dst) return;
  int64_t sr = 0;
  if (src) {
    sr = src_rows[e];
    if (sr < 0 || sr >= n_src) return;
  }
#pragma unroll
  for (int j = 0; j < kCopyVecPerThread; ++j) {
    const int64_t idx = c * kCopyChunk + j * kCopyThreads + threadIdx.x;
    if (idx < row_vec) dst[dr * row_vec + idx] = src ? src[sr * row_vec + idx] : make_uint4(0u, 0u, 0u, 0u);
  }
}

hipError_t launch_rows_copy(void* dst, int64_t n_dst, const int32_t* dst_rows, const void* src, int64_t n_src,
                            const int32_t* src_rows, int64_t row_bytes, int n, void* stream) {
  const int64_t row_vec = row_bytes / 16;
  const int64_t chunks = (row_vec + kCopyChunk - 1) / kCopyChunk;
  const int64_t blocks = chunks * n;
  hipLaunchKernelGGL(k_rows_copy, dim3(static_cast<unsigned>(blocks)), dim3(kCopyThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(dst), n_dst, dst_rows,
                     static_cast<const uint4*>(src), n_src, src_rows, row_vec, chunks);
  return hipGetLastError();
}

}  // namespace gdn
