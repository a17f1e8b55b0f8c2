// Causal depthwise conv1d of width 4 + SiLU over packed sequences (gfx950).
//
// Output token t of sequence s is SiLU(sum_i w[c][i] * padded[t - start + i][c])
// where padded = [history(3 raw inputs, oldest first); x_s]; the history is
// then replaced by the last three rows of padded (haskell-infer-demo README,
// "Architecture", width-4 causal-conv1d; Flare core-design, short-convolution
// paragraph and its prepared-interface list: raw projected QKV, dilation 1,
// SiLU, caller-owned raw-input history, slot mapping, inactive lanes).
//
// Prefill: one workgroup per (block of 8 tokens of one sequence, 512
// channels); each thread owns 2 adjacent channels (one 4-byte access per
// token for bf16) and issues the loads of all 11 rows it reads (3 before the
// block, 8 in it) before computing, so the whole input is in flight at
// once.  Two channels per thread keep the register count low enough for
// twice the resident workgroups of eight channels per thread, which measured
// 27.5 against 32-33 us at 4096 tokens x 8192 channels (4-channel threads
// 28-30 us; 8-token blocks faster than 4, 12 or 16).  Blocks are ordered so that consecutive token blocks of a channel
// slice run on one XCD, where the 3-row halo a block re-reads from its
// predecessor is an L2 hit.  Blocks never straddle sequences (slots from
// common.hpp), which keeps the history reads inside the first block of each
// sequence: that block alone reads the old history and writes the new one,
// so the in-place update needs no second pass.
// Decode (one token per sequence): one thread per (sequence, 8 channels).
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

constexpr int kConvBT = 8;             // tokens per prefill block (>= 3)
constexpr int kConvThreads = 256;
constexpr int kConvVec = 2;            // channels per prefill thread
constexpr int kConvChP = kConvThreads * kConvVec;   // channels per prefill workgroup

// kConvVec consecutive channels of one row, as raw elements (one access).
template <class E>
struct ConvRow {
  typedef typename E::T V __attribute__((ext_vector_type(kConvVec)));
  __device__ __forceinline__ static V ld(const typename E::T* p) { return *reinterpret_cast<const V*>(p); }
  __device__ __forceinline__ static void st(typename E::T* p, V v) { *reinterpret_cast<V*>(p) = v; }
  __device__ __forceinline__ static V zero() { return V{}; }
};
__device__ __forceinline__ uint16_t to_elem(float v, uint16_t) { return f32_to_bf16_bits(v); }
__device__ __forceinline__ float to_elem(float v, float) { return v; }

template <class E>
__device__ __forceinline__ void load_taps(const typename E::T* w, int c0, float (&wt)[4][8]) {
  float tmp[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) E::load8(w + static_cast<int64_t>(c0) * 4 + 8 * i, tmp + 8 * i);
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) wt[i][c] = tmp[4 * c + i];
}

__device__ __forceinline__ void conv_out(const float (&wt)[4][8], const float (&w0)[8], const float (&w1)[8],
                                         const float (&w2)[8], const float (&cur)[8], float (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    out[c] = conv4_silu(wt[0][c], wt[1][c], wt[2][c], wt[3][c], w0[c], w1[c], w2[c], cur[c]);
  }
}

template <class E>
__global__ __launch_bounds__(kConvThreads) void k_conv1d_prefill(
    const typename E::T* __restrict__ x, const typename E::T* __restrict__ w, int channels,
    const int32_t* __restrict__ cu, int n_seq, int64_t t_total, typename E::T* __restrict__ state,
    const int32_t* __restrict__ slots, const int32_t* __restrict__ fresh, typename E::T* __restrict__ y,
    int64_t n_tblk, int n_slices) {
  using T = typename E::T;
  using R = ConvRow<E>;
  constexpr int NV = kConvVec;
  const int64_t lid = xcd_order(blockIdx.x, n_tblk * n_slices);
  const int slice = static_cast<int>(lid / n_tblk);
  const int64_t tblk = lid % n_tblk;
  const int c0 = (slice * kConvThreads + threadIdx.x) * NV;
  if (c0 >= channels) return;
  int seq, len;
  int64_t t0;
  if (!locate_block(cu, n_seq, t_total, kConvBT, tblk, seq, t0, len)) {
    // a fresh zero-length sequence: its history becomes zeros
    if (fresh) {
      const int es = empty_seq_at(cu, n_seq, t_total, kConvBT, tblk);
      const int es_slot = es < 0 ? -1 : (slots ? slots[es] : es);
      if (es_slot >= 0 && fresh[es] != 0) {
        T* h = state + static_cast<int64_t>(es_slot) * 3 * channels + c0;
#pragma unroll
        for (int r = 0; r < 3; ++r) R::st(h + r * static_cast<int64_t>(channels), R::zero());
      }
    }
    return;
  }
  const int slot = slots ? slots[seq] : seq;
  if (slot < 0) return;
  const int64_t start = cu[seq];
  const int64_t p0 = t0 - start;
  const int64_t ld = channels;
  T* hist = state + static_cast<int64_t>(slot) * 3 * ld + c0;

  // every row this thread reads: raw inputs at local positions p0-3 .. p0-1
  // (history rows in the first block; zeros for a fresh sequence, whose
  // history is not read) and the block's own rows (rows past the block's end
  // re-read its last row and are not used)
  // All 11 loads are unconditional (the source of a row before the block is
  // a pointer select) and a fresh sequence's history rows are zeroed after
  // their load: a load under a branch made the compiler wait for it at the
  // join, which serialised the three rows before the block and the block's
  // own rows into four memory round trips per workgroup.
  typename R::V raw[3 + kConvBT];
  const bool zero_hist = p0 < 3 && fresh != nullptr && fresh[seq] != 0;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int64_t lp = p0 - 3 + r;
    raw[r] = R::ld(lp >= 0 ? x + (start + lp) * ld + c0 : hist + (3 + lp) * ld);
  }
#pragma unroll
  for (int u = 0; u < kConvBT; ++u) raw[3 + u] = R::ld(x + (t0 + (u < len ? u : len - 1)) * ld + c0);
#pragma unroll
  for (int r = 0; r < 3; ++r)
    if (p0 - 3 + r < 0 && zero_hist) raw[r] = R::zero();
  float wt[4][NV];
  {
    // taps of the thread's channels: w[c][0..3], channel-major
    typedef T W8 __attribute__((ext_vector_type(4 * NV)));
    const W8 wr = *reinterpret_cast<const W8*>(w + static_cast<int64_t>(c0) * 4);
#pragma unroll
    for (int c = 0; c < NV; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) wt[i][c] = E::cvt(wr[4 * c + i]);
  }

  float h0[NV], h1[NV], h2[NV];
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    h0[c] = E::cvt(raw[0][c]);
    h1[c] = E::cvt(raw[1][c]);
    h2[c] = E::cvt(raw[2][c]);
  }
#pragma unroll
  for (int u = 0; u < kConvBT; ++u) {
    if (u < len) {
      typename R::V o;
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        const float cur = E::cvt(raw[3 + u][c]);
        o[c] = to_elem(conv4_silu(wt[0][c], wt[1][c], wt[2][c], wt[3][c], h0[c], h1[c], h2[c], cur), T{});
        h0[c] = h1[c];
        h1[c] = h2[c];
        h2[c] = cur;
      }
      // plain stores: the chunk kernels read y right after, from cache
      // (non-temporal stores made this kernel 1.2 us faster and the scan,
      // which reads v from y a step ahead, 5 us slower)
      R::st(y + (t0 + u) * ld + c0, o);
    }
  }

  if (p0 == 0) {
    // new history row r = padded[L + r] with padded = [old history; x_s];
    // raw[0..2] still hold the old history in the first block
    const int64_t L = cu[seq + 1] - start;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int64_t idx = L + r;
      typename R::V row;
      if (idx >= 3) row = R::ld(x + (start + idx - 3) * ld + c0);
      else row = idx == 0 ? raw[0] : (idx == 1 ? raw[1] : raw[2]);   // constant indices keep raw in registers
      R::st(hist + r * ld, row);
    }
  }
}

template <class E>
__global__ __launch_bounds__(kConvThreads) void k_conv1d_step(
    const typename E::T* __restrict__ x, const typename E::T* __restrict__ w, int channels, int n_seq,
    typename E::T* __restrict__ state, const int32_t* __restrict__ slots, typename E::T* __restrict__ y) {
  using T = typename E::T;
  const int groups = channels / 8;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kConvThreads + threadIdx.x;
  const int64_t s = gid / groups;
  if (s >= n_seq) return;
  const int c0 = static_cast<int>(gid % groups) * 8;
  const int slot = slots ? slots[s] : static_cast<int>(s);
  if (slot < 0) return;
  const int64_t ld = channels;
  float wt[4][8];
  load_taps<E>(w, c0, wt);
  T* hist = state + static_cast<int64_t>(slot) * 3 * ld + c0;
  float h0[8], h1[8], h2[8], cur[8], out[8];
  E::load8(hist, h0);
  E::load8(hist + ld, h1);
  E::load8(hist + 2 * ld, h2);
  E::load8(x + s * ld + c0, cur);
  conv_out(wt, h0, h1, h2, cur, out);
  E::store8(y + s * ld + c0, out);
  E::store8(hist, h1);
  E::store8(hist + ld, h2);
  E::store8(hist + 2 * ld, cur);
}

// Speculative verification: n_tok tokens per request (rows s n_tok .. s n_tok +
// n_tok - 1 of x and y) from the live history of the request's slot, which is
// only read.  The history after token t (its last three raw inputs) is
// written to column t of the window store, windows[slot][t][0..2][c], as the
// three-token convolution window of that checkpoint column (Flare
// core-design, speculative target state).  A negative slot is an inactive
// lane: nothing is read or written.
template <class E>
__global__ __launch_bounds__(kConvThreads) void k_conv1d_verify(
    const typename E::T* __restrict__ x, const typename E::T* __restrict__ w, int channels, int n_seq,
    int n_tok, const typename E::T* __restrict__ state, const int32_t* __restrict__ slots,
    typename E::T* __restrict__ y, typename E::T* __restrict__ windows, int n_cols) {
  const int groups = channels / 8;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kConvThreads + threadIdx.x;
  const int64_t s = gid / groups;
  if (s >= n_seq) return;
  const int c0 = static_cast<int>(gid % groups) * 8;
  const int slot = slots ? slots[s] : static_cast<int>(s);
  if (slot < 0) return;
  const int64_t ld = channels;
  float wt[4][8];
  load_taps<E>(w, c0, wt);
  const typename E::T* hist = state + static_cast<int64_t>(slot) * 3 * ld + c0;
  float h0[8], h1[8], h2[8], cur[8], out[8];
  E::load8(hist, h0);
  E::load8(hist + ld, h1);
  E::load8(hist + 2 * ld, h2);
  for (int t = 0; t < n_tok; ++t) {
    const int64_t row = s * n_tok + t;
    E::load8(x + row * ld + c0, cur);
    conv_out(wt, h0, h1, h2, cur, out);
    E::store8(y + row * ld + c0, out);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h0[i] = h1[i];
      h1[i] = h2[i];
      h2[i] = cur[i];
    }
    typename E::T* win = windows + (static_cast<int64_t>(slot) * n_cols + t) * 3 * ld + c0;
    E::store8(win, h0);
    E::store8(win + ld, h1);
    E::store8(win + 2 * ld, h2);
  }
}

template <class E>
static hipError_t run_conv(const void* x, const void* w, int channels, const int32_t* cu, int n_seq,
                           int64_t t_total, void* state, const int32_t* slots, void* y, hipStream_t st,
                           const int32_t* fresh) {
  using T = typename E::T;
  if (cu) {
    const int64_t ntblk = block_slots(t_total, n_seq, kConvBT);
    const int nslices = (channels + kConvChP - 1) / kConvChP;
    hipLaunchKernelGGL((k_conv1d_prefill<E>), dim3(static_cast<unsigned>(ntblk * nslices)), dim3(kConvThreads), 0, st,
                       static_cast<const T*>(x), static_cast<const T*>(w), channels, cu, n_seq, t_total,
                       static_cast<T*>(state), slots, fresh, static_cast<T*>(y), ntblk, nslices);
  } else {
    const int64_t threads = static_cast<int64_t>(n_seq) * (channels / 8);
    const unsigned blocks = static_cast<unsigned>((threads + kConvThreads - 1) / kConvThreads);
    hipLaunchKernelGGL((k_conv1d_step<E>), dim3(blocks), dim3(kConvThreads), 0, st, static_cast<const T*>(x),
                       static_cast<const T*>(w), channels, n_seq, static_cast<T*>(state), slots,
                       static_cast<T*>(y));
  }
  return hipGetLastError();
}

template <class E>
static hipError_t run_conv_verify(const void* x, const void* w, int channels, int n_seq, int n_tok, const void* state,
                                  const int32_t* slots, void* y, void* windows, int n_cols, hipStream_t st) {
  using T = typename E::T;
  const int64_t threads = static_cast<int64_t>(n_seq) * (channels / 8);
  const unsigned blocks = static_cast<unsigned>((threads + kConvThreads - 1) / kConvThreads);
  hipLaunchKernelGGL((k_conv1d_verify<E>), dim3(blocks), dim3(kConvThreads), 0, st, static_cast<const T*>(x),
                     static_cast<const T*>(w), channels, n_seq, n_tok, static_cast<const T*>(state), slots,
                     static_cast<T*>(y), static_cast<T*>(windows), n_cols);
  return hipGetLastError();
}

hipError_t launch_conv1d_verify(const void* x, gdn_dtype dt, const void* w, int channels, int n_seq, int n_tok,
                                const void* state, const int32_t* slots, void* y, void* windows, int n_cols,
                                void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == GDN_BF16) return run_conv_verify<BF16>(x, w, channels, n_seq, n_tok, state, slots, y, windows, n_cols, st);
  return run_conv_verify<F32>(x, w, channels, n_seq, n_tok, state, slots, y, windows, n_cols, st);
}

hipError_t launch_conv1d(const void* x, gdn_dtype dt, const void* w, int channels, const int32_t* cu,
                         int n_seq, int64_t t_total, void* state, const int32_t* slots, void* y,
                         void* stream, const int32_t* fresh) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == GDN_BF16) return run_conv<BF16>(x, w, channels, cu, n_seq, t_total, state, slots, y, st, fresh);
  return run_conv<F32>(x, w, channels, cu, n_seq, t_total, state, slots, y, st, fresh);
}

}  // namespace gdn
