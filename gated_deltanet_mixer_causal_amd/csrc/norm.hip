// Gated RMSNorm epilogue (gfx950):
//     y = x / sqrt(mean(x^2) + eps) * w * SiLU(z)   per row of d elements
// (the gated RMSNorm of the GDN layers: haskell-infer-demo README,
// "Highlights" and "Architecture"/gdn_norm.cu).  Each thread owns 8 adjacent
// elements (one 16-byte vector of bf16); the d/8 threads of a row reduce the
// sum of squares with lane shuffles, so a row is read and written once.
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

// Optional row mask of the epilogue (see row_active).
struct RowMask {
  const int32_t* cu;
  int n_seq;
  const int32_t* slots;
  int h_v;
};

// With a row mask (cu != nullptr) the rows are (token, head) pairs of packed
// sequences, h_v rows per token: a row is normalised only when its token lies
// in a sequence whose slot is not negative; rows of inactive sequences and
// padding rows past cu[n_seq] keep their contents.
__device__ __forceinline__ bool row_active(int64_t row, const int32_t* __restrict__ cu, int n_seq,
                                           const int32_t* __restrict__ slots, int h_v) {
  const int64_t t = row / h_v;
  if (n_seq <= 0 || t < cu[0] || t >= cu[n_seq]) return false;
  int lo = 0, hi = n_seq - 1;   // last sequence whose start is <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return slots[lo] >= 0;
}

template <class EX, class EZ, class EY, int D>
__global__ __launch_bounds__(256) void k_gated_rmsnorm(const typename EX::T* x,
                                                      const typename EZ::T* __restrict__ z,
                                                      const float* __restrict__ w, float eps, int64_t rows,
                                                      typename EY::T* y, const int32_t* __restrict__ cu,
                                                      int n_seq, const int32_t* __restrict__ slots, int h_v) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / TPR;
  const int c0 = (threadIdx.x % TPR) * 8;
  const bool valid = row < rows && (cu == nullptr || row_active(row, cu, n_seq, slots, h_v));
  float xv[8] = {0, 0, 0, 0, 0, 0, 0, 0}, zv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (valid) {
    EX::load8(x + row * D + c0, xv);
    EZ::load8(z + row * D + c0, zv);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += xv[i] * xv[i];
  ss = group_sum<TPR>(ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / D) + eps);
  if (valid) {
    float out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = xv[i] * r * w[c0 + i] * silu(zv[i]);
    EY::store8(y + row * D + c0, out);
  }
}

template <class EX, class EZ, class EY>
static hipError_t run_norm(const void* x, const void* z, const float* w, float eps, int64_t rows, int d, void* y,
                           hipStream_t st, const RowMask& m) {
  using TX = typename EX::T;
  using TZ = typename EZ::T;
  using TY = typename EY::T;
  if (d == 128) {
    const unsigned blocks = static_cast<unsigned>((rows + 15) / 16);
    hipLaunchKernelGGL((k_gated_rmsnorm<EX, EZ, EY, 128>), dim3(blocks), dim3(256), 0, st,
                       static_cast<const TX*>(x), static_cast<const TZ*>(z), w, eps, rows, static_cast<TY*>(y), m.cu,
                       m.n_seq, m.slots, m.h_v);
  } else {
    const unsigned blocks = static_cast<unsigned>((rows + 127) / 128);
    hipLaunchKernelGGL((k_gated_rmsnorm<EX, EZ, EY, 16>), dim3(blocks), dim3(256), 0, st,
                       static_cast<const TX*>(x), static_cast<const TZ*>(z), w, eps, rows, static_cast<TY*>(y), m.cu,
                       m.n_seq, m.slots, m.h_v);
  }
  return hipGetLastError();
}

template <class EX, class EZ>
static hipError_t run_norm_y(const void* x, const void* z, const float* w, float eps, int64_t rows, int d, void* y,
                             gdn_dtype y_dt, hipStream_t st, const RowMask& m) {
  if (y_dt == GDN_BF16) return run_norm<EX, EZ, BF16>(x, z, w, eps, rows, d, y, st, m);
  return run_norm<EX, EZ, F32>(x, z, w, eps, rows, d, y, st, m);
}

template <class EX>
static hipError_t run_norm_z(const void* x, const void* z, gdn_dtype z_dt, const float* w, float eps, int64_t rows,
                             int d, void* y, gdn_dtype y_dt, hipStream_t st, const RowMask& m) {
  if (z_dt == GDN_BF16) return run_norm_y<EX, BF16>(x, z, w, eps, rows, d, y, y_dt, st, m);
  return run_norm_y<EX, F32>(x, z, w, eps, rows, d, y, y_dt, st, m);
}

hipError_t launch_gated_rmsnorm(const void* x, gdn_dtype x_dt, const void* z, gdn_dtype z_dt, const float* w,
                                float eps, int64_t rows, int d, void* y, gdn_dtype y_dt, void* stream,
                                const int32_t* cu, int n_seq, const int32_t* slots, int h_v) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rows == 0) return hipSuccess;
  const RowMask m{cu, n_seq, slots, h_v};
  if (x_dt == GDN_BF16) return run_norm_z<BF16>(x, z, z_dt, w, eps, rows, d, y, y_dt, st, m);
  return run_norm_z<F32>(x, z, z_dt, w, eps, rows, d, y, y_dt, st, m);
}

}  // namespace gdn
