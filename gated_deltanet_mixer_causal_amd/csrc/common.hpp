// Device helpers shared by the GDN kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---- scalar conversions --------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ __bf16 f32_to_bf16(float f) { return static_cast<__bf16>(f); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// fp32 value -> bf16 pair (hi, lo) with hi + lo == x to about 2^-17 relative.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

// ---- element traits for I/O dtypes ----------------------------------------

struct BF16 {
  using T = uint16_t;
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load(const T* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
  __device__ __forceinline__ static float cvt(T raw) { return bf16_bits_to_f32(raw); }
  __device__ __forceinline__ static void store(T* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
  // 8 consecutive elements (16 bytes) -> float[8]
  // 8 consecutive elements as raw bits (one 16-byte access)
  using Vec = uint4;
  __device__ __forceinline__ static Vec zero_vec() { return make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ static Vec ld_vec(const T* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ static void st_vec(T* p, Vec v) { *reinterpret_cast<uint4*>(p) = v; }
  __device__ __forceinline__ static void unpack8(Vec r, float* out) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void load8(const T* p, float* out) {
    const uint4 r = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void store8(T* p, const float* in) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16_bits(in[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16_bits(in[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

struct F32 {
  using T = float;
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float load(const T* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static float cvt(T raw) { return raw; }
  __device__ __forceinline__ static void store(T* p, int64_t i, float v) { p[i] = v; }
  struct Vec {
    float4 a, b;
  };
  __device__ __forceinline__ static Vec zero_vec() {
    return Vec{make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
  }
  __device__ __forceinline__ static Vec ld_vec(const T* p) {
    return Vec{reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
  }
  __device__ __forceinline__ static void st_vec(T* p, Vec v) {
    reinterpret_cast<float4*>(p)[0] = v.a;
    reinterpret_cast<float4*>(p)[1] = v.b;
  }
  __device__ __forceinline__ static void unpack8(Vec v, float* out) {
    out[0] = v.a.x; out[1] = v.a.y; out[2] = v.a.z; out[3] = v.a.w;
    out[4] = v.b.x; out[5] = v.b.y; out[6] = v.b.z; out[7] = v.b.w;
  }
  __device__ __forceinline__ static void load8(const T* p, float* out) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
  __device__ __forceinline__ static void store8(T* p, const float* in) {
    reinterpret_cast<float4*>(p)[0] = make_float4(in[0], in[1], in[2], in[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(in[4], in[5], in[6], in[7]);
  }
};

// SiLU with the hardware reciprocal (1 ulp) in place of an IEEE divide: the
// conv kernels, the norms and the fused prefill form it for every output, and
// the divide's ten-instruction sequence dominated the fused prefill's conv.
// Every kernel uses this one definition, so entry points that promise
// bit-identical results stay so.
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// One output of the width-4 causal conv with SiLU: taps w0..w3 against the
// three previous raw inputs h0 (oldest) .. h2 and the current one x.  The
// products are accumulated in this order with explicit fused multiply-adds,
// so every kernel that forms a conv output (the conv kernels, the one-launch
// decode mixer and the fused prefill) rounds it alike.
__device__ __forceinline__ float conv4_silu(float w0, float w1, float w2, float w3, float h0, float h1, float h2,
                                            float x) {
  float acc = w0 * h0;
  acc = __builtin_fmaf(w1, h1, acc);
  acc = __builtin_fmaf(w2, h2, acc);
  acc = __builtin_fmaf(w3, x, acc);
  return silu(acc);
}

// DPP row rotation: lane i of each row of 16 lanes reads lane (i - M) mod 16.
template <int M>
__device__ __forceinline__ float row_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x120 + M, 0xf, 0xf, false));
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64),
// every lane of each group active: the xor butterfly v += v[lane ^ m] for
// m = width/2 .. 1.  For width 16 (the rows of 16 lanes of the d = 128
// kernels) it runs on DPP row rotations by m instead of LDS crossbar
// shuffles, with the same result bit for bit: after the step of offset m the
// partial sums repeat with period m in the row, so the rotated partner
// (i - m) mod 16 holds the value of the xor partner i ^ m, and each addition
// takes the same two operands in the same order.
template <int width>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (width == 16) {
    v += row_ror<8>(v);
    v += row_ror<4>(v);
    v += row_ror<2>(v);
    v += row_ror<1>(v);
    return v;
  } else {
#pragma unroll
    for (int off = width / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, width);
    return v;
  }
}

// ---- arithmetic of one recurrent token --------------------------------------
//
// Every kernel that runs the plain recurrence of one token (the decode step,
// the verification columns, the one-launch decode mixer and the chunk path's
// one-token sequences) forms these quantities with the helpers below.  Each
// multiply-add is an explicit fused multiply-add and each other product is
// rounded on its own, so the kernels round alike whatever contractions the
// compiler would choose, and results that the interface promises to be
// bit-identical across entry points stay so.

// Partial sums of |k|^2, |q|^2 and k.q over one lane's 8 columns.
__device__ __forceinline__ void tok_sums8(const float* kk, const float* qq, float& sk, float& sq, float& kq) {
  sk = kk[0] * kk[0];
  sq = qq[0] * qq[0];
  kq = kk[0] * qq[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    sk = __builtin_fmaf(kk[i], kk[i], sk);
    sq = __builtin_fmaf(qq[i], qq[i], sq);
    kq = __builtin_fmaf(kk[i], qq[i], kq);
  }
}

// One lane's part of a state row (columns a: 4, b: 4) dotted with x[8].
__device__ __forceinline__ float tok_dot8(const float4& a, const float4& b, const float* x) {
  float s = a.x * x[0];
  s = __builtin_fmaf(a.y, x[1], s);
  s = __builtin_fmaf(a.z, x[2], s);
  s = __builtin_fmaf(a.w, x[3], s);
  s = __builtin_fmaf(b.x, x[4], s);
  s = __builtin_fmaf(b.y, x[5], s);
  s = __builtin_fmaf(b.z, x[6], s);
  return __builtin_fmaf(b.w, x[7], s);
}

// e = v - a (S k^)_row: the row's prediction error after the decay.
__device__ __forceinline__ float tok_err(float v, float alpha, float sk_row) {
  return __builtin_fmaf(-alpha, sk_row, v);
}

// o_row = scale (a (S q^)_row + (beta e) (k^ . q^)).
__device__ __forceinline__ float tok_out(float scale, float alpha, float sq_row, float be, float kq) {
  return scale * __builtin_fmaf(kq, be, alpha * sq_row);
}

// New state element a s + (beta e) k^_col.
__device__ __forceinline__ float tok_upd(float alpha, float s, float be, float kcol) {
  return __builtin_fmaf(be, kcol, alpha * s);
}
__device__ __forceinline__ float4 tok_upd4(float alpha, const float4& s, float be, const float* kc) {
  return make_float4(tok_upd(alpha, s.x, be, kc[0]), tok_upd(alpha, s.y, be, kc[1]),
                     tok_upd(alpha, s.z, be, kc[2]), tok_upd(alpha, s.w, be, kc[3]));
}

// 1 / sqrt(mean of the d squares + eps) from their sum.
__device__ __forceinline__ float norm_rinv(float sum_sq, float inv_d, float eps) {
  return 1.0f / sqrtf(__builtin_fmaf(sum_sq, inv_d, eps));
}

// ---- per-(token, v-head) gates ---------------------------------------------

// Where the log-decay g and the write strength beta of the gated delta rule
// come from: fp32 tensors g, beta [rows][h_v] (a == nullptr), or the raw
// outputs a, b of the gate projections (row stride ab_stride elements, bf16
// or fp32) with per-v-head a_log and an optional dt_bias, from which
//     g = -exp(a_log[h]) * softplus(a + dt_bias[h]),   beta = sigmoid(b)
// (the B/A gate projections of the GDN mixer: Flare core-design, fused
// projection weights paragraph).  Plain data, passed to kernels by value.
struct GateSrc {
  const float* g;
  const float* beta;
  const void* a;
  const void* b;
  int64_t ab_stride;
  int ab_bf16;
  const float* a_log;
  const float* dt_bias;
};

// The raw gate inputs of token row t, v-head h: the bits of g and beta, or of
// the two gate projections (a bf16 value zero-extended).  Nothing here uses
// the loaded values, so a caller can keep the loads in flight across other
// work and convert later with gate_from_raw.
__device__ __forceinline__ void gate_load_raw(const GateSrc& s, int64_t t, int h, int h_v, uint32_t& ra,
                                              uint32_t& rb) {
  if (s.a == nullptr) {
    const int64_t i = t * h_v + h;
    ra = __float_as_uint(s.g[i]);
    rb = __float_as_uint(s.beta[i]);
  } else if (s.ab_bf16) {
    const int64_t i = t * s.ab_stride + h;
    ra = static_cast<const uint16_t*>(s.a)[i];
    rb = static_cast<const uint16_t*>(s.b)[i];
  } else {
    const int64_t i = t * s.ab_stride + h;
    ra = __float_as_uint(static_cast<const float*>(s.a)[i]);
    rb = __float_as_uint(static_cast<const float*>(s.b)[i]);
  }
}

// g and beta from the raw inputs of v-head h.  softplus(x) is evaluated as
// max(x, 0) + log1p(exp(-|x|)) and sigmoid(x) through exp(-|x|), so no
// exponential overflows for any finite input.
__device__ __forceinline__ void gate_from_raw(const GateSrc& s, int h, uint32_t ra, uint32_t rb, float& g,
                                              float& beta) {
  if (s.a == nullptr) {
    g = __uint_as_float(ra);
    beta = __uint_as_float(rb);
    return;
  }
  const float av = s.ab_bf16 ? __uint_as_float(ra << 16) : __uint_as_float(ra);
  const float bv = s.ab_bf16 ? __uint_as_float(rb << 16) : __uint_as_float(rb);
  const float x = av + (s.dt_bias ? s.dt_bias[h] : 0.f);
  const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
  g = -expf(s.a_log[h]) * sp;
  const float e = expf(-fabsf(bv));
  beta = bv >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

// g and beta of token row t, v-head h.
__device__ __forceinline__ void load_gate(const GateSrc& s, int64_t t, int h, int h_v, float& g, float& beta) {
  uint32_t ra, rb;
  gate_load_raw(s, t, h, h_v, ra, rb);
  gate_from_raw(s, h, ra, rb, g, beta);
}

// Sequence of a token-block slot.  Block j of sequence s (blocks of `blk`
// tokens restarting at each sequence start) is given slot
//     floor(cu[s] / blk) + s + j,
// which is strictly increasing over (s, j) and stays below
// ceil(t_total / blk) + n_seq, so a grid of that many blocks covers every
// block with no host-side knowledge of the lengths.  Returns false for an
// idle slot.
__device__ __forceinline__ int64_t seq_start(const int32_t* cu, int s, int64_t t_total) {
  return cu ? static_cast<int64_t>(cu[s]) : (s == 0 ? 0 : t_total);
}

// cu == nullptr means a single sequence of t_total tokens.
__device__ __forceinline__ bool locate_block(const int32_t* cu, int n_seq, int64_t t_total, int blk,
                                             int64_t slot, int& seq, int64_t& t0, int& len) {
  // largest s in [0, n_seq) with floor(cu[s]/blk) + s <= slot
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seq_start(cu, mid, t_total) / blk + mid <= slot) lo = mid; else hi = mid - 1;
  }
  const int64_t start = seq_start(cu, lo, t_total), end = seq_start(cu, lo + 1, t_total);
  const int64_t j = slot - (start / blk + lo);
  if (j < 0) return false;
  t0 = start + j * blk;
  if (t0 >= end) return false;
  seq = lo;
  len = static_cast<int>(end - t0 < blk ? end - t0 : blk);
  return true;
}

// The zero-length sequence whose (only) slot is `slot`, or -1.  Slot keys
// floor(cu[s]/blk) + s strictly increase with s, so at most one sequence
// has key == slot.
__device__ __forceinline__ int empty_seq_at(const int32_t* cu, int n_seq, int64_t t_total, int blk, int64_t slot) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seq_start(cu, mid, t_total) / blk + mid <= slot) lo = mid; else hi = mid - 1;
  }
  const int64_t start = seq_start(cu, lo, t_total);
  if (start / blk + lo != slot || seq_start(cu, lo + 1, t_total) != start) return -1;
  return lo;
}

__host__ __device__ constexpr int64_t block_slots(int64_t t_total, int n_seq, int blk) {
  return (t_total + blk - 1) / blk + n_seq;
}

// XCD-aware order.  The dispatcher hands workgroup b of a 1-D grid to XCD
// b % 8, and each of the 8 XCDs has its own L2.  This bijection of [0, n)
// gives XCD x the contiguous logical range [start(x), start(x) + count(x)),
// so logical neighbours (which share operands) run under one L2.
__device__ __forceinline__ int64_t xcd_order(int64_t b, int64_t n) {
  const int64_t x = b % 8, r = b / 8, q = n / 8, m = n % 8;
  return x * q + (x < m ? x : m) + r;
}

}  // namespace gdn
