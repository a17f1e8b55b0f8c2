// Recurrent decode step of the gated delta rule (gfx950).
//
// One token per request; per (request, v-head) the fp32 state S (d_v x d_k)
// is read once, updated and written once:
//     a = exp(g),  e_i = v_i - a (S k^)_i,  S <- a S + beta e k^^T,
//     o_i = scale (S_new q^)_i = scale (a (S q^)_i + beta e_i (k^ . q^))
// which is the rule S_t = a S (I - beta k k^T) + beta v k^T, o_t = scale S_t q_t
// (haskell-infer-demo README, "Architecture"/fla_gdn.cu recurrent decode;
// FP32 recurrent state: Flare core-design, Qwen defaults table).
//
// The step is bound by HBM: 2 x d_v x d_k x 4 bytes of state per (request,
// head) against ~4 flops per state element.  One workgroup per (request,
// head); a state row of d_k floats is split over d_k/8 lanes as two 16-byte
// vectors at columns 4l and d_k/2 + 4l, so the lanes of a row read 2 x 256
// contiguous bytes; every thread issues all its state loads before any use,
// keeping 64 KiB per workgroup in flight.  Both row dot products (S k^ and
// S q^) come from the same registers, reduced across the row's lanes.
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

// State rows are streamed with non-temporal loads and stores: each is touched
// once per step, and keeping them out of the caches measured 17% faster
// (5.6 TB/s against 4.8 TB/s for 64 requests).
typedef float nt_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 stream_load4(const float* p) {
  const nt_f4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void stream_store4(float* p, float4 v) {
  __builtin_nontemporal_store(nt_f4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_f4*>(p));
}

template <class E>
__device__ __forceinline__ void load4(const typename E::T* p, float* out);
template <>
__device__ __forceinline__ void load4<BF16>(const uint16_t* p, float* out) {
  const uint2 r = *reinterpret_cast<const uint2*>(p);
  out[0] = __uint_as_float(r.x << 16);
  out[1] = __uint_as_float(r.x & 0xffff0000u);
  out[2] = __uint_as_float(r.y << 16);
  out[3] = __uint_as_float(r.y & 0xffff0000u);
}
template <>
__device__ __forceinline__ void load4<F32>(const float* p, float* out) {
  const float4 r = *reinterpret_cast<const float4*>(p);
  out[0] = r.x; out[1] = r.y; out[2] = r.z; out[3] = r.w;
}

// SPLIT workgroups share the D state rows of one (request, head), D / SPLIT
// rows each; rows are independent, so only the fused norm (a sum over all D
// outputs) needs them in one workgroup and runs with SPLIT == 1.  Two rows per
// thread (64 bytes of state in flight per lane) in workgroups of 256 threads
// measured fastest at 64 requests x 32 heads: 43.4 us per step (6.18 TB/s)
// with SPLIT = 4, against 47.8 us for eight rows per thread in one 256-thread
// workgroup per head.  With the fused norm, one 1024-thread workgroup per
// head (two rows per thread) made the decode mixer step slower (55.6 against
// 52.7 us), so that case keeps eight rows per thread.
template <class E, class EO, int D, int NT, int SPLIT>
__global__ __launch_bounds__(NT) void k_recurrent_step(
    const typename E::T* __restrict__ q, const typename E::T* __restrict__ k, const typename E::T* __restrict__ v,
    int64_t q_stride, int64_t k_stride, int64_t v_stride, GateSrc gates, float scale, int use_l2,
    float l2_eps, int h_qk, int h_v,
    float* __restrict__ state, const int32_t* __restrict__ slots, typename EO::T* __restrict__ o,
    const typename E::T* __restrict__ z, const float* __restrict__ norm_w, float norm_eps) {
  constexpr int TPR = D / 8;                 // lanes per state row
  constexpr int RPP = NT / TPR;              // rows per pass
  constexpr int RW = D / SPLIT;              // rows of this workgroup
  constexpr int PASSES = (RW + RPP - 1) / RPP;
  static_assert(TPR <= 64 && NT % 64 == 0, "row lanes within a wave");
  static_assert(D % SPLIT == 0, "equal row parts");

  const int part = static_cast<int>(blockIdx.x % SPLIT);
  const int rh = static_cast<int>(blockIdx.x / SPLIT);
  const int r = rh / h_v, h = rh % h_v;
  const int slot = slots ? slots[r] : r;
  if (slot < 0) return;
  const int hq = h / (h_v / h_qk);
  const int tid = threadIdx.x, l = tid % TPR, rg = tid / TPR;
  const int ca = 4 * l, cb = D / 2 + 4 * l;
  const int row0 = part * RW;

  constexpr bool FULL = RPP * PASSES == RW;   // every pass row is a state row
  float* S = state + (static_cast<int64_t>(slot) * h_v + h) * D * D;
  // Issue every load of the step before any use: the state rows of this
  // thread, its q/k columns and the v entries of its rows.  Rows beyond the
  // part (small heads) read its first row and are discarded.
  float4 sa[PASSES], sb[PASSES];
  typename E::T vraw[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = row0 + rg + p * RPP;
    const int rr = (FULL || rg + p * RPP < RW) ? row : row0;
    sa[p] = stream_load4(S + rr * D + ca);
    sb[p] = stream_load4(S + rr * D + cb);
    vraw[p] = v[r * v_stride + h * D + rr];
  }

  float kk[8], qq[8];
  load4<E>(k + r * k_stride + hq * D + ca, kk);
  load4<E>(k + r * k_stride + hq * D + cb, kk + 4);
  load4<E>(q + r * q_stride + hq * D + ca, qq);
  load4<E>(q + r * q_stride + hq * D + cb, qq + 4);
  float gv, bt;
  load_gate(gates, r, h, h_v, gv, bt);
  const int64_t obase = (static_cast<int64_t>(r) * h_v + h) * D;
  // gate of the fused norm, loaded with everything else (thread tid owns row tid)
  typename E::T zraw = 0;
  if (z) zraw = z[obase + (tid < D ? tid : 0)];
  float sk = 0.f, sq = 0.f, kq = 0.f;
  tok_sums8(kk, qq, sk, sq, kq);
  sk = group_sum<TPR>(sk);
  sq = group_sum<TPR>(sq);
  kq = group_sum<TPR>(kq);
  const float rk = use_l2 ? 1.0f / sqrtf(sk + l2_eps) : 1.0f;
  const float rq = use_l2 ? 1.0f / sqrtf(sq + l2_eps) : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) { kk[i] *= rk; qq[i] *= rq; }
  kq *= rk * rq;
  const float alpha = __expf(gv);

  float orow[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = row0 + rg + p * RPP;
    float dk = tok_dot8(sa[p], sb[p], kk);
    float dq = tok_dot8(sa[p], sb[p], qq);
    dk = group_sum<TPR>(dk);
    dq = group_sum<TPR>(dq);
    const float e = tok_err(E::cvt(vraw[p]), alpha, dk);
    const float be = bt * e;
    orow[p] = tok_out(scale, alpha, dq, be, kq);
    if (FULL || rg + p * RPP < RW) {
      float4 na, nb;
      na = tok_upd4(alpha, sa[p], be, kk);
      nb = tok_upd4(alpha, sb[p], be, kk + 4);
      stream_store4(S + row * D + ca, na);
      stream_store4(S + row * D + cb, nb);
    }
  }

  if (SPLIT > 1 || !z) {
    if (l == 0) {
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int row = row0 + rg + p * RPP;
        if (FULL || rg + p * RPP < RW) EO::store(o, obase + row, orow[p]);
      }
    }
    return;
  }
  // fused gated RMSNorm over the head's d_v outputs (SPLIT == 1: row0 == 0)
  __shared__ float so[D];
  __shared__ float sred[NT / 64];
  if (l == 0) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = rg + p * RPP;
      if (FULL || row < D) so[row] = orow[p];
    }
  }
  __syncthreads();
  const float ov = tid < D ? so[tid] : 0.f;
  float ss = group_sum<64>(ov * ov);
  if ((tid & 63) == 0) sred[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) tot += sred[w];
  if (tid < D) {
    const float rr = norm_rinv(tot, 1.0f / D, norm_eps);
    EO::store(o, obase + tid, ov * rr * norm_w[tid] * silu(E::cvt(zraw)));
  }
}

// Speculative verification: n_tok tokens per request (rows r n_tok + t of q, k,
// v, the gates, z and o), starting from the live state of the request's slot,
// which is only read.  The state after token t is written to checkpoint
// column t, ckpt[slot][t] (Flare core-design, speculative target state: a
// round writes the recurrent checkpoint columns of its verification inputs).
// Per (request, v-head) the state is read once, kept in registers across the
// tokens, and streamed out once per token.  A negative slot is an inactive
// lane: nothing is read or written and its o rows stay untouched.
template <class E, class EO, int D, int NT>
__global__ __launch_bounds__(NT) void k_recurrent_verify(
    const typename E::T* __restrict__ q, const typename E::T* __restrict__ k, const typename E::T* __restrict__ v,
    int64_t q_stride, int64_t k_stride, int64_t v_stride, GateSrc gates, float scale, int use_l2,
    float l2_eps, int h_qk, int h_v, int n_tok, const float* __restrict__ state, const int32_t* __restrict__ slots,
    float* __restrict__ ckpt, int n_cols, typename EO::T* __restrict__ o, const typename E::T* __restrict__ z,
    const float* __restrict__ norm_w, float norm_eps) {
  constexpr int TPR = D / 8;                 // lanes per state row
  constexpr int RPP = NT / TPR;              // rows per pass
  constexpr int PASSES = (D + RPP - 1) / RPP;
  static_assert(TPR <= 64 && NT % 64 == 0, "row lanes within a wave");
  constexpr bool FULL = RPP * PASSES == D;

  const int r = blockIdx.x / h_v, h = blockIdx.x % h_v;
  const int slot = slots ? slots[r] : r;
  if (slot < 0) return;
  const int hq = h / (h_v / h_qk);
  const int tid = threadIdx.x, l = tid % TPR, rg = tid / TPR;
  const int ca = 4 * l, cb = D / 2 + 4 * l;
  __shared__ float so[D];
  __shared__ float sred[NT / 64];

  const float* S = state + (static_cast<int64_t>(slot) * h_v + h) * D * D;
  float4 sa[PASSES], sb[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = rg + p * RPP;
    const int rr = (FULL || row < D) ? row : 0;
    sa[p] = stream_load4(S + rr * D + ca);
    sb[p] = stream_load4(S + rr * D + cb);
  }

  // the token inputs are loaded one token ahead, so their latency falls under
  // the previous token's work (the last token reloads its own: no branch)
  struct TokIn {
    typename E::T vraw[PASSES];
    typename E::T kr[8], qr[8];
    uint32_t graw, braw;
    typename E::T zraw;
  };
  auto load_tok = [&](int t, TokIn& ti) {
    const int64_t tr = static_cast<int64_t>(r) * n_tok + t;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = rg + p * RPP;
      ti.vraw[p] = v[tr * v_stride + h * D + ((FULL || row < D) ? row : 0)];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ti.kr[i] = k[tr * k_stride + hq * D + ca + i];
      ti.kr[4 + i] = k[tr * k_stride + hq * D + cb + i];
      ti.qr[i] = q[tr * q_stride + hq * D + ca + i];
      ti.qr[4 + i] = q[tr * q_stride + hq * D + cb + i];
    }
    gate_load_raw(gates, tr, h, h_v, ti.graw, ti.braw);
    ti.zraw = z ? z[(tr * h_v + h) * D + (tid < D ? tid : 0)] : typename E::T(0);
  };
  TokIn cur;
  load_tok(0, cur);
  for (int t = 0; t < n_tok; ++t) {
    const int64_t tr = static_cast<int64_t>(r) * n_tok + t;   // token row
    TokIn nxt;
    load_tok(t + 1 < n_tok ? t + 1 : t, nxt);
    float kk[8], qq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { kk[i] = E::cvt(cur.kr[i]); qq[i] = E::cvt(cur.qr[i]); }
    float gv, bt;
    gate_from_raw(gates, h, cur.graw, cur.braw, gv, bt);
    const int64_t obase = (tr * h_v + h) * D;
    const typename E::T zraw = cur.zraw;
    typename E::T vraw[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) vraw[p] = cur.vraw[p];
    float sk = 0.f, sq = 0.f, kq = 0.f;
    tok_sums8(kk, qq, sk, sq, kq);
    sk = group_sum<TPR>(sk);
    sq = group_sum<TPR>(sq);
    kq = group_sum<TPR>(kq);
    const float rk = use_l2 ? 1.0f / sqrtf(sk + l2_eps) : 1.0f;
    const float rq = use_l2 ? 1.0f / sqrtf(sq + l2_eps) : 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) { kk[i] *= rk; qq[i] *= rq; }
    kq *= rk * rq;
    const float alpha = __expf(gv);

    float* C = ckpt + ((static_cast<int64_t>(slot) * n_cols + t) * h_v + h) * D * D;
    float orow[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = rg + p * RPP;
      float dk = tok_dot8(sa[p], sb[p], kk);
      float dq = tok_dot8(sa[p], sb[p], qq);
      dk = group_sum<TPR>(dk);
      dq = group_sum<TPR>(dq);
      const float e = tok_err(E::cvt(vraw[p]), alpha, dk);
      const float be = bt * e;
      orow[p] = tok_out(scale, alpha, dq, be, kq);
      float4 na, nb;
      na = tok_upd4(alpha, sa[p], be, kk);
      nb = tok_upd4(alpha, sb[p], be, kk + 4);
      sa[p] = na;
      sb[p] = nb;
      if (FULL || row < D) {
        stream_store4(C + row * D + ca, na);
        stream_store4(C + row * D + cb, nb);
      }
    }

    if (!z) {
      if (l == 0) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
          const int row = rg + p * RPP;
          if (FULL || row < D) EO::store(o, obase + row, orow[p]);
        }
      }
      cur = nxt;
      continue;
    }
    // fused gated RMSNorm over the head's d_v outputs of this token
    if (l == 0) {
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int row = rg + p * RPP;
        if (FULL || row < D) so[row] = orow[p];
      }
    }
    __syncthreads();
    const float ov = tid < D ? so[tid] : 0.f;
    const float ss = group_sum<64>(ov * ov);
    if ((tid & 63) == 0) sred[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) tot += sred[w];
    if (tid < D) {
      const float rr = norm_rinv(tot, 1.0f / D, norm_eps);
      EO::store(o, obase + tid, ov * rr * norm_w[tid] * silu(E::cvt(zraw)));
    }
    __syncthreads();   // so and sred are rewritten by the next token
    cur = nxt;
  }
}

template <class E, class EO>
static hipError_t run_verify(const VerifyArgs& a) {
  using T = typename E::T;
  using TO = typename EO::T;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(a.n_req) * a.h_v);
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* z = static_cast<const T*>(a.z);
  // d = 128: 1024 threads (two state rows each) measured fastest without the
  // norm (133 against 148 us at 64 requests x 4 tokens); with the norm, whose
  // three barriers per token weigh more in larger workgroups, 512 threads
  // (146 against 152 us).
  if (a.d == 128 && z == nullptr)
    hipLaunchKernelGGL((k_recurrent_verify<E, EO, 128, 1024>), dim3(blocks), dim3(1024), 0, st, q, k, v, a.q_stride,
                       a.k_stride, a.v_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.n_tok, a.state,
                       a.slots, a.ckpt, a.n_cols, static_cast<TO*>(a.o), z, a.norm_w, a.norm_eps);
  else if (a.d == 128)
    hipLaunchKernelGGL((k_recurrent_verify<E, EO, 128, 512>), dim3(blocks), dim3(512), 0, st, q, k, v, a.q_stride,
                       a.k_stride, a.v_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.n_tok, a.state,
                       a.slots, a.ckpt, a.n_cols, static_cast<TO*>(a.o), z, a.norm_w, a.norm_eps);
  else
    hipLaunchKernelGGL((k_recurrent_verify<E, EO, 16, 64>), dim3(blocks), dim3(64), 0, st, q, k, v, a.q_stride,
                       a.k_stride, a.v_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.n_tok, a.state,
                       a.slots, a.ckpt, a.n_cols, static_cast<TO*>(a.o), z, a.norm_w, a.norm_eps);
  return hipGetLastError();
}

hipError_t launch_recurrent_verify(const VerifyArgs& a) {
  if (a.dt == GDN_BF16) return a.o_dt == GDN_BF16 ? run_verify<BF16, BF16>(a) : run_verify<BF16, F32>(a);
  return a.o_dt == GDN_BF16 ? run_verify<F32, BF16>(a) : run_verify<F32, F32>(a);
}

template <class E, class EO>
static hipError_t run_step(const StepArgs& a) {
  using T = typename E::T;
  using TO = typename EO::T;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(a.n_req) * a.h_v);
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* z = static_cast<const T*>(a.z);
  if (a.d == 128 && z)   // the fused norm needs the head's rows in one workgroup
    hipLaunchKernelGGL((k_recurrent_step<E, EO, 128, 256, 1>), dim3(blocks), dim3(256), 0, st, q, k, v,
                       a.q_stride, a.k_stride, a.v_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v,
                       a.state, a.slots, static_cast<TO*>(a.o), z, a.norm_w, a.norm_eps);
  else if (a.d == 128)
    hipLaunchKernelGGL((k_recurrent_step<E, EO, 128, 256, 4>), dim3(blocks * 4), dim3(256), 0, st, q, k, v,
                       a.q_stride, a.k_stride, a.v_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v,
                       a.state, a.slots, static_cast<TO*>(a.o), z, a.norm_w, a.norm_eps);
  else
    hipLaunchKernelGGL((k_recurrent_step<E, EO, 16, 64, 1>), dim3(blocks), dim3(64), 0, st, q, k, v, a.q_stride,
                       a.k_stride, a.v_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.state,
                       a.slots, static_cast<TO*>(a.o), z, a.norm_w, a.norm_eps);
  return hipGetLastError();
}

hipError_t launch_recurrent_step(const StepArgs& a) {
  if (a.dt == GDN_BF16) return a.o_dt == GDN_BF16 ? run_step<BF16, BF16>(a) : run_step<BF16, F32>(a);
  return a.o_dt == GDN_BF16 ? run_step<F32, BF16>(a) : run_step<F32, F32>(a);
}

}  // namespace gdn
