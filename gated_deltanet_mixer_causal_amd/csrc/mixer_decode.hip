// One decode token of the whole mixer in one kernel (gfx950): the width-4
// conv step with SiLU, the gated delta rule step and, optionally, the gated
// RMSNorm, for one request and one q/k head per workgroup.
//
// The conv (haskell-infer-demo README, "Architecture": causal conv1d of width
// 4 over the raw projected q|k|v; Flare core-design, short-convolution
// paragraph: raw-input history per slot) runs over the channels this
// workgroup owns: the q and k channels of its q/k head and the v channels of
// the v-heads that read it.  Each channel's history is shifted by exactly one
// thread, so the in-place update needs no ordering between workgroups.  The
// conv outputs are rounded to the input dtype (the dtype at which the
// unfused path hands them to the recurrence) and kept in LDS; the recurrence
// (the formula of the gated delta rule: haskell-infer-demo README,
// "Highlights") then runs for each of those v-heads in turn with the
// arithmetic of the unfused decode step, row by row, so the results are
// bit-identical to gdn_conv1d_fwd (decode) followed by gdn_recurrent_step.
// It saves the conv step's launch and its round trip of the conv output
// through memory.
//
// Shape: 512 threads per workgroup, 16 lanes per state row (32 rows per
// pass, 4 passes per 128-row head), one v-head at a time; the first head's
// state rows are loaded before the conv so their latency overlaps it.  At 112
// VGPRs two workgroups share a CU, so one's conv overlaps the other's state
// stream (measured: 1024-thread workgroups running two heads at once, one per
// CU, and 256-thread ones were slower).
#include "common.hpp"
#include "mixer_decode.hpp"

namespace gdn {

typedef float md_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 md_stream_load4(const float* p) {
  const md_f4 v = __builtin_nontemporal_load(reinterpret_cast<const md_f4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void md_stream_store4(float* p, float4 v) {
  __builtin_nontemporal_store(md_f4{v.x, v.y, v.z, v.w}, reinterpret_cast<md_f4*>(p));
}


template <class E, class EO, int D, int NT, int GMAX, int PAR>
__global__ __launch_bounds__(NT * PAR) void k_mixer_decode(
    const typename E::T* __restrict__ x, const typename E::T* __restrict__ w, typename E::T* __restrict__ hist,
    GateSrc gates, float scale, int use_l2, float l2_eps, int h_qk, int h_v, float* __restrict__ state,
    const int32_t* __restrict__ slots, typename EO::T* __restrict__ o, const typename E::T* __restrict__ z,
    const float* __restrict__ norm_w, float norm_eps) {
  // PAR groups of NT threads; group `sub` runs the v-heads sub, sub + PAR, ...
  constexpr int TPR = D / 8, RPP = NT / TPR, PASSES = D / RPP;
  static_assert(D % RPP == 0 && TPR <= 64 && NT % 64 == 0, "row lanes within a wave");
  __shared__ float yq[D], yk[D], yv[GMAX][D];
  __shared__ float so[PAR][D];
  __shared__ float sred[PAR][NT / 64];
  const int r = blockIdx.x / h_qk, hq = blockIdx.x % h_qk;
  const int slot = slots ? slots[r] : r;
  if (slot < 0) return;
  const int grp = h_v / h_qk;
  const int nq = h_qk * D, ch = 2 * nq + h_v * D;
  const int64_t ld = ch;
  const int tid = threadIdx.x;

  const int sub = tid / NT, t2 = tid % NT;
  const int l = t2 % TPR, rg = t2 / TPR;
  const int ca = 4 * l, cb = D / 2 + 4 * l;
  // the state rows of this thread's first v-head are loaded before the conv,
  // so their latency overlaps it
  float4 sa[PASSES], sb[PASSES];
  auto load_rows = [&](int h) {
    const float* S = state + (static_cast<int64_t>(slot) * h_v + h) * D * D;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = rg + p * RPP;
      sa[p] = md_stream_load4(S + row * D + ca);
      sb[p] = md_stream_load4(S + row * D + cb);
    }
  };
  if (sub < grp) load_rows(hq * grp + sub);

  // 1. conv step over this workgroup's channels: q, k of head hq, v of its heads
  const int own = (2 + grp) * D;
  for (int e = tid; e < own; e += NT * PAR) {
    int c;
    if (e < D) c = hq * D + e;
    else if (e < 2 * D) c = nq + hq * D + (e - D);
    else c = 2 * nq + (hq * grp) * D + (e - 2 * D);
    typename E::T* hp = hist + static_cast<int64_t>(slot) * 3 * ld + c;
    const float h0 = E::load(hp, 0), h1 = E::load(hp, ld), h2 = E::load(hp, 2 * ld);
    const typename E::T xraw = x[static_cast<int64_t>(r) * ld + c];
    const float xc = E::cvt(xraw);
    const float y = conv4_silu(E::load(w, 4 * static_cast<int64_t>(c)), E::load(w, 4 * static_cast<int64_t>(c) + 1),
                            E::load(w, 4 * static_cast<int64_t>(c) + 2), E::load(w, 4 * static_cast<int64_t>(c) + 3),
                            h0, h1, h2, xc);
    // the unfused path stores the conv output in the input dtype
    typename E::T yr[1];
    E::store(yr, 0, y);
    const float yd = E::cvt(yr[0]);
    if (e < D) yq[e] = yd;
    else if (e < 2 * D) yk[e - D] = yd;
    else yv[(e - 2 * D) / D][(e - 2 * D) % D] = yd;
    hp[0] = hp[ld];
    hp[ld] = hp[2 * ld];
    hp[2 * ld] = xraw;
  }
  __syncthreads();

  // 2. normalised q, k (each row's TPR lanes hold columns 4l.. and D/2 + 4l..)
  float kk[8], qq[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kk[i] = yk[ca + i]; kk[4 + i] = yk[cb + i];
    qq[i] = yq[ca + i]; qq[4 + i] = yq[cb + i];
  }
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

  // 3. the recurrent step of each v-head that reads this q/k head (the trip
  // count is the same for every group, so the barriers below are uniform)
  for (int base = 0; base < grp; base += PAR) {
    const int hh = base + sub;
    const bool live = hh < grp;
    const int h = hq * grp + (live ? hh : 0);
    float* S = state + (static_cast<int64_t>(slot) * h_v + h) * D * D;
    float orow[PASSES];
    typename E::T zraw = 0;
    const int64_t obase = (static_cast<int64_t>(r) * h_v + h) * D;
    if (live) {
      if (base > 0) load_rows(h);
      float gv, bt;
      load_gate(gates, r, h, h_v, gv, bt);
      if (z) zraw = z[obase + (t2 < D ? t2 : 0)];
      const float alpha = __expf(gv);
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int row = rg + p * RPP;
        float dk = tok_dot8(sa[p], sb[p], kk);
        float dq = tok_dot8(sa[p], sb[p], qq);
        dk = group_sum<TPR>(dk);
        dq = group_sum<TPR>(dq);
        const float e = tok_err(yv[hh][row], alpha, dk);
        const float be = bt * e;
        orow[p] = tok_out(scale, alpha, dq, be, kq);
        float4 na, nb;
        na = tok_upd4(alpha, sa[p], be, kk);
        nb = tok_upd4(alpha, sb[p], be, kk + 4);
        md_stream_store4(S + row * D + ca, na);
        md_stream_store4(S + row * D + cb, nb);
      }
      if (!z && l == 0) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) EO::store(o, obase + rg + p * RPP, orow[p]);
      }
    }
    if (!z) continue;
    // fused gated RMSNorm over the head's outputs (the unfused step's sum order)
    if (live && l == 0) {
#pragma unroll
      for (int p = 0; p < PASSES; ++p) so[sub][rg + p * RPP] = orow[p];
    }
    __syncthreads();
    const float ov = t2 < D ? so[sub][t2] : 0.f;
    float ss = group_sum<64>(ov * ov);
    if ((t2 & 63) == 0) sred[sub][t2 >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int wv = 0; wv < NT / 64; ++wv) tot += sred[sub][wv];
    if (live && t2 < D) {
      const float rr = norm_rinv(tot, 1.0f / D, norm_eps);
      EO::store(o, obase + t2, ov * rr * norm_w[t2] * silu(E::cvt(zraw)));
    }
    __syncthreads();   // so and sred are rewritten by the next round of v-heads
  }
}

template <class E, class EO>
static hipError_t run_mixer_decode(const MixerDecodeArgs& a) {
  using T = typename E::T;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(a.n_req) * a.h_qk);
  hipLaunchKernelGGL((k_mixer_decode<E, EO, 128, 512, kMixerDecodeMaxGroup, 1>), dim3(blocks), dim3(512), 0, st,
                     static_cast<const T*>(a.x), static_cast<const T*>(a.w), static_cast<T*>(a.conv_state), a.gate,
                     a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.state, a.slots, static_cast<typename EO::T*>(a.o),
                     static_cast<const T*>(a.z), a.norm_w, a.norm_eps);
  return hipGetLastError();
}

hipError_t launch_mixer_decode(const MixerDecodeArgs& a) {
  if (a.dt == GDN_BF16) return a.o_dt == GDN_BF16 ? run_mixer_decode<BF16, BF16>(a) : run_mixer_decode<BF16, F32>(a);
  return a.o_dt == GDN_BF16 ? run_mixer_decode<F32, BF16>(a) : run_mixer_decode<F32, F32>(a);
}

}  // namespace gdn
