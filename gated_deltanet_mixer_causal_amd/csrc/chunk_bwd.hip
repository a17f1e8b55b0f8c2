// Chunked backward of the gated delta rule on the matrix cores (gfx950),
// bf16 inputs, d_k = d_v = 128, 64-token chunks.
//
// For L = sum(dO * O) + sum(dS_T * S_T) with the forward of chunk.hip, the
// gradients follow from two chains over the chunks and one pass per chunk.
// Inside a chunk entering with state S (d_v x d_k) and leaving with dS the
// gradient of the loss with respect to the leaving state, with the forward's
// normalised rows K^ = diag(rk) K, Q^ = diag(rq) Q, decays
// D_ij = exp(gamma_i - gamma_j) (j <= i), b = exp(gamma), d = exp(gamma_C -
// gamma), and its T = (I + L)^-1, Tb = T diag(beta), X, U, P:
//     dU  = P^T dO + diag(d) K^ dS^T
//     dX  = Tb^T dU                                   (= dV)
//     dS0 = b_C dS + scale dO^T diag(b) Q^ - dX^T diag(b) K^   (into the previous chunk)
//     dTb = dU X^T;  dbeta_j = sum_i dTb_ij T_ij;  dT = dTb diag(beta)
//     dL  = -T^T dT T^T (strictly lower);  dbeta_i += sum_j dL_ij A_ij D_ij
//     dP  = dO U^T (lower);  dAq = scale dP * D;  dA = diag(beta) dL * D
//     dQ^ = scale diag(b) dO S + dAq K^
//     dK^ = diag(d) U dS - diag(b) dX S + dAq^T Q^ + (dA + dA^T) K^
//     dgamma_i = row i minus column i of dP*P and of dL*L
//                + q^_i . (scale b_i (dO S)_i) - b_i k^_i . (dX S)_i - d_i k^_i . (U dS)_i,
//                and at the chunk's last token + sum_j d_j k^_j . (U dS)_j + b_C <dS, S>
//     dg_t = sum_{i >= t} dgamma_i inside the chunk
// (A = K^ K^^T; the reverse-mode derivative of the chunk algebra, checked
// against the token-by-token gradient to 1e-15 on the CPU).  dq, dk then go
// through the L2 normalisation after the v-heads of each q/k head are summed.
//
// Launches (after the forward prep, written in its backward mode with P^T and
// Tb^T fragments, and the forward scan writing the state entering every chunk):
//   k_bwd_dstate  one workgroup per (sequence, v-head, 16-wide d_v slice),
//                 chunks last to first, the slice of dS in fp32 registers:
//                 writes dS leaving each chunk, dV and dS_initial.  Three
//                 products per chunk with a barrier after each, like the
//                 forward scan.
//   k_bwd_grad    one workgroup per (chunk, v-head): recomputes the chunk's
//                 Gram tiles, L, P and T, streams S, dS, dO over four 32-wide
//                 d_v parts to form X, U, dU and the sums over d_v (dO S,
//                 dX S, U dS, dP, dTb), then the C x C algebra and dQ^, dK^,
//                 dbeta, dg.
//   k_bwd_dqk     per (token, q/k head): sums dQ^, dK^ over the v-heads and
//                 applies the L2-norm backward.
// Operand precision as in the forward: derived operands are bf16 hi+lo pairs,
// raw bf16 q/k/v single, fp32 accumulation; all sums run in a fixed order.
#include "chunk_impl.hpp"

namespace gdn {
namespace {

using PB = PolBF16;
constexpr int BD = 128, BC = 64;
using BW = WsLayout<PB, BD, BC>;
using Frag = bf16x8;

__device__ __forceinline__ floatx4 mma3(floatx4 c, Frag ah, Frag al, Frag bh, Frag bl) {
  c = mfma_bf16(ah, bh, c);
  c = mfma_bf16(ah, bl, c);
  return mfma_bf16(al, bh, c);
}
// A derived (hi, lo), B raw
__device__ __forceinline__ floatx4 mma2(floatx4 c, Frag ah, Frag al, Frag b) {
  c = mfma_bf16(ah, b, c);
  return mfma_bf16(al, b, c);
}

// Fragment from k-contiguous rows: lane (r, g) gets p[(row0 + r) ld + k0 + 8g + e].
__device__ __forceinline__ Frag frag_rows(const __bf16* p, int ld, int row0, int k0) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const Frag*>(p + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}
// Fragment from the transpose: lane (r, g) gets p[(k0 + 8g + e) ld + col0 + r],
// two transposing reads of four rows each (ld and col0 multiples of 4).
__device__ __forceinline__ Frag frag_cols(const __bf16* p, int ld, int k0, int col0) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const __bf16* a = p + (k0 + 8 * g + (r >> 2)) * ld + col0 + 4 * (r & 3);
  const uint2 x = lds_read_tr16(a);
  const uint2 y = lds_read_tr16(a + 4 * ld);
  return __builtin_bit_cast(Frag, make_uint4(x.x, x.y, y.x, y.y));
}
__device__ __forceinline__ void put_hl(__bf16* hi, __bf16* lo, int idx, float v) {
  __bf16 a, b;
  split_bf16(v, a, b);
  hi[idx] = a;
  lo[idx] = b;
}
// four consecutive fp32 values as hi/lo, 8-byte stores
__device__ __forceinline__ void put4_hl(__bf16* hi, __bf16* lo, int idx, float4 v) {
  const float t[4] = {v.x, v.y, v.z, v.w};
  PB::put4(hi, lo, idx, t);
}
__device__ __forceinline__ void split8(const float* v, Frag& h, Frag& l) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 a, b;
    split_bf16(v[e], a, b);
    h[e] = a;
    l[e] = b;
  }
}
// sum over the 16 lanes of a row group (lanes 16g .. 16g + 15)
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}
// sum over the four row groups (lanes r, r + 16, r + 32, r + 48)
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}

// ---------------------------------------------------------------------------
// k_bwd_dstate: the gradient of the state, chunks last to first
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_dstate(int h_qk, int h_v, const int32_t* __restrict__ cu, int n_seq,
                                                    int64_t t_total, const float* __restrict__ d_o,
                                                    const float* __restrict__ d_final, float* __restrict__ dv,
                                                    float* __restrict__ d_init, float* __restrict__ dstates,
                                                    ChunkWs ws) {
  constexpr int D = BD, C = BC, KS = 32, NKS_D = D / KS, NKS_C = C / KS, NTILE = D / 16;
  constexpr int LDT = C, LDK = D, LDKT = D + 8;
  __shared__ __attribute__((aligned(16))) __bf16 sG[2 * 16 * LDK];         // dS rows (d_v), hi | lo
  __shared__ __attribute__((aligned(16))) __bf16 sDO[2][2 * 16 * LDT];     // dO rows (d_v), double-buffered
  __shared__ __attribute__((aligned(16))) __bf16 sDOc[2][2 * 16 * LDT];    // c2 dO
  __shared__ __attribute__((aligned(16))) __bf16 sDU[2 * 16 * LDT];        // dU rows (d_v)
  __shared__ __attribute__((aligned(16))) __bf16 sDX[2 * 16 * LDT];        // -c1 dX rows (d_v)
  __shared__ __attribute__((aligned(16))) __bf16 sKt[C * LDKT];            // the chunk's K rows
  __shared__ __attribute__((aligned(16))) __bf16 sQt[C * LDKT];            // the chunk's Q rows
  __bf16* const sG_lo = sG + 16 * LDK;
  __bf16* const sDU_lo = sDU + 16 * LDT;
  __bf16* const sDX_lo = sDX + 16 * LDT;

  const int64_t per_seq = static_cast<int64_t>(h_v) * NTILE;
  const int64_t bidx = blockIdx.x;
  const int64_t rank = bidx / per_seq;
  if (rank >= n_seq) return;
  const int s = ws.order ? ws.order[rank] : static_cast<int>(rank);
  const int64_t lid = xcd_order(bidx % per_seq, per_seq);
  const int tile = static_cast<int>(lid % NTILE);
  const int h = static_cast<int>(lid / NTILE);
  const int hq = h / (h_v / h_qk);
  const int dv0 = tile * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  auto offT = [&](int row, int ks) { return swz_off<LDT>(row, ks * (KS / 8) + g4); };
  auto offS = [&](int row, int ks) { return swz_off<LDK>(row, ks * (KS / 8) + g4); };

  // dS of this lane: dS[dv0 + r16][16 mt + 4 g4 + i], mt = wave + 4 jj
  floatx4 G[2];
  const int64_t grow = (static_cast<int64_t>(s) * h_v + h) * D + dv0 + r16;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int mt = wave + 4 * jj;
    G[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (d_final) {
      const float4 f = *reinterpret_cast<const float4*>(d_final + grow * D + 16 * mt + 4 * g4);
      G[jj] = floatx4{f.x, f.y, f.z, f.w};
    }
    const float t4[4] = {G[jj][0], G[jj][1], G[jj][2], G[jj][3]};
    PB::put4(sG, sG_lo, swz_off<LDK>(r16, (16 * mt + 4 * g4) >> 3) + ((4 * g4) & 7), t4);
  }

  const int64_t start = seq_start(cu, s, t_total), end = seq_start(cu, s + 1, t_total);
  const int64_t nchunks = (end - start + C - 1) / C;
  const int64_t slot0 = start / C + s;
  const int orow0 = 16 * wave + 4 * g4;
  const int ks0 = (16 * wave) / KS;       // first k-step of this tile's rows of P^T and Tb^T
  const int64_t vrow = static_cast<int64_t>(h_v) * D;

  // operands of one chunk (registers), loaded one chunk ahead
  Frag kf[NKS_D], qf[NKS_D], ph[NKS_C], pl[NKS_C], th[NKS_C], tl[NKS_C];
  float4 c1v, c3v, dov;
  float bcv, c2t;
  auto load_chunk = [&](int64_t jj, Frag* kf_, Frag* qf_, Frag* ph_, Frag* pl_, Frag* th_, Frag* tl_, float4& c1_,
                        float4& c3_, float& bc_, float4& do_, float& c2_) {
    const int64_t t0_ = start + jj * C;
    const int len_ = static_cast<int>(end - t0_ < C ? end - t0_ : C);
    const __bf16* kq_ = static_cast<const __bf16*>(ws.kq) + ((slot0 + jj) * h_qk + hq) * BW::kq_elems + lane * 8;
#pragma unroll
    for (int ks = 0; ks < NKS_D; ++ks) {
      kf_[ks] = PB::ld(kq_ + BW::kq_block(0, wave, ks));
      qf_[ks] = PB::ld(kq_ + BW::kq_block(1, wave, ks));
    }
    const int64_t u_ = (slot0 + jj) * h_v + h;
    const __bf16* p_ = static_cast<const __bf16*>(ws.p) + u_ * BW::op_elems + lane * 8;
    const __bf16* t_ = static_cast<const __bf16*>(ws.tbt) + u_ * BW::op_elems + lane * 8;
#pragma unroll
    for (int ks = 0; ks < NKS_C; ++ks) {
      if (ks >= ks0) {
        ph_[ks] = PB::ld(p_ + BW::op_block(wave, ks, 0));
        pl_[ks] = PB::ld(p_ + BW::op_block(wave, ks, 1));
        th_[ks] = PB::ld(t_ + BW::op_block(wave, ks, 0));
        tl_[ks] = PB::ld(t_ + BW::op_block(wave, ks, 1));
      }
    }
    const float* sc_ = ws.sc + u_ * (4 * C);
    c1_ = *reinterpret_cast<const float4*>(sc_ + orow0);
    c3_ = *reinterpret_cast<const float4*>(sc_ + 2 * C + orow0);
    bc_ = sc_[3 * C];
    // dO staging: token tid / 4, d_v columns 4 (tid % 4) .. + 3
    const int tk = tid >> 2;
    c2_ = sc_[C + tk];
    do_ = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tk < len_) do_ = *reinterpret_cast<const float4*>(d_o + (t0_ + tk) * vrow + h * D + dv0 + 4 * (tid & 3));
  };
  auto stage_do = [&](int buf, float4 v4, float c2) {
    const int tk = tid >> 2, c0 = 4 * (tid & 3);
    const float v[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = swz_off<LDT>(c0 + e, tk >> 3) + (tk & 7);
      put_hl(sDO[buf], sDO[buf] + 16 * LDT, idx, v[e]);
      put_hl(sDOc[buf], sDOc[buf] + 16 * LDT, idx, c2 * v[e]);
    }
  };

  int buf = 0;
  if (nchunks > 0) {
    load_chunk(nchunks - 1, kf, qf, ph, pl, th, tl, c1v, c3v, bcv, dov, c2t);
    stage_do(0, dov, c2t);
  }
  __syncthreads();

  for (int64_t j = nchunks - 1; j >= 0; --j) {
    const int64_t t0 = start + j * C;
    const int len = static_cast<int>(end - t0 < C ? end - t0 : C);
    // the gradient of the state leaving this chunk
    {
      float* o = dstates + (((slot0 + j) * h_v + h) * D + dv0 + r16) * D;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        *reinterpret_cast<float4*>(o + 16 * (wave + 4 * jj) + 4 * g4) = make_float4(G[jj][0], G[jj][1], G[jj][2], G[jj][3]);
    }
    // next (earlier) chunk's operands, in flight during this one
    const int64_t jn = j > 0 ? j - 1 : j;
    Frag kfn[NKS_D], qfn[NKS_D], phn[NKS_C], pln[NKS_C], thn[NKS_C], tln[NKS_C];
    float4 c1n, c3n, don;
    float bcn, c2n;
    load_chunk(jn, kfn, qfn, phn, pln, thn, tln, c1n, c3n, bcn, don, c2n);

    // ---- A: dU = P^T dO + diag(c3) K dS^T for token tile `wave` ----
    {
      floatx4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS_D; ++ks) {
        const int off = offS(r16, ks);
        y = mfma_bf16(kf[ks], PB::ld(sG + off), y);
        y = mfma_bf16(kf[ks], PB::ld(sG_lo + off), y);
        *reinterpret_cast<Frag*>(sKt + (16 * wave + r16) * LDKT + ks * KS + g4 * 8) = kf[ks];
        *reinterpret_cast<Frag*>(sQt + (16 * wave + r16) * LDKT + ks * KS + g4 * 8) = qf[ks];
      }
      const float c3[4] = {c3v.x, c3v.y, c3v.z, c3v.w};
      floatx4 du;
#pragma unroll
      for (int i = 0; i < 4; ++i) du[i] = c3[i] * y[i];
#pragma unroll
      for (int ks = 0; ks < NKS_C; ++ks) {
        if (ks >= ks0) {
          const int off = offT(r16, ks);
          du = mma3(du, ph[ks], pl[ks], PB::ld(sDO[buf] + off), PB::ld(sDO[buf] + 16 * LDT + off));
        }
      }
      const float t4[4] = {du[0], du[1], du[2], du[3]};
      PB::put4(sDU, sDU_lo, swz_off<LDT>(r16, orow0 >> 3) + (orow0 & 7), t4);
    }
    __syncthreads();

    // ---- B: dX = Tb^T dU (= dV); -c1 dX for the state update ----
    {
      floatx4 dx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS_C; ++ks) {
        if (ks >= ks0) {
          const int off = offT(r16, ks);
          dx = mma3(dx, th[ks], tl[ks], PB::ld(sDU + off), PB::ld(sDU_lo + off));
        }
      }
      const float c1[4] = {c1v.x, c1v.y, c1v.z, c1v.w};
      float t4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (orow0 + i < len) dv[(t0 + orow0 + i) * vrow + h * D + dv0 + r16] = dx[i];
        t4[i] = -c1[i] * dx[i];
      }
      PB::put4(sDX, sDX_lo, swz_off<LDT>(r16, orow0 >> 3) + (orow0 & 7), t4);
    }
    __syncthreads();

    // ---- C: dS <- b_C dS + Q^T (c2 dO) - K^T (c1 dX) ----
    {
      const __bf16* doc = sDOc[buf];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int mt = wave + 4 * jj;
        floatx4 acc = G[jj] * bcv;
#pragma unroll
        for (int ks = 0; ks < NKS_C; ++ks) {
          const int off = offT(r16, ks);
          const Frag kt = frag_cols(sKt, LDKT, ks * KS, 16 * mt);
          const Frag qt = frag_cols(sQt, LDKT, ks * KS, 16 * mt);
          acc = mfma_bf16(kt, PB::ld(sDX + off), acc);
          acc = mfma_bf16(kt, PB::ld(sDX_lo + off), acc);
          acc = mfma_bf16(qt, PB::ld(doc + off), acc);
          acc = mfma_bf16(qt, PB::ld(doc + 16 * LDT + off), acc);
        }
        G[jj] = acc;
        const float t4[4] = {acc[0], acc[1], acc[2], acc[3]};
        PB::put4(sG, sG_lo, swz_off<LDK>(r16, (16 * mt + 4 * g4) >> 3) + ((4 * g4) & 7), t4);
      }
      stage_do(buf ^ 1, don, c2n);
    }
#pragma unroll
    for (int ks = 0; ks < NKS_D; ++ks) {
      kf[ks] = kfn[ks];
      qf[ks] = qfn[ks];
    }
#pragma unroll
    for (int ks = 0; ks < NKS_C; ++ks) {
      ph[ks] = phn[ks];
      pl[ks] = pln[ks];
      th[ks] = thn[ks];
      tl[ks] = tln[ks];
    }
    c1v = c1n;
    c3v = c3n;
    bcv = bcn;
    buf ^= 1;
    __syncthreads();
  }

  if (d_init) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
      *reinterpret_cast<float4*>(d_init + grow * D + 16 * (wave + 4 * jj) + 4 * g4) =
          make_float4(G[jj][0], G[jj][1], G[jj][2], G[jj][3]);
  }
}

// ---------------------------------------------------------------------------
// k_bwd_grad: one workgroup per (chunk slot, v-head)
// ---------------------------------------------------------------------------
// LDS (bytes).  Rows: K, Q raw [64][LDK]; T, P hi|lo [64][L64]; then one
// region reused by the solve (L, T fp32 [64][LDC]), the d_v parts (S, dS
// [32][LDK], dO, X, beta X, U, dU [64][L32], hi|lo) and the C x C algebra
// (dAq diag(rk), diag(rq) dAq, dT then E, Z [64][L64], hi|lo); scalars last.
struct GradLds {
  static constexpr int LDK = BD + 8, L64 = BC + 8, L32 = 40, LDC = BC + 4;
  static constexpr int HL64 = 2 * BC * L64 * 2;     // one hi|lo C x C array
  static constexpr int HL32 = 2 * BC * L32 * 2;     // one hi|lo C x 32 array
  static constexpr int HLS = 2 * 32 * LDK * 2;      // one hi|lo 32 x d_k array
  static constexpr int kK = 0, kQ = kK + BC * LDK * 2, kT = kQ + BC * LDK * 2, kP = kT + HL64;
  static constexpr int kU = kP + HL64;
  // solve
  static constexpr int kL = kU, kTf = kU + BC * LDC * 4;
  // d_v parts
  static constexpr int kS = kU, kdS = kS + HLS, kDO = kdS + HLS, kX = kDO + HL32, kXb = kX + HL32, kUU = kXb + HL32,
                       kDU = kUU + HL32, kPartsEnd = kDU + HL32;
  // C x C
  static constexpr int kAqk = kU, kAqq = kAqk + HL64, kDT = kAqq + HL64, kZ = kDT + HL64, kCxCEnd = kZ + HL64;
  static constexpr int kUEnd = kPartsEnd > kCxCEnd ? kPartsEnd : kCxCEnd;
  static constexpr int kGam = kUEnd;                       // double[64]
  static constexpr int kB = kGam + 8 * BC, kD = kB + 4 * BC, kRk = kD + 4 * BC, kRq = kRk + 4 * BC,
                       kBeta = kRq + 4 * BC;
  static constexpr int kRowG = kBeta + 4 * BC, kRowB = kRowG + 4 * BC;   // per-token sums of row terms
  static constexpr int kColG = kRowB + 4 * BC, kColB = kColG + 16 * BC;  // [4 waves][64] column terms
  static constexpr int kDd = kColB + 16 * BC;                             // per-token d_j k^_j . (U dS)_j
  static constexpr int kRed = kDd + 4 * BC;                               // 16 floats
  static constexpr int bytes = kRed + 64;
  static_assert(kTf + BC * LDC * 4 <= kUEnd, "solve fits the shared region");
};

template <class In>
__global__ __launch_bounds__(256) void k_bwd_grad(
    const typename In::T* __restrict__ q, const typename In::T* __restrict__ k, const typename In::T* __restrict__ v,
    int64_t q_stride, int64_t k_stride, int64_t v_stride, GateSrc gates, float scale, int use_l2, float l2_eps,
    int h_qk, int h_v, const int32_t* __restrict__ cu, int n_seq, int64_t t_total, const float* __restrict__ d_o,
    const float* __restrict__ dvx, const float* __restrict__ states, const float* __restrict__ dstates,
    float* __restrict__ dqh, float* __restrict__ dkh, float* __restrict__ dg, float* __restrict__ dbeta) {
  using LY = GradLds;
  constexpr int D = BD, C = BC, LDK = LY::LDK, L64 = LY::L64, L32 = LY::L32, LDC = LY::LDC;
  __shared__ __attribute__((aligned(16))) char lds[LY::bytes];
  __bf16* const sK = reinterpret_cast<__bf16*>(lds + LY::kK);
  __bf16* const sQ = reinterpret_cast<__bf16*>(lds + LY::kQ);
  __bf16* const sT = reinterpret_cast<__bf16*>(lds + LY::kT);
  __bf16* const sT_lo = sT + C * L64;
  __bf16* const sP = reinterpret_cast<__bf16*>(lds + LY::kP);
  __bf16* const sP_lo = sP + C * L64;
  float* const sL = reinterpret_cast<float*>(lds + LY::kL);
  float* const sTf = reinterpret_cast<float*>(lds + LY::kTf);
  __bf16* const sS = reinterpret_cast<__bf16*>(lds + LY::kS);
  __bf16* const sS_lo = sS + 32 * LDK;
  __bf16* const sdS = reinterpret_cast<__bf16*>(lds + LY::kdS);
  __bf16* const sdS_lo = sdS + 32 * LDK;
  __bf16* const sDO = reinterpret_cast<__bf16*>(lds + LY::kDO);
  __bf16* const sDO_lo = sDO + C * L32;
  __bf16* const sX = reinterpret_cast<__bf16*>(lds + LY::kX);
  __bf16* const sX_lo = sX + C * L32;
  __bf16* const sXb = reinterpret_cast<__bf16*>(lds + LY::kXb);
  __bf16* const sXb_lo = sXb + C * L32;
  __bf16* const sU = reinterpret_cast<__bf16*>(lds + LY::kUU);
  __bf16* const sU_lo = sU + C * L32;
  __bf16* const sDU = reinterpret_cast<__bf16*>(lds + LY::kDU);
  __bf16* const sDU_lo = sDU + C * L32;
  __bf16* const sAqk = reinterpret_cast<__bf16*>(lds + LY::kAqk);
  __bf16* const sAqk_lo = sAqk + C * L64;
  __bf16* const sAqq = reinterpret_cast<__bf16*>(lds + LY::kAqq);
  __bf16* const sAqq_lo = sAqq + C * L64;
  __bf16* const sDT = reinterpret_cast<__bf16*>(lds + LY::kDT);   // dT, then E = (dA + dA^T) diag(rk)
  __bf16* const sDT_lo = sDT + C * L64;
  __bf16* const sZ = reinterpret_cast<__bf16*>(lds + LY::kZ);
  __bf16* const sZ_lo = sZ + C * L64;
  double* const s_gam = reinterpret_cast<double*>(lds + LY::kGam);
  float* const s_b = reinterpret_cast<float*>(lds + LY::kB);
  float* const s_d = reinterpret_cast<float*>(lds + LY::kD);
  float* const s_rk = reinterpret_cast<float*>(lds + LY::kRk);
  float* const s_rq = reinterpret_cast<float*>(lds + LY::kRq);
  float* const s_beta = reinterpret_cast<float*>(lds + LY::kBeta);
  float* const s_rowg = reinterpret_cast<float*>(lds + LY::kRowG);
  float* const s_rowb = reinterpret_cast<float*>(lds + LY::kRowB);
  float* const s_colg = reinterpret_cast<float*>(lds + LY::kColG);
  float* const s_colb = reinterpret_cast<float*>(lds + LY::kColB);
  float* const s_dd = reinterpret_cast<float*>(lds + LY::kDd);
  float* const s_red = reinterpret_cast<float*>(lds + LY::kRed);

  const int64_t cs = blockIdx.x / h_v;
  const int h = static_cast<int>(blockIdx.x % h_v);
  int seq, len;
  int64_t t0;
  if (!locate_block(cu, n_seq, t_total, C, cs, seq, t0, len)) return;
  const int hq = h / (h_v / h_qk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int64_t vrow = static_cast<int64_t>(h_v) * D;
  const int64_t smat = (cs * h_v + h) * static_cast<int64_t>(D) * D;

  // 1. raw K, Q rows (zero past len) and their L2 scales; gates and decays
  {
    constexpr int TPR = D / 8, RPP = 256 / TPR;
#pragma unroll
    for (int it = 0; it < C / RPP; ++it) {
      const int row = it * RPP + tid / TPR, c8 = (tid % TPR) * 8;
      const int64_t tok = t0 + (row < len ? row : 0);
      typename PB::Raw8 kr = PB::load8(reinterpret_cast<const uint16_t*>(k) + tok * k_stride + (int64_t)hq * D + c8);
      typename PB::Raw8 qr = PB::load8(reinterpret_cast<const uint16_t*>(q) + tok * q_stride + (int64_t)hq * D + c8);
      float kv[8], qv[8];
      PB::commit8(sK + row * LDK + c8, kr, row < len, kv);
      PB::commit8(sQ + row * LDK + c8, qr, row < len, qv);
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { sk += kv[i] * kv[i]; sq += qv[i] * qv[i]; }
      sk = group_sum<TPR>(sk);
      sq = group_sum<TPR>(sq);
      if (tid % TPR == 0) {
        const bool valid = row < len;
        s_rk[row] = !valid ? 0.f : (use_l2 ? 1.0f / sqrtf(sk + l2_eps) : 1.0f);
        s_rq[row] = !valid ? 0.f : (use_l2 ? 1.0f / sqrtf(sq + l2_eps) : 1.0f);
      }
    }
    if (wave == 0) {
      float gv = 0.f, bv = 0.f;
      if (lane < len) load_gate(gates, t0 + lane, h, h_v, gv, bv);
      double gam = gv;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(gam, off, 64);
        if (lane >= off) gam += o;
      }
      const double glast = __shfl(gam, C - 1, 64);
      s_gam[lane] = gam;
      s_beta[lane] = bv;
      s_b[lane] = __expf(static_cast<float>(gam));
      s_d[lane] = __expf(static_cast<float>(glast - gam));
      if (lane == 0) s_red[0] = __expf(static_cast<float>(glast));   // b_C
    }
  }
  __syncthreads();

  // 2. Gram tiles of row tile `wave`: (wave, tj), tj <= wave.  Lane (r, g)
  //    holds element (i, j) = (16 wave + 4g + e, 16 tj + r).  LA = rk_i rk_j
  //    (k_i . k_j) D_ij below the diagonal, P = scale D_ij rq_i rk_j (q_i . k_j)
  //    on and below it; L = beta_i LA goes to LDS for the solve, P to LDS as
  //    hi|lo rows (zero above the diagonal).
  floatx4 Pt[4], LAt[4];
  const float bC = s_red[0];
  {
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      Pt[tj] = LAt[tj] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (tj <= wave) {
        floatx4 gk = {0.f, 0.f, 0.f, 0.f}, gq = gk;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const Frag kb = frag_rows(sK, LDK, 16 * tj, 32 * ks);
          gk = mfma_bf16(frag_rows(sK, LDK, 16 * wave, 32 * ks), kb, gk);
          gq = mfma_bf16(frag_rows(sQ, LDK, 16 * wave, 32 * ks), kb, gq);
        }
        const int j = 16 * tj + r16;
        const double gj = s_gam[j];
        const float rkj = s_rk[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * wave + 4 * g4 + e;
          const float dec = __expf(j <= i ? static_cast<float>(s_gam[i] - gj) : -INFINITY);
          const float la = j < i ? s_rk[i] * rkj * gk[e] * dec : 0.f;
          const float pv = j <= i ? scale * dec * s_rq[i] * rkj * gq[e] : 0.f;
          LAt[tj][e] = la;
          Pt[tj][e] = pv;
          sL[i * LDC + j] = s_beta[i] * la;
          put_hl(sP, sP_lo, i * L64 + j, pv);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) put_hl(sP, sP_lo, (16 * wave + 4 * g4 + e) * L64 + 16 * tj + r16, 0.f);
      }
    }
  }
  __syncthreads();

  // 3. T = (I + L)^-1 (fp32), then T as hi|lo rows (zero above the diagonal)
  unit_lower_inverse<C, LDC>(sL, sTf);
  for (int f = tid; f < C * C; f += 256) {
    const int i = f / C, j = f % C;
    put_hl(sT, sT_lo, i * L64 + j, j <= i ? sTf[i * LDC + j] : 0.f);
  }
  __syncthreads();

  // 4. the d_v parts: X, U, dU of 32 columns, then the sums over d_v
  floatx4 dOS[8], dXS[8], UdS[8], dPt[4], dTbt[4];
#pragma unroll
  for (int n = 0; n < 8; ++n) dOS[n] = dXS[n] = UdS[n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) dPt[tj] = dTbt[tj] = floatx4{0.f, 0.f, 0.f, 0.f};
  float sds = 0.f;   // this thread's part of <dS, S>
  const int ks0 = (16 * wave) / 32;
  const int i0 = 16 * wave + 4 * g4;   // this lane's first row in MFMA output tiles
  for (int p = 0; p < 4; ++p) {
    // a. stage S and dS rows 32p .. 32p + 31 (d_v) and dO columns 32p .. (tokens)
    {
      const int row = tid >> 3, c16 = (tid & 7) * 16;
      const float* sp = states + smat + (int64_t)(32 * p + row) * D + c16;
      const float* dp = dstates + smat + (int64_t)(32 * p + row) * D + c16;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 a = reinterpret_cast<const float4*>(sp)[u];
        const float4 b = reinterpret_cast<const float4*>(dp)[u];
        sds += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
        put4_hl(sS, sS_lo, row * LDK + c16 + 4 * u, a);
        put4_hl(sdS, sdS_lo, row * LDK + c16 + 4 * u, b);
      }
      const int tk = tid >> 2, c8 = (tid & 3) * 8;
      float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
      if (tk < len) {
        const float* src = d_o + (t0 + tk) * vrow + h * D + 32 * p + c8;
        x0 = reinterpret_cast<const float4*>(src)[0];
        x1 = reinterpret_cast<const float4*>(src)[1];
      }
      put4_hl(sDO, sDO_lo, tk * L32 + c8, x0);
      put4_hl(sDO, sDO_lo, tk * L32 + c8 + 4, x1);
    }
    __syncthreads();
    // b. X = V - diag(b rk) K S^T and K dS^T for this wave's 16 tokens
    floatx4 kds[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      floatx4 ks_ = {0.f, 0.f, 0.f, 0.f}, kd = ks_;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const Frag a = frag_rows(sK, LDK, 16 * wave, 32 * ks);
        ks_ = mfma_bf16(a, frag_rows(sS, LDK, 16 * nt, 32 * ks), ks_);
        ks_ = mfma_bf16(a, frag_rows(sS_lo, LDK, 16 * nt, 32 * ks), ks_);
        kd = mfma_bf16(a, frag_rows(sdS, LDK, 16 * nt, 32 * ks), kd);
        kd = mfma_bf16(a, frag_rows(sdS_lo, LDK, 16 * nt, 32 * ks), kd);
      }
      kds[nt] = kd;
      const int c = 16 * nt + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        const float vv = i < len ? In::load(v, (t0 + i) * v_stride + (int64_t)h * D + 32 * p + c) : 0.f;
        const float x = vv - s_b[i] * s_rk[i] * ks_[e];
        put_hl(sX, sX_lo, i * L32 + c, x);
        put_hl(sXb, sXb_lo, i * L32 + c, s_beta[i] * x);
      }
    }
    __syncthreads();
    // c. U = T (beta X) and dU = P^T dO + diag(d rk) K dS^T
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      floatx4 u = {0.f, 0.f, 0.f, 0.f}, du;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (32 * ks <= 16 * wave + 15)
          u = mma3(u, frag_rows(sT, L64, 16 * wave, 32 * ks), frag_rows(sT_lo, L64, 16 * wave, 32 * ks),
                   frag_cols(sXb, L32, 32 * ks, 16 * nt), frag_cols(sXb_lo, L32, 32 * ks, 16 * nt));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) du[e] = s_d[i0 + e] * s_rk[i0 + e] * kds[nt][e];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks >= ks0)
          du = mma3(du, frag_cols(sP, L64, 32 * ks, 16 * wave), frag_cols(sP_lo, L64, 32 * ks, 16 * wave),
                    frag_cols(sDO, L32, 32 * ks, 16 * nt), frag_cols(sDO_lo, L32, 32 * ks, 16 * nt));
      }
      const int c = 16 * nt + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        put_hl(sU, sU_lo, (i0 + e) * L32 + c, u[e]);
        put_hl(sDU, sDU_lo, (i0 + e) * L32 + c, du[e]);
      }
    }
    __syncthreads();
    // d. sums over this part's 32 d_v columns
    {
      const Frag aoh = frag_rows(sDO, L32, 16 * wave, 0), aol = frag_rows(sDO_lo, L32, 16 * wave, 0);
      const Frag auh = frag_rows(sU, L32, 16 * wave, 0), aul = frag_rows(sU_lo, L32, 16 * wave, 0);
      const Frag adh = frag_rows(sDU, L32, 16 * wave, 0), adl = frag_rows(sDU_lo, L32, 16 * wave, 0);
      Frag axh, axl;
      {
        const int row = 16 * wave + r16;
        float xv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (row < len) {
          const float* src = dvx + (t0 + row) * vrow + h * D + 32 * p + 8 * g4;
          const float4 a = reinterpret_cast<const float4*>(src)[0], b = reinterpret_cast<const float4*>(src)[1];
          xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
          xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
        }
        split8(xv, axh, axl);
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const Frag bsh = frag_cols(sS, LDK, 0, 16 * n), bsl = frag_cols(sS_lo, LDK, 0, 16 * n);
        const Frag bdh = frag_cols(sdS, LDK, 0, 16 * n), bdl = frag_cols(sdS_lo, LDK, 0, 16 * n);
        dOS[n] = mma3(dOS[n], aoh, aol, bsh, bsl);
        dXS[n] = mma3(dXS[n], axh, axl, bsh, bsl);
        UdS[n] = mma3(UdS[n], auh, aul, bdh, bdl);
      }
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        if (tj <= wave) {
          dPt[tj] = mma3(dPt[tj], aoh, aol, frag_rows(sU, L32, 16 * tj, 0), frag_rows(sU_lo, L32, 16 * tj, 0));
          dTbt[tj] = mma3(dTbt[tj], adh, adl, frag_rows(sX, L32, 16 * tj, 0), frag_rows(sX_lo, L32, 16 * tj, 0));
        }
      }
    }
    __syncthreads();
  }

  // 5. the C x C algebra.  Row sums of a wave's tiles belong to its own rows;
  //    column sums are left per wave and added in a fixed order.
  {
    float rowg[4] = {0.f, 0.f, 0.f, 0.f}, colg[4] = {0.f, 0.f, 0.f, 0.f}, colb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const int j = 16 * tj + r16;
      if (tj <= wave) {
        const double gj = s_gam[j];
        const float rkj = s_rk[j], bj = s_beta[j];
        float cg = 0.f, cb = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + e;
          const bool on = j <= i;
          const float dp = on ? dPt[tj][e] : 0.f;
          const float m1 = dp * Pt[tj][e];
          rowg[e] += m1;
          cg += m1;
          const float dec = __expf(on ? static_cast<float>(s_gam[i] - gj) : -INFINITY);
          const float aq = on ? scale * dp * dec : 0.f;
          put_hl(sAqk, sAqk_lo, i * L64 + j, aq * rkj);
          put_hl(sAqq, sAqq_lo, i * L64 + j, s_rq[i] * aq);
          const float dtb = on ? dTbt[tj][e] : 0.f;
          const float tij = static_cast<float>(sT[i * L64 + j]) + static_cast<float>(sT_lo[i * L64 + j]);
          cb += dtb * tij;
          put_hl(sDT, sDT_lo, i * L64 + j, dtb * bj);
        }
        colg[tj] = cg;
        colb[tj] = cb;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = (i0 + e) * L64 + j;
          put_hl(sAqk, sAqk_lo, idx, 0.f);
          put_hl(sAqq, sAqq_lo, idx, 0.f);
          put_hl(sDT, sDT_lo, idx, 0.f);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) rowg[e] = sum16(rowg[e]);
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const float cg = sum_groups(colg[tj]), cb = sum_groups(colb[tj]);
      if (g4 == 0) {
        s_colg[wave * C + 16 * tj + r16] = cg;
        s_colb[wave * C + 16 * tj + r16] = cb;
      }
    }
    if (r16 == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s_rowg[i0 + e] = rowg[e];
    }
  }
  __syncthreads();
  // Z = dT T^T on the tiles (wave, tj <= wave), zero above the diagonal
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) {
    if (tj <= wave) {
      floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        z = mma3(z, frag_rows(sDT, L64, 16 * wave, 32 * ks), frag_rows(sDT_lo, L64, 16 * wave, 32 * ks),
                 frag_rows(sT, L64, 16 * tj, 32 * ks), frag_rows(sT_lo, L64, 16 * tj, 32 * ks));
#pragma unroll
      for (int e = 0; e < 4; ++e) put_hl(sZ, sZ_lo, (i0 + e) * L64 + 16 * tj + r16, z[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) put_hl(sZ, sZ_lo, (i0 + e) * L64 + 16 * tj + r16, 0.f);
    }
  }
  __syncthreads();
  // dL = -T^T Z (strictly lower); its dgamma and dbeta terms; E = (dA + dA^T) diag(rk)
  {
    float rowg[4] = {0.f, 0.f, 0.f, 0.f}, rowb[4] = {0.f, 0.f, 0.f, 0.f}, colg[4] = {0.f, 0.f, 0.f, 0.f};
    floatx4 dAt[4];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      dAt[tj] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (tj <= wave) {
        floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks >= ks0)
            z = mma3(z, frag_cols(sT, L64, 32 * ks, 16 * wave), frag_cols(sT_lo, L64, 32 * ks, 16 * wave),
                     frag_cols(sZ, L64, 32 * ks, 16 * tj), frag_cols(sZ_lo, L64, 32 * ks, 16 * tj));
        }
        const int j = 16 * tj + r16;
        const double gj = s_gam[j];
        float cg = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + e;
          const bool on = j < i;
          const float dl = on ? -z[e] : 0.f;
          const float bi = s_beta[i];
          const float m2 = dl * bi * LAt[tj][e];
          rowg[e] += m2;
          cg += m2;
          rowb[e] += dl * LAt[tj][e];
          const float dec = __expf(on ? static_cast<float>(s_gam[i] - gj) : -INFINITY);
          dAt[tj][e] = on ? bi * dec * dl : 0.f;
        }
        colg[tj] = cg;
      }
    }
    // E overwrites dT, which no wave reads after the Z product
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      if (tj <= wave) {
        const int j = 16 * tj + r16;
        const float rkj = s_rk[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + e;
          if (j <= i) {
            put_hl(sDT, sDT_lo, i * L64 + j, dAt[tj][e] * rkj);
            put_hl(sDT, sDT_lo, j * L64 + i, dAt[tj][e] * s_rk[i]);
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rowg[e] = sum16(rowg[e]);
      rowb[e] = sum16(rowb[e]);
    }
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const float cg = sum_groups(colg[tj]);
      if (g4 == 0) s_colg[wave * C + 16 * tj + r16] += cg;
    }
    if (r16 == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_rowg[i0 + e] += rowg[e];
        s_rowb[i0 + e] = rowb[e];
      }
    }
  }
  // <dS, S> over the workgroup
  {
    float x = sds;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
    if (lane == 0) s_red[4 + wave] = x;
  }
  __syncthreads();

  // 6. dQ^ = scale diag(b) dO S + dAq diag(rk) K and dK^ = diag(d) U dS -
  //    diag(b) dX S + (diag(rq) dAq)^T Q + E K, for this wave's 16 rows; the
  //    row dots of the dgamma terms are taken before the products are added.
  {
    float t_row[4] = {0.f, 0.f, 0.f, 0.f}, dd_row[4] = {0.f, 0.f, 0.f, 0.f};
    float* qo = dqh + (t0 * h_v + h) * static_cast<int64_t>(D);
    float* ko = dkh + (t0 * h_v + h) * static_cast<int64_t>(D);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int c = 16 * n + r16;
      floatx4 aq, ak;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        const float qv = static_cast<float>(sQ[i * LDK + c]), kv = static_cast<float>(sK[i * LDK + c]);
        const float bi = s_b[i];
        const float qs = scale * bi * dOS[n][e];
        t_row[e] += s_rq[i] * qv * qs - bi * s_rk[i] * kv * dXS[n][e];
        dd_row[e] += s_d[i] * s_rk[i] * kv * UdS[n][e];
        aq[e] = qs;
        ak[e] = s_d[i] * UdS[n][e] - bi * dXS[n][e];
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const Frag kb = frag_cols(sK, LDK, 32 * ks, 16 * n);
        aq = mma2(aq, frag_rows(sAqk, L64, 16 * wave, 32 * ks), frag_rows(sAqk_lo, L64, 16 * wave, 32 * ks), kb);
        ak = mma2(ak, frag_cols(sAqq, L64, 32 * ks, 16 * wave), frag_cols(sAqq_lo, L64, 32 * ks, 16 * wave),
                  frag_cols(sQ, LDK, 32 * ks, 16 * n));
        ak = mma2(ak, frag_rows(sDT, L64, 16 * wave, 32 * ks), frag_rows(sDT_lo, L64, 16 * wave, 32 * ks), kb);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        if (i < len) {
          qo[(int64_t)i * vrow + c] = aq[e];
          ko[(int64_t)i * vrow + c] = ak[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t_row[e] = sum16(t_row[e]);
      dd_row[e] = sum16(dd_row[e]);
    }
    if (r16 == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_rowg[i0 + e] += t_row[e] - dd_row[e];
        s_dd[i0 + e] = dd_row[e];
      }
    }
  }
  __syncthreads();

  // 7. per token: dgamma, then dg = its suffix sum over the chunk, and dbeta
  if (wave == 0) {
    const int t = lane;
    float x = s_rowg[t] - (((s_colg[t] + s_colg[C + t]) + s_colg[2 * C + t]) + s_colg[3 * C + t]);
    const float db = s_rowb[t] + (((s_colb[t] + s_colb[C + t]) + s_colb[2 * C + t]) + s_colb[3 * C + t]);
    float dd = s_dd[t];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) dd += __shfl_xor(dd, m, 64);
    if (t == C - 1) x += dd + bC * (((s_red[4] + s_red[5]) + s_red[6]) + s_red[7]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(x, off, 64);
      if (t + off < 64) x += y;
    }
    if (t < len) {
      dg[(t0 + t) * h_v + h] = x;
      dbeta[(t0 + t) * h_v + h] = db;
    }
  }
}

// ---------------------------------------------------------------------------
// k_bwd_dqk: per (token, q/k head), dq^ and dk^ summed over the v-heads that
// read the q/k head (in head order), then dx = rx (dx^ - x^ (x^ . dx^)) with
// x^ = rx x, rx = 1 / sqrt(|x|^2 + eps) (or dx = dx^ without the L2 norm).
// 128 threads, one d_k element each.
// ---------------------------------------------------------------------------
template <class In>
__global__ __launch_bounds__(128) void k_bwd_dqk(const typename In::T* __restrict__ q,
                                                 const typename In::T* __restrict__ k, int64_t q_stride,
                                                 int64_t k_stride, int use_l2, float l2_eps, int h_qk, int h_v,
                                                 const float* __restrict__ dqh, const float* __restrict__ dkh,
                                                 float* __restrict__ dq, float* __restrict__ dk) {
  __shared__ float red[2][4];
  const int64_t t = blockIdx.x / h_qk;
  const int hq = static_cast<int>(blockIdx.x % h_qk);
  const int c = threadIdx.x, lane = c & 63, wv = c >> 6;
  const int grp = h_v / h_qk;
  float gq = 0.f, gk = 0.f;
  for (int i = 0; i < grp; ++i) {
    const int64_t row = (t * h_v + hq * grp + i) * BD + c;
    gq += dqh[row];
    gk += dkh[row];
  }
  float outq = gq, outk = gk;
  if (use_l2) {
    const float xq = In::load(q, t * q_stride + (int64_t)hq * BD + c);
    const float xk = In::load(k, t * k_stride + (int64_t)hq * BD + c);
    float v[4] = {xq * xq, xk * xk, xq * gq, xk * gk};
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] += __shfl_xor(v[u], m, 64);
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) red[wv][u] = v[u];
    }
    __syncthreads();
    const float sqq = red[0][0] + red[1][0], skk = red[0][1] + red[1][1];
    const float dq_ = red[0][2] + red[1][2], dk_ = red[0][3] + red[1][3];
    const float rq = 1.0f / sqrtf(sqq + l2_eps), rk = 1.0f / sqrtf(skk + l2_eps);
    // x^ . dx^ = rx (x . dx^)
    outq = rq * (gq - (rq * xq) * (rq * dq_));
    outk = rk * (gk - (rk * xk) * (rk * dk_));
  }
  dq[(t * h_qk + hq) * BD + c] = outq;
  dk[(t * h_qk + hq) * BD + c] = outk;
}

// Workspace of the chunked backward: the forward prep's regions (with Tb^T),
// the state entering and the gradient leaving each chunk, and dQ^, dK^ per
// v-head.
struct BwdChunkWs {
  ChunkWs w;
  float* dstates;
  float* dqh;
  float* dkh;
};
size_t bwd_chunk_al(size_t x) { return (x + 255) & ~size_t(255); }
size_t bwd_chunk_bytes(int h_qk, int h_v, int n_seq, int64_t t_total) {
  const int64_t slots = block_slots(t_total, n_seq, BC);
  const size_t ops = bwd_chunk_al(sizeof(__bf16) * slots * h_v * BW::op_elems);
  const size_t st = bwd_chunk_al(sizeof(float) * slots * h_v * BD * BD);
  const size_t dx = bwd_chunk_al(sizeof(float) * t_total * h_v * BD);
  return BW::bytes(slots, h_qk, h_v, n_seq) + ops + 2 * st + 2 * dx;
}
BwdChunkWs bwd_chunk_carve(void* base, int h_qk, int h_v, int n_seq, int64_t t_total) {
  const int64_t slots = block_slots(t_total, n_seq, BC);
  BwdChunkWs r;
  r.w = BW::carve(base, slots, h_qk, h_v, n_seq);
  char* b = static_cast<char*>(base) + BW::bytes(slots, h_qk, h_v, n_seq);
  r.w.tbt = b;
  b += bwd_chunk_al(sizeof(__bf16) * slots * h_v * BW::op_elems);
  r.w.states = reinterpret_cast<float*>(b);
  b += bwd_chunk_al(sizeof(float) * slots * h_v * BD * BD);
  r.dstates = reinterpret_cast<float*>(b);
  b += bwd_chunk_al(sizeof(float) * slots * h_v * BD * BD);
  r.dqh = reinterpret_cast<float*>(b);
  b += bwd_chunk_al(sizeof(float) * t_total * h_v * BD);
  r.dkh = reinterpret_cast<float*>(b);
  return r;
}

}  // namespace

size_t bwd_chunked_ws_bytes(int h_qk, int h_v, int n_seq, int64_t t_total) {
  return bwd_chunk_bytes(h_qk, h_v, n_seq, t_total);
}

hipError_t launch_chunk_bwd_chunked(const BwdArgs& a) {
  using T = uint16_t;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const int64_t slots = block_slots(a.t_total, a.n_seq, BC);
  BwdChunkWs w = bwd_chunk_carve(a.workspace, a.h_qk, a.h_v, a.n_seq, a.t_total);
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  if (slots > 0) {
    static const int per_cu = [] {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_chunk_prep<PB, BD, BC, true>, 256, 0) != hipSuccess ||
          n < 1)
        n = 1;
      return n;
    }();
    const int64_t units = slots * a.h_qk;
    const int64_t resident = static_cast<int64_t>(per_cu) * device_cu_count();
    const int64_t grid = units < resident ? units : resident;
    hipLaunchKernelGGL((k_chunk_prep<PB, BD, BC, true>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, q, k,
                       a.q_stride, a.k_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.cu, a.n_seq,
                       a.t_total, nullptr, w.w, slots);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (w.w.order) {
    hipError_t e = launch_seq_order(a.cu, a.n_seq, BC, w.w.order, st);
    if (e != hipSuccess) return e;
  }
  const int64_t nblk = static_cast<int64_t>(a.n_seq) * a.h_v * (BD / 16);
  if (nblk > 0) {
    hipLaunchKernelGGL((k_chunk_scan<PB, F32, BD, BC, 1, true>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st,
                       q, k, v, a.q_stride, a.k_stride, a.v_stride, a.h_qk, a.h_v, a.cu, a.n_seq, a.t_total, a.init,
                       nullptr, nullptr, nullptr, static_cast<float*>(nullptr), w.w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_bwd_dstate, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st, a.h_qk, a.h_v, a.cu,
                       a.n_seq, a.t_total, a.d_o, a.d_final, a.dv, a.d_init, w.dstates, w.w);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (slots > 0) {
    hipLaunchKernelGGL(k_bwd_grad<BF16>, dim3(static_cast<unsigned>(slots * a.h_v)), dim3(256), 0, st, q, k, v,
                       a.q_stride, a.k_stride, a.v_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.cu,
                       a.n_seq, a.t_total, a.d_o, a.dv, w.w.states, w.dstates, w.dqh, w.dkh, a.dg, a.dbeta);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.t_total > 0) {
    hipLaunchKernelGGL(k_bwd_dqk<BF16>, dim3(static_cast<unsigned>(a.t_total * a.h_qk)), dim3(128), 0, st, q, k,
                       a.q_stride, a.k_stride, a.use_l2, a.l2_eps, a.h_qk, a.h_v, w.dqh, w.dkh, a.dq, a.dk);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdn
