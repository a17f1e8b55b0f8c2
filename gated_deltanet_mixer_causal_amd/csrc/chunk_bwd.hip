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
//   dstate_body   the reverse scan, run as the prefix of that forward scan
//                 in the same launch: one workgroup per (sequence, v-head,
//                 16-wide d_v slice), chunks last to first, the slice of dS
//                 in fp32 registers: writes dS leaving each chunk, dV and
//                 dS_initial.  Three products per chunk with a barrier after
//                 each, like the forward scan.
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
// dstate_body: the gradient of the state, chunks last to first.  It runs in
// one launch with the forward scan that writes the state entering every
// chunk (k_bwd_scans below): the two read only the prep's workspace and
// write disjoint buffers.
// ---------------------------------------------------------------------------
// LDS (bf16 elements): dS rows (d_v) hi | lo; dO rows, double-buffered; c2 dO,
// double-buffered; dU rows; -c1 dX rows; the chunk's K rows; its Q rows.
struct DstateLds {
  static constexpr int LDT = BC, LDK = BD, LDKT = BD + 8;
  static constexpr int G = 0, DO = G + 2 * 16 * LDK, DOC = DO + 2 * 2 * 16 * LDT, DU = DOC + 2 * 2 * 16 * LDT,
                       DX = DU + 2 * 16 * LDT, KT = DX + 2 * 16 * LDT, QT = KT + BC * LDKT, end = QT + BC * LDKT;
  static constexpr size_t bytes = sizeof(__bf16) * end;
};

__device__ __forceinline__ void dstate_body(int64_t bidx, char* lds, int h_qk, int h_v,
                                            const int32_t* __restrict__ cu, int n_seq, int64_t t_total,
                                            const float* __restrict__ d_o, const float* __restrict__ d_final,
                                            float* __restrict__ dv, float* __restrict__ d_init,
                                            float* __restrict__ dstates, ChunkWs ws) {
  constexpr int D = BD, C = BC, KS = 32, NKS_D = D / KS, NKS_C = C / KS, NTILE = D / 16;
  constexpr int LDT = DstateLds::LDT, LDK = DstateLds::LDK, LDKT = DstateLds::LDKT;
  __bf16* const base = reinterpret_cast<__bf16*>(lds);
  __bf16* const sG = base + DstateLds::G;
  __bf16(*const sDO)[2 * 16 * LDT] = reinterpret_cast<__bf16(*)[2 * 16 * LDT]>(base + DstateLds::DO);
  __bf16(*const sDOc)[2 * 16 * LDT] = reinterpret_cast<__bf16(*)[2 * 16 * LDT]>(base + DstateLds::DOC);
  __bf16* const sDU = base + DstateLds::DU;
  __bf16* const sDX = base + DstateLds::DX;
  __bf16* const sKt = base + DstateLds::KT;
  __bf16* const sQt = base + DstateLds::QT;
  __bf16* const sG_lo = sG + 16 * LDK;
  __bf16* const sDU_lo = sDU + 16 * LDT;
  __bf16* const sDX_lo = sDX + 16 * LDT;

  const int64_t per_seq = static_cast<int64_t>(h_v) * NTILE;
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

  // Operands of one chunk (registers).  Each set is reloaded for the next
  // (earlier) chunk right after its last use in this one, so the loads are
  // spread over the three phases and every load has about a chunk step of
  // latency: K, Q, P^T and c3 after phase A, Tb^T and c1 after phase B, b_C
  // and dO (two chunks ahead) in phase C.
  Frag kf[NKS_D], qf[NKS_D], ph[NKS_C], pl[NKS_C], th[NKS_C], tl[NKS_C];
  float4 c1v, c3v;
  float bcv;
  auto unit_of = [&](int64_t jj) { return (slot0 + jj) * h_v + h; };
  auto load_kqp = [&](int64_t jj) {
    const __bf16* kq_ = static_cast<const __bf16*>(ws.kq) + ((slot0 + jj) * h_qk + hq) * BW::kq_elems + lane * 8;
#pragma unroll
    for (int ks = 0; ks < NKS_D; ++ks) {
      kf[ks] = PB::ld(kq_ + BW::kq_block(0, wave, ks));
      qf[ks] = PB::ld(kq_ + BW::kq_block(1, wave, ks));
    }
    const __bf16* p_ = static_cast<const __bf16*>(ws.p) + unit_of(jj) * BW::op_elems + lane * 8;
#pragma unroll
    for (int ks = 0; ks < NKS_C; ++ks) {
      if (ks >= ks0) {
        ph[ks] = PB::ld(p_ + BW::op_block(wave, ks, 0));
        pl[ks] = PB::ld(p_ + BW::op_block(wave, ks, 1));
      }
    }
    c3v = *reinterpret_cast<const float4*>(ws.sc + unit_of(jj) * (4 * C) + 2 * C + orow0);
  };
  auto load_tbt = [&](int64_t jj) {
    const __bf16* t_ = static_cast<const __bf16*>(ws.tbt) + unit_of(jj) * BW::op_elems + lane * 8;
#pragma unroll
    for (int ks = 0; ks < NKS_C; ++ks) {
      if (ks >= ks0) {
        th[ks] = PB::ld(t_ + BW::op_block(wave, ks, 0));
        tl[ks] = PB::ld(t_ + BW::op_block(wave, ks, 1));
      }
    }
    c1v = *reinterpret_cast<const float4*>(ws.sc + unit_of(jj) * (4 * C) + orow0);
  };
  // dO of chunk jj for the staging, in the layout of the MFMA outputs: this
  // lane's tokens orow0 .. orow0 + 3 at d_v column dv0 + r16 (one 8-byte LDS
  // run per array), and c2 of those tokens; rows past the end re-read the
  // last row and are zeroed at the staging
  auto load_do = [&](int64_t jj, float4& do_, float4& c2_) {
    const int64_t t0_ = start + jj * C;
    const int len_ = static_cast<int>(end - t0_ < C ? end - t0_ : C);
    c2_ = *reinterpret_cast<const float4*>(ws.sc + unit_of(jj) * (4 * C) + C + orow0);
    float t4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = orow0 + i < len_ ? orow0 + i : len_ - 1;
      t4[i] = d_o[(t0_ + r) * vrow + h * D + dv0 + r16];
    }
    do_ = make_float4(t4[0], t4[1], t4[2], t4[3]);
  };
  auto stage_do = [&](int buf, int64_t jj, float4 v4, float4 c2) {
    const int64_t t0_ = start + jj * C;
    const float v[4] = {v4.x, v4.y, v4.z, v4.w}, c[4] = {c2.x, c2.y, c2.z, c2.w};
    float a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = t0_ + orow0 + i < end ? v[i] : 0.f;
      b[i] = c[i] * a[i];
    }
    const int idx = swz_off<LDT>(r16, orow0 >> 3) + (orow0 & 7);
    PB::put4(sDO[buf], sDO[buf] + 16 * LDT, idx, a);
    PB::put4(sDOc[buf], sDOc[buf] + 16 * LDT, idx, b);
  };

  int buf = 0;
  float4 don, c2n;   // dO of the next chunk down, loaded a chunk before its staging
  if (nchunks > 0) {
    load_kqp(nchunks - 1);
    load_tbt(nchunks - 1);
    bcv = ws.sc[unit_of(nchunks - 1) * (4 * C) + 3 * C];
    float4 d0, c0;
    load_do(nchunks - 1, d0, c0);
    stage_do(0, nchunks - 1, d0, c0);
    load_do(nchunks > 1 ? nchunks - 2 : 0, don, c2n);
  }
  __syncthreads();

  for (int64_t j = nchunks - 1; j >= 0; --j) {
    const int64_t t0 = start + j * C;
    const int len = static_cast<int>(end - t0 < C ? end - t0 : C);
    const int64_t jn = j > 0 ? j - 1 : j;   // the next chunk down (the last step reloads its own)
    // the gradient of the state leaving this chunk
    {
      float* o = dstates + (((slot0 + j) * h_v + h) * D + dv0 + r16) * D;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        *reinterpret_cast<float4*>(o + 16 * (wave + 4 * jj) + 4 * g4) = make_float4(G[jj][0], G[jj][1], G[jj][2], G[jj][3]);
    }

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
    load_kqp(jn);   // K, Q, P^T and c3 of this chunk are consumed

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
    load_tbt(jn);   // Tb^T and c1 of this chunk are consumed

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
      stage_do(buf ^ 1, jn, don, c2n);
      bcv = ws.sc[unit_of(jn) * (4 * C) + 3 * C];
      load_do(j > 1 ? j - 2 : 0, don, c2n);
    }
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

// The reverse scan as the prefix of the forward scan that writes the state
// entering every chunk (k_chunk_scan's Pre argument): blocks [0, nblk) run
// it, and the forward scan takes the blocks after them.  The two read only
// the prep's workspace and write disjoint buffers; the reverse scan, the
// longer chain, takes the first blocks.  nblk is a multiple of 8, so both
// halves keep their XCD-aware block mapping.
struct DstatePrefix {
  static constexpr size_t kLdsBytes = DstateLds::bytes;
  int64_t nblk;
  const float* d_o;
  const float* d_final;
  float* dv;
  float* d_init;
  float* dstates;
  __device__ __forceinline__ void run(int64_t b, char* lds, int h_qk, int h_v, const int32_t* cu, int n_seq,
                                      int64_t t_total, const ChunkWs& ws) const {
    dstate_body(b, lds, h_qk, h_v, cu, n_seq, t_total, d_o, d_final, dv, d_init, dstates, ws);
  }
};

// ---------------------------------------------------------------------------
// k_bwd_grad: one workgroup of 8 waves per (chunk slot, v-head)
// ---------------------------------------------------------------------------
// Wave w works on token tile w % 4 (16 rows); the two waves of a tile split
// the products: half 0 (w < 4) holds L's decayed Gram tiles and forms X, U,
// dTb, then Z, dL and E; half 1 holds P and forms K dS^T, dU, dP and the
// staging of dAq.  The sums over d_v into d_k columns (dO S, dX S, U dS) and
// dQ^, dK^ are split by d_k: half h owns d_k tiles 4h .. 4h + 3.
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
  static constexpr int kRowG = kBeta + 4 * BC;   // [2 halves][64] row terms of dgamma
  static constexpr int kRowB = kRowG + 8 * BC;   // [64] row terms of dbeta
  static constexpr int kColG = kRowB + 4 * BC;   // [8 waves][64] column terms of dgamma
  static constexpr int kColB = kColG + 32 * BC;  // [4 waves][64] column terms of dbeta
  // 20 floats: b_C, <dS, S> per wave (4 ..), sum of d_j k^_j . (U dS)_j per wave (12 ..)
  static constexpr int kRed = kColB + 16 * BC;
  static constexpr int bytes = kRed + 80;
  static_assert(kTf + BC * LDC * 4 <= kUEnd, "solve fits the shared region");
  static_assert(bytes <= 160 * 1024, "one workgroup per CU");
};

template <class In>
__global__ __launch_bounds__(512) void k_bwd_grad(
    const typename In::T* __restrict__ q, const typename In::T* __restrict__ k, const typename In::T* __restrict__ v,
    int64_t q_stride, int64_t k_stride, int64_t v_stride, GateSrc gates, float scale, int use_l2, float l2_eps,
    int h_qk, int h_v, const int32_t* __restrict__ cu, int n_seq, int64_t t_total, const float* __restrict__ d_o,
    const float* __restrict__ dvx, const float* __restrict__ states, const float* __restrict__ dstates,
    float* __restrict__ dqh, float* __restrict__ dkh, float* __restrict__ dg, float* __restrict__ dbeta) {
  using LY = GradLds;
  constexpr int D = BD, C = BC, LDK = LY::LDK, L64 = LY::L64, L32 = LY::L32, LDC = LY::LDC, NTH = 512;
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
  float* const s_red = reinterpret_cast<float*>(lds + LY::kRed);

  const int64_t cs = blockIdx.x / h_v;
  const int h = static_cast<int>(blockIdx.x % h_v);
  int seq, len;
  int64_t t0;
  if (!locate_block(cu, n_seq, t_total, C, cs, seq, t0, len)) return;
  const int hq = h / (h_v / h_qk);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tile = wv & 3;
  const bool h0 = wv < 4;   // half 0 or half 1 (wave-uniform)
  const int r16 = lane & 15, g4 = lane >> 4;
  const int64_t vrow = static_cast<int64_t>(h_v) * D;
  const int64_t smat = (cs * h_v + h) * static_cast<int64_t>(D) * D;
  const int i0 = 16 * tile + 4 * g4;   // this lane's first row in MFMA output tiles
  const int ks0 = (16 * tile) / 32;

  // 1. raw K, Q rows (zero past len) and their L2 scales; gates and decays
  {
    constexpr int TPR = D / 8, RPP = NTH / TPR;
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
    if (wv == 0) {
      float gv, bv;
      load_gate(gates, t0 + (lane < len ? lane : len - 1), h, h_v, gv, bv);
      if (lane >= len) gv = bv = 0.f;
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

  // Inputs of one 32-wide d_v part, fetched into registers a part ahead:
  // S and dS rows (8 floats each per thread), dO (4 per thread), and this
  // lane's V values (half 0, X tiles) or dV values (half 1, A operand).
  // Rows past len re-read row len - 1 and are zeroed where they are used: a
  // select right after a load would wait for it there.
  struct PartIn {
    float4 s[2], ds[2], o;
  };
  // V at this lane's X tile elements (used by half 0), kept as raw bits and
  // converted where it is used: loaded under a branch, or converted on
  // arrival, it made the wave wait for the load right there
  auto fetch_vv = [&](int p, uint32_t* vv) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e < len ? i0 + e : len - 1;
        vv[4 * nt + e] = to_u32(v[(t0 + i) * v_stride + (int64_t)h * D + 32 * p + 16 * nt + r16]);
      }
  };
  auto fetch_xv = [&](int p, float* xv) {   // dV as this lane's A operand values
    const int xrow = 16 * tile + r16 < len ? 16 * tile + r16 : len - 1;
    const float* src = dvx + (t0 + xrow) * vrow + h * D + 32 * p + 8 * g4;
    const float4 a = reinterpret_cast<const float4*>(src)[0], b = reinterpret_cast<const float4*>(src)[1];
    xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
    xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
  };
  auto fetch_part = [&](int p, PartIn& r) {
    const int row = tid >> 4, c8 = (tid & 15) * 8;
    const float* sp = states + smat + (int64_t)(32 * p + row) * D + c8;
    const float* dp = dstates + smat + (int64_t)(32 * p + row) * D + c8;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      r.s[u] = reinterpret_cast<const float4*>(sp)[u];
      r.ds[u] = reinterpret_cast<const float4*>(dp)[u];
    }
    const int tk = tid >> 3, c4 = (tid & 7) * 4;
    r.o = *reinterpret_cast<const float4*>(d_o + (t0 + (tk < len ? tk : len - 1)) * vrow + h * D + 32 * p + c4);
  };
  PartIn nxt;

  // 2. Gram tiles of row tile `tile`: (tile, tj), tj <= tile; lane (r, g)
  //    holds element (i, j) = (16 tile + 4g + e, 16 tj + r).  Half 0: LA =
  //    rk_i rk_j (k_i . k_j) D_ij below the diagonal (L = beta_i LA to LDS for
  //    the solve); half 1: P = scale D_ij rq_i rk_j (q_i . k_j) on and below
  //    it (hi|lo rows to LDS, zero above the diagonal).  Ct keeps LA (half 0)
  //    or P (half 1).
  const float bC = s_red[0];
  {
    auto gram = [&](const __bf16* aop, int tj) {
      floatx4 gm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        gm = mfma_bf16(frag_rows(aop, LDK, 16 * tile, 32 * ks), frag_rows(sK, LDK, 16 * tj, 32 * ks), gm);
      return gm;
    };
    if (h0) {
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        if (tj <= tile) {
          const floatx4 gm = gram(sK, tj);
          const int j = 16 * tj + r16;
          const double gj = s_gam[j];
          const float rkj = s_rk[j];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            const float dec = __expf(j < i ? static_cast<float>(s_gam[i] - gj) : -INFINITY);
            sL[i * LDC + j] = s_beta[i] * s_rk[i] * rkj * gm[e] * dec;
          }
        }
      }
    } else {
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        float pv[4] = {0.f, 0.f, 0.f, 0.f};
        const int j = 16 * tj + r16;
        if (tj <= tile) {
          const floatx4 gm = gram(sQ, tj);
          const double gj = s_gam[j];
          const float rkj = s_rk[j];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            const float dec = __expf(j <= i ? static_cast<float>(s_gam[i] - gj) : -INFINITY);
            pv[e] = scale * dec * s_rq[i] * rkj * gm[e];
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) put_hl(sP, sP_lo, (i0 + e) * L64 + j, pv[e]);
      }
    }
  }
  __syncthreads();

  // 3. T = (I + L)^-1 (fp32), then T as hi|lo rows (zero above the diagonal)
  unit_lower_inverse<C, LDC>(sL, sTf);
  // after the solve, whose forward substitution holds many registers
  uint32_t vv[8];
  float xv[8];
  fetch_part(0, nxt);
  fetch_vv(0, vv);
  fetch_xv(0, xv);
  {
    // eight consecutive columns per thread: two 16-byte reads, 16-byte stores
    static_assert(C * C == 8 * NTH, "one pass of eight columns per thread");
    const int i = tid >> 3, j0 = (tid & 7) * 8;
    const float4 t0 = *reinterpret_cast<const float4*>(sTf + i * LDC + j0);
    const float4 t1 = *reinterpret_cast<const float4*>(sTf + i * LDC + j0 + 4);
    float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) tv[e] = j0 + e <= i ? tv[e] : 0.f;   // T above the diagonal is not written
    Frag th, tl;
    split8(tv, th, tl);
    *reinterpret_cast<Frag*>(sT + i * L64 + j0) = th;
    *reinterpret_cast<Frag*>(sT_lo + i * L64 + j0) = tl;
  }
  __syncthreads();

  // 4. the d_v parts: X, U, dU of 32 columns, then the sums over d_v:
  //    dOS, dXS, UdS on this half's d_k tiles nb .. nb + 3, and T4 = dTb
  //    (half 0) or dP (half 1).
  const int nb = h0 ? 0 : 4;
  floatx4 dOS[4], dXS[4], UdS[4], T4[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) dOS[n] = dXS[n] = UdS[n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) T4[tj] = floatx4{0.f, 0.f, 0.f, 0.f};
  float sds = 0.f;   // this thread's part of <dS, S>
#pragma unroll 1
  for (int p = 0; p < 4; ++p) {
    // the part whose inputs are fetched during this one (the last part
    // re-reads its own: a load under a branch is waited for at the join)
    const int pn = p < 3 ? p + 1 : 3;
    // a. stage S and dS rows 32p .. 32p + 31 (d_v) and dO columns 32p .. from
    //    the registers fetched a part ahead, then fetch the next part
    {
      const int row = tid >> 4, c8 = (tid & 15) * 8;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float4 a = nxt.s[u], b = nxt.ds[u];
        sds += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
        put4_hl(sS, sS_lo, row * LDK + c8 + 4 * u, a);
        put4_hl(sdS, sdS_lo, row * LDK + c8 + 4 * u, b);
      }
      const int tk = tid >> 3, c4 = (tid & 7) * 4;
      put4_hl(sDO, sDO_lo, tk * L32 + c4, tk < len ? nxt.o : make_float4(0.f, 0.f, 0.f, 0.f));
    }
    fetch_part(pn, nxt);
    __syncthreads();
    // b. half 0: X = V - diag(b rk) K S^T (and beta X); half 1: K dS^T
    floatx4 kds[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const __bf16* bh = h0 ? sS : sdS;
      const __bf16* bl = h0 ? sS_lo : sdS_lo;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const Frag a = frag_rows(sK, LDK, 16 * tile, 32 * ks);
        acc = mfma_bf16(a, frag_rows(bh, LDK, 16 * nt, 32 * ks), acc);
        acc = mfma_bf16(a, frag_rows(bl, LDK, 16 * nt, 32 * ks), acc);
      }
      kds[nt] = acc;
      if (h0) {
        const int c = 16 * nt + r16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + e;
          const float x = (i < len ? from_u32<In>(vv[4 * nt + e]) : 0.f) - s_b[i] * s_rk[i] * acc[e];
          put_hl(sX, sX_lo, i * L32 + c, x);
          put_hl(sXb, sXb_lo, i * L32 + c, s_beta[i] * x);
        }
      }
    }
    fetch_vv(pn, vv);
    __syncthreads();
    // c. half 0: U = T (beta X); half 1: dU = P^T dO + diag(d rk) K dS^T
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      floatx4 u = {0.f, 0.f, 0.f, 0.f};
      if (h0) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (32 * ks <= 16 * tile + 15)
            u = mma3(u, frag_rows(sT, L64, 16 * tile, 32 * ks), frag_rows(sT_lo, L64, 16 * tile, 32 * ks),
                     frag_cols(sXb, L32, 32 * ks, 16 * nt), frag_cols(sXb_lo, L32, 32 * ks, 16 * nt));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = s_d[i0 + e] * s_rk[i0 + e] * kds[nt][e];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks >= ks0)
            u = mma3(u, frag_cols(sP, L64, 32 * ks, 16 * tile), frag_cols(sP_lo, L64, 32 * ks, 16 * tile),
                     frag_cols(sDO, L32, 32 * ks, 16 * nt), frag_cols(sDO_lo, L32, 32 * ks, 16 * nt));
        }
      }
      __bf16* oh = h0 ? sU : sDU;
      __bf16* ol = h0 ? sU_lo : sDU_lo;
      const int c = 16 * nt + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) put_hl(oh, ol, (i0 + e) * L32 + c, u[e]);
    }
    __syncthreads();
    // d. sums over this part's 32 d_v columns
    {
      const Frag aoh = frag_rows(sDO, L32, 16 * tile, 0), aol = frag_rows(sDO_lo, L32, 16 * tile, 0);
      const Frag auh = frag_rows(sU, L32, 16 * tile, 0), aul = frag_rows(sU_lo, L32, 16 * tile, 0);
      Frag axh, axl;
      {
        float xm[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xm[e] = 16 * tile + r16 < len ? xv[e] : 0.f;
        split8(xm, axh, axl);
      }
      fetch_xv(pn, xv);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int c0 = 16 * (nb + n);
        const Frag bsh = frag_cols(sS, LDK, 0, c0), bsl = frag_cols(sS_lo, LDK, 0, c0);
        dOS[n] = mma3(dOS[n], aoh, aol, bsh, bsl);
        dXS[n] = mma3(dXS[n], axh, axl, bsh, bsl);
        UdS[n] = mma3(UdS[n], auh, aul, frag_cols(sdS, LDK, 0, c0), frag_cols(sdS_lo, LDK, 0, c0));
      }
      const Frag ath = h0 ? frag_rows(sDU, L32, 16 * tile, 0) : aoh;
      const Frag atl = h0 ? frag_rows(sDU_lo, L32, 16 * tile, 0) : aol;
      const __bf16* bt = h0 ? sX : sU;
      const __bf16* btl = h0 ? sX_lo : sU_lo;
#pragma unroll
      for (int tj = 0; tj < 4; ++tj)
        if (tj <= tile)
          T4[tj] = mma3(T4[tj], ath, atl, frag_rows(bt, L32, 16 * tj, 0), frag_rows(btl, L32, 16 * tj, 0));
    }
    __syncthreads();
  }

  // 5. the C x C algebra.  Row sums of a wave's tiles belong to its own rows;
  //    column sums are left per wave and added in a fixed order.
  //    Half 1: dP (masked) with P: its dgamma terms and dAq (two scalings);
  //    half 0: dTb (masked) with T: dbeta's column terms and dT.
  {
    float rowa[4] = {0.f, 0.f, 0.f, 0.f}, cola[4] = {0.f, 0.f, 0.f, 0.f};
    if (!h0) {
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        const int j = 16 * tj + r16;
        float ak[4] = {0.f, 0.f, 0.f, 0.f}, aqq[4] = {0.f, 0.f, 0.f, 0.f};
        if (tj <= tile) {
          const double gj = s_gam[j];
          const float rkj = s_rk[j];
          float ca = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            const bool on = j <= i;
            const float x = on ? T4[tj][e] : 0.f;
            const float m1 = x * (static_cast<float>(sP[i * L64 + j]) + static_cast<float>(sP_lo[i * L64 + j]));
            rowa[e] += m1;
            ca += m1;
            const float aq = scale * x * __expf(on ? static_cast<float>(s_gam[i] - gj) : -INFINITY);
            ak[e] = aq * rkj;
            aqq[e] = s_rq[i] * aq;
          }
          cola[tj] = ca;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          put_hl(sAqk, sAqk_lo, (i0 + e) * L64 + j, ak[e]);
          put_hl(sAqq, sAqq_lo, (i0 + e) * L64 + j, aqq[e]);
        }
      }
    } else {
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        const int j = 16 * tj + r16;
        float dt[4] = {0.f, 0.f, 0.f, 0.f};
        if (tj <= tile) {
          const float bj = s_beta[j];
          float ca = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            const float x = j <= i ? T4[tj][e] : 0.f;
            const float tij = static_cast<float>(sT[i * L64 + j]) + static_cast<float>(sT_lo[i * L64 + j]);
            ca += x * tij;
            dt[e] = x * bj;
          }
          cola[tj] = ca;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) put_hl(sDT, sDT_lo, (i0 + e) * L64 + j, dt[e]);
      }
    }
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const float c_ = sum_groups(cola[tj]);
      if (g4 == 0) {
        if (h0) s_colb[tile * C + 16 * tj + r16] = c_;
        else s_colg[wv * C + 16 * tj + r16] = c_;
      }
    }
    if (!h0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) rowa[e] = sum16(rowa[e]);
      if (r16 == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s_rowg[C + i0 + e] = rowa[e];
      }
    }
  }
  // <dS, S> over the workgroup
  {
    float x = sds;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
    if (lane == 0) s_red[4 + wv] = x;
  }
  __syncthreads();

  // 6. dQ^ = scale diag(b) dO S + dAq diag(rk) K and dK^ = diag(d) U dS -
  //    diag(b) dX S + (diag(rq) dAq)^T Q + E K on this half's d_k tiles, the
  //    row dots of their dgamma terms taken before the products are added;
  //    meanwhile half 0 forms Z = dT T^T, then dL = -T^T Z and E.
  floatx4 dq4[4], dk4[4];
  {
    float t_row[4] = {0.f, 0.f, 0.f, 0.f}, dd_row[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int c = 16 * (nb + n) + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        const float qv = static_cast<float>(sQ[i * LDK + c]), kv = static_cast<float>(sK[i * LDK + c]);
        const float bi = s_b[i], qs = scale * bi * dOS[n][e], ud = s_d[i] * UdS[n][e];
        t_row[e] += s_rq[i] * qv * qs - bi * s_rk[i] * kv * dXS[n][e];
        dd_row[e] += s_rk[i] * kv * ud;
        dq4[n][e] = qs;
        dk4[n][e] = ud - bi * dXS[n][e];
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const Frag kb = frag_cols(sK, LDK, 32 * ks, 16 * (nb + n));
        dq4[n] = mma2(dq4[n], frag_rows(sAqk, L64, 16 * tile, 32 * ks), frag_rows(sAqk_lo, L64, 16 * tile, 32 * ks),
                      kb);
        dk4[n] = mma2(dk4[n], frag_cols(sAqq, L64, 32 * ks, 16 * tile), frag_cols(sAqq_lo, L64, 32 * ks, 16 * tile),
                      frag_cols(sQ, LDK, 32 * ks, 16 * (nb + n)));
      }
      // one tile's operand reads at a time (registers)
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t_row[e] = sum16(t_row[e]);
      dd_row[e] = sum16(dd_row[e]);
    }
    if (r16 == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (h0) s_rowg[i0 + e] = t_row[e] - dd_row[e];
        else s_rowg[C + i0 + e] += t_row[e] - dd_row[e];
      }
    }
    const float ddw = sum_groups(((dd_row[0] + dd_row[1]) + dd_row[2]) + dd_row[3]);
    if (lane == 0) s_red[12 + wv] = ddw;
  }
  if (h0) {
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      if (tj <= tile) {
        floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          z = mma3(z, frag_rows(sDT, L64, 16 * tile, 32 * ks), frag_rows(sDT_lo, L64, 16 * tile, 32 * ks),
                   frag_rows(sT, L64, 16 * tj, 32 * ks), frag_rows(sT_lo, L64, 16 * tj, 32 * ks));
#pragma unroll
        for (int e = 0; e < 4; ++e) put_hl(sZ, sZ_lo, (i0 + e) * L64 + 16 * tj + r16, z[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) put_hl(sZ, sZ_lo, (i0 + e) * L64 + 16 * tj + r16, 0.f);
      }
    }
  }
  __syncthreads();
  if (h0) {
    // dL = -T^T Z (strictly lower); its dgamma and dbeta terms; E = (dA + dA^T) diag(rk)
    float rowg[4] = {0.f, 0.f, 0.f, 0.f}, rowb[4] = {0.f, 0.f, 0.f, 0.f}, colg[4] = {0.f, 0.f, 0.f, 0.f};
    floatx4 dAt[4];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      dAt[tj] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (tj <= tile) {
        floatx4 z = {0.f, 0.f, 0.f, 0.f}, gk = z;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks >= ks0)
            z = mma3(z, frag_cols(sT, L64, 32 * ks, 16 * tile), frag_cols(sT_lo, L64, 32 * ks, 16 * tile),
                     frag_cols(sZ, L64, 32 * ks, 16 * tj), frag_cols(sZ_lo, L64, 32 * ks, 16 * tj));
        }
        // the K K^T tile again (raw operands, exact products)
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
          gk = mfma_bf16(frag_rows(sK, LDK, 16 * tile, 32 * ks), frag_rows(sK, LDK, 16 * tj, 32 * ks), gk);
        const int j = 16 * tj + r16;
        const double gj = s_gam[j];
        const float rkj = s_rk[j];
        float cg = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + e;
          const bool on = j < i;
          const float dl = on ? -z[e] : 0.f;
          const float bi = s_beta[i];
          const float dec = __expf(on ? static_cast<float>(s_gam[i] - gj) : -INFINITY);
          const float la = on ? s_rk[i] * rkj * gk[e] * dec : 0.f;
          const float m2 = dl * bi * la;
          rowg[e] += m2;
          cg += m2;
          rowb[e] += dl * la;
          dAt[tj][e] = on ? bi * dec * dl : 0.f;
        }
        colg[tj] = cg;
      }
    }
    // E overwrites dT, which no wave reads after the Z product
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      if (tj <= tile) {
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
      if (g4 == 0) s_colg[wv * C + 16 * tj + r16] = cg;
    }
    if (r16 == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_rowg[i0 + e] += rowg[e];
        s_rowb[i0 + e] = rowb[e];
      }
    }
  }
  __syncthreads();
  {
    float* oq = dqh + (t0 * h_v + h) * static_cast<int64_t>(D);
    float* ok = dkh + (t0 * h_v + h) * static_cast<int64_t>(D);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        dk4[n] = mma2(dk4[n], frag_rows(sDT, L64, 16 * tile, 32 * ks), frag_rows(sDT_lo, L64, 16 * tile, 32 * ks),
                      frag_cols(sK, LDK, 32 * ks, 16 * (nb + n)));
      const int c = 16 * (nb + n) + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (i0 + e < len) {
          oq[(int64_t)(i0 + e) * vrow + c] = dq4[n][e];
          ok[(int64_t)(i0 + e) * vrow + c] = dk4[n][e];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();

  // 7. per token: dgamma, then dg = its suffix sum over the chunk, and dbeta
  if (wv == 0) {
    const int t = lane;
    float cg = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) cg += s_colg[w * C + t];
    float x = (s_rowg[t] + s_rowg[C + t]) - cg;
    const float db = s_rowb[t] + (((s_colb[t] + s_colb[C + t]) + s_colb[2 * C + t]) + s_colb[3 * C + t]);
    float dd = 0.f, sd = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      dd += s_red[12 + w];
      sd += s_red[4 + w];
    }
    if (t == C - 1) x += dd + bC * sd;
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
// k_bwd_dqk: per (token, q/k head) row, dq^ and dk^ summed over the v-heads
// that read the q/k head (in head order), then dx = rx (dx^ - x^ (x^ . dx^))
// with x^ = rx x, rx = 1 / sqrt(|x|^2 + eps) (or dx = dx^ without the L2
// norm).  16 lanes per row, 8 consecutive elements each; 16 rows per
// workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_dqk(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                 int64_t q_stride, int64_t k_stride, int use_l2, float l2_eps,
                                                 int h_qk, int h_v, int64_t t_total, const float* __restrict__ dqh,
                                                 const float* __restrict__ dkh, float* __restrict__ dq,
                                                 float* __restrict__ dk) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  if (row >= t_total * h_qk) return;   // whole 16-lane groups leave together
  const int64_t t = row / h_qk;
  const int hq = static_cast<int>(row % h_qk);
  const int c8 = (threadIdx.x & 15) * 8;
  const int grp = h_v / h_qk;
  float gq[8], gk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gq[e] = gk[e] = 0.f;
  for (int i = 0; i < grp; ++i) {
    const int64_t off = (t * h_v + hq * grp + i) * BD + c8;
    const float4 a0 = *reinterpret_cast<const float4*>(dqh + off), a1 = *reinterpret_cast<const float4*>(dqh + off + 4);
    const float4 b0 = *reinterpret_cast<const float4*>(dkh + off), b1 = *reinterpret_cast<const float4*>(dkh + off + 4);
    gq[0] += a0.x; gq[1] += a0.y; gq[2] += a0.z; gq[3] += a0.w;
    gq[4] += a1.x; gq[5] += a1.y; gq[6] += a1.z; gq[7] += a1.w;
    gk[0] += b0.x; gk[1] += b0.y; gk[2] += b0.z; gk[3] += b0.w;
    gk[4] += b1.x; gk[5] += b1.y; gk[6] += b1.z; gk[7] += b1.w;
  }
  if (use_l2) {
    const uint4 rq = *reinterpret_cast<const uint4*>(q + t * q_stride + (int64_t)hq * BD + c8);
    const uint4 rk = *reinterpret_cast<const uint4*>(k + t * k_stride + (int64_t)hq * BD + c8);
    const uint32_t wq[4] = {rq.x, rq.y, rq.z, rq.w}, wk[4] = {rk.x, rk.y, rk.z, rk.w};
    float xq[8], xk[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xq[2 * u] = __uint_as_float(wq[u] << 16);
      xq[2 * u + 1] = __uint_as_float(wq[u] & 0xffff0000u);
      xk[2 * u] = __uint_as_float(wk[u] << 16);
      xk[2 * u + 1] = __uint_as_float(wk[u] & 0xffff0000u);
    }
    float sqq = 0.f, skk = 0.f, sqg = 0.f, skg = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sqq += xq[e] * xq[e];
      skk += xk[e] * xk[e];
      sqg += xq[e] * gq[e];
      skg += xk[e] * gk[e];
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      sqq += __shfl_xor(sqq, m, 64);
      skk += __shfl_xor(skk, m, 64);
      sqg += __shfl_xor(sqg, m, 64);
      skg += __shfl_xor(skg, m, 64);
    }
    const float rqn = 1.0f / sqrtf(sqq + l2_eps), rkn = 1.0f / sqrtf(skk + l2_eps);
    // x^ . dx^ = rx (x . dx^)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gq[e] = rqn * (gq[e] - (rqn * xq[e]) * (rqn * sqg));
      gk[e] = rkn * (gk[e] - (rkn * xk[e]) * (rkn * skg));
    }
  }
  float* oq = dq + row * BD + c8;
  float* ok = dk + row * BD + c8;
  *reinterpret_cast<float4*>(oq) = make_float4(gq[0], gq[1], gq[2], gq[3]);
  *reinterpret_cast<float4*>(oq + 4) = make_float4(gq[4], gq[5], gq[6], gq[7]);
  *reinterpret_cast<float4*>(ok) = make_float4(gk[0], gk[1], gk[2], gk[3]);
  *reinterpret_cast<float4*>(ok + 4) = make_float4(gk[4], gk[5], gk[6], gk[7]);
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
    hipLaunchKernelGGL((k_chunk_scan<PB, F32, BD, BC, 1, true, DstatePrefix>), dim3(static_cast<unsigned>(2 * nblk)),
                       dim3(256), 0, st, q, k, v, a.q_stride, a.k_stride, a.v_stride, a.h_qk, a.h_v, a.cu, a.n_seq,
                       a.t_total, a.init, nullptr, nullptr, nullptr, static_cast<float*>(nullptr), w.w,
                       DstatePrefix{nblk, a.d_o, a.d_final, a.dv, a.d_init, w.dstates});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (slots > 0) {
    hipLaunchKernelGGL(k_bwd_grad<BF16>, dim3(static_cast<unsigned>(slots * a.h_v)), dim3(512), 0, st, q, k, v,
                       a.q_stride, a.k_stride, a.v_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.cu,
                       a.n_seq, a.t_total, a.d_o, a.dv, w.w.states, w.dstates, w.dqh, w.dkh, a.dg, a.dbeta);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.t_total > 0) {
    const int64_t rows = a.t_total * a.h_qk;
    hipLaunchKernelGGL(k_bwd_dqk, dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0, st, q, k,
                       a.q_stride, a.k_stride, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.t_total, w.dqh, w.dkh, a.dq,
                       a.dk);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdn
