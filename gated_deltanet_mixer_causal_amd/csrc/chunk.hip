// Chunked prefill of the gated delta rule (UT/WY form) for gfx950.
//
// Recurrence, per sequence and v-head with fp32 state S (d_v x d_k):
//     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = scale S_t q_t
// (the gated delta rule of the GDN layers: haskell-infer-demo README,
// "Highlights" and "Architecture"/fla_gdn.cu; fp32 state and bf16
// intermediates: Flare core-design, GDN numerics paragraph).
//
// Chunk algebra.  Within a chunk of C tokens entering with state S0, raw
// q/k rows (as stored), rk = 1/|k| and rq = 1/|q| (L2 norm), gamma = inclusive
// cumsum of g and b = exp(gamma):
//     L_ij = beta_i exp(gamma_i - gamma_j) rk_i rk_j (k_i . k_j),  j < i
//     Tb   = (I + L)^-1 diag(beta)
//     X    = V - diag(b rk) K S0^T          error of the decayed entering state
//     U    = Tb X                           the per-token delta-rule writes
//     O    = diag(scale b rq) Q S0^T + P U, P_ij = scale exp(gamma_i-gamma_j) rq_i rk_j (q_i . k_j), j <= i
//     S_C  = b_C S0 + U^T diag(exp(gamma_C - gamma) rk) K
// U solves u_i = beta_i (v_i - a_i S_{i-1} k^_i) for every token of the chunk.
//
// Two kernels:
//   k_chunk_prep  one workgroup per (chunk, q/k head): the Gram matrices K K^T
//                 and Q K^T on the matrix cores (raw operands, exact products),
//                 then per v-head of the group the decay scalars, L, P and the
//                 unit-lower-triangular solve (16x16 diagonal blocks by forward
//                 substitution in registers, off-diagonal blocks by fp32 MFMA).
//                 Writes Tb, P and the per-token scalars to the workspace.
//   k_chunk_scan  one workgroup per (sequence, v-head, 16-wide d_v tile),
//                 walking the sequence's chunks in order with its slice of the
//                 state held in fp32 registers; every contraction with the state
//                 or a derived operand runs on the matrix cores.
//
// Operand precision (policy PolBF16): raw bf16 q/k/v are exact single bf16
// operands; derived operands (S, X, U, Tb, P) are bf16 hi+lo pairs and a
// product uses hi*hi + hi*lo + lo*hi (or hi*raw + lo*raw), accumulated in fp32
// (the multi-term bf16 technique of Henry, Tang and Heinecke, ARITH 2019).
// Policy PolF32 uses the fp32 matrix-core instruction for fp32 inputs.
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

__device__ __forceinline__ floatx4 mfma_bf16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Operands in LDS are "k-contiguous": A as [m][k] and B as [n][k].  A 16x16
// tile product accumulates acc[i] += sum_k A[4g+i][k] * B[r][k] -- the
// matrix-core output layout: lane (r = lane%16, g = lane/16) holds column r,
// rows 4g..4g+3.
struct PolBF16 {
  using In = BF16;
  using Elem = __bf16;
  static constexpr int KSTEP = 32;
  static constexpr int PAD = 8;
  static constexpr int NSPLIT = 2;   // hi and lo arrays

  template <bool ALO, bool BLO>
  __device__ __forceinline__ static void mma(floatx4& acc, const Elem* a_hi, const Elem* a_lo, int lda,
                                             const Elem* b_hi, const Elem* b_lo, int ldb, int nks) {
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    for (int ks = 0; ks < nks; ++ks) {
      const int off = ks * 32 + 8 * g;
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(a_hi + r * lda + off);
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(b_hi + r * ldb + off);
      acc = mfma_bf16(ah, bh, acc);
      if constexpr (ALO) {
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(a_lo + r * lda + off);
        acc = mfma_bf16(al, bh, acc);
      }
      if constexpr (BLO) {
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(b_lo + r * ldb + off);
        acc = mfma_bf16(ah, bl, acc);
      }
    }
  }
  // Split store of 4 consecutive values.
  __device__ __forceinline__ static void put4(Elem* hi, Elem* lo, int idx, const float* v) {
    bf16x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __bf16 a, b;
      split_bf16(v[i], a, b);
      h[i] = a;
      l[i] = b;
    }
    *reinterpret_cast<bf16x4*>(hi + idx) = h;
    *reinterpret_cast<bf16x4*>(lo + idx) = l;
  }
  __device__ __forceinline__ static void put_raw(Elem* p, int idx, float v) { p[idx] = f32_to_bf16(v); }
  // 8 consecutive raw input elements: copy bits to LDS, return values.
  __device__ __forceinline__ static void stage8(Elem* dst, const uint16_t* src, bool valid, float* f) {
    uint4 r = valid ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(dst) = r;
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

struct PolF32 {
  using In = F32;
  using Elem = float;
  static constexpr int KSTEP = 4;
  static constexpr int PAD = 4;
  static constexpr int NSPLIT = 1;   // fp32 operands need no lo part

  template <bool ALO, bool BLO>
  __device__ __forceinline__ static void mma(floatx4& acc, const Elem* a_hi, const Elem*, int lda,
                                             const Elem* b_hi, const Elem*, int ldb, int nks) {
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    for (int ks = 0; ks < nks; ++ks) {
      const int off = ks * 4 + g;
      acc = mfma_f32(a_hi[r * lda + off], b_hi[r * ldb + off], acc);
    }
  }
  __device__ __forceinline__ static void put4(Elem* hi, Elem*, int idx, const float* v) {
    *reinterpret_cast<float4*>(hi + idx) = make_float4(v[0], v[1], v[2], v[3]);
  }
  __device__ __forceinline__ static void put_raw(Elem* p, int idx, float v) { p[idx] = v; }
  __device__ __forceinline__ static void stage8(Elem* dst, const float* src, bool valid, float* f) {
    float4 a = valid ? reinterpret_cast<const float4*>(src)[0] : make_float4(0, 0, 0, 0);
    float4 b = valid ? reinterpret_cast<const float4*>(src)[1] : make_float4(0, 0, 0, 0);
    reinterpret_cast<float4*>(dst)[0] = a;
    reinterpret_cast<float4*>(dst)[1] = b;
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

// Workspace regions, indexed by (chunk slot, v-head).
struct ChunkWs {
  float* tb;   // [slots][h_v][C][C]  T diag(beta), row-major
  float* p;    // [slots][h_v][C][C]  P (scale folded in), row-major
  float* sc;   // [slots][h_v][4][C]  b rk | scale b rq | exp(gamma_C - gamma) rk | b_C
};

// ---------------------------------------------------------------------------
// k_chunk_prep
// ---------------------------------------------------------------------------
template <class Pol, int D, int C>
__global__ __launch_bounds__(256) void k_chunk_prep(
    const typename Pol::In::T* __restrict__ q, const typename Pol::In::T* __restrict__ k,
    int64_t q_stride, int64_t k_stride, const float* __restrict__ g, const float* __restrict__ beta,
    float scale, int use_l2, float l2_eps, int h_qk, int h_v,
    const int32_t* __restrict__ cu, int n_seq, int64_t t_total, ChunkWs ws) {
  using Elem = typename Pol::Elem;
  constexpr int LDK = D + Pol::PAD;
  constexpr int LDC = C + 4;
  constexpr int NT = C / 16;
  static_assert(C % 16 == 0 && D % 16 == 0 && C <= 64, "tile shape");
  static_assert(D % Pol::KSTEP == 0, "k-steps must tile D");

  __shared__ __attribute__((aligned(16))) Elem sK[C * LDK];
  __shared__ __attribute__((aligned(16))) Elem sQ[C * LDK];
  __shared__ float sGK[C * LDC], sGQ[C * LDC], sL[C * LDC], sT[C * LDC];
  __shared__ float s_rk[C], s_rq[C], s_gam[C], s_beta[C];

  int seq, len;
  int64_t t0;
  if (!locate_block(cu, n_seq, t_total, C, blockIdx.x, seq, t0, len)) return;
  const int hq = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int grp = h_v / h_qk;

  // 1. raw K, Q rows of the chunk into LDS (zero beyond len) and their L2 scales
  {
    constexpr int TPR = D / 8, RPP = 256 / TPR;
    for (int r0 = 0; r0 < C; r0 += RPP) {
      const int row = r0 + tid / TPR, c8 = (tid % TPR) * 8;
      float kv[8] = {0, 0, 0, 0, 0, 0, 0, 0}, qv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (row < C) {
        const bool valid = row < len;
        const int64_t tok = t0 + (valid ? row : 0);
        Pol::stage8(sK + row * LDK + c8, k + tok * k_stride + (int64_t)hq * D + c8, valid, kv);
        Pol::stage8(sQ + row * LDK + c8, q + tok * q_stride + (int64_t)hq * D + c8, valid, qv);
      }
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { sk += kv[i] * kv[i]; sq += qv[i] * qv[i]; }
      sk = group_sum<TPR>(sk);
      sq = group_sum<TPR>(sq);
      if (row < C && tid % TPR == 0) {
        const bool valid = row < len;
        s_rk[row] = !valid ? 0.f : (use_l2 ? 1.0f / sqrtf(sk + l2_eps) : 1.0f);
        s_rq[row] = !valid ? 0.f : (use_l2 ? 1.0f / sqrtf(sq + l2_eps) : 1.0f);
      }
    }
  }
  __syncthreads();

  // 2. lower-triangular tiles of K K^T and Q K^T (raw operands, exact products)
  {
    constexpr int NLT = NT * (NT + 1) / 2;
    for (int task = wave; task < 2 * NLT; task += 4) {
      const bool isq = task >= NLT;
      const int idx = isq ? task - NLT : task;
      int ti = 0;
      while ((ti + 1) * (ti + 2) / 2 <= idx) ++ti;
      const int tj = idx - ti * (ti + 1) / 2;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      Pol::template mma<false, false>(acc, (isq ? sQ : sK) + ti * 16 * LDK, nullptr, LDK,
                                      sK + tj * 16 * LDK, nullptr, LDK, D / Pol::KSTEP);
      float* dst = isq ? sGQ : sGK;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * ti + 4 * g4 + i) * LDC + 16 * tj + r16] = acc[i];
    }
  }
  __syncthreads();

  for (int gi = 0; gi < grp; ++gi) {
    const int h = hq * grp + gi;
    const int64_t unit = (int64_t)blockIdx.x * h_v + h;
    float* sc_out = ws.sc + unit * (4 * C);

    // 3. decay: inclusive prefix sum of g over the chunk (padded tokens add 0)
    if (wave == 0) {
      float gv = 0.f, bv = 0.f;
      if (lane < len) {
        gv = g[(t0 + lane) * h_v + h];
        bv = beta[(t0 + lane) * h_v + h];
      }
      float gam = gv;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(gam, off, 64);
        if (lane >= off) gam += o;
      }
      const float glast = __shfl(gam, C - 1, 64);
      if (lane < C) {
        s_gam[lane] = gam;
        s_beta[lane] = bv;
        const float b = __expf(gam);
        sc_out[lane] = b * s_rk[lane];
        sc_out[C + lane] = scale * b * s_rq[lane];
        sc_out[2 * C + lane] = __expf(glast - gam) * s_rk[lane];
        sc_out[3 * C + lane] = __expf(glast);
      }
    }
    __syncthreads();

    // 4. L (strictly lower) into LDS; P (lower incl. diagonal) to the workspace.
    //    The decay is only formed for j <= i (masked before the exponential).
    {
      float* p_out = ws.p + unit * (C * C);
      for (int e = tid; e < C * C; e += 256) {
        const int i = e / C, j = e % C;
        float lv = 0.f, pv = 0.f;
        if (j <= i) {
          const float dec = __expf(s_gam[i] - s_gam[j]);
          pv = scale * dec * s_rq[i] * s_rk[j] * sGQ[i * LDC + j];
          if (j < i) lv = s_beta[i] * dec * s_rk[i] * s_rk[j] * sGK[i * LDC + j];
        }
        sL[i * LDC + j] = lv;
        p_out[e] = pv;
      }
    }
    __syncthreads();

    // 5. T = (I + L)^-1.  Diagonal 16x16 blocks: lane 16b + c owns column c of
    //    block b and runs forward substitution T_i = e_i - sum_{j<i} L_ij T_j.
    if (wave == 0 && lane < 16 * NT) {
      const int b = lane >> 4, c = lane & 15, base = 16 * b;
      float tcol[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < i; ++j) acc -= sL[(base + i) * LDC + base + j] * tcol[j];
        tcol[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sT[(base + i) * LDC + base + c] = tcol[i];
    }
    __syncthreads();
    //    Off-diagonal blocks by block diagonals d = bi - bj:
    //    T_{bi,bj} = -T_{bi,bi} * sum_{kb=bj}^{bi-1} L_{bi,kb} T_{kb,bj}   (fp32 MFMA)
    for (int d = 1; d < NT; ++d) {
      for (int bi = d + wave; bi < NT; bi += 4) {
        const int bj = bi - d;
        floatx4 w = {0.f, 0.f, 0.f, 0.f};
        for (int kb = bj; kb < bi; ++kb) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int kk = 4 * ks + g4;
            w = mfma_f32(sL[(16 * bi + r16) * LDC + 16 * kb + kk], sT[(16 * kb + kk) * LDC + 16 * bj + r16], w);
          }
        }
        // w holds W[4g+i][r16]; use it as the B operand with k = 4g + step
        floatx4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) t = mfma_f32(sT[(16 * bi + r16) * LDC + 16 * bi + 4 * g4 + s], w[s], t);
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[(16 * bi + 4 * g4 + i) * LDC + 16 * bj + r16] = -t[i];
      }
      __syncthreads();
    }

    // 6. Tb = T diag(beta) (zero above the diagonal) to the workspace
    {
      float* tb_out = ws.tb + unit * (C * C);
      for (int e = tid; e < C * C; e += 256) {
        const int i = e / C, j = e % C;
        tb_out[e] = (j <= i) ? sT[i * LDC + j] * s_beta[j] : 0.f;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// k_chunk_scan
// ---------------------------------------------------------------------------
template <class Pol, class EO, int D, int C>
__global__ __launch_bounds__(256) void k_chunk_scan(
    const typename Pol::In::T* __restrict__ q, const typename Pol::In::T* __restrict__ k,
    const typename Pol::In::T* __restrict__ v, int64_t q_stride, int64_t k_stride, int64_t v_stride,
    int h_qk, int h_v, const int32_t* __restrict__ cu, int n_seq, int64_t t_total,
    const float* __restrict__ init, float* __restrict__ fin,
    typename EO::T* __restrict__ o, ChunkWs ws, int64_t n_blocks) {
  using Elem = typename Pol::Elem;
  using In = typename Pol::In;
  constexpr int BV = 16;
  constexpr int NTILE = D / BV;
  constexpr int LDK = D + Pol::PAD;    // rows of d_k elements
  constexpr int LDT = C + Pol::PAD;    // rows of C token elements
  constexpr int NMT = C / 16;          // token m-tiles (one per wave)
  constexpr int NST = D / 16;          // d_k tiles of the state
  constexpr int SPW = (NST + 3) / 4;   // state tiles per wave
  static_assert(NMT <= 4, "one token tile per wave");
  static_assert(C % Pol::KSTEP == 0 && D % Pol::KSTEP == 0, "k-steps must tile C and D");

  __shared__ __attribute__((aligned(16))) Elem sK[C * LDK];
  __shared__ __attribute__((aligned(16))) Elem sQ[C * LDK];
  __shared__ __attribute__((aligned(16))) Elem sKt[D * LDT];
  __shared__ __attribute__((aligned(16))) Elem sTb[Pol::NSPLIT][C * LDT];
  __shared__ __attribute__((aligned(16))) Elem sP[Pol::NSPLIT][C * LDT];
  __shared__ __attribute__((aligned(16))) Elem sX[Pol::NSPLIT][BV * LDT];
  __shared__ __attribute__((aligned(16))) Elem sU[Pol::NSPLIT][BV * LDT];
  __shared__ __attribute__((aligned(16))) Elem sU2[Pol::NSPLIT][BV * LDT];
  __shared__ __attribute__((aligned(16))) Elem sS[Pol::NSPLIT][BV * LDK];
  __shared__ float s_c1[C], s_c2[C], s_c3[C], s_bc;

  // XCD-aware order: the dispatcher places block b on XCD b % 8, so give each
  // XCD a contiguous range of logical ids; the d_v tiles of one head then
  // share an L2 and its K/Q/Tb/P reads.
  const int64_t b = blockIdx.x;
  const int64_t lid = (n_blocks % 8 == 0) ? (b % 8) * (n_blocks / 8) + b / 8 : b;
  const int tile = static_cast<int>(lid % NTILE);
  const int64_t sh = lid / NTILE;
  const int h = static_cast<int>(sh % h_v);
  const int s = static_cast<int>(sh / h_v);
  if (s >= n_seq) return;
  const int hq = h / (h_v / h_qk);
  const int dv0 = tile * BV;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;

  // fp32 master state: tiles mt = wave + 4 j of S^T (rows d_k, columns d_v):
  // lane holds S[dv0 + r16][16 mt + 4 g4 + i].
  floatx4 Sacc[SPW];
  const int64_t srow = ((int64_t)s * h_v + h) * D + dv0 + r16;   // state row of this lane
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int mt = wave + 4 * j;
    Sacc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (mt < NST) {
      if (init) {
        const float4 v4 = *reinterpret_cast<const float4*>(init + srow * D + 16 * mt + 4 * g4);
        Sacc[j] = floatx4{v4.x, v4.y, v4.z, v4.w};
      }
      const float tmp[4] = {Sacc[j][0], Sacc[j][1], Sacc[j][2], Sacc[j][3]};
      Pol::put4(sS[0], sS[Pol::NSPLIT - 1], r16 * LDK + 16 * mt + 4 * g4, tmp);
    }
  }

  const int64_t start = seq_start(cu, s, t_total), end = seq_start(cu, s + 1, t_total);
  const int64_t nchunks = (end - start + C - 1) / C;
  const int64_t slot0 = start / C + s;

  for (int64_t j = 0; j < nchunks; ++j) {
    const int64_t t0 = start + j * C;
    const int len = static_cast<int>(end - t0 < C ? end - t0 : C);
    const int64_t unit = (slot0 + j) * h_v + h;

    // ---- stage the chunk's operands ----
    {
      constexpr int TPR = D / 8, RPP = 256 / TPR;
      for (int r0 = 0; r0 < C; r0 += RPP) {
        const int row = r0 + tid / TPR, c8 = (tid % TPR) * 8;
        if (row < C) {
          const bool valid = row < len;
          const int64_t tok = t0 + (valid ? row : 0);
          float kv[8], qv[8];
          Pol::stage8(sK + row * LDK + c8, k + tok * k_stride + (int64_t)hq * D + c8, valid, kv);
          Pol::stage8(sQ + row * LDK + c8, q + tok * q_stride + (int64_t)hq * D + c8, valid, qv);
#pragma unroll
          for (int i = 0; i < 8; ++i) Pol::put_raw(sKt, (c8 + i) * LDT + row, kv[i]);
        }
      }
      const float* tb = ws.tb + unit * (C * C);
      const float* pp = ws.p + unit * (C * C);
      for (int e = tid * 4; e < C * C; e += 256 * 4) {
        const int i = e / C, jj = e % C;
        const float4 a = *reinterpret_cast<const float4*>(tb + e);
        const float4 bq = *reinterpret_cast<const float4*>(pp + e);
        const float av[4] = {a.x, a.y, a.z, a.w}, pv[4] = {bq.x, bq.y, bq.z, bq.w};
        Pol::put4(sTb[0], sTb[Pol::NSPLIT - 1], i * LDT + jj, av);
        Pol::put4(sP[0], sP[Pol::NSPLIT - 1], i * LDT + jj, pv);
      }
      const float* sc = ws.sc + unit * (4 * C);
      if (tid < C) {
        s_c1[tid] = sc[tid];
        s_c2[tid] = sc[C + tid];
        s_c3[tid] = sc[2 * C + tid];
      }
      if (tid == 0) s_bc = sc[3 * C];
    }
    __syncthreads();

    // ---- K S^T and Q S^T for token tile `wave`; X = V - diag(b rk) K S^T ----
    floatx4 Oacc = {0.f, 0.f, 0.f, 0.f};
    if (wave < NMT) {
      floatx4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
      Pol::template mma<false, true>(ak, sK + 16 * wave * LDK, nullptr, LDK, sS[0], sS[Pol::NSPLIT - 1], LDK, D / Pol::KSTEP);
      Pol::template mma<false, true>(aq, sQ + 16 * wave * LDK, nullptr, LDK, sS[0], sS[Pol::NSPLIT - 1], LDK, D / Pol::KSTEP);
      float xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * g4 + i;
        const float vv = row < len ? In::load(v, (t0 + row) * v_stride + (int64_t)h * D + dv0 + r16) : 0.f;
        xv[i] = vv - s_c1[row] * ak[i];
        Oacc[i] = s_c2[row] * aq[i];
      }
      Pol::put4(sX[0], sX[Pol::NSPLIT - 1], r16 * LDT + 16 * wave + 4 * g4, xv);
    }
    __syncthreads();

    // ---- U = Tb X (lower triangular: k up to the tile's last row) ----
    const int nks_w = (16 * wave + 16 + Pol::KSTEP - 1) / Pol::KSTEP;
    if (wave < NMT) {
      floatx4 au = {0.f, 0.f, 0.f, 0.f};
      Pol::template mma<true, true>(au, sTb[0] + 16 * wave * LDT, sTb[Pol::NSPLIT - 1] + 16 * wave * LDT, LDT,
                                    sX[0], sX[Pol::NSPLIT - 1], LDT, nks_w);
      float u2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) u2[i] = s_c3[16 * wave + 4 * g4 + i] * au[i];
      const float uv[4] = {au[0], au[1], au[2], au[3]};
      Pol::put4(sU[0], sU[Pol::NSPLIT - 1], r16 * LDT + 16 * wave + 4 * g4, uv);
      Pol::put4(sU2[0], sU2[Pol::NSPLIT - 1], r16 * LDT + 16 * wave + 4 * g4, u2);
    }
    __syncthreads();

    // ---- O += P U; store rows of the chunk ----
    if (wave < NMT) {
      Pol::template mma<true, true>(Oacc, sP[0] + 16 * wave * LDT, sP[Pol::NSPLIT - 1] + 16 * wave * LDT, LDT,
                                    sU[0], sU[Pol::NSPLIT - 1], LDT, nks_w);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * g4 + i;
        if (row < len) EO::store(o, (t0 + row) * ((int64_t)h_v * D) + (int64_t)h * D + dv0 + r16, Oacc[i]);
      }
    }
    // ---- S^T <- b_C S^T + K^T U2 ----
    const float bc = s_bc;
#pragma unroll
    for (int jj = 0; jj < SPW; ++jj) {
      const int mt = wave + 4 * jj;
      if (mt < NST) {
        floatx4 acc = Sacc[jj] * bc;
        Pol::template mma<false, true>(acc, sKt + 16 * mt * LDT, nullptr, LDT, sU2[0], sU2[Pol::NSPLIT - 1], LDT,
                                       C / Pol::KSTEP);
        Sacc[jj] = acc;
        const float tmp[4] = {acc[0], acc[1], acc[2], acc[3]};
        Pol::put4(sS[0], sS[Pol::NSPLIT - 1], r16 * LDK + 16 * mt + 4 * g4, tmp);
      }
    }
    __syncthreads();
  }

  if (fin) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int mt = wave + 4 * j;
      if (mt < NST)
        *reinterpret_cast<float4*>(fin + srow * D + 16 * mt + 4 * g4) =
            make_float4(Sacc[j][0], Sacc[j][1], Sacc[j][2], Sacc[j][3]);
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
size_t chunk_ws_bytes(int h_v, int d, int chunk, int n_seq, int64_t t_total, int with_norm) {
  const int64_t slots = block_slots(t_total, n_seq, chunk);
  auto al = [](size_t b) { return (b + 255) & ~size_t(255); };
  size_t bytes = 0;
  bytes += al(sizeof(float) * slots * h_v * chunk * chunk);   // tb
  bytes += al(sizeof(float) * slots * h_v * chunk * chunk);   // p
  bytes += al(sizeof(float) * slots * h_v * 4 * chunk);       // scalars
  if (with_norm) bytes += al(sizeof(float) * t_total * h_v * d);
  return bytes;
}

template <class Pol, int D, int C>
static hipError_t run_chunk(const ChunkArgs& a) {
  using T = typename Pol::In::T;
  const int64_t slots = block_slots(a.t_total, a.n_seq, C);
  auto al = [](size_t b) { return (b + 255) & ~size_t(255); };
  char* base = static_cast<char*>(a.workspace);
  ChunkWs ws;
  ws.tb = reinterpret_cast<float*>(base);
  base += al(sizeof(float) * slots * a.h_v * C * C);
  ws.p = reinterpret_cast<float*>(base);
  base += al(sizeof(float) * slots * a.h_v * C * C);
  ws.sc = reinterpret_cast<float*>(base);
  base += al(sizeof(float) * slots * a.h_v * 4 * C);
  float* o_pre = reinterpret_cast<float*>(base);   // pre-norm outputs when z is given

  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  if (slots > 0) {
    dim3 grid(static_cast<unsigned>(slots), a.h_qk);
    hipLaunchKernelGGL((k_chunk_prep<Pol, D, C>), grid, dim3(256), 0, st, q, k, a.q_stride, a.k_stride,
                       a.g, a.beta, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.cu, a.n_seq, a.t_total, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nblk = (int64_t)a.n_seq * a.h_v * (D / 16);
  if (a.z) {
    hipLaunchKernelGGL((k_chunk_scan<Pol, F32, D, C>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st,
                       q, k, v, a.q_stride, a.k_stride, a.v_stride, a.h_qk, a.h_v, a.cu, a.n_seq, a.t_total,
                       a.init, a.fin, o_pre, ws, nblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.t_total > 0)
      return launch_gated_rmsnorm(o_pre, GDN_F32, a.z, a.dt, a.norm_w, a.norm_eps, a.t_total * a.h_v, D,
                                  a.o, a.o_dt, a.stream);
    return hipSuccess;
  }
  if (a.o_dt == GDN_BF16)
    hipLaunchKernelGGL((k_chunk_scan<Pol, BF16, D, C>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st,
                       q, k, v, a.q_stride, a.k_stride, a.v_stride, a.h_qk, a.h_v, a.cu, a.n_seq, a.t_total,
                       a.init, a.fin, static_cast<uint16_t*>(a.o), ws, nblk);
  else
    hipLaunchKernelGGL((k_chunk_scan<Pol, F32, D, C>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st,
                       q, k, v, a.q_stride, a.k_stride, a.v_stride, a.h_qk, a.h_v, a.cu, a.n_seq, a.t_total,
                       a.init, a.fin, static_cast<float*>(a.o), ws, nblk);
  return hipGetLastError();
}

hipError_t launch_chunk_fwd(const ChunkArgs& a) {
  if (a.dt == GDN_BF16) {
    if (a.d == 128 && a.chunk == 64) return run_chunk<PolBF16, 128, 64>(a);
  } else {
    if (a.d == 128 && a.chunk == 64) return run_chunk<PolF32, 128, 64>(a);
    if (a.d == 16 && a.chunk == 16) return run_chunk<PolF32, 16, 16>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
