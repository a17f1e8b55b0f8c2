// Kernel templates of the chunk path (gfx950): matrix-core operand policies,
// the chunk workspace layout, the prep kernel and the scan kernel.  Included by
// chunk.hip (the forward launcher) and chunk_bwd.hip (the chunked backward);
// the chunk algebra they implement is stated at the top of chunk.hip.
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

__device__ __forceinline__ floatx4 mfma_bf16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Matrix-core operand conventions.  One 16 x 16 x KSTEP product takes per
// lane (r = lane % 16, g = lane / 16) an A fragment: row r, k elements
// g*FE .. g*FE+FE-1 of the k-step, and a B fragment: column r, the same k
// elements; it accumulates acc[i] += A[4g+i][.] B[.][r] (output row 4g+i,
// column r).  Operands in LDS are stored k-contiguous: A as [m][k], B as [n][k].
struct PolBF16 {
  using In = BF16;
  using Elem = __bf16;
  using Frag = bf16x8;
  static constexpr int KSTEP = 32;
  static constexpr int FE = 8;        // elements per lane per fragment
  static constexpr int PAD = 8;
  static constexpr int NSPLIT = 2;    // hi and lo arrays
  // The scan keeps the chunk's K in LDS and builds the K^T operands of the
  // state update with transposing LDS reads (16-bit elements), so the
  // workspace holds no K^T copy.
  static constexpr bool kKtInLds = true;
  // The scan's LDS rows (S, X, U) are unpadded, with XOR-swizzled 16-byte units.
  static constexpr bool kSwizzle = true;

  __device__ __forceinline__ static floatx4 mma(Frag a, Frag b, floatx4 c) { return mfma_bf16(a, b, c); }
  __device__ __forceinline__ static Frag ld(const Elem* p) { return *reinterpret_cast<const Frag*>(p); }
  __device__ __forceinline__ static Frag ld_in(const uint16_t* p) { return *reinterpret_cast<const Frag*>(p); }

  // acc += A B over NKS k-steps, both operands in LDS (raw, no lo parts)
  template <int NKS>
  __device__ __forceinline__ static void mma_lds(floatx4& acc, const Elem* a, int lda, const Elem* b, int ldb) {
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    Frag fa[NKS], fb[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      fa[ks] = ld(a + r * lda + ks * KSTEP + g * FE);
      fb[ks] = ld(b + r * ldb + ks * KSTEP + g * FE);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) acc = mma(fa[ks], fb[ks], acc);
  }
  // Split store of 4 consecutive values into LDS hi and lo arrays.
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
  // One fragment (FE values) split into hi and lo, stored to memory.
  __device__ __forceinline__ static void store_split(Elem* hi, Elem* lo, const float* v) {
    Frag h, l;
#pragma unroll
    for (int i = 0; i < FE; ++i) {
      __bf16 a, b;
      split_bf16(v[i], a, b);
      h[i] = a;
      l[i] = b;
    }
    *reinterpret_cast<Frag*>(hi) = h;
    *reinterpret_cast<Frag*>(lo) = l;
  }
  // FE raw elements gathered from LDS with a stride, stored as one fragment.
  __device__ __forceinline__ static void gather(Elem* dst, const Elem* src, int stride) {
    Frag h;
#pragma unroll
    for (int i = 0; i < FE; ++i) h[i] = src[i * stride];
    *reinterpret_cast<Frag*>(dst) = h;
  }
  // 8 consecutive raw input elements: load (Raw8), then copy the bits to LDS
  // and return the values (commit8), zeroed when the row is not valid.
  struct Raw8 {
    uint4 a;
  };
  __device__ __forceinline__ static Raw8 load8(const uint16_t* src) {
    return Raw8{*reinterpret_cast<const uint4*>(src)};
  }
  __device__ __forceinline__ static void commit8(Elem* dst, Raw8 raw, bool valid, float* f) {
    uint4 r = raw.a;
    if (!valid) r = make_uint4(0, 0, 0, 0);
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
  using Frag = float;
  static constexpr int KSTEP = 4;
  static constexpr int FE = 1;
  static constexpr int PAD = 4;
  static constexpr int NSPLIT = 1;    // fp32 operands need no lo part
  static constexpr bool kKtInLds = false;   // K^T fragments come from the workspace
  static constexpr bool kSwizzle = false;   // padded LDS rows

  __device__ __forceinline__ static floatx4 mma(Frag a, Frag b, floatx4 c) { return mfma_f32(a, b, c); }
  __device__ __forceinline__ static Frag ld(const Elem* p) { return *p; }
  __device__ __forceinline__ static Frag ld_in(const float* p) { return *p; }
  template <int NKS>
  __device__ __forceinline__ static void mma_lds(floatx4& acc, const Elem* a, int lda, const Elem* b, int ldb) {
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) acc = mma(a[r * lda + ks * KSTEP + g], b[r * ldb + ks * KSTEP + g], acc);
  }
  __device__ __forceinline__ static void put4(Elem* hi, Elem*, int idx, const float* v) {
    *reinterpret_cast<float4*>(hi + idx) = make_float4(v[0], v[1], v[2], v[3]);
  }
  __device__ __forceinline__ static void store_split(Elem* hi, Elem*, const float* v) { *hi = v[0]; }
  __device__ __forceinline__ static void gather(Elem* dst, const Elem* src, int) { *dst = *src; }
  struct Raw8 {
    float4 a, b;
  };
  __device__ __forceinline__ static Raw8 load8(const float* src) {
    return Raw8{reinterpret_cast<const float4*>(src)[0], reinterpret_cast<const float4*>(src)[1]};
  }
  __device__ __forceinline__ static void commit8(Elem* dst, Raw8 raw, bool valid, float* f) {
    float4 a = raw.a, b = raw.b;
    if (!valid) {
      a = make_float4(0, 0, 0, 0);
      b = make_float4(0, 0, 0, 0);
    }
    reinterpret_cast<float4*>(dst)[0] = a;
    reinterpret_cast<float4*>(dst)[1] = b;
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

__device__ __forceinline__ uint32_t to_u32(uint16_t x) { return x; }
__device__ __forceinline__ uint32_t to_u32(float x) { return __float_as_uint(x); }
template <class In>
__device__ __forceinline__ float from_u32(uint32_t x);
template <>
__device__ __forceinline__ float from_u32<BF16>(uint32_t x) { return __uint_as_float(x << 16); }
template <>
__device__ __forceinline__ float from_u32<F32>(uint32_t x) { return __uint_as_float(x); }

// Workspace, all indexed by chunk slot (see locate_block):
//   kq [slots][h_qk][2][C*D]       K, Q fragments (raw): blocks (token tile mt, d_k k-step ks)
//   kt [slots][h_qk][D*C]          K^T fragments: blocks (dk tile mt, k-step ks); fp32 only
//   tb [slots][h_v][NSPLIT*C*C]    Tb fragments:  blocks (token tile mt, k-step ks, hi|lo)
//   p  [slots][h_v][NSPLIT*C*C]    P fragments:   same order
//   sc [slots][h_v][4][C] fp32     b rk | scale b rq | exp(gamma_C - gamma) rk | b_C
//   order [n_seq] int32            sequences, most chunks first (only when n_seq > 1)
// A fragment block is 64 lanes x FE elements, lane l holding row l % 16 and
// k elements (l / 16) * FE .. + FE - 1 of its k-step, so one wave reads a
// block with one contiguous 16-byte load per lane (bf16).
struct ChunkWs {
  void* kq;
  void* kt;
  void* tb;
  void* p;
  float* sc;
  int32_t* order;   // NULL for a single sequence
  void* tbt;        // Tb^T fragments (backward prep), else NULL
  float* states;    // [slots][h_v][D][D] state entering each chunk (backward's forward scan), else NULL
};

template <class Pol, int D, int C>
struct WsLayout {
  using Elem = typename Pol::Elem;
  static constexpr int NKS_C = C / Pol::KSTEP;
  static constexpr int BLK = 64 * Pol::FE;                            // elements per fragment block
  static constexpr int NKS_D = D / Pol::KSTEP;
  static constexpr int64_t kt_elems = (int64_t)D * C;                 // per (slot, qk head)
  static constexpr int64_t kq_elems = 2 * (int64_t)C * D;             // per (slot, qk head): K then Q
  static constexpr int64_t op_elems = (int64_t)Pol::NSPLIT * C * C;   // per (slot, v head)
  // offset of block (mt, ks, split) of a Tb/P region, and of block (mt, ks) of a K^T region
  __host__ __device__ static constexpr int op_block(int mt, int ks, int split) {
    return ((mt * NKS_C + ks) * Pol::NSPLIT + split) * BLK;
  }
  __host__ __device__ static constexpr int kt_block(int mt, int ks) { return (mt * NKS_C + ks) * BLK; }
  // block (token tile mt, d_k k-step ks) of the K (which 0) or Q (which 1) half of a kq region
  __host__ __device__ static constexpr int kq_block(int which, int mt, int ks) {
    return which * C * D + (mt * NKS_D + ks) * BLK;
  }
  static size_t al(size_t x) { return (x + 255) & ~size_t(255); }
  static size_t order_bytes(int n_seq) { return n_seq > 1 ? al(sizeof(int32_t) * n_seq) : 0; }
  static size_t kt_bytes(int64_t slots, int h_qk) {
    return Pol::kKtInLds ? 0 : al(sizeof(Elem) * slots * h_qk * kt_elems);
  }
  static size_t bytes(int64_t slots, int h_qk, int h_v, int n_seq) {
    return al(sizeof(Elem) * slots * h_qk * kq_elems) + kt_bytes(slots, h_qk) +
           2 * al(sizeof(Elem) * slots * h_v * op_elems) + al(sizeof(float) * slots * h_v * 4 * C) +
           order_bytes(n_seq);
  }
  static ChunkWs carve(void* base, int64_t slots, int h_qk, int h_v, int n_seq) {
    char* b = static_cast<char*>(base);
    ChunkWs w;
    w.kq = b;
    b += al(sizeof(Elem) * slots * h_qk * kq_elems);
    w.kt = b;
    b += kt_bytes(slots, h_qk);
    w.tb = b;
    b += al(sizeof(Elem) * slots * h_v * op_elems);
    w.p = b;
    b += al(sizeof(Elem) * slots * h_v * op_elems);
    w.sc = reinterpret_cast<float*>(b);
    b += al(sizeof(float) * slots * h_v * 4 * C);
    w.order = n_seq > 1 ? reinterpret_cast<int32_t*>(b) : nullptr;
    w.tbt = nullptr;
    w.states = nullptr;
    return w;
  }
};

// Sum of squares of 8 values, in a fixed order of fused multiply-adds.
__device__ __forceinline__ float sumsq8(const float* v) {
  float s = v[0] * v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) s = __builtin_fmaf(v[i], v[i], s);
  return s;
}

// N consecutive values from LDS, as 16-byte reads when they fill them
template <int N, class T>
__device__ __forceinline__ void lds_row(const T* p, T* out) {
  constexpr int V = 16 / (int)sizeof(T);
  if constexpr (N % V == 0) {
    typedef T vec __attribute__((ext_vector_type(V)));
#pragma unroll
    for (int k = 0; k < N / V; ++k) {
      const vec v = reinterpret_cast<const vec*>(p)[k];
#pragma unroll
      for (int e = 0; e < V; ++e) out[V * k + e] = v[e];
    }
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) out[k] = p[k];
  }
}

// T = (I + L)^-1 for the strictly lower C x C matrix L in LDS (rows of LDC
// floats; only its strictly lower part is read), into the lower part of T
// (the part above the diagonal is not written).  Every thread of the 256
// calls it; it ends with a barrier.  Diagonal 16x16 blocks: lane 16b + c of
// wave 0 owns column c of block b and runs forward substitution
// T_i = e_i - sum_{j<i} L_ij T_j.  Off-diagonal blocks by block diagonals
// d = bi - bj:  T_{bi,bj} = -T_{bi,bi} * sum_{kb=bj}^{bi-1} L_{bi,kb} T_{kb,bj}
// (fp32 MFMA).
template <int C, int LDC>
__device__ __forceinline__ void unit_lower_inverse(const float* sL, float* sT) {
  constexpr int NT = C / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  if (wave == 0 && lane < 16 * NT) {
    int c = lane & 15;
    // opaque per call: the kernels call this inside their unit loops, and the
    // 16 selects (i == c) below would otherwise be hoisted into 16 registers
    // held across every unit
    asm volatile("" : "+v"(c));
    const int b = lane >> 4, base = 16 * b;
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
}

// ---------------------------------------------------------------------------
// k_chunk_prep: persistent workgroups over (chunk slot, q/k head) units
// ---------------------------------------------------------------------------
//
// With kBwd (the backward's prep) one-token sequences are prepared too, the
// P region holds P^T and ws.tbt receives Tb^T, both in the same fragment
// blocks: block (mt, ks), lane l holds M^T[16 mt + l%16][ks*KSTEP + (l/16)*FE
// + e] = M[ks*KSTEP + (l/16)*FE + e][16 mt + l%16] (zero above M's diagonal).
template <class Pol, int D, int C, bool kBwd = false>
__global__ __launch_bounds__(256, 2) void k_chunk_prep(
    const typename Pol::In::T* __restrict__ q, const typename Pol::In::T* __restrict__ k,
    int64_t q_stride, int64_t k_stride, GateSrc gates, float scale, int use_l2, float l2_eps, int h_qk, int h_v,
    const int32_t* __restrict__ cu, int n_seq, int64_t t_total, const int32_t* __restrict__ seq_slots, ChunkWs ws,
    int64_t n_slots) {
  using Elem = typename Pol::Elem;
  using W = WsLayout<Pol, D, C>;
  constexpr int LDK = D + Pol::PAD;
  constexpr int LDC = C + 4;
  constexpr int NT = C / 16;
  constexpr int FE = Pol::FE;
  constexpr int NKS_C = C / Pol::KSTEP;
  using Frag = typename Pol::Frag;
  constexpr int KQ_BYTES = 2 * C * LDK * (int)sizeof(Elem);
  constexpr int LT_BYTES = 2 * C * LDC * 4;
  static_assert(C % 16 == 0 && D % 16 == 0 && C <= 64, "tile shape");
  static_assert(D % Pol::KSTEP == 0 && C % Pol::KSTEP == 0, "k-steps must tile D and C");

  // K/Q rows during the Gram phase, then L and T (overlaid).
  __shared__ __attribute__((aligned(16))) char smem[KQ_BYTES > LT_BYTES ? KQ_BYTES : LT_BYTES];
  __shared__ __attribute__((aligned(16))) float sGK[C * LDC];
  __shared__ __attribute__((aligned(16))) float sGQ[C * LDC];
  __shared__ __attribute__((aligned(16))) float s_rk[C];
  __shared__ __attribute__((aligned(16))) float s_rq[C];
  // the chunk's running sum of g, kept in fp64: with strong decays it reaches
  // hundreds, and the decay between two tokens is a difference of two sums
  __shared__ __attribute__((aligned(16))) double s_gam[C];
  __shared__ __attribute__((aligned(16))) float s_beta[C];
  Elem* sK = reinterpret_cast<Elem*>(smem);
  Elem* sQ = sK + C * LDK;
  float* sL = reinterpret_cast<float*>(smem);
  float* sT = sL + C * LDC;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int grp = h_v / h_qk;
  constexpr int TPR = D / 8, RPP = 256 / TPR, NR = (C + RPP - 1) / RPP;

  // Persistent loop over units u = (chunk slot u / h_qk, q/k head u % h_qk),
  // slot-major so that slots left empty by the slot numbering come last.  A
  // unit loads K and Q and forms their Gram matrices once, then runs the
  // decay, the solve and the outputs for each v-head that reads this q/k head.
  // The raw K, Q rows and the g, beta values of the next unit are loaded
  // while the current one is computed.
  const int64_t n_units = n_slots * h_qk;
  const int64_t stride = gridDim.x;
  typename Pol::Raw8 kr[NR], qr[NR];   // raw rows of the unit to be committed next
  float gn = 0.f, bn = 0.f;            // g, beta of its first v-head (wave 0, one token per lane)
  int n_seq_i = 0, n_len = 0;
  int64_t n_t0 = 0;
  bool n_ok = false;
  int64_t u = blockIdx.x;
#define GDN_PREP_FETCH(uu)                                                                              \
  do {                                                                                                 \
    n_ok = (uu) < n_units && locate_block(cu, n_seq, t_total, C, (uu) / h_qk, n_seq_i, n_t0, n_len);     \
    if (n_ok && seq_slots) n_ok = seq_slots[n_seq_i] >= 0;   /* inactive lane: no scan reads it */        \
    if (!kBwd && n_ok && n_len == 1)   /* a one-token sequence: the scan runs the plain recurrence */    \
      n_ok = seq_start(cu, n_seq_i + 1, t_total) - seq_start(cu, n_seq_i, t_total) > 1;                  \
    if (n_ok) {                                                                                        \
      const int fq_ = static_cast<int>((uu) % h_qk);                                                   \
      _Pragma("unroll") for (int it = 0; it < NR; ++it) {                                              \
        const int row = it * RPP + tid / TPR, c8 = (tid % TPR) * 8;                                    \
        if (RPP <= C || row < C) {                                                                     \
          const int64_t tok = n_t0 + (row < n_len ? row : 0);                                          \
          kr[it] = Pol::load8(k + tok * k_stride + (int64_t)fq_ * D + c8);                             \
          qr[it] = Pol::load8(q + tok * q_stride + (int64_t)fq_ * D + c8);                             \
        }                                                                                              \
      }                                                                                                \
      if (wave == 0)                                                                                   \
        load_gate(gates, n_t0 + (lane < n_len ? lane : n_len - 1), fq_ * grp, h_v, gn, bn);            \
    }                                                                                                  \
  } while (0)
  GDN_PREP_FETCH(u);
  for (; u < n_units; u += stride) {
    const bool ok = n_ok;
    const int len = n_len;
    const int64_t t0 = n_t0;
    float gv = gn, bv = bn;
    const int64_t cslot = u / h_qk;
    const int hq = static_cast<int>(u % h_qk);
    if (ok) {
      // 1. commit the raw K, Q rows to LDS (zero beyond len) and form their
      //    L2 scales
#pragma unroll
      for (int it = 0; it < NR; ++it) {
        const int row = it * RPP + tid / TPR, c8 = (tid % TPR) * 8;
        float kv[8] = {0, 0, 0, 0, 0, 0, 0, 0}, qv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (RPP <= C || row < C) {
          Pol::commit8(sK + row * LDK + c8, kr[it], row < len, kv);
          Pol::commit8(sQ + row * LDK + c8, qr[it], row < len, qv);
        }
        float sk = sumsq8(kv), sq = sumsq8(qv);
        sk = group_sum<TPR>(sk);
        sq = group_sum<TPR>(sq);
        if ((RPP <= C || row < C) && tid % TPR == 0) {
          const bool valid = row < len;
          s_rk[row] = !valid ? 0.f : (use_l2 ? 1.0f / sqrtf(sk + l2_eps) : 1.0f);
          s_rq[row] = !valid ? 0.f : (use_l2 ? 1.0f / sqrtf(sq + l2_eps) : 1.0f);
        }
      }
    }
    // the next unit's loads go out now and land during this unit's work
    GDN_PREP_FETCH(u + stride);
    if (!ok) continue;
    __syncthreads();

    // 2. lower-triangular tiles of K K^T and Q K^T (raw operands, exact
    //    products), tasks spread statically over the 4 waves
    {
      constexpr int NLT = NT * (NT + 1) / 2, NTASK = 2 * NLT, TPW = (NTASK + 3) / 4;
#pragma unroll
      for (int it = 0; it < TPW; ++it) {
        const int task = wave + 4 * it;
        if (task < NTASK) {
          const bool isq = task >= NLT;
          const int idx = isq ? task - NLT : task;
          int ti = 0;
#pragma unroll
          for (int r = 1; r < NT; ++r) ti += (r * (r + 1) / 2 <= idx) ? 1 : 0;
          const int tj = idx - ti * (ti + 1) / 2;
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          Pol::template mma_lds<D / Pol::KSTEP>(acc, (isq ? sQ : sK) + ti * 16 * LDK, LDK, sK + tj * 16 * LDK, LDK);
          float* dst = isq ? sGQ : sGK;
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[(16 * ti + 4 * g4 + i) * LDC + 16 * tj + r16] = acc[i];
        }
      }
    }
    // 3. K and Q of the chunk as the scan's A fragments (block (token tile mt,
    //    d_k k-step ks), lane l: row 16 mt + l%16, d_k ks*KSTEP + (l/16)*FE + e;
    //    rows past the chunk's end are zero), so the scan reads contiguous
    //    blocks instead of rows spread over the input, and K^T as fragments:
    //    block (mt, ks), lane l: K[token ks*KSTEP + (l/16)*FE + e][dk 16 mt + l%16]
    {
      Elem* kqb = static_cast<Elem*>(ws.kq) + (cslot * h_qk + hq) * W::kq_elems;
      constexpr int NKS_D = D / Pol::KSTEP;
      for (int f = tid; f < 2 * NT * NKS_D * 64; f += 256) {
        const int l = f & 63, blk = f >> 6;
        const int which = blk / (NT * NKS_D), mt = (blk / NKS_D) % NT, ks = blk % NKS_D;
        const Elem* src = (which ? sQ : sK) + (16 * mt + (l & 15)) * LDK + ks * Pol::KSTEP + (l >> 4) * FE;
        *reinterpret_cast<Frag*>(kqb + W::kq_block(which, mt, ks) + l * FE) = Pol::ld(src);
      }
    }
    if constexpr (!Pol::kKtInLds) {
      Elem* kt = static_cast<Elem*>(ws.kt) + (cslot * h_qk + hq) * W::kt_elems;
      for (int f = tid; f < (D / 16) * NKS_C * 64; f += 256) {
        const int l = f & 63, blk = f >> 6;
        const int mt = blk / NKS_C, ks = blk % NKS_C;
        const int dk = 16 * mt + (l & 15), tok0 = ks * Pol::KSTEP + (l >> 4) * FE;
        Pol::gather(kt + W::kt_block(mt, ks) + l * FE, sK + tok0 * LDK + dk, LDK);
      }
    }

    for (int vh = 0; vh < grp; ++vh) {
      const int h = hq * grp + vh;
      const int64_t unit = cslot * h_v + h;
      // g, beta of the following v-head of the group, loaded now for later
      float g_next = 0.f, b_next = 0.f;
      if (wave == 0 && vh + 1 < grp) load_gate(gates, t0 + (lane < len ? lane : len - 1), h + 1, h_v, g_next, b_next);
      if (lane >= len) gv = bv = 0.f;

      // 4. decay: inclusive prefix sum of g over the chunk (padded tokens add 0)
      if (wave == 0) {
        double gam = gv;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const double o = __shfl_up(gam, off, 64);
          if (lane >= off) gam += o;
        }
        const double glast = __shfl(gam, C - 1, 64);
        if (lane < C) {
          float* sc_out = ws.sc + unit * (4 * C);
          s_gam[lane] = gam;
          s_beta[lane] = bv;
          const float b = __expf(static_cast<float>(gam));
          sc_out[lane] = b * s_rk[lane];
          sc_out[C + lane] = scale * b * s_rq[lane];
          sc_out[2 * C + lane] = __expf(static_cast<float>(glast - gam)) * s_rk[lane];
          sc_out[3 * C + lane] = __expf(static_cast<float>(glast));
        }
      }
      __syncthreads();   // K/Q no longer read: L and T may overlay them

      // 5. One pass over the lower triangle in fragment order: each decay factor
      //    exp(gamma_i - gamma_j) serves both L (strictly lower, into LDS) and P
      //    (lower incl. diagonal, split fragments to the workspace).  No
      //    branches: the exponent is masked to -inf above the diagonal and the
      //    masks are selects (the Gram tiles above the diagonal are never
      //    written, so their contents must not reach a product).
      if constexpr (kBwd) {
        // transposed blocks: lane l of block (mt, ks) covers column i of P and
        // L and rows j0 .. j0 + FE - 1 (the Gram tiles are read down a column)
        Elem* pb = static_cast<Elem*>(ws.p) + unit * W::op_elems;
        for (int f = tid; f < NT * NKS_C * 64; f += 256) {
          const int l = f & 63, blk = f >> 6;
          const int mt = blk / NKS_C, ks = blk % NKS_C;
          if (ks * Pol::KSTEP + Pol::KSTEP - 1 < 16 * mt) continue;   // wholly below the transposed diagonal
          const int i = 16 * mt + (l & 15), j0 = ks * Pol::KSTEP + (l >> 4) * FE;
          const double gi = s_gam[i];
          const float rki = s_rk[i];
          double gj[FE];
          float rkj[FE], rqj[FE], bj[FE], pv[FE];
          lds_row<FE>(s_gam + j0, gj);
          lds_row<FE>(s_rk + j0, rkj);
          lds_row<FE>(s_rq + j0, rqj);
          lds_row<FE>(s_beta + j0, bj);
#pragma unroll
          for (int e = 0; e < FE; ++e) {
            const int j = j0 + e;
            const float gq = sGQ[j * LDC + i], gk = sGK[j * LDC + i];
            const float dec = __expf(i <= j ? static_cast<float>(gj[e] - gi) : -INFINITY);
            pv[e] = i <= j ? scale * dec * rqj[e] * rki * gq : 0.f;
            sL[j * LDC + i] = i < j ? bj[e] * dec * rkj[e] * rki * gk : 0.f;
          }
          Pol::store_split(pb + W::op_block(mt, ks, 0) + l * FE, pb + W::op_block(mt, ks, Pol::NSPLIT - 1) + l * FE,
                           pv);
        }
      } else {
        Elem* pb = static_cast<Elem*>(ws.p) + unit * W::op_elems;
        for (int f = tid; f < NT * NKS_C * 64; f += 256) {
          const int l = f & 63, blk = f >> 6;
          const int mt = blk / NKS_C, ks = blk % NKS_C;
          if (ks * Pol::KSTEP > 16 * mt + 15) continue;   // wholly above the diagonal: never read
          const int i = 16 * mt + (l & 15), j0 = ks * Pol::KSTEP + (l >> 4) * FE;
          const double gi = s_gam[i];
          const float rki = s_rk[i], rqi = s_rq[i], bi = s_beta[i];
          double gj[FE];
          float rkj[FE], gq[FE], gk[FE], pv[FE], lv[FE];
          lds_row<FE>(s_gam + j0, gj);
          lds_row<FE>(s_rk + j0, rkj);
          lds_row<FE>(sGQ + i * LDC + j0, gq);
          lds_row<FE>(sGK + i * LDC + j0, gk);
#pragma unroll
          for (int e = 0; e < FE; ++e) {
            const int j = j0 + e;
            const float dec = __expf(j <= i ? static_cast<float>(gi - gj[e]) : -INFINITY);
            pv[e] = j <= i ? scale * dec * rqi * rkj[e] * gq[e] : 0.f;
            lv[e] = j < i ? bi * dec * rki * rkj[e] * gk[e] : 0.f;
          }
#pragma unroll
          for (int e = 0; e < FE; ++e) sL[i * LDC + j0 + e] = lv[e];
          Pol::store_split(pb + W::op_block(mt, ks, 0) + l * FE, pb + W::op_block(mt, ks, Pol::NSPLIT - 1) + l * FE,
                           pv);
        }
      }
      __syncthreads();

      // 6. T = (I + L)^-1
      unit_lower_inverse<C, LDC>(sL, sT);

      // 7. Tb = T diag(beta) (zero above the diagonal) as split fragments
      {
        Elem* tb = static_cast<Elem*>(ws.tb) + unit * W::op_elems;
        for (int f = tid; f < NT * NKS_C * 64; f += 256) {
          const int l = f & 63, blk = f >> 6;
          const int mt = blk / NKS_C, ks = blk % NKS_C;
          if (ks * Pol::KSTEP > 16 * mt + 15) continue;   // wholly above the diagonal: never read
          const int i = 16 * mt + (l & 15), j0 = ks * Pol::KSTEP + (l >> 4) * FE;
          float tr[FE], bj[FE], tv[FE];
          lds_row<FE>(sT + i * LDC + j0, tr);
          lds_row<FE>(s_beta + j0, bj);
#pragma unroll
          for (int e = 0; e < FE; ++e) tv[e] = j0 + e <= i ? tr[e] * bj[e] : 0.f;   // T above the diagonal is not written
          Pol::store_split(tb + W::op_block(mt, ks, 0) + l * FE, tb + W::op_block(mt, ks, Pol::NSPLIT - 1) + l * FE,
                           tv);
        }
        if constexpr (kBwd) {
          Elem* tbt = static_cast<Elem*>(ws.tbt) + unit * W::op_elems;
          for (int f = tid; f < NT * NKS_C * 64; f += 256) {
            const int l = f & 63, blk = f >> 6;
            const int mt = blk / NKS_C, ks = blk % NKS_C;
            if (ks * Pol::KSTEP + Pol::KSTEP - 1 < 16 * mt) continue;
            const int i = 16 * mt + (l & 15), j0 = ks * Pol::KSTEP + (l >> 4) * FE;
            const float bi = s_beta[i];
            float tv[FE];
#pragma unroll
            for (int e = 0; e < FE; ++e) tv[e] = i <= j0 + e ? sT[(j0 + e) * LDC + i] * bi : 0.f;
            Pol::store_split(tbt + W::op_block(mt, ks, 0) + l * FE,
                             tbt + W::op_block(mt, ks, Pol::NSPLIT - 1) + l * FE, tv);
          }
        }
      }
      __syncthreads();   // L, T, gamma and beta are rewritten by the next v-head or unit
      gv = g_next;
      bv = b_next;
    }
  }
#undef GDN_PREP_FETCH
}

// Transposing LDS read of 16-bit elements (gfx950 ds_read_b64_tr_b16): in each
// group of 16 lanes, lane i receives element i % 4 of the 8-byte rows that the
// lanes (i / 4) + 4 j address, j = 0..3 (checked on the device with a probe of
// distinct values).  Returned as the raw 64 bits (four bf16, element 0 low).
__device__ __forceinline__ uint2 lds_read_tr16(const __bf16* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf16_t;
  auto q = reinterpret_cast<__attribute__((address_space(3))) v4bf16_t*>(
      (__attribute__((address_space(3))) __bf16*)(const_cast<__bf16*>(p)));
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(q));
}

// Swizzled LDS rows of the bf16 scan.  The 16-byte units (8 elements) of a row
// are permuted by an XOR with a function of the row so that a fragment read
// touches every bank once.  On gfx950 a 16-byte read is served 16 lanes at a
// time (lanes whose index differs only in bits 0-2 and 4: here 8 consecutive
// rows x 2 adjacent units) over 64 banks, a layout fitted to the LDS
// bank-conflict counter of probe kernels.  The unpadded, swizzled rows halved
// the scan's conflict cycles against padded rows.  The 8-byte split stores of
// 4 values stay within one unit.
//   rows of 64 elements (8 units):   unit ^ (row % 8)
//   rows of 128 elements (16 units): unit ^ (2 (row % 8) + bit 2 of row)
template <int NE>
__device__ __forceinline__ int swz_off(int row, int unit) {
  static_assert(NE == 64 || NE == 128, "swizzled rows of 64 or 128 elements");
  if constexpr (NE == 64) return row * NE + ((unit ^ (row & 7)) << 3);
  else return row * NE + ((unit ^ (((row & 7) << 1) | ((row >> 2) & 1))) << 3);
}

// Four consecutive output values of one row (one 16- or 8-byte store).
template <class EO>
__device__ __forceinline__ void store_row4(typename EO::T* p, floatx4 v);
template <>
__device__ __forceinline__ void store_row4<F32>(float* p, floatx4 v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <>
__device__ __forceinline__ void store_row4<BF16>(uint16_t* p, floatx4 v) {
  const uint32_t a = static_cast<uint32_t>(f32_to_bf16_bits(v[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16);
  const uint32_t b = static_cast<uint32_t>(f32_to_bf16_bits(v[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(a, b);
}

// ---------------------------------------------------------------------------
// k_chunk_scan: one workgroup per (sequence, v-head, d_v slice of 16*NV)
// ---------------------------------------------------------------------------
//
// With kStates (the backward's forward pass) the scan writes the state
// entering every chunk to ws.states ([slot][h_v][d_v][d_k] fp32) instead of
// forming outputs, and runs one-token sequences too.
//
// With a prefix argument (Pre, at most one; the chunked backward's reverse
// scan), blocks [0, pre.nblk) run pre.run(...) and the scan takes the blocks
// after them, so that two latency-bound chains share the chip in one launch.
// The two then share one LDS buffer; without a prefix the scan's arrays are
// separate (a carved buffer, or the scan as a function called from the
// kernel, measured about 2 us slower per 4096-token call).
template <class P, class...>
struct FirstOf {
  using type = P;
};

template <class Pol, class EO, int D, int C, int NV, bool kStates = false, class... Pre>
__global__ __launch_bounds__(256) void k_chunk_scan(
    const typename Pol::In::T* __restrict__ q, const typename Pol::In::T* __restrict__ k,
    const typename Pol::In::T* __restrict__ v, int64_t q_stride, int64_t k_stride, int64_t v_stride,
    int h_qk, int h_v, const int32_t* __restrict__ cu, int n_seq, int64_t t_total,
    const float* __restrict__ init, float* __restrict__ fin, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ fresh, typename EO::T* __restrict__ o, ChunkWs ws, Pre... pre) {
  static_assert(sizeof...(Pre) <= 1, "at most one prefix");
  using Elem = typename Pol::Elem;
  using In = typename Pol::In;
  using Frag = typename Pol::Frag;
  using W = WsLayout<Pol, D, C>;
  constexpr int BV = 16 * NV;           // d_v columns of this workgroup (NV matrix-core N tiles)
  constexpr int NTILE = D / BV;
  constexpr bool kSwz = Pol::kSwizzle;
  static_assert(!kSwz || (C == 64 && D == 128), "swizzled rows: 64-token chunks, d = 128");
  constexpr int LDK = kSwz ? D : D + Pol::PAD;    // LDS rows of d_k elements
  constexpr int LDT = kSwz ? C : C + Pol::PAD;    // LDS rows of C token elements
  constexpr int NMT = C / 16;          // token tiles (one per wave)
  constexpr int NST = D / 16;          // d_k tiles of the state
  constexpr int SPW = (NST + 3) / 4;   // state tiles per wave
  constexpr int NSP = Pol::NSPLIT;
  constexpr int FE = Pol::FE;
  constexpr int KS = Pol::KSTEP;
  constexpr int NKS_D = D / KS;        // k-steps over d_k
  constexpr int NKS_C = C / KS;        // k-steps over the chunk's tokens
  constexpr bool kAllWaves = NMT == 4;         // every wave owns a token tile
  constexpr bool kAllTiles = NST % 4 == 0;     // every wave owns SPW state tiles
  static_assert(NMT <= 4, "one token tile per wave");
  static_assert(C % KS == 0 && D % KS == 0, "k-steps must tile C and D");

  // LDS: X, U, U2 (hi | lo rows of C tokens), S (hi | lo rows of d_k) and
  // the chunk's K rows (bf16 policy) in rows of LDKT elements.  A stride of
  // 68 banks keeps the 16-byte row stores free of bank conflicts; the
  // transposing reads take two passes at any stride (LDS bank-conflict
  // counter of probe kernels).
  constexpr int LDKT = D + 8;
  constexpr int kTE = NSP * BV * LDT, kSE = NSP * BV * LDK, kKE = Pol::kKtInLds ? C * LDKT : 1;
  Elem *sX, *sU, *sU2, *sS, *sKt;
  int64_t b = blockIdx.x;
  if constexpr (sizeof...(Pre) == 0) {
    __shared__ __attribute__((aligned(16))) Elem aX[kTE];
    __shared__ __attribute__((aligned(16))) Elem aU[kTE];
    __shared__ __attribute__((aligned(16))) Elem aU2[kTE];
    __shared__ __attribute__((aligned(16))) Elem aS[kSE];
    __shared__ __attribute__((aligned(16))) Elem aKt[kKE];
    sX = aX, sU = aU, sU2 = aU2, sS = aS, sKt = aKt;
  } else {
    using P0 = typename FirstOf<Pre...>::type;
    constexpr size_t kScan = sizeof(Elem) * (3 * kTE + kSE + kKE);
    constexpr size_t kBytes = kScan > P0::kLdsBytes ? kScan : P0::kLdsBytes;
    __shared__ __attribute__((aligned(16))) char buf[kBytes];
    const P0& p0 = (pre, ...);
    if (b < p0.nblk) {
      p0.run(b, buf, h_qk, h_v, cu, n_seq, t_total, ws);
      return;
    }
    b -= p0.nblk;
    Elem* const e = reinterpret_cast<Elem*>(buf);
    sX = e, sU = e + kTE, sU2 = e + 2 * kTE, sS = e + 3 * kTE, sKt = e + 3 * kTE + kSE;
  }
  Elem* const sX_lo = sX + (NSP - 1) * BV * LDT;
  Elem* const sU_lo = sU + (NSP - 1) * BV * LDT;
  Elem* const sU2_lo = sU2 + (NSP - 1) * BV * LDT;
  Elem* const sS_lo = sS + (NSP - 1) * BV * LDK;

  // Block order: sequences in ws.order (longest first), each a run of
  // h_v * NTILE consecutive blocks.  Inside a run the XCD-aware bijection
  // gives each XCD (the dispatcher places block b on XCD b % 8) a contiguous
  // range of heads, so the d_v tiles of one head share an L2 and its
  // K/Q/Tb/P reads, and every sequence is spread over all XCDs.
  const int64_t per_seq = static_cast<int64_t>(h_v) * NTILE;
  const int64_t rank = b / per_seq;
  if (rank >= n_seq) return;
  const int s = ws.order ? ws.order[rank] : static_cast<int>(rank);
  // State row of the sequence: its slot in the caller's state pool (identity
  // without a slot map).  A negative slot is an inactive lane, which reads
  // and writes nothing; a fresh sequence starts from the zero state.
  const int sslot = slots ? slots[s] : s;
  if (sslot < 0) return;
  const bool from_init = init != nullptr && !(fresh && fresh[s] != 0);
  const int64_t lid = xcd_order(b % per_seq, per_seq);
  const int tile = static_cast<int>(lid % NTILE);
  const int h = static_cast<int>(lid / NTILE);
  const int hq = h / (h_v / h_qk);
  const int dv0 = tile * BV;
  // one-token sequences belong to k_single_token
  if (!kStates && seq_start(cu, s + 1, t_total) - seq_start(cu, s, t_total) == 1) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const bool tok_wave = kAllWaves || wave < NMT;
  // Element offset of this lane's fragment (k-step ks) in row `row` of X, U, U2
  // (offT) or S (offS), and the split store of 4 consecutive values of a row.
  auto offT = [&](int row, int ks) -> int {
    if constexpr (kSwz) return swz_off<LDT>(row, ks * (KS / 8) + g4);
    else return row * LDT + ks * KS + g4 * FE;
  };
  auto offS = [&](int row, int ks) -> int {
    if constexpr (kSwz) return swz_off<LDK>(row, ks * (KS / 8) + g4);
    else return row * LDK + ks * KS + g4 * FE;
  };
  auto storeT = [&](Elem* hi, Elem* lo, int row, int col0, const float* v) {
    if constexpr (kSwz) Pol::put4(hi, lo, swz_off<LDT>(row, col0 >> 3) + (col0 & 7), v);
    else Pol::put4(hi, lo, row * LDT + col0, v);
  };
  auto storeS = [&](Elem* hi, Elem* lo, int row, int col0, const float* v) {
    if constexpr (kSwz) Pol::put4(hi, lo, swz_off<LDK>(row, col0 >> 3) + (col0 & 7), v);
    else Pol::put4(hi, lo, row * LDK + col0, v);
  };

  // fp32 master state: tiles (mt = wave + 4 j, nt) of S^T (rows d_k, columns
  // d_v): lane holds S[dv0 + 16 nt + r16][16 mt + 4 g4 + i].
  floatx4 Sacc[SPW][NV];
  const int64_t srow = ((int64_t)sslot * h_v + h) * D + dv0 + r16;   // state row of this lane (nt = 0)
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int mt = wave + 4 * j;
#pragma unroll
    for (int nt = 0; nt < NV; ++nt) {
      Sacc[j][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (kAllTiles || mt < NST) {
        if (from_init) {
          const float4 v4 = *reinterpret_cast<const float4*>(init + (srow + 16 * nt) * D + 16 * mt + 4 * g4);
          Sacc[j][nt] = floatx4{v4.x, v4.y, v4.z, v4.w};
        }
        const float tmp[4] = {Sacc[j][nt][0], Sacc[j][nt][1], Sacc[j][nt][2], Sacc[j][nt][3]};
        storeS(sS, sS_lo, 16 * nt + r16, 16 * mt + 4 * g4, tmp);
      }
    }
  }

  const int64_t start = seq_start(cu, s, t_total), end = seq_start(cu, s + 1, t_total);
  const int64_t nchunks = (end - start + C - 1) / C;
  const int64_t slot0 = start / C + s;
  const int orow0 = 16 * wave + 4 * g4;           // this lane's first output row

  // This wave's operand fragments for one chunk (registers).  Rows of K, Q
  // and V past the chunk's end re-read a valid row: their scalars (b rk,
  // scale b rq, exp(.) rk) and their Tb rows and columns are exactly zero, so
  // they contribute nothing and only need to be finite.
  Frag kf[NKS_D], qf[NKS_D];             // K, Q rows of the token tile
  Frag tbh[NKS_C], tbl[NKS_C];           // Tb rows (hi, lo)
  Frag ph[NKS_C], pl[NKS_C];             // P rows (hi, lo)
  Frag ktf[SPW][NKS_C];                  // K^T rows of the state tiles
  float4 c1v = {0.f, 0.f, 0.f, 0.f}, c3v = c1v;   // b rk, exp(.) rk of rows orow0 .. orow0 + 3
  float c2s = 0.f;                       // scale b rq of row 16 wave + r16 (outputs are built transposed)
  float bcv = 0.f;                       // b_C
  uint32_t vraw[NV][4] = {};             // raw V of rows orow0 .. orow0 + 3, per N tile
  int vlen = 0;
  const int nks_w = (16 * wave + 16 + KS - 1) / KS;   // k-steps reaching this tile's last row
  const uint32_t vs32 = static_cast<uint32_t>(v_stride);   // at most 2^24
  // V element (row orow0 + i, column dv0 + 16 nt + r16) of a chunk: the chunk's
  // uniform base plus a 32-bit lane offset (strides are at most 2^24)

#define GDN_LOAD_KV(jj)                                                                                 \
  do {                                                                                                 \
    const int64_t t0_ = start + (jj) * C;                                                              \
    const int len_ = static_cast<int>(end - t0_ < C ? end - t0_ : C);                                  \
    if (tok_wave) {                                                                                    \
      const Elem* kq_ = static_cast<const Elem*>(ws.kq) + ((slot0 + (jj)) * h_qk + hq) * W::kq_elems + lane * FE; \
      _Pragma("unroll") for (int ks_ = 0; ks_ < NKS_D; ++ks_) {                                        \
        kf[ks_] = Pol::ld(kq_ + W::kq_block(0, wave, ks_));                                            \
      }                                                                                                \
      const float* sc_ = ws.sc + ((slot0 + (jj)) * h_v + h) * (4 * C);                                \
      c1v = *reinterpret_cast<const float4*>(sc_ + orow0);                                             \
      c3v = *reinterpret_cast<const float4*>(sc_ + 2 * C + orow0);                                     \
      const typename In::T* vc_ = v + t0_ * v_stride + (int64_t)h * D + dv0 + r16;                     \
      _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                               \
        const int r_ = orow0 + i_ < len_ ? orow0 + i_ : len_ - 1;                                      \
        const uint32_t o_ = __umul24(static_cast<uint32_t>(r_), vs32);                                 \
        _Pragma("unroll") for (int nt_ = 0; nt_ < NV; ++nt_) vraw[nt_][i_] = to_u32(vc_[o_ + 16 * nt_]); \
      }                                                                                                \
      vlen = len_;                                                                                     \
    }                                                                                                  \
    bcv = ws.sc[((slot0 + (jj)) * h_v + h) * (4 * C) + 3 * C];                                         \
  } while (0)
#define GDN_LOAD_Q(jj)                                                                                 \
  do {                                                                                                 \
    if (!kStates && tok_wave) {                                                                        \
      const Elem* kq_ = static_cast<const Elem*>(ws.kq) + ((slot0 + (jj)) * h_qk + hq) * W::kq_elems + lane * FE; \
      _Pragma("unroll") for (int ks_ = 0; ks_ < NKS_D; ++ks_) qf[ks_] = Pol::ld(kq_ + W::kq_block(1, wave, ks_)); \
      c2s = ws.sc[((slot0 + (jj)) * h_v + h) * (4 * C) + C + 16 * wave + r16];                         \
    }                                                                                                  \
  } while (0)
#define GDN_LOAD_TB(jj)                                                                                \
  do {                                                                                                 \
    if (tok_wave) {                                                                                    \
      const Elem* tb_ = static_cast<const Elem*>(ws.tb) + ((slot0 + (jj)) * h_v + h) * W::op_elems + lane * FE; \
      _Pragma("unroll") for (int ks_ = 0; ks_ < NKS_C; ++ks_) {                                        \
        if (ks_ < nks_w) {                                                                             \
          tbh[ks_] = Pol::ld(tb_ + W::op_block(wave, ks_, 0));                                         \
          tbl[ks_] = Pol::ld(tb_ + W::op_block(wave, ks_, NSP - 1));                                   \
        }                                                                                              \
      }                                                                                                \
    }                                                                                                  \
  } while (0)
#define GDN_LOAD_PKT(jj)                                                                               \
  do {                                                                                                 \
    if (!kStates && tok_wave) {                                                                        \
      const Elem* p_ = static_cast<const Elem*>(ws.p) + ((slot0 + (jj)) * h_v + h) * W::op_elems + lane * FE; \
      _Pragma("unroll") for (int ks_ = 0; ks_ < NKS_C; ++ks_) {                                        \
        if (ks_ < nks_w) {                                                                             \
          ph[ks_] = Pol::ld(p_ + W::op_block(wave, ks_, 0));                                           \
          pl[ks_] = Pol::ld(p_ + W::op_block(wave, ks_, NSP - 1));                                     \
        }                                                                                              \
      }                                                                                                \
    }                                                                                                  \
    if constexpr (!Pol::kKtInLds) {                                                                    \
      const Elem* kt_ = static_cast<const Elem*>(ws.kt) + ((slot0 + (jj)) * h_qk + hq) * W::kt_elems + lane * FE; \
      _Pragma("unroll") for (int j_ = 0; j_ < SPW; ++j_) {                                             \
        if (kAllTiles || wave + 4 * j_ < NST) {                                                        \
          _Pragma("unroll") for (int ks_ = 0; ks_ < NKS_C; ++ks_)                                      \
              ktf[j_][ks_] = Pol::ld(kt_ + W::kt_block(wave + 4 * j_, ks_));                           \
        }                                                                                              \
      }                                                                                                \
    }                                                                                                  \
  } while (0)

  if (nchunks > 0) {
    GDN_LOAD_KV(0);
    GDN_LOAD_Q(0);
    GDN_LOAD_TB(0);
    GDN_LOAD_PKT(0);
  }
  __syncthreads();

  for (int64_t j = 0; j < nchunks; ++j) {
    const int64_t t0 = start + j * C;
    const int len = static_cast<int>(end - t0 < C ? end - t0 : C);
    // the chunk whose operands are fetched during this step (the last step
    // re-reads its own chunk, so every load is unconditional)
    const int64_t jn = j + 1 < nchunks ? j + 1 : j;
    if constexpr (kStates) {
      float* st = ws.states + (((slot0 + j) * h_v + h) * D + dv0 + r16) * D;
#pragma unroll
      for (int jj = 0; jj < SPW; ++jj) {
        const int mt = wave + 4 * jj;
        if (kAllTiles || mt < NST) {
#pragma unroll
          for (int nt = 0; nt < NV; ++nt)
            *reinterpret_cast<float4*>(st + 16 * nt * D + 16 * mt + 4 * g4) =
                make_float4(Sacc[jj][nt][0], Sacc[jj][nt][1], Sacc[jj][nt][2], Sacc[jj][nt][3]);
        }
      }
    }

    // ---- A: K S^T for token tile `wave`; X = V - diag(b rk) K S^T ----
    floatx4 Oacc[NV];
    Frag sfh[NV][NKS_D], sfl[NV][NKS_D];   // S fragments, reused for S Q^T in phase B
    const float4 c3 = c3v;
    const float bc = bcv;
    if (tok_wave) {
      floatx4 ak[NV];
#pragma unroll
      for (int nt = 0; nt < NV; ++nt) ak[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS_D; ++ks) {
#pragma unroll
        for (int nt = 0; nt < NV; ++nt) {
          const int off = offS(16 * nt + r16, ks);
          sfh[nt][ks] = Pol::ld(sS + off);
          ak[nt] = Pol::mma(kf[ks], sfh[nt][ks], ak[nt]);
          if constexpr (NSP == 2) {
            sfl[nt][ks] = Pol::ld(sS_lo + off);
            ak[nt] = Pol::mma(kf[ks], sfl[nt][ks], ak[nt]);
          }
        }
      }
      if constexpr (Pol::kKtInLds) {
        // the K rows of this token tile, for the K^T operands of the state update
#pragma unroll
        for (int ks = 0; ks < NKS_D; ++ks)
          *reinterpret_cast<Frag*>(sKt + (16 * wave + r16) * LDKT + ks * KS + g4 * FE) = kf[ks];
      }
      const float c1[4] = {c1v.x, c1v.y, c1v.z, c1v.w};
#pragma unroll
      for (int nt = 0; nt < NV; ++nt) {
        float xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float vv = (orow0 + i < vlen) ? from_u32<In>(vraw[nt][i]) : 0.f;
          xv[i] = vv - c1[i] * ak[nt][i];
        }
        storeT(sX, sX_lo, 16 * nt + r16, orow0, xv);
      }
    }
    __syncthreads();
    GDN_LOAD_KV(jn);   // K, V and the scalars of this step are consumed

    // ---- B: U = Tb X (lower triangular: k up to the tile's last row) ----
    if (tok_wave) {
      floatx4 au[NV];
#pragma unroll
      for (int nt = 0; nt < NV; ++nt) au[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS_C; ++ks) {
        if (ks < nks_w) {
#pragma unroll
          for (int nt = 0; nt < NV; ++nt) {
            const int off = offT(16 * nt + r16, ks);
            const Frag xh = Pol::ld(sX + off);
            au[nt] = Pol::mma(tbh[ks], xh, au[nt]);
            if constexpr (NSP == 2) {
              const Frag xl = Pol::ld(sX_lo + off);
              au[nt] = Pol::mma(tbh[ks], xl, au[nt]);
              au[nt] = Pol::mma(tbl[ks], xh, au[nt]);
            }
          }
        }
      }
      const float c3a[4] = {c3.x, c3.y, c3.z, c3.w};
#pragma unroll
      for (int nt = 0; nt < NV; ++nt) {
        float u2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u2[i] = c3a[i] * au[nt][i];
        const float uv[4] = {au[nt][0], au[nt][1], au[nt][2], au[nt][3]};
        storeT(sU, sU_lo, 16 * nt + r16, orow0, uv);
        storeT(sU2, sU2_lo, 16 * nt + r16, orow0, u2);
      }
    }
    GDN_LOAD_TB(jn);
    __syncthreads();

    // ---- C: O += P U, store rows; S^T <- b_C S^T + K^T U2 ----
    if (!kStates && tok_wave) {
      floatx4 aq[NV];
#pragma unroll
      for (int nt = 0; nt < NV; ++nt) {
        aq[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS_D; ++ks) {
          aq[nt] = Pol::mma(sfh[nt][ks], qf[ks], aq[nt]);   // transposed: O[16 wave + r16][dv 4 g4 + i]
          if constexpr (NSP == 2) aq[nt] = Pol::mma(sfl[nt][ks], qf[ks], aq[nt]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Oacc[nt][i] = c2s * aq[nt][i];
      }
    }
    GDN_LOAD_Q(jn);
    if (!kStates && tok_wave) {
#pragma unroll
      for (int ks = 0; ks < NKS_C; ++ks) {
        if (ks < nks_w) {
#pragma unroll
          for (int nt = 0; nt < NV; ++nt) {
            const int off = offT(16 * nt + r16, ks);
            const Frag uh = Pol::ld(sU + off);
            Oacc[nt] = Pol::mma(uh, ph[ks], Oacc[nt]);
            if constexpr (NSP == 2) {
              const Frag ul = Pol::ld(sU_lo + off);
              Oacc[nt] = Pol::mma(ul, ph[ks], Oacc[nt]);
              Oacc[nt] = Pol::mma(uh, pl[ks], Oacc[nt]);
            }
          }
        }
      }
      const int row = 16 * wave + r16;
      if (row < len) {
        typename EO::T* ob = o + (t0 + row) * ((int64_t)h_v * D) + (int64_t)h * D + dv0 + 4 * g4;
#pragma unroll
        for (int nt = 0; nt < NV; ++nt) store_row4<EO>(ob + 16 * nt, Oacc[nt]);
      }
    }
#pragma unroll
    for (int jj = 0; jj < SPW; ++jj) {
      const int mt = wave + 4 * jj;
      if (kAllTiles || mt < NST) {
#pragma unroll
        for (int nt = 0; nt < NV; ++nt) {
          floatx4 acc = Sacc[jj][nt] * bc;
#pragma unroll
          for (int ks = 0; ks < NKS_C; ++ks) {
            const int off = offT(16 * nt + r16, ks);
            Frag kt;
            if constexpr (Pol::kKtInLds) {
              // lane (r16, g4): K[tokens ks*KS + 8 g4 + 0..7][d_k 16 mt + r16], as two
              // transposing reads of four tokens (lane r16 addresses row r16 / 4,
              // columns 4 (r16 % 4) .. + 3 of the 16-column block)
              const Elem* kp = sKt + (ks * KS + 8 * g4 + (r16 >> 2)) * LDKT + 16 * mt + 4 * (r16 & 3);
              const uint2 a = lds_read_tr16(kp);
              const uint2 b = lds_read_tr16(kp + 4 * LDKT);
              kt = __builtin_bit_cast(Frag, make_uint4(a.x, a.y, b.x, b.y));
            } else {
              kt = ktf[jj][ks];
            }
            acc = Pol::mma(kt, Pol::ld(sU2 + off), acc);
            if constexpr (NSP == 2) acc = Pol::mma(kt, Pol::ld(sU2_lo + off), acc);
          }
          Sacc[jj][nt] = acc;
          const float tmp[4] = {acc[0], acc[1], acc[2], acc[3]};
          storeS(sS, sS_lo, 16 * nt + r16, 16 * mt + 4 * g4, tmp);
        }
      }
    }
    GDN_LOAD_PKT(jn);
    __syncthreads();
  }
#undef GDN_LOAD_KV
#undef GDN_LOAD_TB
#undef GDN_LOAD_Q
#undef GDN_LOAD_PKT

  if (fin) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int mt = wave + 4 * j;
      if (kAllTiles || mt < NST) {
#pragma unroll
        for (int nt = 0; nt < NV; ++nt)
          *reinterpret_cast<float4*>(fin + (srow + 16 * nt) * D + 16 * mt + 4 * g4) =
              make_float4(Sacc[j][nt][0], Sacc[j][nt][1], Sacc[j][nt][2], Sacc[j][nt][3]);
      }
    }
  }
}

}  // namespace gdn
