// Chunked prefill of the gated delta rule for bf16 inputs, d_k = d_v = 128,
// chunks of 64 tokens (gfx950): a prep kernel that builds every per-chunk
// operand in matrix-core fragment order, and a scan kernel whose four waves
// take four roles in a pipeline with one barrier per chunk.
//
// Recurrence, per sequence and v-head, fp32 state S (d_v x d_k):
//     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = scale S_t q_t
// (the gated delta rule of the GDN layers: haskell-infer-demo README,
// "Highlights" and "Architecture"/fla_gdn.cu; fp32 state with bf16
// intermediates: Flare core-design, GDN numerics paragraph).
//
// Chunk algebra.  A chunk of C tokens with raw bf16 rows K, Q, V enters with
// state S.  With rk = 1/|k|, rq = 1/|q| (L2 norm), gamma the inclusive running
// sum of g over the chunk and b = exp(gamma):
//     L_ij = beta_i e^{gamma_i - gamma_j} rk_i rk_j (k_i . k_j)   (j < i),  T = (I + L)^-1
//     P_ij = scale e^{gamma_i - gamma_j} rq_i rk_j (q_i . k_j)     (j <= i)
//     c1 = b rk,  c2 = scale b rq,  c3 = e^{gamma_C - gamma} rk,  bC = e^{gamma_C}
//     Y  = K S^T                     X  = V - diag(c1) Y          (error of the decayed state)
//     U2 = Tb' X,   Tb' = diag(c3) T diag(beta)                   (the token writes, pre-scaled)
//     O  = diag(c2) Q S^T + R X,   R = P T diag(beta)
//     S' = bC S + U2^T K
// Across chunks, with the raw inter-chunk Gram matrix G_{c+1} = K_{c+1} K_c^T,
//     Y_{c+1} = K_{c+1} S_{c+1}^T = bC_c (K_{c+1} S_c^T) + G_{c+1} U2_c,
// so the chain from one chunk's writes U2_c to the next chunk's error X_{c+1}
// needs the state S_c only through a product computed a step ahead.
//
// Kernels:
//   k_prep_bf16  persistent workgroups over (chunk slot, q/k head) units: the
//                Gram tiles K K^T, Q K^T and K_c K_{c-1}^T on the matrix cores
//                (raw bf16, exact products), then per v-head the decays, L,
//                P, the triangular solve, Tb' and R.  Writes K, Q, G, Tb' and
//                R as fragments (derived ones as bf16 hi + lo) and c1, c2, bC.
//   k_scan_bf16  one workgroup of four waves per (sequence, v-head, 16-wide
//                d_v slice), walking the chunks in ticks:
//                  wave 0 (chain)  Y_c = bC Z_c + G_c U2_{c-1}, X_c, U2_c = Tb'_c X_c
//                  waves 1, 2 (state) one d_k half each of S in fp32:
//                                  S_{c} = bC S_{c-1} + U2_{c-1}^T K_{c-1},
//                                  Z_{c+1} = K_{c+1} S_c^T (partial over the half)
//                  wave 3 (output) O_c = diag(c2) Q_c S_c^T + R_c X_c
//                Every tick each wave does its part for a different chunk and
//                hands its results to the others through LDS buffers indexed
//                by the tick's parity; one workgroup barrier ends the tick.
//
// Fragment conventions (v_mfma_f32_16x16x32_bf16).  Lane l = 16 g + r holds an
// A fragment: row r, 8 k elements; a B fragment: column r, 8 k elements; and
// accumulates output rows 4 g + i (i = 0..3) of column r.  The 8 k elements of
// slot e are k = 32 s + kap(g, e), kap(g, e) = 4 g + (e & 3) + 16 (e >> 2), so
// an output pair of 16-row tiles (2s, 2s+1) held by a lane is, unchanged, the
// B fragment (or the transposed A fragment) of k-step s of a following
// product: every product of the chain and of the state update takes its
// derived operand straight from the registers of the product before it.
// Operands the prep writes use the same k order.
//
// Precision (as the general chunk kernels): raw bf16 q/k/v are exact single
// operands; every derived operand (S, X, U2, G, Tb', R) is a bf16 hi + lo pair
// and a product uses hi*hi + hi*lo + lo*hi (or hi*raw + lo*raw), accumulated
// in fp32 (the multi-term bf16 technique of Henry, Tang and Heinecke, ARITH
// 2019); the state master copy is fp32.
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int kD = 128;
constexpr int kC = 64;
constexpr int kBlk = 512;        // bf16 elements per fragment block (64 lanes x 8)
constexpr int kScStride = 132;   // floats per (slot, v-head): c1[64] | c2[64] | bC | pad

__device__ __forceinline__ floatx4 mma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma_f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// hi*hi + hi*lo + lo*hi
__device__ __forceinline__ floatx4 mma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, floatx4 c) {
  c = mma16(ah, bh, c);
  c = mma16(ah, bl, c);
  return mma16(al, bh, c);
}

// Two fp32 values as a packed bf16 hi pair and a packed bf16 lo pair
// (hi = RNE(x), lo = RNE(x - hi)): one paired conversion for each part.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a - ha, b - hb}, bf16x2));
}

// Two output tiles of a lane (rows 4g..4g+3 of tiles 2s and 2s+1) as one
// fragment of k-step s, split into bf16 hi and lo parts.
__device__ __forceinline__ void split_pair(const floatx4& a, const floatx4& b, bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
  split2(a[0], a[1], h[0], l[0]);
  split2(a[2], a[3], h[1], l[1]);
  split2(b[0], b[1], h[2], l[2]);
  split2(b[2], b[3], h[3], l[3]);
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

// Eight values as one hi and one lo fragment.
__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) split2(v[2 * i], v[2 * i + 1], h[i], l[i]);
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

// Index of block (token tile t, k-step s) among the lower-triangular blocks of
// a 64 x 64 operand whose k-steps are 32 wide: s <= t / 2, six blocks.
__host__ __device__ constexpr int tri_blk(int t, int s) { return t < 2 ? t : 2 * t - 2 + s; }

// Transposing LDS read of 16-bit elements (gfx950 ds_read_b64_tr_b16): in each
// group of 16 lanes, lane i receives element i % 4 of the 8-byte rows that the
// lanes (i / 4) + 4 j address, j = 0..3 (checked on the device with a probe of
// distinct values).  Returned as the raw 64 bits (four bf16, element 0 low).
__device__ __forceinline__ uint2 lds_tr16(const uint16_t* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf16_t;
  auto q = reinterpret_cast<__attribute__((address_space(3))) v4bf16_t*>(
      (__attribute__((address_space(3))) uint16_t*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(q));
}

__device__ __forceinline__ bf16x8 ld_frag(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void st_frag(uint16_t* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }

// 8 bytes (4 bf16) from LDS
__device__ __forceinline__ uint2 lds8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }

}  // namespace

// Workspace of the bf16 path, indexed by chunk slot (see locate_block):
//   kfr [slots][h_qk][16 blocks (t, sf)]      K fragments: K[16t + r][32 sf + kap(g, e)]
//   qfr [slots][h_qk][16 blocks (t, sf)]      Q fragments, same order
//   gfr [slots][h_qk][8 blocks (t, s)][hi|lo] G fragments: G[16t + r][32 s + kap(g, e)]
//   tfr [slots][h_v][6 blocks tri(t, s)][hi|lo] Tb' fragments, same order
//   rfr [slots][h_v][6 blocks tri(t, s)][hi|lo] R fragments, same order
//   sc  [slots][h_v][132] fp32                c1[64] | c2[64] | bC
//   order [n_seq] int32                       sequences, most chunks first (n_seq > 1)
//   o   [t_total][h_v][128] fp32              outputs before the fused norm (with z)
struct Bf16Ws {
  uint16_t* kfr;
  uint16_t* qfr;
  uint16_t* gfr;
  uint16_t* tfr;
  uint16_t* rfr;
  float* sc;
  int32_t* order;
  float* o_pre;
};

namespace {

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

struct Bf16Sizes {
  size_t kfr, gfr, tfr, sc, order, o_pre;
  Bf16Sizes(int64_t slots, int h_qk, int h_v, int n_seq, int64_t t_total, bool with_norm) {
    kfr = al256(sizeof(uint16_t) * slots * h_qk * 16 * kBlk);
    gfr = al256(sizeof(uint16_t) * slots * h_qk * 16 * kBlk);
    tfr = al256(sizeof(uint16_t) * slots * h_v * 12 * kBlk);
    sc = al256(sizeof(float) * slots * h_v * kScStride);
    order = n_seq > 1 ? al256(sizeof(int32_t) * n_seq) : 0;
    o_pre = with_norm ? al256(sizeof(float) * t_total * h_v * kD) : 0;
  }
  size_t total() const { return 2 * kfr + gfr + 2 * tfr + sc + order + o_pre; }
};

Bf16Ws carve(void* base, int64_t slots, int h_qk, int h_v, int n_seq, int64_t t_total, bool with_norm) {
  const Bf16Sizes z(slots, h_qk, h_v, n_seq, t_total, with_norm);
  char* b = static_cast<char*>(base);
  Bf16Ws w;
  w.kfr = reinterpret_cast<uint16_t*>(b); b += z.kfr;
  w.qfr = reinterpret_cast<uint16_t*>(b); b += z.kfr;
  w.gfr = reinterpret_cast<uint16_t*>(b); b += z.gfr;
  w.tfr = reinterpret_cast<uint16_t*>(b); b += z.tfr;
  w.rfr = reinterpret_cast<uint16_t*>(b); b += z.tfr;
  w.sc = reinterpret_cast<float*>(b); b += z.sc;
  w.order = n_seq > 1 ? reinterpret_cast<int32_t*>(b) : nullptr; b += z.order;
  w.o_pre = with_norm ? reinterpret_cast<float*>(b) : nullptr;
  return w;
}

}  // namespace

size_t chunk_bf16_ws_bytes(int h_qk, int h_v, int n_seq, int64_t t_total, int with_norm) {
  const int64_t slots = block_slots(t_total, n_seq, kC);
  return Bf16Sizes(slots, h_qk, h_v, n_seq, t_total, with_norm != 0).total();
}

// ---------------------------------------------------------------------------
// k_prep_bf16: persistent workgroups over (chunk slot, q/k head) units
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void k_prep_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                   int64_t q_stride, int64_t k_stride, GateSrc gates, float scale,
                                                   int use_l2, float l2_eps, int h_qk, int h_v,
                                                   const int32_t* __restrict__ cu, int n_seq, int64_t t_total,
                                                   const int32_t* __restrict__ seq_slots, Bf16Ws ws,
                                                   int64_t n_slots) {
  constexpr int D = kD, C = kC;
  constexpr int LDK = D + 8;    // bf16 elements per K/Q row in LDS
  constexpr int LDC = C + 4;    // floats per L/T/P row
  constexpr int ROWS_BYTES = 3 * C * LDK * 2;
  constexpr int MAT_BYTES = 3 * C * LDC * 4;
  // K, Q and previous-chunk K rows during the Gram phase; then L, T and P.
  __shared__ __attribute__((aligned(16))) char smem[ROWS_BYTES > MAT_BYTES ? ROWS_BYTES : MAT_BYTES];
  __shared__ __attribute__((aligned(16))) float s_rk[C];
  __shared__ __attribute__((aligned(16))) float s_rq[C];
  // the chunk's running sum of g, in fp64: with strong decays it reaches
  // hundreds, and the decay between two tokens is a difference of two sums
  __shared__ __attribute__((aligned(16))) double s_gam[C];
  __shared__ __attribute__((aligned(16))) float s_beta[C];
  __shared__ __attribute__((aligned(16))) float s_c3[C];
  // the sequence boundaries, staged once: every unit locates its sequence
  // from them, and a global read there would stall the unit's start
  constexpr int kCuLds = 256;
  __shared__ int32_t s_cu[kCuLds + 1];
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sQ = sK + C * LDK;
  uint16_t* sKp = sQ + C * LDK;
  float* sL = reinterpret_cast<float*>(smem);
  float* sT = sL + C * LDC;
  float* sP = sT + C * LDC;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int grp = h_v / h_qk;
  constexpr int TPR = D / 8, RPP = 256 / TPR, NR = C / RPP;   // 16 lanes per row, 16 rows per pass, 4 passes

  if (cu != nullptr && n_seq <= kCuLds) {
    for (int i = threadIdx.x; i <= n_seq; i += 256) s_cu[i] = cu[i];
    __syncthreads();
    cu = s_cu;
  }
  const int64_t n_units = n_slots * h_qk;
  const int64_t stride = gridDim.x;
  // Several workgroups share a compute unit: while one waits for its rows
  // the others compute, so a unit loads its own rows when it starts.
  for (int64_t u = blockIdx.x; u < n_units; u += stride) {
    int seq_i = 0, len = 0;
    int64_t t0 = 0;
    bool ok = locate_block(cu, n_seq, t_total, C, u / h_qk, seq_i, t0, len);
    if (ok && seq_slots) ok = seq_slots[seq_i] >= 0;   // inactive lane: no scan reads it
    if (ok && len == 1)   // a one-token sequence: the plain recurrence runs it
      ok = seq_start(cu, seq_i + 1, t_total) - seq_start(cu, seq_i, t_total) > 1;
    if (!ok) continue;
    const bool has_prev = t0 > seq_start(cu, seq_i, t_total);
    const int64_t cslot = u / h_qk;
    const int hq = static_cast<int>(u % h_qk);
    uint32_t gr0, br0;
    gate_load_raw(gates, t0 + (lane < len ? lane : len - 1), hq * grp, h_v, gr0, br0);
    {
      // 1. the raw K, Q (zero past len) and previous-chunk K rows to LDS,
      //    and the L2 scales of K and Q
#pragma unroll
      for (int it = 0; it < NR; ++it) {
        const int row = it * RPP + tid / TPR, c8 = (tid % TPR) * 8;
        const bool valid = row < len;
        const int64_t tok = t0 + (valid ? row : 0);
        const int64_t col = static_cast<int64_t>(hq) * D + c8;
        uint4 kv4 = *reinterpret_cast<const uint4*>(k + tok * k_stride + col);
        uint4 qv4 = *reinterpret_cast<const uint4*>(q + tok * q_stride + col);
        if (has_prev)
          *reinterpret_cast<uint4*>(sKp + row * LDK + c8) =
              *reinterpret_cast<const uint4*>(k + (t0 - C + row) * k_stride + col);
        if (!valid) kv4 = qv4 = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(sK + row * LDK + c8) = kv4;
        *reinterpret_cast<uint4*>(sQ + row * LDK + c8) = qv4;
        float kv[8], qv[8];
        BF16::unpack8(kv4, kv);
        BF16::unpack8(qv4, qv);
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          sk = __builtin_fmaf(kv[i], kv[i], sk);
          sq = __builtin_fmaf(qv[i], qv[i], sq);
        }
        sk = group_sum<TPR>(sk);
        sq = group_sum<TPR>(sq);
        if (tid % TPR == 0) {
          s_rk[row] = !valid ? 0.f : (use_l2 ? 1.0f / sqrtf(sk + l2_eps) : 1.0f);
          s_rq[row] = !valid ? 0.f : (use_l2 ? 1.0f / sqrtf(sq + l2_eps) : 1.0f);
        }
      }
    }
    __syncthreads();

    // 2. lower-triangular Gram tiles K K^T (tasks 0..9) and Q K^T (10..19),
    //    kept in registers for the per-v-head passes: wave w owns tasks
    //    w + 4 j.  Raw operands, exact products, fp32 sums.
    floatx4 gram[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int task = wave + 4 * j;
      const bool isq = task >= 10;
      const int idx = isq ? task - 10 : task;
      const int ti = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
      const int tj = idx - ti * (ti + 1) / 2;
      const uint16_t* ap = (isq ? sQ : sK) + (16 * ti + r16) * LDK + 8 * g4;
      const uint16_t* bp = sK + (16 * tj + r16) * LDK + 8 * g4;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) acc = mma16(ld_frag(ap + 32 * ks), ld_frag(bp + 32 * ks), acc);
      gram[j] = acc;
    }
    // 3. G = K_c K_{c-1}^T, computed transposed so that each lane ends with
    //    G[16t + r][16 jb + 4g + i]: wave w owns row tile t = w, and the pair
    //    of column tiles (2s, 2s+1) is the fragment of k-step s.
    if (has_prev) {
      const uint16_t* bp = sK + (16 * wave + r16) * LDK + 8 * g4;
      floatx4 gt[4];
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const uint16_t* ap = sKp + (16 * jb + r16) * LDK + 8 * g4;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) acc = mma16(ld_frag(ap + 32 * ks), ld_frag(bp + 32 * ks), acc);
        gt[jb] = acc;
      }
      uint16_t* gb = ws.gfr + (cslot * h_qk + hq) * 16 * kBlk + lane * 8;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 hi, lo;
        split_pair(gt[2 * s], gt[2 * s + 1], hi, lo);
        st_frag(gb + ((wave * 2 + s) * 2 + 0) * kBlk, hi);
        st_frag(gb + ((wave * 2 + s) * 2 + 1) * kBlk, lo);
      }
    }
    // 4. K and Q fragments: block (t, sf), lane (r, g): row 16t + r, columns
    //    32 sf + kap(g, e) (two 8-byte pieces of the row)
    {
      uint16_t* kb = ws.kfr + (cslot * h_qk + hq) * 16 * kBlk;
      uint16_t* qb = ws.qfr + (cslot * h_qk + hq) * 16 * kBlk;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int f = tid + 256 * j;                 // 2 x 16 blocks x 64 lanes
        const int l = f & 63, blk = (f >> 6) & 15, which = f >> 10;
        const int t = blk >> 2, sf = blk & 3, r = l & 15, g = l >> 4;
        const uint16_t* src = (which ? sQ : sK) + (16 * t + r) * LDK + 32 * sf + 4 * g;
        const uint2 a = lds8(src), b = lds8(src + 16);
        *reinterpret_cast<uint4*>((which ? qb : kb) + blk * kBlk + l * 8) = make_uint4(a.x, a.y, b.x, b.y);
      }
    }
    __syncthreads();   // rows no longer read: L, T and P may overlay them

    uint32_t graw = gr0, braw = br0;
    for (int vh = 0; vh < grp; ++vh) {
      const int h = hq * grp + vh;
      const int64_t unit = cslot * h_v + h;
      // the next v-head's gate inputs load during this one (the last v-head
      // reloads its own: an unconditional load stays here)
      uint32_t graw_next, braw_next;
      gate_load_raw(gates, t0 + (lane < len ? lane : len - 1), vh + 1 < grp ? h + 1 : h, h_v, graw_next, braw_next);
      float gv, bv;
      gate_from_raw(gates, h, graw, braw, gv, bv);
      if (lane >= len) gv = bv = 0.f;

      // 5. decays: inclusive running sum of g over the chunk (padded tokens
      //    add 0), and the per-token scalars
      if (wave == 0) {
        double gam = gv;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const double o = __shfl_up(gam, off, 64);
          if (lane >= off) gam += o;
        }
        const double glast = __shfl(gam, C - 1, 64);
        float* sc = ws.sc + unit * kScStride;
        s_gam[lane] = gam;
        s_beta[lane] = bv;
        const float b = __expf(static_cast<float>(gam));
        s_c3[lane] = __expf(static_cast<float>(glast - gam)) * s_rk[lane];
        sc[lane] = b * s_rk[lane];
        sc[C + lane] = scale * b * s_rq[lane];
        if (lane == 0) sc[2 * C] = __expf(static_cast<float>(glast));
      }
      __syncthreads();

      // 6. L (strictly lower) and P (lower with the diagonal) from the Gram
      //    tiles in registers; each decay factor is masked to -inf above the
      //    diagonal before the exponential, and the masks are selects.  All
      //    LDS reads are gathered before the first write, so they overlap.
      {
        float val[5][4];
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          const int task = wave + 4 * j;
          const bool isq = task >= 10;
          const int idx = isq ? task - 10 : task;
          const int ti = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
          const int tj = idx - ti * (ti + 1) / 2;
          const int col = 16 * tj + r16, row0 = 16 * ti + 4 * g4;
          const double gj = s_gam[col];
          const float rkj = s_rk[col];
          double gr[4];
          float sr[4], br[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            gr[i] = s_gam[row0 + i];
            sr[i] = isq ? s_rq[row0 + i] : s_rk[row0 + i];
            br[i] = s_beta[row0 + i];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = row0 + i;
            const float dec = __expf(col <= row ? static_cast<float>(gr[i] - gj) : -INFINITY);
            if (isq) val[j][i] = col <= row ? scale * dec * sr[i] * rkj * gram[j][i] : 0.f;
            else val[j][i] = col < row ? br[i] * dec * sr[i] * rkj * gram[j][i] : 0.f;
          }
        }
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          const int task = wave + 4 * j;
          const bool isq = task >= 10;
          const int idx = isq ? task - 10 : task;
          const int ti = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
          const int tj = idx - ti * (ti + 1) / 2;
          float* dst = isq ? sP : sL;
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[(16 * ti + 4 * g4 + i) * LDC + 16 * tj + r16] = val[j][i];
        }
      }
      __syncthreads();

      // 7. T = (I + L)^-1.  Diagonal 16x16 blocks: lane 16b + c owns column c
      //    of block b and runs forward substitution T_i = e_i - sum_{j<i} L_ij T_j.
      if (wave == 0) {
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
      //    T_{bi,bj} = -T_{bi,bi} sum_{kb=bj}^{bi-1} L_{bi,kb} T_{kb,bj}   (fp32 MFMA)
      for (int d = 1; d < 4; ++d) {
        const int bi = d + wave;
        if (bi < 4) {
          const int bj = bi - d;
          floatx4 w = {0.f, 0.f, 0.f, 0.f};
          for (int kb = bj; kb < bi; ++kb) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const int kk = 4 * ks + g4;
              w = mma_f32(sL[(16 * bi + r16) * LDC + 16 * kb + kk], sT[(16 * kb + kk) * LDC + 16 * bj + r16], w);
            }
          }
          // w holds W[4g+i][r16]; use it as the B operand with k = 4g + step
          floatx4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) t = mma_f32(sT[(16 * bi + r16) * LDC + 16 * bi + 4 * g4 + s], w[s], t);
#pragma unroll
          for (int i = 0; i < 4; ++i) sT[(16 * bi + 4 * g4 + i) * LDC + 16 * bj + r16] = -t[i];
        }
        __syncthreads();
      }

      // 8. Tb' = diag(c3) T diag(beta) (zero above the diagonal) as split
      //    fragments: block (t, s), lane (r, g): row 16t + r, columns 32 s + kap(g, e)
      {
        uint16_t* tb = ws.tfr + unit * 12 * kBlk;
        for (int f = tid; f < 6 * 64; f += 256) {
          const int l = f & 63, bi6 = f >> 6;
          const int t = bi6 < 2 ? bi6 : 2 + ((bi6 - 2) >> 1), s = bi6 < 2 ? 0 : ((bi6 - 2) & 1);
          const int r = l & 15, g = l >> 4, row = 16 * t + r;
          const float c3 = s_c3[row];
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int col = 32 * s + 4 * g + (e & 3) + 16 * (e >> 2);
            v[e] = col <= row ? c3 * sT[row * LDC + col] * s_beta[col] : 0.f;   // T above the diagonal is not written
          }
          bf16x8 hi, lo;
          split8(v, hi, lo);
          st_frag(tb + (bi6 * 2 + 0) * kBlk + l * 8, hi);
          st_frag(tb + (bi6 * 2 + 1) * kBlk + l * 8, lo);
        }
      }
      // 9. R = P T diag(beta), computed transposed (R^T = (T diag(beta))^T P^T,
      //    fp32 MFMA) so each lane ends with R[16 ib + r][16 jb + 4g + i]:
      //    wave w owns row tile ib = w and the column tiles jb <= w.
      {
        const int ib = wave;
        floatx4 rt[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          if (jb <= ib) {
            const float bj = s_beta[16 * jb + r16];
            for (int kb = jb; kb <= ib; ++kb) {
#pragma unroll
              for (int ks = 0; ks < 4; ++ks) {
                const int kk = 16 * kb + 4 * ks + g4;
                acc = mma_f32(sT[kk * LDC + 16 * jb + r16] * bj, sP[(16 * ib + r16) * LDC + kk], acc);
              }
            }
          }
          rt[jb] = acc;
        }
        uint16_t* rb = ws.rfr + unit * 12 * kBlk + lane * 8;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (2 * s <= ib) {
            bf16x8 hi, lo;
            split_pair(rt[2 * s], rt[2 * s + 1], hi, lo);
            st_frag(rb + (tri_blk(ib, s) * 2 + 0) * kBlk, hi);
            st_frag(rb + (tri_blk(ib, s) * 2 + 1) * kBlk, lo);
          }
        }
      }
      __syncthreads();   // L, T, P and the decay arrays are rewritten by the next v-head or unit
      graw = graw_next;
      braw = braw_next;
    }
  }
}

// ---------------------------------------------------------------------------
// k_scan_bf16: one workgroup of four role waves per (sequence, v-head, d_v slice)
// ---------------------------------------------------------------------------
template <class EO>
__global__ __launch_bounds__(256) void k_scan_bf16(const uint16_t* __restrict__ v, int64_t v_stride, int h_qk,
                                                   int h_v, const int32_t* __restrict__ cu, int n_seq,
                                                   int64_t t_total, const float* __restrict__ init,
                                                   float* __restrict__ fin, const int32_t* __restrict__ slots,
                                                   const int32_t* __restrict__ fresh, typename EO::T* __restrict__ o,
                                                   Bf16Ws ws) {
  constexpr int D = kD, C = kC, NTILE = D / 16;
  constexpr int LDKT = 64 + 8;   // bf16 per row of a state wave's K tile (its 64 d_k columns)
  // Hand-over buffers, indexed by the parity of the tick that wrote them:
  __shared__ floatx4 zbuf[2][2][4][64];          // Z partials: [p][state wave][token tile][lane]
  __shared__ bf16x8 u2buf[2][2][2][64];          // U2 fragments: [p][k-step][hi|lo][lane]
  __shared__ bf16x8 xbuf[2][2][2][64];           // X fragments
  __shared__ bf16x8 sbuf[2][2][2][2][64];        // S fragments: [p][state wave][k-step][hi|lo][lane]
  __shared__ __attribute__((aligned(16))) uint16_t ktile[2][2][64 * LDKT];   // [state wave][p] K rows

  // Block order: sequences in ws.order (longest first), each a run of
  // h_v * NTILE consecutive blocks; inside a run the XCD-aware bijection gives
  // each XCD a contiguous range of heads, so the d_v slices of one head share
  // an L2 and its operand reads, and every sequence spreads over all XCDs.
  const int64_t per_seq = static_cast<int64_t>(h_v) * NTILE;
  const int64_t bidx = blockIdx.x;
  const int64_t rank = bidx / per_seq;
  if (rank >= n_seq) return;
  const int s = ws.order ? ws.order[rank] : static_cast<int>(rank);
  const int sslot = slots ? slots[s] : s;
  if (sslot < 0) return;   // inactive lane: reads and writes nothing
  const bool from_init = init != nullptr && !(fresh && fresh[s] != 0);
  const int64_t lid = xcd_order(bidx % per_seq, per_seq);
  const int tile = static_cast<int>(lid % NTILE);
  const int h = static_cast<int>(lid / NTILE);
  const int hq = h / (h_v / h_qk);
  const int dv0 = tile * 16;
  const int64_t start = seq_start(cu, s, t_total), end = seq_start(cu, s + 1, t_total);
  if (end - start == 1) return;   // one-token sequences belong to k_single_token
  const int n = static_cast<int>((end - start + C - 1) / C);
  const int64_t slot0 = start / C + s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int64_t srow = (static_cast<int64_t>(sslot) * h_v + h) * D + dv0 + r16;   // state row of this lane
  auto sc_of = [&](int c) { return ws.sc + ((slot0 + c) * h_v + h) * kScStride; };
  if (n == 0) {
    // a zero-length sequence: its final state is the initial one (zeros without it)
    if (fin && (wave == 1 || wave == 2)) {
      const int w = wave - 1;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int64_t e = srow * D + 64 * w + 16 * mt + 4 * g4;
        *reinterpret_cast<float4*>(fin + e) =
            from_init ? *reinterpret_cast<const float4*>(init + e) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }
  // Next-chunk operands are fetched unconditionally (the last chunk fetches
  // itself again): a prefetch under a branch leaves two versions of its
  // registers to merge at the join, which makes the wave wait for the load.
  auto next_c = [&](int c) { return c + 1 < n ? c + 1 : n - 1; };

  if (wave == 0) {
    // ------------------------------------------------------------ chain
    const uint16_t* vb = v + static_cast<int64_t>(h) * D + dv0 + r16;
    const uint32_t vs32 = static_cast<uint32_t>(v_stride);   // at most 2^24
    bf16x8 gh[4][2], gl[4][2];     // G_c fragments (t, s)
    bf16x8 th[6], tl[6];           // Tb'_c fragments
    uint32_t vr[4][4];             // V of rows 16t + 4g + i, column dv0 + r (raw bf16 bits)
    float4 c1v[4];                 // c1 of those rows
    float bcp = 1.f;               // bC of the previous chunk
    bf16x8 uh[2], ul[2];           // U2 of the previous chunk, k-steps 0, 1
    auto load_g = [&](int c) {
      const uint16_t* gp = ws.gfr + ((slot0 + c) * h_qk + hq) * 16 * kBlk + lane * 8;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          gh[t][s2] = ld_frag(gp + ((t * 2 + s2) * 2 + 0) * kBlk);
          gl[t][s2] = ld_frag(gp + ((t * 2 + s2) * 2 + 1) * kBlk);
        }
    };
    auto load_t = [&](int c) {
      const uint16_t* tp = ws.tfr + ((slot0 + c) * h_v + h) * 12 * kBlk + lane * 8;
#pragma unroll
      for (int b = 0; b < 6; ++b) {
        th[b] = ld_frag(tp + (b * 2 + 0) * kBlk);
        tl[b] = ld_frag(tp + (b * 2 + 1) * kBlk);
      }
    };
    auto load_v = [&](int c) {
      const int64_t t0 = start + static_cast<int64_t>(c) * C;
      const int len = static_cast<int>(end - t0 < C ? end - t0 : C);
      const uint16_t* vc = vb + t0 * v_stride;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * t + 4 * g4 + i;
          const uint32_t off = __umul24(static_cast<uint32_t>(row < len ? row : len - 1), vs32);
          vr[t][i] = vc[off];   // converted where it is used, so the load is not waited for here
        }
      const float* sc = sc_of(c);
#pragma unroll
      for (int t = 0; t < 4; ++t) c1v[t] = *reinterpret_cast<const float4*>(sc + 16 * t + 4 * g4);
    };
    load_g(next_c(0));
    load_t(0);
    load_v(0);
    for (int tick = 0; tick <= n + 1; ++tick) {
      const int c = tick - 1;
      if (c >= 0 && c < n) {
        const int p = tick & 1, pz = (tick - 1) & 1;
        // Y = bC_{c-1} Z_c + G_c U2_{c-1}   (Y_0 = Z_0): the accumulators start
        // from the state waves' partials, then take the G products
        floatx4 y[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const floatx4 za = zbuf[pz][0][t][lane], zb = zbuf[pz][1][t][lane];
          y[t] = (za + zb) * bcp;
        }
        if (c > 0) {
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int t = 0; t < 4; ++t) y[t] = mma3(gh[t][s2], gl[t][s2], uh[s2], ul[s2], y[t]);
        }
        load_g(next_c(c));
        // X = V - c1 Y
        floatx4 x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float c1[4] = {c1v[t].x, c1v[t].y, c1v[t].z, c1v[t].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) x[t][i] = __builtin_fmaf(-c1[i], y[t][i], __uint_as_float(vr[t][i] << 16));
        }
        load_v(next_c(c));
        bf16x8 xh[2], xl[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          split_pair(x[2 * s2], x[2 * s2 + 1], xh[s2], xl[s2]);
          xbuf[p][s2][0][lane] = xh[s2];
          xbuf[p][s2][1][lane] = xl[s2];
        }
        // U2 = Tb' X (lower-triangular blocks)
        floatx4 u[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) u[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (s2 <= (t >> 1)) u[t] = mma3(th[tri_blk(t, s2)], tl[tri_blk(t, s2)], xh[s2], xl[s2], u[t]);
        load_t(next_c(c));
        bcp = sc_of(c)[2 * C];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          split_pair(u[2 * s2], u[2 * s2 + 1], uh[s2], ul[s2]);
          u2buf[p][s2][0][lane] = uh[s2];
          u2buf[p][s2][1][lane] = ul[s2];
        }
      }
      __syncthreads();
    }
  } else if (wave <= 2) {
    // ------------------------------------------------------------ state
    const int w = wave - 1;            // d_k half 64 w .. 64 w + 63
    floatx4 sacc[4];                   // S^T rows (d_k) 64 w + 16 mt + 4g + i, column dv0 + r
    bf16x8 sh[2], sl[2];               // S as fragments of k-steps s (d_k 64 w + 32 s + kap)
    bf16x8 kf[4][2];                   // K_tick fragments of this half
    float bq0 = 1.f, bq1 = 1.f;        // bC of chunks tick - 2 and tick - 1
    auto load_k = [&](int c) {
      const uint16_t* kp = ws.kfr + ((slot0 + c) * h_qk + hq) * 16 * kBlk + lane * 8;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) kf[t][s2] = ld_frag(kp + (t * 4 + 2 * w + s2) * kBlk);
    };
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sacc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (from_init) {
        const float4 v4 = *reinterpret_cast<const float4*>(init + srow * D + 64 * w + 16 * mt + 4 * g4);
        sacc[mt] = floatx4{v4.x, v4.y, v4.z, v4.w};
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) split_pair(sacc[2 * s2], sacc[2 * s2 + 1], sh[s2], sl[s2]);
    load_k(0);
    for (int tick = 0; tick <= n + 1; ++tick) {
      const int p = tick & 1;
      if (tick >= 2) {
        // S_{tick-1} = bC S_{tick-2} + K_{tick-2}^T U2_{tick-2}
        const bf16x8 u2h0 = u2buf[(tick - 1) & 1][0][0][lane], u2l0 = u2buf[(tick - 1) & 1][0][1][lane];
        const bf16x8 u2h1 = u2buf[(tick - 1) & 1][1][0][lane], u2l1 = u2buf[(tick - 1) & 1][1][1][lane];
        const uint16_t* kt = ktile[w][p];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          floatx4 acc = sacc[mt] * bq0;
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            // lane (r, g): K[32 s + kap(g, e)][16 mt + r] as two transposing
            // reads of four tokens (lane r addresses row r / 4, columns
            // 4 (r % 4) .. + 3 of the 16-column block)
            const uint16_t* a = kt + (32 * s2 + 4 * g4 + (r16 >> 2)) * LDKT + 16 * mt + 4 * (r16 & 3);
            const uint2 lo4 = lds_tr16(a), hi4 = lds_tr16(a + 16 * LDKT);
            const bf16x8 kt8 = __builtin_bit_cast(bf16x8, make_uint4(lo4.x, lo4.y, hi4.x, hi4.y));
            acc = mma16(kt8, s2 ? u2h1 : u2h0, acc);
            acc = mma16(kt8, s2 ? u2l1 : u2l0, acc);
          }
          sacc[mt] = acc;
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) split_pair(sacc[2 * s2], sacc[2 * s2 + 1], sh[s2], sl[s2]);
      }
      if (tick - 1 == n) {
        // the state after the sequence's last token
        if (fin) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            *reinterpret_cast<float4*>(fin + srow * D + 64 * w + 16 * mt + 4 * g4) =
                make_float4(sacc[mt][0], sacc[mt][1], sacc[mt][2], sacc[mt][3]);
        }
      } else if (tick <= n) {
        if (tick >= 1) {
          // S_{tick-1} for the output of chunk tick - 1
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            sbuf[p][w][s2][0][lane] = sh[s2];
            sbuf[p][w][s2][1][lane] = sl[s2];
          }
        }
        if (tick < n) {
          // Z_tick partial = K_tick S^T over this half (tick 0: K_0 S_0^T = Y_0)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              z = mma16(kf[t][s2], sh[s2], z);
              z = mma16(kf[t][s2], sl[s2], z);
            }
            zbuf[p][w][t][lane] = z;
          }
          // K_tick rows of this half into the tile slot read two ticks later
          // (the reads of this tick's update above are issued first)
          uint16_t* kt = ktile[w][p];
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              const uint4 kv = __builtin_bit_cast(uint4, kf[t][s2]);
              uint16_t* dst = kt + (16 * t + r16) * LDKT + 32 * s2 + 4 * g4;
              *reinterpret_cast<uint2*>(dst) = make_uint2(kv.x, kv.y);
              *reinterpret_cast<uint2*>(dst + 16) = make_uint2(kv.z, kv.w);
            }
        }
      }
      load_k(next_c(tick < n ? tick : n - 1));
      bq0 = bq1;
      bq1 = tick < n ? sc_of(tick)[2 * C] : 1.f;
      __syncthreads();
    }
  } else {
    // ------------------------------------------------------------ output
    bf16x8 qf[4][4];                   // Q_c fragments (t, ks)
    bf16x8 rh[6], rl[6];               // R_c fragments
    float c2v[4];                      // c2 of tokens 16t + r
    auto load_q = [&](int c) {
      const uint16_t* qp = ws.qfr + ((slot0 + c) * h_qk + hq) * 16 * kBlk + lane * 8;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[t][ks] = ld_frag(qp + (t * 4 + ks) * kBlk);
      const float* sc = sc_of(c);
#pragma unroll
      for (int t = 0; t < 4; ++t) c2v[t] = sc[C + 16 * t + r16];
    };
    auto load_r = [&](int c) {
      const uint16_t* rp = ws.rfr + ((slot0 + c) * h_v + h) * 12 * kBlk + lane * 8;
#pragma unroll
      for (int b = 0; b < 6; ++b) {
        rh[b] = ld_frag(rp + (b * 2 + 0) * kBlk);
        rl[b] = ld_frag(rp + (b * 2 + 1) * kBlk);
      }
    };
    load_q(0);
    load_r(0);
    for (int tick = 0; tick <= n + 1; ++tick) {
      const int c = tick - 2;
      if (c >= 0 && c < n) {
        const int pp = (tick - 1) & 1;
        const int64_t t0 = start + static_cast<int64_t>(c) * C;
        const int len = static_cast<int>(end - t0 < C ? end - t0 : C);
        // O^T = S Q^T diag(c2) + X^T R^T: S and X as A operands (rows d_v)
        floatx4 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 sh = sbuf[pp][ks >> 1][ks & 1][0][lane], sl = sbuf[pp][ks >> 1][ks & 1][1][lane];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            acc[t] = mma16(sh, qf[t][ks], acc[t]);
            acc[t] = mma16(sl, qf[t][ks], acc[t]);
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = acc[t] * c2v[t];
        load_q(next_c(c));
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const bf16x8 xh = xbuf[pp][s2][0][lane], xl = xbuf[pp][s2][1][lane];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (s2 <= (t >> 1)) acc[t] = mma3(xh, xl, rh[tri_blk(t, s2)], rl[tri_blk(t, s2)], acc[t]);
        }
        load_r(next_c(c));
        // lane (r, g) holds O[token 16t + r][d_v dv0 + 4g .. 4g + 3]
        typename EO::T* ob = o + (t0 + r16) * (static_cast<int64_t>(h_v) * D) + static_cast<int64_t>(h) * D + dv0 + 4 * g4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (16 * t + r16 < len) {
            typename EO::T* dst = ob + static_cast<int64_t>(16 * t) * h_v * D;
            if constexpr (EO::kBytes == 4) {
              *reinterpret_cast<float4*>(dst) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
            } else {
              const uint32_t a = static_cast<uint32_t>(f32_to_bf16_bits(acc[t][0])) |
                                 (static_cast<uint32_t>(f32_to_bf16_bits(acc[t][1])) << 16);
              const uint32_t b = static_cast<uint32_t>(f32_to_bf16_bits(acc[t][2])) |
                                 (static_cast<uint32_t>(f32_to_bf16_bits(acc[t][3])) << 16);
              *reinterpret_cast<uint2*>(dst) = make_uint2(a, b);
            }
          }
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
hipError_t run_chunk_bf16(const ChunkArgs& a) {
  const int64_t slots = block_slots(a.t_total, a.n_seq, kC);
  Bf16Ws ws = carve(a.workspace, slots, a.h_qk, a.h_v, a.n_seq, a.t_total, a.z != nullptr);
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  if (slots > 0) {
    // persistent grid: as many workgroups as can be resident at once
    static const int per_cu = [] {
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_prep_bf16, 256, 0) != hipSuccess || nb < 1) nb = 1;
      return nb;
    }();
    const int64_t units = slots * a.h_qk;
    const int64_t resident = static_cast<int64_t>(per_cu) * device_cu_count();
    const int64_t grid = units < resident ? units : resident;
    hipLaunchKernelGGL(k_prep_bf16, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, q, k, a.q_stride,
                       a.k_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.cu, a.n_seq, a.t_total,
                       a.slots, ws, slots);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ws.order) {
    hipError_t e = launch_seq_order(a.cu, a.n_seq, kC, ws.order, st);
    if (e != hipSuccess) return e;
  }
  if (a.n_seq > 1 || a.t_total == 1 || a.slots != nullptr) {
    hipError_t e = launch_single_token(a, ws.o_pre);
    if (e != hipSuccess) return e;
  }
  const int64_t nblk = static_cast<int64_t>(a.n_seq) * a.h_v * (kD / 16);
  if (a.z) {
    hipLaunchKernelGGL(k_scan_bf16<F32>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st, v, a.v_stride,
                       a.h_qk, a.h_v, a.cu, a.n_seq, a.t_total, a.init, a.fin, a.slots, a.fresh, ws.o_pre, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.t_total > 0)
      return launch_gated_rmsnorm(ws.o_pre, GDN_F32, a.z, a.dt, a.norm_w, a.norm_eps, a.t_total * a.h_v, kD, a.o,
                                  a.o_dt, a.stream, a.slots ? a.cu : nullptr, a.n_seq, a.slots, a.h_v);
    return hipSuccess;
  }
  if (a.o_dt == GDN_BF16)
    hipLaunchKernelGGL(k_scan_bf16<BF16>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st, v, a.v_stride,
                       a.h_qk, a.h_v, a.cu, a.n_seq, a.t_total, a.init, a.fin, a.slots, a.fresh,
                       static_cast<uint16_t*>(a.o), ws);
  else
    hipLaunchKernelGGL(k_scan_bf16<F32>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st, v, a.v_stride,
                       a.h_qk, a.h_v, a.cu, a.n_seq, a.t_total, a.init, a.fin, a.slots, a.fresh,
                       static_cast<float*>(a.o), ws);
  return hipGetLastError();
}

}  // namespace gdn
