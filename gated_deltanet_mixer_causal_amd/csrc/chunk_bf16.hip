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
//     W  = Tb X,   Tb = T diag(beta)                               (the token writes)
//     U2 = diag(c3) W                                              (the writes, decayed to the chunk end)
//     O  = diag(c2) Q S^T + P W
//     S' = bC S + U2^T K
// Across chunks, with the raw inter-chunk Gram matrix G_{c+1} = K_{c+1} K_c^T,
//     Y_{c+1} = K_{c+1} S_{c+1}^T = bC_c (K_{c+1} S_c^T) + G_{c+1} U2_c,
// so the chain from one chunk's writes U2_c to the next chunk's error X_{c+1}
// needs the state S_c only through a product computed a step ahead.
//
// Kernels:
//   k_prep_bf16  persistent workgroups over (chunk slot, q/k head) units: the
//                Gram blocks K K^T, Q K^T and K_c K_{c-1}^T on the matrix cores
//                (raw bf16, exact products), then two v-heads at a time the
//                decays, L (to LDS) and P (to the workspace) straight from the
//                Gram registers, the triangular solve (diagonal blocks by
//                forward substitution, each off-diagonal block column by one
//                wave) and Tb.  Writes K, Q, G, Tb and P as fragments
//                (derived ones as bf16 hi + lo) and c1, c2, c3, bC.
//   k_scan_bf16  one workgroup of four waves per (sequence, v-head, 16-wide
//                d_v slice), walking the chunks in ticks:
//                  wave 0 (chain)  Y_c = bC Z_c + G_c U2_{c-1}, X_c, W_c = Tb_c X_c,
//                                  U2_c = diag(c3) W_c
//                  waves 1, 2 (state) one d_k half each of S in fp32:
//                                  S_{c} = bC S_{c-1} + U2_{c-1}^T K_{c-1},
//                                  Z_{c+1} = K_{c+1} S_c^T (partial over the half)
//                  wave 3 (output) O_c = diag(c2) Q_c S_c^T + P_c W_c
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
// operands; every derived operand (S, X, W, U2, G, Tb, P) is a bf16 hi + lo pair
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
constexpr int kScStride = 196;   // floats per (slot, v-head): c1[64] | c2[64] | c3[64] | bC | pad

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

// A value every lane loads from the same address, kept a vector load: with a
// uniform address the compiler would use a scalar load, whose completion the
// workgroup barrier waits for (it shares a counter with LDS), which would put
// the load's whole latency before the barrier.
__device__ __forceinline__ float bcast_load(const float* p) {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return p[z];
}

// Raw buffer loads (MUBUF): a per-lane 32-bit byte offset and a uniform one
// against a resource of base and size built from scalars, so a load costs no
// vector address arithmetic.  A load whose offset (both parts) reaches past
// the size returns zero without touching memory (checked on the device).
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrcFlags = 0x00020000;   // 32-bit raw data format
__device__ __forceinline__ Rsrc rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcFlags);
}
__device__ __forceinline__ bf16x8 bl_frag(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ float4 bl_f4(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ float bl_f32(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t bl_u16(Rsrc r, uint32_t voff, uint32_t soff) {
  return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
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
//   tfr [slots][h_v][6 blocks tri(t, s)][hi|lo] Tb fragments, same order
//   pfr [slots][h_v][6 blocks tri(t, s)][hi|lo] P fragments, same order
//   sc  [slots][h_v][196] fp32                c1[64] | c2[64] | c3[64] | bC
//   order [n_seq] int32                       sequences, most chunks first (n_seq > 1)
//   o   [t_total][h_v][128] fp32              outputs before the fused norm (with z)
struct Bf16Ws {
  uint16_t* kfr;
  uint16_t* qfr;
  uint16_t* gfr;
  uint16_t* tfr;
  uint16_t* pfr;
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
  w.pfr = reinterpret_cast<uint16_t*>(b); b += z.tfr;
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
// Gram blocks of a unit.  Fragment block b (0..5) of a 64 x 64 lower-
// triangular operand covers token tile t and k-step s (tri_blk order); it
// holds the 16 x 16 tiles (t, 2s) and (t, 2s + 1), the second one only when
// it is not above the diagonal.  Wave w forms the blocks of one kind (waves
// 0, 1: K K^T for L; waves 2, 3: Q K^T for P), three blocks each, five tiles.
__device__ __forceinline__ int prep_block(int w, int j) {
  return (w & 1) ? (j == 0 ? 4 : j == 1 ? 5 : 3) : (j == 0 ? 1 : j == 1 ? 2 : 0);
}
__device__ __forceinline__ void blk_ts(int b, int& t, int& s) {
  t = b < 2 ? b : 2 + ((b - 2) >> 1);
  s = b < 2 ? 0 : ((b - 2) & 1);
}

// One 16 x 16 x 16 product on the fp32 matrix cores.  A is a row-major block
// in LDS (row stride lda); b holds B in the output layout of an earlier
// product (lane (r, g): B[4g + i][r] in b[i]).  The k index of step s is
// 4 g + s in lane group g, so A comes as one 16-byte read of row r.
__device__ __forceinline__ floatx4 mm16_lds(const float* a_blk, int lda, floatx4 b, floatx4 acc, int r, int g) {
  const float4 a = *reinterpret_cast<const float4*>(a_blk + r * lda + 4 * g);
  acc = mma_f32(a.x, b[0], acc);
  acc = mma_f32(a.y, b[1], acc);
  acc = mma_f32(a.z, b[2], acc);
  return mma_f32(a.w, b[3], acc);
}

// A 16 x 16 block of LDS in the output layout (lane (r, g): rows 4g + i, column r).
__device__ __forceinline__ floatx4 ld_out(const float* blk, int ld, int r, int g) {
  return floatx4{blk[(4 * g + 0) * ld + r], blk[(4 * g + 1) * ld + r], blk[(4 * g + 2) * ld + r],
                 blk[(4 * g + 3) * ld + r]};
}
__device__ __forceinline__ void st_out(float* blk, int ld, floatx4 v, int r, int g) {
#pragma unroll
  for (int i = 0; i < 4; ++i) blk[(4 * g + i) * ld + r] = v[i];
}

__global__ __launch_bounds__(256, 2) void k_prep_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                      int64_t q_stride, int64_t k_stride, GateSrc gates, float scale,
                                                      int use_l2, float l2_eps, int h_qk, int h_v,
                                                      const int32_t* __restrict__ cu, int n_seq, int64_t t_total,
                                                      const int32_t* __restrict__ seq_slots, Bf16Ws ws,
                                                      int64_t n_slots) {
  constexpr int D = kD, C = kC;
  constexpr int LDK = D + 8;    // bf16 elements per K/Q row in LDS
  constexpr int LDC = C + 4;    // floats per L/T row
  constexpr int ROWS_BYTES = 3 * C * LDK * 2;
  constexpr int MAT_BYTES = 2 * 2 * C * LDC * 4;
  // K, Q and previous-chunk K rows during the Gram phase; then L and T of
  // the two v-heads in progress.
  __shared__ __attribute__((aligned(16))) char smem[ROWS_BYTES > MAT_BYTES ? ROWS_BYTES : MAT_BYTES];
  __shared__ __attribute__((aligned(16))) float s_rk[C];
  __shared__ __attribute__((aligned(16))) float s_rq[C];
  // the chunk's running sum of g, in fp64: with strong decays it reaches
  // hundreds, and the decay between two tokens is a difference of two sums
  __shared__ __attribute__((aligned(16))) double s_gam[2][C];
  __shared__ __attribute__((aligned(16))) float s_beta[2][C];
  // the sequence boundaries, staged once: every unit locates its sequence
  // from them, and a global read there would stall the unit's start
  constexpr int kCuLds = 256;
  __shared__ int32_t s_cu[kCuLds + 1];
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sQ = sK + C * LDK;
  uint16_t* sKp = sQ + C * LDK;
  auto sL = [&](int v) { return reinterpret_cast<float*>(smem) + v * 2 * C * LDC; };
  auto sT = [&](int v) { return reinterpret_cast<float*>(smem) + (v * 2 + 1) * C * LDC; };

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
  // Two workgroups share a compute unit: while one waits for its rows the
  // other computes, so a unit loads its own rows when it starts.
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
    const int tok_l = lane < len ? lane : len - 1;
    // gate inputs of the first pair of v-heads: waves 0 and 1 take one each
    // (waves 2 and 3 load the same, unused, so no load sits under a branch)
    uint32_t graw, braw;
    gate_load_raw(gates, t0 + tok_l, hq * grp + ((wave & 1) < grp ? (wave & 1) : 0), h_v, graw, braw);

    // 1. raw K, Q (zero past len) and previous-chunk K rows to LDS, and the
    //    L2 scales of K and Q
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
    __syncthreads();

    // 2. Gram blocks, transposed products (A = K rows of the column tile,
    //    B = K or Q rows of the row tile) so lane (r, g) ends with row
    //    16t + r, columns 16 tj + 4g + i: the k order of a fragment.  Raw
    //    operands, exact products, fp32 sums.
    const bool isq = wave >= 2;
    floatx4 gram[3][2];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      int t, s;
      blk_ts(prep_block(wave, j), t, s);
      const uint16_t* bp = (isq ? sQ : sK) + (16 * t + r16) * LDK + 8 * g4;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int tj = 2 * s + h2;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        if (tj <= t) {
          const uint16_t* ap = sK + (16 * tj + r16) * LDK + 8 * g4;
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) acc = mma16(ld_frag(ap + 32 * ks), ld_frag(bp + 32 * ks), acc);
        }
        gram[j][h2] = acc;
      }
    }
    //    G = K_c K_{c-1}^T the same way: wave w owns row tile w, and the
    //    column tiles (2s, 2s+1) form the fragment of k-step s.
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
    //    K and Q fragments: block (t, sf), lane (r, g): row 16t + r, columns
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

    for (int p0 = 0; p0 < grp; p0 += 2) {
      const int nv = grp - p0 < 2 ? grp - p0 : 2;   // v-heads in this pass
      // 3. decays of the pass's v-heads (wave v for v-head p0 + v): inclusive
      //    running sum of g over the chunk (padded tokens add 0), and c1, c2,
      //    c3, bC
      if (p0 > 0) gate_load_raw(gates, t0 + tok_l, hq * grp + p0 + ((wave & 1) < nv ? (wave & 1) : 0), h_v, graw, braw);
      {
        float gv, bv;
        gate_from_raw(gates, hq * grp + p0 + ((wave & 1) < nv ? (wave & 1) : 0), graw, braw, gv, bv);
        if (lane >= len) gv = bv = 0.f;
        if (wave < nv) {
          const int64_t unit = cslot * h_v + hq * grp + p0 + wave;
          double gam = gv;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const double o = __shfl_up(gam, off, 64);
            if (lane >= off) gam += o;
          }
          const double glast = __shfl(gam, C - 1, 64);
          float* sc = ws.sc + unit * kScStride;
          s_gam[wave][lane] = gam;
          s_beta[wave][lane] = bv;
          const float b = __expf(static_cast<float>(gam));
          const float rk = s_rk[lane];
          sc[lane] = b * rk;
          sc[C + lane] = scale * b * s_rq[lane];
          sc[2 * C + lane] = __expf(static_cast<float>(glast - gam)) * rk;
          if (lane == 0) sc[3 * C] = __expf(static_cast<float>(glast));
        }
      }
      __syncthreads();   // rows no longer read (L and T overlay them); decays visible

      // 4. L (strictly lower, to LDS) and P (lower with the diagonal, split
      //    fragments to the workspace) from the Gram blocks in registers.
      //    Each decay is masked to -inf above the diagonal before the
      //    exponential; the masks are selects.
      for (int v = 0; v < nv; ++v) {
        const int64_t unit = cslot * h_v + hq * grp + p0 + v;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int b = prep_block(wave, j);
          int t, s;
          blk_ts(b, t, s);
          const int row = 16 * t + r16, c0 = 32 * s + 4 * g4;
          const double gi = s_gam[v][row];
          const float ri = isq ? scale * s_rq[row] : s_beta[v][row] * s_rk[row];
          float val[2][4];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int cb = c0 + 16 * h2;
            const float4 rkj = *reinterpret_cast<const float4*>(s_rk + cb);
            const double2 ga = *reinterpret_cast<const double2*>(&s_gam[v][cb]);
            const double2 gb = *reinterpret_cast<const double2*>(&s_gam[v][cb + 2]);
            const double gj[4] = {ga.x, ga.y, gb.x, gb.y};
            const float rj[4] = {rkj.x, rkj.y, rkj.z, rkj.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int col = cb + e;
              const bool keep = isq ? col <= row : col < row;
              const float dec = __expf(keep ? static_cast<float>(gi - gj[e]) : -INFINITY);
              val[h2][e] = keep ? ri * dec * rj[e] * gram[j][h2][e] : 0.f;
            }
          }
          if (isq) {
            bf16x8 hi, lo;
            split_pair(floatx4{val[0][0], val[0][1], val[0][2], val[0][3]},
                       floatx4{val[1][0], val[1][1], val[1][2], val[1][3]}, hi, lo);
            uint16_t* pb = ws.pfr + unit * 12 * kBlk + lane * 8;
            st_frag(pb + (b * 2 + 0) * kBlk, hi);
            st_frag(pb + (b * 2 + 1) * kBlk, lo);
          } else {
            float* dst = sL(v) + row * LDC + c0;
            *reinterpret_cast<float4*>(dst) = make_float4(val[0][0], val[0][1], val[0][2], val[0][3]);
            if (2 * s + 1 <= t)
              *reinterpret_cast<float4*>(dst + 16) = make_float4(val[1][0], val[1][1], val[1][2], val[1][3]);
          }
        }
      }
      __syncthreads();

      // 5. T = (I + L)^-1, diagonal 16 x 16 blocks: wave w serves v-head
      //    w / 2, blocks 2 (w % 2) and 2 (w % 2) + 1; lane 16 b' + c owns
      //    column c and runs forward substitution T_i = e_i - sum_{j<i} L_ij T_j
      //    (rows of L read 16 bytes at a time, the same address across the
      //    block's lanes).
      if ((wave >> 1) < nv && lane < 32) {
        const int v = wave >> 1;
        const int base = 16 * (2 * (wave & 1) + (lane >> 4)), c = lane & 15;
        const float* lb = sL(v) + base * LDC + base;
        float tcol[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
          for (int j4 = 0; j4 < i; j4 += 4) {
            const float4 l4 = *reinterpret_cast<const float4*>(lb + i * LDC + j4);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (j4 + e < i) acc = __builtin_fmaf(-lv[e], tcol[j4 + e], acc);
          }
          tcol[i] = acc;
        }
        float* tb = sT(v) + base * LDC + base;
#pragma unroll
        for (int i = 0; i < 16; ++i) tb[i * LDC + c] = tcol[i];
      }
      __syncthreads();

      // 6. Off-diagonal blocks, one block column at a time by one wave (no
      //    workgroup barrier: a column needs only its own blocks and the
      //    diagonal ones):  T_ij = -T_ii sum_{k=j}^{i-1} L_ik T_kj.
      //    Wave 2v + 0 forms column 0 of v-head v; wave 2v + 1 columns 1, 2.
      if ((wave >> 1) < nv) {
        const int v = wave >> 1;
        const float* L = sL(v);
        float* T = sT(v);
        auto lblk = [&](int i, int kb) { return L + 16 * i * LDC + 16 * kb; };
        auto tblk = [&](int i, int j) { return T + 16 * i * LDC + 16 * j; };
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
        if ((wave & 1) == 0) {
          const floatx4 d0 = ld_out(tblk(0, 0), LDC, r16, g4);
          floatx4 w = mm16_lds(lblk(1, 0), LDC, d0, zero, r16, g4);
          const floatx4 t10 = -mm16_lds(tblk(1, 1), LDC, w, zero, r16, g4);
          w = mm16_lds(lblk(2, 0), LDC, d0, zero, r16, g4);
          w = mm16_lds(lblk(2, 1), LDC, t10, w, r16, g4);
          const floatx4 t20 = -mm16_lds(tblk(2, 2), LDC, w, zero, r16, g4);
          w = mm16_lds(lblk(3, 0), LDC, d0, zero, r16, g4);
          w = mm16_lds(lblk(3, 1), LDC, t10, w, r16, g4);
          w = mm16_lds(lblk(3, 2), LDC, t20, w, r16, g4);
          const floatx4 t30 = -mm16_lds(tblk(3, 3), LDC, w, zero, r16, g4);
          st_out(tblk(1, 0), LDC, t10, r16, g4);
          st_out(tblk(2, 0), LDC, t20, r16, g4);
          st_out(tblk(3, 0), LDC, t30, r16, g4);
        } else {
          const floatx4 d1 = ld_out(tblk(1, 1), LDC, r16, g4);
          const floatx4 d2 = ld_out(tblk(2, 2), LDC, r16, g4);
          floatx4 w = mm16_lds(lblk(2, 1), LDC, d1, zero, r16, g4);
          const floatx4 t21 = -mm16_lds(tblk(2, 2), LDC, w, zero, r16, g4);
          w = mm16_lds(lblk(3, 2), LDC, d2, zero, r16, g4);
          const floatx4 t32 = -mm16_lds(tblk(3, 3), LDC, w, zero, r16, g4);
          w = mm16_lds(lblk(3, 1), LDC, d1, zero, r16, g4);
          w = mm16_lds(lblk(3, 2), LDC, t21, w, r16, g4);
          const floatx4 t31 = -mm16_lds(tblk(3, 3), LDC, w, zero, r16, g4);
          st_out(tblk(2, 1), LDC, t21, r16, g4);
          st_out(tblk(3, 2), LDC, t32, r16, g4);
          st_out(tblk(3, 1), LDC, t31, r16, g4);
        }
      }
      __syncthreads();

      // 7. Tb = T diag(beta) (zero above the diagonal) as split fragments:
      //    block (t, s), lane (r, g): row 16t + r, columns 32 s + kap(g, e)
      for (int f = tid; f < nv * 6 * 64; f += 256) {
        const int v = f / 384, rem = f - 384 * v;
        const int b = rem >> 6, l = rem & 63;
        int t, s;
        blk_ts(b, t, s);
        const int r = l & 15, g = l >> 4, row = 16 * t + r, c0 = 32 * s + 4 * g;
        const float* tr = sT(v) + row * LDC;
        float val[8];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int cb = c0 + 16 * h2;
          const float4 t4 = *reinterpret_cast<const float4*>(tr + cb);
          const float4 b4 = *reinterpret_cast<const float4*>(&s_beta[v][cb]);
          val[4 * h2 + 0] = cb + 0 <= row ? t4.x * b4.x : 0.f;   // T above the diagonal is not written
          val[4 * h2 + 1] = cb + 1 <= row ? t4.y * b4.y : 0.f;
          val[4 * h2 + 2] = cb + 2 <= row ? t4.z * b4.z : 0.f;
          val[4 * h2 + 3] = cb + 3 <= row ? t4.w * b4.w : 0.f;
        }
        bf16x8 hi, lo;
        split8(val, hi, lo);
        uint16_t* tb = ws.tfr + (cslot * h_v + hq * grp + p0 + v) * 12 * kBlk + l * 8;
        st_frag(tb + (b * 2 + 0) * kBlk, hi);
        st_frag(tb + (b * 2 + 1) * kBlk, lo);
      }
      __syncthreads();   // L, T and the decays are rewritten by the next pass or unit
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
  __shared__ floatx4 wbuf[2][4][64];             // W = Tb X: [p][token tile][lane]
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
    bf16x8 th[6], tl[6];           // Tb_c fragments
    uint32_t vr[4][4];             // V of rows 16t + 4g + i, column dv0 + r (raw bf16 bits)
    float4 c1v[4], c3v[4];         // c1, c3 of those rows (c3 loads with Tb: it is used after V's reload)
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
      const float* sc = sc_of(c);
#pragma unroll
      for (int t = 0; t < 4; ++t) c3v[t] = *reinterpret_cast<const float4*>(sc + 2 * C + 16 * t + 4 * g4);
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
        const float bc_now = bcast_load(sc_of(c) + 3 * C);   // first of this tick's loads: used next tick
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
        for (int s2 = 0; s2 < 2; ++s2) split_pair(x[2 * s2], x[2 * s2 + 1], xh[s2], xl[s2]);
        // W = Tb X (lower-triangular blocks), to the output wave in fp32;
        // U2 = diag(c3) W
        floatx4 u[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) u[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (s2 <= (t >> 1)) u[t] = mma3(th[tri_blk(t, s2)], tl[tri_blk(t, s2)], xh[s2], xl[s2], u[t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          wbuf[p][t][lane] = u[t];
          u[t] = u[t] * floatx4{c3v[t].x, c3v[t].y, c3v[t].z, c3v[t].w};
        }
        load_t(next_c(c));
        bcp = bc_now;
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
    const uint32_t lo16 = lane * 16;
    auto load_k = [&](int c) {
      const Rsrc r = rsrc(ws.kfr + ((slot0 + c) * h_qk + hq) * 16 * kBlk, 16 * kBlk * 2);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) kf[t][s2] = bl_frag(r, lo16, (t * 4 + 2 * w + s2) * kBlk * 2);
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
      const float bc_tick = bcast_load(sc_of(tick < n ? tick : n - 1) + 3 * C);
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
      bq1 = tick < n ? bc_tick : 1.f;
      __syncthreads();
    }
  } else {
    // ------------------------------------------------------------ output
    bf16x8 qf[4][4];                   // Q_c fragments (t, ks)
    bf16x8 ph[6], pl[6];               // P_c fragments
    float c2v[4];                      // c2 of tokens 16t + r
    const uint32_t lo16 = lane * 16;
    auto load_q = [&](int c) {
      const Rsrc r = rsrc(ws.qfr + ((slot0 + c) * h_qk + hq) * 16 * kBlk, 16 * kBlk * 2);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[t][ks] = bl_frag(r, lo16, (t * 4 + ks) * kBlk * 2);
      const Rsrc rs = rsrc(sc_of(c), kScStride * 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) c2v[t] = bl_f32(rs, 4 * r16, (C + 16 * t) * 4);
    };
    auto load_p = [&](int c) {
      const Rsrc r = rsrc(ws.pfr + ((slot0 + c) * h_v + h) * 12 * kBlk, 12 * kBlk * 2);
#pragma unroll
      for (int b = 0; b < 6; ++b) {
        ph[b] = bl_frag(r, lo16, (b * 2 + 0) * kBlk * 2);
        pl[b] = bl_frag(r, lo16, (b * 2 + 1) * kBlk * 2);
      }
    };
    load_q(0);
    load_p(0);
    for (int tick = 0; tick <= n + 1; ++tick) {
      const int c = tick - 2;
      if (c >= 0 && c < n) {
        const int pp = (tick - 1) & 1;
        const int64_t t0 = start + static_cast<int64_t>(c) * C;
        const int len = static_cast<int>(end - t0 < C ? end - t0 : C);
        // O^T = S Q^T diag(c2) + W^T P^T: S and W as A operands (rows d_v)
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
          bf16x8 wh, wl;
          split_pair(wbuf[pp][2 * s2][lane], wbuf[pp][2 * s2 + 1][lane], wh, wl);
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (s2 <= (t >> 1)) acc[t] = mma3(wh, wl, ph[tri_blk(t, s2)], pl[tri_blk(t, s2)], acc[t]);
        }
        load_p(next_c(c));
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
