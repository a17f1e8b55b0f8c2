// Backward of the gated delta rule (gfx950), from chunk-boundary states.
//
// Forward, per sequence and v-head with fp32 state S (d_v x d_k) and each
// token t (k^, q^ the L2-normalised keys and queries):
//     S' = a S,  e = v - S' k^,  S_t = S' + beta e k^^T,  o_t = scale S_t q^
// (the gated delta rule of the GDN layers: haskell-infer-demo README,
// "Highlights" and "Architecture"/fla_gdn.cu).  With G = dL/dS_t the reverse
// step is, token by token from the last:
//     G   += scale do_t q^^T                 dq^_t = scale S_t^T do_t
//     u    = G k^                            dv_t  = beta u,  dbeta_t = e . u
//     dk^_t = beta (G^T e - S'^T u)
//     dS'  = G - beta u k^^T                 dg_t  = <dS', S'>
//     G    = a dS'                           (dL/dS_{t-1})
// and dL/dS_0 is the G left after the first token.  Each row of S evolves
// on its own, so the state is split into 16-row slices; dq^, dk^, dbeta and dg
// are sums over all rows, formed per slice and added up by a final kernel,
// which also takes dq^, dk^ back through the L2 normalisation.
//
// Kernels:
//   k_bwd_ckpt    forward over each sequence, writing the state entering
//                 every 16-token block (per slice) to the workspace.
//   k_bwd_slice   per (sequence, v-head, 16-row slice), blocks last to
//                 first, and inside a block its second 8 tokens, then its
//                 first 8: recompute from the block's checkpoint through the
//                 half, keeping the state before each of its tokens in LDS,
//                 then run the reverse step over them.  The sums over the
//                 slice's rows (partial dq^, dk^, dbeta, dg) are left per half wave
//                 in LDS and finished once per half, so the reverse chain
//                 waits at no barrier between tokens.  A block's inputs
//                 (normalised k, q; v, do of the slice; a, beta) are staged in
//                 LDS first; both kernels load the next block's inputs into
//                 registers while the current block runs.
//   k_bwd_reduce  per (token, q/k head): sums the slice partials over the
//                 slices and the v-heads that read this q/k head, applies the
//                 L2-norm backward dx = (dx^ - x^ (x^ . dx^)) / |x|_eps, and
//                 sums dbeta, dg over slices.
// All sums run in a fixed order: reruns are bitwise identical.
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

constexpr int kBwdRows = 16;    // state rows per workgroup
constexpr int kBwdSub = 16;     // tokens per staged sub-block
constexpr int kBwdChunk = 16;   // tokens between checkpoints (one sub-block: no recompute beyond it)

// Sum over groups of W consecutive lanes (W = 2, 4, 8, 16) with DPP lane moves
// inside each 16-lane row instead of LDS-crossbar shuffles: quad permutations
// for lane distances 1 and 2, then the half-row mirror (lane i of each 8 reads
// lane 7 - i, the other quad) and the row mirror (lane i reads 15 - i, the
// other half).  Every lane ends with the group's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Two row-pair sums in one instruction, without the LDS crossbar: gfx950's
// v_permlane16_swap trades the odd 16-lane rows of its first operand with the
// even rows of its second (lane layout checked on the device).  Given x and y
// it leaves x0 | y0 | x2 | y2 in one result and x1 | y1 | x3 | y3 in the other
// (rows of 16 lanes), so their sum holds x0 + x1 in row 0, y0 + y1 in row 1,
// x2 + x3 in row 2 and y2 + y3 in row 3.
__device__ __forceinline__ float pair_sums16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int W>
__device__ __forceinline__ float row_sum(float v) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16, "groups inside one DPP row");
  v += dpp_move<0xB1>(v);                       // quad_perm [1,0,3,2]
  if constexpr (W >= 4) v += dpp_move<0x4E>(v); // quad_perm [2,3,0,1]
  if constexpr (W >= 8) v += dpp_move<0x141>(v);  // row_half_mirror
  if constexpr (W >= 16) v += dpp_move<0x140>(v); // row_mirror
  return v;
}

// Workspace carve-up (floats):
//   ckpt [slots][h_v][D][D]          state entering each kBwdChunk-token block
//   pdq, pdk [T][h_v][D/16][D]       slice partials of dq^, dk^
//   pdb, pdg [T][h_v][D/16]          slice partials of dbeta, dg
struct BwdWs {
  float* ckpt;
  float* pdq;
  float* pdk;
  float* pdb;
  float* pdg;
};

static size_t bwd_al(size_t x) { return (x + 255) & ~size_t(255); }

size_t bwd_ws_bytes(int h_v, int d, int n_seq, int64_t t_total) {
  const int64_t slots = block_slots(t_total, n_seq, kBwdChunk);
  const int tiles = d / kBwdRows;
  const size_t b = bwd_al(sizeof(float) * slots * h_v * d * d) + 2 * bwd_al(sizeof(float) * t_total * h_v * tiles * d) +
                   2 * bwd_al(sizeof(float) * t_total * h_v * tiles);
  // bf16, d = 128 runs the chunked path (chunk_bwd.hip); h_qk <= h_v bounds its q/k regions
  const size_t c = d == 128 ? bwd_chunked_ws_bytes(h_v, h_v, n_seq, t_total) : 0;
  return b > c ? b : c;
}

static BwdWs bwd_carve(void* base, int h_v, int d, int n_seq, int64_t t_total) {
  const int64_t slots = block_slots(t_total, n_seq, kBwdChunk);
  const int tiles = d / kBwdRows;
  char* b = static_cast<char*>(base);
  BwdWs w;
  w.ckpt = reinterpret_cast<float*>(b);
  b += bwd_al(sizeof(float) * slots * h_v * d * d);
  w.pdq = reinterpret_cast<float*>(b);
  b += bwd_al(sizeof(float) * t_total * h_v * tiles * d);
  w.pdk = reinterpret_cast<float*>(b);
  b += bwd_al(sizeof(float) * t_total * h_v * tiles * d);
  w.pdb = reinterpret_cast<float*>(b);
  b += bwd_al(sizeof(float) * t_total * h_v * tiles);
  w.pdg = reinterpret_cast<float*>(b);
  return w;
}

// Inputs of one sub-block, staged in LDS.
template <int D>
struct BwdStage {
  float k[kBwdSub][D];          // normalised keys
  float q[kBwdSub][D];          // normalised queries
  float v[kBwdSub][kBwdRows];   // v of the slice's rows
  float dov[kBwdSub][kBwdRows]; // do of the slice's rows
  float a[kBwdSub];             // exp(g)
  float b[kBwdSub];             // beta
};

// Staging of tokens t0 .. t0 + n - 1 (n <= kBwdSub; rows past n repeat row
// t0) in two parts, so that a block's global loads are in flight while the
// previous block is computed: stage_fetch reads this thread's raw inputs into
// registers, stage_put normalises k and q and writes the LDS block.  Thread
// layout of k, q: token tid / TPR, columns 4l .. 4l+3 and D/2 + 4l .. of it
// (l = tid % TPR), the same layout as the state rows, so the norms are
// TPR-lane sums.
template <class In, int D, int NT>
struct StageRegs {
  static constexpr int kPer = (kBwdSub * kBwdRows + NT - 1) / NT;   // v, do entries per thread
  float kk[8], qq[8], vv[kPer], dd[kPer], gv, bt;
};

template <class In, int D, int NT>
__device__ __forceinline__ void stage_fetch(StageRegs<In, D, NT>& R, const typename In::T* __restrict__ q,
                                            const typename In::T* __restrict__ k,
                                            const typename In::T* __restrict__ v, const float* __restrict__ dout,
                                            int64_t q_stride, int64_t k_stride, int64_t v_stride,
                                            const GateSrc& gates, int h_v, int h, int hq, int dv0, int64_t t0, int n,
                                            bool with_q) {
  constexpr int TPR = D / 8;
  const int tid = threadIdx.x;
  const int j = tid / TPR, l = tid % TPR;
  const int ca = 4 * l, cb = D / 2 + 4 * l;
  if (j < kBwdSub) {
    const int64_t t = t0 + (j < n ? j : 0);
    const typename In::T* kr = k + t * k_stride + static_cast<int64_t>(hq) * D;
    const typename In::T* qr = q + t * q_stride + static_cast<int64_t>(hq) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      R.kk[i] = In::load(kr, ca + i);
      R.kk[4 + i] = In::load(kr, cb + i);
      R.qq[i] = with_q ? In::load(qr, ca + i) : 0.f;
      R.qq[4 + i] = with_q ? In::load(qr, cb + i) : 0.f;
    }
  }
#pragma unroll
  for (int u = 0; u < R.kPer; ++u) {
    const int e = tid + u * NT;
    if (e < kBwdSub * kBwdRows) {
      const int jj = e / kBwdRows, r = e % kBwdRows;
      const int64_t t = t0 + (jj < n ? jj : 0);
      R.vv[u] = In::load(v + t * v_stride + static_cast<int64_t>(h) * D, dv0 + r);
      R.dd[u] = dout ? dout[(t * h_v + h) * static_cast<int64_t>(D) + dv0 + r] : 0.f;
    }
  }
  if (tid < kBwdSub) load_gate(gates, t0 + (tid < n ? tid : 0), h, h_v, R.gv, R.bt);
}

template <class In, int D, int NT>
__device__ __forceinline__ void stage_put(BwdStage<D>& sm, const StageRegs<In, D, NT>& R, int use_l2,
                                          float l2_eps) {
  constexpr int TPR = D / 8;
  const int tid = threadIdx.x;
  const int j = tid / TPR, l = tid % TPR;
  const int ca = 4 * l, cb = D / 2 + 4 * l;
  if (j < kBwdSub) {
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) { sk += R.kk[i] * R.kk[i]; sq += R.qq[i] * R.qq[i]; }
    sk = row_sum<TPR>(sk);
    sq = row_sum<TPR>(sq);
    const float rk = use_l2 ? 1.0f / sqrtf(sk + l2_eps) : 1.0f;
    const float rq = use_l2 ? 1.0f / sqrtf(sq + l2_eps) : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sm.k[j][ca + i] = R.kk[i] * rk;
      sm.k[j][cb + i] = R.kk[4 + i] * rk;
      sm.q[j][ca + i] = R.qq[i] * rq;
      sm.q[j][cb + i] = R.qq[4 + i] * rq;
    }
  }
#pragma unroll
  for (int u = 0; u < R.kPer; ++u) {
    const int e = tid + u * NT;
    if (e < kBwdSub * kBwdRows) {
      sm.v[e / kBwdRows][e % kBwdRows] = R.vv[u];
      sm.dov[e / kBwdRows][e % kBwdRows] = R.dd[u];
    }
  }
  if (tid < kBwdSub) {
    sm.a[tid] = __expf(R.gv);
    sm.b[tid] = R.bt;
  }
}

// One forward token on this thread's 8 state values (row r): S <- a S + beta e k^,
// e = v_r - a (S . k^).
template <int D>
__device__ __forceinline__ void bwd_fwd_token(float (&s)[8], const BwdStage<D>& sm, int j, int r, int ca, int cb) {
  constexpr int TPR = D / 8;
  float kk[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) { kk[i] = sm.k[j][ca + i]; kk[4 + i] = sm.k[j][cb + i]; }
  float dk = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) dk += s[i] * kk[i];
  dk = row_sum<TPR>(dk);
  const float a = sm.a[j];
  const float be = sm.b[j] * (sm.v[j][r < kBwdRows ? r : 0] - a * dk);
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = a * s[i] + be * kk[i];
}

template <class In, int D, int NT>
__global__ __launch_bounds__(NT) void k_bwd_ckpt(
    const typename In::T* __restrict__ q, const typename In::T* __restrict__ k, const typename In::T* __restrict__ v,
    int64_t q_stride, int64_t k_stride, int64_t v_stride, GateSrc gates, int use_l2, float l2_eps, int h_qk,
    int h_v, const int32_t* __restrict__ cu, int n_seq, int64_t t_total, const float* __restrict__ init, BwdWs ws) {
  constexpr int TPR = D / 8, TILES = D / kBwdRows;
  static_assert(NT >= kBwdRows * TPR && NT % 64 == 0, "one thread per (row, lane)");
  __shared__ BwdStage<D> sm;
  const int64_t b = blockIdx.x;
  const int s = static_cast<int>(b / (static_cast<int64_t>(h_v) * TILES));
  const int h = static_cast<int>((b / TILES) % h_v), tile = static_cast<int>(b % TILES);
  if (s >= n_seq) return;
  const int hq = h / (h_v / h_qk), dv0 = tile * kBwdRows;
  const int tid = threadIdx.x, r = tid / TPR, l = tid % TPR;
  const int ca = 4 * l, cb = D / 2 + 4 * l;
  const bool row_ok = NT == kBwdRows * TPR || r < kBwdRows;
  const int64_t start = seq_start(cu, s, t_total), end = seq_start(cu, s + 1, t_total);
  const int64_t srow = (static_cast<int64_t>(s) * h_v + h) * D * D + static_cast<int64_t>(dv0 + (row_ok ? r : 0)) * D;
  float st[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (init && row_ok) {
    const float4 x = *reinterpret_cast<const float4*>(init + srow + ca);
    const float4 y = *reinterpret_cast<const float4*>(init + srow + cb);
    st[0] = x.x; st[1] = x.y; st[2] = x.z; st[3] = x.w; st[4] = y.x; st[5] = y.y; st[6] = y.z; st[7] = y.w;
  }
  static_assert(kBwdChunk == kBwdSub, "one staged block per checkpoint");
  const int64_t slot0 = start / kBwdChunk + s;
  // block c + 1's inputs are fetched into registers while block c is computed
  StageRegs<In, D, NT> nx;
  auto fetch = [&](int64_t c0) {
    const int n = static_cast<int>(end - c0 < kBwdSub ? end - c0 : kBwdSub);
    stage_fetch<In, D, NT>(nx, q, k, v, nullptr, q_stride, k_stride, v_stride, gates, h_v, h, hq, dv0, c0, n,
                           false);
  };
  if (start < end) fetch(start);
  for (int64_t c0 = start; c0 < end; c0 += kBwdChunk) {
    const int64_t slot = slot0 + (c0 - start) / kBwdChunk;
    if (row_ok) {
      float* dst = ws.ckpt + (slot * h_v + h) * static_cast<int64_t>(D) * D + static_cast<int64_t>(dv0 + r) * D;
      *reinterpret_cast<float4*>(dst + ca) = make_float4(st[0], st[1], st[2], st[3]);
      *reinterpret_cast<float4*>(dst + cb) = make_float4(st[4], st[5], st[6], st[7]);
    }
    const int n = static_cast<int>(end - c0 < kBwdSub ? end - c0 : kBwdSub);
    stage_put<In, D, NT>(sm, nx, use_l2, l2_eps);
    __syncthreads();
    if (c0 + kBwdChunk < end) fetch(c0 + kBwdChunk);
    if (n == kBwdSub) {
#pragma unroll
      for (int j = 0; j < kBwdSub; ++j) bwd_fwd_token<D>(st, sm, j, r, ca, cb);
    } else {
      for (int j = 0; j < n; ++j) bwd_fwd_token<D>(st, sm, j, r, ca, cb);
    }
    __syncthreads();
  }
}

template <class In, int D, int NT>
__global__ __launch_bounds__(NT) void k_bwd_slice(
    const typename In::T* __restrict__ q, const typename In::T* __restrict__ k, const typename In::T* __restrict__ v,
    int64_t q_stride, int64_t k_stride, int64_t v_stride, GateSrc gates, float scale, int use_l2, float l2_eps,
    int h_qk, int h_v, const int32_t* __restrict__ cu, int n_seq, int64_t t_total, const float* __restrict__ dout,
    const float* __restrict__ dfin, float* __restrict__ dv_out, float* __restrict__ dinit, BwdWs ws) {
  constexpr int TPR = D / 8, TILES = D / kBwdRows;
  constexpr int NW = NT / 64;
  constexpr int HALF = kBwdSub / 2;   // tokens whose states are stashed at once
  static_assert(kBwdChunk == kBwdSub, "one staged block per checkpoint");
  static_assert(NT >= kBwdRows * TPR && NT % 64 == 0, "one thread per (row, lane)");
  __shared__ BwdStage<D> sm;
  __shared__ float stash[HALF][kBwdRows][D];   // state before each token of the half block
  // column sums of each token of the half, two per wave (its 16-lane rows
  // 0 + 1 and 2 + 3)
  __shared__ float red_q[HALF][2 * NW][D];
  __shared__ float red_k[HALF][2 * NW][D];
  __shared__ float red_s[HALF][2 * NW][2];
  const int64_t b = blockIdx.x;
  const int s = static_cast<int>(b / (static_cast<int64_t>(h_v) * TILES));
  const int h = static_cast<int>((b / TILES) % h_v), tile = static_cast<int>(b % TILES);
  if (s >= n_seq) return;
  const int hq = h / (h_v / h_qk), dv0 = tile * kBwdRows;
  const int tid = threadIdx.x, r = tid / TPR, l = tid % TPR;
  const int ca = 4 * l, cb = D / 2 + 4 * l;
  const bool row_ok = NT == kBwdRows * TPR || r < kBwdRows;
  const int rr = row_ok ? r : 0;
  const int wv = tid >> 6, ln = tid & 63;
  const int64_t start = seq_start(cu, s, t_total), end = seq_start(cu, s + 1, t_total);
  const int64_t smat = (static_cast<int64_t>(s) * h_v + h) * D * D + static_cast<int64_t>(dv0 + rr) * D;

  float gs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // G, this thread's 8 values of row r
  if (dfin && row_ok) {
    const float4 x = *reinterpret_cast<const float4*>(dfin + smat + ca);
    const float4 y = *reinterpret_cast<const float4*>(dfin + smat + cb);
    gs[0] = x.x; gs[1] = x.y; gs[2] = x.z; gs[3] = x.w; gs[4] = y.x; gs[5] = y.y; gs[6] = y.z; gs[7] = y.w;
  }
  const int64_t slot0 = start / kBwdChunk + s;
  const int64_t nblk = (end - start + kBwdChunk - 1) / kBwdChunk;
  // block c - 1's inputs are fetched into registers while block c is computed
  StageRegs<In, D, NT> nx;
  auto fetch = [&](int64_t c) {
    const int64_t c0 = start + c * kBwdChunk;
    const int n = static_cast<int>(end - c0 < kBwdChunk ? end - c0 : kBwdChunk);
    stage_fetch<In, D, NT>(nx, q, k, v, dout, q_stride, k_stride, v_stride, gates, h_v, h, hq, dv0, c0, n, true);
  };
  if (nblk > 0) fetch(nblk - 1);
  for (int64_t c = nblk - 1; c >= 0; --c) {
    const int64_t c0 = start + c * kBwdChunk;
    const int n = static_cast<int>(end - c0 < kBwdChunk ? end - c0 : kBwdChunk);
    const float* ck = ws.ckpt + ((slot0 + c) * h_v + h) * static_cast<int64_t>(D) * D + static_cast<int64_t>(dv0 + rr) * D;
    stage_put<In, D, NT>(sm, nx, use_l2, l2_eps);
    __syncthreads();
    if (c > 0) fetch(c - 1);
    // the block's second half first, then its first half
    // The second half's pass computes the states before tokens 0 .. HALF-1 on
    // its way from the checkpoint; they are kept in registers for the first
    // half, which then needs no recompute.
    float early[HALF][8];
    bool have_early = false;
    for (int hf = (n > HALF ? 1 : 0); hf >= 0; --hf) {
      const int j0 = hf * HALF;
      const int nh = (n - j0 < HALF ? n - j0 : HALF);
      auto put_stash = [&](int j, const float (&v8)[8]) {
        if (row_ok) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            stash[j][r][ca + i] = v8[i];
            stash[j][r][cb + i] = v8[4 + i];
          }
        }
      };
      if (have_early) {
        // first half of a block whose second half ran: nh == HALF
#pragma unroll
        for (int j = 0; j < HALF; ++j) put_stash(j, early[j]);
      } else {
        // states: from the block's checkpoint through the half, keeping the
        // state before each of its tokens
        float st[8];
        {
          const float4 x = *reinterpret_cast<const float4*>(ck + ca);
          const float4 y = *reinterpret_cast<const float4*>(ck + cb);
          st[0] = x.x; st[1] = x.y; st[2] = x.z; st[3] = x.w; st[4] = y.x; st[5] = y.y; st[6] = y.z; st[7] = y.w;
        }
        // (j0 is 0 or HALF; full halves run unrolled, without per-token branches)
        if (j0 == HALF) {
#pragma unroll
          for (int j = 0; j < HALF; ++j) {
#pragma unroll
            for (int i = 0; i < 8; ++i) early[j][i] = st[i];
            bwd_fwd_token<D>(st, sm, j, r, ca, cb);
          }
          have_early = true;
        }
        if (nh == HALF) {
#pragma unroll
          for (int j = 0; j < HALF; ++j) {
            put_stash(j, st);
            if (j + 1 < HALF) bwd_fwd_token<D>(st, sm, j0 + j, r, ca, cb);
          }
        } else {
          for (int j = 0; j < nh; ++j) {
            put_stash(j, st);
            if (j + 1 < nh) bwd_fwd_token<D>(st, sm, j0 + j, r, ca, cb);
          }
        }
      }
      __syncthreads();   // the stash is complete
      // reverse over the half's tokens; the sums over the slice's rows are left
      // per wave in LDS and finished once for the whole half
      // (a full half runs unrolled without per-token branches, so one token's
      // partial sums and stores can overlap the next token's dependent chain)
      auto rev = [&](int j) {
        const int jt = j0 + j;   // token within the block
        const int64_t t = c0 + jt;
        float kk[8], qq[8], sp[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kk[i] = sm.k[jt][ca + i]; kk[4 + i] = sm.k[jt][cb + i];
          qq[i] = sm.q[jt][ca + i]; qq[4 + i] = sm.q[jt][cb + i];
          sp[i] = stash[j][rr][ca + i]; sp[4 + i] = stash[j][rr][cb + i];
        }
        const float a = sm.a[jt], bt = sm.b[jt];
        const float vr = sm.v[jt][rr], dor = sm.dov[jt][rr];
        float dk = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) { sp[i] *= a; dk += sp[i] * kk[i]; }   // sp: S' = a S_{t-1}
        dk = row_sum<TPR>(dk);
        const float e = vr - dk;
        float pq[8], pk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          gs[i] += scale * dor * qq[i];
          pq[i] = scale * dor * (sp[i] + bt * e * kk[i]);   // scale do_r S_t[r, :]
        }
        float u = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) u += gs[i] * kk[i];
        u = row_sum<TPR>(u);
        float pg = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pk[i] = bt * (gs[i] * e - sp[i] * u);
          const float ds = gs[i] - bt * u * kk[i];
          pg += ds * sp[i];
          gs[i] = a * ds;
        }
        pg = row_sum<TPR>(pg);
        if (row_ok && l == 0) dv_out[(t * h_v + h) * static_cast<int64_t>(D) + dv0 + r] = bt * u;
        // sums over the rows of each half wave (lane bits TPR .. 4; the row
        // scalars are replicated over the row's lanes)
        float sbu = row_ok ? e * u : 0.f, sgg = row_ok ? pg : 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (!row_ok) pq[i] = pk[i] = 0.f;
        }
#pragma unroll
        for (int off = TPR; off < 16; off <<= 1) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            pq[i] += __shfl_xor(pq[i], off);
            pk[i] += __shfl_xor(pk[i], off);
          }
          sbu += __shfl_xor(sbu, off);
          sgg += __shfl_xor(sgg, off);
        }
        // rows 0 and 2 of 16 lanes now hold the q partials of the wave's two
        // halves, rows 1 and 3 the k partials; the halves are summed with the
        // other waves' partials
        float ps[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ps[i] = pair_sums16(pq[i], pk[i]);
        const float ps2 = pair_sums16(sbu, sgg);
        if ((ln & 15) < TPR) {
          const int pw = 2 * wv + (ln >> 5), odd = (ln >> 4) & 1;
          float* dst = odd ? red_k[j][pw] : red_q[j][pw];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dst[ca + i] = ps[i];
            dst[cb + i] = ps[4 + i];
          }
          if ((ln & 15) == 0) red_s[j][pw][odd] = ps2;
        }
      };
      if (nh == HALF) {
#pragma unroll
        for (int j = HALF - 1; j >= 0; --j) rev(j);
      } else {
        for (int j = nh - 1; j >= 0; --j) rev(j);
      }
      __syncthreads();   // every wave's sums of the half are in LDS
      for (int e2 = tid; e2 < nh * D; e2 += NT) {
        const int j = e2 / D, col = e2 % D;
        const int64_t pbase = ((c0 + j0 + j) * h_v + h) * TILES + tile;
        float sq = 0.f, sk2 = 0.f;
#pragma unroll
        for (int w = 0; w < 2 * NW; ++w) { sq += red_q[j][w][col]; sk2 += red_k[j][w][col]; }
        ws.pdq[pbase * D + col] = sq;
        ws.pdk[pbase * D + col] = sk2;
      }
      if (tid < nh) {
        const int64_t pbase = ((c0 + j0 + tid) * h_v + h) * TILES + tile;
        float sb_ = 0.f, sg = 0.f;
#pragma unroll
        for (int w = 0; w < 2 * NW; ++w) { sb_ += red_s[tid][w][0]; sg += red_s[tid][w][1]; }
        ws.pdb[pbase] = sb_;
        ws.pdg[pbase] = sg;
      }
      __syncthreads();   // stash and sums are rewritten by the next half
    }
  }
  if (dinit && row_ok) {
    *reinterpret_cast<float4*>(dinit + smat + ca) = make_float4(gs[0], gs[1], gs[2], gs[3]);
    *reinterpret_cast<float4*>(dinit + smat + cb) = make_float4(gs[4], gs[5], gs[6], gs[7]);
  }
}

// Block-wide sum over NT threads (NT a multiple of 64).
template <int NT>
__device__ __forceinline__ float block_sum(float x, float* scratch) {
  x = group_sum<64>(x);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += scratch[w];
  __syncthreads();
  return t;
}

template <class In, int D, int NT>
__global__ __launch_bounds__(NT) void k_bwd_reduce(
    const typename In::T* __restrict__ q, const typename In::T* __restrict__ k, int64_t q_stride, int64_t k_stride,
    int use_l2, float l2_eps, int h_qk, int h_v, int64_t t_total, BwdWs ws, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dg, float* __restrict__ dbeta) {
  constexpr int TILES = D / kBwdRows;
  static_assert(NT >= D && NT % 64 == 0, "one thread per column");
  __shared__ float scratch[NT / 64];
  const int64_t t = blockIdx.x / h_qk;
  const int hq = static_cast<int>(blockIdx.x % h_qk);
  const int grp = h_v / h_qk;
  const int c = threadIdx.x;
  const bool col = c < D;
  float gq = 0.f, gk = 0.f;
  if (col) {
    for (int hh = 0; hh < grp; ++hh) {
      const int h = hq * grp + hh;
      for (int ti = 0; ti < TILES; ++ti) {
        const int64_t p = ((t * h_v + h) * TILES + ti) * D + c;
        gq += ws.pdq[p];
        gk += ws.pdk[p];
      }
    }
  }
  const float xq = col ? In::load(q + t * q_stride + static_cast<int64_t>(hq) * D, c) : 0.f;
  const float xk = col ? In::load(k + t * k_stride + static_cast<int64_t>(hq) * D, c) : 0.f;
  if (use_l2) {
    // x^ = x / r, r = sqrt(sum x^2 + eps):  dx = (dx^ - x^ (x^ . dx^)) / r
    const float rq = sqrtf(block_sum<NT>(xq * xq, scratch) + l2_eps);
    const float rk = sqrtf(block_sum<NT>(xk * xk, scratch) + l2_eps);
    const float dotq = block_sum<NT>((xq / rq) * gq, scratch);
    const float dotk = block_sum<NT>((xk / rk) * gk, scratch);
    gq = (gq - (xq / rq) * dotq) / rq;
    gk = (gk - (xk / rk) * dotk) / rk;
  }
  if (col) {
    dq[(t * h_qk + hq) * static_cast<int64_t>(D) + c] = gq;
    dk[(t * h_qk + hq) * static_cast<int64_t>(D) + c] = gk;
  }
  if (c < grp) {
    const int h = hq * grp + c;
    float sb = 0.f, sg = 0.f;
    for (int ti = 0; ti < TILES; ++ti) {
      const int64_t p = (t * h_v + h) * TILES + ti;
      sb += ws.pdb[p];
      sg += ws.pdg[p];
    }
    dbeta[t * h_v + h] = sb;
    dg[t * h_v + h] = sg;
  }
}

// ---------------------------------------------------------------------------
// Conv backward.  Forward, per sequence with padded input p = [history (3
// rows); x_s]: pre[t] = sum_i w[i] p[t + i], y[t] = SiLU(pre[t]), and the new
// history is p[L], p[L+1], p[L+2] (the width-4 causal conv: haskell-infer-demo
// README, "Architecture"; raw-input history: Flare core-design,
// short-convolution paragraph).  With dpre[t] = dy[t] SiLU'(pre[t]):
//     dp[j]  = sum_i w[i] dpre[j - i]  (0 <= j - i < L)  + d_hist_out[j - L]
//     dx[t]  = dp[t + 3],   d_hist_in[j] = dp[j] (j < 3)
//     dw[i]  = sum over all sequences and t of dpre[t] p[t + i]
// The rounding of y to the input dtype is not differentiated.
// ---------------------------------------------------------------------------
constexpr int kCbBT = 32;           // tokens per strip
constexpr int kCbThreads = 256;     // 8 channels per thread
constexpr int kCbPF = 4;            // rows fetched ahead

__device__ __forceinline__ float silu_grad(float x) {
  const float s = 1.0f / (1.0f + __expf(-x));
  return s * (1.0f + x * (1.0f - s));
}

// Strip (kCbBT tokens of one sequence, kCbThreads * 8 channels): dx of its
// rows and its share of dw (the products of its own rows), written as one
// partial per strip.  Empty strip slots write zero partials.  Each thread
// walks its 8 channels down the strip with a window of four input rows and
// four dpre values, so a strip reads its kCbBT rows of x plus 6 and of dy plus
// 3.  The rows of x and dy come kCbPF steps ahead into a ring of raw registers
// (unconditional loads from clamped rows, converted and zeroed at use: a load
// under a branch, or converted on arrival, is waited for right there).
template <class E>
__global__ __launch_bounds__(kCbThreads) void k_conv_bwd_dx(
    const typename E::T* __restrict__ x, const typename E::T* __restrict__ w, int channels,
    const int32_t* __restrict__ cu, int n_seq, int64_t t_total, const typename E::T* __restrict__ hist,
    const float* __restrict__ dy, const float* __restrict__ dhist_out, float* __restrict__ dx,
    float* __restrict__ dw_part, int64_t n_tblk) {
  const int slice = static_cast<int>(blockIdx.x / n_tblk);
  const int64_t tblk = blockIdx.x % n_tblk;
  const int c0 = (slice * kCbThreads + threadIdx.x) * 8;
  if (c0 >= channels) return;
  const int64_t ld = channels;
  float* part = dw_part + (tblk * ld + c0) * 4;
  int seq, len;
  int64_t t0;
  if (!locate_block(cu, n_seq, t_total, kCbBT, tblk, seq, t0, len)) {
#pragma unroll
    for (int e = 0; e < 32; e += 4) *reinterpret_cast<float4*>(part + e) = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const int64_t start = seq_start(cu, seq, t_total), L = seq_start(cu, seq + 1, t_total) - start;
  const int64_t u0 = t0 - start;   // local index of the strip's first token
  float wt[4][8];
  {
    float tmp[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) E::load8(w + static_cast<int64_t>(c0) * 4 + 8 * i, tmp + 8 * i);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) wt[i][c] = tmp[4 * c + i];
  }
  // raw row of the padded input p at padded index j (history rows for j < 3
  // with a history, else a clamped row of x_s), and whether it is nonzero
  auto p_src = [&](int64_t j) -> const typename E::T* {
    const int64_t jx = j - 3 < L ? (j - 3 < 0 ? 0 : j - 3) : L - 1;   // a row of x_s (L >= 1 here)
    return (j < 3 && hist) ? hist + (static_cast<int64_t>(seq) * 3 + j) * ld + c0 : x + (start + jx) * ld + c0;
  };
  auto p_valid = [&](int64_t j) { return j < 3 ? hist != nullptr : j - 3 < L; };
  auto dy_src = [&](int64_t t) { return dy + (start + (t < L ? t : L - 1)) * ld + c0; };

  // window: padded rows u + 0 .. u + 3 of the dpre token u being formed (the
  // first three enter before the walk), and dpre of the four tokens before it
  float pw[4][8], dw4[4][8];
  float dwa[4][8] = {};
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int64_t j = u0 + r;
    E::unpack8(E::ld_vec(p_src(j)), pw[r + 1]);
    const bool ok = p_valid(j);
#pragma unroll
    for (int c = 0; c < 8; ++c) pw[r + 1][c] = ok ? pw[r + 1][c] : 0.f;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int c = 0; c < 8; ++c) dw4[k][c] = 0.f;
  // ring of rows fetched ahead: step r needs padded row u0 + r + 3 and dy of token u0 + r
  typename E::Vec pring[kCbPF];
  float4 gring[kCbPF][2];
#pragma unroll
  for (int k = 0; k < kCbPF; ++k) {
    pring[k] = E::ld_vec(p_src(u0 + k + 3));
    const float* g = dy_src(u0 + k);
    gring[k][0] = reinterpret_cast<const float4*>(g)[0];
    gring[k][1] = reinterpret_cast<const float4*>(g)[1];
  }
  // steps r = 0 .. kCbBT + 3: dpre of token u0 + r, and dx of token u0 + r - 3
  // (tokens from u0 + 3 on need dpre up to u0 + kCbBT + 2)
  constexpr int kSteps = kCbBT + 4;
  static_assert(kSteps % kCbPF == 0, "whole ring turns");
#pragma unroll 1
  for (int r0 = 0; r0 < kSteps; r0 += kCbPF) {
#pragma unroll
    for (int k = 0; k < kCbPF; ++k) {
      const int r = r0 + k;
      const int64_t t = u0 + r;
      // shift in padded row t + 3
#pragma unroll
      for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) pw[i][c] = pw[i + 1][c];
      {
        float nr[8];
        E::unpack8(pring[k], nr);
        const bool ok = p_valid(t + 3);
#pragma unroll
        for (int c = 0; c < 8; ++c) pw[3][c] = ok ? nr[c] : 0.f;
      }
      const float4 ga = gring[k][0], gb = gring[k][1];
      // fetch the step kCbPF ahead into this slot (past the walk: a clamped re-read)
      {
        const int64_t tn = t + kCbPF;
        pring[k] = E::ld_vec(p_src(tn + 3));
        const float* g = dy_src(tn);
        gring[k][0] = reinterpret_cast<const float4*>(g)[0];
        gring[k][1] = reinterpret_cast<const float4*>(g)[1];
      }
      // dpre of token t (zero outside [0, L)), shifted into the dpre window
#pragma unroll
      for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) dw4[i][c] = dw4[i + 1][c];
      const float g[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float pre = wt[0][c] * pw[0][c] + wt[1][c] * pw[1][c] + wt[2][c] * pw[2][c] + wt[3][c] * pw[3][c];
        dw4[3][c] = t < L ? g[c] * silu_grad(pre) : 0.f;
      }
      if (r < len) {   // the strip's own tokens contribute to dw
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < 8; ++c) dwa[i][c] += dw4[3][c] * pw[i][c];
      }
      // dx[u] = dp_pad[u + 3] = sum_i w[i] dpre[u + 3 - i] (+ d_hist_out[u + 3 - L]), u = t - 3
      if (r >= 3 && r - 3 < len) {
        const int64_t u = t - 3;
        float o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          o[c] = wt[3][c] * dw4[0][c] + wt[2][c] * dw4[1][c] + wt[1][c] * dw4[2][c] + wt[0][c] * dw4[3][c];
        const int64_t jo = u + 3 - L;
        if (dhist_out && jo >= 0 && jo < 3) {
          const float* src = dhist_out + (static_cast<int64_t>(seq) * 3 + jo) * ld + c0;
          const float4 a4 = *reinterpret_cast<const float4*>(src);
          const float4 b4 = *reinterpret_cast<const float4*>(src + 4);
          const float e[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int c = 0; c < 8; ++c) o[c] += e[c];
        }
        float* dst = dx + (start + u) * ld + c0;
        *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c)
    *reinterpret_cast<float4*>(part + 4 * c) = make_float4(dwa[0][c], dwa[1][c], dwa[2][c], dwa[3][c]);
}

// d_hist_in of each sequence: dp_pad[j] for j < 3, one thread per (sequence,
// 8 channels); handles sequences of any length, including empty ones.
template <class E>
__global__ __launch_bounds__(kCbThreads) void k_conv_bwd_hist(
    const typename E::T* __restrict__ x, const typename E::T* __restrict__ w, int channels,
    const int32_t* __restrict__ cu, int n_seq, int64_t t_total, const typename E::T* __restrict__ hist,
    const float* __restrict__ dy, const float* __restrict__ dhist_out, float* __restrict__ dhist_in) {
  const int groups = channels / 8;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kCbThreads + threadIdx.x;
  const int64_t s = gid / groups;
  if (s >= n_seq) return;
  const int c0 = static_cast<int>(gid % groups) * 8;
  const int64_t ld = channels;
  const int64_t start = seq_start(cu, static_cast<int>(s), t_total);
  const int64_t L = seq_start(cu, static_cast<int>(s) + 1, t_total) - start;
  float wt[4][8];
  {
    float tmp[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) E::load8(w + static_cast<int64_t>(c0) * 4 + 8 * i, tmp + 8 * i);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) wt[i][c] = tmp[4 * c + i];
  }
  float pr[6][8];
#pragma unroll
  for (int r = 0; r < 6; ++r) {
#pragma unroll
    for (int c = 0; c < 8; ++c) pr[r][c] = 0.f;
    if (r < 3) {
      if (hist) E::load8(hist + (s * 3 + r) * ld + c0, pr[r]);
    } else if (r - 3 < L) {
      E::load8(x + (start + r - 3) * ld + c0, pr[r]);
    }
  }
  float dp[3][8];
#pragma unroll
  for (int t = 0; t < 3; ++t) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      dp[t][c] = 0.f;
      if (t < L) {
        const float pre = wt[0][c] * pr[t][c] + wt[1][c] * pr[t + 1][c] + wt[2][c] * pr[t + 2][c] + wt[3][c] * pr[t + 3][c];
        dp[t][c] = dy[(start + t) * ld + c0 + c] * silu_grad(pre);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    float o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      o[c] = 0.f;
#pragma unroll
      for (int i = 0; i <= j; ++i) o[c] += wt[i][c] * dp[j - i][c];
      if (dhist_out && j - L >= 0) o[c] += dhist_out[(s * 3 + (j - L)) * ld + c0 + c];
    }
    float* dst = dhist_in + (s * 3 + j) * ld + c0;
    *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
  }
}

// dw[c][i] = sum over blocks of the partials, in a fixed order: eight running
// sums over the blocks b = 8 m + j (eight independent loads in flight), then
// added together.
__global__ __launch_bounds__(256) void k_conv_bwd_dw(const float* __restrict__ dw_part, int channels, int64_t n_tblk,
                                                     float* __restrict__ dw) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // (channel, tap)
  if (e >= static_cast<int64_t>(channels) * 4) return;
  const int64_t stride = static_cast<int64_t>(channels) * 4;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int64_t b = 0;
  for (; b + 8 <= n_tblk; b += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += dw_part[(b + j) * stride + e];
  }
  for (int j = 0; b + j < n_tblk; ++j) acc[j] += dw_part[(b + j) * stride + e];
  dw[e] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

size_t conv_bwd_ws_bytes(int channels, int n_seq, int64_t t_total) {
  return sizeof(float) * static_cast<size_t>(block_slots(t_total, n_seq, kCbBT)) * channels * 4;
}

template <class E>
static hipError_t run_conv_bwd(const ConvBwdArgs& a) {
  using T = typename E::T;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const int64_t ntblk = block_slots(a.t_total, a.n_seq, kCbBT);
  const int nslices = (a.channels + kCbThreads * 8 - 1) / (kCbThreads * 8);
  float* part = static_cast<float*>(a.workspace);
  if (a.t_total > 0) {
    hipLaunchKernelGGL((k_conv_bwd_dx<E>), dim3(static_cast<unsigned>(ntblk * nslices)), dim3(kCbThreads), 0, st,
                       static_cast<const T*>(a.x), static_cast<const T*>(a.w), a.channels, a.cu, a.n_seq, a.t_total,
                       static_cast<const T*>(a.hist), a.dy, a.dhist_out, a.dx, part, ntblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned nb = static_cast<unsigned>((static_cast<int64_t>(a.channels) * 4 + 255) / 256);
    hipLaunchKernelGGL(k_conv_bwd_dw, dim3(nb), dim3(256), 0, st, part, a.channels, ntblk, a.dw);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    const unsigned nb = static_cast<unsigned>((static_cast<int64_t>(a.channels) * 4 + 255) / 256);
    hipLaunchKernelGGL(k_conv_bwd_dw, dim3(nb), dim3(256), 0, st, part, a.channels, int64_t(0), a.dw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.dhist_in) {
    const int64_t threads = static_cast<int64_t>(a.n_seq) * (a.channels / 8);
    hipLaunchKernelGGL((k_conv_bwd_hist<E>), dim3(static_cast<unsigned>((threads + kCbThreads - 1) / kCbThreads)),
                       dim3(kCbThreads), 0, st, static_cast<const T*>(a.x), static_cast<const T*>(a.w), a.channels,
                       a.cu, a.n_seq, a.t_total, static_cast<const T*>(a.hist), a.dy, a.dhist_out, a.dhist_in);
  }
  return hipGetLastError();
}

hipError_t launch_conv1d_bwd(const ConvBwdArgs& a) {
  if (a.dt == GDN_BF16) return run_conv_bwd<BF16>(a);
  return run_conv_bwd<F32>(a);
}

template <class In, int D>
static hipError_t run_bwd(const BwdArgs& a) {
  using T = typename In::T;
  constexpr int NT = D == 128 ? 256 : 64;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  BwdWs ws = bwd_carve(a.workspace, a.h_v, D, a.n_seq, a.t_total);
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const int64_t nblk = static_cast<int64_t>(a.n_seq) * a.h_v * (D / kBwdRows);
  if (a.t_total > 0) {
    hipLaunchKernelGGL((k_bwd_ckpt<In, D, NT>), dim3(static_cast<unsigned>(nblk)), dim3(NT), 0, st, q, k, v,
                       a.q_stride, a.k_stride, a.v_stride, a.gate, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.cu, a.n_seq,
                       a.t_total, a.init, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_bwd_slice<In, D, NT>), dim3(static_cast<unsigned>(nblk)), dim3(NT), 0, st, q, k, v,
                     a.q_stride, a.k_stride, a.v_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.cu,
                     a.n_seq, a.t_total, a.d_o, a.d_final, a.dv, a.d_init, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.t_total == 0) return e;
  constexpr int NTR = D < 64 ? 64 : D;
  hipLaunchKernelGGL((k_bwd_reduce<In, D, NTR>), dim3(static_cast<unsigned>(a.t_total * a.h_qk)), dim3(NTR), 0, st,
                     q, k, a.q_stride, a.k_stride, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.t_total, ws, a.dq, a.dk,
                     a.dg, a.dbeta);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd(const BwdArgs& a) {
  if (a.dt == GDN_BF16) {
    if (a.d == 128) return launch_chunk_bwd_chunked(a);
  } else {
    if (a.d == 128) return run_bwd<F32, 128>(a);
    if (a.d == 16) return run_bwd<F32, 16>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
