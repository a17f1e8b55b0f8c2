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
// Kernels:
//   k_chunk_prep  persistent workgroups over (chunk, q/k head) units: the
//                 Gram matrices K K^T and Q K^T on the matrix cores (raw
//                 operands, exact products) once per unit, then for each v-head
//                 reading that q/k head the decay scalars, L, P and the
//                 unit-lower-triangular solve (16x16 diagonal blocks by forward
//                 substitution in registers, off-diagonal blocks by fp32 MFMA).
//                 It writes K, Q, Tb and P (Tb, P split into bf16 hi/lo; for
//                 fp32 inputs also K^T) in matrix-core fragment order, and
//                 loads the next unit's K, Q while it computes.
//   k_chunk_scan  one workgroup per (sequence, v-head, 16-wide d_v slice),
//                 walking the sequence's chunks in order with its slice of the
//                 state in fp32 registers; every contraction with the state or
//                 a derived operand runs on the matrix cores.
//   k_seq_order   (calls with several sequences) the sequences longest first,
//                 the order in which the scan starts them.
//
// Data movement of the scan.  Every chunk operand the scan reads (K, Q, Tb,
// P) is a matrix-core operand that exactly one wave uses: wave w owns token
// rows 16w..16w+15 of K, Q, Tb and P.  The K^T operands of the state update
// (d_k rows 16(w + 4j)) come from the chunk's K rows, which the waves leave in
// LDS, through transposing LDS reads (bf16); for fp32 inputs from a K^T copy
// in the workspace.  So each wave loads its fragments straight from memory into the
// registers the MFMAs read -- nothing is staged through LDS -- and issues the
// next chunk's loads for a register set as soon as the current chunk's MFMAs
// have consumed it, giving every load a full chunk step of latency.  Only the
// operands every wave needs (the state S, X, U and the decayed U) pass
// through LDS, three barriers per chunk.  The outputs are built transposed,
// O^T = S Q^T and U^T P^T (S and U as A operands, Q and P as B operands), so
// a lane ends with four consecutive d_v values of one token: one vector store.
//
// Operand precision (policy PolBF16): raw bf16 q/k/v are exact single bf16
// operands; derived operands (S, X, U, Tb, P) are bf16 hi+lo pairs and a
// product uses hi*hi + hi*lo + lo*hi (or hi*raw + lo*raw), accumulated in fp32
// (the multi-term bf16 technique of Henry, Tang and Heinecke, ARITH 2019).
// Policy PolF32 uses the fp32 matrix-core instruction for fp32 inputs.
#include <mutex>

#include "chunk_impl.hpp"

namespace gdn {

// ---------------------------------------------------------------------------
// k_seq_order: the sequences, most chunks first, for the scan's block order.
// The scan's workgroups start in index order and each runs one sequence's
// chunks back to back, so the longest sequence bounds the call: listing it
// first starts it at once, spread over every XCD, and the shorter ones fill
// the compute units behind it (longest-first list scheduling).  A counting
// sort on a key that is exact below 32 chunks and has eight steps per octave
// above; equal keys may come out in any order, which changes no result.
// ---------------------------------------------------------------------------
constexpr int kOrderBins = 256;

__device__ __forceinline__ int order_key(int64_t nch) {
  if (nch < 32) return nch > 0 ? static_cast<int>(nch) : 0;
  const int e = 63 - __builtin_clzll(static_cast<unsigned long long>(nch));   // >= 5
  const int key = 32 + 8 * (e - 5) + static_cast<int>((nch >> (e - 3)) & 7);
  return key < kOrderBins ? key : kOrderBins - 1;
}

__global__ __launch_bounds__(kOrderBins) void k_seq_order(const int32_t* __restrict__ cu, int n_seq, int C,
                                                          int32_t* __restrict__ order) {
  __shared__ int cnt[kOrderBins];
  __shared__ int scan[2][kOrderBins];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  for (int s = tid; s < n_seq; s += kOrderBins) atomicAdd(&cnt[order_key((cu[s + 1] - cu[s] + C - 1) / C)], 1);
  __syncthreads();
  // inclusive scan of the counts in descending key order: x_t = cnt[last - t]
  const int x = cnt[kOrderBins - 1 - tid];
  int cur = 0;
  scan[0][tid] = x;
  __syncthreads();
  for (int off = 1; off < kOrderBins; off <<= 1) {
    const int y = scan[cur][tid] + (tid >= off ? scan[cur][tid - off] : 0);
    scan[cur ^ 1][tid] = y;
    cur ^= 1;
    __syncthreads();
  }
  cnt[kOrderBins - 1 - tid] = scan[cur][tid] - x;   // first position of the key
  __syncthreads();
  for (int s = tid; s < n_seq; s += kOrderBins)
    order[atomicAdd(&cnt[order_key((cu[s + 1] - cu[s] + C - 1) / C)], 1)] = s;
}

// ---------------------------------------------------------------------------
// k_single_token: one-token sequences (the decode tokens of a mixed batch).
// Their recurrence, a = exp(g), e = v - a S k^, S <- a S + beta e k^^T,
// o = scale S q^, runs in fp32 on the vector units, as in the decode step:
// SPLIT workgroups per (sequence, v-head), each over D / SPLIT state rows,
// D / 8 lanes per row (columns 4l .. 4l+3 and D/2 + 4l ..).  The prep kernel
// leaves these sequences out and the scan returns at once for them; every
// other sequence returns here at once.  A separate launch keeps these light
// workgroups off the scan's register and LDS footprint.
// ---------------------------------------------------------------------------
template <class In, class EO, int D, int NT, int SPLIT>
__global__ __launch_bounds__(NT) void k_single_token(
    const typename In::T* __restrict__ q, const typename In::T* __restrict__ k,
    const typename In::T* __restrict__ v, int64_t q_stride, int64_t k_stride, int64_t v_stride, GateSrc gates,
    float scale, int use_l2, float l2_eps, int h_qk, int h_v, const int32_t* __restrict__ cu, int n_seq,
    int64_t t_total, const float* __restrict__ init, float* __restrict__ fin, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ fresh, typename EO::T* __restrict__ o) {
  constexpr int TPR = D / 8, RPP = NT / TPR, RW = D / SPLIT, PASSES = (RW + RPP - 1) / RPP;
  static_assert(TPR <= 64 && NT % 64 == 0 && D % SPLIT == 0, "row lanes within a wave");
  const int part = static_cast<int>(blockIdx.x % SPLIT);
  const int64_t sh = blockIdx.x / SPLIT;
  const int s = static_cast<int>(sh / h_v), h = static_cast<int>(sh % h_v);
  if (s >= n_seq) return;
  const int64_t t = seq_start(cu, s, t_total);
  if (seq_start(cu, s + 1, t_total) - t != 1) return;
  const int sslot = slots ? slots[s] : s;
  if (sslot < 0) return;
  const float* src = (init != nullptr && !(fresh && fresh[s] != 0)) ? init : nullptr;
  const int hq = h / (h_v / h_qk);
  const int tid = threadIdx.x, l = tid % TPR, rg = tid / TPR;
  const int ca = 4 * l, cb = D / 2 + 4 * l;
  const int64_t smat = (static_cast<int64_t>(sslot) * h_v + h) * D * D;

  float4 sa[PASSES], sb[PASSES];
  float vv[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = part * RW + (rg + p * RPP < RW ? rg + p * RPP : 0);
    sa[p] = sb[p] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (src) {
      sa[p] = *reinterpret_cast<const float4*>(src + smat + static_cast<int64_t>(row) * D + ca);
      sb[p] = *reinterpret_cast<const float4*>(src + smat + static_cast<int64_t>(row) * D + cb);
    }
    vv[p] = In::load(v + t * v_stride + static_cast<int64_t>(h) * D, row);
  }
  float kk[8], qq[8];
  const typename In::T* kr = k + t * k_stride + static_cast<int64_t>(hq) * D;
  const typename In::T* qr = q + t * q_stride + static_cast<int64_t>(hq) * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kk[i] = In::load(kr, ca + i);
    kk[4 + i] = In::load(kr, cb + i);
    qq[i] = In::load(qr, ca + i);
    qq[4 + i] = In::load(qr, cb + i);
  }
  float gv, bt;
  load_gate(gates, t, h, h_v, gv, bt);
  float sk, sq, kq;
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
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    float dk = tok_dot8(sa[p], sb[p], kk);
    float dq = tok_dot8(sa[p], sb[p], qq);
    dk = group_sum<TPR>(dk);
    dq = group_sum<TPR>(dq);
    const float e = tok_err(vv[p], alpha, dk), be = bt * e;
    if (rg + p * RPP < RW) {
      const int64_t row = part * RW + rg + p * RPP;
      if (fin) {
        *reinterpret_cast<float4*>(fin + smat + row * D + ca) = tok_upd4(alpha, sa[p], be, kk);
        *reinterpret_cast<float4*>(fin + smat + row * D + cb) = tok_upd4(alpha, sb[p], be, kk + 4);
      }
      if (l == 0) EO::store(o, (t * h_v + h) * static_cast<int64_t>(D) + row, tok_out(scale, alpha, dq, be, kq));
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <class Pol, int D, int C>
static size_t ws_bytes_for(int h_qk, int h_v, int n_seq, int64_t t_total, int with_norm) {
  const int64_t slots = block_slots(t_total, n_seq, C);
  size_t b = WsLayout<Pol, D, C>::bytes(slots, h_qk, h_v, n_seq);
  if (with_norm) b += WsLayout<Pol, D, C>::al(sizeof(float) * t_total * h_v * D);
  return b;
}

size_t chunk_ws_bytes(gdn_dtype dt, int h_qk, int h_v, int d, int chunk, int n_seq, int64_t t_total,
                      int with_norm) {
  if (dt == GDN_BF16) return ws_bytes_for<PolBF16, 128, 64>(h_qk, h_v, n_seq, t_total, with_norm);
  if (d == 128) return ws_bytes_for<PolF32, 128, 64>(h_qk, h_v, n_seq, t_total, with_norm);
  return ws_bytes_for<PolF32, 16, 16>(h_qk, h_v, n_seq, t_total, with_norm);
}

hipError_t launch_seq_order(const int32_t* cu, int n_seq, int chunk, int32_t* order, hipStream_t st) {
  hipLaunchKernelGGL(k_seq_order, dim3(1), dim3(kOrderBins), 0, st, cu, n_seq, chunk, order);
  return hipGetLastError();
}

template <class In, int D>
static hipError_t single_token_for(const ChunkArgs& a, float* o_pre, hipStream_t st) {
  using T = typename In::T;
  constexpr int NT1 = D == 128 ? 256 : 64, SPL = D == 128 ? 4 : 1;
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const int64_t nb1 = static_cast<int64_t>(a.n_seq) * a.h_v * SPL;
  if (a.z)
    hipLaunchKernelGGL((k_single_token<In, F32, D, NT1, SPL>), dim3(static_cast<unsigned>(nb1)), dim3(NT1), 0, st,
                       q, k, v, a.q_stride, a.k_stride, a.v_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk,
                       a.h_v, a.cu, a.n_seq, a.t_total, a.init, a.fin, a.slots, a.fresh, o_pre);
  else if (a.o_dt == GDN_BF16)
    hipLaunchKernelGGL((k_single_token<In, BF16, D, NT1, SPL>), dim3(static_cast<unsigned>(nb1)), dim3(NT1), 0, st,
                       q, k, v, a.q_stride, a.k_stride, a.v_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk,
                       a.h_v, a.cu, a.n_seq, a.t_total, a.init, a.fin, a.slots, a.fresh,
                       static_cast<uint16_t*>(a.o));
  else
    hipLaunchKernelGGL((k_single_token<In, F32, D, NT1, SPL>), dim3(static_cast<unsigned>(nb1)), dim3(NT1), 0, st,
                       q, k, v, a.q_stride, a.k_stride, a.v_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk,
                       a.h_v, a.cu, a.n_seq, a.t_total, a.init, a.fin, a.slots, a.fresh, static_cast<float*>(a.o));
  return hipGetLastError();
}

hipError_t launch_single_token(const ChunkArgs& a, float* o_pre, hipStream_t st) {
  if (a.dt == GDN_BF16) return single_token_for<BF16, 128>(a, o_pre, st);
  if (a.d == 128) return single_token_for<F32, 128>(a, o_pre, st);
  return single_token_for<F32, 16>(a, o_pre, st);
}

// A second stream per device for the one-token sequences of a call, which
// then run beside the scan instead of after it (they read no prep output and
// write other sequences' rows and states).  Created on first use with the
// default priority and held until the process ends; the fork and the join
// are events, so a captured call captures both branches.  Calls from several
// host threads on one device share it (each fork, launch and join record is
// made under a lock, and a join waits at least for its own launch).
namespace {
struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxSideDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxSideDevices];

// Launches one-token work on the side stream after everything already on st;
// *forked tells whether st must wait for it (side_join).  Falls back to st
// itself while st is being captured (a capture must not pull a stream that
// other threads use into the graph) or where no side stream can be had.
hipError_t side_fork(const ChunkArgs& a, float* o_pre, hipStream_t st, bool* forked) {
  *forked = false;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  int dev = 0;
  if (!a.side_ok || hipStreamIsCapturing(st, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone ||
      hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices)
    return launch_single_token(a, o_pre, st);
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream& sd = g_side[dev];
  hipError_t e = hipSuccess;
  if (!sd.st) {
    hipStream_t s2 = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if ((e = hipStreamCreateWithFlags(&s2, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&f, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&j, hipEventDisableTiming)) != hipSuccess) return e;
    sd.st = s2;
    sd.fork = f;
    sd.join = j;
  }
  if ((e = hipEventRecord(sd.fork, st)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(sd.st, sd.fork, 0)) != hipSuccess) return e;
  if ((e = launch_single_token(a, o_pre, sd.st)) != hipSuccess) return e;
  if ((e = hipEventRecord(sd.join, sd.st)) != hipSuccess) return e;
  *forked = true;
  return hipSuccess;
}

// st waits for the side stream's work so far (at least the last fork's launch).
hipError_t side_join(hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_side_mu);
  return hipStreamWaitEvent(st, g_side[dev].join, 0);
}
}  // namespace

template <class Pol, int D, int C>
static hipError_t run_chunk(const ChunkArgs& a) {
  using T = typename Pol::In::T;
  const int64_t slots = block_slots(a.t_total, a.n_seq, C);
  ChunkWs ws = WsLayout<Pol, D, C>::carve(a.workspace, slots, a.h_qk, a.h_v, a.n_seq);
  float* o_pre = reinterpret_cast<float*>(static_cast<char*>(a.workspace) +
                                          WsLayout<Pol, D, C>::bytes(slots, a.h_qk, a.h_v, a.n_seq));

  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  if (slots > 0) {
    // persistent grid: as many workgroups as can be resident at once, so
    // every workgroup runs from the start and the unit loop balances
    static const int per_cu = [] {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_chunk_prep<Pol, D, C>, 256, 0) != hipSuccess || n < 1)
        n = 1;
      return n;
    }();
    const int64_t units = slots * a.h_qk;
    const int64_t resident = static_cast<int64_t>(per_cu) * device_cu_count();
    const int64_t grid = units < resident ? units : resident;
    hipLaunchKernelGGL((k_chunk_prep<Pol, D, C>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, q, k,
                       a.q_stride, a.k_stride, a.gate, a.scale, a.use_l2, a.l2_eps, a.h_qk, a.h_v, a.cu,
                       a.n_seq, a.t_total, a.slots, ws, slots);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ws.order) {
    hipError_t e = launch_seq_order(a.cu, a.n_seq, C, ws.order, st);
    if (e != hipSuccess) return e;
  }
  // One-token sequences: skipped only when a single sequence holds all of
  // several tokens (cu_seqlens ends at t_total, so it has no one-token
  // sequence); in a mixed call t_total is a capacity.
  bool forked = false;
  if (a.n_seq > 1 || a.t_total == 1 || a.slots != nullptr) {
    hipError_t e = side_fork(a, o_pre, st, &forked);
    if (e != hipSuccess) return e;
  }
  // One 16-wide d_v tile per workgroup: a single long sequence has only
  // heads x d_v/16 independent recurrences, and the chunk loop's latency, not
  // the matrix cores, sets its pace, so the widest grid wins (two tiles per
  // workgroup measured 1.6x slower on one 4096-token sequence).
  constexpr int NV = 1;
  const int64_t nblk = (int64_t)a.n_seq * a.h_v * (D / (16 * NV));
  if (a.z) {
    hipLaunchKernelGGL((k_chunk_scan<Pol, F32, D, C, NV>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st,
                       q, k, v, a.q_stride, a.k_stride, a.v_stride, a.h_qk, a.h_v, a.cu, a.n_seq, a.t_total,
                       a.init, a.fin, a.slots, a.fresh, o_pre, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (forked && (e = side_join(st)) != hipSuccess) return e;
    if (a.t_total > 0)
      return launch_gated_rmsnorm(o_pre, GDN_F32, a.z, a.dt, a.norm_w, a.norm_eps, a.t_total * a.h_v, D,
                                  a.o, a.o_dt, a.stream, a.slots ? a.cu : nullptr, a.n_seq, a.slots, a.h_v);
    return hipSuccess;
  }
  if (a.o_dt == GDN_BF16)
    hipLaunchKernelGGL((k_chunk_scan<Pol, BF16, D, C, NV>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st,
                       q, k, v, a.q_stride, a.k_stride, a.v_stride, a.h_qk, a.h_v, a.cu, a.n_seq, a.t_total,
                       a.init, a.fin, a.slots, a.fresh, static_cast<uint16_t*>(a.o), ws);
  else
    hipLaunchKernelGGL((k_chunk_scan<Pol, F32, D, C, NV>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, st,
                       q, k, v, a.q_stride, a.k_stride, a.v_stride, a.h_qk, a.h_v, a.cu, a.n_seq, a.t_total,
                       a.init, a.fin, a.slots, a.fresh, static_cast<float*>(a.o), ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return forked ? side_join(st) : hipSuccess;
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
