// C ABI of the GDN mixer library: argument validation on the host, then the
// launchers.  Every check runs before any launch, so a rejected call writes
// nothing; no path here reads device memory, allocates or synchronises.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "../../include/gdn.h"
#include "launch.hpp"
#include "mixer_decode.hpp"

namespace {

thread_local int32_t g_last_hip_error = 0;

struct Range {
  const void* p;
  uint64_t bytes;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned16(p)) return false;
  return true;
}

// An output range must not overlap any of the given ranges.
bool disjoint(const Range& out, std::initializer_list<Range> others) {
  for (const Range& r : others)
    if (overlap(out, r)) return false;
  return true;
}

int dt_bytes(gdn_dtype dt) { return dt == GDN_BF16 ? 2 : 4; }
bool dt_valid(gdn_dtype dt) { return dt == GDN_BF16 || dt == GDN_F32; }

// Byte extent of `rows` rows of `width` elements with a row stride (elements).
uint64_t strided_bytes(int64_t rows, int64_t stride, int64_t width, int eb) {
  if (rows <= 0) return 0;
  return static_cast<uint64_t>((rows - 1) * stride + width) * eb;
}

gdn_status finish(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int32_t>(e);
    return GDN_ERR_HIP;
  }
  return GDN_OK;
}

// Workspace of gdn_chunk_fwd_noalloc: a library-owned device array, one copy
// per GPU (the loader places it when the code object is first loaded on a
// device, and it stays until the process ends).  In host code `scratch` names
// a host-side stand-in, not device memory, so its device address is taken
// once per device with hipGetSymbolAddress and only that address is used.
static_assert(GDN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of this device's scratch (looked up on the first call on the
// device), or nullptr with the HIP error recorded.
void* device_scratch() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int32_t>(e);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) {
    g_last_hip_error = static_cast<int32_t>(hipErrorInvalidDevice);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_hip_error = static_cast<int32_t>(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// The gates of a recurrence call as the caller passed them: fp32 g and beta,
// or (raw) the gate projections a, b with a_log and an optional dt_bias.
struct GateArgs {
  bool raw;
  const float* g;
  const float* beta;
  const void* a;
  const void* b;
  int64_t ab_stride;
  gdn_dtype ab_dt;
  const float* a_log;
  const float* dt_bias;

  bool rows_missing() const { return raw ? (!a || !b) : (!g || !beta); }
};

GateArgs plain_gates(const float* g, const float* beta) {
  return GateArgs{false, g, beta, nullptr, nullptr, 0, GDN_F32, nullptr, nullptr};
}

GateArgs raw_gates(const void* a, const void* b, int64_t ab_stride, gdn_dtype ab_dt, const float* a_log,
                   const float* dt_bias) {
  return GateArgs{true, nullptr, nullptr, a, b, ab_stride, ab_dt, a_log, dt_bias};
}

// Validated gates of `rows` token rows: the kernels' gate source and the byte
// ranges the gate inputs occupy (for the overlap checks of the outputs).
struct Gates {
  gdn::GateSrc src{};
  Range r[4]{};
};

gdn_status check_gates(const GateArgs& ga, int64_t rows, int32_t h_v, Gates& out) {
  out = Gates{};
  if (!ga.raw) {
    if (!all_aligned({ga.g, ga.beta})) return GDN_ERR_ALIGN;
    out.src.g = ga.g;
    out.src.beta = ga.beta;
    out.r[0] = Range{ga.g, static_cast<uint64_t>(rows) * h_v * 4};
    out.r[1] = Range{ga.beta, static_cast<uint64_t>(rows) * h_v * 4};
    return GDN_OK;
  }
  if (!ga.a_log) return GDN_ERR_NULL;
  if (!dt_valid(ga.ab_dt)) return GDN_ERR_UNSUPPORTED;
  const int64_t stride = ga.ab_stride == 0 ? h_v : ga.ab_stride;
  if (stride < h_v) return GDN_ERR_INVALID;
  // a and b are read one element at a time, so element alignment suffices
  // (a packed [rows, 2 h_v] b|a tensor puts a at an offset of h_v elements)
  const int eb = dt_bytes(ga.ab_dt);
  const uintptr_t pa = reinterpret_cast<uintptr_t>(ga.a), pb = reinterpret_cast<uintptr_t>(ga.b);
  if (pa % eb || pb % eb || reinterpret_cast<uintptr_t>(ga.a_log) % 4 || reinterpret_cast<uintptr_t>(ga.dt_bias) % 4)
    return GDN_ERR_ALIGN;
  out.src.a = ga.a;
  out.src.b = ga.b;
  out.src.ab_stride = stride;
  out.src.ab_bf16 = ga.ab_dt == GDN_BF16;
  out.src.a_log = ga.a_log;
  out.src.dt_bias = ga.dt_bias;
  out.r[0] = Range{ga.a, strided_bytes(rows, stride, h_v, eb)};
  out.r[1] = Range{ga.b, strided_bytes(rows, stride, h_v, eb)};
  out.r[2] = Range{ga.a_log, static_cast<uint64_t>(h_v) * 4};
  out.r[3] = Range{ga.dt_bias, ga.dt_bias ? static_cast<uint64_t>(h_v) * 4 : 0};
  return GDN_OK;
}

bool disjoint_gates(const Range& out, const Gates& gt) {
  for (const Range& r : gt.r)
    if (overlap(out, r)) return false;
  return true;
}

// Shared checks of the q/k/v arguments of the recurrence entry points.
gdn_status check_qkv(const void* q, const void* k, const void* v, int64_t& q_stride, int64_t& k_stride,
                     int64_t& v_stride, gdn_dtype dt, bool gate_rows_missing, int32_t h_qk,
                     int32_t h_v, int32_t d_k, int32_t d_v, bool has_rows = true) {
  if (has_rows && (!q || !k || !v || gate_rows_missing)) return GDN_ERR_NULL;
  if (h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0 || h_v % h_qk != 0) return GDN_ERR_INVALID;
  if (!dt_valid(dt)) return GDN_ERR_UNSUPPORTED;
  if (q_stride == 0) q_stride = static_cast<int64_t>(h_qk) * d_k;
  if (k_stride == 0) k_stride = static_cast<int64_t>(h_qk) * d_k;
  if (v_stride == 0) v_stride = static_cast<int64_t>(h_v) * d_v;
  if (q_stride < static_cast<int64_t>(h_qk) * d_k || k_stride < static_cast<int64_t>(h_qk) * d_k ||
      v_stride < static_cast<int64_t>(h_v) * d_v)
    return GDN_ERR_INVALID;
  // row offsets inside a chunk or a decode batch row are formed in 32 bits
  constexpr int64_t kMaxStride = int64_t(1) << 24;
  if (q_stride > kMaxStride || k_stride > kMaxStride || v_stride > kMaxStride) return GDN_ERR_INVALID;
  if (q_stride % 8 || k_stride % 8 || v_stride % 8) return GDN_ERR_ALIGN;
  if (!all_aligned({q, k, v})) return GDN_ERR_ALIGN;
  return GDN_OK;
}

}  // namespace

namespace gdn {

int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace gdn

extern "C" {

const char* gdn_version(void) { return "gdn-mi355x 0.1.0 (gfx950)"; }

int32_t gdn_last_hip_error(void) { return g_last_hip_error; }

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_INVALID: return "GDN_ERR_INVALID: invalid size, stride or head grouping";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: head dims, chunk or dtype not supported";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: pointer or stride not 16-byte aligned";
    case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: an output overlaps another buffer";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: kernel launch failed";
    default: return "unknown gdn_status";
  }
}

gdn_status gdn_conv1d_fwd(const void* x, gdn_dtype dt, const void* w, int32_t channels, const int32_t* cu_seqlens,
                          int32_t n_seq, int64_t t_total, void* conv_state, int32_t n_slots,
                          const int32_t* state_slots, void* y, void* stream) {
  if (n_seq < 0 || t_total < 0 || channels <= 0 || n_slots < 0) return GDN_ERR_INVALID;
  if (!dt_valid(dt)) return GDN_ERR_UNSUPPORTED;
  if (channels % 8) return GDN_ERR_INVALID;
  if (n_seq == 0) return GDN_OK;
  if (!x && t_total > 0) return GDN_ERR_NULL;
  if (!y && t_total > 0) return GDN_ERR_NULL;
  if (!w || !conv_state) return GDN_ERR_NULL;
  if (!cu_seqlens && t_total != n_seq) return GDN_ERR_INVALID;
  if (!state_slots && n_slots < n_seq) return GDN_ERR_INVALID;
  if (!all_aligned({x, w, conv_state, y, cu_seqlens, state_slots})) return GDN_ERR_ALIGN;
  const int eb = dt_bytes(dt);
  const Range rx{x, static_cast<uint64_t>(t_total) * channels * eb};
  const Range ry{y, static_cast<uint64_t>(t_total) * channels * eb};
  const Range rw{w, static_cast<uint64_t>(channels) * 4 * eb};
  const Range rs{conv_state, static_cast<uint64_t>(n_slots) * 3 * channels * eb};
  const Range rcu{cu_seqlens, cu_seqlens ? static_cast<uint64_t>(n_seq + 1) * 4 : 0};
  const Range rsl{state_slots, state_slots ? static_cast<uint64_t>(n_seq) * 4 : 0};
  if (!disjoint(ry, {rx, rw, rs, rcu, rsl}) || !disjoint(rs, {rx, rw, rcu, rsl})) return GDN_ERR_ALIAS;
  return finish(gdn::launch_conv1d(x, dt, w, channels, cu_seqlens, n_seq, t_total, conv_state, state_slots, y,
                                   stream));
}

gdn_status gdn_chunk_fwd_workspace_size(int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, int32_t chunk,
                                        int32_t n_seq, int64_t t_total, gdn_dtype dt, int32_t with_norm,
                                        size_t* bytes) {
  if (!bytes) return GDN_ERR_NULL;
  if (h_qk <= 0 || h_v <= 0 || h_v % h_qk != 0 || n_seq < 0 || t_total < 0) return GDN_ERR_INVALID;
  if (!dt_valid(dt)) return GDN_ERR_UNSUPPORTED;
  const bool ok = (d_k == 128 && d_v == 128 && chunk == 64) || (dt == GDN_F32 && d_k == 16 && d_v == 16 && chunk == 16);
  if (!ok) return GDN_ERR_UNSUPPORTED;
  *bytes = gdn::chunk_ws_bytes(dt, h_qk, h_v, d_v, chunk, n_seq, t_total, with_norm);
  return GDN_OK;
}

}  // extern "C"

namespace {

gdn_status chunk_fwd_impl(const void* q, const void* k, const void* v, int64_t q_stride, int64_t k_stride,
                          int64_t v_stride, gdn_dtype dt, const GateArgs& ga, float scale, int32_t use_qk_l2norm,
                          float l2_eps, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, int32_t chunk,
                          const int32_t* cu_seqlens, int32_t n_seq, int64_t t_total, const float* initial_state,
                          float* final_state, void* o, gdn_dtype o_dt, const void* z, const float* norm_w,
                          float norm_eps, void* workspace, size_t ws_bytes, void* stream,
                          const int32_t* state_slots = nullptr, const int32_t* fresh = nullptr,
                          int32_t n_slots = 0, bool side_ok = true) {
  // With state_slots (the mixed prefill + decode form) initial_state and
  // final_state are the same state pool of n_slots rows, read and written at
  // the slot of each sequence.
  if (n_seq < 0 || t_total < 0 || n_slots < 0) return GDN_ERR_INVALID;
  if (n_seq == 0) return GDN_OK;
  gdn_status st = check_qkv(q, k, v, q_stride, k_stride, v_stride, dt, ga.rows_missing(), h_qk, h_v, d_k, d_v,
                            t_total > 0);
  if (st != GDN_OK) return st;
  Gates gt;
  st = check_gates(ga, t_total, h_v, gt);
  if (st != GDN_OK) return st;
  if (!o && t_total > 0) return GDN_ERR_NULL;
  if (!workspace) return GDN_ERR_WORKSPACE;
  if (z && !norm_w) return GDN_ERR_NULL;
  if (!cu_seqlens && n_seq != 1) return GDN_ERR_NULL;
  if (!dt_valid(o_dt)) return GDN_ERR_UNSUPPORTED;
  size_t need = 0;
  st = gdn_chunk_fwd_workspace_size(h_qk, h_v, d_k, d_v, chunk, n_seq, t_total, dt, z != nullptr, &need);
  if (st != GDN_OK) return st;
  if (ws_bytes < need) return GDN_ERR_WORKSPACE;
  if (!all_aligned({o, z, norm_w, initial_state, final_state, workspace, cu_seqlens, state_slots, fresh}))
    return GDN_ERR_ALIGN;
  const int eb = dt_bytes(dt);
  const uint64_t state_bytes = static_cast<uint64_t>(state_slots ? n_slots : n_seq) * h_v * d_v * d_k * 4;
  const Range rsl{state_slots, state_slots ? static_cast<uint64_t>(n_seq) * 4 : 0};
  const Range rfr{fresh, fresh ? static_cast<uint64_t>(n_seq) * 4 : 0};
  const Range rq{q, strided_bytes(t_total, q_stride, static_cast<int64_t>(h_qk) * d_k, eb)};
  const Range rk{k, strided_bytes(t_total, k_stride, static_cast<int64_t>(h_qk) * d_k, eb)};
  const Range rv{v, strided_bytes(t_total, v_stride, static_cast<int64_t>(h_v) * d_v, eb)};
  const Range ro{o, static_cast<uint64_t>(t_total) * h_v * d_v * dt_bytes(o_dt)};
  const Range rz{z, z ? static_cast<uint64_t>(t_total) * h_v * d_v * eb : 0};
  const Range rw{norm_w, z ? static_cast<uint64_t>(d_v) * 4 : 0};
  const Range ri{initial_state, initial_state ? state_bytes : 0};
  const Range rf{final_state, final_state ? state_bytes : 0};
  const Range rws{workspace, need};
  const Range rcu{cu_seqlens, cu_seqlens ? static_cast<uint64_t>(n_seq + 1) * 4 : 0};
  if (!disjoint(ro, {rq, rk, rv, rz, rw, ri, rf, rws, rcu, rsl, rfr}) || !disjoint_gates(ro, gt))
    return GDN_ERR_ALIAS;
  if (!disjoint(rws, {rq, rk, rv, rz, rw, ri, rf, rcu, rsl, rfr}) || !disjoint_gates(rws, gt)) return GDN_ERR_ALIAS;
  if (!disjoint(rf, {rq, rk, rv, rz, rw, rcu, rsl, rfr}) || !disjoint_gates(rf, gt)) return GDN_ERR_ALIAS;
  if (initial_state && final_state && initial_state != final_state && overlap(ri, rf)) return GDN_ERR_ALIAS;

  gdn::ChunkArgs a;
  a.q = q; a.k = k; a.v = v;
  a.q_stride = q_stride; a.k_stride = k_stride; a.v_stride = v_stride;
  a.dt = dt; a.gate = gt.src; a.scale = scale;
  a.use_l2 = use_qk_l2norm != 0; a.l2_eps = l2_eps;
  a.h_qk = h_qk; a.h_v = h_v; a.d = d_k; a.chunk = chunk;
  a.cu = cu_seqlens; a.n_seq = n_seq; a.t_total = t_total;
  a.init = initial_state; a.fin = final_state;
  a.slots = state_slots; a.fresh = fresh;
  a.o = o; a.o_dt = o_dt; a.z = z; a.norm_w = norm_w; a.norm_eps = norm_eps;
  a.workspace = workspace; a.stream = stream;
  a.side_ok = side_ok;
  return finish(gdn::launch_chunk_fwd(a));
}

gdn_status recurrent_step_impl(const void* q, const void* k, const void* v, int64_t q_stride, int64_t k_stride,
                               int64_t v_stride, gdn_dtype dt, const GateArgs& ga, float scale,
                               int32_t use_qk_l2norm, float l2_eps, int32_t h_qk, int32_t h_v, int32_t d_k,
                               int32_t d_v, int32_t n_req, float* state, int32_t n_slots,
                               const int32_t* state_slots, void* o, gdn_dtype o_dt, const void* z,
                               const float* norm_w, float norm_eps, void* stream) {
  if (n_req < 0 || n_slots < 0) return GDN_ERR_INVALID;
  if (n_req == 0) return GDN_OK;
  gdn_status st = check_qkv(q, k, v, q_stride, k_stride, v_stride, dt, ga.rows_missing(), h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  Gates gt;
  st = check_gates(ga, n_req, h_v, gt);
  if (st != GDN_OK) return st;
  if (!state || !o) return GDN_ERR_NULL;
  if (z && !norm_w) return GDN_ERR_NULL;
  if (!dt_valid(o_dt)) return GDN_ERR_UNSUPPORTED;
  if (!((d_k == 128 && d_v == 128) || (d_k == 16 && d_v == 16))) return GDN_ERR_UNSUPPORTED;
  if (!state_slots && n_slots < n_req) return GDN_ERR_INVALID;
  if (!all_aligned({state, o, z, norm_w, state_slots})) return GDN_ERR_ALIGN;
  const int eb = dt_bytes(dt);
  const Range rq{q, strided_bytes(n_req, q_stride, static_cast<int64_t>(h_qk) * d_k, eb)};
  const Range rk{k, strided_bytes(n_req, k_stride, static_cast<int64_t>(h_qk) * d_k, eb)};
  const Range rv{v, strided_bytes(n_req, v_stride, static_cast<int64_t>(h_v) * d_v, eb)};
  const Range rs{state, static_cast<uint64_t>(n_slots) * h_v * d_v * d_k * 4};
  const Range ro{o, static_cast<uint64_t>(n_req) * h_v * d_v * dt_bytes(o_dt)};
  const Range rz{z, z ? static_cast<uint64_t>(n_req) * h_v * d_v * eb : 0};
  const Range rw{norm_w, z ? static_cast<uint64_t>(d_v) * 4 : 0};
  const Range rsl{state_slots, state_slots ? static_cast<uint64_t>(n_req) * 4 : 0};
  if (!disjoint(ro, {rq, rk, rv, rs, rz, rw, rsl}) || !disjoint_gates(ro, gt)) return GDN_ERR_ALIAS;
  if (!disjoint(rs, {rq, rk, rv, rz, rw, rsl}) || !disjoint_gates(rs, gt)) return GDN_ERR_ALIAS;

  gdn::StepArgs a;
  a.q = q; a.k = k; a.v = v;
  a.q_stride = q_stride; a.k_stride = k_stride; a.v_stride = v_stride;
  a.dt = dt; a.gate = gt.src; a.scale = scale;
  a.use_l2 = use_qk_l2norm != 0; a.l2_eps = l2_eps;
  a.h_qk = h_qk; a.h_v = h_v; a.d = d_k; a.n_req = n_req;
  a.state = state; a.slots = state_slots;
  a.o = o; a.o_dt = o_dt; a.z = z; a.norm_w = norm_w; a.norm_eps = norm_eps;
  a.stream = stream;
  return finish(gdn::launch_recurrent_step(a));
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v, int64_t q_stride, int64_t k_stride,
                         int64_t v_stride, gdn_dtype dt, const float* g, const float* beta, float scale,
                         int32_t use_qk_l2norm, float l2_eps, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                         int32_t chunk, const int32_t* cu_seqlens, int32_t n_seq, int64_t t_total,
                         const float* initial_state, float* final_state, void* o, gdn_dtype o_dt, const void* z,
                         const float* norm_w, float norm_eps, void* workspace, size_t ws_bytes, void* stream) {
  return chunk_fwd_impl(q, k, v, q_stride, k_stride, v_stride, dt, plain_gates(g, beta), scale, use_qk_l2norm,
                        l2_eps, h_qk, h_v, d_k, d_v, chunk, cu_seqlens, n_seq, t_total, initial_state,
                        final_state, o, o_dt, z, norm_w, norm_eps, workspace, ws_bytes, stream);
}

gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, int64_t q_stride, int64_t k_stride,
                                 int64_t v_stride, gdn_dtype dt, const float* g, const float* beta, float scale,
                                 int32_t use_qk_l2norm, float l2_eps, int32_t h_qk, int32_t h_v, int32_t d_k,
                                 int32_t d_v, int32_t chunk, const int32_t* cu_seqlens, int32_t n_seq,
                                 int64_t t_total, const float* initial_state, float* final_state, void* o,
                                 gdn_dtype o_dt, const void* z, const float* norm_w, float norm_eps, void* stream) {
  if (n_seq < 0 || t_total < 0) return GDN_ERR_INVALID;
  if (n_seq == 0) return GDN_OK;
  size_t need = 0;
  gdn_status st = gdn_chunk_fwd_workspace_size(h_qk, h_v, d_k, d_v, chunk, n_seq, t_total, dt, z != nullptr, &need);
  if (st != GDN_OK) return st;
  if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return GDN_ERR_HIP;
  // no side stream: this entry creates nothing
  return chunk_fwd_impl(q, k, v, q_stride, k_stride, v_stride, dt, plain_gates(g, beta), scale, use_qk_l2norm,
                        l2_eps, h_qk, h_v, d_k, d_v, chunk, cu_seqlens, n_seq, t_total, initial_state,
                        final_state, o, o_dt, z, norm_w, norm_eps, ws, GDN_NOALLOC_SCRATCH_BYTES, stream,
                        nullptr, nullptr, 0, false);
}

gdn_status gdn_chunk_fwd_gated(const void* q, const void* k, const void* v, int64_t q_stride, int64_t k_stride,
                               int64_t v_stride, gdn_dtype dt, const void* a, const void* b, int64_t ab_stride,
                               gdn_dtype ab_dt, const float* a_log, const float* dt_bias, float scale,
                               int32_t use_qk_l2norm, float l2_eps, int32_t h_qk, int32_t h_v, int32_t d_k,
                               int32_t d_v, int32_t chunk, const int32_t* cu_seqlens, int32_t n_seq,
                               int64_t t_total, const float* initial_state, float* final_state, void* o,
                               gdn_dtype o_dt, const void* z, const float* norm_w, float norm_eps, void* workspace,
                               size_t ws_bytes, void* stream) {
  return chunk_fwd_impl(q, k, v, q_stride, k_stride, v_stride, dt, raw_gates(a, b, ab_stride, ab_dt, a_log, dt_bias),
                        scale, use_qk_l2norm, l2_eps, h_qk, h_v, d_k, d_v, chunk, cu_seqlens, n_seq, t_total,
                        initial_state, final_state, o, o_dt, z, norm_w, norm_eps, workspace, ws_bytes, stream);
}

gdn_status gdn_recurrent_step(const void* q, const void* k, const void* v, int64_t q_stride, int64_t k_stride,
                              int64_t v_stride, gdn_dtype dt, const float* g, const float* beta, float scale,
                              int32_t use_qk_l2norm, float l2_eps, int32_t h_qk, int32_t h_v, int32_t d_k,
                              int32_t d_v, int32_t n_req, float* state, int32_t n_slots,
                              const int32_t* state_slots, void* o, gdn_dtype o_dt, const void* z,
                              const float* norm_w, float norm_eps, void* stream) {
  return recurrent_step_impl(q, k, v, q_stride, k_stride, v_stride, dt, plain_gates(g, beta), scale, use_qk_l2norm,
                             l2_eps, h_qk, h_v, d_k, d_v, n_req, state, n_slots, state_slots, o, o_dt, z, norm_w,
                             norm_eps, stream);
}

gdn_status gdn_recurrent_step_gated(const void* q, const void* k, const void* v, int64_t q_stride,
                                    int64_t k_stride, int64_t v_stride, gdn_dtype dt, const void* a, const void* b,
                                    int64_t ab_stride, gdn_dtype ab_dt, const float* a_log, const float* dt_bias,
                                    float scale, int32_t use_qk_l2norm, float l2_eps, int32_t h_qk, int32_t h_v,
                                    int32_t d_k, int32_t d_v, int32_t n_req, float* state, int32_t n_slots,
                                    const int32_t* state_slots, void* o, gdn_dtype o_dt, const void* z,
                                    const float* norm_w, float norm_eps, void* stream) {
  return recurrent_step_impl(q, k, v, q_stride, k_stride, v_stride, dt,
                             raw_gates(a, b, ab_stride, ab_dt, a_log, dt_bias), scale, use_qk_l2norm, l2_eps, h_qk,
                             h_v, d_k, d_v, n_req, state, n_slots, state_slots, o, o_dt, z, norm_w, norm_eps, stream);
}

gdn_status gdn_recurrent_verify(const void* q, const void* k, const void* v, int64_t q_stride, int64_t k_stride,
                                int64_t v_stride, gdn_dtype dt, const float* g, const float* beta, float scale,
                                int32_t use_qk_l2norm, float l2_eps, int32_t h_qk, int32_t h_v, int32_t d_k,
                                int32_t d_v, int32_t n_req, int32_t n_tok, const float* state, int32_t n_slots,
                                const int32_t* state_slots, float* checkpoints, int32_t n_cols, void* o,
                                gdn_dtype o_dt, const void* z, const float* norm_w, float norm_eps, void* stream) {
  if (n_req < 0 || n_slots < 0) return GDN_ERR_INVALID;
  if (n_req == 0) return GDN_OK;
  if (n_tok < 1 || n_cols < n_tok) return GDN_ERR_INVALID;
  const GateArgs ga = plain_gates(g, beta);
  gdn_status st = check_qkv(q, k, v, q_stride, k_stride, v_stride, dt, ga.rows_missing(), h_qk, h_v, d_k, d_v);
  if (st != GDN_OK) return st;
  const int64_t rows = static_cast<int64_t>(n_req) * n_tok;
  Gates gt;
  st = check_gates(ga, rows, h_v, gt);
  if (st != GDN_OK) return st;
  if (!state || !checkpoints || !o) return GDN_ERR_NULL;
  if (z && !norm_w) return GDN_ERR_NULL;
  if (!dt_valid(o_dt)) return GDN_ERR_UNSUPPORTED;
  if (!((d_k == 128 && d_v == 128) || (d_k == 16 && d_v == 16))) return GDN_ERR_UNSUPPORTED;
  if (!state_slots && n_slots < n_req) return GDN_ERR_INVALID;
  if (!all_aligned({state, checkpoints, o, z, norm_w, state_slots})) return GDN_ERR_ALIGN;
  const int eb = dt_bytes(dt);
  const uint64_t slot_bytes = static_cast<uint64_t>(h_v) * d_v * d_k * 4;
  const Range rq{q, strided_bytes(rows, q_stride, static_cast<int64_t>(h_qk) * d_k, eb)};
  const Range rk{k, strided_bytes(rows, k_stride, static_cast<int64_t>(h_qk) * d_k, eb)};
  const Range rv{v, strided_bytes(rows, v_stride, static_cast<int64_t>(h_v) * d_v, eb)};
  const Range rs{state, static_cast<uint64_t>(n_slots) * slot_bytes};
  const Range rc{checkpoints, static_cast<uint64_t>(n_slots) * n_cols * slot_bytes};
  const Range ro{o, static_cast<uint64_t>(rows) * h_v * d_v * dt_bytes(o_dt)};
  const Range rz{z, z ? static_cast<uint64_t>(rows) * h_v * d_v * eb : 0};
  const Range rw{norm_w, z ? static_cast<uint64_t>(d_v) * 4 : 0};
  const Range rsl{state_slots, state_slots ? static_cast<uint64_t>(n_req) * 4 : 0};
  if (!disjoint(ro, {rq, rk, rv, rs, rc, rz, rw, rsl}) || !disjoint_gates(ro, gt)) return GDN_ERR_ALIAS;
  if (!disjoint(rc, {rq, rk, rv, rs, rz, rw, rsl}) || !disjoint_gates(rc, gt)) return GDN_ERR_ALIAS;

  gdn::VerifyArgs a;
  a.q = q; a.k = k; a.v = v;
  a.q_stride = q_stride; a.k_stride = k_stride; a.v_stride = v_stride;
  a.dt = dt; a.gate = gt.src; a.scale = scale;
  a.use_l2 = use_qk_l2norm != 0; a.l2_eps = l2_eps;
  a.h_qk = h_qk; a.h_v = h_v; a.d = d_k; a.n_req = n_req; a.n_tok = n_tok;
  a.state = state; a.slots = state_slots; a.ckpt = checkpoints; a.n_cols = n_cols;
  a.o = o; a.o_dt = o_dt; a.z = z; a.norm_w = norm_w; a.norm_eps = norm_eps;
  a.stream = stream;
  return finish(gdn::launch_recurrent_verify(a));
}

gdn_status gdn_conv1d_verify(const void* x, gdn_dtype dt, const void* w, int32_t channels, int32_t n_req,
                             int32_t n_tok, const void* conv_state, int32_t n_slots, const int32_t* state_slots,
                             void* y, void* windows, int32_t n_cols, void* stream) {
  if (n_req < 0 || channels <= 0 || n_slots < 0) return GDN_ERR_INVALID;
  if (!dt_valid(dt)) return GDN_ERR_UNSUPPORTED;
  if (channels % 8) return GDN_ERR_INVALID;
  if (n_req == 0) return GDN_OK;
  if (n_tok < 1 || n_cols < n_tok) return GDN_ERR_INVALID;
  if (!x || !w || !conv_state || !y || !windows) return GDN_ERR_NULL;
  if (!state_slots && n_slots < n_req) return GDN_ERR_INVALID;
  if (!all_aligned({x, w, conv_state, y, windows, state_slots})) return GDN_ERR_ALIGN;
  const int eb = dt_bytes(dt);
  const uint64_t rows = static_cast<uint64_t>(n_req) * n_tok;
  const Range rx{x, rows * channels * eb};
  const Range ry{y, rows * channels * eb};
  const Range rw{w, static_cast<uint64_t>(channels) * 4 * eb};
  const Range rs{conv_state, static_cast<uint64_t>(n_slots) * 3 * channels * eb};
  const Range rwin{windows, static_cast<uint64_t>(n_slots) * n_cols * 3 * channels * eb};
  const Range rsl{state_slots, state_slots ? static_cast<uint64_t>(n_req) * 4 : 0};
  if (!disjoint(ry, {rx, rw, rs, rwin, rsl}) || !disjoint(rwin, {rx, rw, rs, rsl})) return GDN_ERR_ALIAS;
  return finish(gdn::launch_conv1d_verify(x, dt, w, channels, n_req, n_tok, conv_state, state_slots, y, windows,
                                          n_cols, stream));
}

gdn_status gdn_state_rows_copy(void* dst, int64_t n_dst_rows, const int32_t* dst_rows, const void* src,
                               int64_t n_src_rows, const int32_t* src_rows, int64_t row_bytes, int32_t n,
                               void* stream) {
  if (n < 0 || n_dst_rows < 0 || n_src_rows < 0 || row_bytes <= 0) return GDN_ERR_INVALID;
  if (n == 0) return GDN_OK;
  if (!dst || !dst_rows) return GDN_ERR_NULL;
  if (src && !src_rows) return GDN_ERR_NULL;
  if (row_bytes % 16) return GDN_ERR_ALIGN;
  if (!all_aligned({dst, dst_rows, src, src_rows})) return GDN_ERR_ALIGN;
  // one workgroup per 16 KiB of each entry's row: the grid must stay below 2^31
  const int64_t chunks = (row_bytes / 16 + 1023) / 1024;
  if (chunks > (int64_t(1) << 31) / n) return GDN_ERR_INVALID;
  const Range rd{dst, static_cast<uint64_t>(n_dst_rows) * row_bytes};
  const Range rsrc{src, src ? static_cast<uint64_t>(n_src_rows) * row_bytes : 0};
  const Range rdi{dst_rows, static_cast<uint64_t>(n) * 4};
  const Range rsi{src_rows, src ? static_cast<uint64_t>(n) * 4 : 0};
  if (!disjoint(rd, {rdi, rsi})) return GDN_ERR_ALIAS;
  if (src && src != dst && overlap(rd, rsrc)) return GDN_ERR_ALIAS;
  return finish(gdn::launch_rows_copy(dst, n_dst_rows, dst_rows, src, n_src_rows, src_rows, row_bytes, n, stream));
}

gdn_status gdn_conv1d_mixed(const void* x, gdn_dtype dt, const void* w, int32_t channels, const int32_t* cu_seqlens,
                            int32_t n_seq, int64_t t_total, void* conv_state, int32_t n_slots,
                            const int32_t* state_slots, const int32_t* fresh, void* y, void* stream) {
  if (n_seq < 0 || t_total < 0 || channels <= 0 || n_slots < 0) return GDN_ERR_INVALID;
  if (!dt_valid(dt)) return GDN_ERR_UNSUPPORTED;
  if (channels % 8) return GDN_ERR_INVALID;
  if (n_seq == 0) return GDN_OK;
  if (!cu_seqlens || !state_slots || !w || !conv_state) return GDN_ERR_NULL;
  if (t_total > 0 && (!x || !y)) return GDN_ERR_NULL;
  if (!all_aligned({x, w, conv_state, y, cu_seqlens, state_slots, fresh})) return GDN_ERR_ALIGN;
  const int eb = dt_bytes(dt);
  const Range rx{x, static_cast<uint64_t>(t_total) * channels * eb};
  const Range ry{y, static_cast<uint64_t>(t_total) * channels * eb};
  const Range rw{w, static_cast<uint64_t>(channels) * 4 * eb};
  const Range rs{conv_state, static_cast<uint64_t>(n_slots) * 3 * channels * eb};
  const Range rcu{cu_seqlens, static_cast<uint64_t>(n_seq + 1) * 4};
  const Range rsl{state_slots, static_cast<uint64_t>(n_seq) * 4};
  const Range rfr{fresh, fresh ? static_cast<uint64_t>(n_seq) * 4 : 0};
  if (!disjoint(ry, {rx, rw, rs, rcu, rsl, rfr}) || !disjoint(rs, {rx, rw, rcu, rsl, rfr})) return GDN_ERR_ALIAS;
  return finish(gdn::launch_conv1d(x, dt, w, channels, cu_seqlens, n_seq, t_total, conv_state, state_slots, y,
                                   stream, fresh));
}

gdn_status gdn_chunk_mixed(const void* q, const void* k, const void* v, int64_t q_stride, int64_t k_stride,
                           int64_t v_stride, gdn_dtype dt, const float* g, const float* beta, float scale,
                           int32_t use_qk_l2norm, float l2_eps, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                           int32_t chunk, const int32_t* cu_seqlens, int32_t n_seq, int64_t t_total, float* state,
                           int32_t n_slots, const int32_t* state_slots, const int32_t* fresh, void* o,
                           gdn_dtype o_dt, const void* z, const float* norm_w, float norm_eps, void* workspace,
                           size_t ws_bytes, void* stream) {
  if (n_seq < 0 || t_total < 0 || n_slots < 0) return GDN_ERR_INVALID;
  if (n_seq == 0) return GDN_OK;
  if (!cu_seqlens || !state_slots || !state) return GDN_ERR_NULL;
  return chunk_fwd_impl(q, k, v, q_stride, k_stride, v_stride, dt, plain_gates(g, beta), scale, use_qk_l2norm,
                        l2_eps, h_qk, h_v, d_k, d_v, chunk, cu_seqlens, n_seq, t_total, state, state, o, o_dt, z,
                        norm_w, norm_eps, workspace, ws_bytes, stream, state_slots, fresh, n_slots);
}

gdn_status gdn_chunk_bwd_workspace_size(int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, int32_t n_seq,
                                        int64_t t_total, size_t* bytes) {
  if (!bytes) return GDN_ERR_NULL;
  if (h_qk <= 0 || h_v <= 0 || h_v % h_qk != 0 || n_seq < 0 || t_total < 0) return GDN_ERR_INVALID;
  if (!((d_k == 128 && d_v == 128) || (d_k == 16 && d_v == 16))) return GDN_ERR_UNSUPPORTED;
  *bytes = gdn::bwd_ws_bytes(h_v, d_v, n_seq, t_total);
  return GDN_OK;
}

gdn_status gdn_chunk_bwd(const void* q, const void* k, const void* v, int64_t q_stride, int64_t k_stride,
                         int64_t v_stride, gdn_dtype dt, const float* g, const float* beta, float scale,
                         int32_t use_qk_l2norm, float l2_eps, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                         const int32_t* cu_seqlens, int32_t n_seq, int64_t t_total, const float* initial_state,
                         const float* d_o, const float* d_final, float* dq, float* dk, float* dv, float* dg,
                         float* dbeta, float* d_initial, void* workspace, size_t ws_bytes, void* stream) {
  if (n_seq < 0 || t_total < 0) return GDN_ERR_INVALID;
  if (n_seq == 0) return GDN_OK;
  if (!dt_valid(dt)) return GDN_ERR_UNSUPPORTED;
  if (dt == GDN_BF16 && d_k != 128) return GDN_ERR_UNSUPPORTED;
  gdn_status st = check_qkv(q, k, v, q_stride, k_stride, v_stride, dt, !g || !beta, h_qk, h_v, d_k, d_v,
                            t_total > 0);
  if (st != GDN_OK) return st;
  Gates gt;
  st = check_gates(plain_gates(g, beta), t_total, h_v, gt);
  if (st != GDN_OK) return st;
  if (t_total > 0 && (!d_o || !dq || !dk || !dv || !dg || !dbeta)) return GDN_ERR_NULL;
  if (!cu_seqlens && n_seq != 1) return GDN_ERR_NULL;
  if (!workspace) return GDN_ERR_WORKSPACE;
  size_t need = 0;
  st = gdn_chunk_bwd_workspace_size(h_qk, h_v, d_k, d_v, n_seq, t_total, &need);
  if (st != GDN_OK) return st;
  if (ws_bytes < need) return GDN_ERR_WORKSPACE;
  if (!all_aligned({initial_state, d_o, d_final, dq, dk, dv, dg, dbeta, d_initial, workspace, cu_seqlens}))
    return GDN_ERR_ALIGN;
  const int eb = dt_bytes(dt);
  const uint64_t state_bytes = static_cast<uint64_t>(n_seq) * h_v * d_v * d_k * 4;
  const Range rq{q, strided_bytes(t_total, q_stride, static_cast<int64_t>(h_qk) * d_k, eb)};
  const Range rk{k, strided_bytes(t_total, k_stride, static_cast<int64_t>(h_qk) * d_k, eb)};
  const Range rv{v, strided_bytes(t_total, v_stride, static_cast<int64_t>(h_v) * d_v, eb)};
  const Range ri{initial_state, initial_state ? state_bytes : 0};
  const Range rdo{d_o, static_cast<uint64_t>(t_total) * h_v * d_v * 4};
  const Range rdf{d_final, d_final ? state_bytes : 0};
  const Range rcu{cu_seqlens, cu_seqlens ? static_cast<uint64_t>(n_seq + 1) * 4 : 0};
  const Range rws{workspace, need};
  const Range outs[] = {{dq, static_cast<uint64_t>(t_total) * h_qk * d_k * 4},
                        {dk, static_cast<uint64_t>(t_total) * h_qk * d_k * 4},
                        {dv, static_cast<uint64_t>(t_total) * h_v * d_v * 4},
                        {dg, static_cast<uint64_t>(t_total) * h_v * 4},
                        {dbeta, static_cast<uint64_t>(t_total) * h_v * 4},
                        {d_initial, d_initial ? state_bytes : 0},
                        rws};
  for (const Range& o : outs) {
    if (!disjoint(o, {rq, rk, rv, ri, rdo, rdf, rcu}) || !disjoint_gates(o, gt)) return GDN_ERR_ALIAS;
    for (const Range& o2 : outs)
      if (&o != &o2 && overlap(o, o2)) return GDN_ERR_ALIAS;
  }
  gdn::BwdArgs a;
  a.q = q; a.k = k; a.v = v;
  a.q_stride = q_stride; a.k_stride = k_stride; a.v_stride = v_stride;
  a.dt = dt; a.gate = gt.src; a.scale = scale;
  a.use_l2 = use_qk_l2norm != 0; a.l2_eps = l2_eps;
  a.h_qk = h_qk; a.h_v = h_v; a.d = d_k;
  a.cu = cu_seqlens; a.n_seq = n_seq; a.t_total = t_total;
  a.init = initial_state; a.d_o = d_o; a.d_final = d_final;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.d_init = d_initial;
  a.workspace = workspace; a.stream = stream;
  return finish(gdn::launch_chunk_bwd(a));
}

gdn_status gdn_conv1d_bwd_workspace_size(int32_t channels, int32_t n_seq, int64_t t_total, size_t* bytes) {
  if (!bytes) return GDN_ERR_NULL;
  if (channels <= 0 || channels % 8 || n_seq < 0 || t_total < 0) return GDN_ERR_INVALID;
  *bytes = gdn::conv_bwd_ws_bytes(channels, n_seq, t_total);
  return GDN_OK;
}

gdn_status gdn_conv1d_bwd(const void* x, gdn_dtype dt, const void* w, int32_t channels, const int32_t* cu_seqlens,
                          int32_t n_seq, int64_t t_total, const void* conv_state_in, const float* dy,
                          const float* d_state_out, float* dx, float* dw, float* d_state_in, void* workspace,
                          size_t ws_bytes, void* stream) {
  if (n_seq < 0 || t_total < 0 || channels <= 0) return GDN_ERR_INVALID;
  if (!dt_valid(dt)) return GDN_ERR_UNSUPPORTED;
  if (channels % 8) return GDN_ERR_INVALID;
  if (n_seq == 0) return GDN_OK;
  if (!w || !dw) return GDN_ERR_NULL;
  if (t_total > 0 && (!x || !dy || !dx)) return GDN_ERR_NULL;
  if (!cu_seqlens && n_seq != 1) return GDN_ERR_NULL;
  if (!workspace) return GDN_ERR_WORKSPACE;
  size_t need = 0;
  gdn_status st = gdn_conv1d_bwd_workspace_size(channels, n_seq, t_total, &need);
  if (st != GDN_OK) return st;
  if (ws_bytes < need) return GDN_ERR_WORKSPACE;
  if (!all_aligned({x, w, conv_state_in, dy, d_state_out, dx, dw, d_state_in, workspace, cu_seqlens}))
    return GDN_ERR_ALIGN;
  const int eb = dt_bytes(dt);
  const uint64_t rows = static_cast<uint64_t>(t_total) * channels;
  const uint64_t hist = static_cast<uint64_t>(n_seq) * 3 * channels;
  const Range rx{x, rows * eb}, rw{w, static_cast<uint64_t>(channels) * 4 * eb};
  const Range rh{conv_state_in, conv_state_in ? hist * eb : 0};
  const Range rdy{dy, rows * 4}, rdh{d_state_out, d_state_out ? hist * 4 : 0};
  const Range rcu{cu_seqlens, cu_seqlens ? static_cast<uint64_t>(n_seq + 1) * 4 : 0};
  const Range outs[] = {{dx, rows * 4}, {dw, static_cast<uint64_t>(channels) * 4 * 4},
                        {d_state_in, d_state_in ? hist * 4 : 0}, {workspace, need}};
  for (const Range& o : outs) {
    if (!disjoint(o, {rx, rw, rh, rdy, rdh, rcu})) return GDN_ERR_ALIAS;
    for (const Range& o2 : outs)
      if (&o != &o2 && overlap(o, o2)) return GDN_ERR_ALIAS;
  }
  gdn::ConvBwdArgs a;
  a.x = x; a.dt = dt; a.w = w; a.channels = channels;
  a.cu = cu_seqlens; a.n_seq = n_seq; a.t_total = t_total;
  a.hist = conv_state_in; a.dy = dy; a.dhist_out = d_state_out;
  a.dx = dx; a.dw = dw; a.dhist_in = d_state_in;
  a.workspace = workspace; a.stream = stream;
  return finish(gdn::launch_conv1d_bwd(a));
}

gdn_status gdn_mixer_decode_step(const void* x, gdn_dtype dt, const void* conv_w, void* conv_state,
                                 const float* g, const float* beta, float scale, int32_t use_qk_l2norm, float l2_eps,
                                 int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, int32_t n_req, float* state,
                                 int32_t n_slots, const int32_t* state_slots, void* o, gdn_dtype o_dt, const void* z,
                                 const float* norm_w, float norm_eps, void* stream) {
  if (n_req < 0 || n_slots < 0) return GDN_ERR_INVALID;
  if (n_req == 0) return GDN_OK;
  if (!dt_valid(dt) || !dt_valid(o_dt)) return GDN_ERR_UNSUPPORTED;
  if (h_qk <= 0 || h_v <= 0 || h_v % h_qk != 0) return GDN_ERR_INVALID;
  if (d_k != 128 || d_v != 128 || h_v / h_qk > gdn::kMixerDecodeMaxGroup) return GDN_ERR_UNSUPPORTED;
  if (!x || !conv_w || !conv_state || !g || !beta || !state || !o) return GDN_ERR_NULL;
  if (z && !norm_w) return GDN_ERR_NULL;
  if (!state_slots && n_slots < n_req) return GDN_ERR_INVALID;
  if (!all_aligned({x, conv_w, conv_state, g, beta, state, state_slots, o, z, norm_w})) return GDN_ERR_ALIGN;
  const int eb = dt_bytes(dt);
  const int64_t ch = 2 * static_cast<int64_t>(h_qk) * d_k + static_cast<int64_t>(h_v) * d_v;
  const Range rx{x, static_cast<uint64_t>(n_req) * ch * eb};
  const Range rw{conv_w, static_cast<uint64_t>(ch) * 4 * eb};
  const Range rh{conv_state, static_cast<uint64_t>(n_slots) * 3 * ch * eb};
  const Range rs{state, static_cast<uint64_t>(n_slots) * h_v * d_v * d_k * 4};
  const Range rg{g, static_cast<uint64_t>(n_req) * h_v * 4}, rb{beta, static_cast<uint64_t>(n_req) * h_v * 4};
  const Range ro{o, static_cast<uint64_t>(n_req) * h_v * d_v * dt_bytes(o_dt)};
  const Range rz{z, z ? static_cast<uint64_t>(n_req) * h_v * d_v * eb : 0};
  const Range rnw{norm_w, z ? static_cast<uint64_t>(d_v) * 4 : 0};
  const Range rsl{state_slots, state_slots ? static_cast<uint64_t>(n_req) * 4 : 0};
  if (!disjoint(ro, {rx, rw, rh, rs, rg, rb, rz, rnw, rsl})) return GDN_ERR_ALIAS;
  if (!disjoint(rh, {rx, rw, rs, rg, rb, rz, rnw, rsl})) return GDN_ERR_ALIAS;
  if (!disjoint(rs, {rx, rw, rg, rb, rz, rnw, rsl})) return GDN_ERR_ALIAS;
  gdn::MixerDecodeArgs a;
  a.x = x; a.dt = dt; a.w = conv_w; a.conv_state = conv_state;
  a.gate = gdn::GateSrc{g, beta, nullptr, nullptr, 0, 0, nullptr, nullptr};
  a.scale = scale; a.use_l2 = use_qk_l2norm != 0; a.l2_eps = l2_eps;
  a.h_qk = h_qk; a.h_v = h_v; a.n_req = n_req;
  a.state = state; a.slots = state_slots;
  a.o = o; a.o_dt = o_dt; a.z = z; a.norm_w = norm_w; a.norm_eps = norm_eps;
  a.stream = stream;
  return finish(gdn::launch_mixer_decode(a));
}

gdn_status gdn_gated_rmsnorm(const void* x, gdn_dtype x_dt, const void* z, gdn_dtype z_dt, const float* w, float eps,
                             int64_t rows, int32_t d, void* y, gdn_dtype y_dt, void* stream) {
  if (rows < 0) return GDN_ERR_INVALID;
  if (!dt_valid(x_dt) || !dt_valid(z_dt) || !dt_valid(y_dt)) return GDN_ERR_UNSUPPORTED;
  if (d != 16 && d != 128) return GDN_ERR_UNSUPPORTED;
  if (rows == 0) return GDN_OK;
  if (!x || !z || !w || !y) return GDN_ERR_NULL;
  if (!all_aligned({x, z, w, y})) return GDN_ERR_ALIGN;
  const Range rx{x, static_cast<uint64_t>(rows) * d * dt_bytes(x_dt)};
  const Range rz{z, static_cast<uint64_t>(rows) * d * dt_bytes(z_dt)};
  const Range rw{w, static_cast<uint64_t>(d) * 4};
  const Range ry{y, static_cast<uint64_t>(rows) * d * dt_bytes(y_dt)};
  const bool in_place = (y == x && y_dt == x_dt);
  if (!in_place && overlap(ry, rx)) return GDN_ERR_ALIAS;
  if (!disjoint(ry, {rz, rw})) return GDN_ERR_ALIAS;
  return finish(gdn::launch_gated_rmsnorm(x, x_dt, z, z_dt, w, eps, rows, d, y, y_dt, stream));
}

}  // extern "C"
