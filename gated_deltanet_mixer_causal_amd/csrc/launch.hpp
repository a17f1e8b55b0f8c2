// Internal launchers behind the C ABI (host side).  Arguments reaching these
// functions have been validated by the API layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdn.h"
#include "common.hpp"

namespace gdn {

struct ChunkArgs {
  const void *q, *k, *v;
  int64_t q_stride, k_stride, v_stride;
  gdn_dtype dt;
  GateSrc gate;   // g and beta, or the raw gate projections
  float scale;
  int use_l2;
  float l2_eps;
  int h_qk, h_v, d, chunk;
  const int32_t* cu;
  int n_seq;
  int64_t t_total;
  const float* init;
  float* fin;
  const int32_t* slots;   // state row per sequence (NULL = identity); negative = inactive lane
  const int32_t* fresh;   // per sequence: nonzero = start from the zero state (NULL = none)
  void* o;
  gdn_dtype o_dt;
  const void* z;
  const float* norm_w;
  float norm_eps;
  void* workspace;
  void* stream;
  bool side_ok = true;   // the one-token sequences may run on the library's side stream (not for the no-alloc entry)
};

struct StepArgs {
  const void *q, *k, *v;
  int64_t q_stride, k_stride, v_stride;
  gdn_dtype dt;
  GateSrc gate;   // g and beta, or the raw gate projections
  float scale;
  int use_l2;
  float l2_eps;
  int h_qk, h_v, d, n_req;
  float* state;
  const int32_t* slots;
  void* o;
  gdn_dtype o_dt;
  const void* z;
  const float* norm_w;
  float norm_eps;
  void* stream;
};

// Speculative verification of n_tok tokens per request (checkpoint columns).
struct VerifyArgs {
  const void *q, *k, *v;
  int64_t q_stride, k_stride, v_stride;
  gdn_dtype dt;
  GateSrc gate;
  float scale;
  int use_l2;
  float l2_eps;
  int h_qk, h_v, d, n_req, n_tok;
  const float* state;
  const int32_t* slots;
  float* ckpt;
  int n_cols;
  void* o;
  gdn_dtype o_dt;
  const void* z;
  const float* norm_w;
  float norm_eps;
  void* stream;
};

// Backward of the gated delta rule over packed sequences.
struct BwdArgs {
  const void *q, *k, *v;
  int64_t q_stride, k_stride, v_stride;
  gdn_dtype dt;
  GateSrc gate;
  float scale;
  int use_l2;
  float l2_eps;
  int h_qk, h_v, d;
  const int32_t* cu;
  int n_seq;
  int64_t t_total;
  const float* init;      // [n_seq, h_v, d, d] or NULL (zeros)
  const float* d_o;       // [t_total, h_v, d]
  const float* d_final;   // [n_seq, h_v, d, d] or NULL (zero)
  float *dq, *dk;         // [t_total, h_qk, d]
  float* dv;              // [t_total, h_v, d]
  float *dg, *dbeta;      // [t_total, h_v]
  float* d_init;          // [n_seq, h_v, d, d] or NULL
  void* workspace;
  void* stream;
};

// Backward of the width-4 conv + SiLU over packed sequences.
struct ConvBwdArgs {
  const void* x;
  gdn_dtype dt;
  const void* w;
  int channels;
  const int32_t* cu;
  int n_seq;
  int64_t t_total;
  const void* hist;        // [n_seq, 3, channels] history before the call, or NULL (zeros)
  const float* dy;         // [t_total, channels]
  const float* dhist_out;  // [n_seq, 3, channels] or NULL
  float* dx;               // [t_total, channels]
  float* dw;               // [channels, 4]
  float* dhist_in;         // [n_seq, 3, channels] or NULL
  void* workspace;
  void* stream;
};

// Compute units of the current device (cached per device).
int device_cu_count();

size_t chunk_ws_bytes(gdn_dtype dt, int h_qk, int h_v, int d, int chunk, int n_seq, int64_t t_total,
                      int with_norm);
// Pieces of the chunk path (csrc/chunk.hip).
hipError_t launch_seq_order(const int32_t* cu, int n_seq, int chunk, int32_t* order, hipStream_t st);
// The one-token sequences of a call (outputs to o_pre when a.z is set, else to a.o).
hipError_t launch_single_token(const ChunkArgs& a, float* o_pre, hipStream_t st);
hipError_t launch_chunk_fwd(const ChunkArgs& a);
size_t bwd_ws_bytes(int h_v, int d, int n_seq, int64_t t_total);
hipError_t launch_chunk_bwd(const BwdArgs& a);
// The chunked backward on the matrix cores (csrc/chunk_bwd.hip): bf16, d = 128.
size_t bwd_chunked_ws_bytes(int h_qk, int h_v, int n_seq, int64_t t_total);
hipError_t launch_chunk_bwd_chunked(const BwdArgs& a);
size_t conv_bwd_ws_bytes(int channels, int n_seq, int64_t t_total);
hipError_t launch_conv1d_bwd(const ConvBwdArgs& a);
hipError_t launch_recurrent_step(const StepArgs& a);
hipError_t launch_recurrent_verify(const VerifyArgs& a);
hipError_t launch_conv1d_verify(const void* x, gdn_dtype dt, const void* w, int channels, int n_seq, int n_tok,
                                const void* state, const int32_t* slots, void* y, void* windows, int n_cols,
                                void* stream);
hipError_t launch_rows_copy(void* dst, int64_t n_dst, const int32_t* dst_rows, const void* src, int64_t n_src,
                            const int32_t* src_rows, int64_t row_bytes, int n, void* stream);
hipError_t launch_conv1d(const void* x, gdn_dtype dt, const void* w, int channels, const int32_t* cu,
                         int n_seq, int64_t t_total, void* state, const int32_t* slots, void* y,
                         void* stream, const int32_t* fresh = nullptr);
// With cu != nullptr, rows are (token, v-head) pairs (h_v per token) of packed
// sequences and only rows of sequences with a non-negative slot are written.
hipError_t launch_gated_rmsnorm(const void* x, gdn_dtype x_dt, const void* z, gdn_dtype z_dt, const float* w,
                                float eps, int64_t rows, int d, void* y, gdn_dtype y_dt, void* stream,
                                const int32_t* cu = nullptr, int n_seq = 0, const int32_t* slots = nullptr,
                                int h_v = 1);

}  // namespace gdn
