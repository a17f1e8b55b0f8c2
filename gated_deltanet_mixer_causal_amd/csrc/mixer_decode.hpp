// Launcher interface of the one-kernel decode mixer step (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn.h"
#include "common.hpp"

namespace gdn {

constexpr int kMixerDecodeMaxGroup = 8;   // v-heads per q/k head

struct MixerDecodeArgs {
  const void* x;          // [n_req, channels] raw projected q|k|v
  gdn_dtype dt;
  const void* w;          // [channels, 4]
  void* conv_state;       // [n_slots, 3, channels]
  GateSrc gate;
  float scale;
  int use_l2;
  float l2_eps;
  int h_qk, h_v, n_req;
  float* state;           // [n_slots, h_v, 128, 128]
  const int32_t* slots;   // [n_req] or NULL (identity); negative = inactive
  void* o;
  gdn_dtype o_dt;
  const void* z;
  const float* norm_w;
  float norm_eps;
  void* stream;
};

hipError_t launch_mixer_decode(const MixerDecodeArgs& a);

}  // namespace gdn
