// Internal launch descriptors shared by the C-ABI layer and the kernels.
// Arguments are validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

struct PrefillLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* sinks;
  const int32_t* cu_seqlens;
  int batch, max_seqlen, num_q_heads, num_kv_heads, window;
  float softmax_scale;
  void* o;
  float* lse;
};

struct DecodeLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* sinks;
  const int32_t* cu_seqlens_k;
  int batch, max_seqlen_k, num_q_heads, num_kv_heads, window, num_splits;
  float softmax_scale;
  void* o;          // bf16 output when num_splits == 1
  float* lse;       // optional, num_splits == 1
  float* o_part;    // fp32 partials when num_splits > 1
  float* lse_part;
};

struct MergeLaunch {
  const float* o_parts;
  const float* lse_parts;
  int num_parts, n, num_heads;
  void* o;
  float* lse;
};

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream);
hipError_t launch_merge(const MergeLaunch& a, hipStream_t stream);

int prefill_max_qtiles();
int prefill_qtile();
int decode_max_group();

}  // namespace sinkattn
