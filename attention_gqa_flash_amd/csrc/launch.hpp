// Internal launch descriptors shared by the C-ABI layer and the kernels.
// Arguments are validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

// Prefill: queries packed by cu_seqlens, keys / values by cu_seqlens_k
// (the same array for self-attention); per sequence the queries are the last
// Lq_b of its Lk_b >= Lq_b tokens (bottom-right causal alignment).
struct PrefillLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* sinks;
  const int32_t* cu_seqlens;
  const int32_t* cu_seqlens_k;
  int batch, max_seqlen, max_seqlen_k, total_tokens, num_q_heads, num_kv_heads, window;
  float softmax_scale;
  void* o;
  float* lse;
  // Paged K/V (block_table non-null): k / v are the page pools and
  // cu_seqlens_k holds the key lengths [batch].
  const int32_t* block_table = nullptr;
  int max_pages = 0, page_shift = 0, num_pages = 0;
  // num_splits > 1: each query tile's keys are cut into that many shares
  // whose fp32 partials [num_splits, total_tokens, num_q_heads, (head_dim)]
  // go to o_part / lse_part, then merged into o and lse.
  int num_splits = 1;
  float* o_part = nullptr;
  float* lse_part = nullptr;
};

struct DecodeLaunch {
  const void* q;
  const void* k;    // bf16, or E4M3 codes when fp8
  const void* v;
  const float* sinks;
  const int32_t* cu_seqlens_k;
  int batch, max_seqlen_k, num_q_heads, num_kv_heads, window, num_splits;
  float softmax_scale;
  void* o;          // bf16 output when num_splits == 1 or merged in the kernel
  float* lse;       // optional, likewise
  float* o_part;    // fp32 partials when num_splits > 1
  float* lse_part;
  bool fp8 = false;       // K/V caches hold E4M3 codes
  float k_scale = 1.0f;   // K = k_scale * e4m3(code)
  float v_scale = 1.0f;   // V = v_scale * e4m3(code)
  // Multi-token-query decode (bf16 cache): sequence b's last
  // cu_seqlens_q[b+1] - cu_seqlens_q[b] <= max_q tokens are queries, rows of
  // q / o / lse / partials indexed by cu_seqlens_q (total_q rows);
  // max_q * group <= 32.
  const int32_t* cu_seqlens_q = nullptr;
  int max_q = 1;
  int total_q = 0;
  // Paged cache (bf16, one token per sequence): k / v are pages
  // [num_pages, 1 << page_shift, num_kv_heads, 64], block_table [batch,
  // max_pages] page ids, and cu_seqlens_k holds the lengths [batch].
  const int32_t* block_table = nullptr;
  int max_pages = 0, page_shift = 0, num_pages = 0;
};

struct MergeLaunch {
  const float* o_parts;
  const float* lse_parts;
  int num_parts, n, num_heads;
  void* o;
  float* lse;
};

// Fused rotary step: frequencies f_i of dimension pairs (i, i + 32) and the
// temperature factor, computed on the host.
struct RopeTable {
  double freq[32];
  float attention_factor;
};

struct RopeLaunch {
  const void* qkv;             // bf16 [num_tokens, num_q_heads + 2 num_kv_heads, 64]
  const int32_t* positions;    // [num_tokens]
  const int32_t* slot_mapping; // [num_tokens], cache row or -1
  int num_tokens, num_q_heads, num_kv_heads, cache_rows;
  RopeTable table;
  void* q_out;                 // bf16 [num_tokens, num_q_heads, 64]
  void* k_cache;               // bf16 [cache_rows, num_kv_heads, 64]
  void* v_cache;
};

// Output projection with bias: y [num_rows, out_features] = o W^T + b,
// o [num_rows, in_features], W [out_features, in_features] (bf16), b fp32.
struct OprojLaunch {
  const void* o;
  const void* w;
  const float* bias;
  int num_rows, in_features, out_features;
  void* y;
  float* part;  // fp32 [splits, num_rows, out_features] when oproj_splits(...) > 1
};
// K ranges one projection launch splits into (1: no partials).
int oproj_splits(int num_rows, int in_features, int out_features);

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream);
hipError_t launch_oproj(const OprojLaunch& a, hipStream_t stream);
hipError_t launch_rope_qkv_append(const RopeLaunch& a, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream);
// True when launch_decode writes o (and lse) itself although num_splits > 1
// (splits of at most 32 keys are evaluated as one range): no merge follows.
bool decode_merges_in_kernel(const DecodeLaunch& a);
hipError_t launch_merge(const MergeLaunch& a, hipStream_t stream);

// Device-side precondition checks (debug mode).  Bits of the flag word:
enum CheckBits : unsigned {
  kCheckOffsetsStart = 1u << 0,  // cu_seqlens[0] != 0
  kCheckOffsetsOrder = 1u << 1,  // cu_seqlens decreasing somewhere
  kCheckLengthMax = 1u << 2,     // a length above the declared maximum
  kCheckLengthMin = 1u << 3,     // a length below the minimum (decode: 1)
  kCheckOffsetsTotal = 1u << 4,  // cu_seqlens[batch] above the declared total
  kCheckSinks = 1u << 5,         // a sink is NaN or +inf
  kCheckQ = 1u << 6,             // NaN / Inf in q
  kCheckK = 1u << 7,             // NaN / Inf in k
  kCheckV = 1u << 8,             // NaN / Inf in v
  kCheckParts = 1u << 9,         // NaN / Inf in o_parts, NaN / +inf in lse_parts
  kCheckAppend = 1u << 10,       // append prefill: a sequence with fewer keys than queries
  kCheckPages = 1u << 11,        // paged decode: a page id outside the pool or a table too short
  kCheckSlots = 1u << 12,        // rotary append: a slot outside [-1, cache_rows) or used twice
  kCheckO = 1u << 13,            // output projection: NaN / Inf in o
  kCheckW = 1u << 14,            // output projection: NaN / Inf in w
  kCheckAll = (1u << 15) - 1u,
};
// Size of the static split-KV scratch of the allocation-free decode (32 MiB:
// the partials of 64 sequences x 64 query heads at 16 splits need 17 MB).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
// Device address of that scratch on `device` (looked up on first use).
hipError_t noalloc_scratch(int device, void** ptr);

hipError_t check_clear(hipStream_t stream);
hipError_t check_offsets(const int32_t* cu, int batch, int max_len, int min_len, int total_limit,
                         hipStream_t stream);
hipError_t check_sinks(const float* sinks, int n, hipStream_t stream);
// Rotary append: every slot in [-1, cache_rows), and no cache row named twice.
hipError_t check_slots(const int32_t* slots, int n, int cache_rows, hipStream_t stream);
// Append prefill: every sequence has cu_k[b+1] - cu_k[b] >= cu_q[b+1] - cu_q[b].
// cu_k holds offsets [batch + 1], or (k_lengths) the lengths [batch].
hipError_t check_append(const int32_t* cu_q, const int32_t* cu_k, bool k_lengths, int batch, hipStream_t stream);
// Paged decode: 1 <= seq_lens[b] <= max_len and every page id a sequence
// uses (the first ceil(L_b / page_size) of its table row) in [0, num_pages).
hipError_t check_paged(const int32_t* seq_lens, const int32_t* block_table, int batch, int max_pages,
                       int page_size, int num_pages, int max_len, hipStream_t stream);
hipError_t check_bf16(const void* x, size_t n, unsigned bit, hipStream_t stream);
// The rows of a page pool that the table and lengths of a paged call reach
// (row_elems elements of elem_bytes bytes each: 2 = bf16, 1 = E4M3).
hipError_t check_paged_values(const void* pool, const int32_t* seq_lens, const int32_t* block_table, int batch,
                              int max_pages, int page_size, int num_pages, int max_len, int row_elems, int elem_bytes,
                              unsigned bit, hipStream_t stream);
// E4M3 codes: NaN (all exponent and mantissa bits set).
hipError_t check_e4m3(const void* x, size_t n, unsigned bit, hipStream_t stream);
hipError_t check_f32(const float* x, size_t n, unsigned bit, bool allow_neg_inf, hipStream_t stream);
// Reads the flag word and cu_seqlens[batch] of the last offsets check;
// synchronises the stream.
hipError_t check_read(unsigned* flags, int* total, hipStream_t stream);

// Workgroups of one prefill launch, and the most one launch can take.
long long prefill_blocks(int batch, int total_tokens, int num_kv_heads, int group);
long long prefill_max_blocks();
int decode_max_group();
// Most (query token, query head) columns one multi-token decode wave serves.
int decode_max_cols();

}  // namespace sinkattn
