// C ABI of the sink-attention library: argument validation, workspace
// sizing, and launches on the caller's stream.  See include/sinkattn.h for
// the contract of every entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "launch.hpp"
#include "sinkattn.h"

namespace {

thread_local std::string g_last_error;

sinkattn_status fail(sinkattn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sinkattn_status ok() {
  g_last_error.clear();
  return SINKATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

sinkattn_status check_heads(int32_t hq, int32_t hkv, int32_t head_dim) {
  if (hq < 1 || hkv < 1) return fail(SINKATTN_ERR_INVALID_ARG, "head counts must be >= 1 (got %d, %d)", hq, hkv);
  if (hq % hkv != 0)
    return fail(SINKATTN_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", hq, hkv);
  if (head_dim != 64) return fail(SINKATTN_ERR_UNSUPPORTED, "head_dim %d is not supported (only 64)", head_dim);
  return SINKATTN_OK;
}

sinkattn_status check_scale(float scale) {
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(SINKATTN_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  return SINKATTN_OK;
}

sinkattn_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SINKATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Debug mode: SINKATTN_DEBUG_CHECKS=1 in the environment (read on every
// call) runs the device-side precondition checks before a launch.
bool debug_checks() {
  const char* v = std::getenv("SINKATTN_DEBUG_CHECKS");
  return v != nullptr && v[0] == '1' && v[1] == '\0';
}

sinkattn_status check_failed(unsigned flags) {
  static const struct {
    unsigned bit;
    const char* what;
  } kNames[] = {
      {sinkattn::kCheckOffsetsStart, "cu_seqlens[0] != 0"},
      {sinkattn::kCheckOffsetsOrder, "cu_seqlens is not non-decreasing"},
      {sinkattn::kCheckLengthMax, "a sequence is longer than the declared maximum"},
      {sinkattn::kCheckLengthMin, "a decode sequence is empty (needs L_b >= 1)"},
      {sinkattn::kCheckOffsetsTotal, "cu_seqlens[batch] exceeds total_tokens"},
      {sinkattn::kCheckSinks, "a sink is NaN or +inf"},
      {sinkattn::kCheckQ, "q holds NaN or Inf"},
      {sinkattn::kCheckK, "k holds NaN or Inf"},
      {sinkattn::kCheckV, "v holds NaN or Inf"},
      {sinkattn::kCheckParts, "o_parts holds NaN or Inf, or lse_parts NaN or +inf"},
      {sinkattn::kCheckAppend, "a sequence has fewer keys than queries (its key length vs cu_seqlens_q)"},
      {sinkattn::kCheckPages, "a page id is outside the pool, or a block table row is too short"},
      {sinkattn::kCheckSlots, "a slot is outside [-1, cache_rows) or names a cache row twice"},
      {sinkattn::kCheckO, "o holds NaN or Inf"},
      {sinkattn::kCheckW, "w holds NaN or Inf"},
  };
  std::string msg = "debug checks failed:";
  for (const auto& n : kNames)
    if (flags & n.bit) (msg += " ") += n.what, msg += ";";
  g_last_error = msg;
  return SINKATTN_ERR_INVALID_ARG;
}

// Runs the queued checks and turns their flags into a status.
sinkattn_status check_result(hipStream_t stream, int* total) {
  unsigned flags = 0;
  int t = 0;
  const hipError_t e = sinkattn::check_read(&flags, &t, stream);
  if (e != hipSuccess) return fail(SINKATTN_ERR_HIP, "debug checks: %s", hipGetErrorString(e));
  if (total != nullptr) *total = t;
  return flags != 0u ? check_failed(flags) : SINKATTN_OK;
}

sinkattn_status hip_queue(hipError_t e) {
  return e == hipSuccess ? SINKATTN_OK : fail(SINKATTN_ERR_HIP, "debug checks: %s", hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* sinkattn_last_error(void) { return g_last_error.c_str(); }

const char* sinkattn_version(void) { return "sinkattn 0.1.0 (gfx950)"; }

// Self-attention prefill (cu_q == cu_k) and append prefill share one kernel.
// Splits of the split-KV append prefill: gridDim.y of its launch.
constexpr int32_t kMaxPrefillSplits = 1024;

static sinkattn_status prefill_common(const void* q, const void* k, const void* v, const float* sinks,
                                      const int32_t* cu_q, const int32_t* cu_k, int32_t batch, int32_t max_q,
                                      int32_t max_k, int32_t total_q, int32_t total_k, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t window, float softmax_scale,
                                      void* o, float* lse, void* stream, const int32_t* block_table = nullptr,
                                      int32_t max_pages = 0, int32_t page_size = 0, int32_t num_pages = 0,
                                      int32_t num_splits = 1, void* workspace = nullptr,
                                      size_t workspace_bytes = 0) {
  const bool append = cu_k != cu_q;
  const bool paged = block_table != nullptr;  // k / v are page pools, cu_k the key lengths [batch]
  sinkattn_status st = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (st != SINKATTN_OK) return st;
  if ((st = check_scale(softmax_scale)) != SINKATTN_OK) return st;
  if (batch == 0 || max_q == 0 || total_q == 0) return ok();
  if (!q || !k || !v || !o || !cu_q || !cu_k)
    return fail(SINKATTN_ERR_INVALID_ARG, "q, k, v, o and the sequence offsets must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SINKATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (max_q > total_q)
    return fail(SINKATTN_ERR_INVALID_ARG, "max_seqlen (%d) exceeds total_tokens (%d)", max_q, total_q);
  if (max_k > total_k)
    return fail(SINKATTN_ERR_INVALID_ARG, "max_seqlen_k (%d) exceeds total_k (%d)", max_k, total_k);
  if (max_k == 0) return fail(SINKATTN_ERR_INVALID_ARG, "queries need keys: max_seqlen_k is 0");
  const int group = num_q_heads / num_kv_heads;
  if (sinkattn::prefill_blocks(batch, total_q, num_kv_heads, group) > sinkattn::prefill_max_blocks())
    return fail(SINKATTN_ERR_UNSUPPORTED, "too many (query tile, head) work items for one launch");
  // K/V rows of one sequence are addressed with 32-bit byte offsets.
  if (static_cast<long long>(max_k) * num_kv_heads * head_dim * 2 >= (1LL << 31))
    return fail(SINKATTN_ERR_UNSUPPORTED, "max_seqlen_k * num_kv_heads * head_dim * 2 must stay below 2^31");
  if (debug_checks()) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t qn = static_cast<size_t>(total_q) * num_q_heads * head_dim;
    const size_t kvn = static_cast<size_t>(total_k) * num_kv_heads * head_dim;
    if ((st = hip_queue(sinkattn::check_clear(s))) != SINKATTN_OK) return st;
    if ((st = hip_queue(sinkattn::check_offsets(cu_q, batch, max_q, 0, total_q, s))) != SINKATTN_OK) return st;
    if (paged) {
      if ((st = hip_queue(sinkattn::check_paged(cu_k, block_table, batch, max_pages, page_size, num_pages, max_k,
                                                s))) != SINKATTN_OK)
        return st;
      if ((st = hip_queue(sinkattn::check_append(cu_q, cu_k, true, batch, s))) != SINKATTN_OK) return st;
    } else if (append) {
      if ((st = hip_queue(sinkattn::check_offsets(cu_k, batch, max_k, 0, total_k, s))) != SINKATTN_OK) return st;
      if ((st = hip_queue(sinkattn::check_append(cu_q, cu_k, false, batch, s))) != SINKATTN_OK) return st;
    }
    if ((st = hip_queue(sinkattn::check_sinks(sinks, num_q_heads, s))) != SINKATTN_OK) return st;
    if ((st = hip_queue(sinkattn::check_bf16(q, qn, sinkattn::kCheckQ, s))) != SINKATTN_OK) return st;
    if (paged) {  // only the pool rows the table and lengths reach
      const int row = num_kv_heads * head_dim;
      if ((st = hip_queue(sinkattn::check_paged_values(k, cu_k, block_table, batch, max_pages, page_size, num_pages,
                                                       max_k, row, 2, sinkattn::kCheckK, s))) != SINKATTN_OK)
        return st;
      if ((st = hip_queue(sinkattn::check_paged_values(v, cu_k, block_table, batch, max_pages, page_size, num_pages,
                                                       max_k, row, 2, sinkattn::kCheckV, s))) != SINKATTN_OK)
        return st;
    } else {
      if ((st = hip_queue(sinkattn::check_bf16(k, kvn, sinkattn::kCheckK, s))) != SINKATTN_OK) return st;
      if ((st = hip_queue(sinkattn::check_bf16(v, kvn, sinkattn::kCheckV, s))) != SINKATTN_OK) return st;
    }
    if ((st = check_result(s, nullptr)) != SINKATTN_OK) return st;
  }
  sinkattn::PrefillLaunch a{q, k, v, sinks, cu_q, cu_k, batch, max_q, max_k, total_q, num_q_heads,
                            num_kv_heads, window, softmax_scale, o, lse};
  if (paged) {
    a.block_table = block_table;
    a.max_pages = max_pages;
    a.num_pages = num_pages;
    while ((1 << a.page_shift) < page_size) ++a.page_shift;
  }
  if (num_splits > 1) {
    const size_t need = sinkattn_decode_workspace_bytes(total_q, num_q_heads, head_dim, num_splits);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(SINKATTN_ERR_WORKSPACE, "workspace of %zu bytes is too small (need %zu)", workspace_bytes, need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(SINKATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const size_t rows = static_cast<size_t>(num_splits) * total_q * num_q_heads;
    char* ws = static_cast<char*>(workspace);
    a.num_splits = num_splits;
    a.o_part = reinterpret_cast<float*>(ws);
    a.lse_part = reinterpret_cast<float*>(ws + round_up(rows * head_dim * sizeof(float), 256));
  }
  return hip_status(sinkattn::launch_prefill(a, static_cast<hipStream_t>(stream)), "prefill launch");
}

sinkattn_status sinkattn_prefill_varlen(const void* q, const void* k, const void* v, const float* sinks,
                                        const int32_t* cu_seqlens, int32_t batch, int32_t max_seqlen,
                                        int32_t total_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t window, float softmax_scale, void* o,
                                        float* lse, void* stream) {
  if (batch < 0 || max_seqlen < 0 || total_tokens < 0)
    return fail(SINKATTN_ERR_INVALID_ARG, "batch, max_seqlen and total_tokens must be >= 0");
  return prefill_common(q, k, v, sinks, cu_seqlens, cu_seqlens, batch, max_seqlen, max_seqlen, total_tokens,
                        total_tokens, num_q_heads, num_kv_heads, head_dim, window, softmax_scale, o, lse, stream);
}

sinkattn_status sinkattn_prefill_append(const void* q, const void* k, const void* v, const float* sinks,
                                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                                        int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t total_q,
                                        int32_t total_k, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t window, float softmax_scale, void* o, float* lse,
                                        void* stream) {
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return fail(SINKATTN_ERR_INVALID_ARG, "batch, lengths and totals must be >= 0");
  if (cu_seqlens_q != nullptr && cu_seqlens_q == cu_seqlens_k && max_seqlen_q == max_seqlen_k &&
      total_q == total_k)
    return sinkattn_prefill_varlen(q, k, v, sinks, cu_seqlens_q, batch, max_seqlen_q, total_q, num_q_heads,
                                   num_kv_heads, head_dim, window, softmax_scale, o, lse, stream);
  if (cu_seqlens_q != nullptr && cu_seqlens_q == cu_seqlens_k)
    return fail(SINKATTN_ERR_INVALID_ARG, "one offsets array for queries and keys needs equal maxima and totals");
  return prefill_common(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k, total_q,
                        total_k, num_q_heads, num_kv_heads, head_dim, window, softmax_scale, o, lse, stream);
}

sinkattn_status sinkattn_prefill_append_splitkv(const void* q, const void* k, const void* v, const float* sinks,
                                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                                int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                                int32_t total_q, int32_t total_k, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim, int32_t window,
                                                float softmax_scale, int32_t num_splits, void* workspace,
                                                size_t workspace_bytes, void* o, float* lse, void* stream) {
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 || total_k < 0)
    return fail(SINKATTN_ERR_INVALID_ARG, "batch, lengths and totals must be >= 0");
  if (num_splits < 1) return fail(SINKATTN_ERR_INVALID_ARG, "num_splits must be >= 1 (got %d)", num_splits);
  if (num_splits > kMaxPrefillSplits)
    return fail(SINKATTN_ERR_UNSUPPORTED, "num_splits must be <= %d (got %d)", kMaxPrefillSplits, num_splits);
  if (cu_seqlens_q != nullptr && cu_seqlens_q == cu_seqlens_k &&
      !(max_seqlen_q == max_seqlen_k && total_q == total_k))
    return fail(SINKATTN_ERR_INVALID_ARG, "one offsets array for queries and keys needs equal maxima and totals");
  return prefill_common(q, k, v, sinks, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k, total_q,
                        total_k, num_q_heads, num_kv_heads, head_dim, window, softmax_scale, o, lse, stream, nullptr,
                        0, 0, 0, num_splits, workspace, workspace_bytes);
}

size_t sinkattn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim, int32_t num_splits) {
  if (batch < 0 || num_q_heads < 0 || head_dim < 0 || num_splits <= 1) return 0;
  const size_t rows = static_cast<size_t>(num_splits) * batch * num_q_heads;
  return round_up(rows * head_dim * sizeof(float), 256) + round_up(rows * sizeof(float), 256);
}

// Decode over a bf16 cache, or (fp8) an E4M3 cache with per-tensor scales.
static sinkattn_status decode_common(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_k,
                                     const float* sinks, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t window, float softmax_scale, int32_t num_splits, void* workspace,
                                     size_t workspace_bytes, void* o, float* lse, void* stream, bool fp8,
                                     float k_scale, float v_scale, const int32_t* cu_seqlens_q = nullptr,
                                     int32_t max_seqlen_q = 1, int32_t total_q = 0,
                                     const int32_t* block_table = nullptr, int32_t max_pages = 0,
                                     int32_t page_size = 0, int32_t num_pages = 0, bool static_scratch = false) {
  const bool multi = cu_seqlens_q != nullptr;
  const bool paged = block_table != nullptr;  // cu_seqlens_k then holds the lengths [batch]
  if (batch < 0 || max_seqlen_k < 0) return fail(SINKATTN_ERR_INVALID_ARG, "batch and max_seqlen_k must be >= 0");
  if (multi && (max_seqlen_q < 0 || total_q < 0))
    return fail(SINKATTN_ERR_INVALID_ARG, "max_seqlen_q and total_q must be >= 0");
  sinkattn_status st = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (st != SINKATTN_OK) return st;
  if ((st = check_scale(softmax_scale)) != SINKATTN_OK) return st;
  if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
    return fail(SINKATTN_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0 (got %g, %g)", k_scale,
                v_scale);
  if (num_splits < 1 || num_splits > 65536)
    return fail(SINKATTN_ERR_INVALID_ARG, "num_splits must be in [1, 65536] (got %d)", num_splits);
  if (num_q_heads / num_kv_heads > sinkattn::decode_max_group())
    return fail(SINKATTN_ERR_UNSUPPORTED, "decode supports at most %d query heads per KV head",
                sinkattn::decode_max_group());
  if (multi && static_cast<long long>(max_seqlen_q) * (num_q_heads / num_kv_heads) > sinkattn::decode_max_cols())
    return fail(SINKATTN_ERR_UNSUPPORTED, "max_seqlen_q * (num_q_heads / num_kv_heads) must be at most %d (got %d * %d)",
                sinkattn::decode_max_cols(), max_seqlen_q, num_q_heads / num_kv_heads);
  if (multi && max_seqlen_q > total_q)
    return fail(SINKATTN_ERR_INVALID_ARG, "max_seqlen_q (%d) exceeds total_q (%d)", max_seqlen_q, total_q);
  if (batch == 0 || (multi && (max_seqlen_q == 0 || total_q == 0))) return ok();
  if (!q || !k_cache || !v_cache || !o || !cu_seqlens_k)
    return fail(SINKATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, o and the sequence offsets / lengths must not be NULL");
  if (max_seqlen_k < 1) return fail(SINKATTN_ERR_INVALID_ARG, "decode needs max_seqlen_k >= 1");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(SINKATTN_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
  const long long blocks = static_cast<long long>(batch) * num_kv_heads * num_splits;
  if (blocks > 0x7fffffffLL) return fail(SINKATTN_ERR_UNSUPPORTED, "too many (batch, head, split) work items");

  if (debug_checks()) {
    // Offsets first: they size the K/V scan.
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = hip_queue(sinkattn::check_clear(s))) != SINKATTN_OK) return st;
    if (multi) {
      if ((st = hip_queue(sinkattn::check_offsets(cu_seqlens_q, batch, max_seqlen_q, 0, total_q, s))) != SINKATTN_OK)
        return st;
      if ((st = hip_queue(sinkattn::check_append(cu_seqlens_q, cu_seqlens_k, paged, batch, s))) != SINKATTN_OK)
        return st;
    }
    if (paged) {
      if ((st = hip_queue(sinkattn::check_paged(cu_seqlens_k, block_table, batch, max_pages, page_size, num_pages,
                                                max_seqlen_k, s))) != SINKATTN_OK)
        return st;
    } else if ((st = hip_queue(sinkattn::check_offsets(cu_seqlens_k, batch, max_seqlen_k, 1, -1, s))) !=
               SINKATTN_OK) {
      return st;
    }
    if ((st = hip_queue(sinkattn::check_sinks(sinks, num_q_heads, s))) != SINKATTN_OK) return st;
    const size_t qn = static_cast<size_t>(multi ? total_q : batch) * num_q_heads * head_dim;
    if ((st = hip_queue(sinkattn::check_bf16(q, qn, sinkattn::kCheckQ, s))) != SINKATTN_OK) return st;
    int total_kv = 0;
    if ((st = check_result(s, &total_kv)) != SINKATTN_OK) return st;
    const size_t kvn = static_cast<size_t>(total_kv) * num_kv_heads * head_dim;
    if (paged) {  // only the pool rows the table and lengths reach
      const int row = num_kv_heads * head_dim, eb = fp8 ? 1 : 2;
      if ((st = hip_queue(sinkattn::check_paged_values(k_cache, cu_seqlens_k, block_table, batch, max_pages, page_size,
                                                       num_pages, max_seqlen_k, row, eb, sinkattn::kCheckK, s))) !=
          SINKATTN_OK)
        return st;
      if ((st = hip_queue(sinkattn::check_paged_values(v_cache, cu_seqlens_k, block_table, batch, max_pages, page_size,
                                                       num_pages, max_seqlen_k, row, eb, sinkattn::kCheckV, s))) !=
          SINKATTN_OK)
        return st;
    } else if (fp8) {
      if ((st = hip_queue(sinkattn::check_e4m3(k_cache, kvn, sinkattn::kCheckK, s))) != SINKATTN_OK) return st;
      if ((st = hip_queue(sinkattn::check_e4m3(v_cache, kvn, sinkattn::kCheckV, s))) != SINKATTN_OK) return st;
    } else {
      if ((st = hip_queue(sinkattn::check_bf16(k_cache, kvn, sinkattn::kCheckK, s))) != SINKATTN_OK) return st;
      if ((st = hip_queue(sinkattn::check_bf16(v_cache, kvn, sinkattn::kCheckV, s))) != SINKATTN_OK) return st;
    }
    if ((st = check_result(s, nullptr)) != SINKATTN_OK) return st;
  }
  sinkattn::DecodeLaunch a{q, k_cache, v_cache, sinks, cu_seqlens_k, batch, max_seqlen_k, num_q_heads, num_kv_heads,
                           window, num_splits, softmax_scale, o, lse, nullptr, nullptr, fp8,
                           fp8 ? k_scale : 1.0f, fp8 ? v_scale : 1.0f, cu_seqlens_q, max_seqlen_q, total_q,
                           block_table, max_pages, 0, num_pages};
  if (paged)
    while ((1 << a.page_shift) < page_size) ++a.page_shift;
  // Output rows: one per sequence, or (multi) one per query token.
  const int32_t rows_out = multi ? total_q : batch;
  if (num_splits == 1) return hip_status(sinkattn::launch_decode(a, static_cast<hipStream_t>(stream)), "decode launch");

  const size_t need = sinkattn_decode_workspace_bytes(rows_out, num_q_heads, head_dim, num_splits);
  if (static_scratch) {
    // the allocation-free form: the library's static array on the stream's
    // device (the current device for the null stream)
    if (need > sinkattn::kNoAllocScratchBytes)
      return fail(SINKATTN_ERR_WORKSPACE,
                  "the split-KV partials need %zu bytes, above the %zu-byte static scratch of the allocation-free "
                  "decode (use fewer splits, or sinkattn_decode_splitkv with a workspace)",
                  need, sinkattn::kNoAllocScratchBytes);
    int device = -1;
    hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &device)
                                     : hipGetDevice(&device);
    if (e == hipSuccess) e = sinkattn::noalloc_scratch(device, &workspace);
    if (e != hipSuccess) return hip_status(e, "static scratch lookup");
    workspace_bytes = sinkattn::kNoAllocScratchBytes;
  }
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SINKATTN_ERR_WORKSPACE, "workspace of %zu bytes is too small (need %zu)", workspace_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SINKATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t rows = static_cast<size_t>(num_splits) * rows_out * num_q_heads;
  char* ws = static_cast<char*>(workspace);
  a.o_part = reinterpret_cast<float*>(ws);
  a.lse_part = reinterpret_cast<float*>(ws + round_up(rows * head_dim * sizeof(float), 256));
  hipError_t e = sinkattn::launch_decode(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "decode launch");
  if (sinkattn::decode_merges_in_kernel(a)) return ok();
  sinkattn::MergeLaunch m{a.o_part, a.lse_part, num_splits, rows_out, num_q_heads, o, lse};
  return hip_status(sinkattn::launch_merge(m, static_cast<hipStream_t>(stream)), "merge launch");
}

sinkattn_status sinkattn_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_k,
                                        const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t window, float softmax_scale,
                                        int32_t num_splits, void* workspace, size_t workspace_bytes, void* o,
                                        float* lse, void* stream) {
  return decode_common(q, k_cache, v_cache, cu_seqlens_k, batch, max_seqlen_k, sinks, num_q_heads, num_kv_heads,
                       head_dim, window, softmax_scale, num_splits, workspace, workspace_bytes, o, lse, stream, false,
                       1.0f, 1.0f);
}

sinkattn_status sinkattn_decode_splitkv_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                                const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_k,
                                                const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t window, float softmax_scale,
                                                int32_t num_splits, void* o, float* lse, void* stream) {
  static_assert(SINKATTN_NOALLOC_SCRATCH_BYTES == sinkattn::kNoAllocScratchBytes, "scratch size mismatch");
  return decode_common(q, k_cache, v_cache, cu_seqlens_k, batch, max_seqlen_k, sinks, num_q_heads, num_kv_heads,
                       head_dim, window, softmax_scale, num_splits, nullptr, 0, o, lse, stream, false, 1.0f, 1.0f,
                       nullptr, 1, 0, nullptr, 0, 0, 0, /*static_scratch=*/true);
}

sinkattn_status sinkattn_decode_splitkv_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                                            float v_scale, const int32_t* cu_seqlens_k, int32_t batch,
                                            int32_t max_seqlen_k, const float* sinks, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim, int32_t window,
                                            float softmax_scale, int32_t num_splits, void* workspace,
                                            size_t workspace_bytes, void* o, float* lse, void* stream) {
  return decode_common(q, k_cache, v_cache, cu_seqlens_k, batch, max_seqlen_k, sinks, num_q_heads, num_kv_heads,
                       head_dim, window, softmax_scale, num_splits, workspace, workspace_bytes, o, lse, stream, true,
                       k_scale, v_scale);
}

sinkattn_status sinkattn_decode_splitkv_multi(const void* q, const void* k_cache, const void* v_cache,
                                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                                              int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t total_q,
                                              const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t window, float softmax_scale,
                                              int32_t num_splits, void* workspace, size_t workspace_bytes, void* o,
                                              float* lse, void* stream) {
  // (with batch 0 and no offsets the call validates its arguments and returns)
  if (cu_seqlens_q == nullptr && batch > 0)
    return fail(SINKATTN_ERR_INVALID_ARG, "cu_seqlens_q must not be NULL");
  return decode_common(q, k_cache, v_cache, cu_seqlens_k, batch, max_seqlen_k, sinks, num_q_heads, num_kv_heads,
                       head_dim, window, softmax_scale, num_splits, workspace, workspace_bytes, o, lse, stream, false,
                       1.0f, 1.0f, cu_seqlens_q, max_seqlen_q, total_q);
}

// Arguments of the paged cache, shared by the paged decode entry points.
static sinkattn_status check_pages(const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                                   int32_t max_pages, int32_t page_size, int32_t num_pages, int32_t max_seqlen_k) {
  if (page_size < 16 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
    return fail(SINKATTN_ERR_UNSUPPORTED, "page_size must be a power of two in [16, 2^20] (got %d)", page_size);
  if (batch < 0 || max_pages < 0 || num_pages < 0)
    return fail(SINKATTN_ERR_INVALID_ARG, "batch, max_pages and num_pages must be >= 0");
  if (batch > 0 && (max_pages < 1 || num_pages < 1))
    return fail(SINKATTN_ERR_INVALID_ARG, "max_pages and num_pages must be >= 1");
  if (static_cast<long long>(max_pages) * page_size < max_seqlen_k)
    return fail(SINKATTN_ERR_INVALID_ARG, "max_pages * page_size (%lld) is below max_seqlen_k (%d)",
                static_cast<long long>(max_pages) * page_size, max_seqlen_k);
  if (static_cast<long long>(num_pages) * page_size > 0x7fffffffLL)
    return fail(SINKATTN_ERR_UNSUPPORTED, "num_pages * page_size must stay below 2^31 tokens");
  if (batch > 0 && (block_table == nullptr || seq_lens == nullptr))
    return fail(SINKATTN_ERR_INVALID_ARG, "block_table and seq_lens must not be NULL");
  return ok();
}

sinkattn_status sinkattn_decode_splitkv_multi_fp8(const void* q, const void* k_cache, const void* v_cache,
                                                  float k_scale, float v_scale, const int32_t* cu_seqlens_q,
                                                  const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_q,
                                                  int32_t max_seqlen_k, int32_t total_q, const float* sinks,
                                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                                  int32_t window, float softmax_scale, int32_t num_splits,
                                                  void* workspace, size_t workspace_bytes, void* o, float* lse,
                                                  void* stream) {
  if (cu_seqlens_q == nullptr && batch > 0)
    return fail(SINKATTN_ERR_INVALID_ARG, "cu_seqlens_q must not be NULL");
  return decode_common(q, k_cache, v_cache, cu_seqlens_k, batch, max_seqlen_k, sinks, num_q_heads, num_kv_heads,
                       head_dim, window, softmax_scale, num_splits, workspace, workspace_bytes, o, lse, stream, true,
                       k_scale, v_scale, cu_seqlens_q, max_seqlen_q, total_q);
}

sinkattn_status sinkattn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                      const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                                      int32_t max_pages, int32_t page_size, int32_t num_pages, int32_t max_seqlen_k,
                                      const float* sinks, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t window, float softmax_scale, int32_t num_splits, void* workspace,
                                      size_t workspace_bytes, void* o, float* lse, void* stream) {
  sinkattn_status st = check_pages(block_table, seq_lens, batch, max_pages, page_size, num_pages, max_seqlen_k);
  if (st != SINKATTN_OK) return st;
  // (batch 0 validates the remaining arguments and returns)
  return decode_common(q, k_pages, v_pages, seq_lens, batch, max_seqlen_k, sinks, num_q_heads, num_kv_heads,
                       head_dim, window, softmax_scale, num_splits, workspace, workspace_bytes, o, lse, stream, false,
                       1.0f, 1.0f, nullptr, 1, 0, block_table, max_pages, page_size, num_pages);
}

sinkattn_status sinkattn_decode_paged_fp8(const void* q, const void* k_pages, const void* v_pages, float k_scale,
                                          float v_scale, const int32_t* block_table, const int32_t* seq_lens,
                                          int32_t batch, int32_t max_pages, int32_t page_size, int32_t num_pages,
                                          int32_t max_seqlen_k, const float* sinks, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t window,
                                          float softmax_scale, int32_t num_splits, void* workspace,
                                          size_t workspace_bytes, void* o, float* lse, void* stream) {
  sinkattn_status st = check_pages(block_table, seq_lens, batch, max_pages, page_size, num_pages, max_seqlen_k);
  if (st != SINKATTN_OK) return st;
  return decode_common(q, k_pages, v_pages, seq_lens, batch, max_seqlen_k, sinks, num_q_heads, num_kv_heads,
                       head_dim, window, softmax_scale, num_splits, workspace, workspace_bytes, o, lse, stream, true,
                       k_scale, v_scale, nullptr, 1, 0, block_table, max_pages, page_size, num_pages);
}

sinkattn_status sinkattn_decode_paged_multi(const void* q, const void* k_pages, const void* v_pages,
                                            const int32_t* block_table, const int32_t* seq_lens,
                                            const int32_t* cu_seqlens_q, int32_t batch, int32_t max_pages,
                                            int32_t page_size, int32_t num_pages, int32_t max_seqlen_q,
                                            int32_t max_seqlen_k, int32_t total_q, const float* sinks,
                                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                            int32_t window, float softmax_scale, int32_t num_splits, void* workspace,
                                            size_t workspace_bytes, void* o, float* lse, void* stream) {
  sinkattn_status st = check_pages(block_table, seq_lens, batch, max_pages, page_size, num_pages, max_seqlen_k);
  if (st != SINKATTN_OK) return st;
  if (cu_seqlens_q == nullptr && batch > 0) return fail(SINKATTN_ERR_INVALID_ARG, "cu_seqlens_q must not be NULL");
  return decode_common(q, k_pages, v_pages, seq_lens, batch, max_seqlen_k, sinks, num_q_heads, num_kv_heads,
                       head_dim, window, softmax_scale, num_splits, workspace, workspace_bytes, o, lse, stream, false,
                       1.0f, 1.0f, cu_seqlens_q, max_seqlen_q, total_q, block_table, max_pages, page_size, num_pages);
}

sinkattn_status sinkattn_decode_paged_multi_fp8(const void* q, const void* k_pages, const void* v_pages,
                                                float k_scale, float v_scale, const int32_t* block_table,
                                                const int32_t* seq_lens, const int32_t* cu_seqlens_q, int32_t batch,
                                                int32_t max_pages, int32_t page_size, int32_t num_pages,
                                                int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t total_q,
                                                const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t window, float softmax_scale,
                                                int32_t num_splits, void* workspace, size_t workspace_bytes, void* o,
                                                float* lse, void* stream) {
  sinkattn_status st = check_pages(block_table, seq_lens, batch, max_pages, page_size, num_pages, max_seqlen_k);
  if (st != SINKATTN_OK) return st;
  if (cu_seqlens_q == nullptr && batch > 0) return fail(SINKATTN_ERR_INVALID_ARG, "cu_seqlens_q must not be NULL");
  return decode_common(q, k_pages, v_pages, seq_lens, batch, max_seqlen_k, sinks, num_q_heads, num_kv_heads,
                       head_dim, window, softmax_scale, num_splits, workspace, workspace_bytes, o, lse, stream, true,
                       k_scale, v_scale, cu_seqlens_q, max_seqlen_q, total_q, block_table, max_pages, page_size,
                       num_pages);
}

sinkattn_status sinkattn_prefill_append_paged(const void* q, const void* k_pages, const void* v_pages,
                                              const int32_t* block_table, const int32_t* seq_lens_k,
                                              const int32_t* cu_seqlens_q, int32_t batch, int32_t max_pages,
                                              int32_t page_size, int32_t num_pages, int32_t max_seqlen_q,
                                              int32_t max_seqlen_k, int32_t total_q, const float* sinks,
                                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                              int32_t window, float softmax_scale, void* o, float* lse,
                                              void* stream) {
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0)
    return fail(SINKATTN_ERR_INVALID_ARG, "batch, lengths and totals must be >= 0");
  sinkattn_status st = check_pages(block_table, seq_lens_k, batch, max_pages, page_size, num_pages, max_seqlen_k);
  if (st != SINKATTN_OK) return st;
  if (cu_seqlens_q == nullptr && batch > 0) return fail(SINKATTN_ERR_INVALID_ARG, "cu_seqlens_q must not be NULL");
  // (the pool's rows stand for total_k)
  return prefill_common(q, k_pages, v_pages, sinks, cu_seqlens_q, seq_lens_k, batch, max_seqlen_q, max_seqlen_k,
                        total_q, num_pages * page_size, num_q_heads, num_kv_heads, head_dim, window, softmax_scale, o,
                        lse, stream, block_table, max_pages, page_size, num_pages);
}

sinkattn_status sinkattn_prefill_append_paged_splitkv(
    const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table, const int32_t* seq_lens_k,
    const int32_t* cu_seqlens_q, int32_t batch, int32_t max_pages, int32_t page_size, int32_t num_pages,
    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t total_q, const float* sinks, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t window, float softmax_scale, int32_t num_splits, void* workspace,
    size_t workspace_bytes, void* o, float* lse, void* stream) {
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0)
    return fail(SINKATTN_ERR_INVALID_ARG, "batch, lengths and totals must be >= 0");
  if (num_splits < 1) return fail(SINKATTN_ERR_INVALID_ARG, "num_splits must be >= 1 (got %d)", num_splits);
  if (num_splits > kMaxPrefillSplits)
    return fail(SINKATTN_ERR_UNSUPPORTED, "num_splits must be <= %d (got %d)", kMaxPrefillSplits, num_splits);
  sinkattn_status st = check_pages(block_table, seq_lens_k, batch, max_pages, page_size, num_pages, max_seqlen_k);
  if (st != SINKATTN_OK) return st;
  if (cu_seqlens_q == nullptr && batch > 0) return fail(SINKATTN_ERR_INVALID_ARG, "cu_seqlens_q must not be NULL");
  return prefill_common(q, k_pages, v_pages, sinks, cu_seqlens_q, seq_lens_k, batch, max_seqlen_q, max_seqlen_k,
                        total_q, num_pages * page_size, num_q_heads, num_kv_heads, head_dim, window, softmax_scale, o,
                        lse, stream, block_table, max_pages, page_size, num_pages, num_splits, workspace,
                        workspace_bytes);
}

// Rotary frequencies of the pairs (i, i + 32): theta^(-2i/64), rescaled by
// YaRN's NTK-by-parts rule when factor > 1, with the ramp over the pair index
// that YaRN's own code and the GPT-OSS / DeepSeek-V3 models use: the index at
// which a frequency turns `beta` times over the original context is
// 32 ln(L / (2 pi beta)) / ln(theta); between the indices of beta_fast and
// beta_slow (rounded outwards when `truncate` is set; clamped to [0, 63])
// the frequency moves linearly in the index from f to f / factor.  YaRN's
// temperature is 0.1 ln(factor) + 1.
static sinkattn::RopeTable rope_table(double theta, double factor, int original_max_position, double beta_fast,
                                      double beta_slow, bool truncate) {
  sinkattn::RopeTable t{};
  const double two_pi = 6.283185307179586476925286766559;
  double low = 0.0, high = 1.0;
  if (factor > 1.0) {
    auto index_of = [&](double turns) {
      return 32.0 * std::log(original_max_position / (two_pi * turns)) / std::log(theta);
    };
    low = index_of(beta_fast);
    high = index_of(beta_slow);
    if (truncate) {
      low = std::floor(low);
      high = std::ceil(high);
    }
    low = std::max(low, 0.0);
    high = std::min(high, 63.0);
    if (high == low) high += 0.001;  // a zero-width ramp is a step
  }
  for (int i = 0; i < 32; ++i) {
    const double f = std::pow(theta, -static_cast<double>(2 * i) / 64.0);
    if (factor > 1.0) {
      const double g = std::min(1.0, std::max(0.0, (i - low) / (high - low)));
      t.freq[i] = f * (1.0 - g) + g * f / factor;
    } else {
      t.freq[i] = f;
    }
  }
  t.attention_factor = factor > 1.0 ? static_cast<float>(0.1 * std::log(factor) + 1.0) : 1.0f;
  return t;
}

sinkattn_status sinkattn_rope_qkv_append(const void* qkv, const int32_t* positions, const int32_t* slot_mapping,
                                         int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, double rope_theta, double yarn_factor,
                                         int32_t yarn_original_max_position, double yarn_beta_fast,
                                         double yarn_beta_slow, int32_t yarn_truncate, void* q_out, void* k_cache,
                                         void* v_cache, int32_t cache_rows, void* stream) {
  if (num_tokens < 0 || cache_rows < 0) return fail(SINKATTN_ERR_INVALID_ARG, "num_tokens and cache_rows must be >= 0");
  if (num_q_heads < 1 || num_kv_heads < 1)
    return fail(SINKATTN_ERR_INVALID_ARG, "head counts must be >= 1 (got %d, %d)", num_q_heads, num_kv_heads);
  if (head_dim != 64) return fail(SINKATTN_ERR_UNSUPPORTED, "head_dim %d is not supported (only 64)", head_dim);
  if (!std::isfinite(rope_theta) || !(rope_theta > 1.0))
    return fail(SINKATTN_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
  if (!std::isfinite(yarn_factor) || !(yarn_factor > 0.0))
    return fail(SINKATTN_ERR_INVALID_ARG, "yarn_factor must be finite and > 0");
  if (yarn_factor > 1.0 &&
      (yarn_original_max_position < 1 || !std::isfinite(yarn_beta_fast) || !std::isfinite(yarn_beta_slow) ||
       !(yarn_beta_fast > yarn_beta_slow) || !(yarn_beta_slow > 0.0)))
    return fail(SINKATTN_ERR_INVALID_ARG,
                "YaRN needs original_max_position >= 1 and finite beta_fast > beta_slow > 0");
  if (num_tokens == 0) return ok();
  if (!qkv || !positions || !slot_mapping || !q_out || !k_cache || !v_cache)
    return fail(SINKATTN_ERR_INVALID_ARG, "qkv, positions, slot_mapping, q_out, k_cache and v_cache must not be NULL");
  if (!aligned16(qkv) || !aligned16(q_out) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(SINKATTN_ERR_INVALID_ARG, "qkv, q_out, k_cache and v_cache must be 16-byte aligned");
  sinkattn_status st;
  if (debug_checks()) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t n = static_cast<size_t>(num_tokens) * (num_q_heads + 2 * num_kv_heads) * head_dim;
    if ((st = hip_queue(sinkattn::check_clear(s))) != SINKATTN_OK) return st;
    if ((st = hip_queue(sinkattn::check_slots(slot_mapping, num_tokens, cache_rows, s))) != SINKATTN_OK) return st;
    if ((st = hip_queue(sinkattn::check_bf16(qkv, n, sinkattn::kCheckQ, s))) != SINKATTN_OK) return st;
    if ((st = check_result(s, nullptr)) != SINKATTN_OK) return st;
  }
  sinkattn::RopeLaunch a{qkv, positions, slot_mapping, num_tokens, num_q_heads, num_kv_heads, cache_rows,
                         rope_table(rope_theta, yarn_factor, yarn_original_max_position, yarn_beta_fast,
                                    yarn_beta_slow, yarn_truncate != 0),
                         q_out, k_cache, v_cache};
  return hip_status(sinkattn::launch_rope_qkv_append(a, static_cast<hipStream_t>(stream)), "rope launch");
}

size_t sinkattn_oproj_workspace_bytes(int32_t num_rows, int32_t in_features, int32_t out_features) {
  if (num_rows <= 0 || in_features < 128 || in_features % 128 != 0 || out_features < 32 || out_features % 32 != 0)
    return 0;
  const int splits = sinkattn::oproj_splits(num_rows, in_features, out_features);
  return splits > 1 ? round_up(static_cast<size_t>(splits) * num_rows * out_features * sizeof(float), 256) : 0;
}

sinkattn_status sinkattn_oproj_bias(const void* o, const void* w, const float* bias, int32_t num_rows,
                                    int32_t in_features, int32_t out_features, void* y, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (num_rows < 0 || in_features < 1 || out_features < 1)
    return fail(SINKATTN_ERR_INVALID_ARG, "need num_rows >= 0 and positive feature counts");
  if (in_features % 128 != 0 || out_features % 32 != 0)
    return fail(SINKATTN_ERR_UNSUPPORTED, "in_features must be a multiple of 128 and out_features of 32 (got %d, %d)",
                in_features, out_features);
  if ((static_cast<long long>(num_rows) + 63) / 64 > 65535)
    return fail(SINKATTN_ERR_UNSUPPORTED, "at most 65535 * 64 rows per call");
  if (num_rows == 0) return ok();
  if (!o || !w || !y) return fail(SINKATTN_ERR_INVALID_ARG, "o, w and y must not be NULL");
  if (!aligned16(o) || !aligned16(w) || !aligned16(y))
    return fail(SINKATTN_ERR_INVALID_ARG, "o, w and y must be 16-byte aligned");
  if (debug_checks()) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    sinkattn_status st;
    if ((st = hip_queue(sinkattn::check_clear(s))) != SINKATTN_OK) return st;
    if ((st = hip_queue(sinkattn::check_bf16(o, static_cast<size_t>(num_rows) * in_features, sinkattn::kCheckO,
                                             s))) != SINKATTN_OK)
      return st;
    if ((st = hip_queue(sinkattn::check_bf16(w, static_cast<size_t>(out_features) * in_features,
                                             sinkattn::kCheckW, s))) != SINKATTN_OK)
      return st;
    if ((st = check_result(s, nullptr)) != SINKATTN_OK) return st;
  }
  const size_t need = sinkattn_oproj_workspace_bytes(num_rows, in_features, out_features);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(SINKATTN_ERR_WORKSPACE, "workspace of %zu bytes is too small (need %zu)", workspace_bytes, need);
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SINKATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  sinkattn::OprojLaunch a{o, w, bias, num_rows, in_features, out_features, y, static_cast<float*>(workspace)};
  return hip_status(sinkattn::launch_oproj(a, static_cast<hipStream_t>(stream)), "projection launch");
}

sinkattn_status sinkattn_merge_lse(const float* o_parts, const float* lse_parts, int32_t num_parts, int32_t n,
                                   int32_t num_heads, int32_t head_dim, void* o, float* lse, void* stream) {
  if (num_parts < 1 || n < 0 || num_heads < 1)
    return fail(SINKATTN_ERR_INVALID_ARG, "need num_parts >= 1, n >= 0, num_heads >= 1");
  if (head_dim != 64) return fail(SINKATTN_ERR_UNSUPPORTED, "head_dim %d is not supported (only 64)", head_dim);
  if (n == 0) return ok();
  if (!o_parts || !lse_parts || !o) return fail(SINKATTN_ERR_INVALID_ARG, "o_parts, lse_parts and o must not be NULL");
  if (!aligned16(o_parts) || !aligned16(o)) return fail(SINKATTN_ERR_INVALID_ARG, "o_parts and o must be 16-byte aligned");
  const long long rows = static_cast<long long>(n) * num_heads;
  if (rows > 0x7fffffffLL) return fail(SINKATTN_ERR_UNSUPPORTED, "too many rows");
  if (debug_checks()) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t prow = static_cast<size_t>(num_parts) * rows;
    sinkattn_status st;
    if ((st = hip_queue(sinkattn::check_clear(s))) != SINKATTN_OK) return st;
    if ((st = hip_queue(sinkattn::check_f32(o_parts, prow * head_dim, sinkattn::kCheckParts, false, s))) !=
        SINKATTN_OK)
      return st;
    if ((st = hip_queue(sinkattn::check_f32(lse_parts, prow, sinkattn::kCheckParts, true, s))) != SINKATTN_OK)
      return st;
    if ((st = check_result(s, nullptr)) != SINKATTN_OK) return st;
  }
  sinkattn::MergeLaunch m{o_parts, lse_parts, num_parts, n, num_heads, o, lse};
  return hip_status(sinkattn::launch_merge(m, static_cast<hipStream_t>(stream)), "merge launch");
}

}  // extern "C"
