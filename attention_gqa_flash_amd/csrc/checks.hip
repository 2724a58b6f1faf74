// Device-side precondition checks, run by the C ABI before a launch when
// SINKATTN_DEBUG_CHECKS=1 is set in the environment.  They cover what the
// host cannot see without reading device memory: sequence offsets (monotone,
// starting at 0, lengths within the declared maximum, decode lengths >= 1,
// append prefill: at least as many keys as queries per sequence),
// sinks (finite or -inf; NaN and +inf are undefined), and NaN / Inf in the
// bf16 inputs (NaN codes in E4M3 caches) and in merge partials.
//
// Each check kernel ORs a bit into g_check_flags; the host clears the word
// before and reads it back after (hipMemcpyFromSymbol), synchronising the
// stream.  Debug mode is for diagnosis: calls that overlap on one device
// share the flag word.
#include "launch.hpp"

namespace sinkattn {

namespace {

__device__ unsigned g_check_flags;
__device__ int g_check_total;  // cu_seqlens[batch] of the last offsets check

__global__ void clear_flags_kernel() {
  g_check_flags = 0u;
  g_check_total = 0;
}

__global__ void check_offsets_kernel(const int32_t* __restrict__ cu, int batch, int max_len, int min_len,
                                     int total_limit) {
  unsigned bits = 0;
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < batch; b += gridDim.x * blockDim.x) {
    const int lo = cu[b], hi = cu[b + 1];
    if (b == 0 && lo != 0) bits |= kCheckOffsetsStart;
    if (hi < lo) bits |= kCheckOffsetsOrder;
    else if (hi - lo > max_len) bits |= kCheckLengthMax;
    else if (hi - lo < min_len) bits |= kCheckLengthMin;
    if (b == batch - 1) {
      if (total_limit >= 0 && hi > total_limit) bits |= kCheckOffsetsTotal;
      g_check_total = hi;
    }
  }
  if (bits != 0u) atomicOr(&g_check_flags, bits);
}

// Append prefill: no sequence may have fewer key rows than query rows.
__global__ void check_append_kernel(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                                    bool k_lengths, int batch) {
  unsigned bits = 0;
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < batch; b += gridDim.x * blockDim.x) {
    const int lk = k_lengths ? cu_k[b] : cu_k[b + 1] - cu_k[b];
    if (lk < cu_q[b + 1] - cu_q[b]) bits |= kCheckAppend;
  }
  if (bits != 0u) atomicOr(&g_check_flags, bits);
}

// Paged decode: lengths within [1, max_len], tables long enough, page ids
// inside the pool.  One thread per sequence.
__global__ void check_paged_kernel(const int32_t* __restrict__ lens, const int32_t* __restrict__ table, int batch,
                                   int max_pages, int page_size, int num_pages, int max_len) {
  unsigned bits = 0;
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < batch; b += gridDim.x * blockDim.x) {
    const int n = lens[b];
    if (n < 1) bits |= kCheckLengthMin;
    if (n > max_len) bits |= kCheckLengthMax;
    const int pages = n > 0 ? (min(n, max_len) + page_size - 1) / page_size : 0;
    if (pages > max_pages) bits |= kCheckPages;
    for (int p = 0; p < min(pages, max_pages); ++p) {
      const int id = table[static_cast<size_t>(b) * max_pages + p];
      if (id < 0 || id >= num_pages) bits |= kCheckPages;
    }
  }
  if (bits != 0u) atomicOr(&g_check_flags, bits);
}

// Rotary append: slots in [-1, cache_rows) and pairwise distinct (the check
// compares every pair: debug mode only, quadratic in the tokens).
__global__ void check_slots_kernel(const int32_t* __restrict__ slots, int n, int cache_rows) {
  unsigned bits = 0;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const int s = slots[i];
    if (s < -1 || s >= cache_rows) bits |= kCheckSlots;
    if (s >= 0)
      for (int j = i + 1; j < n; ++j)
        if (slots[j] == s) bits |= kCheckSlots;
  }
  if (bits != 0u) atomicOr(&g_check_flags, bits);
}

// Floating-point classes are tested on the bit patterns: the library is
// built without NaN semantics (-fno-honor-nans), so x != x would fold away.
__device__ __forceinline__ bool is_nan_bits(uint32_t u) { return (u & 0x7fffffffu) > 0x7f800000u; }
constexpr uint32_t kPosInfBits = 0x7f800000u;
constexpr uint32_t kNegInfBits = 0xff800000u;

__global__ void check_sinks_kernel(const float* __restrict__ sinks, int n) {
  unsigned bits = 0;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const uint32_t u = __float_as_uint(sinks[i]);
    if (is_nan_bits(u) || u == kPosInfBits) bits |= kCheckSinks;
  }
  if (bits != 0u) atomicOr(&g_check_flags, bits);
}

// bf16 NaN or Inf: exponent bits all ones.
__global__ void check_bf16_kernel(const uint16_t* __restrict__ x, size_t n, unsigned bit) {
  unsigned bad = 0;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    bad |= (x[i] & 0x7f80u) == 0x7f80u;
  if (bad != 0u) atomicOr(&g_check_flags, bit);
}

// E4M3 NaN: the codes 0x7f and 0xff (the format has no infinities).
__global__ void check_e4m3_kernel(const uint8_t* __restrict__ x, size_t n, unsigned bit) {
  unsigned bad = 0;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    bad |= (x[i] & 0x7fu) == 0x7fu;
  if (bad != 0u) atomicOr(&g_check_flags, bit);
}

// fp32 values must not be NaN or +inf, nor -inf unless allow_neg_inf.
__global__ void check_f32_kernel(const float* __restrict__ x, size_t n, unsigned bit, int allow_neg_inf) {
  unsigned bad = 0;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const uint32_t u = __float_as_uint(x[i]);
    bad |= is_nan_bits(u) || u == kPosInfBits || (!allow_neg_inf && u == kNegInfBits);
  }
  if (bad != 0u) atomicOr(&g_check_flags, bit);
}

// NaN / Inf (bf16, elem_bytes 2) or NaN codes (E4M3, elem_bytes 1) in the
// page-pool rows a paged call can read: the first lens[b] slots of sequence
// b through its table row.  Free or unowned pages are not inspected.  A
// length or page id that check_paged reports is skipped here, so a broken
// table cannot move this scan out of the pool.  Work is (sequence, page)
// pairs in a grid-stride loop, one page per workgroup at a time.
__global__ void check_paged_values_kernel(const void* __restrict__ pool, const int32_t* __restrict__ lens,
                                          const int32_t* __restrict__ table, int batch, int max_pages,
                                          int page_size, int num_pages, int max_len, int row_elems, int elem_bytes,
                                          unsigned bit) {
  unsigned bad = 0;
  const long long pairs = static_cast<long long>(batch) * max_pages;
  for (long long pr = blockIdx.x; pr < pairs; pr += gridDim.x) {
    const int b = static_cast<int>(pr / max_pages);
    const int p = static_cast<int>(pr % max_pages);
    const int n = lens[b];
    if (n < 1 || n > max_len) continue;
    const long long first = static_cast<long long>(p) * page_size;
    if (first >= n) continue;
    const int id = table[pr];
    if (id < 0 || id >= num_pages) continue;
    const int rows = static_cast<int>(min(static_cast<long long>(page_size), n - first));
    const size_t base = static_cast<size_t>(id) * page_size * row_elems;
    const size_t count = static_cast<size_t>(rows) * row_elems;
    if (elem_bytes == 2) {
      const uint16_t* x = static_cast<const uint16_t*>(pool) + base;
      for (size_t i = threadIdx.x; i < count; i += blockDim.x) bad |= (x[i] & 0x7f80u) == 0x7f80u;
    } else {
      const uint8_t* x = static_cast<const uint8_t*>(pool) + base;
      for (size_t i = threadIdx.x; i < count; i += blockDim.x) bad |= (x[i] & 0x7fu) == 0x7fu;
    }
  }
  if (bad != 0u) atomicOr(&g_check_flags, bit);
}

unsigned grid_for(size_t n) {
  const size_t blocks = (n + 255) / 256;
  return static_cast<unsigned>(blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks));
}

}  // namespace

hipError_t check_clear(hipStream_t stream) {
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(1), 0, stream);
  return hipGetLastError();
}

hipError_t check_offsets(const int32_t* cu, int batch, int max_len, int min_len, int total_limit,
                         hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_offsets_kernel, dim3(grid_for(batch)), dim3(256), 0, stream, cu, batch, max_len,
                     min_len, total_limit);
  return hipGetLastError();
}

hipError_t check_append(const int32_t* cu_q, const int32_t* cu_k, bool k_lengths, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_append_kernel, dim3(grid_for(batch)), dim3(256), 0, stream, cu_q, cu_k, k_lengths, batch);
  return hipGetLastError();
}

hipError_t check_paged(const int32_t* seq_lens, const int32_t* block_table, int batch, int max_pages,
                       int page_size, int num_pages, int max_len, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_paged_kernel, dim3(grid_for(batch)), dim3(256), 0, stream, seq_lens, block_table, batch,
                     max_pages, page_size, num_pages, max_len);
  return hipGetLastError();
}

hipError_t check_paged_values(const void* pool, const int32_t* seq_lens, const int32_t* block_table, int batch,
                              int max_pages, int page_size, int num_pages, int max_len, int row_elems, int elem_bytes,
                              unsigned bit, hipStream_t stream) {
  if (pool == nullptr || batch <= 0 || max_pages <= 0) return hipSuccess;
  const long long pairs = static_cast<long long>(batch) * max_pages;
  const unsigned blocks = static_cast<unsigned>(pairs < 4096 ? pairs : 4096);
  hipLaunchKernelGGL(check_paged_values_kernel, dim3(blocks), dim3(256), 0, stream, pool, seq_lens, block_table,
                     batch, max_pages, page_size, num_pages, max_len, row_elems, elem_bytes, bit);
  return hipGetLastError();
}

hipError_t check_slots(const int32_t* slots, int n, int cache_rows, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_slots_kernel, dim3(grid_for(n)), dim3(256), 0, stream, slots, n, cache_rows);
  return hipGetLastError();
}

hipError_t check_sinks(const float* sinks, int n, hipStream_t stream) {
  if (sinks == nullptr || n <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_sinks_kernel, dim3(grid_for(n)), dim3(256), 0, stream, sinks, n);
  return hipGetLastError();
}

hipError_t check_bf16(const void* x, size_t n, unsigned bit, hipStream_t stream) {
  if (x == nullptr || n == 0) return hipSuccess;
  hipLaunchKernelGGL(check_bf16_kernel, dim3(grid_for(n)), dim3(256), 0, stream, static_cast<const uint16_t*>(x),
                     n, bit);
  return hipGetLastError();
}

hipError_t check_e4m3(const void* x, size_t n, unsigned bit, hipStream_t stream) {
  if (x == nullptr || n == 0) return hipSuccess;
  hipLaunchKernelGGL(check_e4m3_kernel, dim3(grid_for(n)), dim3(256), 0, stream, static_cast<const uint8_t*>(x), n,
                     bit);
  return hipGetLastError();
}

hipError_t check_f32(const float* x, size_t n, unsigned bit, bool allow_neg_inf, hipStream_t stream) {
  if (x == nullptr || n == 0) return hipSuccess;
  hipLaunchKernelGGL(check_f32_kernel, dim3(grid_for(n)), dim3(256), 0, stream, x, n, bit, allow_neg_inf ? 1 : 0);
  return hipGetLastError();
}

hipError_t check_read(unsigned* flags, int* total, hipStream_t stream) {
  hipError_t e = hipMemcpyFromSymbolAsync(flags, HIP_SYMBOL(g_check_flags), sizeof(unsigned), 0,
                                          hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyFromSymbolAsync(total, HIP_SYMBOL(g_check_total), sizeof(int), 0, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return e;
}

}  // namespace sinkattn
