// Fused rotary step before attention: rotate the query heads into q_out, and
// write the rotated key heads and the value heads of each new token into its
// cache row (gfx950).
//
// Operation: the rotary position embedding of the attention layers (NVIDIA
// gpt-oss announcement, model description: RoPE; Perplexity, "GPT-OSS on
// day 0", Hopper section: YaRN position encoding), applied together with the
// Q output and the KV-cache write as one pass (vLLM, "GPT-OSS performance
// optimizations on NVIDIA Blackwell", minimum latency: RoPE + Q + cache
// fusion).  Dimension i < 32 of a head pairs with i + 32 and turns by
// position * f_i; the frequencies (YaRN-rescaled on the host) and the
// temperature factor come in as kernel arguments.
//
// HBM-bound elementwise work: one workgroup per token; each work-item owns 8
// pairs of one head row (two 16-byte loads, two 16-byte stores), four per
// 128-byte row, so a wave reads 16 whole rows.  The token's angles are formed
// and reduced modulo 2 pi in fp64 (positions up to 2^31 keep their phase),
// then sin / cos in fp32, once per token into LDS.
#include "device_common.hpp"
#include "launch.hpp"

namespace sinkattn {

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One workgroup per token: its 32 (cos, sin) pairs are computed once into
// LDS (every head of the token turns by the same angles), then the
// workgroup's threads take the token's (head, quarter) items.
__global__ __launch_bounds__(256) void rope_qkv_append_kernel(
    const uint16_t* __restrict__ qkv, const int32_t* __restrict__ positions, const int32_t* __restrict__ slots,
    int hq, int hkv, RopeTable table, uint16_t* __restrict__ q_out, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, int cache_rows) {
  __shared__ float cs[2][32];
  const long long t = blockIdx.x;
  const int heads = hq + 2 * hkv;
  if (threadIdx.x < 32) {
    double a = static_cast<double>(positions[t]) * table.freq[threadIdx.x];
    a -= kTwoPi * rint(a * (1.0 / kTwoPi));
    float s, c;
    sincosf(static_cast<float>(a), &s, &c);
    cs[0][threadIdx.x] = c * table.attention_factor;
    cs[1][threadIdx.x] = s * table.attention_factor;
  }
  const int slot = slots[t];
  __syncthreads();
  for (int item = threadIdx.x; item < heads * 4; item += blockDim.x) {
    const int head = item >> 2;
    const int d0 = 8 * (item & 3);
    const uint16_t* src = qkv + (t * heads + head) * kHeadDim;
    const u32x4_t lo = load16(src + d0);
    const u32x4_t hi = load16(src + 32 + d0);
    uint16_t* dst;
    if (head < hq) {
      dst = q_out + (t * hq + head) * kHeadDim;
    } else {
      if (slot < 0 || slot >= cache_rows) continue;  // -1: no cache row; beyond the cache: a broken precondition
      if (head >= hq + hkv) {  // value head: copied as it is
        uint16_t* vd = v_cache + (static_cast<size_t>(slot) * hkv + (head - hq - hkv)) * kHeadDim;
        *reinterpret_cast<u32x4_t*>(vd + d0) = lo;
        *reinterpret_cast<u32x4_t*>(vd + 32 + d0) = hi;
        continue;
      }
      dst = k_cache + (static_cast<size_t>(slot) * hkv + (head - hq)) * kHeadDim;
    }
    u32x4_t out_lo, out_hi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float c0 = cs[0][d0 + 2 * j], s0 = cs[1][d0 + 2 * j];
      const float c1 = cs[0][d0 + 2 * j + 1], s1 = cs[1][d0 + 2 * j + 1];
      const float a0 = bf16_lo(lo[j]), a1 = bf16_hi(lo[j]);  // x_i of the pairs
      const float b0 = bf16_lo(hi[j]), b1 = bf16_hi(hi[j]);  // x_{i+32}
      out_lo[j] = static_cast<uint32_t>(to_bf16_bits(a0 * c0 - b0 * s0)) |
                  (static_cast<uint32_t>(to_bf16_bits(a1 * c1 - b1 * s1)) << 16);
      out_hi[j] = static_cast<uint32_t>(to_bf16_bits(b0 * c0 + a0 * s0)) |
                  (static_cast<uint32_t>(to_bf16_bits(b1 * c1 + a1 * s1)) << 16);
    }
    *reinterpret_cast<u32x4_t*>(dst + d0) = out_lo;
    *reinterpret_cast<u32x4_t*>(dst + 32 + d0) = out_hi;
  }
}

}  // namespace

hipError_t launch_rope_qkv_append(const RopeLaunch& a, hipStream_t stream) {
  if (a.num_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_qkv_append_kernel, dim3(static_cast<unsigned>(a.num_tokens)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a.qkv), a.positions, a.slot_mapping, a.num_q_heads,
                     a.num_kv_heads, a.table, static_cast<uint16_t*>(a.q_out), static_cast<uint16_t*>(a.k_cache),
                     static_cast<uint16_t*>(a.v_cache), a.cache_rows);
  return hipGetLastError();
}

}  // namespace sinkattn
