// Device helpers shared by the sink-attention kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16): lane l holds row l % 32, k = 8 * (l / 32) + t, t = 0..7
//   B (16 x 32): lane l holds column l % 32, k = 8 * (l / 32) + t
//   C (32 x 32): lane l holds column l % 32; register r holds row
//                8 * (r / 4) + 4 * (l / 32) + r % 4
// The attention kernels compute S^T = K Q^T and O^T = V^T P^T so that every
// per-query quantity (running max, denominator, output column) lives in one
// lane pair (l, l ^ 32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x16_t mfma_32x32x16(const bf16x8_t& a, const bf16x8_t& b,
                                                  const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Max / sum of a per-lane value over the lane pair (l, l ^ 32).
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + p.x + p.y for a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_pair(bf16x2_t p, float acc) {
  const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(p, ones, acc, false);
}

// True if the predicate holds on any lane of the wave.
__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite or +-0).
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// A row of a [rows][64] bf16 tile in LDS is 128 bytes = 8 chunks of 16 bytes.
// Chunk c of row r is stored at chunk position c ^ swz_f(r), where swz_f is a
// linear map (over GF(2)) of the row's low four bits into the three chunk
// bits.  This map was picked by timing every such map on gfx950 for the two
// read patterns of the attention kernels -- K rows as the MFMA A operand
// (ds_read_b128 over rows key_of_row(0..31)) and V rows read transposed
// (ds_read_b64_tr_b16 over groups of 4 rows) -- and is within a few percent
// of the fastest map for each; the plain c ^ (r & 7) swizzle is 1.7x / 1.5x
// slower there.  It is a bijection on any 8 consecutive aligned rows, so the
// row-wise tile writes stay conflict-free.
__device__ __forceinline__ int swz_f(int row) {
  const int b0 = row & 1, b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
  return (b0 ^ b1 ^ b2) | ((b1 ^ b2 ^ b3) << 1) | ((b0 ^ b1 ^ b3) << 2);
}

__device__ __forceinline__ int swz(int row, int d) {
  return row * kHeadDim + ((((d >> 3) ^ swz_f(row)) & 7) << 3) + (d & 7);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives element i % 4 of the 4-element pieces addressed by lanes
// 4r + i / 4 (r = 0..3).  Used with every lane of a group pointing at
// row (base + i / 4), columns [c0 + 4 (i % 4), +4), lane i receives column
// c0 + i of rows base .. base + 3.
__device__ __forceinline__ bf16x4_t lds_read_tr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ bf16x8_t cat4(const bf16x4_t& a, const bf16x4_t& b) {
  bf16x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// 16-byte global -> LDS copy that bypasses registers (global_load_lds_dwordx4):
// lane L of the wave writes the 16 bytes it loads from `src` to
// lds_base + 16 L.  lds_base must be the same for every lane of the wave.
// Completion is tracked by vmcnt.
__device__ __forceinline__ void load16_to_lds(const uint16_t* src, uint16_t* lds_base) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void*)(lds_base), 16, 0, 0);
}

// The same copy issued from inline assembly, so the compiler does not know
// about it: it adds no vmcnt waits of its own before LDS reads (it would
// otherwise make every transposing read wait for every copy in flight).  The
// caller orders each read of the destination after the copy with a vmcnt
// wait and a barrier.  The LDS address goes through M0; the asm names M0 as
// clobbered, so the compiler reloads any value of its own it keeps there.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load16_to_lds_untracked(const uint16_t* src, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS address (byte offset in the workgroup's LDS) of a __shared__ object.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  typedef __attribute__((address_space(3))) const void lds_cvoid;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cvoid*)(p)));
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// 16-byte load of data that is streamed once (nontemporal hint: bypasses
// cache retention).  On MI355X this raised sustained read bandwidth of a plain
// streaming kernel from 6.5 to 7.2 TB/s.
__device__ __forceinline__ u32x4_t load16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ u32x4_t zero_u32x4() {
  u32x4_t z = {0u, 0u, 0u, 0u};
  return z;
}

// Row permutation of a 32-key block used when K feeds the A operand of
// S^T = K Q^T: MFMA row m reads key sigma(m) so that, in the C layout, lane
// half h holds keys 8h + 0..7 (registers 0..7) and 16 + 8h + 0..7
// (registers 8..15).  Those are exactly the k slots the B operand of
// O^T = V^T P^T expects for the two 16-key steps.
__device__ __forceinline__ int key_of_row(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// Key offset (within a 32-key block) of C register r in lane half h.
__device__ __forceinline__ int key_of_reg(int r, int half) {
  return 16 * (r >> 3) + 8 * half + (r & 7);
}

}  // namespace sinkattn
