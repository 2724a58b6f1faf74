// Varlen causal / sliding-window prefill with per-head sinks (gfx950).
//
// Operation: Perplexity, "GPT-OSS on day 0", section "GPT-OSS kernels / Sink
// attention" (the sink is an extra softmax logit; the online softmax starts
// its running max at the sink and its denominator at 1), with the 128-token
// window layers of the NVIDIA gpt-oss announcement (model description).
//
// Work decomposition: one workgroup per (sequence, KV head, chunk of up to 8
// query heads of that KV head's group, tile of 32 query tokens).  The four
// waves of a workgroup share every K/V tile staged in LDS; wave w owns two
// query heads of the group for the same 32 tokens, so one K/V tile read from
// HBM feeds the whole GQA group.  Work items are launched heaviest first
// (query tiles in descending order), and the KV head is the fastest-varying
// block index so that the blocks of one KV head land on the same XCD (blocks
// are dealt to the 8 XCDs round-robin) and share its L2.
//
// Per key tile of 64 keys and per wave (64 query columns):
//   S^T = K Q^T          16 MFMA 32x32x16 (K from LDS, Q held in registers)
//   mask                 only on tiles that cross the diagonal / window edge
//   online softmax       running max in log2 units, exp2, per-lane partial
//                        denominators (the lane pair shares the max)
//   O^T += V^T P^T       16 MFMA (V read transposed from LDS)
#include "device_common.hpp"
#include "launch.hpp"

namespace sinkattn {

namespace {

constexpr int kQTile = 32;     // query tokens per workgroup
constexpr int kKTile = 64;     // keys per LDS tile
constexpr int kThreads = 256;  // 4 waves
constexpr int kHeadsPerBlock = 8;

__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ sinks,
    const int32_t* __restrict__ cu_seqlens, int hq, int hkv, int group, int n_hchunk,
    int n_qtiles, int window, float scale_log2, uint16_t* __restrict__ o,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kKTile * kHeadDim];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kKTile * kHeadDim];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query token within the tile
  const int half = lane >> 5;  // which k-half / row-half of the MFMA layouts

  int x = blockIdx.x;
  const int g = x % hkv;
  x /= hkv;
  const int hchunk = x % n_hchunk;
  const int b = x / n_hchunk;
  const int qt = n_qtiles - 1 - static_cast<int>(blockIdx.y);

  const int seq0 = cu_seqlens[b];
  const int len = cu_seqlens[b + 1] - seq0;
  const int q0 = qt * kQTile;
  if (q0 >= len) return;  // uniform over the workgroup

  // Query heads of this wave (two column blocks of 32).
  int head[2];
  bool head_ok[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int slot = hchunk * kHeadsPerBlock + wave * 2 + c;
    head_ok[c] = slot < group;
    head[c] = g * group + (head_ok[c] ? slot : 0);
  }
  const bool wave_active = head_ok[0];
  const int qtok = q0 + col;
  const bool row_ok = qtok < len;

  // Q^T as the B operand: lane holds query column `col`, d = 16 s + 8 half + t.
  bf16x8_t qreg[2][4];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t val = zero_u32x4();
      if (head_ok[c] && row_ok) {
        const size_t off = (static_cast<size_t>(seq0 + qtok) * hq + head[c]) * kHeadDim + 16 * s + 8 * half;
        val = load16(q + off);
      }
      qreg[c][s] = __builtin_bit_cast(bf16x8_t, val);
    }
  }

  // Online-softmax state per column block.  The running max m is kept in
  // log2 units (scaled logits); the sink seeds it, and its "1" is counted once
  // (in the lower lane of the pair).
  float m2[2], lsum[2];
  f32x16_t acc[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const float z = (sinks != nullptr && head_ok[c]) ? sinks[head[c]] : kNegInf;
    if (z > kNegInf) {
      m2[c] = z * kLog2e;
      lsum[c] = half == 0 ? 1.0f : 0.0f;
    } else {
      m2[c] = kNegInf;
      lsum[c] = 0.0f;
    }
    acc[c][0] = zero16();
    acc[c][1] = zero16();
  }

  const int last_q = min(len - 1, q0 + kQTile - 1);
  const int first_key = window > 0 ? max(0, q0 - window + 1) : 0;
  const int t_begin = first_key / kKTile;
  const int t_end = last_q / kKTile;

  for (int t = t_begin; t <= t_end; ++t) {
    const int key0 = t * kKTile;
    __syncthreads();
    // Stage K and V tiles: 64 rows x 128 B each; thread -> (row, 16-B chunk).
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const int ch = tid & 7;
      const int key = key0 + r;
      u32x4_t kv = zero_u32x4(), vv = zero_u32x4();
      if (key < len) {
        const size_t off = (static_cast<size_t>(seq0 + key) * hkv + g) * kHeadDim + ch * 8;
        kv = load16(k + off);
        vv = load16(v + off);
      }
      const int dst = swz(r, ch * 8);
      *reinterpret_cast<u32x4_t*>(k_lds + dst) = kv;
      *reinterpret_cast<u32x4_t*>(v_lds + dst) = vv;
    }
    __syncthreads();
    if (!wave_active) continue;

    // S^T = K Q^T for two 32-key blocks and two column blocks.
    f32x16_t sacc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb][0] = zero16();
      sacc[kb][1] = zero16();
      const int row = kb * 32 + key_of_row(col);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(k_lds + swz(row, 16 * s + 8 * half));
        sacc[kb][0] = mfma_32x32x16(a, qreg[0][s], sacc[kb][0]);
        sacc[kb][1] = mfma_32x32x16(a, qreg[1][s], sacc[kb][1]);
      }
    }

    // Mask only tiles that reach past the first query (diagonal) or behind
    // the window of the last query.
    const bool need_mask = (key0 + kKTile - 1 > q0) || (window > 0 && key0 <= last_q - window);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + key_of_reg(r, half);
          const bool ok = key <= qtok && (window <= 0 || key > qtok - window);
          if (!ok) {
            sacc[kb][0][r] = kNegInf;
            sacc[kb][1][r] = kNegInf;
          }
        }
      }
    }

    // Online softmax (log2 domain) and P in bf16 as the B operand of O^T.
    bf16x8_t pb[2][2][2];  // [c][kb][u]
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][c][r]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m2[c], mx * scale_log2);
      const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
      const float alpha = fast_exp2(m2[c] - m_use);
      m2[c] = m_new;
      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          bf16x8_t pv;
#pragma unroll
          for (int tt = 0; tt < 8; ++tt) {
            const float p = fast_exp2(sacc[kb][c][8 * u + tt] * scale_log2 - m_use);
            psum += p;
            pv[tt] = static_cast<__bf16>(p);
          }
          pb[c][kb][u] = pv;
        }
      }
      lsum[c] = lsum[c] * alpha + psum;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][db][r] *= alpha;
    }

    // O^T += V^T P^T.  Lane (d = l % 32 of block db, half) needs V rows
    // kb*32 + 16u + 8 half + 0..7 at its column: two transposing reads.
    const int grp_lane = lane & 15;
    const int dcol0 = 16 * ((lane >> 4) & 1) + 4 * (grp_lane & 3);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int rbase = kb * 32 + 16 * u + 8 * half + (grp_lane >> 2);
          const int dcol = 32 * db + dcol0;
          const bf16x4_t lo = lds_read_tr(v_lds + swz(rbase, dcol));
          const bf16x4_t hi = lds_read_tr(v_lds + swz(rbase + 4, dcol));
          const bf16x8_t a = cat4(lo, hi);
          acc[0][db] = mfma_32x32x16(a, pb[0][kb][u], acc[0][db]);
          acc[1][db] = mfma_32x32x16(a, pb[1][kb][u], acc[1][db]);
        }
      }
    }
  }

  if (!wave_active) return;

  // Epilogue: full denominator over the lane pair, normalise, store bf16.
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const float den = pair_sum(lsum[c]);
    if (!head_ok[c] || !row_ok) continue;
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    const size_t orow = (static_cast<size_t>(seq0 + qtok) * hq + head[c]) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u16x4_t w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = to_bf16_bits(acc[c][db][4 * j + i] * inv);
        const int d = 32 * db + 8 * j + 4 * half;
        *reinterpret_cast<u16x4_t*>(o + orow + d) = w;
      }
    }
    if (lse != nullptr && half == 0) {
      const float l = den > 0.0f ? (m2[c] + __log2f(den)) * kLn2 : kNegInf;
      lse[static_cast<size_t>(seq0 + qtok) * hq + head[c]] = l;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int n_hchunk = (group + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const int n_qtiles = (a.max_seqlen + kQTile - 1) / kQTile;
  dim3 grid(static_cast<unsigned>(a.num_kv_heads) * n_hchunk * a.batch, n_qtiles, 1);
  hipLaunchKernelGGL(prefill_kernel, grid, dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.sinks, a.cu_seqlens, a.num_q_heads,
                     a.num_kv_heads, group, n_hchunk, n_qtiles, a.window,
                     a.softmax_scale * kLog2e, static_cast<uint16_t*>(a.o), a.lse);
  return hipGetLastError();
}

int prefill_max_qtiles() { return 65535; }
int prefill_qtile() { return kQTile; }

}  // namespace sinkattn
