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
constexpr int kKTile = 64;     // keys per LDS tile (two 32-key halves)
constexpr int kThreads = 256;  // 4 waves
constexpr int kHeadsPerBlock = 8;
// Lazy reference max.  Probabilities are taken against a per-row reference
// m (log2 units) that only moves when the new keys push a row's partial
// denominator past 2^32 (or when the row has no reference yet); the running
// output and denominator are then rescaled.  Values below the reference by
// more than 126 underflow to 0, which is exact to fp32 precision relative to
// the reference's own weight (>= 1) already counted.  o = acc / l is
// unchanged in exact arithmetic.
constexpr float kRescaleSum = 4294967296.0f;  // 2^32

struct TileRegs {
  u32x4_t k[2];
  u32x4_t v[2];
};

// Global -> registers for one 64-key tile: thread -> (row, 16-byte chunk).
__device__ __forceinline__ void load_tile(TileRegs& r, const uint16_t* __restrict__ k,
                                          const uint16_t* __restrict__ v, int seq0, int len, int hkv,
                                          int g, int key0, int tid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (tid >> 3) + 32 * i;
    const int key = key0 + row;
    r.k[i] = zero_u32x4();
    r.v[i] = zero_u32x4();
    if (key < len) {
      const size_t off = (static_cast<size_t>(seq0 + key) * hkv + g) * kHeadDim + (tid & 7) * 8;
      r.k[i] = load16(k + off);
      r.v[i] = load16(v + off);
    }
  }
}

__device__ __forceinline__ void store_tile(const TileRegs& r, uint16_t* k_lds, uint16_t* v_lds, int tid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (tid >> 3) + 32 * i;
    const int dst = swz(row, (tid & 7) * 8);
    *reinterpret_cast<u32x4_t*>(k_lds + dst) = r.k[i];
    *reinterpret_cast<u32x4_t*>(v_lds + dst) = r.v[i];
  }
}

template <bool kWindow>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ sinks,
    const int32_t* __restrict__ cu_seqlens, int hq, int hkv, int group, int n_hchunk,
    int n_qtiles, int window, float scale_log2, uint16_t* __restrict__ o,
    float* __restrict__ lse) {
  // Two LDS buffers per operand: tile t+1 is written while tile t is read.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kKTile * kHeadDim];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][kKTile * kHeadDim];

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

  const int last_q = min(len - 1, q0 + kQTile - 1);
  const int first_key = kWindow ? max(0, q0 - window + 1) : 0;
  const int t_begin = first_key / kKTile;
  const int t_end = last_q / kKTile;

  // Start the first K/V tile on its way before anything else.
  TileRegs regs;
  load_tile(regs, k, v, seq0, len, hkv, g, t_begin * kKTile, tid);

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

  // Online-softmax state per column block.  The reference max m is kept in
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

  store_tile(regs, k_lds[0], v_lds[0], tid);
  __syncthreads();

  // LDS read offsets (elements, within a 32-row half of a tile).  K^T rows
  // as the A operand: row key_of_row(col), d = 16 s + 8 half.  V^T operand:
  // lane (d = l % 32 of block db, half) needs rows 16 u + 8 half + 0..7 at
  // its column, as two transposing reads of 4 rows (i = 0, 1); under the
  // chunk swizzle read (db, u, i) sits at vbase + 1024 u + 256 i + 32 (db ^ i).
  int koff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = swz(key_of_row(col), 16 * s + 8 * half);
  const int grp_lane = lane & 15;
  const int dcol0 = 16 * ((lane >> 4) & 1) + 4 * (grp_lane & 3);
  const int vbase = (8 * half + (grp_lane >> 2)) * kHeadDim + ((((dcol0 >> 3) ^ (grp_lane >> 2)) & 3) << 3) +
                    (dcol0 & 7);

  for (int t = t_begin; t <= t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bool more = t < t_end;
    if (more) load_tile(regs, k, v, seq0, len, hkv, g, (t + 1) * kKTile, tid);

    if (wave_active) {
      const uint16_t* kt = k_lds[buf];
      const uint16_t* vt = v_lds[buf];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kbase = t * kKTile + kb * 32;
        // Halves no query of the tile can see are skipped.
        const bool dead = (kbase > last_q) || (kWindow && kbase + 31 <= q0 - window);
        if (dead) continue;

        // S^T = K Q^T for 32 keys and two column blocks.
        f32x16_t sacc[2] = {zero16(), zero16()};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kt + kb * 32 * kHeadDim + koff[s]);
          sacc[0] = mfma_32x32x16(a, qreg[0][s], sacc[0]);
          sacc[1] = mfma_32x32x16(a, qreg[1][s], sacc[1]);
        }

        const bool need_mask = (kbase + 31 > q0) || (kWindow && kbase <= last_q - window);
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase + key_of_reg(r, half);
            const bool ok = key <= qtok && (!kWindow || key > qtok - window);
            if (!ok) {
              sacc[0][r] = kNegInf;
              sacc[1][r] = kNegInf;
            }
          }
        }

        // Online softmax (log2 domain), P in bf16 as the B operand of O^T.
        // Fast path: P against the current reference m, no row max.
        bf16x8_t pb[2][2];  // [c][u]
        float tsum[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const float m_use = m2[c] == kNegInf ? 0.0f : m2[c];
          float l = 0.0f;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            bf16x8_t pv;
#pragma unroll
            for (int tt = 0; tt < 8; ++tt)
              pv[tt] = static_cast<__bf16>(fast_exp2(fmaf(sacc[c][8 * u + tt], scale_log2, -m_use)));
#pragma unroll
            for (int tt = 0; tt < 8; tt += 2) {
              bf16x2_t pr = {pv[tt], pv[tt + 1]};
              l = add_pair(pr, l);
            }
            pb[c][u] = pv;
          }
          tsum[c] = l;
        }
        // Slow path (rare): a row without reference yet, or keys far above
        // it.  Move the reference to the row max, redo P, rescale the state.
        const bool slow0 = m2[0] == kNegInf || !(tsum[0] <= kRescaleSum);
        const bool slow1 = m2[1] == kNegInf || !(tsum[1] <= kRescaleSum);
        if (wave_any(slow0 || slow1)) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            float mx = sacc[c][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[c][r]);
            mx = pair_max(mx) * scale_log2;
            const bool slow = c == 0 ? slow0 : slow1;
            // the pair agrees on `slow` (same reference, and the pair's
            // sums are compared lane by lane, so make it pair-uniform)
            const bool move = pair_max(slow ? 1.0f : 0.0f) > 0.0f && mx > m2[c];
            const float m_new = move ? mx : m2[c];
            const float alpha = move ? fast_exp2(m2[c] - m_new) : 1.0f;
            m2[c] = m_new;
            lsum[c] *= alpha;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[c][db][r] *= alpha;
            const float m_use = m_new == kNegInf ? 0.0f : m_new;
            float l = 0.0f;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              bf16x8_t pv;
#pragma unroll
              for (int tt = 0; tt < 8; ++tt)
                pv[tt] = static_cast<__bf16>(fast_exp2(fmaf(sacc[c][8 * u + tt], scale_log2, -m_use)));
#pragma unroll
              for (int tt = 0; tt < 8; tt += 2) {
                bf16x2_t pr = {pv[tt], pv[tt + 1]};
                l = add_pair(pr, l);
              }
              pb[c][u] = pv;
            }
            tsum[c] = l;
          }
        }
        lsum[0] += tsum[0];
        lsum[1] += tsum[1];

        // O^T += V^T P^T: lane (d = l % 32 of block db, half) reads V rows
        // kb*32 + 16u + 8 half + 0..7 at its column (two transposing reads).
#pragma unroll
        for (int db = 0; db < 2; ++db) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const uint16_t* vp = vt + vbase + kb * 32 * kHeadDim + 1024 * u;
            const bf16x8_t a = cat4(lds_read_tr(vp + 32 * db), lds_read_tr(vp + 256 + 32 * (db ^ 1)));
            acc[0][db] = mfma_32x32x16(a, pb[0][u], acc[0][db]);
            acc[1][db] = mfma_32x32x16(a, pb[1][u], acc[1][db]);
          }
        }
      }
    }

    if (more) store_tile(regs, k_lds[buf ^ 1], v_lds[buf ^ 1], tid);
    __syncthreads();
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
  const bool windowed = a.window > 0 && a.window < a.max_seqlen;
  auto kernel = windowed ? prefill_kernel<true> : prefill_kernel<false>;
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.sinks, a.cu_seqlens, a.num_q_heads,
                     a.num_kv_heads, group, n_hchunk, n_qtiles, a.window,
                     a.softmax_scale * kLog2e, static_cast<uint16_t*>(a.o), a.lse);
  return hipGetLastError();
}

int prefill_max_qtiles() { return 65535; }
int prefill_qtile() { return kQTile; }

}  // namespace sinkattn
