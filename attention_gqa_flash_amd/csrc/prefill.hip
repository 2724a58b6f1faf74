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

constexpr int kQTile = 32;  // query tokens per workgroup
#ifndef SINKATTN_PREFILL_KTILE
#define SINKATTN_PREFILL_KTILE 128
#endif
constexpr int kKTile = SINKATTN_PREFILL_KTILE;  // keys per LDS tile (32-key halves)
constexpr int kHalves = kKTile / 32;
constexpr int kHeadsPerBlock = 8;
// kCols query heads ("column blocks" of 32 columns) per wave; the workgroup
// has 8 / kCols waves.
template <int kCols>
constexpr int threads_for() { return 64 * (kHeadsPerBlock / kCols); }
#ifndef SINKATTN_PREFILL_COLS
#define SINKATTN_PREFILL_COLS 2
#endif
constexpr int kColsPerWave = SINKATTN_PREFILL_COLS;
// Lazy reference max.  Probabilities are taken against a per-row reference
// m (log2 units) that only moves when the new keys push a row's partial
// denominator past 2^32 (or when the row has no reference yet); the running
// output and denominator are then rescaled.  Values below the reference by
// more than 126 underflow to 0, which is exact to fp32 precision relative to
// the reference's own weight (>= 1) already counted.  o = acc / l is
// unchanged in exact arithmetic.
constexpr float kRescaleSum = 4294967296.0f;  // 2^32

// Issue the copy of one K/V tile (kKTile rows x 8 16-byte chunks of each)
// HBM -> LDS without passing through registers (global_load_lds).  Slot n
// = 64 (kPer wave + i) + lane of the tile holds row n / 8, chunk position
// n % 8, which under the chunk swizzle is global chunk (n % 8) ^ swz_f(row).  Rows past the sequence end are clamped to its
// last key: they only ever meet masked logits.
template <int kThreads>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                           uint16_t* k_dst, uint16_t* v_dst, int seq0, int len, int hkv,
                                           int g, int key0, int wave, int lane) {
  constexpr int kPer = kKTile * 8 / kThreads;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int slot0 = 64 * (kPer * wave + i);
    const int row = (slot0 >> 3) + (lane >> 3);
    const int chunk = (lane & 7) ^ swz_f(row);
    const int key = min(key0 + row, len - 1);
    const size_t off = (static_cast<size_t>(seq0 + key) * hkv + g) * kHeadDim + chunk * 8;
    load16_to_lds_untracked(k + off, k_dst + slot0 * 8);
    load16_to_lds_untracked(v + off, v_dst + slot0 * 8);
  }
}

// P (bf16, the B operand of O^T) for one 32-key half of one column block
// against the reference max m_use (log2 units); returns this lane's partial
// sum of the bf16-rounded probabilities (two independent chains, one per
// 16-key step, to keep the dependency chain short).
__device__ __forceinline__ float probs(const f32x16_t& sacc, bf16x8_t (&pb)[2], float m_use, float scale_log2) {
  float l[2] = {0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    bf16x8_t pv;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
      pv[tt] = static_cast<__bf16>(fast_exp2(fmaf(sacc[8 * u + tt], scale_log2, -m_use)));
#pragma unroll
    for (int tt = 0; tt < 8; tt += 2) {
      bf16x2_t pr = {pv[tt], pv[tt + 1]};
      l[u] = add_pair(pr, l[u]);
    }
    pb[u] = pv;
  }
  return l[0] + l[1];
}

template <bool kWindow, int kCols>
__global__ __launch_bounds__(threads_for<kCols>()) __attribute__((amdgpu_waves_per_eu(4 / kCols, 4 / kCols))) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ sinks,
    const int32_t* __restrict__ cu_seqlens, int hq, int hkv, int group, int n_hchunk,
    int n_qtiles, int window, float scale_log2, uint16_t* __restrict__ o,
    float* __restrict__ lse) {
  // Two LDS tile buffers (K rows then V rows): tile t+1 is written while
  // tile t is read.  They are separate arrays, and every access names one of
  // them statically (tiles are processed in pairs), so the compiler can tell
  // that the asynchronous copy into one buffer does not touch the other and
  // does not make reads of the current tile wait for the next one.
  __shared__ __attribute__((aligned(16))) uint16_t kv_lds0[2 * kKTile * kHeadDim];
  __shared__ __attribute__((aligned(16))) uint16_t kv_lds1[2 * kKTile * kHeadDim];

  constexpr int kThreads = threads_for<kCols>();
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
  issue_tile<kThreads>(k, v, kv_lds0, kv_lds0 + kKTile * kHeadDim, seq0, len, hkv, g, t_begin * kKTile,
                       wave, lane);

  // Query heads of this wave (kCols column blocks of 32).
  int head[kCols];
  bool head_ok[kCols];
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
    const int slot = hchunk * kHeadsPerBlock + wave * kCols + c;
    head_ok[c] = slot < group;
    head[c] = g * group + (head_ok[c] ? slot : 0);
  }
  const bool wave_active = head_ok[0];
  const int qtok = q0 + col;
  const bool row_ok = qtok < len;

  // Q^T as the B operand: lane holds query column `col`, d = 16 s + 8 half + t.
  bf16x8_t qreg[kCols][4];
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
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
  float m2[kCols], lsum[kCols];
  f32x16_t acc[kCols][2];
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
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

  wait_vmem();
  __syncthreads();

  // LDS read offsets (elements, within a 32-row half of a tile).  K rows as
  // the A operand: row key_of_row(col), d = 16 s + 8 half.  V^T operand:
  // lane (d = l % 32 of block db, half) needs rows 16 u + 8 half + 0..7 at
  // its column, as two transposing reads of 4 rows (i = 0, 1); the swizzle
  // depends on the row's low four bits only, so read (db, u, i) sits at
  // voff[db][i] + 1024 u.
  int koff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = swz(key_of_row(col), 16 * s + 8 * half);
  const int grp_lane = lane & 15;
  const int dcol0 = 16 * ((lane >> 4) & 1) + 4 * (grp_lane & 3);
  int voff[2][2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int i = 0; i < 2; ++i) voff[db][i] = swz(8 * half + (grp_lane >> 2) + 4 * i, 32 * db + dcol0);

  // Keys are walked in 32-key halves h_begin..h_end (every half holds a key
  // some query of the tile sees); tiles of kKTile keys are what is staged.
  const int h_begin = first_key >> 5;
  const int h_end = last_q >> 5;

  // Operands are read from LDS one step ahead of the MFMAs that use them:
  // K of the next half during the current half, V of a half before its
  // softmax, so the LDS latency overlaps other work.
  bf16x8_t kop[4];
  bf16x8_t vop[2][2];
  auto read_k = [&](const uint16_t* kt) {
#pragma unroll
    for (int s = 0; s < 4; ++s) kop[s] = *reinterpret_cast<const bf16x8_t*>(kt + koff[s]);
  };
  auto read_v = [&](const uint16_t* vt) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        vop[db][u] = cat4(lds_read_tr(vt + voff[db][0] + 1024 * u), lds_read_tr(vt + voff[db][1] + 1024 * u));
  };

  // Softmax of column block c for one unmasked half: P against the current
  // reference, and in the rare slow case (a row without reference yet, or
  // keys far above it) the reference moves to the row max (uniformly over
  // the lane pair), the state is rescaled and P is redone.
  auto softmax_block = [&](int c, const f32x16_t& s_c, bf16x8_t (&pb_c)[2]) {
    float tsum = probs(s_c, pb_c, m2[c] == kNegInf ? 0.0f : m2[c], scale_log2);
    const bool slow = m2[c] == kNegInf || !(tsum <= kRescaleSum);
    if (wave_any(slow)) {
      float mx = s_c[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s_c[r]);
      mx = pair_max(mx) * scale_log2;
      const bool move = pair_max(slow ? 1.0f : 0.0f) > 0.0f && mx > m2[c];
      const float m_new = move ? mx : m2[c];
      const float alpha = move ? fast_exp2(m2[c] - m_new) : 1.0f;
      m2[c] = m_new;
      lsum[c] *= alpha;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][db][r] *= alpha;
      tsum = probs(s_c, pb_c, m_new == kNegInf ? 0.0f : m_new, scale_log2);
    }
    lsum[c] += tsum;
  };

  // Causal / window mask of column block c (a half crossing the diagonal or
  // the window's lower edge).
  auto mask_block = [&](int kbase, f32x16_t& s_c) {
    // Register r of this lane holds key kbase + key_of_reg(r, half); compare
    // the compile-time part key_of_reg(r, 0) against the query's distance.
    const int lim = qtok - kbase - 8 * half;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = key_of_reg(r, 0);
      const bool ok = off <= lim && (!kWindow || off > lim - window);
      if (!ok) s_c[r] = kNegInf;
    }
  };

  // One 32-key half.  vt points at its V rows in LDS, kt_next at the K rows
  // of the next half (read unconditionally, which keeps the half free of
  // extra branches).  The column blocks are staggered so
  // that the softmax (VALU) of block c overlaps the MFMAs of S for block
  // c + 1 and of O^T for block c - 1:
  //   S_0 | S_1 + softmax_0 | PV_0 + softmax_1 | PV_1.
  // The K rows of the next half are read once the last S MFMA has taken its
  // operands, so they can reuse the same registers.  The (rare) mask of block
  // c sits just before the block that holds softmax_c.
  auto step = [&](int hh, const uint16_t* vt, const uint16_t* kt_next) {
    const int kbase = hh * 32;
    const bool need_mask = (kbase + 31 > q0) || (kWindow && kbase <= last_q - window);
    f32x16_t sacc[kCols];
    bf16x8_t pb[kCols][2];
    auto s_chain = [&](int c) {
      sacc[c] = zero16();
#pragma unroll
      for (int s = 0; s < 4; ++s) sacc[c] = mfma_32x32x16(kop[s], qreg[c][s], sacc[c]);
    };
    auto pv_chain = [&](int c) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[c][db] = mfma_32x32x16(vop[db][u], pb[c][u], acc[c][db]);
    };
    s_chain(0);
    read_v(vt);
    if (need_mask) mask_block(kbase, sacc[0]);
#pragma unroll
    for (int c = 1; c < kCols; ++c) s_chain(c);
    softmax_block(0, sacc[0], pb[0]);
    read_k(kt_next);
#pragma unroll
    for (int c = 1; c < kCols; ++c) {
      if (need_mask) mask_block(kbase, sacc[c]);
      pv_chain(c - 1);
      softmax_block(c, sacc[c], pb[c]);
    }
    pv_chain(kCols - 1);
  };

  // All halves of tile t, which sits in buffer `cur`; at the tile boundary
  // the next tile (buffer `nxt`, issued one tile ago) is waited for and
  // published, and the tile after it is issued into `cur`, whose reads the
  // barrier has retired.
  auto run_tile = [&](int t, uint16_t* cur, uint16_t* nxt) {
    // The halves of a tile are unrolled so that every LDS address is a
    // per-lane base plus an immediate offset.  The K rows read after the
    // last half of the range come from a fixed slot of the current tile;
    // they are either overwritten after the barrier or never used.
    const int ib = max(h_begin - t * kHalves, 0);
    const int ie = min(h_end - t * kHalves, kHalves - 1);
    if (wave_active) {
#pragma unroll
      for (int i = 0; i < kHalves; ++i) {
        if (i >= ib && i <= ie)
          step(t * kHalves + i, cur + kKTile * kHeadDim + i * 32 * kHeadDim,
               cur + ((i + 1) % kHalves) * 32 * kHeadDim);
      }
    }
    if (t < t_end) {
      wait_vmem();
      __syncthreads();
      if (t + 2 <= t_end)
        issue_tile<kThreads>(k, v, cur, cur + kKTile * kHeadDim, seq0, len, hkv, g, (t + 2) * kKTile, wave,
                             lane);
      if (wave_active) read_k(nxt);
    }
  };

  if (t_begin < t_end)
    issue_tile<kThreads>(k, v, kv_lds1, kv_lds1 + kKTile * kHeadDim, seq0, len, hkv, g, (t_begin + 1) * kKTile,
                         wave, lane);
  if (wave_active) read_k(kv_lds0 + (h_begin - t_begin * kHalves) * 32 * kHeadDim);
  for (int t = t_begin; t <= t_end; t += 2) {
    run_tile(t, kv_lds0, kv_lds1);
    if (t + 1 <= t_end) run_tile(t + 1, kv_lds1, kv_lds0);
  }

  if (!wave_active) return;

  // Epilogue: full denominator over the lane pair, normalise, store bf16.
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
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
  auto kernel = windowed ? prefill_kernel<true, kColsPerWave> : prefill_kernel<false, kColsPerWave>;
  hipLaunchKernelGGL(kernel, grid, dim3(threads_for<kColsPerWave>()), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.sinks, a.cu_seqlens, a.num_q_heads,
                     a.num_kv_heads, group, n_hchunk, n_qtiles, a.window,
                     a.softmax_scale * kLog2e, static_cast<uint16_t*>(a.o), a.lse);
  return hipGetLastError();
}

int prefill_max_qtiles() { return 65535; }
int prefill_qtile() { return kQTile; }

}  // namespace sinkattn
