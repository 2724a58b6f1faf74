// Split-KV decode with per-head sinks, and the log-sum-exp merge (gfx950).
//
// Operation: Perplexity, "GPT-OSS on day 0", section "GPT-OSS kernels / Sink
// attention": attention is parallelised over heads and over the KV length;
// when the KV length is split into chunks, the sink-initialised running max
// (and the denominator's initial 1) belongs to the first chunk only.  The
// partial results are combined with the log-sum-exp merge that the running
// (max, denominator) pair implies (the page does not print the formula).
//
// Decode kernels: a wave streams keys of one KV head once and applies them to
// all G query heads of that KV head (the G heads are the N columns of
// S^T = K Q^T).  Workgroups: one per (sequence, KV head, split) whose 2 or 4
// waves walk interleaved 32-key tiles of the chunk with their own online-
// softmax states, merged through LDS at the end (decode_kernel_w2/_w4); one
// per (sequence, KV head, 4 splits) with a split per wave (decode_kernel_ps);
// one per (sequence, pair of KV heads, split) with four interleaved waves
// per head (decode_kernel_w8p, one long split), or per (sequence, KV head)
// with eight (decode_kernel_w8, one long split over few KV heads); or, with four or more
// splits, one per (sequence, split) with a wave per KV head
// (decode_kernel_hw).  The last two read adjacent pieces of the same token
// rows of the cache from one workgroup, which streams faster.  E4M3 caches
// with one query token, G <= 8 and an even number of KV heads take
// decode_kernel_pair: a wave streams both heads of a pair (128 contiguous
// bytes per token) with its 16 MFMA columns split between them.  K and V rows are read with fully
// coalesced 16-byte loads (8 lanes per 128-byte row; a key row of one head is
// 128 contiguous bytes, rows are Hkv * 128 bytes apart), the next tile of a
// wave is in flight while the current one is computed, and each tile passes
// through a wave-private LDS tile: K is read back in MFMA A-operand order, V
// with the transposing read that O^T = V^T P^T needs.
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace sinkattn {

namespace {

constexpr int kThreads = 256;  // merge kernel: 4 waves, one row each
constexpr int kWaves = 4;
constexpr int kKeys = 32;  // keys per wave iteration
// The decode workgroup has kDecWaves waves: 4 for long key chunks, 2 when a
// chunk holds at most kShortChunk keys (fewer waves to merge per workgroup,
// twice the workgroups resident per CU).
constexpr int kShortChunk = 1024;
// With at least kSplitPerWaveMin splits of more than kShortChunk keys, each
// wave of a four-wave workgroup owns a split (64 x 8192 at S = 4: 6.0 TB/s
// against 5.5 with the waves interleaved; at S = 16, 512-key splits, the
// two-wave interleaved kernel is 12% faster).
constexpr int kSplitPerWaveMin = 4;
// ... when that still launches at least this many workgroups; fewer (few KV
// heads: 64 x 8192 with 16 / 2 heads at S = 4 has 128) leave most CUs idle,
// and the four-wave interleaved kernel takes the splits one workgroup each.
constexpr long long kSplitPerWaveMinGroups = 256;
// A single long split serves pairs of KV heads per workgroup (w8p) when
// that gives at least this many workgroups; fewer (64 x 8192 with 16 / 2
// heads: 64) take one KV head per workgroup (w8) for twice as many.
constexpr long long kPairMinGroups = 128;
// Online softmax: the reference maximum (log2 units) is raised only when a
// logit passes it by more than this, so most tiles skip the rescale of the
// output accumulators; the unnormalised weights stay below 2^kLazyLog2.
constexpr float kLazyLog2 = 8.0f;
// With at least kHeadPerWaveMinSplits splits of at least kHeadPerWaveMinKeys
// keys over 4 to 8 KV heads, a workgroup is one (sequence, split) and its
// waves are the KV heads (decode_kernel_hw): 64 x 8192 at S = 4 from 182 to
// 167 us, 16 x 32768 at S = 32 from 180 to 171 us.  (Forcing four waves per
// SIMD spills and runs 20-40% slower.)
constexpr int kHeadPerWaveMinSplits = 4;
constexpr int kHeadPerWaveMinKeys = 128;
// ... and only when sequences x splits give enough workgroups: at least
// twice this many, or at least this many when the split-per-wave kernel
// (long splits) is not the alternative.  Below that (one or a few long
// sequences split a few ways) the layouts with a workgroup per (sequence,
// KV head, split) keep more CUs busy: 1 x 131072 at S = 16 0.304 -> 0.077
// ms, 4 x 32768 at S = 8 0.160 -> 0.056 ms, 8 x 8192 at S = 4 0.084 ->
// 0.033 ms.  Between the two bounds the split-per-wave kernel is faster
// (16 x 32768 at S = 8 0.188 -> 0.178 ms, 32 x 8192 at S = 4 0.103 ->
// 0.095 ms) and the short-split two-wave kernel slower (4 x 32768 at S = 32,
// 8 x 8192 at S = 16 keep this layout).
constexpr long long kHeadPerWaveMinUnits = 128;
// Consecutive splits of a sequence share a decode_kernel_hw workgroup when
// the launch would otherwise exceed about kHeadPerWaveTarget workgroups (two
// per CU): 64 x 8192 at S = 16, 184 to 180 us.
constexpr long long kHeadPerWaveTarget = 512;
// Splits of at most kKeys keys over a range of at most kDirectMaxKeys keys
// (window layers cut into many splits) are not formed: the merge of
// normalised split partials is exact, so it equals attention over the whole
// range, which one workgroup per (sequence, KV head) evaluates in a third of
// the time the partials and their merge take (16 x 32768 cached tokens,
// 128-key window, 32 splits: 4.9 against 13.5 us back to back).
constexpr int kDirectMaxKeys = 1024;
// A range of at most kDirectWholeKeys keys (a 128-key window layer, also
// with a few query tokens before it) is evaluated whole at any split count:
// 64 x 4 draft tokens with a 128-key window, 4 splits of 33 keys, took
// 0.040 ms split and merged against 0.019 ms as one range.
constexpr int kDirectWholeKeys = 256;

// One 32-key tile of one wave, in registers, K and V rows in coalesced
// order.  bf16 cache: lane l holds the 16-byte chunk l % 8 of rows
// l / 8 + 8 i (a head's row is 128 bytes).  FP8 (E4M3) cache: lane l holds the
// 16-byte chunk l % 4 (16 codes) of rows l / 4 + 16 i (a head's row is 64
// bytes).  Rows at or beyond `end` (> k0) repeat row end - 1: their logits
// are masked to -inf, so their weights are 0 and the (finite) V values drop
// out.
template <bool kFp8>
struct TileRegs {
  u32x4_t k[kFp8 ? 2 : 4];
  u32x4_t v[kFp8 ? 2 : 4];
};

template <bool kFp8>
__device__ __forceinline__ void load_tile(TileRegs<kFp8>& t, const void* __restrict__ k,
                                          const void* __restrict__ v, int base, int hkv, int g,
                                          int k0, int end, int lane) {
  if constexpr (kFp8) {
    const uint8_t* kb = static_cast<const uint8_t*>(k);
    const uint8_t* vb = static_cast<const uint8_t*>(v);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = min(k0 + (lane >> 2) + 16 * i, end - 1);
      const size_t off = (static_cast<size_t>(base + key) * hkv + g) * kHeadDim + (lane & 3) * 16;  // bytes
      // Cached loads: a head's 64-byte row is half of a 128-byte line whose
      // other half another wave or workgroup reads soon after (nontemporal
      // loads fetched 10-24% of the bytes twice; 64 x 8192: S = 1 0.119 ->
      // 0.113 ms, S = 16 0.138 -> 0.122 ms).
      t.k[i] = load16(reinterpret_cast<const uint16_t*>(kb + off));
      t.v[i] = load16(reinterpret_cast<const uint16_t*>(vb + off));
    }
  } else {
    const uint16_t* kh = static_cast<const uint16_t*>(k);
    const uint16_t* vh = static_cast<const uint16_t*>(v);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(k0 + (lane >> 3) + 8 * i, end - 1);
      const size_t off = (static_cast<size_t>(base + key) * hkv + g) * kHeadDim + (lane & 7) * 8;
      t.k[i] = load16_stream(kh + off);
      t.v[i] = load16_stream(vh + off);
    }
  }
}

// Paged cache: pages [num_pages, 1 << page_shift, hkv, 64] (bf16, or E4M3
// codes with kFp8); key j of the sequence is slot j & (page_size - 1) of page
// row[j >> page_shift].  A 32-key tile spans at most three pages when
// page_size >= 16: PageIds holds the ids of pages p0, p0 + 1, p0 + 2 of one
// sequence, uniform over the wave, clamped to the pool so that a bad table
// cannot move an access out of bounds.  The ids must stay in registers: a
// choice among them by index makes the compiler keep them in memory, one
// copy per work-item (8 KB of LDS per 512-thread workgroup, or scratch when
// LDS is full), so a row's page id is formed from their differences.
struct PageIds {
  int p0, id0, id1, id2;
};

// Reads the ids of pages p0 .. p0 + 2 (entries past the sequence's last page
// `plast` repeat it, so no entry past the table row is read).
__device__ __forceinline__ void fetch_page_ids(PageIds& p, const int32_t* __restrict__ row, int p0, int plast,
                                               int num_pages) {
  auto id = [&](int page) { return min(max(row[min(page, plast)], 0), num_pages - 1); };
  p.p0 = p0;
  p.id0 = id(p0);
  p.id1 = id(p0 + 1);
  p.id2 = id(p0 + 2);
}

// Lanes take the same keys and 16-byte pieces as load_tile; rows at or beyond
// `end` repeat row end - 1.  pid covers page k0 >> page_shift.
// Cache row (token slot in the pool) of key `key` of the tile whose pages
// pid covers.
__device__ __forceinline__ size_t paged_token(const PageIds& pid, int page_shift, int key) {
  const int rel = (key >> page_shift) - pid.p0;  // 0, 1 or 2
  // (as differences: written as a choice among the three ids, the compiler
  // builds a per-work-item table in memory to index)
  const int id = pid.id0 + (rel >= 1 ? pid.id1 - pid.id0 : 0) + (rel >= 2 ? pid.id2 - pid.id1 : 0);
  return (static_cast<size_t>(id) << page_shift) + (key & ((1 << page_shift) - 1));
}

template <bool kFp8>
__device__ __forceinline__ void load_tile_paged(TileRegs<kFp8>& t, const void* __restrict__ k,
                                                const void* __restrict__ v, const PageIds& pid, int page_shift,
                                                int hkv, int g, int k0, int end, int lane) {
  auto token = [&](int key) { return paged_token(pid, page_shift, key); };
  if constexpr (kFp8) {
    const uint8_t* kb = static_cast<const uint8_t*>(k);
    const uint8_t* vb = static_cast<const uint8_t*>(v);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = min(k0 + (lane >> 2) + 16 * i, end - 1);
      const size_t off = (token(key) * hkv + g) * kHeadDim + (lane & 3) * 16;  // bytes
      t.k[i] = load16(reinterpret_cast<const uint16_t*>(kb + off));
      t.v[i] = load16(reinterpret_cast<const uint16_t*>(vb + off));
    }
  } else {
    const uint16_t* kh = static_cast<const uint16_t*>(k);
    const uint16_t* vh = static_cast<const uint16_t*>(v);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(k0 + (lane >> 3) + 8 * i, end - 1);
      const size_t off = (token(key) * hkv + g) * kHeadDim + (lane & 7) * 8;
      t.k[i] = load16_stream(kh + off);
      t.v[i] = load16_stream(vh + off);
    }
  }
}

// 16 E4M3 codes (one 16-byte chunk) -> 16 bf16 in two 16-byte halves.  E4M3
// values are exactly representable in bf16; the conversion runs with scale 1.
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4_t c, u32x4_t& lo, u32x4_t& hi) {
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[j], 1.0f, false));
    w[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[j], 1.0f, true));
  }
  lo = u32x4_t{w[0], w[1], w[2], w[3]};
  hi = u32x4_t{w[4], w[5], w[6], w[7]};
}

// The tile into the wave's LDS staging (bf16, swizzled rows of 64 values).
template <bool kFp8>
__device__ __forceinline__ void stage_tile(const TileRegs<kFp8>& cur, uint16_t* kt, uint16_t* vt, int lane) {
  if constexpr (kFp8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (lane >> 2) + 16 * i;
      const int c0 = (lane & 3) * 16;
      u32x4_t lo, hi;
      e4m3x16_to_bf16(cur.k[i], lo, hi);
      *reinterpret_cast<u32x4_t*>(kt + swz(r, c0)) = lo;
      *reinterpret_cast<u32x4_t*>(kt + swz(r, c0 + 8)) = hi;
      e4m3x16_to_bf16(cur.v[i], lo, hi);
      *reinterpret_cast<u32x4_t*>(vt + swz(r, c0)) = lo;
      *reinterpret_cast<u32x4_t*>(vt + swz(r, c0 + 8)) = hi;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (lane >> 3) + 8 * i;
      const int dst = swz(r, (lane & 7) * 8);
      *reinterpret_cast<u32x4_t*>(kt + dst) = cur.k[i];
      *reinterpret_cast<u32x4_t*>(vt + dst) = cur.v[i];
    }
  }
}

// MFMA column layouts of a decode wave (the N side of S^T = K Q^T: one
// column per (query token, query head) pair).
//   kN = 16: one v_mfma_f32_16x16x32_bf16 block: lane l holds column l % 16;
//            S^T C registers i of key block kb are key 8 (l / 16) + 4 kb + i
//            (rows permuted by key16_of_row) and O^T registers i of d block
//            db are d = 16 db + 4 (l / 16) + i.  Half the matrix-core work
//            and half the softmax lanes of the 32-column layout: the layout
//            for GQA groups of at most 16 (G = 8: 8 of 16 columns real
//            instead of 8 of 32).
//   kN = 32: one v_mfma_f32_32x32x16_bf16 block (key_of_row, key_of_reg).
//   kN = 64: two 32-column blocks sharing every K and V operand read: draft
//            tokens with Lq * G of 33 to 64 columns (5 to 8 tokens at G = 8)
//            in one pass over the keys.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_16x16x32(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Key (within a 32-key tile) read by A-operand row m of key block kb, so that
// C register i of lane group q is key 8 q + 4 kb + i: the 8 keys of a lane
// group are then exactly the k slots 8 q + 0..7 of the B operand of
// O^T = V^T P^T.
__device__ __forceinline__ int key16_of_row(int m, int kb) { return 8 * (m >> 2) + 4 * kb + (m & 3); }

// Max / sum over the four lanes l % 16 of a column (16-column layout).
__device__ __forceinline__ float quad_max(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return pair_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quad_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return pair_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

template <int kN>
struct DecodeCols {
  static constexpr bool k16 = kN == 16;
  static constexpr int kBlocks = kN == 64 ? 2 : 1;  // column blocks per wave
  static constexpr int kBlockCols = k16 ? 16 : 32;
  static constexpr int kQRegs = k16 ? 2 : 4;        // bf16x8 Q^T operands per block
  typedef typename std::conditional<k16, f32x4_t, f32x16_t>::type Acc;  // one C block
  static constexpr int kAccBlocks = k16 ? 4 : 2;    // d blocks of O^T
  static constexpr int kAccRegs = k16 ? 4 : 16;
  static constexpr int kSBlocks = k16 ? 2 : 1;      // key blocks of S^T per 32-key tile
};

// kSplitPerWave: each wave owns one whole split (split = 4 * group of
// splits + wave) and writes that split's partial itself; kHeadPerWave: the
// workgroup is one (sequence, split) and wave w takes KV head w of it, so the
// waves together read whole 1 KB token rows (all KV heads) at about the same
// time, which streams faster than 128-byte pieces 1 KB apart read by
// separate workgroups (6.9 against 6.2 TB/s, measured with plain loads);
// otherwise the waves of the workgroup interleave over one split and merge
// through LDS.
//
// kMulti (multi-token-query decode): sequence b's last nq_b tokens are
// queries (rows cu_seqlens_q[b] .. of q, o and the partials), and MFMA
// column c = t * group + h serves token t and query head h of the group, so
// one pass over the keys serves every query token (nq_b * group <= ncols <=
// kN columns).  Token t sits at position len - nq_b + t and sees the keys at
// or before it (and, with a window W, after position - W): the causal mask
// aligned at the bottom right, applied per column.
//
// kPaged: the cache is paged (load_tile_paged); cu_seqlens_k then holds the
// sequence lengths [batch] instead of offsets.
template <int kDecWaves, bool kSplitPerWave, bool kHeadPerWave = false, int kHeadsPerWG = 1, bool kFp8 = false,
          bool kMulti = false, bool kPaged = false, int kN = 32>
__device__ __forceinline__ void decode_body(
    const uint16_t* __restrict__ q, const void* __restrict__ k,
    const void* __restrict__ v, const float* __restrict__ sinks,
    const int32_t* __restrict__ cu_seqlens_k, int batch, int hq, int hkv, int group,
    int window, float scale_log2, int num_splits, uint16_t* __restrict__ o,
    float* __restrict__ lse, float* __restrict__ o_part, float* __restrict__ lse_part, int splits_per_wg,
    float v_scale, const int32_t* __restrict__ cu_seqlens_q, int ncols, int out_rows,
    const int32_t* __restrict__ block_table, int max_pages, int page_shift, int num_pages) {
  typedef DecodeCols<kN> L;
  constexpr int kCB = L::kBlocks;
  // Wave-private K and V staging tiles (2 x 4 KiB per wave); the whole
  // buffer is reused for the cross-wave merge of up to 32 columns x 64 d per
  // wave and column block (index (wave * cols + column) * 64 + d).
  __shared__ __attribute__((aligned(16))) float lds_buf[kDecWaves * 32 * kHeadDim];
  __shared__ float red_m[kDecWaves][32];
  __shared__ float red_l[kDecWaves][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lc = L::k16 ? (lane & 15) : (lane & 31);  // column within a block
  const int lq = L::k16 ? (lane >> 4) : (lane >> 5);  // k group of the MFMA operands

  constexpr bool kOwnSplit = kSplitPerWave || kHeadPerWave;  // the wave streams its range alone
  // kHeadsPerWG > 1 (interleaved mode): the workgroup serves kHeadsPerWG
  // adjacent KV heads; wave w takes head w % kHeadsPerWG and is the
  // (w / kHeadsPerWG)-th of the kIl waves interleaving over that head's keys.
  constexpr int kIl = kDecWaves / kHeadsPerWG;
  const int hsub = wave % kHeadsPerWG;
  const int wl = wave / kHeadsPerWG;
  int x = blockIdx.x;
  int split;
  int split_stop = 0;  // kHeadPerWave: the workgroup's splits are [split, split_stop)
  if (kHeadPerWave) {
    const int n_sgroups = (num_splits + splits_per_wg - 1) / splits_per_wg;
    split = (x % n_sgroups) * splits_per_wg;
    split_stop = min(num_splits, split + splits_per_wg);
    x = (x / n_sgroups) * hkv + wave;  // (sequence, KV head = wave)
  } else if (kSplitPerWave) {
    const int n_sgroups = (num_splits + kDecWaves - 1) / kDecWaves;
    split = (x % n_sgroups) * kDecWaves + wave;
    x /= n_sgroups;
  } else {
    split = x % num_splits;
    x /= num_splits;
    if (kHeadsPerWG > 1) {
      const int pairs = hkv / kHeadsPerWG;
      x = (x / pairs) * hkv + (x % pairs) * kHeadsPerWG + hsub;
    }
  }
  const int g = x % hkv;
  const int b = x / hkv;

  const int base = kPaged ? 0 : cu_seqlens_k[b];
  const int len = kPaged ? cu_seqlens_k[b] : cu_seqlens_k[b + 1] - base;
  const int32_t* bt_row = kPaged ? block_table + static_cast<size_t>(b) * max_pages : nullptr;
  const int plast = kPaged ? min(max(len - 1, 0) >> page_shift, max_pages - 1) : 0;
  constexpr int kStride = kOwnSplit ? kKeys : kKeys * kIl;  // keys between a wave's tiles
  // Paged bf16: the ids of the pages a tile needs are read one tile ahead (a
  // wave's next tile normally starts kStride keys on), so that the address
  // of each K/V row does not wait for a table read; a tile that starts
  // elsewhere (the next split's first) reads its ids first.  64 x 8192,
  // 16-token pages: S = 1 0.200 -> 0.186 ms, S = 16 0.215 -> 0.203 ms.  The
  // E4M3 tiles read their ids when they are loaded: reading them ahead made
  // no measurable difference there.
  constexpr bool kIdsAhead = kPaged && !kFp8;
  PageIds pids{-1, 0, 0, 0};
  auto load = [&](TileRegs<kFp8>& t, int k_first, int k_end) {
    if constexpr (kPaged) {
      const int p0 = k_first >> page_shift;
      if (!kIdsAhead || p0 != pids.p0) fetch_page_ids(pids, bt_row, p0, plast, num_pages);
      load_tile_paged(t, k, v, pids, page_shift, hkv, g, k_first, k_end, lane);
      if constexpr (kIdsAhead) fetch_page_ids(pids, bt_row, (k_first + kStride) >> page_shift, plast, num_pages);
    } else {
      load_tile(t, k, v, base, hkv, g, k_first, k_end, lane);
    }
  };
  // Query tokens of this sequence (one unless kMulti); more than len breaks
  // a precondition and is clamped.
  int q_row0 = b, nq = 1;
  if constexpr (kMulti) {
    q_row0 = cu_seqlens_q[b];
    nq = min(cu_seqlens_q[b + 1] - q_row0, len);
    if (nq <= 0) return;  // uniform over the workgroup: no query, no output row
  }
  const int lo = window > 0 ? max(0, len - nq - window + 1) : 0;
  const int n = len - lo;
  const int chunk = n > 0 ? (n + num_splits - 1) / num_splits : 0;
  auto split_end = [&](int sp) { return sp < num_splits ? min(len, lo + (sp + 1) * chunk) : len; };
  // (a wave past the last split gets an empty range and writes nothing)
  const int a = split < num_splits ? min(len, lo + split * chunk) : len;
  int e = split_end(split);

  // Column -> (query token, head of the group) per column block;
  // single-token: token 0.
  int tok[kCB], head[kCB], qrow[kCB], qpos[kCB];
  bool col_ok[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const int c = 32 * cb + lc;
    tok[cb] = kMulti ? c / group : 0;
    col_ok[cb] = kMulti ? tok[cb] < nq : c < group;
    head[cb] = g * group + (col_ok[cb] ? c - tok[cb] * group : 0);
    qrow[cb] = kMulti ? q_row0 + (col_ok[cb] ? tok[cb] : 0) : b;  // row of q / o / partials
    qpos[cb] = len - nq + (col_ok[cb] ? tok[cb] : 0);              // the query's position (kMulti masks)
  }

  uint16_t* kt = reinterpret_cast<uint16_t*>(lds_buf) + wave * 2 * kKeys * kHeadDim;
  uint16_t* vt = kt + kKeys * kHeadDim;
  const int grp_lane = lane & 15;
  const int dcol0 = 16 * ((lane >> 4) & 1) + 4 * (grp_lane & 3);

  // Register double buffering: the loads of the next tile of this wave are in
  // flight while the current one is computed.  The first tile is requested
  // before Q and the sink, so the three latencies overlap.
  TileRegs<kFp8> cur, nxt;
  int k0 = kOwnSplit ? a : a + kKeys * wl;
  if (k0 < e) load(cur, k0, e);

  // Q^T (B operand): column lc of each block, d = (32 or 16) s + 8 lq + t.
  // Every lane loads; columns past the group repeat the group's first head
  // (S columns are independent, and theirs are never written).
  bf16x8_t qreg[kCB][L::kQRegs];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int s = 0; s < L::kQRegs; ++s) {
      const int d0 = (L::k16 ? 32 : 16) * s + 8 * lq;
      const u32x4_t val = load16(q + (static_cast<size_t>(qrow[cb]) * hq + head[cb]) * kHeadDim + d0);
      qreg[cb][s] = __builtin_bit_cast(bf16x8_t, val);
    }
  // The sink belongs to split 0 only (its wave 0 when the waves share a
  // split).  It is folded into the state after the keys (the order of the
  // logits does not matter), so nothing waits for it before the loop.
  float z[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
    z[cb] = (split == 0 && (kOwnSplit || wl == 0) && sinks != nullptr && col_ok[cb]) ? sinks[head[cb]] : kNegInf;
  // Q and the sink are taken into registers before the loop (the first
  // tile, requested before them, has then landed too).  Without this use the
  // compiler's wait counters treat their loads as possibly still in flight
  // inside the loop and wait for every outstanding load there, the next
  // tile's included, which leaves no tile in flight during the computation.
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
#pragma unroll
    for (int s = 0; s < L::kQRegs; ++s) asm volatile("" ::"v"(qreg[cb][s]));
    asm volatile("" ::"v"(z[cb]));
  }
  float m2[kCB], lsum[kCB];
  typename L::Acc acc[kCB][L::kAccBlocks];
  auto reset_state = [&]() {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      m2[cb] = kNegInf;
      lsum[cb] = 0.0f;
#pragma unroll
      for (int db = 0; db < L::kAccBlocks; ++db)
#pragma unroll
        for (int r = 0; r < L::kAccRegs; ++r) acc[cb][db][r] = 0.0f;
    }
  };
  reset_state();
  // d of O^T register r of d block db in this lane.
  auto d_of = [&](int db, int r) {
    return L::k16 ? 16 * db + 4 * lq + r : 32 * db + 8 * (r >> 2) + 4 * lq + (r & 3);
  };
  auto col_sum = [&](float x) { return L::k16 ? quad_sum(x) : pair_sum(x); };
  auto col_max = [&](float x) { return L::k16 ? quad_max(x) : pair_max(x); };

  // The sink: one more logit z (already in natural-log units) with no value.
  auto fold_sink = [&]() {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      if (z[cb] > kNegInf) {
        const float z2 = z[cb] * kLog2e;
        const float m_new = fmaxf(m2[cb], z2);
        const float alpha = fast_exp2(m2[cb] - m_new);  // 0 when no key was seen
        lsum[cb] = lsum[cb] * alpha + (lq == 0 ? fast_exp2(z2 - m_new) : 0.0f);
#pragma unroll
        for (int db = 0; db < L::kAccBlocks; ++db)
#pragma unroll
          for (int r = 0; r < L::kAccRegs; ++r) acc[cb][db][r] *= alpha;
        m2[cb] = m_new;
      }
    }
  };
  // This wave's split sp alone: normalise and write its partial.
  auto write_partial = [&](int sp) {
    if (sp >= num_splits) return;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const float den = col_sum(lsum[cb]);
      if (!col_ok[cb]) continue;
      float inv = den > 0.0f ? 1.0f / den : 0.0f;
      if constexpr (kFp8) inv *= v_scale;  // V = v_scale * e4m3(code)
      const size_t prow = (static_cast<size_t>(sp) * out_rows + qrow[cb]) * hq + head[cb];
#pragma unroll
      for (int db = 0; db < L::kAccBlocks; ++db)
#pragma unroll
        for (int r = 0; r < L::kAccRegs; ++r) o_part[prow * kHeadDim + d_of(db, r)] = acc[cb][db][r] * inv;
      if (lq == 0) lse_part[prow] = den > 0.0f ? (m2[cb] + __log2f(den)) * kLn2 : kNegInf;
    }
  };
  // Key offset (within the tile) of S register r of key block kb in this lane.
  auto key_of = [&](int kb, int r) { return L::k16 ? 8 * lq + 4 * kb + r : key_of_reg(r, lq); };

  // One 32-key tile (keys k0 .. k0 + 31; those at or past `end` masked) into
  // the wave's online-softmax state.
  auto tile_step = [&](const TileRegs<kFp8>& cur, int k0, int end) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // previous tile's LDS reads are done
    stage_tile<kFp8>(cur, kt, vt, lane);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // K and V tiles written

    // S^T = K Q^T.
    typename L::Acc sacc[kCB][L::kSBlocks];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int kb = 0; kb < L::kSBlocks; ++kb)
#pragma unroll
        for (int r = 0; r < L::kAccRegs; ++r) sacc[cb][kb][r] = 0.0f;
    if constexpr (L::k16) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8_t ak = *reinterpret_cast<const bf16x8_t*>(kt + swz(key16_of_row(lc, kb), 32 * s + 8 * lq));
          sacc[0][kb] = mfma_16x16x32(ak, qreg[0][s], sacc[0][kb]);
        }
    } else {
      const int krow = key_of_row(lc);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t ak = *reinterpret_cast<const bf16x8_t*>(kt + swz(krow, 16 * s + 8 * lq));
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) sacc[cb][0] = mfma_32x32x16(ak, qreg[cb][s], sacc[cb][0]);
      }
    }

    if (k0 + kKeys > end) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int kb = 0; kb < L::kSBlocks; ++kb)
#pragma unroll
          for (int r = 0; r < L::kAccRegs; ++r)
            if (k0 + key_of(kb, r) >= end) sacc[cb][kb][r] = kNegInf;
    }
    if constexpr (kMulti) {
      // Per-column causal / window mask where the tile reaches past the
      // first query's position or below the last query's window.
      if (k0 + kKeys - 1 > len - nq || (window > 0 && k0 <= len - 1 - window)) {
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
          for (int kb = 0; kb < L::kSBlocks; ++kb)
#pragma unroll
            for (int r = 0; r < L::kAccRegs; ++r) {
              const int key = k0 + key_of(kb, r);
              if (key > qpos[cb] || (window > 0 && key <= qpos[cb] - window)) sacc[cb][kb][r] = kNegInf;
            }
      }
    }

    // P (B operand of O^T = V^T P^T): 32-column layout: pb[cb][u][t] is key
    // 16 u + 8 lq + t; 16-column layout: pb[0][0][4 kb + i] is key
    // 8 lq + 4 kb + i.
    bf16x8_t pb[kCB][L::k16 ? 1 : 2];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      float mx = sacc[cb][0][0];
#pragma unroll
      for (int kb = 0; kb < L::kSBlocks; ++kb)
#pragma unroll
        for (int r = 0; r < L::kAccRegs; ++r) mx = fmaxf(mx, sacc[cb][kb][r]);
      mx = col_max(mx) * scale_log2;
      // The reference m2 moves lazily (the wave's columns together): only
      // when a column's tile maximum passes its reference by more than
      // kLazyLog2 are the references raised to the running maxima and the
      // state rescaled; otherwise the weights stay below 2^kLazyLog2 and the
      // rescale of the accumulators is skipped.
      if (__builtin_amdgcn_ballot_w64(mx > m2[cb] + kLazyLog2) != 0) {
        const float m_new = fmaxf(m2[cb], mx);
        const float alpha = fast_exp2(m2[cb] - ((m_new == kNegInf) ? 0.0f : m_new));
        m2[cb] = m_new;
        lsum[cb] *= alpha;
#pragma unroll
        for (int db = 0; db < L::kAccBlocks; ++db)
#pragma unroll
          for (int r = 0; r < L::kAccRegs; ++r) acc[cb][db][r] *= alpha;
      }
      const float m_use = (m2[cb] == kNegInf) ? 0.0f : m2[cb];
      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < L::kSBlocks; ++kb)
#pragma unroll
        for (int r = 0; r < L::kAccRegs; ++r) {
          const float p = fast_exp2(fmaf(sacc[cb][kb][r], scale_log2, -m_use));
          psum += p;
          if constexpr (L::k16)
            pb[cb][0][4 * kb + r] = static_cast<__bf16>(p);
          else
            pb[cb][r >> 3][r & 7] = static_cast<__bf16>(p);
        }
      lsum[cb] += psum;
    }

    if constexpr (L::k16) {
      // V^T rows d = 16 db + lc, keys 8 lq + 0..7: two transposing reads of
      // 4 key rows each.
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int rbase = 8 * lq + (lc >> 2);
        const int dcol = 16 * db + 4 * (lc & 3);
        const bf16x8_t av = cat4(lds_read_tr(vt + swz(rbase, dcol)), lds_read_tr(vt + swz(rbase + 4, dcol)));
        acc[0][db] = mfma_16x16x32(av, pb[0][0], acc[0][db]);
      }
    } else {
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int rbase = 16 * u + 8 * lq + (grp_lane >> 2);
          const int dcol = 32 * db + dcol0;
          const bf16x8_t av = cat4(lds_read_tr(vt + swz(rbase, dcol)), lds_read_tr(vt + swz(rbase + 4, dcol)));
#pragma unroll
          for (int cb = 0; cb < kCB; ++cb) acc[cb][db] = mfma_32x32x16(av, pb[cb][u], acc[cb][db]);
        }
      }
    }
  };

  if constexpr (kHeadPerWave) {
    // The workgroup's splits one after another: the next split's first tile
    // (it starts where this one ends) is loaded during this split's last, and
    // each split's partial is written when it ends.
    int sp = split;
    while (true) {
      for (; k0 < e; k0 += kKeys) {
        const int k1 = k0 + kKeys;
        if (k1 < e)
          load(nxt, k1, e);
        else if (sp + 1 < split_stop && e < split_end(sp + 1))
          load(nxt, e, split_end(sp + 1));
        tile_step(cur, k0, e);
        cur = nxt;
      }
      fold_sink();
      write_partial(sp);
      if (++sp >= split_stop) return;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) z[cb] = kNegInf;  // the sink belongs to split 0 only
      reset_state();
      k0 = e;
      e = split_end(sp);
    }
  }

  for (; k0 < e; k0 += kStride) {
    const int k1 = k0 + kStride;
    if (k1 < e) load(nxt, k1, e);
    tile_step(cur, k0, e);
    cur = nxt;
  }

  fold_sink();
  if constexpr (kOwnSplit) {
    write_partial(split);
    return;
  }

  // Cross-wave merge, one column block at a time.  Each wave publishes
  // (m, l, unnormalised O) per column.
  const int cols = kMulti ? min(ncols, 32) : group;  // columns per wave and block in red_o
  float* red_o = lds_buf;  // [wave][column][64 d]
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const float den = col_sum(lsum[cb]);
    const int cb_cols = kMulti ? min(ncols - 32 * cb, cols) : cols;  // columns of this block
    __syncthreads();  // all waves are done with their V tiles (or with the previous block's merge)
    if (lq == 0 && lc < 32) {
      red_m[wave][lc] = m2[cb];
      red_l[wave][lc] = den;
    }
    if (col_ok[cb]) {
#pragma unroll
      for (int db = 0; db < L::kAccBlocks; ++db)
#pragma unroll
        for (int r = 0; r < L::kAccRegs; ++r) red_o[(wave * cols + lc) * kHeadDim + d_of(db, r)] = acc[cb][db][r];
    }
    __syncthreads();

    for (int idx = tid; idx < kHeadsPerWG * cb_cols * kHeadDim; idx += 64 * kDecWaves) {
      const int hs = idx / (cb_cols * kHeadDim);  // KV head within the workgroup
      const int hc = (idx / kHeadDim) % cb_cols;  // column within the block
      const int d = idx % kHeadDim;
      const int c = 32 * cb + hc;                 // column of the wave
      const int ct = kMulti ? c / group : 0;      // its query token
      if (kMulti && ct >= nq) continue;
      float big_m = kNegInf;
#pragma unroll
      for (int i = 0; i < kIl; ++i) big_m = fmaxf(big_m, red_m[hs + kHeadsPerWG * i][hc]);
      float out = 0.0f, out_lse = kNegInf;
      if (big_m > kNegInf) {
        float num = 0.0f, tot = 0.0f;
#pragma unroll
        for (int i = 0; i < kIl; ++i) {
          const int w = hs + kHeadsPerWG * i;
          const float sc = fast_exp2(red_m[w][hc] - big_m);
          tot += sc * red_l[w][hc];
          num += sc * red_o[(w * cols + hc) * kHeadDim + d];
        }
        out = num / tot;
        if constexpr (kFp8) out *= v_scale;  // V = v_scale * e4m3(code)
        out_lse = (big_m + __log2f(tot)) * kLn2;
      }
      const int h = (g - hsub + hs) * group + (c - ct * group);
      const int row = kMulti ? q_row0 + ct : b;
      if (num_splits == 1) {
        o[(static_cast<size_t>(row) * hq + h) * kHeadDim + d] = to_bf16_bits(out);
        if (lse != nullptr && d == 0) lse[static_cast<size_t>(row) * hq + h] = out_lse;
      } else {
        const size_t prow = (static_cast<size_t>(split) * out_rows + row) * hq + h;
        o_part[prow * kHeadDim + d] = out;
        if (d == 0) lse_part[prow] = out_lse;
      }
    }
  }
}

// Log-sum-exp merge: one wave per (row, head), lane = d.  The partials of a
// row are read in batches of kMergeBatch (every load of a batch in flight at
// once: one memory latency for up to 32 splits); the running (max, weight
// sum, weighted sum) is updated per batch with the same rescaling as the
// online softmax.
constexpr int kMergeBatch = 32;
// Rows below which a merge of more than kMergeBatch parts gives each row a
// workgroup of several waves (fewer rows than the chip has wave slots).
constexpr int kMergeWideMaxRows = 2048;

// Max / sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// All decode kernels take the same arguments; k and v point at bf16 or, with
// kFp8, E4M3 caches (scale_log2 then includes the K scale; v_scale is applied
// to the outputs).
#define SINKATTN_DECODE_PARAMS                                                                             \
  const uint16_t *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,                  \
      const float *__restrict__ sinks, const int32_t *__restrict__ cu_seqlens_k, int batch, int hq, int hkv, \
      int group, int window, float scale_log2, int num_splits, uint16_t *__restrict__ o, float *__restrict__ lse, \
      float *__restrict__ o_part, float *__restrict__ lse_part, int splits_per_wg, float v_scale,             \
      const int32_t *__restrict__ cu_seqlens_q, int ncols, int out_rows, const int32_t *__restrict__ block_table, \
      int max_pages, int page_shift, int num_pages
#define SINKATTN_DECODE_ARGS                                                                                  \
  q, k, v, sinks, cu_seqlens_k, batch, hq, hkv, group, window, scale_log2, num_splits, o, lse, o_part, lse_part, \
      splits_per_wg, v_scale, cu_seqlens_q, ncols, out_rows, block_table, max_pages, page_shift, num_pages

// Short splits (at most kShortChunk keys): two-wave workgroups at three
// waves per SIMD, i.e. more workgroups and so more loads in flight (two with
// 64 columns, whose state needs the registers).
template <bool kFp8, bool kMulti, bool kPaged, int kN>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(kN == 64 ? 2 : 3, kN == 64 ? 2 : 3))) void decode_kernel_w2(
    SINKATTN_DECODE_PARAMS) {
  decode_body<2, false, false, 1, kFp8, kMulti, kPaged, kN>(SINKATTN_DECODE_ARGS);
}

// Four or more long splits: four-wave workgroups, one split per wave (each
// wave writes its split's partial; no cross-wave merge).
template <bool kFp8, bool kMulti, bool kPaged, int kN>
__global__ __launch_bounds__(256) void decode_kernel_ps(SINKATTN_DECODE_PARAMS) {
  decode_body<4, true, false, 1, kFp8, kMulti, kPaged, kN>(SINKATTN_DECODE_ARGS);
}

// Four or more splits over 4 to 8 KV heads: one workgroup per (sequence,
// split), one wave per KV head.
template <bool kFp8, bool kMulti, bool kPaged, int kN>
__global__ __launch_bounds__(512) void decode_kernel_hw(SINKATTN_DECODE_PARAMS) {
  decode_body<8, false, true, 1, kFp8, kMulti, kPaged, kN>(SINKATTN_DECODE_ARGS);
}

// One split of more than kShortChunk keys over an even number of KV heads:
// eight-wave workgroups serving two adjacent KV heads with four interleaved
// waves each, so that a workgroup reads 256 contiguous bytes of every token
// row it touches (a plain-load probe: 6.4-6.6 TB/s against 6.0-6.2 for one
// head per workgroup; 64 x 8192 at S = 1 from 180 to 165 us).
template <bool kFp8, bool kMulti, bool kPaged, int kN>
__global__ __launch_bounds__(512) void decode_kernel_w8p(SINKATTN_DECODE_PARAMS) {
  decode_body<8, false, false, 2, kFp8, kMulti, kPaged, kN>(SINKATTN_DECODE_ARGS);
}

// One long split when the pairs of KV heads give too few workgroups (few KV
// heads): eight interleaved waves on one KV head, twice the workgroups.
template <bool kFp8, bool kMulti, bool kPaged, int kN>
__global__ __launch_bounds__(512) void decode_kernel_w8(SINKATTN_DECODE_PARAMS) {
  decode_body<8, false, false, 1, kFp8, kMulti, kPaged, kN>(SINKATTN_DECODE_ARGS);
}

// Long splits: four-wave workgroups at the compiler's own register budget
// (two waves per SIMD; at three, S = 4 on 64 x 8192 would end on a
// two-thirds-full round of workgroups).
template <bool kFp8, bool kMulti, bool kPaged, int kN>
__global__ __launch_bounds__(256) void decode_kernel_w4(SINKATTN_DECODE_PARAMS) {
  decode_body<4, false, false, 1, kFp8, kMulti, kPaged, kN>(SINKATTN_DECODE_ARGS);
}

// E4M3 decode over pairs of KV heads (one query token, G <= 8, an even
// number of KV heads).  A head's E4M3 row is 64 bytes, half of the 128-byte
// line the next head's row completes, and waves that each read 64-byte
// pieces 512 bytes apart stream at about 5.7 TB/s, against 6.2-7.0 TB/s for
// waves reading whole 128-byte pieces with nontemporal loads (plain-load
// probes, 64 x 8192 tokens x 8 KV heads).  So a wave here takes both heads
// of a pair: lane l loads 16 bytes of token l / 8 + 8 i (i = 0..3), chunk
// l % 8, of the pair's 128 contiguous bytes, and the 16 MFMA columns carry
// the two heads' query heads (column c: head 2 p + c / 8, query head c % 8
// of its group).  K rows of the two heads feed the A operand of two
// 16x16x32 MFMAs whose B operands are Q^T with the other head's columns
// zeroed, so each column accumulates only its own head's logits; P^T is
// split the same way for O^T = V^T P^T.  Per key and head this is the same
// matrix-core work as the single-head 16-column layout, with every softmax
// lane used.
//
// Workgroup: one (sequence, pair, split) whose kW waves walk interleaved
// 32-key tiles of the split and merge through LDS at the end.
struct PairRegs {
  u32x4_t k[4];
  u32x4_t v[4];
};

// Staging tiles of a wave: K of head 0, K of head 1, V of head 0, V of head
// 1 of the pair, bf16 rows of 64 (the swz layout), each followed by one
// 128-byte row of padding so that a head-1 row sits in the other half of the
// LDS banks from the head-0 row of the same token (the two are written by
// the same 16 lanes).
constexpr int kPairTileElems = kKeys * kHeadDim + 64;
constexpr int kPairStageElems = 4 * kPairTileElems;

// kPW > 1 (with kW = 1): the workgroup is one (sequence, split) and its kPW
// waves take its kPW pairs of KV heads, so that together they read whole
// token rows (8 heads: 512 contiguous bytes).
template <int kW, bool kPaged, int kPW = 1>
__device__ __forceinline__ void decode_pair_body(
    const uint16_t* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ sinks, const int32_t* __restrict__ cu_seqlens_k, int hq, int hkv, int group,
    int window, float scale_log2, int num_splits, uint16_t* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ o_part, float* __restrict__ lse_part, float v_scale, int out_rows,
    const int32_t* __restrict__ block_table, int max_pages, int page_shift, int num_pages) {
  static_assert(kPW == 1 || kW == 1, "pair waves take whole splits");
  __shared__ __attribute__((aligned(16))) uint16_t stage_all[(kW > kPW ? kW : kPW) * kPairStageElems];
  __shared__ float red_m[kW][16];
  __shared__ float red_l[kW][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lc = lane & 15;  // MFMA column
  const int lq = lane >> 4;  // k group of the MFMA operands
  const int npairs = hkv >> 1;
  int x = blockIdx.x;
  const int split = x % num_splits;
  x /= num_splits;
  const int g0 = kPW > 1 ? 2 * wave : 2 * (x % npairs);  // first KV head of the pair
  const int b = kPW > 1 ? x : x / npairs;

  const int hp = lc >> 3;  // head of the pair this column serves
  const bool col_ok = (lc & 7) < group;
  const int head = (g0 + hp) * group + (col_ok ? (lc & 7) : 0);

  const int base = kPaged ? 0 : cu_seqlens_k[b];
  const int len = kPaged ? cu_seqlens_k[b] : cu_seqlens_k[b + 1] - base;
  const int32_t* bt_row = kPaged ? block_table + static_cast<size_t>(b) * max_pages : nullptr;
  const int plast = kPaged ? min(max(len - 1, 0) >> page_shift, max_pages - 1) : 0;
  const int lo = window > 0 ? max(0, len - window) : 0;
  const int n = len - lo;
  const int chunk = n > 0 ? (n + num_splits - 1) / num_splits : 0;
  const int a = min(len, lo + split * chunk);
  const int e = min(len, lo + (split + 1) * chunk);

  const uint8_t* kb8 = static_cast<const uint8_t*>(k);
  const uint8_t* vb8 = static_cast<const uint8_t*>(v);
  // Paged: the ids of the pages a tile needs are read one tile ahead (a
  // wave's next tile starts kKeys * kW keys on), so that no row address of a
  // tile waits for a table read.
  PageIds pids{-1, 0, 0, 0};
  auto load = [&](PairRegs& t, int k0, int end) {
    if constexpr (kPaged) {
      if ((k0 >> page_shift) != pids.p0) fetch_page_ids(pids, bt_row, k0 >> page_shift, plast, num_pages);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(k0 + (lane >> 3) + 8 * i, end - 1);
      const size_t tok = kPaged ? paged_token(pids, page_shift, key) : static_cast<size_t>(base + key);
      const size_t off = (tok * hkv + g0) * kHeadDim + (lane & 7) * 16;  // bytes
      t.k[i] = load16_stream(reinterpret_cast<const uint16_t*>(kb8 + off));
      t.v[i] = load16_stream(reinterpret_cast<const uint16_t*>(vb8 + off));
    }
    if constexpr (kPaged) fetch_page_ids(pids, bt_row, (k0 + kKeys * kW) >> page_shift, plast, num_pages);
  };

  uint16_t* const stage = stage_all + wave * kPairStageElems;
  uint16_t* const kt0 = stage;
  uint16_t* const kt1 = stage + kPairTileElems;
  uint16_t* const vt0 = stage + 2 * kPairTileElems;
  uint16_t* const vt1 = stage + 3 * kPairTileElems;

  PairRegs cur, nxt;
  int k0 = kPW > 1 ? a : a + kKeys * wave;
  if (k0 < e) load(cur, k0, e);

  // Q^T (B operand): column lc, d = 32 s + 8 lq + t; qz[h][s] keeps only the
  // columns of head h of the pair.
  bf16x8_t qz[2][2];
  {
    const bf16x8_t zero = __builtin_bit_cast(bf16x8_t, zero_u32x4());
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4_t val = load16(q + (static_cast<size_t>(b) * hq + head) * kHeadDim + 32 * s + 8 * lq);
      const bf16x8_t qv = __builtin_bit_cast(bf16x8_t, val);
      qz[0][s] = hp == 0 ? qv : zero;
      qz[1][s] = hp == 1 ? qv : zero;
    }
  }
  // The sink (split 0, wave 0), folded in after the keys.
  const float z = (split == 0 && (kPW > 1 || wave == 0) && sinks != nullptr && col_ok) ? sinks[head] : kNegInf;
  // Q and the sink in registers before the loop (see decode_body).
#pragma unroll
  for (int s = 0; s < 2; ++s) asm volatile("" ::"v"(qz[0][s]), "v"(qz[1][s]));
  asm volatile("" ::"v"(z));
  float m2 = kNegInf, lsum = 0.0f;
  f32x4_t acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[db][r] = 0.0f;

  auto tile_step = [&](const PairRegs& t, int k0, int end) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // previous tile's LDS reads are done
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (lane >> 3) + 8 * i;
      const int ch = lane & 7;
      const int d0 = (ch & 3) * 16;
      uint16_t* kt = (ch >> 2) ? kt1 : kt0;
      uint16_t* vt = (ch >> 2) ? vt1 : vt0;
      u32x4_t lo, hi;
      e4m3x16_to_bf16(t.k[i], lo, hi);
      *reinterpret_cast<u32x4_t*>(kt + swz(r, d0)) = lo;
      *reinterpret_cast<u32x4_t*>(kt + swz(r, d0 + 8)) = hi;
      e4m3x16_to_bf16(t.v[i], lo, hi);
      *reinterpret_cast<u32x4_t*>(vt + swz(r, d0)) = lo;
      *reinterpret_cast<u32x4_t*>(vt + swz(r, d0 + 8)) = hi;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // K and V tiles written

    // S^T = K Q^T: C register i of key block kb is key 8 lq + 4 kb + i.
    f32x4_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int off = swz(key16_of_row(lc, kb), 32 * s + 8 * lq);
        const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(kt0 + off);
        const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(kt1 + off);
        sacc[kb] = mfma_16x16x32(a0, qz[0][s], sacc[kb]);
        sacc[kb] = mfma_16x16x32(a1, qz[1][s], sacc[kb]);
      }
    }
    if (k0 + kKeys > end) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (k0 + 8 * lq + 4 * kb + r >= end) sacc[kb][r] = kNegInf;
    }

    // Online softmax (log2 units) and P: pb[4 kb + i] is key 8 lq + 4 kb + i.
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = quad_max(mx) * scale_log2;
    // Lazy reference, as in decode_body.
    if (__builtin_amdgcn_ballot_w64(mx > m2 + kLazyLog2) != 0) {
      const float m_new = fmaxf(m2, mx);
      const float alpha = fast_exp2(m2 - ((m_new == kNegInf) ? 0.0f : m_new));
      m2 = m_new;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[db][r] *= alpha;
    }
    const float m_use = (m2 == kNegInf) ? 0.0f : m2;
    float psum = 0.0f;
    bf16x8_t pb;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = fast_exp2(fmaf(sacc[kb][r], scale_log2, -m_use));
        psum += pr;
        pb[4 * kb + r] = static_cast<__bf16>(pr);
      }
    lsum += psum;
    const bf16x8_t zero = __builtin_bit_cast(bf16x8_t, zero_u32x4());
    const bf16x8_t p0 = hp == 0 ? pb : zero;
    const bf16x8_t p1 = hp == 1 ? pb : zero;

    // O^T += V^T P^T: V^T rows d = 16 db + lc, keys 8 lq + 0..7.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int rbase = 8 * lq + (lc >> 2);
      const int dcol = 16 * db + 4 * (lc & 3);
      const bf16x8_t a0 = cat4(lds_read_tr(vt0 + swz(rbase, dcol)), lds_read_tr(vt0 + swz(rbase + 4, dcol)));
      const bf16x8_t a1 = cat4(lds_read_tr(vt1 + swz(rbase, dcol)), lds_read_tr(vt1 + swz(rbase + 4, dcol)));
      acc[db] = mfma_16x16x32(a0, p0, acc[db]);
      acc[db] = mfma_16x16x32(a1, p1, acc[db]);
    }
  };

  constexpr int kStride = kKeys * kW;
  for (; k0 < e; k0 += kStride) {
    const int k1 = k0 + kStride;
    if (k1 < e) load(nxt, k1, e);
    tile_step(cur, k0, e);
    cur = nxt;
  }

  // The sink: one more logit with no value.
  if (z > kNegInf) {
    const float z2 = z * kLog2e;
    const float m_new = fmaxf(m2, z2);
    const float alpha = fast_exp2(m2 - m_new);  // 0 when no key was seen
    lsum = lsum * alpha + (lq == 0 ? fast_exp2(z2 - m_new) : 0.0f);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[db][r] *= alpha;
    m2 = m_new;
  }
  const float den = quad_sum(lsum);

  auto emit = [&](int col_head, int d, float out, float out_lse) {
    if (num_splits == 1) {
      o[(static_cast<size_t>(b) * hq + col_head) * kHeadDim + d] = to_bf16_bits(out);
      if (lse != nullptr && d == 0) lse[static_cast<size_t>(b) * hq + col_head] = out_lse;
    } else {
      const size_t prow = (static_cast<size_t>(split) * out_rows + b) * hq + col_head;
      o_part[prow * kHeadDim + d] = out;
      if (d == 0) lse_part[prow] = out_lse;
    }
  };

  if constexpr (kW == 1) {
    // A lane holds d = 16 db + 4 lq + 0..3 of its column: one 8- or 16-byte
    // store per db.
    if (!col_ok) return;
    const float inv = den > 0.0f ? v_scale / den : 0.0f;
    const float out_lse = den > 0.0f ? (m2 + __log2f(den)) * kLn2 : kNegInf;
    if (num_splits == 1) {
      uint16_t* orow = o + (static_cast<size_t>(b) * hq + head) * kHeadDim + 4 * lq;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        u16x4_t w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = to_bf16_bits(acc[db][r] * inv);
        *reinterpret_cast<u16x4_t*>(orow + 16 * db) = w;
      }
      if (lse != nullptr && lq == 0) lse[static_cast<size_t>(b) * hq + head] = out_lse;
    } else {
      const size_t prow = (static_cast<size_t>(split) * out_rows + b) * hq + head;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        f32x4_t w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = acc[db][r] * inv;
        *reinterpret_cast<f32x4_t*>(o_part + prow * kHeadDim + 16 * db + 4 * lq) = w;
      }
      if (lq == 0) lse_part[prow] = out_lse;
    }
    return;
  }

  // Cross-wave merge: each wave publishes (m, l, unnormalised O) per column.
  float* red_o = reinterpret_cast<float*>(stage_all);  // [wave][16 columns][64 d]
  __syncthreads();  // every wave is done with its staging tiles
  if (lq == 0) {
    red_m[wave][lc] = m2;
    red_l[wave][lc] = den;
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) red_o[(wave * 16 + lc) * kHeadDim + 16 * db + 4 * lq + r] = acc[db][r];
  __syncthreads();
  for (int idx = tid; idx < 16 * kHeadDim; idx += 64 * kW) {
    const int c = idx / kHeadDim;
    const int d = idx % kHeadDim;
    if ((c & 7) >= group) continue;
    float big_m = kNegInf;
#pragma unroll
    for (int w = 0; w < kW; ++w) big_m = fmaxf(big_m, red_m[w][c]);
    float out = 0.0f, out_lse = kNegInf;
    if (big_m > kNegInf) {
      float num = 0.0f, tot = 0.0f;
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        const float sc = fast_exp2(red_m[w][c] - big_m);
        tot += sc * red_l[w][c];
        num += sc * red_o[(w * 16 + c) * kHeadDim + d];
      }
      out = num / tot * v_scale;
      out_lse = (big_m + __log2f(tot)) * kLn2;
    }
    emit((g0 + (c >> 3)) * group + (c & 7), d, out, out_lse);
  }
}

template <int kW, bool kPaged>
__global__ __launch_bounds__(64 * kW) void decode_kernel_pair(SINKATTN_DECODE_PARAMS) {
  decode_pair_body<kW, kPaged>(q, k, v, sinks, cu_seqlens_k, hq, hkv, group, window, scale_log2, num_splits, o, lse,
                               o_part, lse_part, v_scale, out_rows, block_table, max_pages, page_shift, num_pages);
}

// Four or more splits over 4 or 8 KV heads: one workgroup per (sequence,
// split), one wave per pair of KV heads.
template <int kPW, bool kPaged>
__global__ __launch_bounds__(64 * kPW) void decode_kernel_pair_hw(SINKATTN_DECODE_PARAMS) {
  decode_pair_body<1, kPaged, kPW>(q, k, v, sinks, cu_seqlens_k, hq, hkv, group, window, scale_log2, num_splits, o,
                                   lse, o_part, lse_part, v_scale, out_rows, block_table, max_pages, page_shift,
                                   num_pages);
}

#undef SINKATTN_DECODE_PARAMS
#undef SINKATTN_DECODE_ARGS

// The parts s_first, s_first + stride, ... (batches of kMergeBatch from
// s_first on, every stride parts) of one row folded into a running (max,
// weight sum, weighted sum); lane = d.
__device__ __forceinline__ void merge_batches(const float* __restrict__ o_parts, const float* __restrict__ lse_parts,
                                              int num_parts, int rows, int row, int lane, int s_first, int stride,
                                              float& big_m, float& tot, float& num) {
  for (int s0 = s_first; s0 < num_parts; s0 += stride) {
    const int cnt = min(kMergeBatch, num_parts - s0);
    // The batch's lse values (lane j holds part s0 + j) and O values (register
    // j holds part s0 + j at d = lane) are all requested before any is used.
    // Registers past the batch re-read its last part; their weight is 0.
    const float l = lane < cnt ? lse_parts[static_cast<size_t>(s0 + lane) * rows + row] : kNegInf;
    float ov[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const size_t pr = static_cast<size_t>(s0 + min(j, cnt - 1)) * rows + row;
      ov[j] = o_parts[pr * kHeadDim + lane];
    }
    const float bm = fmaxf(big_m, wave_max(l));
    // (no branch on bm: the O loads above stay ahead of the reduction)
    const float ref = bm > kNegInf ? bm : 0.0f;
    const float rescale = fast_exp2((big_m - ref) * kLog2e);  // 0 while big_m = -inf
    const float w = fast_exp2((l - ref) * kLog2e);             // 0 for empty parts and idle lanes
    tot = tot * rescale + wave_sum(w);
    num *= rescale;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
      num += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j)) * ov[j];
    big_m = bm;
  }
}

__device__ __forceinline__ void merge_store(uint16_t* __restrict__ o, float* __restrict__ lse, int row, int lane,
                                            float big_m, float tot, float num) {
  float out = 0.0f, out_lse = kNegInf;
  if (big_m > kNegInf) {
    out = num / tot;
    out_lse = big_m + __log2f(tot) * kLn2;
  }
  o[static_cast<size_t>(row) * kHeadDim + lane] = to_bf16_bits(out);
  if (lse != nullptr && lane == 0) lse[row] = out_lse;
}

__global__ __launch_bounds__(kThreads) void merge_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int num_parts,
    int rows, uint16_t* __restrict__ o, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  float big_m = kNegInf, tot = 0.0f, num = 0.0f;
  merge_batches(o_parts, lse_parts, num_parts, rows, row, lane, 0, kMergeBatch, big_m, tot, num);
  merge_store(o, lse, row, lane, big_m, tot, num);
}

// Few rows over many parts (one long sequence split many ways): a workgroup
// per row whose kMergeWideWaves waves take every kMergeWideWaves-th batch of
// its parts, so the batches' memory latencies overlap instead of following
// one another; wave 0 combines the waves' (max, weight sum, weighted sum).
constexpr int kMergeWideWaves = 8;

__global__ __launch_bounds__(64 * kMergeWideWaves) void merge_kernel_wide(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int num_parts,
    int rows, uint16_t* __restrict__ o, float* __restrict__ lse) {
  __shared__ float red_m[kMergeWideWaves], red_t[kMergeWideWaves], red_n[kMergeWideWaves][kHeadDim];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x;
  float big_m = kNegInf, tot = 0.0f, num = 0.0f;
  merge_batches(o_parts, lse_parts, num_parts, rows, row, lane, wave * kMergeBatch, kMergeWideWaves * kMergeBatch,
                big_m, tot, num);
  if (lane == 0) {
    red_m[wave] = big_m;
    red_t[wave] = tot;
  }
  red_n[wave][lane] = num;
  __syncthreads();
  if (wave != 0) return;
  float m = kNegInf;
#pragma unroll
  for (int w = 0; w < kMergeWideWaves; ++w) m = fmaxf(m, red_m[w]);
  float t = 0.0f, n = 0.0f;
  if (m > kNegInf) {
#pragma unroll
    for (int w = 0; w < kMergeWideWaves; ++w) {
      const float sc = fast_exp2((red_m[w] - m) * kLog2e);  // 0 for a wave that saw no part
      t += sc * red_t[w];
      n += sc * red_n[w][lane];
    }
  }
  merge_store(o, lse, row, lane, m, t, n);
}

}  // namespace

// Keys of the longest range a decode query attends.
// The most keys one sequence's queries see together (the first query's
// window start to the end).
static long long max_range(const DecodeLaunch& a) {
  const long long nq = a.cu_seqlens_q != nullptr ? a.max_q : 1;
  return a.window > 0 ? std::min<long long>(a.max_seqlen_k, a.window + nq - 1) : a.max_seqlen_k;
}

bool decode_merges_in_kernel(const DecodeLaunch& a) {
  const long long keys_per_split = (max_range(a) + a.num_splits - 1) / a.num_splits;
  return a.num_splits > 1 && max_range(a) <= kDirectMaxKeys &&
         (keys_per_split <= kKeys || max_range(a) <= kDirectWholeKeys);
}

// Columns per decode wave: the 16-column layout for E4M3 caches with at most
// 16 (token, head) columns (G = 8: half the padded matrix-core and softmax
// work of the 32-column layout, which the E4M3 tile's conversions leave the
// limit there); 32 otherwise; 64 for 33 to 64 columns of draft tokens.
static int decode_cols(const DecodeLaunch& a) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int ncols = a.cu_seqlens_q != nullptr ? a.max_q * group : group;
  if (ncols > 32) return 64;
  if (ncols <= 16 && a.fp8) return 16;
  return 32;
}

template <int kN, bool kFp8, bool kMulti, bool kPaged>
static hipError_t launch_decode_t(const DecodeLaunch& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  // Splits of at most 32 keys: the whole range in one workgroup per
  // (sequence, KV head), o written directly.
  const int splits = decode_merges_in_kernel(a) ? 1 : a.num_splits;
  const long long keys_per_split = (max_range(a) + splits - 1) / splits;
  const bool short_chunks = keys_per_split <= kShortChunk;
  const float scale_log2 = a.softmax_scale * a.k_scale * kLog2e;
  unsigned grid = static_cast<unsigned>(a.batch) * a.num_kv_heads * splits;
  unsigned threads = 128;
  int per_wg = 1;
  decltype(&decode_kernel_w4<kFp8, kMulti, kPaged, kN>) kernel = decode_kernel_w2<kFp8, kMulti, kPaged, kN>;
  // (the split-per-wave kernel's condition below)
  const bool ps_ok = splits >= kSplitPerWaveMin && !short_chunks &&
                     static_cast<long long>(a.batch) * a.num_kv_heads * ((splits + 3) / 4) >= kSplitPerWaveMinGroups;
  const long long hw_units = static_cast<long long>(a.batch) * splits;
  if (splits >= kHeadPerWaveMinSplits && a.num_kv_heads >= 4 && a.num_kv_heads <= 8 &&
      keys_per_split >= kHeadPerWaveMinKeys && (hw_units >= 2 * kHeadPerWaveMinUnits || (hw_units >= kHeadPerWaveMinUnits && !ps_ok))) {
    const long long units = static_cast<long long>(a.batch) * splits;
    per_wg = static_cast<int>(std::max<long long>(1, std::min<long long>(splits, units / kHeadPerWaveTarget)));
    grid = static_cast<unsigned>(static_cast<long long>(a.batch) * ((splits + per_wg - 1) / per_wg));
    threads = 64 * a.num_kv_heads;
    kernel = decode_kernel_hw<kFp8, kMulti, kPaged, kN>;
  } else if (splits == 1 && !short_chunks &&
             static_cast<long long>(a.batch) * (a.num_kv_heads / 2) < kPairMinGroups) {
    grid = static_cast<unsigned>(a.batch) * a.num_kv_heads;
    threads = 512;
    kernel = decode_kernel_w8<kFp8, kMulti, kPaged, kN>;
  } else if (splits == 1 && !short_chunks && a.num_kv_heads % 2 == 0) {
    grid = static_cast<unsigned>(a.batch) * (a.num_kv_heads / 2);
    threads = 512;
    kernel = decode_kernel_w8p<kFp8, kMulti, kPaged, kN>;
  } else if (splits >= kSplitPerWaveMin && !short_chunks &&
             static_cast<long long>(a.batch) * a.num_kv_heads * ((splits + 3) / 4) >= kSplitPerWaveMinGroups) {
    grid = static_cast<unsigned>(a.batch) * a.num_kv_heads * ((splits + 3) / 4);
    threads = 256;
    kernel = decode_kernel_ps<kFp8, kMulti, kPaged, kN>;
  } else if (!short_chunks || (splits == 1 && max_range(a) <= kDirectWholeKeys && kN <= 32)) {
    // (a whole range of at most kDirectWholeKeys keys, a 128-token window
    // layer: four waves take its 4-5 tiles one or two each, a shorter chain
    // than two waves' 2-3; 16 x 32768 8.4 -> 7.8 us, 64 x 4 draft tokens
    // 19.4 -> 17.4 us, eight waves slower again at 64 sequences)
    threads = 256;
    kernel = decode_kernel_w4<kFp8, kMulti, kPaged, kN>;
  }
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, stream, static_cast<const uint16_t*>(a.q), a.k, a.v,
                     a.sinks, a.cu_seqlens_k, a.batch, a.num_q_heads, a.num_kv_heads, group, a.window, scale_log2,
                     splits, static_cast<uint16_t*>(a.o), a.lse, a.o_part, a.lse_part, per_wg, a.v_scale,
                     a.cu_seqlens_q, kMulti ? a.max_q * group : group, kMulti ? a.total_q : a.batch, a.block_table,
                     a.max_pages, a.page_shift, a.num_pages);
  return hipGetLastError();
}

// The E4M3 pair kernel: waves per workgroup so that about kPairWavesTarget
// waves are launched (8 per CU), and no wave is left without a tile.
constexpr long long kPairWavesTarget = 2048;

template <int kW, bool kPaged>
static hipError_t launch_pair_w(const DecodeLaunch& a, int splits, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const unsigned grid = static_cast<unsigned>(static_cast<long long>(a.batch) * (a.num_kv_heads / 2) * splits);
  hipLaunchKernelGGL((decode_kernel_pair<kW, kPaged>), dim3(grid), dim3(64 * kW), 0, stream,
                     static_cast<const uint16_t*>(a.q), a.k, a.v, a.sinks, a.cu_seqlens_k, a.batch, a.num_q_heads,
                     a.num_kv_heads, group, a.window, a.softmax_scale * a.k_scale * kLog2e, splits,
                     static_cast<uint16_t*>(a.o), a.lse, a.o_part, a.lse_part, 1, a.v_scale, nullptr, group, a.batch,
                     a.block_table, a.max_pages, a.page_shift, a.num_pages);
  return hipGetLastError();
}

template <int kPW, bool kPaged>
static hipError_t launch_pair_hw(const DecodeLaunch& a, int splits, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const unsigned grid = static_cast<unsigned>(static_cast<long long>(a.batch) * splits);
  hipLaunchKernelGGL((decode_kernel_pair_hw<kPW, kPaged>), dim3(grid), dim3(64 * kPW), 0, stream,
                     static_cast<const uint16_t*>(a.q), a.k, a.v, a.sinks, a.cu_seqlens_k, a.batch, a.num_q_heads,
                     a.num_kv_heads, group, a.window, a.softmax_scale * a.k_scale * kLog2e, splits,
                     static_cast<uint16_t*>(a.o), a.lse, a.o_part, a.lse_part, 1, a.v_scale, nullptr, group, a.batch,
                     a.block_table, a.max_pages, a.page_shift, a.num_pages);
  return hipGetLastError();
}

template <bool kPaged>
static hipError_t launch_decode_pair(const DecodeLaunch& a, hipStream_t stream) {
  const int splits = decode_merges_in_kernel(a) ? 1 : a.num_splits;
  // (its workgroups hold half the waves of decode_kernel_hw's, so it needs
  // twice the workgroups: 1 x 131072 at S = 128 0.045 -> 0.033 ms, 4 x 32768
  // at S = 32 0.045 -> 0.035 ms on the interleaved pair kernel)
  if (splits >= kHeadPerWaveMinSplits && static_cast<long long>(a.batch) * splits >= 2 * kHeadPerWaveMinUnits) {
    if (a.num_kv_heads == 8) return launch_pair_hw<4, kPaged>(a, splits, stream);
    if (a.num_kv_heads == 4) return launch_pair_hw<2, kPaged>(a, splits, stream);
  }
  const long long units = static_cast<long long>(a.batch) * (a.num_kv_heads / 2) * splits;
  const long long tiles = ((max_range(a) + splits - 1) / splits + kKeys - 1) / kKeys;
  int w = 1;
  while (w < 8 && units * w * 2 <= kPairWavesTarget && w * 2 <= tiles) w *= 2;
  switch (w) {
    case 8: return launch_pair_w<8, kPaged>(a, splits, stream);
    case 4: return launch_pair_w<4, kPaged>(a, splits, stream);
    case 2: return launch_pair_w<2, kPaged>(a, splits, stream);
    default: return launch_pair_w<1, kPaged>(a, splits, stream);
  }
}

static bool decode_pairs(const DecodeLaunch& a) {
  // (a single split over too few pairs of KV heads takes the one-head
  // eight-wave kernel instead, for twice the workgroups)
  const bool few_pairs = a.num_splits == 1 && static_cast<long long>(a.batch) * (a.num_kv_heads / 2) < kPairMinGroups;
  return a.fp8 && a.cu_seqlens_q == nullptr && a.num_kv_heads % 2 == 0 && a.num_q_heads / a.num_kv_heads <= 8 &&
         !few_pairs;
}

template <bool kFp8, bool kMulti, bool kPaged>
static hipError_t launch_decode_cols(const DecodeLaunch& a, hipStream_t stream) {
  if constexpr (kFp8 && !kMulti) {
    if (decode_pairs(a)) return launch_decode_pair<kPaged>(a, stream);
  }
  const int cols = decode_cols(a);
  if constexpr (kMulti) {
    if (cols == 64) return launch_decode_t<64, kFp8, kMulti, kPaged>(a, stream);
  }
  if constexpr (kFp8) {
    if (cols == 16) return launch_decode_t<16, kFp8, kMulti, kPaged>(a, stream);
  }
  return launch_decode_t<32, kFp8, kMulti, kPaged>(a, stream);
}

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream) {
  const bool multi = a.cu_seqlens_q != nullptr;
  if (a.block_table != nullptr) {
    if (multi)
      return a.fp8 ? launch_decode_cols<true, true, true>(a, stream) : launch_decode_cols<false, true, true>(a, stream);
    return a.fp8 ? launch_decode_cols<true, false, true>(a, stream) : launch_decode_cols<false, false, true>(a, stream);
  }
  if (multi)
    return a.fp8 ? launch_decode_cols<true, true, false>(a, stream) : launch_decode_cols<false, true, false>(a, stream);
  return a.fp8 ? launch_decode_cols<true, false, false>(a, stream) : launch_decode_cols<false, false, false>(a, stream);
}

hipError_t launch_merge(const MergeLaunch& a, hipStream_t stream) {
  const int rows = a.n * a.num_heads;
  if (a.num_parts > kMergeBatch && rows < kMergeWideMaxRows) {
    hipLaunchKernelGGL(merge_kernel_wide, dim3(static_cast<unsigned>(rows)), dim3(64 * kMergeWideWaves), 0, stream,
                       a.o_parts, a.lse_parts, a.num_parts, rows, static_cast<uint16_t*>(a.o), a.lse);
    return hipGetLastError();
  }
  const unsigned blocks = static_cast<unsigned>((rows + kWaves - 1) / kWaves);
  hipLaunchKernelGGL(merge_kernel, dim3(blocks), dim3(kThreads), 0, stream, a.o_parts, a.lse_parts,
                     a.num_parts, rows, static_cast<uint16_t*>(a.o), a.lse);
  return hipGetLastError();
}

int decode_max_group() { return 32; }

int decode_max_cols() { return 64; }

// Split-KV partials of sinkattn_decode_splitkv_noalloc: a fixed device array
// instead of a caller workspace.  Each device the library runs on holds its
// own copy for the life of the process.  Nothing in it needs to start at
// zero (every split writes its partial rows before the merge reads them), and
// calls that overlap on one device share it, so they race.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The device address of `scratch` on `device`, looked up once per device
// (hipGetSymbolAddress with that device current) and kept.  In host code the
// name `scratch` is only a host-side stand-in: kernels get this address.
hipError_t noalloc_scratch(int device, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[device] == nullptr) {
    int current = -1;
    hipError_t e = hipGetDevice(&current);
    if (e != hipSuccess) return e;
    if (current != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (current != device) {
      const hipError_t r = hipSetDevice(current);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

}  // namespace sinkattn
