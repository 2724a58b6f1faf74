// Varlen causal / sliding-window prefill with per-head sinks (gfx950).
//
// Operation: Perplexity, "GPT-OSS on day 0", section "GPT-OSS kernels / Sink
// attention" (the sink is an extra softmax logit; the online softmax starts
// its running max at the sink and its denominator at 1), with the 128-token
// window layers of the NVIDIA gpt-oss announcement (model description).
//
// Append prefill (chunked prefill, multi-token-query decode): sequence b has
// Lk_b key rows (cu_seqlens_k) and its last Lq_b <= Lk_b tokens are the
// queries (cu_seqlens_q), so query row r sits at position off + r with
// off = Lk_b - Lq_b, and the causal / window mask is aligned at the bottom
// right.  Self-attention prefill is the case cu_seqlens_k = cu_seqlens_q
// (off = 0).  Draft tokens of a speculative or multi-token-prediction decoder
// are verified this way (Perplexity, "GPT-OSS on day 0", in-house inference
// engine; Baseten, "How to run GPT OSS 120B at 500+ tokens per second on
// NVIDIA GPUs", next performance optimizations).
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
// Per 32-key step h and per wave (two column blocks of 32 query columns):
//   S^T = K Q^T          8 MFMA 32x32x16 (K from LDS, Q held in registers)
//   mask                 only on steps that cross the diagonal / window edge
//   online softmax       reference max in log2 units, exp2, per-lane partial
//                        denominators (the lane pair shares the reference)
//   O^T += V^T P^T       8 MFMA (V read transposed from LDS)
// The steps are software-pipelined: while the VALU normalises step h, the
// matrix core computes S for step h + 1 and O^T for step h - 1, all from one
// basic block, so each wave keeps both units busy on its own.  K/V tiles of
// 64 keys rotate through four LDS buffers, copied HBM -> LDS three tiles
// ahead of use.
#include "device_common.hpp"
#include "launch.hpp"

namespace sinkattn {

namespace {

constexpr int kQTile = 32;  // query tokens per workgroup
constexpr int kKTile = 64;  // keys per LDS tile (two 32-key steps)
constexpr int kBufs = 4;    // LDS tile buffers in the ring
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
// n % 8, which under the chunk swizzle is global chunk (n % 8) ^ swz_f(row).
// Rows past the sequence end are clamped to its last key: they only ever
// meet masked logits.  Each thread issues 2 kPer copies per tile.
template <int kThreads>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ k_seq, const uint16_t* __restrict__ v_seq,
                                           uint32_t k_dst, uint32_t v_dst, int len, int row_stride, int key0,
                                           int wave, int lane) {
  constexpr int kPer = kKTile * 8 / kThreads;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int slot0 = 64 * (kPer * wave + i);
    const int row = (slot0 >> 3) + (lane >> 3);
    const int chunk = (lane & 7) ^ swz_f(row);
    const int key = min(key0 + row, len - 1);
    // 32-bit byte offset from the sequence's first row of this KV head (the
    // host bounds max_seqlen * row_stride * 2 below 2^31).  Kept opaque so
    // the compiler recomputes it here (uniform base + 32-bit lane offset)
    // instead of carrying one 64-bit pointer per copy through the loop.
    uint32_t off = static_cast<uint32_t>(key * row_stride + chunk * 8) * 2u;
    asm volatile("" : "+v"(off));
    load16_to_lds_untracked(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(k_seq) + off),
                            k_dst + slot0 * 16);
    load16_to_lds_untracked(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(v_seq) + off),
                            v_dst + slot0 * 16);
  }
}

// The same copy from a paged cache: pages [num_pages, 1 << page_shift, hkv,
// 64], key j of the sequence in slot j & (page_size - 1) of page
// row[j >> page_shift].  A tile's 64 keys (key0 a multiple of 64) lie in at
// most four pages when page_size >= 16; their ids are read once per tile,
// uniform over the workgroup and clamped to the pool (a bad table cannot move
// a copy out of bounds), and a row's id is formed from their differences so
// that they stay in registers.  k_pool / v_pool point at head g of token 0.
template <int kThreads>
__device__ __forceinline__ void issue_tile_paged(const uint16_t* __restrict__ k_pool,
                                                 const uint16_t* __restrict__ v_pool, uint32_t k_dst, uint32_t v_dst,
                                                 int len, int hkv, int key0, int wave, int lane,
                                                 const int32_t* __restrict__ row, int page_shift, int plast,
                                                 int num_pages) {
  constexpr int kPer = kKTile * 8 / kThreads;
  const int p0 = key0 >> page_shift;
  auto id_of = [&](int page) { return min(max(row[min(page, plast)], 0), num_pages - 1); };
  const int id0 = id_of(p0), id1 = id_of(p0 + 1), id2 = id_of(p0 + 2), id3 = id_of(p0 + 3);
  const int slot_mask = (1 << page_shift) - 1;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int slot0 = 64 * (kPer * wave + i);
    const int r = (slot0 >> 3) + (lane >> 3);
    const int chunk = (lane & 7) ^ swz_f(r);
    const int key = min(key0 + r, len - 1);
    const int rel = (key >> page_shift) - p0;  // 0 .. 3
    const int id = id0 + (rel >= 1 ? id1 - id0 : 0) + (rel >= 2 ? id2 - id1 : 0) + (rel >= 3 ? id3 - id2 : 0);
    const size_t tok = (static_cast<size_t>(id) << page_shift) + (key & slot_mask);
    const size_t off = tok * static_cast<size_t>(hkv) * kHeadDim + chunk * 8;  // elements
    load16_to_lds_untracked(k_pool + off, k_dst + slot0 * 16);
    load16_to_lds_untracked(v_pool + off, v_dst + slot0 * 16);
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

// Compile-time integer (step parity, buffer index) passed to generic lambdas.
template <int N>
struct Parity {
  static constexpr int value = N;
};

template <int kThreads>
constexpr int copies_per_tile() { return 2 * (kKTile * 8 / kThreads); }

// Wait until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that also retires this wave's LDS reads first (so a tile
// copy issued after it cannot overwrite data still being read) and that the
// compiler does not move memory operations across.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// First work item of sequence b: floor((cu[b] + 31 b) / 32).  Consecutive
// starts differ by at least ceil(len_b / 32) and by at most one more, so the
// items of a batch number floor((T + 31 B) / 32) at most, with T the tokens.
__device__ __forceinline__ int item_start(int cu_b, int b) {
  return static_cast<int>((static_cast<long long>(cu_b) + static_cast<long long>(kQTile - 1) * b) / kQTile);
}

// The sequence that owns work item w: the largest b < batch with
// item_start(cu[b], b) <= w (starts are non-decreasing for valid offsets),
// or -1.  A 64-way search: each round probes one offset per lane, so up to
// 64 sequences take one round of loads and 4096 take two.
__device__ __forceinline__ int find_sequence(const int32_t* __restrict__ cu, int batch, int w, int lane) {
  int lo = 0, n = batch;  // the answer lies in [lo, lo + n)
  while (true) {
    const int stride = (n + 63) / 64;
    const int probe = lo + lane * stride;
    bool le = false;
    if (probe < lo + n) le = item_start(cu[probe], probe) <= w;
    const int cnt = __popcll(__builtin_amdgcn_ballot_w64(le));
    if (cnt == 0) return -1;
    lo += (cnt - 1) * stride;
    if (stride == 1) return lo;
    n = min(stride, n - (cnt - 1) * stride);
  }
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// kSplit: the key tiles of every query tile are cut into gridDim.y
// contiguous shares (blockIdx.y = split); each workgroup writes its share's
// normalised fp32 output and lse as a partial ([split][out_rows][hq] rows of
// o_part / lse_part), the sink counted in split 0 only, and the log-sum-exp
// merge combines them (Perplexity, "GPT-OSS on day 0", Sink attention: with
// the KV length split into chunks, the sink initialises only the first).
template <bool kWindow, int kCols, bool kPaged, bool kSplit = false>
__global__ __launch_bounds__(threads_for<kCols>()) __attribute__((amdgpu_waves_per_eu(4 / kCols, 4 / kCols))) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ sinks,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_seqlens_k, int hq, int hkv, int group,
    int n_hchunk, int batch, int max_seqlen, int max_seqlen_k, int window, float scale_log2,
    uint16_t* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ block_table, int max_pages,
    int page_shift, int num_pages, float* __restrict__ o_part, float* __restrict__ lse_part, int out_rows) {
  // Ring of LDS tile buffers, each K rows then V rows.  Tile t lives in
  // buffer (t - t_begin) % kBufs; the loop below is unrolled over the ring so
  // every LDS address is a per-lane base plus an immediate offset.
  // Window layers get a fifth buffer: a query tile whose keys span at most
  // three tiles then has all of them and its Q block in flight at once.
  __shared__ __attribute__((aligned(16))) uint16_t kv_lds[kWindow ? kBufs + 1 : kBufs][2 * kKTile * kHeadDim];

  constexpr int kThreads = threads_for<kCols>();
  constexpr int kCopies = copies_per_tile<kThreads>();
  constexpr int kRowsPerWave = kQTile / (kThreads / 64);  // Q / O block rows moved per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: head maths in SGPRs
  const int col = lane & 31;   // query token within the tile
  const int half = lane >> 5;  // which k-half / row-half of the MFMA layouts

  // blockIdx.x = (w * n_hchunk + hchunk) * hkv + g: consecutive workgroups
  // take consecutive KV heads, so with 8 KV heads each XCD (they receive
  // workgroups round-robin) serves one head.  Work item w names a query tile
  // in batch order (item_start), the top tile of a sequence first: the
  // workgroups in flight on an XCD belong to one or two sequences and share
  // their K/V through its L2, and within a sequence the longest tiles start
  // first.
  int x = blockIdx.x;
  const int g = x % hkv;
  x /= hkv;
  const int hchunk = x % n_hchunk;
  const int w = x / n_hchunk;
  const int b = find_sequence(cu_seqlens, batch, w, lane);
  if (b < 0) return;  // uniform over the workgroup

  const int seq0 = cu_seqlens[b];
  // kPaged: the keys live in pages; cu_seqlens_k then holds the lengths.
  const int seq0_k = kPaged ? 0 : cu_seqlens_k[b];
  // Lengths above the declared maxima, or fewer keys than queries, break a
  // precondition; clamping keeps every access inside the bounds the host
  // checked (such a sequence's rows are left unwritten).
  const int len = min(cu_seqlens[b + 1] - seq0, max_seqlen);
  const int len_k = min(kPaged ? cu_seqlens_k[b] : cu_seqlens_k[b + 1] - seq0_k, max_seqlen_k);
  const int n_tiles = len > 0 ? (len + kQTile - 1) / kQTile : 0;
  const int j = w - item_start(seq0, b);
  if (j >= n_tiles || len_k < len) return;  // a spare item between two sequences
  const int off = len_k - len;  // position of query row 0 in the sequence
  const int qt = n_tiles - 1 - j;
  const int q0 = qt * kQTile;

  const int last_q = min(len - 1, q0 + kQTile - 1);
  const int last_pos = last_q + off;  // the last key any query of the tile sees
  const int first_key = kWindow ? max(0, q0 + off - window + 1) : 0;
  int t_begin = first_key / kKTile;
  int t_end = last_pos / kKTile;
  // 32-key steps h_begin..h_end: every one holds a key some query of the
  // tile sees.
  int h_begin = first_key >> 5;
  int h_end = last_pos >> 5;
  const int split = kSplit ? static_cast<int>(blockIdx.y) : 0;
  if constexpr (kSplit) {
    // This split's share of the tiles: ceil(n / S) consecutive tiles, the
    // trailing shares possibly empty (t_begin > t_end: no step runs and the
    // partial is empty).
    const int n_t = t_end - t_begin + 1;
    const int per = (n_t + static_cast<int>(gridDim.y) - 1) / static_cast<int>(gridDim.y);
    const int tb = t_begin + split * per;
    t_end = min(t_end, tb + per - 1);
    t_begin = tb;
    h_begin = max(h_begin, 2 * t_begin);
    h_end = min(h_end, 2 * t_end + 1);
  }

  // K / V rows of this sequence and KV head; a key's row is hkv * 64
  // elements further on.
  const size_t kv0 = (static_cast<size_t>(seq0_k) * hkv + g) * kHeadDim;
  const uint16_t* k_seq = k + kv0;
  const uint16_t* v_seq = v + kv0;
  // LDS byte address of the ring (uniform).
  const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_address(&kv_lds[0][0]));
  const int32_t* bt_row = kPaged ? block_table + static_cast<size_t>(b) * max_pages : nullptr;
  const int plast = kPaged ? min((len_k - 1) >> page_shift, max_pages - 1) : 0;  // len_k >= len >= 1 here
  auto issue = [&](int tt, int buf) {
    const uint32_t dst = ring + static_cast<uint32_t>(buf) * (2 * kKTile * kHeadDim * 2);
    if constexpr (kPaged)
      issue_tile_paged<kThreads>(k_seq, v_seq, dst, dst + kKTile * kHeadDim * 2, len_k, hkv, tt * kKTile, wave,
                                 lane, bt_row, page_shift, plast, num_pages);
    else
      issue_tile<kThreads>(k_seq, v_seq, dst, dst + kKTile * kHeadDim * 2, len_k, hkv * kHeadDim, tt * kKTile,
                           wave, lane);
  };
  // The first two tiles go out before anything else, then the workgroup's
  // Q block (32 tokens x 8 head slots x 128 B, 1 KB contiguous per token)
  // into buffers 2 and 3, which receive their tiles once Q is in registers.
  // A window tile whose keys span at most three tiles (the 128-token window)
  // sends its third tile at once too and puts Q in buffers 3 and 4: one
  // round trip to memory instead of two.
  const bool all_at_once = kWindow && t_end - t_begin <= 2;
  const int q_buf = all_at_once ? 3 : 2;
  if (t_begin <= t_end) issue(t_begin, 0);
  if (t_begin + 1 <= t_end) issue(t_begin + 1, 1);
  if (all_at_once && t_begin + 2 <= t_end) issue(t_begin + 2, 2);
  uint16_t* const q_lds = &kv_lds[q_buf][0];
  {
    const uint32_t q_dst = ring + q_buf * (2 * kKTile * kHeadDim * 2);
    const int slot = lane >> 3;
    const int head_q = g * group + min(hchunk * kHeadsPerBlock + slot, group - 1);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int r = kRowsPerWave * wave + i;  // token row of the block
      const int chunk = (lane & 7) ^ (r & 7);
      const int tok = min(q0 + r, len - 1);
      const uint16_t* src = q + (static_cast<size_t>(seq0 + tok) * hq + head_q) * kHeadDim + chunk * 8;
      load16_to_lds_untracked(src, q_dst + static_cast<uint32_t>(r) * (kHeadsPerBlock * kHeadDim * 2));
    }
  }

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
  const int qpos = q0 + off + col;  // this lane's query position in the sequence

  // Q^T as the B operand (lane holds query column `col`, d = 16 s + 8 half
  // + t), read from the Q block in LDS once it has landed.
  bf16x8_t qreg[kCols][4];

  // Online-softmax state per column block.  The reference max m is kept in
  // log2 units (scaled logits); the sink seeds it, and its "1" is counted once
  // (in the lower lane of the pair).
  float m2[kCols], lsum[kCols];
  f32x16_t acc[kCols][2];
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
    const float z = (sinks != nullptr && head_ok[c] && split == 0) ? sinks[head[c]] : kNegInf;
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

  // LDS read offsets (elements, within a 32-row step of a tile).  K rows as
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

  // Pipeline registers.  S is double-buffered by step parity (static in the
  // unrolled loop, so no register copies): S of step h in s_buf[h & 1].  P
  // has one buffer: the O^T MFMAs of step h - 1 read it before the softmax
  // of step h overwrites it.  V^T of the previous step, K of the next.
  f32x16_t s_buf[2][kCols];
  bf16x8_t p_buf[kCols][2];
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
  // K rows / V rows of step hh, which sits in buffer `buf`.
  auto k_rows = [&](int buf, int hh) { return kv_lds[buf] + (hh & 1) * 32 * kHeadDim; };
  auto v_rows = [&](int buf, int hh) { return kv_lds[buf] + kKTile * kHeadDim + (hh & 1) * 32 * kHeadDim; };
  auto s_chains = [&](f32x16_t (&s_out)[kCols]) {
#pragma unroll
    for (int c = 0; c < kCols; ++c) s_out[c] = zero16();
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int c = 0; c < kCols; ++c) s_out[c] = mfma_32x32x16(kop[s], qreg[c][s], s_out[c]);
  };
  auto pv_chains = [&](const bf16x8_t (&p)[kCols][2]) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < kCols; ++c) acc[c][db] = mfma_32x32x16(vop[db][u], p[c][u], acc[c][db]);
  };

  // Causal / window mask of step hh (a step crossing the diagonal or the
  // window's lower edge).  Register r of this lane holds key
  // 32 hh + key_of_reg(r, half).
  auto need_mask = [&](int hh) {
    const int kbase = hh * 32;
    return (kbase + 31 > q0 + off) || (kWindow && kbase <= last_pos - window);
  };
  auto mask = [&](int hh, f32x16_t& s_c) {
    const int lim = qpos - hh * 32 - 8 * half;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = key_of_reg(r, 0);
      const bool ok = off <= lim && (!kWindow || off > lim - window);
      if (!ok) s_c[r] = kNegInf;
    }
  };

  // Reference max as used by the fast path: -m (0 for a row without
  // reference yet) and the partial-sum limit above which the slow path runs
  // (-1, i.e. always, for a row without reference).  Updated only when m
  // moves.
  float m_neg[kCols], sum_lim[kCols];
  auto set_ref = [&](int c) {
    const bool none = m2[c] == kNegInf;
    m_neg[c] = none ? 0.0f : -m2[c];
    sum_lim[c] = none ? -1.0f : kRescaleSum;
  };
#pragma unroll
  for (int c = 0; c < kCols; ++c) set_ref(c);

  // One pipelined step hh with parity `par` (= hh & 1); its tile sits in
  // buffer `buf`, the next tile in `buf_next`.
  auto step = [&](int hh, auto par_c, auto buf_c) __attribute__((always_inline)) {
    constexpr int par = decltype(par_c)::value;
    constexpr int buf = decltype(buf_c)::value;
    constexpr int buf_next = (buf + 1) & (kBufs - 1);
    f32x16_t (&s_cur)[kCols] = s_buf[par];
    f32x16_t (&s_next)[kCols] = s_buf[par ^ 1];
    bf16x8_t (&p_cur)[kCols][2] = p_buf;
    if (need_mask(hh)) {
#pragma unroll
      for (int c = 0; c < kCols; ++c) mask(hh, s_cur[c]);
    }
    // Matrix core: S of step hh + 1 and O^T of step hh - 1.  The operands of
    // the next step are read as soon as these MFMAs have taken the current
    // ones (same registers): K of step hh + 2 (same half of the next tile)
    // and V^T of this step.  Past the last step these reads return unused
    // data from resident buffers.  The softmax below covers their latency.
    s_chains(s_next);
    read_k(k_rows(buf_next, hh));
    pv_chains(p_buf);
    read_v(v_rows(buf, hh));
    // VALU: P of step hh against the current reference (fast path).
    float tsum[kCols];
    bool slow[kCols];
    uint64_t slow_lanes = 0;  // ballot of each compare: no boolean materialised
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      tsum[c] = probs(s_cur[c], p_cur[c], -m_neg[c], scale_log2);
      slow[c] = !(tsum[c] <= sum_lim[c]);
      slow_lanes |= __builtin_amdgcn_ballot_w64(slow[c]);
    }
    // Slow path (rare): a row without reference yet, or keys far above it.
    // Move the reference to the row max (uniformly over the lane pair),
    // rescale the state (O^T of step hh - 1 included), redo P.
    if (slow_lanes != 0) {
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        float mx = s_cur[c][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s_cur[c][r]);
        mx = pair_max(mx) * scale_log2;
        const bool move = pair_max(slow[c] ? 1.0f : 0.0f) > 0.0f && mx > m2[c];
        const float m_new = move ? mx : m2[c];
        const float alpha = move ? fast_exp2(m2[c] - m_new) : 1.0f;
        m2[c] = m_new;
        set_ref(c);
        lsum[c] *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[c][db][r] *= alpha;
        tsum[c] = probs(s_cur[c], p_cur[c], -m_neg[c], scale_log2);
      }
    }
#pragma unroll
    for (int c = 0; c < kCols; ++c) lsum[c] += tsum[c];
  };

  // Wait for the first tiles and the Q block (all copies issued so far),
  // publish them, take Q into registers, then hand buffers 2 and 3 to their
  // tiles.
  wait_vmem_keep<0>();
  lds_barrier();
#pragma unroll
  for (int c = 0; c < kCols; ++c) {
    const int slot = wave * kCols + c;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qreg[c][s] = *reinterpret_cast<const bf16x8_t*>(q_lds + col * (kHeadsPerBlock * kHeadDim) + slot * kHeadDim +
                                                     (((2 * s + half) ^ (col & 7)) << 3));
  }
  lds_barrier();
  if (!all_at_once) {
    if (t_begin + 2 <= t_end) issue(t_begin + 2, 2);
    if (t_begin + 3 <= t_end) issue(t_begin + 3, 3);
  }

  if (wave_active) {
    // Prologue: S of step h_begin, K of step h_begin + 1, empty P of step
    // h_begin - 1 and zero V^T (the first step's O^T update adds nothing).
    read_k(kv_lds[0] + (h_begin & 1) * 32 * kHeadDim);
    const bool odd = h_begin & 1;
    if (odd) s_chains(s_buf[1]); else s_chains(s_buf[0]);
    const int h1 = h_begin + 1;
    read_k(kv_lds[((h1 >> 1) - t_begin) & (kBufs - 1)] + (h1 & 1) * 32 * kHeadDim);
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
#pragma unroll
      for (int u = 0; u < 2; ++u) p_buf[c][u] = __builtin_bit_cast(bf16x8_t, zero_u32x4());
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      vop[db][0] = __builtin_bit_cast(bf16x8_t, zero_u32x4());
      vop[db][1] = __builtin_bit_cast(bf16x8_t, zero_u32x4());
    }
  }

  // Tile t (buffer bi, a compile-time constant) and its two steps.
  auto tile = [&](int t0, auto bi_c) __attribute__((always_inline)) {
    constexpr int bi = decltype(bi_c)::value;
    const int t = t0 + bi;
    if (t > t_end) return;
    // Tile boundary: tile t + 1 (read from step 2t on) must have landed for
    // every wave; tile t - 1's buffer is then free for tile t + 3.
    if (t > t_begin) {
      if (t + 2 >= t_begin + kBufs && t + 2 <= t_end)
        wait_vmem_keep<kCopies>();  // tile t + 2 may still be in flight
      else
        wait_vmem_keep<0>();
      lds_barrier();
      if (t + 3 <= t_end) issue(t + 3, (bi + 3) & (kBufs - 1));
    }
    if (!wave_active) return;
    if (2 * t >= h_begin && 2 * t <= h_end) step(2 * t, Parity<0>{}, Parity<bi>{});
    if (2 * t + 1 >= h_begin && 2 * t + 1 <= h_end) step(2 * t + 1, Parity<1>{}, Parity<bi>{});
  };

  for (int t0 = t_begin; t0 <= t_end; t0 += kBufs) {
    tile(t0, Parity<0>{});
    tile(t0, Parity<1>{});
    tile(t0, Parity<2>{});
    tile(t0, Parity<3>{});
  }

  // Epilogue.  Every K/V read is done once all waves pass this barrier;
  // buffers 0 and 1 then stage the O block (same layout as the Q block) so
  // that it is stored as whole 1 KB token rows.
  if constexpr (kSplit) {
    // This split's partial straight from the registers: a lane holds
    // d = 32 db + 8 j + 4 half + 0..3 of query column col, one 16-byte store
    // each; rows past the sequence and columns past the group are skipped.
    if (!wave_active) return;
    pv_chains(p_buf);  // O^T of the last step
    const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int colr = lane_e & 31;
    const int halfr = lane_e >> 5;
    if (q0 + colr >= len) return;
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      const float den = pair_sum(lsum[c]);
      if (!head_ok[c]) continue;
      const float inv = den > 0.0f ? 1.0f / den : 0.0f;
      const size_t prow = (static_cast<size_t>(split) * out_rows + seq0 + q0 + colr) * hq + head[c];
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4_t w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = acc[c][db][4 * j + i] * inv;
          *reinterpret_cast<f32x4_t*>(o_part + prow * kHeadDim + 32 * db + 8 * j + 4 * halfr) = w;
        }
      if (halfr == 0) lse_part[prow] = den > 0.0f ? (m2[c] + __log2f(den)) * kLn2 : kNegInf;
    }
    return;
  }
  lds_barrier();
  uint16_t* const o_lds = &kv_lds[0][0];
  if (wave_active) {
    pv_chains(p_buf);  // O^T of the last step
    const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int colr = lane_e & 31;  // recomputed: nothing from the prologue stays alive
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      // Full denominator over the lane pair, normalise, bf16 into LDS.
      const float den = pair_sum(lsum[c]);
      const float inv = den > 0.0f ? 1.0f / den : 0.0f;
      const int slot = wave * kCols + c;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u16x4_t w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = to_bf16_bits(acc[c][db][4 * j + i] * inv);
          // d = 32 db + 8 j + 4 half: chunk 4 db + j, bytes 8 half of it.
          *reinterpret_cast<u16x4_t*>(o_lds + colr * (kHeadsPerBlock * kHeadDim) + slot * kHeadDim +
                                      (((4 * db + j) ^ (colr & 7)) << 3) + 4 * half) = w;
        }
      }
      if (lse != nullptr && half == 0 && head_ok[c] && q0 + colr < len) {
        const float l = den > 0.0f ? (m2[c] + __log2f(den)) * kLn2 : kNegInf;
        lse[static_cast<size_t>(seq0 + q0 + colr) * hq + head[c]] = l;
      }
    }
  }
  lds_barrier();
  // Whole rows: wave w stores tokens 8 w .. 8 w + 7, lane L the 16 B chunk
  // (L & 7) of head slot L >> 3 (un-swizzled on the way out).
  {
    // Lane id recomputed here so no address of this loop is built before the
    // main loop and carried across it.
    const int lane_s = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int slot = lane_s >> 3;
    const bool slot_ok = hchunk * kHeadsPerBlock + slot < group;
    const int head_o = g * group + hchunk * kHeadsPerBlock + slot;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int r = kRowsPerWave * wave + i;
      const int pos = lane_s & 7;
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(o_lds + r * (kHeadsPerBlock * kHeadDim) +
                                                           slot * kHeadDim + pos * 8);
      if (slot_ok && q0 + r < len) {
        const int chunk = pos ^ (r & 7);
        *reinterpret_cast<u32x4_t*>(o + (static_cast<size_t>(seq0 + q0 + r) * hq + head_o) * kHeadDim +
                                    chunk * 8) = val;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int n_hchunk = (group + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const long long blocks = prefill_blocks(a.batch, a.total_tokens, a.num_kv_heads, group);
  if (blocks <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(blocks), 1, 1);
  const bool windowed = a.window > 0 && a.window < a.max_seqlen_k;
  const bool paged = a.block_table != nullptr;
  const bool split = a.num_splits > 1;
  auto kernel = paged ? (windowed ? prefill_kernel<true, kColsPerWave, true> : prefill_kernel<false, kColsPerWave, true>)
                      : (windowed ? prefill_kernel<true, kColsPerWave, false> : prefill_kernel<false, kColsPerWave, false>);
  if (split) {
    kernel = paged ? (windowed ? prefill_kernel<true, kColsPerWave, true, true>
                               : prefill_kernel<false, kColsPerWave, true, true>)
                   : (windowed ? prefill_kernel<true, kColsPerWave, false, true>
                               : prefill_kernel<false, kColsPerWave, false, true>);
    grid.y = static_cast<unsigned>(a.num_splits);
  }
  hipLaunchKernelGGL(kernel, grid, dim3(threads_for<kColsPerWave>()), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.sinks, a.cu_seqlens, a.cu_seqlens_k, a.num_q_heads,
                     a.num_kv_heads, group, n_hchunk, a.batch, a.max_seqlen, a.max_seqlen_k, a.window,
                     a.softmax_scale * kLog2e, static_cast<uint16_t*>(a.o), a.lse, a.block_table, a.max_pages,
                     a.page_shift, a.num_pages, a.o_part, a.lse_part, a.total_tokens);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !split) return err;
  // The partials of every (query row, head) combined into o and lse.
  MergeLaunch m{a.o_part, a.lse_part, a.num_splits, a.total_tokens, a.num_q_heads, a.o, a.lse};
  return launch_merge(m, stream);
}

long long prefill_blocks(int batch, int total_tokens, int num_kv_heads, int group) {
  const long long items = (static_cast<long long>(total_tokens) + static_cast<long long>(kQTile - 1) * batch) / kQTile;
  return items * num_kv_heads * ((group + kHeadsPerBlock - 1) / kHeadsPerBlock);
}

// hipLaunchKernelGGL takes at most 2^32 - 1 work-items along x.
long long prefill_max_blocks() { return 0xffffffffLL / threads_for<kColsPerWave>(); }

}  // namespace sinkattn
