// Output projection with bias after attention (gfx950):
//     y[n, e] = sum_k o[n, k] * W[e, k] + b[e]
// o is the attention output with its query heads concatenated (k = h * 64 +
// d), W one row per output feature; bf16 in, fp32 accumulation, bf16 out
// (Perplexity, "GPT-OSS on day 0", section "GPT-OSS on Hopper": the output
// projection carries a bias).
//
// Shaped for the decode step, where the rows are few and the weight is the
// traffic: computed transposed, y^T = W o^T, with v_mfma_f32_32x32x16_bf16
// (A = 32 rows of W, B = 32 rows of o, both 16-byte loads of 8 consecutive
// k straight from memory: no LDS staging; W with cached loads, so that the
// re-reads of W by further 64-row blocks hit the caches: 8192 rows 1.91 ->
// 0.96 ms against nontemporal loads).  A workgroup owns 32 kOprojTiles
// output features and 64 rows, each wave all of them (its o loads feed
// kOprojTiles weight tiles); the 8 waves split K into 8 slices, so W is read
// once per 64 rows (from HBM for the first block) while o stays in L2, and
// the slices are summed through LDS, where the bias is added and the result
// rounded to bf16.  The split-KV merge is not fused in: every feature tile
// would re-read all of the split partials of its rows (a probe that forms o
// from 16 partials inside the K loop ran 172-181 us at 64 rows x 4096 ->
// 2880, against 29-36 us for the merge followed by this kernel), so the
// merge writes o once (bf16) and this kernel reads it from L2.
#include "device_common.hpp"
#include "launch.hpp"

namespace sinkattn {

namespace {

constexpr int kOprojWaves = 8;
// 32-feature MFMA tiles per wave (they share each o load).  Measured at
// 64 / 256 / 8192 rows x 4096 -> 2880: one tile 0.032 / 0.088 / 2.18 ms, two
// 0.033 / 0.076 / 1.91 ms, four 0.044 / 0.085 / 1.82 ms.
constexpr int kOprojTiles = 2;
constexpr int kOprojCols = 32 * kOprojTiles;       // output features per workgroup
constexpr int kOprojRows = 64;                     // rows per workgroup (two MFMA column blocks)
constexpr int kOprojUnroll = 8 / kOprojTiles;
// Above this many rows the LDS-tiled GEMM below takes over (256 rows: this
// kernel 0.051 ms, the GEMM 0.092 ms).
constexpr int kOprojGemmMinRows = 256;

// blockIdx.z takes K range [z K / gridDim.z, (z + 1) K / gridDim.z) (its 8
// waves split it again); with more than one K range each workgroup writes
// fp32 partial sums to part[z] and oproj_finish_kernel adds them up.
__global__ __launch_bounds__(64 * kOprojWaves) void oproj_kernel(const uint16_t* __restrict__ o,
                                                                 const uint16_t* __restrict__ w,
                                                                 const float* __restrict__ bias,
                                                                 uint16_t* __restrict__ y, float* __restrict__ part,
                                                                 int n_rows, int k_dim, int e_dim) {
  __shared__ float red[kOprojWaves][2][16][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int e0 = blockIdx.x * kOprojCols;
  const int n0 = blockIdx.y * kOprojRows;
  const int k_range = k_dim / gridDim.z;       // a multiple of 128
  const int slice = k_range / kOprojWaves;     // a multiple of 16
  const int k_begin = blockIdx.z * k_range + wave * slice;
  const int kh = 8 * (lane >> 5);
  // Rows past n_rows repeat the last row: their columns of y^T are dropped.
  const int nr0 = min(n0 + (lane & 31), n_rows - 1);
  const int nr1 = min(n0 + 32 + (lane & 31), n_rows - 1);
  const bool two = n0 + 32 < n_rows;  // uniform: a second block of 32 rows
  // Feature rows past e_dim (the last tile of an e_dim not a multiple of
  // kOprojCols) repeat row e_dim - 1 and are not stored.
  const uint16_t* wp[kOprojTiles];
#pragma unroll
  for (int c = 0; c < kOprojTiles; ++c)
    wp[c] = w + static_cast<size_t>(min(e0 + 32 * c + (lane & 31), e_dim - 1)) * k_dim + k_begin + kh;
  const uint16_t* op0 = o + static_cast<size_t>(nr0) * k_dim + k_begin + kh;
  const uint16_t* op1 = o + static_cast<size_t>(nr1) * k_dim + k_begin + kh;

  f32x16_t acc[kOprojTiles][2];
#pragma unroll
  for (int c = 0; c < kOprojTiles; ++c) acc[c][0] = acc[c][1] = zero16();
  for (int k = 0; k < slice; k += 16 * kOprojUnroll) {
    const int steps = min(kOprojUnroll, (slice - k) / 16);
    bf16x8_t a[kOprojUnroll][kOprojTiles], b0[kOprojUnroll], b1[kOprojUnroll];
#pragma unroll
    for (int u = 0; u < kOprojUnroll; ++u) {
      if (u < steps) {
#pragma unroll
        for (int c = 0; c < kOprojTiles; ++c) a[u][c] = __builtin_bit_cast(bf16x8_t, load16(wp[c] + k + 16 * u));
        b0[u] = __builtin_bit_cast(bf16x8_t, load16(op0 + k + 16 * u));
        if (two) b1[u] = __builtin_bit_cast(bf16x8_t, load16(op1 + k + 16 * u));
      }
    }
#pragma unroll
    for (int u = 0; u < kOprojUnroll; ++u) {
      if (u < steps) {
#pragma unroll
        for (int c = 0; c < kOprojTiles; ++c) {
          acc[c][0] = mfma_32x32x16(a[u][c], b0[u], acc[c][0]);
          if (two) acc[c][1] = mfma_32x32x16(a[u][c], b1[u], acc[c][1]);
        }
      }
    }
  }

  // Sum the K slices, one 32-feature tile at a time: register r of lane l
  // holds y^T[tile + 8 (r / 4) + 4 (l / 32) + r % 4][row block + l % 32].
#pragma unroll
  for (int c = 0; c < kOprojTiles; ++c) {
    if (c > 0) __syncthreads();  // the previous tile's sums are read
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      red[wave][0][r][lane] = acc[c][0][r];
      red[wave][1][r][lane] = two ? acc[c][1][r] : 0.0f;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 2 * 16 * 64; idx += 64 * kOprojWaves) {
      const int nb = idx >> 10;
      const int r = (idx >> 6) & 15;
      const int ln = idx & 63;
      const int n = n0 + 32 * nb + (ln & 31);
      const int e = e0 + 32 * c + 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
      if (n >= n_rows || e >= e_dim) continue;
      float sum = 0.0f;
#pragma unroll
      for (int wv = 0; wv < kOprojWaves; ++wv) sum += red[wv][nb][r][ln];
      if (gridDim.z > 1) {
        part[(static_cast<size_t>(blockIdx.z) * n_rows + n) * e_dim + e] = sum;
        continue;
      }
      if (bias != nullptr) sum += bias[e];
      y[static_cast<size_t>(n) * e_dim + e] = to_bf16_bits(sum);
    }
  }
}

// y = bf16(sum of the K-range partials + bias), four outputs per thread.
__global__ __launch_bounds__(256) void oproj_finish_kernel(const float* __restrict__ part, const float* __restrict__ bias,
                                                           uint16_t* __restrict__ y, int splits, long long count,
                                                           int e_dim) {
  const long long i = (static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= count) return;  // count is a multiple of 32 (e_dim is)
  float4 acc = *reinterpret_cast<const float4*>(part + i);
  for (int z = 1; z < splits; ++z) {
    const float4 p = *reinterpret_cast<const float4*>(part + z * count + i);
    acc.x += p.x;
    acc.y += p.y;
    acc.z += p.z;
    acc.w += p.w;
  }
  if (bias != nullptr) {
    const int e = static_cast<int>(i % e_dim);
    acc.x += bias[e];
    acc.y += bias[e + 1];
    acc.z += bias[e + 2];
    acc.w += bias[e + 3];
  }
  u16x4_t out;
  out[0] = to_bf16_bits(acc.x);
  out[1] = to_bf16_bits(acc.y);
  out[2] = to_bf16_bits(acc.z);
  out[3] = to_bf16_bits(acc.w);
  *reinterpret_cast<u16x4_t*>(y + i) = out;
}

// Prefill-sized row counts: an LDS-tiled GEMM.  A workgroup owns 128 rows x
// 128 output features; its 4 waves each compute 64 x 64 (2 x 2 MFMA
// blocks).  K advances kGemmK at a time: the workgroup copies the 128 x kGemmK
// tiles of o and W into LDS with coalesced 16-byte loads (the next tiles are
// loaded into registers while the current ones are multiplied), so each
// operand element is read from memory once per tile instead of once per
// 32 x 32 MFMA block.  LDS rows are padded by 8 elements (16 bytes) so that
// the 16-byte reads of 32 consecutive rows spread over the banks.
// K per LDS step (8192 rows x 4096 -> 2880: 32 -> 0.316 ms, 64 -> 0.277,
// 128 -> 0.287)
constexpr int kGemmK = 64;
constexpr int kGemmPad = kGemmK + 8;      // LDS row stride in elements
constexpr int kGemmChunks = kGemmK / 8;   // 16-byte chunks per tile row
// Rows and output features per workgroup (8192 rows: 128 x 128 0.281 ms,
// 256 x 128 0.290, 128 x 256 0.295 with 8 waves).
constexpr int kGemmTN = 128;
constexpr int kGemmTE = 128;
constexpr int kGemmWaves = (kGemmTN / 64) * (kGemmTE / 64);
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kGemmPassRows = kGemmThreads / kGemmChunks;  // tile rows one pass of the threads copies
constexpr int kGemmPassesO = kGemmTN / kGemmPassRows;
constexpr int kGemmPassesW = kGemmTE / kGemmPassRows;

__global__ __launch_bounds__(kGemmThreads) void oproj_gemm_kernel(const uint16_t* __restrict__ o,
                                                                  const uint16_t* __restrict__ w,
                                                                  const float* __restrict__ bias,
                                                                  uint16_t* __restrict__ y, int n_rows, int k_dim,
                                                                  int e_dim) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_o[kGemmTN * kGemmPad];
  __shared__ __attribute__((aligned(16))) uint16_t lds_w[kGemmTE * kGemmPad];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * kGemmTN;
  const int e0 = blockIdx.y * kGemmTE;
  // Copy assignment: thread t moves 16-byte chunk t % kGemmChunks of tile
  // rows t / kGemmChunks + kGemmPassRows i (rows past the matrix repeat its
  // last row).
  const int crow = tid / kGemmChunks;
  const int cchunk = 8 * (tid % kGemmChunks);
  const uint16_t* og[kGemmPassesO];
  const uint16_t* wg[kGemmPassesW];
#pragma unroll
  for (int i = 0; i < kGemmPassesO; ++i)
    og[i] = o + static_cast<size_t>(min(n0 + crow + kGemmPassRows * i, n_rows - 1)) * k_dim + cchunk;
#pragma unroll
  for (int i = 0; i < kGemmPassesW; ++i)
    wg[i] = w + static_cast<size_t>(min(e0 + crow + kGemmPassRows * i, e_dim - 1)) * k_dim + cchunk;
  // Wave (we, wn) computes features e0 + 64 we .. + 63 and rows n0 + 64 wn ..
  const int we = wave % (kGemmTE / 64);
  const int wn = wave / (kGemmTE / 64);
  const int kh = 8 * (lane >> 5);
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = zero16();

  u32x4_t ro[kGemmPassesO], rw[kGemmPassesW];
#pragma unroll
  for (int i = 0; i < kGemmPassesO; ++i) ro[i] = load16(og[i]);
#pragma unroll
  for (int i = 0; i < kGemmPassesW; ++i) rw[i] = load16(wg[i]);
  for (int k = 0; k < k_dim; k += kGemmK) {
    __syncthreads();  // the previous tiles' LDS reads are done
#pragma unroll
    for (int i = 0; i < kGemmPassesO; ++i)
      *reinterpret_cast<u32x4_t*>(lds_o + (crow + kGemmPassRows * i) * kGemmPad + cchunk) = ro[i];
#pragma unroll
    for (int i = 0; i < kGemmPassesW; ++i)
      *reinterpret_cast<u32x4_t*>(lds_w + (crow + kGemmPassRows * i) * kGemmPad + cchunk) = rw[i];
    __syncthreads();
    if (k + kGemmK < k_dim) {
#pragma unroll
      for (int i = 0; i < kGemmPassesO; ++i) ro[i] = load16(og[i] + k + kGemmK);
#pragma unroll
      for (int i = 0; i < kGemmPassesW; ++i) rw[i] = load16(wg[i] + k + kGemmK);
    }
#pragma unroll
    for (int ks = 0; ks < kGemmK; ks += 16) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const bf16x8_t*>(lds_w + (64 * we + 32 * i + (lane & 31)) * kGemmPad + ks + kh);
        b[i] = *reinterpret_cast<const bf16x8_t*>(lds_o + (64 * wn + 32 * i + (lane & 31)) * kGemmPad + ks + kh);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16(a[i], b[j], acc[i][j]);
    }
  }
  // acc[i][j] register r of lane l: y^T[e0 + 64 we + 32 i + 8 (r / 4) +
  // 4 (l / 32) + r % 4][n0 + 64 wn + 32 j + l % 32].
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + 64 * wn + 32 * j + (lane & 31);
    if (n >= n_rows) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = e0 + 64 * we + 32 * i + 8 * q + 4 * (lane >> 5);
        if (e >= e_dim) continue;  // e_dim is a multiple of 32: a group of 4 is all in or all out
        u16x4_t out;
#pragma unroll
        for (int r = 0; r < 4; ++r) out[r] = to_bf16_bits(acc[i][j][4 * q + r] + (bias != nullptr ? bias[e + r] : 0.0f));
        *reinterpret_cast<u16x4_t*>(y + static_cast<size_t>(n) * e_dim + e) = out;
      }
    }
  }
}

}  // namespace

// K ranges per launch: the most (a power of two, each range a multiple of
// 128 of K) that keep the launch within one workgroup per CU (256).  64 rows
// x 4096 -> 2880: 4 ranges (180 workgroups) 0.025 ms, 16 ranges (720) 0.034.
int oproj_splits(int num_rows, int in_features, int out_features) {
  if (num_rows > kOprojGemmMinRows) return 1;  // the tiled GEMM: no partials
  const long long tiles = static_cast<long long>((out_features + kOprojCols - 1) / kOprojCols) *
                          ((num_rows + kOprojRows - 1) / kOprojRows);
  int splits = 1;
  while (tiles * splits * 2 <= 256 && in_features % (128 * splits * 2) == 0 && splits < 32) splits *= 2;
  return splits;
}

hipError_t launch_oproj(const OprojLaunch& a, hipStream_t stream) {
  if (a.num_rows <= 0) return hipSuccess;
  if (a.num_rows > kOprojGemmMinRows) {
    const dim3 grid(static_cast<unsigned>((a.num_rows + kGemmTN - 1) / kGemmTN),
                    static_cast<unsigned>((a.out_features + kGemmTE - 1) / kGemmTE));
    hipLaunchKernelGGL(oproj_gemm_kernel, grid, dim3(kGemmThreads), 0, stream, static_cast<const uint16_t*>(a.o),
                       static_cast<const uint16_t*>(a.w), a.bias, static_cast<uint16_t*>(a.y), a.num_rows,
                       a.in_features, a.out_features);
    return hipGetLastError();
  }
  const int splits = oproj_splits(a.num_rows, a.in_features, a.out_features);
  const dim3 grid(static_cast<unsigned>((a.out_features + kOprojCols - 1) / kOprojCols),
                  static_cast<unsigned>((a.num_rows + kOprojRows - 1) / kOprojRows), static_cast<unsigned>(splits));
  hipLaunchKernelGGL(oproj_kernel, grid, dim3(64 * kOprojWaves), 0, stream, static_cast<const uint16_t*>(a.o),
                     static_cast<const uint16_t*>(a.w), a.bias, static_cast<uint16_t*>(a.y), a.part, a.num_rows,
                     a.in_features, a.out_features);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const long long count = static_cast<long long>(a.num_rows) * a.out_features;
  hipLaunchKernelGGL(oproj_finish_kernel, dim3(static_cast<unsigned>((count / 4 + 255) / 256)), dim3(256), 0, stream,
                     a.part, a.bias, static_cast<uint16_t*>(a.y), splits, count, a.out_features);
  return hipGetLastError();
}

}  // namespace sinkattn
