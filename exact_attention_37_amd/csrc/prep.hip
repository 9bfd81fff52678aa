// Memory-bound helper kernels: the backward preprocess rowsum(dO * O) (the
// float32 backward and the chunk driver; the bf16 backward forms it in its dQ
// kernel), the LSE merge of partial outputs, dtype conversion and fills, and
// the packed-batch work lists.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace miattn {

namespace {

// Loads 8 consecutive elements as float.
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = *(const f32x4*)p;
  const f32x4 b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int t = 0; t < 4; ++t) { x[t] = a[t]; x[t + 4] = b[t]; }
}
__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
  const bf16x8 a = *(const bf16x8*)p;
#pragma unroll
  for (int t = 0; t < 8; ++t) x[t] = (float)a[t];
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int t = 0; t < 4; ++t) { a[t] = x[t]; b[t] = x[t + 4]; }
  *(f32x4*)p = a;
  *(f32x4*)(p + 4) = b;
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8]) {
  bf16x8 a;
#pragma unroll
  for (int t = 0; t < 8; ++t) a[t] = (bf16)x[t];
  *(bf16x8*)p = a;
}

// D[b, h, n] = sum_c dO[b, n, h, c] * O[b, n, h, c]. D/8 lanes per row.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                      float* __restrict__ dsum, int B, int H, int N,
                                                      int row0, int nrows) {
  constexpr int L = D / 8;
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = t / L;          // over B * nrows * H (n-major inside b)
  const int part = (int)(t % L);
  const long long total = (long long)B * nrows * H;
  const bool ok = row < total;
  const long long r = ok ? row : 0;
  const int h = (int)(r % H);
  const long long bn = r / H;
  const int n = row0 + (int)(bn % nrows);
  const int b = (int)(bn / nrows);
  const long long off = (((long long)b * N + n) * H + h) * D + part * 8;
  float x[8], y[8];
  load8(o + off, x);
  load8(dout + off, y);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = fmaf(x[e], y[e], acc);
#pragma unroll
  for (int w = L / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, L);
  if (ok && part == 0) dsum[((long long)b * H + h) * N + n] = acc;
}

// Softmax over the union of two disjoint key sets, from their partial
// outputs and logsumexps. Each row is handled by D/8 adjacent lanes of one
// wave, which all read lse_a/lse_b before any of them writes lse, so the
// merge may be done in place.
template <typename TA, typename TB, typename TO, int D>
__global__ __launch_bounds__(256) void merge_kernel(const TA* o_a, const float* lse_a, const TB* o_b,
                                                    const float* lse_b, TO* o, float* lse, int B, int H,
                                                    int N, int row0, int nrows) {
  constexpr int L = D / 8;
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = t / L;
  const int part = (int)(t % L);
  const long long total = (long long)B * nrows * H;
  if (row >= total) return;
  const int h = (int)(row % H);
  const long long bn = row / H;
  const int n = row0 + (int)(bn % nrows);
  const int b = (int)(bn / nrows);
  const long long li = ((long long)b * H + h) * N + n;
  const float la = lse_a[li], lb = lse_b[li];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, l = -INFINITY;
  if (m != -INFINITY) {
    const float ea = __expf(la - m), eb = __expf(lb - m);
    const float tot = ea + eb;
    l = m + __logf(tot);
    const float inv = 1.f / tot;
    wa = ea * inv;
    wb = eb * inv;
  }
  const long long off = (((long long)b * N + n) * H + h) * D + part * 8;
  float x[8], y[8], z[8];
  load8(o_a + off, x);
  load8(o_b + off, y);
  // a partial over an empty key set (lse = -inf) contributes nothing,
  // whatever its o holds (zeros by convention, but also stale values or NaN)
  const bool use_a = la != -INFINITY, use_b = lb != -INFINITY;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (use_a ? wa * x[e] : 0.f) + (use_b ? wb * y[e] : 0.f);
  store8(o + off, z);
  if (part == 0) lse[li] = l;
}

template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ src, T* __restrict__ dst, long long n) {
  const long long i = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i + 8 <= n) {
    float x[8];
    load8(src + i, x);
    store8(dst + i, x);
  } else {
    for (long long j = i; j < n; ++j) dst[j] = from_f<T>(src[j]);
  }
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ dst, long long n, float value) {
  const long long i = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 4 <= n) {
    f32x4 v = {value, value, value, value};
    *(f32x4*)(dst + i) = v;
  } else {
    for (long long j = i; j < n; ++j) dst[j] = value;
  }
}

// Block-sparse tile lists: one wave per block row r (the key tiles of
// BS_TILE keys whose mask block (r, j / 2) is kept, up to the block row's
// last query under causal) or per block column c (the query tiles of BS_TILE
// rows whose mask block (i / 4, c) is kept, from the column's first key on
// under causal). Lanes test 64 consecutive tiles at a time; a ballot and a
// prefix count compact the kept ones, so the lists come out ascending.
__global__ __launch_bounds__(64) void bs_lists_kernel(const uint8_t* __restrict__ mask, int N, int causal,
                                                      int nbr, int nbc, int ld, int* __restrict__ row_cnt,
                                                      int* __restrict__ row_plain, int* __restrict__ row_tiles,
                                                      int* __restrict__ col_cnt, int* __restrict__ col_tiles) {
  static_assert(BS_ROWS == 4 * BS_TILE && BS_COLS == 2 * BS_TILE, "tiles nest in mask blocks");
  const int w = blockIdx.x, lane = threadIdx.x;
  const uint64_t below = (1ull << lane) - 1ull;
  int cnt = 0, plain = 0;
  if (w < nbr) {
    const int r = w;
    const int last = min(r * BS_ROWS + BS_ROWS - 1, N - 1);
    // tiles wholly below every row's diagonal and before the ragged end
    const int plim = min(N / BS_TILE, causal ? r * (BS_ROWS / BS_TILE) : ld);
    for (int j0 = 0; j0 < ld; j0 += 64) {
      const int j = j0 + lane;
      const bool keep = j < ld && (!causal || j * BS_TILE <= last) &&
                        mask[(long long)r * nbc + j / (BS_COLS / BS_TILE)] != 0;
      const uint64_t bits = __ballot(keep);
      if (keep) row_tiles[(long long)r * ld + cnt + __popcll(bits & below)] = j;
      cnt += __popcll(bits);
      plain += __popcll(__ballot(keep && j < plim));
    }
    if (lane == 0) {
      row_cnt[r] = cnt;
      row_plain[r] = plain;
    }
  } else {
    const int c = w - nbr;
    for (int i0 = 0; i0 < ld; i0 += 64) {
      const int i = i0 + lane;
      const bool keep = i < ld && (!causal || i * BS_TILE + BS_TILE - 1 >= c * BS_COLS) &&
                        mask[(long long)(i / (BS_ROWS / BS_TILE)) * nbc + c] != 0;
      const uint64_t bits = __ballot(keep);
      if (keep) col_tiles[(long long)c * ld + cnt + __popcll(bits & below)] = i;
      cnt += __popcll(bits);
    }
    if (lane == 0) col_cnt[c] = cnt;
  }
}

// Work list of a packed variable-length batch: every sequence s (rows
// [cu[s], cu[s+1]) clamped to [0, N], as in narrow_to_sequence) contributes
// ceil(length / rows) tiles, sequences in order and within a sequence from
// the last tile down (desc) or from tile 0 up. Entry e is (list[2 + 2e],
// list[3 + 2e]) = (sequence, tile); list[0] is the number of entries. At
// most cap entries are written (malformed offsets can ask for more).
__global__ __launch_bounds__(1024) void varlen_tiles_kernel(const int* __restrict__ cu, int nseq, int N, int rows,
                                                           int desc, int cap, int* __restrict__ list) {
  __shared__ int wsum[16];
  __shared__ int base;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int s0 = 0; s0 < nseq; s0 += 1024) {
    const int sq = s0 + tid;
    int nt = 0;
    if (sq < nseq) {
      const int e = min(max(cu[sq + 1], 0), N);
      const int a = min(max(cu[sq], 0), e);
      nt = (e - a + rows - 1) / rows;
    }
    int x = nt;                                  // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int wofs = 0;
    for (int w = 0; w < wave; ++w) wofs += wsum[w];
    const int off = base + wofs + x - nt;        // exclusive offset of this sequence
    for (int k = 0; k < nt && off + k < cap; ++k) {
      list[2 + 2 * (off + k)] = sq;
      list[3 + 2 * (off + k)] = desc ? nt - 1 - k : k;
    }
    __syncthreads();
    if (tid == 1023) base = off + nt;
    __syncthreads();
  }
  if (tid == 0) list[0] = min(base, cap);
}

inline unsigned blocks_for(long long threads) { return (unsigned)((threads + 255) / 256); }

template <typename TA, typename TB, typename TO>
hipError_t merge3(const void* oa, const float* la, const void* ob, const float* lb, void* o, float* l,
                  int B, int H, int N, int d, int row0, int nrows, hipStream_t s) {
  const long long threads = (long long)B * nrows * H * (d / 8);
  if (d == 64)
    hipLaunchKernelGGL((merge_kernel<TA, TB, TO, 64>), dim3(blocks_for(threads)), dim3(256), 0, s,
                       (const TA*)oa, la, (const TB*)ob, lb, (TO*)o, l, B, H, N, row0, nrows);
  else
    hipLaunchKernelGGL((merge_kernel<TA, TB, TO, 128>), dim3(blocks_for(threads)), dim3(256), 0, s,
                       (const TA*)oa, la, (const TB*)ob, lb, (TO*)o, l, B, H, N, row0, nrows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pre(const void* o, const void* dout, float* dsum, int B, int H, int N, int d,
                          int row0, int nrows, int dtype, hipStream_t s) {
  const long long threads = (long long)B * nrows * H * (d / 8);
  const dim3 grid(blocks_for(threads)), block(256);
  auto go = [&](auto tc, auto dc) {
    using T = decltype(tc);
    constexpr int D = decltype(dc)::value;
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), grid, block, 0, s, (const T*)o, (const T*)dout, dsum, B, H, N, row0,
                       nrows);
  };
  if (dtype == 0) {
    if (d == 64) go(float{}, std::integral_constant<int, 64>{});
    else go(float{}, std::integral_constant<int, 128>{});
  } else {
    if (d == 64) go(bf16{}, std::integral_constant<int, 64>{});
    else go(bf16{}, std::integral_constant<int, 128>{});
  }
  return hipGetLastError();
}

hipError_t launch_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o,
                        float* lse, int B, int H, int N, int d, int row0, int nrows, int ta, int tb, int to,
                        hipStream_t s) {
  const int key = ta * 4 + tb * 2 + to;
  switch (key) {
    case 0: return merge3<float, float, float>(o_a, lse_a, o_b, lse_b, o, lse, B, H, N, d, row0, nrows, s);
    case 1: return merge3<float, float, bf16>(o_a, lse_a, o_b, lse_b, o, lse, B, H, N, d, row0, nrows, s);
    case 7: return merge3<bf16, bf16, bf16>(o_a, lse_a, o_b, lse_b, o, lse, B, H, N, d, row0, nrows, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_convert(const float* src, void* dst, long long n, int dtype, hipStream_t s) {
  const dim3 grid(blocks_for((n + 7) / 8)), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL((convert_kernel<float>), grid, block, 0, s, src, (float*)dst, n);
  else
    hipLaunchKernelGGL((convert_kernel<bf16>), grid, block, 0, s, src, (bf16*)dst, n);
  return hipGetLastError();
}

long long bs_list_ints(int N) {
  const long long nbr = (N + BS_ROWS - 1) / BS_ROWS, nbc = (N + BS_COLS - 1) / BS_COLS;
  const long long ld = (N + BS_TILE - 1) / BS_TILE;
  return 2 * nbr + nbc + (nbr + nbc) * ld;
}

hipError_t launch_bs_lists(const uint8_t* mask, int N, int causal, int* ints, Params& p, hipStream_t s) {
  const int nbr = (N + BS_ROWS - 1) / BS_ROWS, nbc = (N + BS_COLS - 1) / BS_COLS;
  const int ld = (N + BS_TILE - 1) / BS_TILE;
  int* row_cnt = ints;
  int* row_plain = row_cnt + nbr;
  int* col_cnt = row_plain + nbr;
  int* row_tiles = col_cnt + nbc;
  int* col_tiles = row_tiles + (long long)nbr * ld;
  p.bs_mask = mask;
  p.bs_nbc = nbc;
  p.bs_row_cnt = row_cnt;
  p.bs_row_plain = row_plain;
  p.bs_row_tiles = row_tiles;
  p.bs_col_cnt = col_cnt;
  p.bs_col_tiles = col_tiles;
  p.bs_ld = ld;
  hipLaunchKernelGGL(bs_lists_kernel, dim3(nbr + nbc), dim3(64), 0, s, mask, N, causal, nbr, nbc, ld, row_cnt,
                     row_plain, row_tiles, col_cnt, col_tiles);
  return hipGetLastError();
}

int varlen_list_cap(int total, int rows, int nseq) { return (total + rows - 1) / rows + nseq; }

hipError_t launch_varlen_tiles(const int* cu_seqlens, int nseq, int total, int rows, int desc, int* list,
                               hipStream_t s) {
  hipLaunchKernelGGL(varlen_tiles_kernel, dim3(1), dim3(1024), 0, s, cu_seqlens, nseq, total, rows, desc,
                     varlen_list_cap(total, rows, nseq), list);
  return hipGetLastError();
}

int device_cu_count() {
  // per device, read once: the attribute query is a host call
  static std::atomic<int> counts[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = counts[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  counts[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_fill(float* dst, long long n, float value, hipStream_t s) {
  hipLaunchKernelGGL(fill_kernel, dim3(blocks_for((n + 3) / 4)), dim3(256), 0, s, dst, n, value);
  return hipGetLastError();
}

}  // namespace miattn
