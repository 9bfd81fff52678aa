// Memory-bound helper kernels: the backward preprocess rowsum(dO * O), the
// LSE merge of partial outputs, dtype conversion and fills.
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
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = wa * x[e] + wb * y[e];
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
  if (dtype == 0) {
    if (d == 64)
      hipLaunchKernelGGL((bwd_pre_kernel<float, 64>), grid, block, 0, s, (const float*)o, (const float*)dout, dsum, B, H, N, row0, nrows);
    else
      hipLaunchKernelGGL((bwd_pre_kernel<float, 128>), grid, block, 0, s, (const float*)o, (const float*)dout, dsum, B, H, N, row0, nrows);
  } else {
    if (d == 64)
      hipLaunchKernelGGL((bwd_pre_kernel<bf16, 64>), grid, block, 0, s, (const bf16*)o, (const bf16*)dout, dsum, B, H, N, row0, nrows);
    else
      hipLaunchKernelGGL((bwd_pre_kernel<bf16, 128>), grid, block, 0, s, (const bf16*)o, (const bf16*)dout, dsum, B, H, N, row0, nrows);
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

hipError_t launch_fill(float* dst, long long n, float value, hipStream_t s) {
  hipLaunchKernelGGL(fill_kernel, dim3(blocks_for((n + 3) / 4)), dim3(256), 0, s, dst, n, value);
  return hipGetLastError();
}

}  // namespace miattn
