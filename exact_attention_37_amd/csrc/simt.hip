// Vector-ALU attention kernels (one thread per query or key row, K/V or Q/dO
// tiles staged in LDS, float32 arithmetic). They serve the float32 dtype,
// whose exactness contract is tighter than bf16 matrix-core products give.
//
// Forward: FlashAttention's tiled pass with online softmax (FlashAttention
// abstract page: tiling through on-chip memory; FlashAttention-2 reviews
// page, reviewer 2, points 1-2: un-normalised accumulator divided once at the
// end, logsumexp saved). Backward: P is rebuilt from the saved logsumexp
// (DistFlashAttn reviews page, review 1 point 3) in two passes -- one per
// key row for dK/dV, one per query row for dQ -- so no partial sum is ever
// shared between threads.
#include "common.h"
#include "kernels.h"

namespace miattn {

namespace {

constexpr int kRows = 64;   // rows per workgroup (one row per thread)
constexpr int kTile = 32;   // rows of the streamed operand per LDS tile

__device__ __forceinline__ long long qrow(const Params& p, int b, int row) {
  return ((long long)b * p.N + row) * p.H;
}
__device__ __forceinline__ long long krow(const Params& p, int b, int row) {
  return ((long long)b * p.N + row) * p.Hkv;
}

// Block-sparse: whether the mask keeps the block holding query row i and key
// j (kRows and kTile divide the block sizes, so one test covers a tile).
__device__ __forceinline__ bool block_kept(const Params& p, int i, int j) {
  return !p.bs_mask || p.bs_mask[(long long)(i / BS_ROWS) * p.bs_nbc + j / BS_COLS] != 0;
}
static_assert(BS_ROWS % kRows == 0 && BS_ROWS % kTile == 0 && BS_COLS % kRows == 0 && BS_COLS % kTile == 0,
              "row and key tiles nest in mask blocks");

template <typename T, typename TO, int D>
__global__ __launch_bounds__(kRows) void fwd_simt(Params p) {
  int b = blockIdx.z;
  const int h = blockIdx.y;
  const int g = h / p.G;
  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * kRows;
  if (p.cu_seqlens) {                 // packed batch: z is the sequence
    if (!narrow_to_sequence(p, b, i0)) return;
    b = 0;
  }
  const int i = i0 + tid;
  const int ic = min(i, p.Nq - 1);
  const T* Q = (const T*)p.q + (qrow(p, b, p.q_start + ic) + h) * D;
  const T* K = (const T*)p.k + (krow(p, b, p.k_start) + g) * D;
  const T* V = (const T*)p.v + (krow(p, b, p.k_start) + g) * D;
  const long long kstride = (long long)p.Hkv * D;

  const float c = p.scale * kLog2e;   // scores kept in the log2 domain
  float q[D], acc[D];
#pragma unroll
  for (int t = 0; t < D; ++t) { q[t] = to_f(Q[t]) * c; acc[t] = 0.f; }
  float m = -INFINITY, l = 0.f;

  __shared__ float Ks[kTile][D];
  __shared__ float Vs[kTile][D];

  int kend = p.Nk;
  if (p.causal) {
    const int last_q = p.q_start + min(i0 + kRows - 1, p.Nq - 1);
    kend = max(0, min(p.Nk, last_q - p.k_start + 1));
  }
  const int qpos = p.q_start + i;
  // sliding window: keys before the window of the block's first row are skipped
  const int jbeg = p.window > 0 ? max(0, p.q_start + i0 - (p.window - 1) - p.k_start) / kTile * kTile : 0;
  for (int j0 = jbeg; j0 < kend; j0 += kTile) {
    if (!block_kept(p, i0, j0)) continue;   // (uniform over the workgroup)
    for (int e = tid; e < kTile * D; e += kRows) {
      const int r = e / D, col = e % D;
      const bool in = j0 + r < p.Nk;
      Ks[r][col] = in ? to_f(K[(j0 + r) * kstride + col]) : 0.f;
      Vs[r][col] = in ? to_f(V[(j0 + r) * kstride + col]) : 0.f;
    }
    __syncthreads();
    const int jn = min(kTile, kend - j0);
    for (int jj = 0; jj < jn; ++jj) {
      if (p.causal && p.k_start + j0 + jj > qpos) break;
      if (p.window > 0 && p.k_start + j0 + jj <= qpos - p.window) continue;
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < D; ++t) s = fmaf(q[t], Ks[jj][t], s);
      if (s > m) {
        const float a = exp2f(m - s);
        l *= a;
#pragma unroll
        for (int t = 0; t < D; ++t) acc[t] *= a;
        m = s;
      }
      const float pr = exp2f(s - m);
      l += pr;
#pragma unroll
      for (int t = 0; t < D; ++t) acc[t] = fmaf(pr, Vs[jj][t], acc[t]);
    }
    __syncthreads();
  }
  if (i < p.Nq) {
    TO* O = (TO*)p.o + (qrow(p, b, p.q_start + i) + h) * D;
    const float inv = l > 0.f ? 1.f / l : 0.f;   // a row with no key (block-sparse): o = 0, lse = -inf
#pragma unroll
    for (int t = 0; t < D; ++t) O[t] = from_f<TO>(acc[t] * inv);
    p.lse[((long long)b * p.H + h) * p.N + p.q_start + i] = (m + log2f(l)) * kLn2;
  }
}

// dK, dV of one key row per thread, summed over the query heads of its group.
template <typename T, int D>
__global__ __launch_bounds__(kRows) void bwd_dkdv_simt(Params p) {
  int b = blockIdx.z;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int j0 = blockIdx.x * kRows;
  if (p.cu_seqlens) {                 // packed batch: z is the sequence
    if (!narrow_to_sequence(p, b, j0)) return;
    b = 0;
  }
  const int j = j0 + tid;
  const int jc = min(j, p.Nk - 1);
  const long long kstride = (long long)p.Hkv * D;
  const long long qstride = (long long)p.H * D;

  __shared__ float Kr[kRows][D + 1];   // this block's key rows (padded: one row per thread)
  __shared__ float Vr[kRows][D + 1];
  __shared__ float Qs[kTile][D];
  __shared__ float Ds[kTile][D];
  __shared__ float Ls[kTile], Ps[kTile];
  {
    const T* K = (const T*)p.k + (krow(p, b, p.k_start + j0) + g) * D;
    const T* V = (const T*)p.v + (krow(p, b, p.k_start + j0) + g) * D;
    for (int e = tid; e < kRows * D; e += kRows) {
      const int r = e / D, col = e % D;
      const bool in = j0 + r < p.Nk;
      Kr[r][col] = in ? to_f(K[r * kstride + col]) : 0.f;
      Vr[r][col] = in ? to_f(V[r * kstride + col]) : 0.f;
    }
  }
  float dk[D], dv[D];
#pragma unroll
  for (int t = 0; t < D; ++t) { dk[t] = 0.f; dv[t] = 0.f; }
  const float c = p.scale * kLog2e;
  const int kpos = p.k_start + j;
  // first query row that can see any key of this block
  int ibeg = 0;
  if (p.causal) ibeg = max(0, p.k_start + j0 - p.q_start);
  // sliding window: query rows past the window of the block's last key see none of it
  int iend = p.Nq;
  if (p.window > 0) iend = min(p.Nq, max(0, p.k_start + j0 + kRows - 1 + p.window - p.q_start));
  __syncthreads();

  for (int h = g * p.G; h < (g + 1) * p.G; ++h) {
    const T* Q = (const T*)p.q + (qrow(p, b, p.q_start) + h) * D;
    const T* dO = (const T*)p.dout + (qrow(p, b, p.q_start) + h) * D;
    const float* L = p.lse + ((long long)b * p.H + h) * p.N + p.q_start;
    const float* Dv = p.dsum + ((long long)b * p.H + h) * p.N + p.q_start;
    for (int i0 = ibeg; i0 < iend; i0 += kTile) {
      if (!block_kept(p, i0, j0)) continue;   // (uniform over the workgroup)
      for (int e = tid; e < kTile * D; e += kRows) {
        const int r = e / D, col = e % D;
        const bool in = i0 + r < p.Nq;
        Qs[r][col] = in ? to_f(Q[(i0 + r) * qstride + col]) : 0.f;
        Ds[r][col] = in ? to_f(dO[(i0 + r) * qstride + col]) : 0.f;
      }
      if (tid < kTile) {
        const bool in = i0 + tid < p.Nq;
        Ls[tid] = in ? L[i0 + tid] * kLog2e : 0.f;
        Ps[tid] = in ? Dv[i0 + tid] : 0.f;
      }
      __syncthreads();
      const int in_n = min(kTile, p.Nq - i0);
      for (int ii = 0; ii < in_n; ++ii) {
        if (p.causal && kpos > p.q_start + i0 + ii) continue;
        if (p.window > 0 && p.q_start + i0 + ii >= kpos + p.window) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int t = 0; t < D; ++t) {
          s = fmaf(Qs[ii][t], Kr[tid][t], s);
          dp = fmaf(Ds[ii][t], Vr[tid][t], dp);
        }
        const float pr = exp2f(s * c - Ls[ii]);
        const float ds = pr * (dp - Ps[ii]);
#pragma unroll
        for (int t = 0; t < D; ++t) {
          dv[t] = fmaf(pr, Ds[ii][t], dv[t]);
          dk[t] = fmaf(ds, Qs[ii][t], dk[t]);
        }
      }
      __syncthreads();
    }
  }
  if (j < p.Nk) {
    const long long off = (krow(p, b, p.k_start + j) + g) * D;
    if (p.accumulate) {
      float* DK = (float*)p.dk + off;
      float* DV = (float*)p.dv + off;
#pragma unroll
      for (int t = 0; t < D; ++t) { DK[t] += dk[t] * p.scale; DV[t] += dv[t]; }
    } else {
      T* DK = (T*)p.dk + off;
      T* DV = (T*)p.dv + off;
#pragma unroll
      for (int t = 0; t < D; ++t) { DK[t] = from_f<T>(dk[t] * p.scale); DV[t] = from_f<T>(dv[t]); }
    }
  }
}

// dQ of one query row per thread.
template <typename T, int D>
__global__ __launch_bounds__(kRows) void bwd_dq_simt(Params p) {
  int b = blockIdx.z;
  const int h = blockIdx.y;
  const int g = h / p.G;
  const int tid = threadIdx.x;
  const int i0 = blockIdx.x * kRows;
  if (p.cu_seqlens) {                 // packed batch: z is the sequence
    if (!narrow_to_sequence(p, b, i0)) return;
    b = 0;
  }
  const int i = i0 + tid;
  const int ic = min(i, p.Nq - 1);
  const long long kstride = (long long)p.Hkv * D;
  const T* Q = (const T*)p.q + (qrow(p, b, p.q_start + ic) + h) * D;
  const T* dO = (const T*)p.dout + (qrow(p, b, p.q_start + ic) + h) * D;
  const T* K = (const T*)p.k + (krow(p, b, p.k_start) + g) * D;
  const T* V = (const T*)p.v + (krow(p, b, p.k_start) + g) * D;
  const float c = p.scale * kLog2e;
  const long long stat = ((long long)b * p.H + h) * p.N + p.q_start + ic;
  const float lse2 = p.lse[stat] * kLog2e;
  const float dsum = p.dsum[stat];

  float q[D], dov[D], dq[D];
#pragma unroll
  for (int t = 0; t < D; ++t) { q[t] = to_f(Q[t]) * c; dov[t] = to_f(dO[t]); dq[t] = 0.f; }

  __shared__ float Ks[kTile][D];
  __shared__ float Vs[kTile][D];
  int kend = p.Nk;
  if (p.causal) {
    const int last_q = p.q_start + min(i0 + kRows - 1, p.Nq - 1);
    kend = max(0, min(p.Nk, last_q - p.k_start + 1));
  }
  const int qpos = p.q_start + i;
  const int jbeg = p.window > 0 ? max(0, p.q_start + i0 - (p.window - 1) - p.k_start) / kTile * kTile : 0;
  for (int j0 = jbeg; j0 < kend; j0 += kTile) {
    if (!block_kept(p, i0, j0)) continue;   // (uniform over the workgroup)
    for (int e = tid; e < kTile * D; e += kRows) {
      const int r = e / D, col = e % D;
      const bool in = j0 + r < p.Nk;
      Ks[r][col] = in ? to_f(K[(j0 + r) * kstride + col]) : 0.f;
      Vs[r][col] = in ? to_f(V[(j0 + r) * kstride + col]) : 0.f;
    }
    __syncthreads();
    const int jn = min(kTile, kend - j0);
    for (int jj = 0; jj < jn; ++jj) {
      if (p.causal && p.k_start + j0 + jj > qpos) break;
      if (p.window > 0 && p.k_start + j0 + jj <= qpos - p.window) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int t = 0; t < D; ++t) {
        s = fmaf(q[t], Ks[jj][t], s);
        dp = fmaf(dov[t], Vs[jj][t], dp);
      }
      const float ds = exp2f(s - lse2) * (dp - dsum);
#pragma unroll
      for (int t = 0; t < D; ++t) dq[t] = fmaf(ds, Ks[jj][t], dq[t]);
    }
    __syncthreads();
  }
  if (i < p.Nq) {
    const long long off = (qrow(p, b, p.q_start + i) + h) * D;
    if (p.accumulate) {
      float* DQ = (float*)p.dq + off;
#pragma unroll
      for (int t = 0; t < D; ++t) DQ[t] += dq[t] * p.scale;
    } else {
      T* DQ = (T*)p.dq + off;
#pragma unroll
      for (int t = 0; t < D; ++t) DQ[t] = from_f<T>(dq[t] * p.scale);
    }
  }
}

template <typename T, typename TO, int D>
hipError_t fwd_simt_launch(const Params& p, hipStream_t s) {
  dim3 grid((p.Nq + kRows - 1) / kRows, p.H, p.B);
  hipLaunchKernelGGL((fwd_simt<T, TO, D>), grid, dim3(kRows), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_simt_launch(const Params& p, hipStream_t s) {
  dim3 gk((p.Nk + kRows - 1) / kRows, p.Hkv, p.B);
  hipLaunchKernelGGL((bwd_dkdv_simt<T, D>), gk, dim3(kRows), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 gq((p.Nq + kRows - 1) / kRows, p.H, p.B);
  hipLaunchKernelGGL((bwd_dq_simt<T, D>), gq, dim3(kRows), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_simt(const Params& p, int dtype, bool out_f32, hipStream_t s) {
  if (dtype == 0) return p.d == 64 ? fwd_simt_launch<float, float, 64>(p, s) : fwd_simt_launch<float, float, 128>(p, s);
  if (out_f32) return p.d == 64 ? fwd_simt_launch<bf16, float, 64>(p, s) : fwd_simt_launch<bf16, float, 128>(p, s);
  return p.d == 64 ? fwd_simt_launch<bf16, bf16, 64>(p, s) : fwd_simt_launch<bf16, bf16, 128>(p, s);
}

hipError_t launch_bwd_simt(const Params& p, int dtype, hipStream_t s) {
  if (dtype == 0) return p.d == 64 ? bwd_simt_launch<float, 64>(p, s) : bwd_simt_launch<float, 128>(p, s);
  return p.d == 64 ? bwd_simt_launch<bf16, 64>(p, s) : bwd_simt_launch<bf16, 128>(p, s);
}

}  // namespace miattn
