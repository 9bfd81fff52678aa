// bf16 forward pass on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// The method is FlashAttention's tiled forward with online softmax
// (FlashAttention abstract page: tiles of K and V move through on-chip
// memory; FlashAttention-2 reviews page, reviewer 2, points 1-3: rescaling
// deferred to one division at the end, the logsumexp saved, parallelism over
// query tiles) with whole-tile skipping above the causal diagonal
// (FlashAttention-2 reviews page, reviewer 4, section 3.1).
//
// Work split (MI355X-specific, not from the pages):
//  * a workgroup of NW waves owns NW*QB*32 query rows of one (b, h); each
//    wave owns QB blocks of 32 rows, so its row max and row sum never leave
//    the wave (the pages' warp partitioning, with 64-lane wavefronts);
//  * K and V tiles of BC=64 keys are staged in LDS, double-buffered, with
//    one barrier per tile; the next tile's global loads are issued a full
//    tile ahead into registers;
//  * scores are computed transposed, S^T = K Q^T, with K's rows loaded in a
//    bit-permuted order (sigma32) so that each lane's 32x32 accumulator holds
//    8 consecutive keys of one query: exactly the B-operand layout of the
//    next product O^T += V^T P^T. P never moves between lanes.
//  * V is transposed into LDS (V^T rows are head-dimension columns); LDS rows
//    are padded by 16 bytes so every operand read is base + immediate and the
//    16-lane service groups of ds_read_b128 hit distinct banks;
//  * the running max is only raised when a row's tile max exceeds it by more
//    than 8 (log2 units); otherwise the old max is kept, p <= 2^8, and the
//    accumulator is not rescaled. The result is unchanged (numerator and
//    denominator share the max), and most tiles skip the rescale entirely;
//  * the row sum is accumulated from the float32 probabilities before they
//    are rounded to bf16 for the P V product, so the saved logsumexp keeps
//    float32 accuracy even for rows with few keys;
//  * causal workgroups are launched heaviest first, and with H % 8 == 0 the
//    heads are permuted so that every workgroup of one K/V head group lands
//    on the same XCD (workgroups are dealt to the 8 XCDs round-robin).
#include "common.h"
#include "kernels.h"
#include "mfma_common.h"

namespace miattn {

namespace {

constexpr int BC = 64;   // keys per tile

constexpr int PAD = LDS_PAD;

template <int D>
struct Smem {
  static constexpr int KROW = D + PAD;    // K tile row-major [key][d]
  static constexpr int VROW = BC + PAD;   // V tile transposed [d][key]
  bf16 k[2][BC * KROW];
  bf16 vt[2][D * VROW];
};


template <int D, int NW>
struct TileLoader {
  // K: (BC * D / 8) chunks of 16 B; V: (BC/4) * (D/8) blocks of 4 keys x 8 columns.
  static constexpr int KCH = D / 8;
  static constexpr int KCHUNKS = BC * KCH;
  static constexpr int NT = NW * 64;
  static constexpr int KPER = (KCHUNKS + NT - 1) / NT;
  static constexpr int VBLK = (BC / 4) * (D / 8);
  static constexpr int VPER = (VBLK + NT - 1) / NT;
  bf16x8 kreg[KPER];
  bf16x8 vreg[VPER][4];

  // Loads are unconditional, from clamped rows: a select between a pending
  // load and a constant would force a wait for the load right here. Rows past
  // nk hold copies of row nk-1 (finite); their scores are masked to -inf, so
  // they contribute nothing.
  __device__ __forceinline__ void load(const bf16* K, const bf16* V, long long rstride, int j0, int nk, int tid) {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int c = min(tid + i * NT, KCHUNKS - 1);
      const int row = min(j0 + c / KCH, nk - 1), ch = c % KCH;
      kreg[i] = *(const bf16x8*)(K + row * rstride + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int blk = min(tid + i * NT, VBLK - 1);
      const int kq = blk % (BC / 4), oc = blk / (BC / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = min(j0 + kq * 4 + r, nk - 1);
        vreg[i][r] = *(const bf16x8*)(V + key * rstride + oc * 8);
      }
    }
  }

  __device__ __forceinline__ void store(bf16* ks, bf16* vt, int tid) const {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int c = tid + i * NT;
      if (c < KCHUNKS) {
        const int row = c / KCH, ch = c % KCH;
        *(bf16x8*)(ks + row * Smem<D>::KROW + ch * 8) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int blk = tid + i * NT;
      if (blk < VBLK) {
        const int kq = blk % (BC / 4), oc = blk / (BC / 4);
        store_transposed4x8(vt, Smem<D>::VROW, oc * 8, kq * 4, vreg[i]);
      }
    }
  }
};

template <int D, int QB, int NW, bool CAUSAL, typename TO>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void fwd_mfma_kernel(Params p) {
  constexpr int BR = NW * QB * 32;
  constexpr int KS = D / 16;   // k-steps of the QK^T product
  constexpr int DB = D / 32;   // 32-column blocks of O
  __shared__ __attribute__((aligned(16))) Smem<D> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;

  // ---- workgroup -> (b, h, query tile), heaviest causal tiles first
  const int ntq = gridDim.y;
  const int qt = CAUSAL ? (ntq - 1 - (int)blockIdx.y) : (int)blockIdx.y;
  const int h = xcd_head(blockIdx.x, p.H);
  const int b = blockIdx.z;
  const int kvh = h / p.G;
  const int q0 = qt * BR;                         // first local query row of the tile
  const int wq0 = q0 + wave * QB * 32;            // first local query row of this wave

  const long long qrs = (long long)p.H * D;       // row strides (elements)
  const long long krs = (long long)p.Hkv * D;
  const bf16* Q = (const bf16*)p.q + ((long long)b * p.N + p.q_start) * qrs + (long long)h * D;
  const bf16* K = (const bf16*)p.k + ((long long)b * p.N + p.k_start) * krs + (long long)kvh * D;
  const bf16* V = (const bf16*)p.v + ((long long)b * p.N + p.k_start) * krs + (long long)kvh * D;

  // ---- scale: scores kept in the log2 domain; a non-positive scale is folded into Q
  float c = fabsf(p.scale) * kLog2e;
  float qsign = p.scale < 0.f ? -1.f : 1.f;
  if (p.scale == 0.f) { c = 1.f; qsign = 0.f; }

  // ---- Q^T operands (B operand of S^T = K Q^T): lane (g, n) holds Q[row n][ks*16 + g*8 .. +8]
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wq0 + qb * 32 + n;
    const int rc = min(row, p.Nq - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 x = *(const bf16x8*)(Q + rc * qrs + ks * 16 + g * 8);
      if (qsign != 1.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (bf16)((float)x[e] * qsign);
      }
      qf[qb][ks] = x;
    }
  }
  wait_global_loads();

  // ---- key range of the workgroup
  int nkt = (p.Nk + BC - 1) / BC;
  if (CAUSAL) {
    const int last_q = p.q_start + min(q0 + BR - 1, p.Nq - 1);   // absolute position
    const int kend = min(p.Nk, last_q - p.k_start + 1);
    nkt = kend > 0 ? (kend + BC - 1) / BC : 0;
  }
  const int wq_first = p.q_start + wq0;

  f32x16 acc[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{};
  }

  TileLoader<D, NW> ld;
  if (nkt > 0) {
    ld.load(K, V, krs, 0, p.Nk, tid);
    ld.store(sm.k[0], sm.vt[0], tid);
    if (nkt > 1) ld.load(K, V, krs, BC, p.Nk, tid);
  }
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const bf16* ks_ = sm.k[j & 1];
    const bf16* vt_ = sm.vt[j & 1];
    const int kpos0 = p.k_start + j * BC;   // absolute position of the tile's first key
    {   // no per-wave skip: a per-wave branch makes the register allocator
        // shuttle accumulators between AGPRs and VGPRs every iteration; fully
        // masked waves (diagonal tiles only) compute P = 0 instead
      // ---- S^T = K Q^T for 2 blocks of 32 keys; step i = (ks, kb), chains kb interleaved
      f32x16 s[2][QB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
      const bf16* kbase0 = ks_ + sigma32(n) * Smem<D>::KROW + g * 8;
      pipelined_products<2 * KS, 4>(
          [&](int i) { return lds_read16(kbase0, (i & 1) * 32 * Smem<D>::KROW + (i >> 1) * 16); },
          [&](int i, bf16x8 a) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[i & 1][qb] = mfma32(a, qf[qb][i >> 1], s[i & 1][qb]);
          });
      // ---- mask: keys past the diagonal or past Nk
      const bool need_mask = (CAUSAL && kpos0 + BC - 1 > wq_first) || (j * BC + BC > p.Nk);
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qpos = p.q_start + wq0 + qb * 32 + n;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kin = kb * 32 + sigma_row(g, r);
              const bool bad = (j * BC + kin >= p.Nk) || (CAUSAL && kpos0 + kin > qpos);
              if (bad) s[kb][qb][r] = -INFINITY;
            }
        }
      }
      // ---- online softmax (per query block)
      bf16x8 pf[QB][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = s[0][qb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][qb][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][qb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = mx * c;
        const bool raise = mt > m[qb] + 8.f;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
          const float mnew = raise ? mt : m[qb];
          const float alpha = exp2f(m[qb] - mnew);
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
          m[qb] = mnew;
        }
        const float mneg = -m[qb];
        float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            bf16x8 x;
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][half * 8 + e], c, mneg));
              const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][half * 8 + e + 1], c, mneg));
              lsum0 += p0;
              lsum1 += p1;
              x[e] = (bf16)p0;
              x[e + 1] = (bf16)p1;
            }
            pf[qb][kb * 2 + half] = x;
          }
        }
        const float lsum = lsum0 + lsum1;
        l[qb] += lsum;
      }
      // ---- O^T += V^T P^T; step i = (kq, db), chains db interleaved
      const bf16* vbase0 = vt_ + n * Smem<D>::VROW + g * 8;
      pipelined_products<4 * DB, 4>(
          [&](int i) { return lds_read16(vbase0, (i % DB) * 32 * Smem<D>::VROW + (i / DB) * 16); },
          [&](int i, bf16x8 a) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) acc[qb][i % DB] = mfma32(a, pf[qb][i / DB], acc[qb][i % DB]);
          });
    }
    if (j + 1 < nkt) {
      ld.store(sm.k[(j + 1) & 1], sm.vt[(j + 1) & 1], tid);
      if (j + 2 < nkt) ld.load(K, V, krs, (j + 2) * BC, p.Nk, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wq0 + qb * 32 + n;
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    if (row < p.Nq) {
      const float inv = 1.f / lt;
      TO* O = (TO*)p.o + (((long long)b * p.N + p.q_start + row) * p.H + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // accumulator rows (r/4)*8 + g*4 + r%4: four runs of 4 columns
#pragma unroll
        for (int run = 0; run < 4; ++run) {
          TO* dst = O + db * 32 + run * 8 + g * 4;
          if constexpr (sizeof(TO) == 2) {
            bf16x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (bf16)(acc[qb][db][run * 4 + e] * inv);
            *(bf16x4*)dst = x;
          } else {
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = acc[qb][db][run * 4 + e] * inv;
            *(f32x4*)dst = x;
          }
        }
      }
      if (g == 0) p.lse[((long long)b * p.H + h) * p.N + p.q_start + row] = (m[qb] + __log2f(lt)) * kLn2;
    }
  }
}

template <int D, int QB, int NW, typename TO>
hipError_t launch_cfg(const Params& p, hipStream_t s) {
  constexpr int BR = NW * QB * 32;
  const dim3 grid(p.H, (p.Nq + BR - 1) / BR, p.B);
  if (p.causal)
    hipLaunchKernelGGL((fwd_mfma_kernel<D, QB, NW, true, TO>), grid, dim3(NW * 64), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<D, QB, NW, false, TO>), grid, dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma(const Params& p, bool out_f32, hipStream_t s) {
  if (p.d == 128) return out_f32 ? launch_cfg<128, 1, 8, float>(p, s) : launch_cfg<128, 1, 8, bf16>(p, s);
  return out_f32 ? launch_cfg<64, 1, 8, float>(p, s) : launch_cfg<64, 1, 8, bf16>(p, s);
}

}  // namespace miattn
