// bf16 backward pass on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// The backward rebuilds P tile by tile from the saved logsumexp instead of
// re-running the forward (DistFlashAttn reviews page, review 1 point 3;
// FlashAttention-2 reviews page, reviewer 2, point 2) and never forms the
// N x N matrix. With D_i = rowsum(dO_i * O_i) computed beforehand:
//     P = exp(scale Q K^T - LSE),  dP = dO V^T,  dS = P (dP - D)
//     dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K
// Grouped-query heads: dK and dV of a K/V head are summed over the query
// heads that read it (FlashAttention-2 reviews page, reviewer 1, MQA/GQA
// paragraph of the backward section).
//
// Work split (MI355X-specific): two kernels, neither shares a partial sum
// with another workgroup, so no atomics are needed and results are bitwise
// deterministic. Accumulating dQ across key tiles with float32 atomics would
// cost as much memory traffic as the whole computation takes on MI355X.
//  * bwd_dkdv: one workgroup per 128 keys of one (b, K/V head); each of its 4
//    waves holds 32 keys' K and V as matrix-core operands and their dK, dV
//    accumulators in registers, and streams 64-row tiles of Q and dO
//    (loaded straight from global memory into LDS), LSE and D over every
//    query head of the group. Products: S = Q K^T, dP = dO V^T (query rows
//    read in sigma32 order, so each lane's accumulator holds 8 consecutive
//    queries of one key = the B operand of the next products), then
//    dV^T += dO^T P and dK^T += Q^T dS with dO^T / Q^T read by transposing
//    LDS reads (accumulators hold 16 columns of one key per lane).
//  * bwd_dq: one workgroup per query tile of one (b, h), the forward's
//    structure: S^T = K Q^T and dP^T = V dO^T from row-major K and V tiles,
//    then dQ^T += K^T dS^T with K^T read from the same K tile by
//    transposing LDS reads.
#include "common.h"
#include "kernels.h"
#include "mfma_common.h"

namespace miattn {

namespace {

constexpr int PAD = LDS_PAD;

// ============================================================ dK, dV

constexpr int DKV_NW = 4;            // waves per workgroup
constexpr int DKV_KW = 32;           // keys per wave
constexpr int DKV_BK = DKV_NW * DKV_KW;
constexpr int DKV_BQ = 64;           // query rows per streamed tile

// LDS tile of 64 query rows (Q or dO), row-major. Rows are padded to D + 32
// elements and the 16-byte chunk index is XORed with (row / 4) % 4: then the
// sigma32-ordered ds_read_b128 row reads of S = Q K^T, dP = dO V^T and the
// 4-row transposing reads of dV^T = dO^T P, dK^T = Q^T dS are both free of
// bank conflicts, and the tile is written by direct global -> LDS loads.
template <int D>
struct DkdvSmem {
  static constexpr int ROW = D + 32;
  static constexpr int TILE = DKV_BQ * ROW;    // elements per tile
  bf16 q[2][TILE];
  bf16 o[2][TILE];                             // dO
  float stat[2][2][DKV_BQ];    // [0]: LSE * log2(e) (+inf past the last row), [1]: D
};

template <int D>
__device__ __forceinline__ int dkdv_swz(int row, int chunk) {
  return row * DkdvSmem<D>::ROW + ((chunk ^ ((row >> 2) & 3)) << 3);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(DKV_NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(Params p) {
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int ROW = DkdvSmem<D>::ROW, TILE = DkdvSmem<D>::TILE;
  constexpr int TILE_KB = TILE * 2 / 1024;          // 1 KB direct loads per tile
  static_assert(TILE_KB % DKV_NW == 0, "tile loads split evenly over the waves");
  constexpr int NL = TILE_KB / DKV_NW;             // per wave, per tensor
  __shared__ __attribute__((aligned(16))) DkdvSmem<D> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;
  const int gkv = blockIdx.x;          // all tiles of one K/V head share an XCD
  const int kt = blockIdx.y;           // tile 0 has the most causal work: dispatched first
  const int b = blockIdx.z;
  const int k0 = kt * DKV_BK;
  const int kw0 = k0 + wave * DKV_KW;

  const long long krs = (long long)p.Hkv * D, qrs = (long long)p.H * D;
  const bf16* K = (const bf16*)p.k + ((long long)b * p.N + p.k_start) * krs + (long long)gkv * D;
  const bf16* V = (const bf16*)p.v + ((long long)b * p.N + p.k_start) * krs + (long long)gkv * D;
  const bf16* Qb = (const bf16*)p.q + ((long long)b * p.N + p.q_start) * qrs;
  const bf16* Ob = (const bf16*)p.dout + ((long long)b * p.N + p.q_start) * qrs;

  float c = fabsf(p.scale) * kLog2e;
  float ksign = p.scale < 0.f ? -1.f : 1.f;
  if (p.scale == 0.f) { c = 1.f; ksign = 0.f; }

  // K^T and V^T operands (B of S = Q K^T and dP = dO V^T): lane (g, n) holds row kw0+n, columns 16ks+8g..
  bf16x8 kf[KS], vf[KS];
  {
    const int kr = min(kw0 + n, p.Nk - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 x = *(const bf16x8*)(K + kr * krs + ks * 16 + g * 8);
      if (ksign != 1.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (bf16)((float)x[e] * ksign);
      }
      kf[ks] = x;
      vf[ks] = *(const bf16x8*)(V + kr * krs + ks * 16 + g * 8);
    }
  }
  wait_global_loads();

  // dK^T, dV^T accumulators, in AGPRs (mfma32_agpr)
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
    agpr_settle(dk[db], dv[db]);
  }

  const int nqt = (p.Nq + DKV_BQ - 1) / DKV_BQ;
  int first = 0;
  if (CAUSAL) first = min(nqt, max(0, p.k_start + k0 - p.q_start) / DKV_BQ);
  const int per_head = nqt - first;
  const int niter = p.G * per_head;
  const int kpos = p.k_start + kw0 + n;          // this lane's key position
  const int wk_first = p.k_start + kw0;

  // Direct loads: this wave's i-th 1 KB piece of a tile covers LDS bytes
  // [(wave*NL + i) KB, +1 KB); lane l fills 16 bytes at offset 16 l: tile row
  // r, logical chunk ch (padding bytes are filled from chunk 0), read from
  // byte loff[i] = 2 (r * row stride + 8 ch) past the tile's first row. Rows
  // past the last query read as zeros (buffer range check).
  uint32_t loff[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int off = (wave * NL + i) * 1024 + 16 * lane;      // bytes into the tile
    const int row = off / (ROW * 2), pch = (off % (ROW * 2)) / 16;
    const int col = pch < D / 8 ? ((pch ^ ((row >> 2) & 3)) << 3) : 0;
    loff[i] = (uint32_t)(row * qrs + col) * 2u;
  }
  const uint32_t qbytes = (uint32_t)(p.Nq * qrs * 2);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qb, qbytes), ro = make_rsrc(Ob, qbytes);
  auto load_piece = [&](int piece, int buf, int h, int q0) {   // piece < 2 NL: Q then dO
    const int i = piece % NL;
    const bool is_o = piece >= NL;
    const uint32_t soff = (uint32_t)(q0 * qrs + h * D) * 2u;
    buffer_load_lds16(is_o ? ro : rq, loff[i], soff, (is_o ? sm.o[buf] : sm.q[buf]) + (wave * NL + i) * 512);
  };
  float st;          // LSE (tid < 64) or D (64 <= tid < 128) of row q0 + tid % 64
  bool st_valid;
  auto stat_load = [&](int h, int q0) {
    const int row = q0 + (tid & 63);
    st_valid = row < p.Nq;
    const long long si = ((long long)b * p.H + h) * p.N + p.q_start + min(row, p.Nq - 1);
    st = ((tid & 64) ? p.dsum : p.lse)[si];
  };
  auto stat_store = [&](int buf) {
    if (tid < 128) {
      const float v = (tid < 64) ? (st_valid ? st * kLog2e : INFINITY) : (st_valid ? st : 0.f);
      sm.stat[buf][tid >> 6][tid & 63] = v;
    }
  };

  // per-lane LDS read bases (elements). S/dP A operands: row sigma32(n) (+32 qb),
  // logical chunk 2 ks + g = 4 (ks/2) + 2 (ks%2) + g -> base for ks parity e.
  const int srow = sigma32(n), sf = (srow >> 2) & 3;
  int rd_s[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) rd_s[e] = srow * ROW + (((2 * e + g) ^ sf) << 3);
  // transposing reads for dO^T / Q^T (k-step t, column block db): lane j of
  // 16-lane group G4 = (g, hf) addresses row 16t + 8g + 4rd + j/4,
  // columns 32db + 16hf + 4(j%4).
  int rd_t[2];
  {
    const int G4 = lane >> 4, j = lane & 15, hf = G4 & 1;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int row = 8 * g + 4 * rd + (j >> 2);
      const int chunk = (2 * hf + ((j & 3) >> 1)) ^ ((2 * g + rd) & 3);
      rd_t[rd] = row * ROW + (chunk << 3) + 4 * (j & 1);
    }
  }

  if (niter > 0) {   // first tile: head gkv * G, rows from first * 64
    const int h = gkv * p.G, q0 = first * DKV_BQ;
#pragma unroll
    for (int piece = 0; piece < 2 * NL; ++piece) load_piece(piece, 0, h, q0);
    stat_load(h, q0);
    wait_global_loads();
    stat_store(0);
  }
  __syncthreads();

  // One query tile: `it` counts tiles (buffer parity), (h_nx, q0_nx) is the
  // tile to prefetch. Only tiles that cross the causal diagonal of the
  // workgroup's keys run the body with the mask test.
  auto tile = [&](auto mc, int it, int q0, int h_nx, int q0_nx) {
    constexpr bool MASKED = decltype(mc)::value;
    const int buf = it & 1;
    const bool need_mask = MASKED && (wk_first + DKV_KW - 1 > p.q_start + q0);
    const bf16* qt = sm.q[buf];
    const bf16* ot = sm.o[buf];
    const float* lse2 = sm.stat[buf][0];
    const float* dsm = sm.stat[buf][1];

    // Every wave computes every tile: on the one diagonal tile where a wave's
    // keys are all after the tile's queries, the mask zeroes P (a per-wave
    // branch would make the allocator shuttle accumulators through AGPRs).
    //
    // 4 phases of PL = D/8 lock steps, one MFMA each; the tile's 64 queries
    // are two halves qb:
    //   phase 0: S, dP of half 0          + direct loads of the next tile
    //   phase 1: S, dP of half 1          + softmax of half 0
    //   phase 2: dV^T, dK^T over half 0   + softmax of half 1
    //   phase 3: dV^T, dK^T over half 1   + the next tile's LSE / D to LDS
    // One body serves every tile: the mask test is a compare and a select per
    // element against a per-lane threshold (never true below the diagonal).
    constexpr int PL = D / 8;
    const int mthr = need_mask ? kpos - (p.q_start + q0) : -0x40000000;
    f32x16 s[2], dp[2];
    s[0] = f32x16{}; dp[0] = f32x16{}; s[1] = f32x16{}; dp[1] = f32x16{};
    bf16x8 pa[4], da[4];
    f32x4 lq[2], dq4[2];   // LSE and D of the 8 query rows being softmaxed

    // softmax sub-step w (0..7) of half qb: lane (g, key n), register r <->
    // query q0 + 32 qb + sigma_row(g, r); sub-step w forms P and dS for
    // elements 2k, 2k+1 (k = w % 4) of register group h2 = w / 4, whose 8
    // query rows' LSE and D are read at the group's first sub-step.
    auto softmax_sub = [&](auto qbc, auto wc) {
      constexpr int qb = decltype(qbc)::value, w = decltype(wc)::value;
      constexpr int h2 = w >> 2, k = w & 3;
      const int qi0 = qb * 32 + h2 * 16 + g * 8;    // 8 consecutive query rows
      const int tq = mthr - qi0;                     // element e masked iff e < tq
      if constexpr (k == 0) {
        lq[0] = *(const f32x4*)(lse2 + qi0);
        lq[1] = *(const f32x4*)(lse2 + qi0 + 4);
        dq4[0] = *(const f32x4*)(dsm + qi0);
        dq4[1] = *(const f32x4*)(dsm + qi0 + 4);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * k + u;
        const int r = h2 * 8 + e;
        const float x = __builtin_amdgcn_exp2f(fmaf(s[qb][r], c, -lq[e >> 2][e & 3]));
        const float pv = (MASKED && e < tq) ? 0.f : x;
        pa[qb * 2 + h2][e] = (bf16)pv;
        da[qb * 2 + h2][e] = (bf16)(pv * (dp[qb][r] - dq4[e >> 2][e & 3]));
      }
    };

    lockstep_products<4 * PL, 4>(
        [&](auto ic) {
          constexpr int i = decltype(ic)::value, ph = i / PL, j = i % PL;
          if constexpr (ph < 2) {   // S / dP: step j = (ks, which), half ph
            constexpr int ks = j >> 1;
            const bf16* t = (j & 1) ? ot : qt;
            return lds_read16(t + rd_s[ks & 1], ph * 32 * ROW + (ks >> 1) * 32);
          } else {                  // dV / dK: step j = (t, db, which), two transposing reads
            constexpr int t = 2 * (ph - 2) + j / (2 * DB), db = (j >> 1) % DB;
            const bf16* src = (j & 1) ? qt : ot;
            const bf16x4 r0 = lds_read_tr4(src + rd_t[0] + 16 * t * ROW + 32 * db);
            const bf16x4 r1 = lds_read_tr4(src + rd_t[1] + 16 * t * ROW + 32 * db);
            return bf16x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
          }
        },
        [&](auto ic, bf16x8 a) {
          constexpr int i = decltype(ic)::value, ph = i / PL, j = i % PL;
          if constexpr (ph < 2) {
            if constexpr (j & 1) dp[ph] = mfma32(a, vf[j >> 1], dp[ph]);
            else s[ph] = mfma32(a, kf[j >> 1], s[ph]);
          } else {
            constexpr int t = 2 * (ph - 2) + j / (2 * DB), db = (j >> 1) % DB;
            if constexpr (j & 1) mfma32_agpr(dk[db], a, da[t]);
            else mfma32_agpr(dv[db], a, pa[t]);
          }
        },
        [&](auto ic) {
          constexpr int i = decltype(ic)::value, ph = i / PL, j = i % PL;
          if constexpr (ph == 0) {
            constexpr int lo = j * (2 * NL) / PL, hi = (j + 1) * (2 * NL) / PL;
            [&]<int... Ws>(std::integer_sequence<int, Ws...>) {
              (load_piece(lo + Ws, buf ^ 1, h_nx, q0_nx), ...);
            }(std::make_integer_sequence<int, hi - lo>{});
            if constexpr (j == PL - 1) stat_load(h_nx, q0_nx);
          } else if constexpr (ph == 3) {
            if constexpr (j == PL - 1) stat_store(buf ^ 1);
          } else {
            constexpr int lo = j * 8 / PL, hi = (j + 1) * 8 / PL;
            [&]<int... Ws>(std::integer_sequence<int, Ws...>) {
              (softmax_sub(std::integral_constant<int, ph - 1>{}, std::integral_constant<int, lo + Ws>{}), ...);
            }(std::make_integer_sequence<int, hi - lo>{});
          }
        });
    wait_global_loads();
    __syncthreads();
  };
  // tiles of query tile rows first + t, t < ndiag, cross the diagonal
  int ndiag = 0;
  if (CAUSAL) {
    const int x = p.k_start + k0 + DKV_BK - 1 - p.q_start;   // last key, relative to the query rows
    ndiag = x > 0 ? min(per_head, max(0, (x + DKV_BQ - 1) / DKV_BQ - first)) : 0;
  }
  int it = 0;
  for (int hh = 0; hh < p.G; ++hh) {
    const int h = gkv * p.G + hh;
    // prefetch target after tile t of this head (the very last tile repeats itself)
    auto next = [&](int t, int& hn, int& qn) {
      hn = h;
      qn = (first + t + 1) * DKV_BQ;
      if (t + 1 == per_head) {
        if (hh + 1 < p.G) { hn = h + 1; qn = first * DKV_BQ; }
        else qn = (first + t) * DKV_BQ;
      }
    };
    int t = 0;
    for (; t < ndiag; ++t, ++it) {
      int hn, qn;
      next(t, hn, qn);
      tile(std::true_type{}, it, (first + t) * DKV_BQ, hn, qn);
    }
    for (; t < per_head; ++t, ++it) {
      int hn, qn;
      next(t, hn, qn);
      tile(std::false_type{}, it, (first + t) * DKV_BQ, hn, qn);
    }
  }

  // ---- store dK^T, dV^T: lane (g, key n), register r <-> column 32 db + 8 (r/4) + 4g + r%4
#pragma unroll
  for (int db = 0; db < DB; ++db) agpr_settle(dk[db], dv[db]);
  const int key = kw0 + n;
  if (key < p.Nk) {
    const long long off = (((long long)b * p.N + p.k_start + key) * p.Hkv + gkv) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int run = 0; run < 4; ++run) {
        const int col = db * 32 + run * 8 + g * 4;
        if (p.accumulate) {
          f32x4* a = (f32x4*)((float*)p.dk + off + col);
          f32x4* v = (f32x4*)((float*)p.dv + off + col);
          f32x4 xa = *a, xv = *v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xa[e] += dk[db][run * 4 + e] * p.scale;
            xv[e] += dv[db][run * 4 + e];
          }
          *a = xa;
          *v = xv;
        } else {
          bf16x4 xa, xv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xa[e] = (bf16)(dk[db][run * 4 + e] * p.scale);
            xv[e] = (bf16)dv[db][run * 4 + e];
          }
          *(bf16x4*)((bf16*)p.dk + off + col) = xa;
          *(bf16x4*)((bf16*)p.dv + off + col) = xv;
        }
      }
    }
  }
}

// ============================================================ dQ

constexpr int DQ_BC = 64;   // keys per tile

// K and V tiles (64 keys), row-major in the padded, chunk-swizzled layout of
// DkdvSmem: the sigma32-ordered row reads of S^T = K Q^T and dP^T = V dO^T
// and the transposing reads of K^T for dQ^T = K^T dS^T are conflict-free,
// and both tiles are written by direct global -> LDS loads.
template <int D>
struct DqSmem {
  static constexpr int ROW = D + 32;
  static constexpr int TILE = DQ_BC * ROW;
  bf16 k[2][TILE];
  bf16 v[2][TILE];
};

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void bwd_dq_kernel(Params p) {
  constexpr int BR = NW * 32;
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int ROW = DqSmem<D>::ROW, TILE = DqSmem<D>::TILE;
  constexpr int TILES_KB = 2 * TILE * 2 / 1024;     // K and V, in 1 KB direct loads
  static_assert(TILES_KB % NW == 0, "tile loads split evenly over the waves");
  constexpr int NL = TILES_KB / NW;                // per wave
  constexpr int TILE_KB = TILES_KB / 2;
  __shared__ __attribute__((aligned(16))) DqSmem<D> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;
  const int ntq = gridDim.y;
  const int qt = CAUSAL ? (ntq - 1 - (int)blockIdx.y) : (int)blockIdx.y;
  const int h = xcd_head(blockIdx.x, p.H);
  const int b = blockIdx.z;
  const int kvh = h / p.G;
  const int q0 = qt * BR;
  const int wq0 = q0 + wave * 32;

  const long long qrs = (long long)p.H * D, krs = (long long)p.Hkv * D;
  const bf16* Q = (const bf16*)p.q + ((long long)b * p.N + p.q_start) * qrs + (long long)h * D;
  const bf16* dO = (const bf16*)p.dout + ((long long)b * p.N + p.q_start) * qrs + (long long)h * D;
  const bf16* K = (const bf16*)p.k + ((long long)b * p.N + p.k_start) * krs + (long long)kvh * D;
  const bf16* V = (const bf16*)p.v + ((long long)b * p.N + p.k_start) * krs + (long long)kvh * D;

  float c = fabsf(p.scale) * kLog2e;
  float qsign = p.scale < 0.f ? -1.f : 1.f;
  if (p.scale == 0.f) { c = 1.f; qsign = 0.f; }

  // Q and dO as B operands of S^T = K Q^T and dP^T = V dO^T: lane (g, n) holds row wq0+n, columns 16ks+8g..
  const int row = wq0 + n;
  const int rc = min(row, p.Nq - 1);
  bf16x8 qf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8 x = *(const bf16x8*)(Q + rc * qrs + ks * 16 + g * 8);
    if (qsign != 1.f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (bf16)((float)x[e] * qsign);
    }
    qf[ks] = x;
    of[ks] = *(const bf16x8*)(dO + rc * qrs + ks * 16 + g * 8);
  }
  const long long si = ((long long)b * p.H + h) * p.N + p.q_start + rc;
  const float lse2 = p.lse[si] * kLog2e;
  const float dsum = p.dsum[si];
  wait_global_loads();
  const int qpos = p.q_start + row;

  int nkt = (p.Nk + DQ_BC - 1) / DQ_BC;
  if (CAUSAL) {
    const int last_q = p.q_start + min(q0 + BR - 1, p.Nq - 1);
    const int kend = min(p.Nk, last_q - p.k_start + 1);
    nkt = kend > 0 ? (kend + DQ_BC - 1) / DQ_BC : 0;
  }
  const int wq_first = p.q_start + wq0;

  // Direct loads: 1 KB piece s = wave*NL + i of the two tiles (K: s < TILE_KB,
  // then V) covers tile bytes [(s % TILE_KB) KB, +1 KB); lane l fills 16 bytes
  // at 16 l: tile row r, logical chunk ch (padding from chunk 0), read from
  // byte loff[i] = 2 (r * row stride + 8 ch) past the tile's first key.
  uint32_t loff[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int off = ((wave * NL + i) % TILE_KB) * 1024 + 16 * lane;
    const int r_ = off / (ROW * 2), pch = (off % (ROW * 2)) / 16;
    const int col = pch < D / 8 ? ((pch ^ ((r_ >> 2) & 3)) << 3) : 0;
    loff[i] = (uint32_t)(r_ * krs + col) * 2u;
  }
  // keys past the last one read as zeros (buffer range check); the mask drops them
  const uint32_t kbytes = (uint32_t)(((p.Nk - 1) * krs + D) * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K, kbytes), rv = make_rsrc(V, kbytes);
  auto load_piece = [&](int i, int buf, int j0) {
    const int sl = wave * NL + i;                  // wave-uniform
    const bool is_v = sl >= TILE_KB;
    buffer_load_lds16(is_v ? rv : rk, loff[i], (uint32_t)(j0 * krs) * 2u,
                      (is_v ? sm.v[buf] : sm.k[buf]) + (sl % TILE_KB) * 512);
  };

  // per-lane LDS read bases (elements): K / V rows sigma32(n) (+32 kb), logical
  // chunk 2 ks + g -> base for ks parity e; K^T transposing reads: lane j of
  // 16-lane group (g, hf) addresses key row 16t + 8g + 4rd + j/4, columns
  // 32db + 16hf + 4(j%4).
  const int srow = sigma32(n), sf = (srow >> 2) & 3;
  int rd_s[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) rd_s[e] = srow * ROW + (((2 * e + g) ^ sf) << 3);
  int rd_t[2];
  {
    const int G4 = lane >> 4, j = lane & 15, hf = G4 & 1;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int r_ = 8 * g + 4 * rd + (j >> 2);
      const int chunk = (2 * hf + ((j & 3) >> 1)) ^ ((2 * g + rd) & 3);
      rd_t[rd] = r_ * ROW + (chunk << 3) + 4 * (j & 1);
    }
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  if (nkt > 0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) load_piece(i, 0, 0);
    wait_global_loads();
  }
  __syncthreads();

  // Lock steps per key tile (PS = 2 KS products per key block, PD = 2 DB per 16 keys):
  //   phase 0 (PS steps): S^T, dP^T of keys 0-31    + direct loads of the next tile
  //   phase 1 (PS steps): S^T, dP^T of keys 32-63   + dS of keys 0-31
  //   phase 2 (PD steps): dQ^T over keys 0-31       + dS of keys 32-63
  //   phase 3 (PD steps): dQ^T over keys 32-63
  // Key tiles before nplain lie entirely below the causal diagonal of every
  // row of the workgroup and before the ragged end: they run a body without
  // the mask test; the rest (at most 5 tiles) run the masked body.
  constexpr int PS = 2 * KS, PD = 2 * DB;
  int nplain = min(nkt, p.Nk / DQ_BC);
  if (CAUSAL) nplain = min(nplain, max(0, p.q_start + q0 - p.k_start + 1) / DQ_BC);
  auto tile = [&](auto mc, int j) {
    constexpr bool MASKED = decltype(mc)::value;
    const int buf = j & 1;
    const int kpos0 = p.k_start + j * DQ_BC;
    const int jn = min(j + 1, nkt - 1) * DQ_BC;      // next tile (the last tile repeats itself)
    // masked iff key index inside the tile > thr (causal and the ragged end)
    int thr = p.Nk - 1 - j * DQ_BC;
    if (CAUSAL && kpos0 + DQ_BC - 1 > wq_first) thr = min(thr, qpos - kpos0);
    const bf16* kt = sm.k[buf];
    const bf16* vt = sm.v[buf];
    f32x16 s[2], dp[2];
    s[0] = f32x16{}; dp[0] = f32x16{}; s[1] = f32x16{}; dp[1] = f32x16{};
    bf16x8 dsb[4];

    // dS for elements 2w, 2w+1 (w = 0..7) of key block kb: lane (g, query n),
    // register r <-> key 32 kb + sigma_row(g, r)
    auto ds_sub = [&](auto kbc, auto wc) {
      constexpr int kb = decltype(kbc)::value, w = decltype(wc)::value;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = 2 * w + u;
        const float x = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -lse2));
        float pv = x;
        if constexpr (MASKED) {
          const int kin = kb * 32 + ((r < 8) ? (g * 8 + r) : (16 + g * 8 + r - 8));
          pv = kin > thr ? 0.f : x;
        }
        dsb[kb * 2 + (r >> 3)][r & 7] = (bf16)(pv * (dp[kb][r] - dsum));
      }
    };

    lockstep_products<2 * PS + 2 * PD, 4>(
        [&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr (i < 2 * PS) {            // S^T / dP^T: (kb, ks, which)
            constexpr int kb = i / PS, jj = i % PS, ks = jj >> 1;
            const bf16* t = (jj & 1) ? vt : kt;
            return lds_read16(t + rd_s[ks & 1], kb * 32 * ROW + (ks >> 1) * 32);
          } else {                                // dQ^T: (t, db) with t = key block of 16
            constexpr int ii = i - 2 * PS, t = ii / DB, db = ii % DB;
            const bf16x4 r0 = lds_read_tr4(kt + rd_t[0] + 16 * t * ROW + 32 * db);
            const bf16x4 r1 = lds_read_tr4(kt + rd_t[1] + 16 * t * ROW + 32 * db);
            return bf16x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
          }
        },
        [&](auto ic, bf16x8 a) {
          constexpr int i = decltype(ic)::value;
          if constexpr (i < 2 * PS) {
            constexpr int kb = i / PS, jj = i % PS, ks = jj >> 1;
            if constexpr (jj & 1) dp[kb] = mfma32(a, of[ks], dp[kb]);
            else s[kb] = mfma32(a, qf[ks], s[kb]);
          } else {
            constexpr int ii = i - 2 * PS, t = ii / DB, db = ii % DB;
            acc[db] = mfma32(a, dsb[t], acc[db]);
          }
        },
        [&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr (i < PS) {                 // phase 0: next tile's direct loads
            constexpr int lo = i * NL / PS, hi = (i + 1) * NL / PS;
            [&]<int... Ws>(std::integer_sequence<int, Ws...>) {
              (load_piece(lo + Ws, buf ^ 1, jn), ...);
            }(std::make_integer_sequence<int, hi - lo>{});
          } else if constexpr (i < 2 * PS) {      // phase 1: dS of key block 0
            constexpr int ii = i - PS, lo = ii * 8 / PS, hi = (ii + 1) * 8 / PS;
            [&]<int... Ws>(std::integer_sequence<int, Ws...>) {
              (ds_sub(std::integral_constant<int, 0>{}, std::integral_constant<int, lo + Ws>{}), ...);
            }(std::make_integer_sequence<int, hi - lo>{});
          } else if constexpr (i < 2 * PS + PD) { // phase 2: dS of key block 1
            constexpr int ii = i - 2 * PS, lo = ii * 8 / PD, hi = (ii + 1) * 8 / PD;
            [&]<int... Ws>(std::integer_sequence<int, Ws...>) {
              (ds_sub(std::integral_constant<int, 1>{}, std::integral_constant<int, lo + Ws>{}), ...);
            }(std::make_integer_sequence<int, hi - lo>{});
          }
        });
    wait_global_loads();
    __syncthreads();
  };
  for (int j = 0; j < nplain; ++j) tile(std::false_type{}, j);
  for (int j = nplain; j < nkt; ++j) tile(std::true_type{}, j);

  // ---- store dQ = scale * acc^T: lane (g, query n), register r <-> column 32 db + 8 (r/4) + 4g + r%4
  if (row < p.Nq) {
    const long long off = (((long long)b * p.N + p.q_start + row) * p.H + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int run = 0; run < 4; ++run) {
        const int col = db * 32 + run * 8 + g * 4;
        if (p.accumulate) {
          f32x4* a = (f32x4*)((float*)p.dq + off + col);
          f32x4 x = *a;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] += acc[db][run * 4 + e] * p.scale;
          *a = x;
        } else {
          bf16x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = (bf16)(acc[db][run * 4 + e] * p.scale);
          *(bf16x4*)((bf16*)p.dq + off + col) = x;
        }
      }
    }
  }
}

template <int D>
hipError_t launch_d(const Params& p, hipStream_t s) {
  const dim3 gkv(p.Hkv, (p.Nk + DKV_BK - 1) / DKV_BK, p.B);
  if (p.causal)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), gkv, dim3(DKV_NW * 64), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), gkv, dim3(DKV_NW * 64), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int NW = 8;
  const dim3 gq(p.H, (p.Nq + NW * 32 - 1) / (NW * 32), p.B);
  if (p.causal)
    hipLaunchKernelGGL((bwd_dq_kernel<D, true, NW>), gq, dim3(NW * 64), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, false, NW>), gq, dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_mfma(const Params& p, hipStream_t s) {
  return p.d == 128 ? launch_d<128>(p, s) : launch_d<64>(p, s);
}

}  // namespace miattn
