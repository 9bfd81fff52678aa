// bf16 backward pass on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// The backward rebuilds P tile by tile from the saved logsumexp instead of
// re-running the forward (DistFlashAttn reviews page, review 1 point 3;
// FlashAttention-2 reviews page, reviewer 2, point 2) and never forms the
// N x N matrix. With D_i = rowsum(dO_i * O_i):
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
// The dQ kernel runs first: each of its workgroups also forms D of its own
// query rows (it already holds their dO) and writes it for the dK/dV kernel.
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
//    transposing LDS reads. It uses the 16x16x32 product shape, which
//    sustains more FLOP/s at the chip's power limit; its softmax work per
//    product is low enough for the shape's fewer free VALU issue slots, and
//    each wave's two 16-row query blocks share every K/V fragment, so LDS
//    bytes per FLOP match the 32x32 shape's.
#include "common.h"
#include "kernels.h"
#include "mfma_common.h"

namespace miattn {

namespace {

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
// Three buffers (previous, current and next tile); within a buffer dO
// follows Q and the tile's row statistics follow dO, so all three are
// reached from one base address. A buffer's size is a multiple of the
// 256-byte bank cycle, so every buffer has the same bank pattern.
template <int D>
struct DkdvSmem {
  static constexpr int ROW = D + 32;
  static constexpr int TILE = DKV_BQ * ROW;    // elements per tile
  struct Buf {
    bf16 q[TILE];
    bf16 o[TILE];              // dO
    float stat[2][DKV_BQ];     // [0]: LSE * log2(e) (+inf past the last row), [1]: -D
  };
  Buf buf[3];
};

// Waves per SIMD of the dK/dV kernel: its K/V operands and dK/dV
// accumulators fill one wave's registers at d = 128; at d = 64 they fit
// twice, and two workgroups share a CU.
template <int D> constexpr int dkdv_waves() { return D == 64 ? 2 : 1; }

template <int D, bool CAUSAL, bool WIN = false, bool SPARSE = false>
__global__ __launch_bounds__(DKV_NW * 64) __attribute__((amdgpu_waves_per_eu(dkdv_waves<D>(), dkdv_waves<D>())))
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
  // key tile (tile 0, with the most causal work, first) and batch entry from
  // the grid (tile_grid_index(), mfma_common.h)
  const int tix = tile_grid_index<CAUSAL>();
  int kt = tix;
  int b = batch_grid_index<CAUSAL>();
  if (p.vl_ktiles) {                   // packed batch: (sequence, tile) from the work list
    if (tix >= p.vl_ktiles[0]) return;
    b = p.vl_ktiles[2 + 2 * tix];
    kt = p.vl_ktiles[3 + 2 * tix];
  }
  const int k0 = kt * DKV_BK;
  if (p.cu_seqlens) {                  // packed batch: b is the sequence (from the work list)
    if (!narrow_to_sequence(p, b, k0)) return;
    b = 0;
  }
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
  // K and V operands live in AGPRs (matrix-core operands may be read from
  // there directly), leaving the VGPRs to the per-tile values
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(kf[ks]), "+a"(vf[ks]));

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
  int nqt_end = nqt;   // sliding window: query tiles past the window of the last key see none
  if constexpr (WIN) {
    const int q_hi = p.k_start + k0 + DKV_BK - 1 + p.window - 1 - p.q_start;
    nqt_end = min(nqt, max(0, q_hi / DKV_BQ + 1));
  }
  int per_head = max(0, nqt_end - first);
  // block-sparse: the query tiles of the block column, ascending, from the
  // column's first key on (the same list for every head of the group)
  const int* tl = nullptr;
  if constexpr (SPARSE) {
    static_assert(DKV_BK == BS_COLS && DKV_BQ == BS_TILE, "a workgroup covers one block column of the mask");
    tl = p.bs_col_tiles + (long long)kt * p.bs_ld;
    per_head = p.bs_col_cnt[kt];
  }
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
  const u32x4 rq = rsrc_words(Qb, qbytes), ro = rsrc_words(Ob, qbytes);
  // LDS byte address of buffer 0's Q tile, converted from the generic
  // pointer once (buffers follow at sizeof(Buf), dO at + 2 TILE in each)
  const uint32_t lds_q0 = lds_addr(sm.buf[0].q);
  constexpr uint32_t BUF_BYTES = (uint32_t)sizeof(typename DkdvSmem<D>::Buf);
  constexpr uint32_t STAT_BYTES = 4u * TILE;       // stats past Q and dO in a buffer
  // piece < 2 NL (Q then dO) of a tile into the buffer at byte offset bo
  // from buffer 0; soff = 2 (q0 qrs + h D) for the tile at rows q0 of head h
  auto load_piece = [&](int piece, uint32_t bo, uint32_t soff) {
    const int i = piece % NL;
    const bool is_o = piece >= NL;
    buffer_load_lds16_async(is_o ? ro : rq, loff[i], soff, bo,
                            lds_q0 + (is_o ? 2u * TILE : 0u) + (uint32_t)(wave * NL + i) * 1024u);
  };
  auto tile_soff = [&](int h, int q0) { return (uint32_t)(q0 * qrs + h * D) * 2u; };
  float st;          // LSE (tid < 64) or D (64 <= tid < 128) of row q0 + tid % 64
  bool st_valid;
  // LSE (wave 0) or D (wave 1) of batch entry b from row q_start on; row q
  // of head h is element si = h N + q past it (32-bit: B H N < 2^31), read
  // through a range-checked descriptor over the entry's H N - q_start
  // elements (zeros past them)
  const float* st_base = (wave & 1 ? p.dsum : p.lse) + (long long)b * p.H * p.N + p.q_start;
  const int st_end = p.H * p.N - p.q_start;
  const __amdgpu_buffer_rsrc_t rst = make_rsrc(st_base, (uint32_t)st_end * 4u);
  auto stat_load = [&](int si, int q0) {
    st_valid = q0 + lane < p.Nq;
    st = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rst, 4 * lane, 4 * si, 0));
  };
  auto stat_store = [&](uint32_t bo) {   // into the buffer at byte offset bo
    if (tid < 128) {
      const float v = (tid < 64) ? (st_valid ? st * kLog2e : INFINITY) : (st_valid ? -st : 0.f);
      *(__attribute__((address_space(3))) float*)(lds_q0 + bo + STAT_BYTES + 4 * tid) = v;
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

  // Tiles are taken in the order (query head of the group, query tile);
  // tile k sits in LDS buffer k % 3. The work of one tile is spread over two
  // iterations (software pipeline), so that every phase of matrix-core
  // products carries a quarter of the softmax work:
  //   phase 0: S, dP of half 0 of tile k       + softmax group 1 of half 1 of tile k-1
  //            (+ direct loads of tile k+1)
  //   phase 1: dV^T, dK^T over half 1 of k-1   + softmax group 0 of half 0 of tile k
  //   phase 2: S, dP of half 1 of tile k       + softmax group 1 of half 0 of tile k
  //   phase 3: dV^T, dK^T over half 0 of k     + softmax group 0 of half 1 of tile k
  // (half = 32 query rows, group = 16 of them). Tile -1 is an all-zero buffer
  // with LSE = +inf (P = 0); the last iteration loads one more tile, which
  // nothing reads, and a drain after the loop does what is left of the last
  // tile (its phase-1 products and the softmax they need). Each phase
  // prefetches the LSE / D values the next phase's softmax group needs.
  constexpr int PL = D / 8;          // lock steps per phase
  const int empty_q0 = nqt * DKV_BQ; // rows past the end: zeros, LSE = +inf

  // buffer 2 = tile -1: zero Q / dO, LSE = +inf, D = 0
  {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int i = tid; i < TILE / 8; i += DKV_NW * 64) {
      *(f32x4*)(sm.buf[2].q + 8 * i) = z;
      *(f32x4*)(sm.buf[2].o + 8 * i) = z;
    }
    if (tid < 128) sm.buf[2].stat[tid >> 6][tid & 63] = (tid < 64) ? INFINITY : 0.f;
  }
  // block-sparse: query tile of the next tile and of the one after (fetched
  // an iteration ahead, so the list reads never stall the tile loads)
  int tq_nx = 0, tq_nx2 = 0, t_nx2 = 0;
  if constexpr (SPARSE) {
    t_nx2 = per_head > 2 ? 2 : 0;     // list index of tile 2 (k mod per_head)
    tq_nx = niter > 1 ? uni(tl[per_head > 1 ? 1 : 0]) : 0;
    tq_nx2 = niter > 2 ? uni(tl[t_nx2]) : 0;
  }
  {  // tile 0 (the empty tile if this workgroup has none)
    const int h = gkv * p.G, q0 = niter > 0 ? (SPARSE ? uni(tl[0]) : first) * DKV_BQ : empty_q0;
#pragma unroll
    for (int piece = 0; piece < 2 * NL; ++piece) load_piece(piece, 0, tile_soff(h, q0));
    stat_load(h * p.N + q0, q0);
    wait_global_loads();
    stat_store(0);
  }
  __syncthreads();

  // S, dP of the two halves of a tile: lane (g, key n), register r <-> query
  // 32 half + sigma_row(g, r). s1 / dp1 stay live into the next iteration.
  f32x16 s0, dp0, s1 = f32x16{}, dp1 = f32x16{};
  bf16x8 pa[4], da[4];               // P, dS of the 16-query blocks t = 0..3
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    pa[t] = bf16x8{};
    da[t] = bf16x8{};
  }
  // LSE (log2 units) of the 8 query rows of the group being softmaxed,
  // double-buffered: slot (phase & 1) is consumed, the other one prefetched
  f32x4 st_l[2][2];
  const uint32_t stat_lane = lds_q0 + STAT_BYTES + 32 * g;   // buffer 0, + rows 8g..8g+7
  // stb: LDS address of this lane's rows in the stats of one buffer
  auto stat_read = [&](int slot, uint32_t stb, int qb, int g2) {
    const int off = (qb * 32 + g2 * 16) * 4;
    st_l[slot][0] = lds_read_f32x4_at(stb + off);
    st_l[slot][1] = lds_read_f32x4_at(stb + off + 16);
  };
  // -D of the 16 query rows of half qb that this lane's dP registers hold:
  // the dP products accumulate onto it, so they produce dP - D directly
  auto dinit_read = [&](uint32_t stb, int qb) {
    f32x16 x;
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const f32x4 y = lds_read_f32x4_at(stb + DKV_BQ * 4 + (qb * 32 + g2 * 16) * 4 + 16 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[8 * g2 + 4 * hf + e] = y[e];
      }
    return x;
  };
  stat_read(0, stat_lane + 2 * BUF_BYTES, 1, 1);   // tile -1, half 1, group 1

  // softmax sub-step k (0..3) of group g2 of half qb: P and dS of elements
  // e = 2k, 2k+1 of the group (register r = 8 g2 + e), stats from `slot`
  auto softmax_sub = [&](auto qbc, auto g2c, auto kc, auto slotc) {
    constexpr int qb = decltype(qbc)::value, g2 = decltype(g2c)::value;
    constexpr int k = decltype(kc)::value, slot = decltype(slotc)::value;
    const f32x16& sv = qb ? s1 : s0;
    const f32x16& dv_ = qb ? dp1 : dp0;    // dP - D
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = 2 * k + u, r = g2 * 8 + e;
      const float x = __builtin_amdgcn_exp2f(fmaf(sv[r], c, -st_l[slot][e >> 2][e & 3]));
      pa[qb * 2 + g2][e] = (bf16)x;
      da[qb * 2 + g2][e] = (bf16)(x * dv_[r]);
    }
  };
  // causal mask on the scores of one half of a diagonal tile: query
  // 32 qb + sigma_row(g, r) before this lane's key -> -inf (P = 0); under a
  // sliding window also the queries at or past this key + window
  auto mask_half = [&](f32x16& sv, int mthr_h) {
    const int tq = mthr_h - 8 * g;    // register r masked iff r' < tq, r' = r (r < 8) or r + 8
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = r < 8 ? r : r + 8;
      if (rr < tq || (WIN && rr >= tq + p.window)) sv[r] = -INFINITY;
    }
  };

  int h_cur = gkv * p.G, t_cur = 0;   // (query head, tile index within the head) of tile k
  int q0_cur = niter > 0 ? (SPARSE ? uni(tl[0]) : first) * DKV_BQ : empty_q0;   // first row of tile k
  // tile k's Q / dO offset for load_piece() and LSE / D index for
  // stat_load(), advanced by a tile, or to the next head's first tile
  uint32_t so_cur = tile_soff(h_cur, q0_cur);
  int si_cur = h_cur * p.N + q0_cur;
  const uint32_t so_step = (uint32_t)(DKV_BQ * qrs) * 2u;
  const uint32_t so_wrap = (uint32_t)D * 2u - (uint32_t)(per_head - 1) * so_step;   // modulo 2^32
  const int si_wrap = p.N - (per_head - 1) * DKV_BQ;
  // Tile k: one iteration of the pipeline. MASKED iterations apply the
  // causal (and window) mask to the tile's scores; the driver below gives
  // each its own loop, so that tiles clear of the diagonal carry no mask
  // code at all (a mask test inside one loop body is turned into
  // per-element selects that every tile pays for).
  int kt_ = 0;
  uint32_t cbo = 0;   // byte offset of tile k's LDS buffer (k % 3) from buffer 0
  auto iteration = [&](auto mc) {
    constexpr bool MASKED = decltype(mc)::value;
      // buffers of tiles k - 1 and k + 1
      const uint32_t pbo = cbo == 0 ? 2 * BUF_BYTES : cbo - BUF_BYTES;
      const uint32_t nbo = cbo == 2 * BUF_BYTES ? 0 : cbo + BUF_BYTES;
      const int q0 = q0_cur;           // tile k < niter: the loops below run real tiles only
      // The tile after this one. After the last tile nothing reads it: its
      // loads then start at the end of both descriptors' ranges, so they
      // return zeros without touching memory.
      const bool wrap = t_cur + 1 == per_head;
      const int h_nx = wrap ? h_cur + 1 : h_cur, t_nx = wrap ? 0 : t_cur + 1;
      int q0_nx, si_nx;
      uint32_t so_nx;
      if constexpr (SPARSE) {            // list entry of tile k + 3, read now for the next iteration
        q0_nx = tq_nx * DKV_BQ;
        if (++t_nx2 == per_head) t_nx2 = 0;
        const int after = kt_ + 3 < niter ? uni(tl[t_nx2]) : 0;
        tq_nx = tq_nx2;
        tq_nx2 = after;
        so_nx = tile_soff(h_nx, q0_nx);
        si_nx = h_nx * p.N + q0_nx;
      } else {                           // one tile on, or the next head's first
        q0_nx = wrap ? first * DKV_BQ : q0_cur + DKV_BQ;
        so_nx = so_cur + (wrap ? so_wrap : so_step);
        si_nx = si_cur + (wrap ? si_wrap : DKV_BQ);
      }
      const bool nx_real = kt_ + 1 < niter;
      const uint32_t so_ld = nx_real ? so_nx : qbytes;
      const int si_ld = nx_real ? si_nx : st_end;
      const int mthr = kpos - (p.q_start + q0);     // query index inside the tile < mthr -> masked
      // LDS read bases of this iteration (byte addresses; dO at +TILE from Q)
      const uint32_t cq = lds_q0 + cbo;
      const uint32_t pq = lds_q0 + pbo;
      const uint32_t bs[2] = {lds_opaque(cq + 2 * rd_s[0]), lds_opaque(cq + 2 * rd_s[1])};
      const uint32_t bt[2] = {lds_opaque(cq + 2 * rd_t[0]), lds_opaque(cq + 2 * rd_t[1])};
      const uint32_t btp[2] = {lds_opaque(pq + 2 * rd_t[0]), lds_opaque(pq + 2 * rd_t[1])};
      const uint32_t stb = lds_opaque(stat_lane + cbo);
      // -D of half 0 now; that of half 1 two steps before its first product
      const f32x16 di0 = dinit_read(stb, 0);
      f32x16 di1;

      lockstep_products<4 * PL, 4>(
          [&](auto ic) {
            constexpr int i = decltype(ic)::value, ph = i / PL, j = i % PL;
            if constexpr (ph == 0 || ph == 2) {   // S / dP of half ph/2: step j = (ks, which)
              constexpr int ks = j >> 1;
              return lds_read16_at(bs[ks & 1] + 2 * ((j & 1) * TILE + (ph / 2) * 32 * ROW + (ks >> 1) * 32));
            } else {                              // dV / dK: step j = (t, db, which), two transposing reads
              constexpr int t = (ph == 1 ? 2 : 0) + j / (2 * DB), db = (j >> 1) % DB;
              constexpr int off = ((j & 1) ? 0 : TILE) + 16 * t * ROW + 32 * db;   // Q^T for dK, dO^T for dV
              const bf16x4 r0 = lds_read_tr4_at((ph == 1 ? btp[0] : bt[0]) + 2 * off);
              const bf16x4 r1 = lds_read_tr4_at((ph == 1 ? btp[1] : bt[1]) + 2 * off);
              return bf16x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
            }
          },
          [&](auto ic, bf16x8 a) {
            constexpr int i = decltype(ic)::value, ph = i / PL, j = i % PL;
            if constexpr (ph == 0 || ph == 2) {
              constexpr int ks = j >> 1;
              f32x16& acc = (j & 1) ? (ph == 0 ? dp0 : dp1) : (ph == 0 ? s0 : s1);
              const bf16x8& bop = (j & 1) ? vf[ks] : kf[ks];
              const f32x16 init = (j & 1) ? (ph == 0 ? di0 : di1) : f32x16{};
              acc = mfma32(a, bop, ks == 0 ? init : acc);
            } else {
              constexpr int t = (ph == 1 ? 2 : 0) + j / (2 * DB), db = (j >> 1) % DB;
              if constexpr (j & 1) mfma32_agpr(dk[db], a, da[t]);
              else mfma32_agpr(dv[db], a, pa[t]);
            }
          },
          [&](auto ic) {
            constexpr int i = decltype(ic)::value, ph = i / PL, j = i % PL;
            // stats for the next phase's group, into slot (ph + 1) & 1
            if constexpr (j == 0) {
              if constexpr (ph == 0) stat_read(1, stb, 0, 0);
              else if constexpr (ph == 1) stat_read(0, stb, 0, 1);
              else if constexpr (ph == 2) stat_read(1, stb, 1, 0);
              else stat_read(0, stb, 1, 1);
            }
            // softmax sub-steps at steps (2k + 1) PL / 8
            if constexpr ((j * 8) % PL == 0 && ((j * 8) / PL) % 2 == 1) {
              constexpr int k = ((j * 8) / PL) / 2;
              using KC = std::integral_constant<int, k>;
              using SL = std::integral_constant<int, ph & 1>;
              using I0 = std::integral_constant<int, 0>;
              using I1 = std::integral_constant<int, 1>;
              if constexpr (ph == 0) softmax_sub(I1{}, I1{}, KC{}, SL{});
              else if constexpr (ph == 1) softmax_sub(I0{}, I0{}, KC{}, SL{});
              else if constexpr (ph == 2) softmax_sub(I0{}, I1{}, KC{}, SL{});
              else softmax_sub(I1{}, I0{}, KC{}, SL{});
            }
            if constexpr (ph == 0) {            // next tile: direct loads, then its LSE / D
              constexpr int lo = j * (2 * NL) / PL, hi = (j + 1) * (2 * NL) / PL;
              [&]<int... Ws>(std::integer_sequence<int, Ws...>) {
                (load_piece(lo + Ws, nbo, so_ld), ...);
              }(std::make_integer_sequence<int, hi - lo>{});
              if constexpr (j == PL - 1) stat_load(si_ld, q0_nx);
            }
            if constexpr (ph == 1 && j == PL - 2) di1 = dinit_read(stb, 1);
            if constexpr (ph == 3 && j == PL - 1) stat_store(nbo);
            // diagonal tiles: mask each half's scores once its products are done
            if constexpr ((ph == 0 || ph == 2) && j == PL - 1) {
              if constexpr (MASKED) mask_half(ph == 0 ? s0 : s1, mthr - (ph / 2) * 32);
            }
          },
          std::true_type{});
      wait_global_loads();
      __syncthreads();
    h_cur = h_nx;
    t_cur = t_nx;
    q0_cur = q0_nx;
    so_cur = so_nx;
    si_cur = si_nx;
    ++kt_;
    cbo = nbo;
  };
  // The masked tiles of a head: a prefix whose rows start before this
  // wave's last key (the diagonal) and, under a sliding window, a suffix
  // whose last row reaches past this wave's first key's window. Rows rise
  // with the tile index, so both are contiguous. (Per wave: every wave runs
  // the same number of iterations and barriers.)
  auto tile_row = [&](int t) { return (SPARSE ? uni(tl[t]) : first + t) * DKV_BQ; };
  int npre = 0, nsuf = 0;
  if constexpr (CAUSAL) {
    while (npre < per_head && wk_first + DKV_KW - 1 > p.q_start + tile_row(npre)) ++npre;
    if constexpr (WIN) {
      while (nsuf < per_head - npre &&
             p.q_start + tile_row(per_head - 1 - nsuf) + DKV_BQ - 1 - wk_first >= p.window)
        ++nsuf;
    }
  }
  for (int hh = 0; hh < p.G && per_head > 0; ++hh) {
    const int base = hh * per_head;
    if constexpr (CAUSAL)
      while (kt_ < base + npre) iteration(std::true_type{});
    while (kt_ < base + per_head - nsuf) iteration(std::false_type{});
    if constexpr (WIN)
      while (kt_ < base + per_head) iteration(std::true_type{});
  }
  // Drain: the last tile's dV^T, dK^T over its half 1 (what an iteration's
  // phase 1 would do), with the softmax of that half's group 1 first (what
  // its phase 0 would do); the last tile sits in the buffer before tile k's. With no
  // tile at all that is the zero buffer of tile -1, with P = dS = 0.
  {
    const uint32_t lq = lds_q0 + (cbo == 0 ? 2 * BUF_BYTES : cbo - BUF_BYTES);
    const uint32_t btl[2] = {lds_opaque(lq + 2 * rd_t[0]), lds_opaque(lq + 2 * rd_t[1])};
    lockstep_products<PL, 4>(
        [&](auto ic) {   // step j = (t, db, which), two transposing reads
          constexpr int j = decltype(ic)::value;
          constexpr int t = 2 + j / (2 * DB), db = (j >> 1) % DB;
          constexpr int off = ((j & 1) ? 0 : TILE) + 16 * t * ROW + 32 * db;   // Q^T for dK, dO^T for dV
          const bf16x4 r0 = lds_read_tr4_at(btl[0] + 2 * off);
          const bf16x4 r1 = lds_read_tr4_at(btl[1] + 2 * off);
          return bf16x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
        },
        [&](auto ic, bf16x8 a) {
          constexpr int j = decltype(ic)::value;
          constexpr int t = 2 + j / (2 * DB), db = (j >> 1) % DB;
          if constexpr (j & 1) mfma32_agpr(dk[db], a, da[t]);
          else mfma32_agpr(dv[db], a, pa[t]);
        },
        [&](auto ic) {   // the group's four softmax sub-steps, before its products (step 2 DB on)
          constexpr int j = decltype(ic)::value;
          static_assert(2 * DB >= 4, "sub-steps before the group's first product");
          if constexpr (j < 4)
            softmax_sub(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{},
                        std::integral_constant<int, j>{}, std::integral_constant<int, 0>{});
        },
        std::true_type{});
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
        f32x4 xa, xv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xa[e] = dk[db][run * 4 + e] * p.scale;
          xv[e] = dv[db][run * 4 + e];
        }
        if (p.acc_kv == ACC_ADD || p.acc_kv == ACC_LAST) {   // plus the float32 sums so far
          const float* sk = p.acc_kv == ACC_ADD ? (const float*)p.dk : p.k_part;
          const float* sv = p.acc_kv == ACC_ADD ? (const float*)p.dv : p.v_part;
          xa += *(const f32x4*)(sk + off + col);
          xv += *(const f32x4*)(sv + off + col);
        }
        if (p.acc_kv == ACC_ADD || p.acc_kv == ACC_FIRST) {
          *(f32x4*)((float*)p.dk + off + col) = xa;
          *(f32x4*)((float*)p.dv + off + col) = xv;
        } else {
          bf16x4 ya, yv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ya[e] = (bf16)xa[e];
            yv[e] = (bf16)xv[e];
          }
          *(bf16x4*)((bf16*)p.dk + off + col) = ya;
          *(bf16x4*)((bf16*)p.dv + off + col) = yv;
        }
      }
    }
  }
}

// ============================================================ dQ

constexpr int DQ_BC = 64;   // keys per tile

// K and V tiles (64 keys), row-major; rows padded to D + 32 (d = 128) or
// D + 16 (d = 64) elements, the 16-byte chunk index XORed by swz_dq<D>(row)
// (below). Both tiles are written by direct global -> LDS loads.
template <int D>
struct DqSmem {
  static constexpr int ROW = D == 64 ? D + 16 : D + 32;
  static constexpr int TILE = DQ_BC * ROW;
  bf16 k[2][TILE];
  bf16 v[2][TILE];
};

// Stride-4 key order of the dQ kernel's tiles: A-operand row i = 4q + r of
// 16-key block mb is tile row q + 4 r + 16 (mb % 2) (+ 32 per 32-key chunk),
// so the accumulators of blocks 2c and 2c + 1 give lane group q the keys
// 32 c + q + 4 e, e = 0..7, in register order; the K^T operand of the dQ
// product is read with the same key order.
//
// LDS has 64 banks of 4 bytes. An 8-byte read (plain or transposing) is
// served 32 lanes at a time (lanes 0-31, then 32-63); a 16-byte read 16
// lanes at a time: within each half-wave, the lane quads (lane / 4) % 8
// whose three index bits have even parity, then those with odd parity
// (measured on the device with SQ_LDS_BANK_CONFLICT, two lanes on one bank
// at a time). The row reads of S^T = K Q^T and dP^T = V dO^T touch rows
// 0..15 (+16 k) with one logical chunk; a transposing read of K^T touches,
// per 32 lanes, rows q + 4 m (q = two neighbours, m = 0..3) with one 32-byte
// chunk pair each. With the row strides above, rows 4 apart start on the
// same bank, so the swizzle has to spread those rows over different chunk
// pairs while keeping the rows of each 16-byte phase on different chunk
// columns. It depends on bits 2 and 3 of the row only (so every row a lane
// reads shares it) and sets at most one chunk-index bit above bit 1: the top
// bit of the row's chunks (bit 3 for d = 128, bit 2 for d = 64). Both read
// patterns are then free of bank conflicts (exhaustive check of all
// swizzles linear in the row's low bits against the rules above).
template <int D>
__device__ __forceinline__ int swz_dq(int row) {
  if constexpr (D == 128) return (((row >> 2) & 1) * 2) ^ (((row >> 3) & 1) * 8);
  else return ((row >> 3) & 1) * 4;
}

template <int D, bool CAUSAL, int NW, bool WIN = false, bool SPARSE = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(Params p) {
  constexpr int BR = NW * 32;
  constexpr int KS = D / 32;          // 32-wide k-steps of S^T = K Q^T and dP^T = V dO^T
  constexpr int DM = D / 16;          // 16-row blocks of dQ^T
  constexpr int ROW = DqSmem<D>::ROW, TILE = DqSmem<D>::TILE;
  constexpr int TILES_KB = 2 * TILE * 2 / 1024;     // K and V, in 1 KB direct loads
  static_assert(TILE * 2 % 1024 == 0, "whole 1 KB pieces");
  constexpr int NL = (TILES_KB + NW - 1) / NW;     // per wave (the last waves may have fewer)
  constexpr int TILE_KB = TILES_KB / 2;
  __shared__ __attribute__((aligned(16))) DqSmem<D> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int q4 = lane >> 4, i16 = lane & 15;
  const int tix = tile_grid_index<CAUSAL>(), ntq = tile_grid_count<CAUSAL>();
  int qt = CAUSAL ? (ntq - 1 - tix) : tix;
  const int h = xcd_head(blockIdx.x, p.H);
  int b = batch_grid_index<CAUSAL>();
  if (p.vl_qtiles) {                   // packed batch: (sequence, tile) from the work list
    if (tix >= p.vl_qtiles[0]) return;
    b = p.vl_qtiles[2 + 2 * tix];
    qt = p.vl_qtiles[3 + 2 * tix];
  }
  const int kvh = h / p.G;
  const int q0 = qt * BR;
  if (p.cu_seqlens) {                  // packed batch: b is the sequence (from the work list)
    if (!narrow_to_sequence(p, b, q0)) return;
    b = 0;
  }
  const int wq0 = q0 + wave * 32;

  const long long qrs = (long long)p.H * D, krs = (long long)p.Hkv * D;
  const bf16* Q = (const bf16*)p.q + ((long long)b * p.N + p.q_start) * qrs + (long long)h * D;
  const bf16* dO = (const bf16*)p.dout + ((long long)b * p.N + p.q_start) * qrs + (long long)h * D;
  const bf16* K = (const bf16*)p.k + ((long long)b * p.N + p.k_start) * krs + (long long)kvh * D;
  const bf16* V = (const bf16*)p.v + ((long long)b * p.N + p.k_start) * krs + (long long)kvh * D;

  float c = fabsf(p.scale) * kLog2e;
  float qsign = p.scale < 0.f ? -1.f : 1.f;
  if (p.scale == 0.f) { c = 1.f; qsign = 0.f; }

  // Q and dO as B operands of S^T = K Q^T and dP^T = V dO^T: lane (q4, i16)
  // holds row wq0 + 16 nb + i16 (query block nb), columns 32 ks + 8 q4 ..
  bf16x8 qf[2][KS], of[2][KS];
  float lse2[2], dsum[2];
  int qpos[2];
  long long si[2];
  // With p.fuse_dsum the kernel forms D = rowsum(dO * O) of its rows itself
  // (FlashAttention-2 reviews page, reviewer 2 point 2: the backward needs
  // only the saved O and logsumexp): each lane sums its 8 KS products of the
  // row, and the four lane groups q4 that share the row add their sums.
  // Every query row belongs to exactly one workgroup of this kernel, which
  // writes its D for the dK/dV kernel that runs after it.
  const bool fuse = p.fuse_dsum != 0;
  const bf16* Ob = (const bf16*)p.o + ((long long)b * p.N + p.q_start) * qrs + (long long)h * D;
  bf16x8 ov[2][KS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int r_ = wq0 + 16 * nb + i16;
    const int rc = min(r_, p.Nq - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 x = *(const bf16x8*)(Q + rc * qrs + ks * 32 + q4 * 8);
      if (qsign != 1.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (bf16)((float)x[e] * qsign);
      }
      qf[nb][ks] = x;
      of[nb][ks] = *(const bf16x8*)(dO + rc * qrs + ks * 32 + q4 * 8);
      if (fuse) ov[nb][ks] = *(const bf16x8*)(Ob + rc * qrs + ks * 32 + q4 * 8);
    }
    si[nb] = ((long long)b * p.H + h) * p.N + p.q_start + rc;
    lse2[nb] = p.lse[si[nb]] * kLog2e;
    if (!fuse) dsum[nb] = p.dsum[si[nb]];
    qpos[nb] = p.q_start + r_;
  }
  wait_global_loads();
  if (fuse) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float x = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) x = fmaf((float)of[nb][ks][e], (float)ov[nb][ks][e], x);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      dsum[nb] = x;
      if (q4 == 0 && wq0 + 16 * nb + i16 < p.Nq) p.dsum[si[nb]] = x;
    }
  }

  int nkt = (p.Nk + DQ_BC - 1) / DQ_BC;
  if (CAUSAL) {
    const int last_q = p.q_start + min(q0 + BR - 1, p.Nq - 1);
    const int kend = min(p.Nk, last_q - p.k_start + 1);
    nkt = kend > 0 ? (kend + DQ_BC - 1) / DQ_BC : 0;
  }
  const int wq_first = p.q_start + wq0;

  // Direct loads: 1 KB piece s = wave*NL + i of the two tiles (K: s < TILE_KB,
  // then V; pieces s >= TILES_KB do not exist) covers tile bytes
  // [(s % TILE_KB) KB, +1 KB); lane l fills 16 bytes at 16 l: tile row r,
  // physical chunk pch holding logical chunk pch ^ swz_dq(r) (padding chunks
  // from chunk 0), read from byte loff[i] = 2 (r * row stride + 8 * logical
  // chunk) past the tile's first key.
  uint32_t loff[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int off = ((wave * NL + i) % TILE_KB) * 1024 + 16 * lane;
    const int r_ = off / (ROW * 2), pch = (off % (ROW * 2)) / 16;
    const int col = pch < D / 8 ? ((pch ^ swz_dq<D>(r_)) << 3) : 0;
    loff[i] = (uint32_t)(r_ * krs + col) * 2u;
  }
  // keys past the last one read as zeros (buffer range check); the mask drops them
  const uint32_t kbytes = (uint32_t)(((p.Nk - 1) * krs + D) * 2);
  const u32x4 rk = rsrc_words(K, kbytes), rv = rsrc_words(V, kbytes);
  auto load_piece = [&](int i, int buf, int j0) {
    const int sl = wave * NL + i;                  // wave-uniform
    if (TILES_KB % NW != 0 && sl >= TILES_KB) return;
    const bool is_v = sl >= TILE_KB;
    buffer_load_lds16_async(is_v ? rv : rk, loff[i], (uint32_t)(j0 * krs) * 2u, (uint32_t)buf * (2u * TILE),
                            lds_addr((is_v ? sm.v[0] : sm.k[0]) + (sl % TILE_KB) * 512));
  };

  // per-lane LDS read offsets (elements). Every row a lane reads has the
  // same bits 2 and 3, hence one swizzle per lane: its bits 0-1 (slo) move
  // the chunk within its group of 4, its higher part (if any) flips the top
  // bit of the group index (the group index ^ (half its range)).
  // K / V fragment (key block mb, k-step ks): row i16 / 4 + 4 (i16 % 4) +
  // 16 (mb % 2) + 32 (mb / 2), logical chunk 4 ks + q4 -> physical
  // 4 (ks ^ flip) + (q4 ^ slo): base rd_k[0] for the first KS / 2 k-steps,
  // rd_k[1] for the rest. K^T fragment (d block md, key chunk kc), read rd:
  // lane j of 16-lane group q4 addresses key row 32 kc + q4 + 16 rd + 4 (j/4),
  // logical columns 16 md + 4 (j%4); element 4 rd + t of the result is key
  // 32 kc + q4 + 4 (4 rd + t), the order of dS^T. Its chunk 2 md + (j%4)/2 =
  // 4 (md / 2) + (2 (md % 2) + (j%4)/2) -> base rd_t[md % 2][(md / 2) / (DM / 4)].
  const int krow0 = (i16 >> 2) + 4 * (i16 & 3);
  int rd_k[2];
  {
    const int sk = swz_dq<D>(krow0), slo = sk & 3, flip = sk >> 2 ? KS / 2 : 0;
    const int base = krow0 * ROW + 8 * (q4 ^ slo);
    rd_k[0] = base + 32 * flip;
    rd_k[1] = base + 32 * (KS / 2 - flip);
  }
  int rd_t[2][2];
  {
    const int r_ = q4 + 4 * (i16 >> 2);
    const int st = swz_dq<D>(r_), slo = st & 3, flip = st >> 2 ? DM / 4 : 0;
#pragma unroll
    for (int mp = 0; mp < 2; ++mp) {
      const int base = r_ * ROW + 8 * ((2 * mp + ((i16 & 3) >> 1)) ^ slo) + 4 * (i16 & 1);
      rd_t[mp][0] = base + 32 * flip;
      rd_t[mp][1] = base + 32 * (DM / 4 - flip);
    }
  }

  f32x4 acc[DM][2];   // dQ^T: [16-row d block][query block]
#pragma unroll
  for (int md = 0; md < DM; ++md) acc[md][0] = acc[md][1] = f32x4{};

  // sliding window (causal): key tiles wholly before the window of the
  // workgroup's first row are skipped too
  int jt0 = 0;
  if constexpr (WIN) jt0 = max(0, p.q_start + q0 - (p.window - 1) - p.k_start) / DQ_BC;
  // block-sparse: the ascending key-tile list of the workgroup's block row
  // (cut at the diagonal and the last key); its first `npl` entries need no mask
  const int* tl = nullptr;
  int nit = 0, npl = 0;
  if constexpr (SPARSE) {
    static_assert(BR == BS_ROWS && DQ_BC == BS_TILE, "a workgroup covers one block row of the mask");
    tl = p.bs_row_tiles + (long long)qt * p.bs_ld;
    nit = p.bs_row_cnt[qt];
    npl = min(p.bs_row_plain[qt], nit);
    if (nit > 0) {
#pragma unroll
      for (int i = 0; i < NL; ++i) load_piece(i, 0, uni(tl[0]) * DQ_BC);
      wait_global_loads();
    }
  } else if (nkt > jt0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) load_piece(i, jt0 & 1, jt0 * DQ_BC);
    wait_global_loads();
  }
  __syncthreads();

  // Lock steps per key tile (PS = 2 KS steps per 32-key chunk, PD = DM per chunk;
  // every step is one K/V or K^T fragment and its two products, one per query block):
  //   phase 0 (PS steps): S^T, dP^T of keys 0-31    + direct loads of the next tile
  //   phase 1 (PS steps): S^T, dP^T of keys 32-63   + dS of keys 0-31
  //   phase 2 (PD steps): dQ^T over keys 0-31       + dS of keys 32-63
  //   phase 3 (PD steps): dQ^T over keys 32-63
  // Key tiles before nplain lie entirely below the causal diagonal of every
  // row of the workgroup and before the ragged end: they run a body without
  // the mask test; the rest run the masked body.
  constexpr int PS = 2 * KS * 2, PD = DM;   // (2 key blocks of 16) x KS x (S, dP)
  int nplain = min(nkt, p.Nk / DQ_BC);
  if (CAUSAL) nplain = min(nplain, max(0, p.q_start + q0 - p.k_start + 1) / DQ_BC);
  // key tile j from LDS buffer buf, while tile jnext is loaded into the other one
  auto tile = [&](auto mc, int j, int buf, int jnext) {
    constexpr bool MASKED = decltype(mc)::value;
    const int kpos0 = p.k_start + j * DQ_BC;
    const int jn = jnext * DQ_BC;
    // masked iff key index inside the tile > thr (causal and the ragged end),
    // or < lo under a sliding window (before the row's window)
    int thr[2], lo[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      thr[nb] = p.Nk - 1 - j * DQ_BC;
      if (CAUSAL && kpos0 + DQ_BC - 1 > wq_first) thr[nb] = min(thr[nb], qpos[nb] - kpos0);
      lo[nb] = 0;
      if constexpr (WIN) lo[nb] = qpos[nb] - (p.window - 1) - kpos0;
    }
    const bf16* kt = sm.k[buf];
    const bf16* vt = sm.v[buf];
    // [key block mb][query block nb]; the dP^T products accumulate onto -D
    // of their query (every register of a lane holds the same query), so
    // they leave dP - D
    f32x4 s[4][2], dp[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      s[mb][0] = s[mb][1] = f32x4{};
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) dp[mb][nb] = f32x4{-dsum[nb], -dsum[nb], -dsum[nb], -dsum[nb]};
    }
    bf16x8 dsb[2][2];          // dS^T as the B operand: [key chunk kc][query block nb]

    // dS for key chunk kc, slice w of 8 (query block w / 4, register pair
    // 2 (w % 4)): register r of key block mb holds key 32 (mb/2) + q4 +
    // 4 (4 (mb%2) + r), i.e. element e = 4 (mb%2) + r of the chunk's B operand
    auto ds_sub = [&](auto kcc, auto wc) {
      constexpr int kc = decltype(kcc)::value, w = decltype(wc)::value;
      constexpr int nb = w / 4, e0 = 2 * (w % 4);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = e0 + u, mb = 2 * kc + (e >> 2), r = e & 3;
        const float x = __builtin_amdgcn_exp2f(fmaf(s[mb][nb][r], c, -lse2[nb]));
        float pv = x;
        if constexpr (MASKED) {
          const int kin = 32 * kc + q4 + 4 * e;
          pv = (kin > thr[nb] || (WIN && kin < lo[nb])) ? 0.f : x;
        }
        dsb[kc][nb][e] = (bf16)(pv * dp[mb][nb][r]);
      }
    };

    lockstep_products<2 * PS + 2 * PD, 4>(
        [&](auto ic) {
          constexpr int i = decltype(ic)::value;
          if constexpr (i < 2 * PS) {            // S^T / dP^T: (mb, ks, which)
            constexpr int mb = i / (2 * KS), jj = i % (2 * KS), ks = jj >> 1;
            constexpr int moff = (32 * (mb >> 1) + 16 * (mb & 1)) * ROW + 32 * (ks % (KS / 2));
            return lds_read16((jj & 1) ? vt : kt, rd_k[ks / (KS / 2)] + moff);
          } else {                                // dQ^T: (kc, md)
            constexpr int ii = i - 2 * PS, kc = ii / DM, md = ii % DM;
            constexpr int hh = (md >> 1) / (DM / 4);
            constexpr int off = 32 * kc * ROW + 32 * ((md >> 1) % (DM / 4));
            const bf16x4 r0 = lds_read_tr4(kt + rd_t[md & 1][hh] + off);
            const bf16x4 r1 = lds_read_tr4(kt + rd_t[md & 1][hh] + off + 16 * ROW);
            return bf16x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
          }
        },
        [&](auto ic, bf16x8 a) {
          constexpr int i = decltype(ic)::value;
          if constexpr (i < 2 * PS) {
            constexpr int mb = i / (2 * KS), jj = i % (2 * KS), ks = jj >> 1;
            if constexpr (jj & 1) {
              dp[mb][0] = mfma16(a, of[0][ks], dp[mb][0]);
              dp[mb][1] = mfma16(a, of[1][ks], dp[mb][1]);
            } else {
              s[mb][0] = mfma16(a, qf[0][ks], s[mb][0]);
              s[mb][1] = mfma16(a, qf[1][ks], s[mb][1]);
            }
          } else {
            constexpr int ii = i - 2 * PS, kc = ii / DM, md = ii % DM;
            acc[md][0] = mfma16(a, dsb[kc][0], acc[md][0]);
            acc[md][1] = mfma16(a, dsb[kc][1], acc[md][1]);
          }
        },
        [&](auto ic) {
          constexpr int i = decltype(ic)::value;
          constexpr int NSTEP = 2 * PS + 2 * PD;
          progress_priority<i, NSTEP / 2, 3 * NSTEP / 4, 7 * NSTEP / 8>();
          if constexpr (i < PS) {                 // phase 0: next tile's direct loads
            constexpr int lo_ = i * NL / PS, hi_ = (i + 1) * NL / PS;
            [&]<int... Ws>(std::integer_sequence<int, Ws...>) {
              (load_piece(lo_ + Ws, buf ^ 1, jn), ...);
            }(std::make_integer_sequence<int, hi_ - lo_>{});
          } else if constexpr (i < 2 * PS) {      // phase 1: dS of key chunk 0
            constexpr int ii = i - PS, lo_ = ii * 8 / PS, hi_ = (ii + 1) * 8 / PS;
            [&]<int... Ws>(std::integer_sequence<int, Ws...>) {
              (ds_sub(std::integral_constant<int, 0>{}, std::integral_constant<int, lo_ + Ws>{}), ...);
            }(std::make_integer_sequence<int, hi_ - lo_>{});
          } else if constexpr (i < 2 * PS + PD) { // phase 2: dS of key chunk 1
            constexpr int ii = i - 2 * PS, lo_ = ii * 8 / PD, hi_ = (ii + 1) * 8 / PD;
            [&]<int... Ws>(std::integer_sequence<int, Ws...>) {
              (ds_sub(std::integral_constant<int, 1>{}, std::integral_constant<int, lo_ + Ws>{}), ...);
            }(std::make_integer_sequence<int, hi_ - lo_>{});
          }
        },
        std::true_type{});
    wait_global_loads();
    __syncthreads();
  };
  auto next = [&](int j) { return min(j + 1, nkt - 1); };   // the last tile repeats itself
  if constexpr (SPARSE) {
    // list entries: plain [0, npl), masked [npl, nit); the entry after the
    // next is read an iteration ahead
    int jc = nit > 0 ? uni(tl[0]) : 0, jx = nit > 1 ? uni(tl[1]) : jc;
    int it = 0;
    for (; it < npl; ++it) {
      const int jxx = it + 2 < nit ? uni(tl[it + 2]) : jx;
      tile(std::false_type{}, jc, it & 1, jx);
      jc = jx;
      jx = jxx;
    }
    for (; it < nit; ++it) {
      const int jxx = it + 2 < nit ? uni(tl[it + 2]) : jx;
      tile(std::true_type{}, jc, it & 1, jx);
      jc = jx;
      jx = jxx;
    }
  } else if constexpr (WIN) {
    // tiles before jlow hold keys before the window of some row of the
    // workgroup: masked prefix [jt0, a), plain [a, b), masked [b, nkt)
    const int jlow = max(0, (p.q_start + q0 + BR - p.window - p.k_start + DQ_BC - 1) / DQ_BC);
    const int a = min(max(jlow, jt0), nkt);
    const int b_ = max(a, min(nplain, nkt));
    for (int j = jt0; j < a; ++j) tile(std::true_type{}, j, j & 1, next(j));
    for (int j = a; j < b_; ++j) tile(std::false_type{}, j, j & 1, next(j));
    for (int j = b_; j < nkt; ++j) tile(std::true_type{}, j, j & 1, next(j));
  } else {
    for (int j = 0; j < nplain; ++j) tile(std::false_type{}, j, j & 1, next(j));
    for (int j = nplain; j < nkt; ++j) tile(std::true_type{}, j, j & 1, next(j));
  }

  // ---- store dQ = scale * acc^T: lane (q4, i16), register r of block (md, nb)
  // <-> row wq0 + 16 nb + i16, column 16 md + 4 q4 + r
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int r_ = wq0 + 16 * nb + i16;
    if (r_ >= p.Nq) continue;
    const long long off = (((long long)b * p.N + p.q_start + r_) * p.H + h) * D;
#pragma unroll
    for (int md = 0; md < DM; ++md) {
      const int col = 16 * md + 4 * q4;
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = acc[md][nb][e] * p.scale;
      if (p.acc_q == ACC_ADD || p.acc_q == ACC_LAST)    // plus the float32 sum so far
        x += *(const f32x4*)((p.acc_q == ACC_ADD ? (const float*)p.dq : p.q_part) + off + col);
      if (p.acc_q == ACC_ADD || p.acc_q == ACC_FIRST) {
        *(f32x4*)((float*)p.dq + off + col) = x;
      } else {
        bf16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (bf16)x[e];
        *(bf16x4*)((bf16*)p.dq + off + col) = y;
      }
    }
  }
}

template <int D>
hipError_t launch_dkdv_d(const Params& p, hipStream_t s) {
  const dim3 gkv = tile_grid(p.Hkv, p.vl_ktiles ? 1 : p.B, p.vl_ktiles ? p.vl_kcap : (p.Nk + DKV_BK - 1) / DKV_BK, p.causal);
  if (p.bs_col_tiles && p.causal)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, false, true>), gkv, dim3(DKV_NW * 64), 0, s, p);
  else if (p.bs_col_tiles)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, false, true>), gkv, dim3(DKV_NW * 64), 0, s, p);
  else if (p.causal && p.window > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, true>), gkv, dim3(DKV_NW * 64), 0, s, p);
  else if (p.causal)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), gkv, dim3(DKV_NW * 64), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), gkv, dim3(DKV_NW * 64), 0, s, p);
  return hipGetLastError();
}

template <int D, int NW = query_waves(D)>
hipError_t launch_dq_d(const Params& p, hipStream_t s) {
  if (p.bs_row_tiles) {   // one 256-row block row of the mask per workgroup
    const dim3 gq = tile_grid(p.H, p.B, (p.Nq + BS_ROWS - 1) / BS_ROWS, p.causal);
    if (p.causal)
      hipLaunchKernelGGL((bwd_dq_kernel<D, true, 8, false, true>), gq, dim3(8 * 64), 0, s, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, false, 8, false, true>), gq, dim3(8 * 64), 0, s, p);
    return hipGetLastError();
  }
  const dim3 gq = tile_grid(p.H, p.vl_qtiles ? 1 : p.B, p.vl_qtiles ? p.vl_qcap : (p.Nq + NW * 32 - 1) / (NW * 32), p.causal);
  if (p.causal && p.window > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D, true, NW, true>), gq, dim3(NW * 64), 0, s, p);
  else if (p.causal)
    hipLaunchKernelGGL((bwd_dq_kernel<D, true, NW>), gq, dim3(NW * 64), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, false, NW>), gq, dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dkdv_mfma(const Params& p, hipStream_t s) {
  return p.d == 128 ? launch_dkdv_d<128>(p, s) : launch_dkdv_d<64>(p, s);
}

hipError_t launch_bwd_dq_mfma(const Params& p, hipStream_t s) {
  // four-wave workgroups at d = 128 for packed batches (kVarlenQueryWaves) and small grids
  if (p.d == 128 && !p.bs_row_tiles && (p.vl_qtiles || small_query_grid(128, p.B, p.H, p.Nq, device_cu_count())))
    return launch_dq_d<128, 4>(p, s);
  return p.d == 128 ? launch_dq_d<128>(p, s) : launch_dq_d<64>(p, s);
}

hipError_t launch_bwd_mfma(const Params& p, hipStream_t s) {
  const hipError_t e = launch_bwd_dkdv_mfma(p, s);
  if (e != hipSuccess) return e;
  return launch_bwd_dq_mfma(p, s);
}

}  // namespace miattn
