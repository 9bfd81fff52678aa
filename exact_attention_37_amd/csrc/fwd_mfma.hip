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
//  * a workgroup of 8 waves (256 query rows; 4 waves and 128 rows at d = 64,
//    two workgroups per CU) owns query rows of one (b, h), two waves per
//    SIMD; each wave owns 32 rows, so its row max and row sum never leave the wave
//    (the pages' warp partitioning, with 64-lane wavefronts);
//  * K and V tiles of BC=64 keys are double-buffered in LDS, one barrier per
//    tile; the next tile is loaded straight from global memory into LDS
//    while the current tile's scores are computed;
//  * scores are computed transposed, S^T = K Q^T, with K's rows loaded in a
//    bit-permuted order (sigma32) so that each lane's 32x32 accumulator holds
//    8 consecutive keys of one query: exactly the B-operand layout of the
//    next product O^T += V^T P^T. P never moves between lanes.
//  * V^T operands of the P V product come from transposing LDS reads of the
//    row-major V tile, so V is stored once, as loaded;
//  * the running max is not rescanned per tile: P is formed with the max
//    kept so far and the tile is accepted when every lane's probability sum
//    is at most 2^8 (so p <= 2^8); only a tile that fails raises the max,
//    rescales the accumulator and forms its P again. The result is unchanged
//    (numerator and denominator share the max), and the max scan leaves the
//    loop;
//  * each of the loop's two phases of products (S^T of the next tile, P V of
//    the current one) carries half a tile of exponentials, one per product;
//  * the row sum is accumulated from the float32 probabilities before they
//    are rounded to bf16 for the P V product, so the saved logsumexp keeps
//    float32 accuracy even for rows with few keys;
//  * causal grids are ordered (head, batch, tile) so that the heaviest
//    tiles of every (batch, head) are dispatched first, and with H % 8 == 0
//    the heads are permuted so that every workgroup of one K/V head group
//    lands on the same XCD (workgroups are dealt to the 8 XCDs round-robin);
//  * at d = 128 small grids and packed batches take four-wave (128-row)
//    workgroups (small_query_grid(), kVarlenQueryWaves).
#include "common.h"
#include "kernels.h"
#include "mfma_common.h"

namespace miattn {

namespace {

constexpr int BC = 64;   // keys per tile

// K and V tiles of 64 keys, row-major; rows padded to D + 32 elements with
// the 16-byte chunk index XORed by (row / 4) % 4, so that the sigma32-ordered
// row reads of S^T = K Q^T and the 4-row transposing reads of V^T are free
// of bank conflicts. Both tiles are written by direct global -> LDS loads.
template <int D>
struct FwdSmem {
  static constexpr int ROW = D + 32;
  static constexpr int TILE = BC * ROW;
  bf16 k[2][TILE];
  bf16 v[2][TILE];
};

template <int D, int NW, bool CAUSAL, typename TO, bool WIN = false, bool SPARSE = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_mfma_kernel(Params p) {
  // rows that can still have seen no key mid-loop (sliding window,
  // block-sparse), or none at all (block-sparse)
  constexpr bool EMPTY = WIN || SPARSE;
  constexpr int BR = NW * 32;  // query rows per workgroup, 32 per wave
  constexpr int KS = D / 16;   // k-steps of the QK^T product
  constexpr int DB = D / 32;   // 32-column blocks of O
  constexpr int ROW = FwdSmem<D>::ROW, TILE = FwdSmem<D>::TILE;
  constexpr int TILES_KB = 2 * TILE * 2 / 1024;     // K and V, in 1 KB direct loads
  static_assert(TILES_KB % NW == 0, "tile loads split evenly over the waves");
  constexpr int NL = TILES_KB / NW;
  constexpr int TILE_KB = TILES_KB / 2;
  __shared__ __attribute__((aligned(16))) FwdSmem<D> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;

  // ---- workgroup -> (b, h, query tile); tile_grid_index() (mfma_common.h) picks
  // the grid dimension that holds the tile
  const int tix = tile_grid_index<CAUSAL>(), ntq = tile_grid_count<CAUSAL>();
  int qt = CAUSAL ? (ntq - 1 - tix) : tix;
  const int h = xcd_head(blockIdx.x, p.H);
  int b = batch_grid_index<CAUSAL>();
  if (p.vl_qtiles) {                              // packed batch: (sequence, tile) from the work list
    if (tix >= p.vl_qtiles[0]) return;
    b = p.vl_qtiles[2 + 2 * tix];
    qt = p.vl_qtiles[3 + 2 * tix];
  }
  const int kvh = h / p.G;
  const int q0 = qt * BR;                         // first local query row of the tile
  if (p.cu_seqlens) {                             // packed batch: b is the sequence (from the work list)
    if (!narrow_to_sequence(p, b, q0)) return;
    b = 0;
  }
  const int wq0 = q0 + wave * 32;                 // first local query row of this wave

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
  const int row = wq0 + n;
  bf16x8 qf[KS];
  {
    const int rc = min(row, p.Nq - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 x = *(const bf16x8*)(Q + rc * qrs + ks * 16 + g * 8);
      if (qsign != 1.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (bf16)((float)x[e] * qsign);
      }
      qf[ks] = x;
    }
  }
  wait_global_loads();
  const int qpos = p.q_start + row;

  // ---- key range of the workgroup
  int nkt = (p.Nk + BC - 1) / BC;
  if (CAUSAL) {
    const int last_q = p.q_start + min(q0 + BR - 1, p.Nq - 1);   // absolute position
    const int kend = min(p.Nk, last_q - p.k_start + 1);
    nkt = kend > 0 ? (kend + BC - 1) / BC : 0;
  }
  const int wq_first = p.q_start + wq0;
  // sliding window (causal): key tiles wholly before the window of the
  // workgroup's first row are skipped too
  int jt0 = 0;
  if constexpr (WIN) jt0 = max(0, p.q_start + q0 - (p.window - 1) - p.k_start) / BC;
  // the key tiles taken: jt0 .. nkt-1, or (block-sparse) the ascending list
  // of the workgroup's block row, already cut at the diagonal and the last key
  int nit = nkt - jt0;
  const int* tl = nullptr;
  if constexpr (SPARSE) {
    static_assert(BR == BS_ROWS && BC == BS_TILE, "a workgroup covers one block row of the mask");
    tl = p.bs_row_tiles + (long long)qt * p.bs_ld;
    nit = p.bs_row_cnt[qt];
  }

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
  const u32x4 rk = rsrc_words(K, kbytes), rv = rsrc_words(V, kbytes);
  // piece i of this wave: K of the tile starting at key jk0 into K buffer kb,
  // or V of the tile starting at key jv0 into V buffer vb
  auto load_piece = [&](int i, int kb, int jk0, int vb, int jv0) {
    const int sl = wave * NL + i;                  // wave-uniform
    const bool is_v = sl >= TILE_KB;
    buffer_load_lds16_async(is_v ? rv : rk, loff[i], (uint32_t)((is_v ? jv0 : jk0) * krs) * 2u,
                            lds_addr((is_v ? sm.v[vb] : sm.k[kb]) + (sl % TILE_KB) * 512));
  };

  // ---- per-lane LDS read bases (elements): K rows sigma32(n) (+32 kb), logical
  // chunk 2 ks + g -> base for ks parity e; V^T transposing reads: lane j of
  // 16-lane group (g, hf) addresses key row 16kq + 8g + 4rd + j/4, columns
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
  float m = -INFINITY, l = 0.f;

  // Tiles are taken in list order it = 0 .. nit-1 (tile_of(it): contiguous
  // from jt0, or the block-sparse list). K and V of tile it sit in K / V
  // buffer it & 1. The loop is software-pipelined across tiles, and each of
  // its two phases of matrix-core products carries half a tile of softmax:
  //   phase A: S^T of tile it+1 (K from LDS)  + P of keys 32..63 of tile it
  //            + direct loads of K(it+2) and V(it+1)
  //   phase B: O^T += V^T P^T of tile it      + P of keys 0..31 of tile it+1
  // then one wait for the loads and one barrier. K is thereby loaded two
  // tiles ahead and V one tile ahead: K(it+2) overwrites K(it), whose
  // products ran in the previous iteration, and V(it+1) overwrites V(it-1).
  // Tiles past the last repeat the last one (the extra scores are unused).
  // Block-sparse list entries are read two iterations ahead.
  //
  // The running max m is not rescanned per tile. P is formed with the max
  // kept so far, and a tile is accepted when every lane's sum of its
  // probabilities is at most 2^8, which bounds every probability by 2^8, as
  // a max raised lazily by a margin of 8 would. The scores of the first
  // tile set m. A tile that fails the test (a score more than about 8 above
  // m in log2 units; a window row that has seen no key yet) takes a slow
  // path: its max raises m, the accumulator and row sum are rescaled, and
  // its probabilities are formed again. The result is the same softmax:
  // numerator and denominator share m.
  int t1 = 0, t2 = 0, t3 = 0;     // tile_of(it + 1), tile_of(it + 2), tile_of(it + 3)
  auto list_at = [&](int it) { return SPARSE ? uni(tl[min(it, nit - 1)]) : jt0 + min(it, nit - 1); };
  int t0 = 0;
  if (nit > 0) {
    t0 = list_at(0);
    t1 = list_at(1);
    t2 = list_at(2);
    t3 = list_at(3);
  }

  // ---- S^T = K Q^T of one tile from K buffer kb into sx, lock-stepped with ex(step)
  auto scores = [&](f32x16 (&sx)[2], int kbuf, auto ex) {
    const bf16* kt = sm.k[kbuf];
    sx[0] = f32x16{};
    sx[1] = f32x16{};
    lockstep_products<2 * KS, 4>(
        [&](auto ic) {
          constexpr int i = decltype(ic)::value, kb = i % 2, ks = i / 2;
          return lds_read16(kt + rd_s[ks & 1], kb * 32 * ROW + (ks >> 1) * 32);
        },
        [&](auto ic, bf16x8 a) {
          constexpr int i = decltype(ic)::value, kb = i % 2, ks = i / 2;
          sx[kb] = mfma32(a, qf[ks], sx[kb]);
        },
        ex, std::true_type{});
  };
  // ---- mask of one tile's scores: key index inside the tile > thr (causal
  // diagonal, ragged end) or, under a sliding window, < lo (before the row's window)
  auto mask_tile = [&](f32x16 (&sx)[2], int j) {
    const int kpos0 = p.k_start + j * BC;          // absolute position of the tile's first key
    int thr = p.Nk - 1 - j * BC;
    if (CAUSAL && kpos0 + BC - 1 > wq_first) thr = min(thr, qpos - kpos0);
    int lo = 0;
    if constexpr (WIN) lo = qpos - (p.window - 1) - kpos0;
    if (__builtin_amdgcn_ballot_w64(thr < BC - 1 || (WIN && lo > 0)) != 0) {
      // key index kb * 32 + sigma_row(g, r) = 8 g + kb * 32 + r (+ 8 for r >= 8):
      // the lane's part moves into the thresholds, the rest is a constant
      const int thr_g = thr - 8 * g, lo_g = lo - 8 * g;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kc = kb * 32 + r + (r >= 8 ? 8 : 0);
          if (kc > thr_g || (WIN && kc < lo_g)) sx[kb][r] = -INFINITY;
        }
    }
  };
  // ---- max of a tile's scores over the row (lane (g, query n) and lane
  // (1 - g, n) hold the row's two key halves), in log2 units
  auto tile_max = [&](const f32x16 (&sx)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 32; ++e) mx = fmaxf(mx, sx[e / 16][e % 16]);
    return max_halves(mx) * c;
  };
  // ---- probabilities: element r of score half kb of sx -> pf[2 kb + r / 8][r % 8],
  // summed into ls in float32 before the bf16 rounding. Empty asm uses pin
  // the results of a lock-stepped call to its step, so that the compiler
  // cannot move the exponentials out of the products they run beside.
  float mneg = 0.f;               // -m (0 for a row that has seen no key)
  auto prob = [&](const f32x16 (&sx)[2], bf16x8 (&pf)[4], float& ls, auto kbc, auto rc) {
    constexpr int kb = decltype(kbc)::value, r = decltype(rc)::value;
    const float x = __builtin_amdgcn_exp2f(fmaf(sx[kb][r], c, mneg));
    ls += x;
    pf[2 * kb + r / 8][r % 8] = (bf16)x;
    if constexpr (r % 2 == 1) asm volatile("" : "+v"(pf[2 * kb + r / 8]), "+v"(ls));
  };
  // elements [i * 16 / n, (i + 1) * 16 / n) of half kb: step i of n
  auto prob_steps = [&](const f32x16 (&sx)[2], bf16x8 (&pf)[4], float& ls, auto kbc, auto ic, auto nc) {
    constexpr int i = decltype(ic)::value, n_ = decltype(nc)::value;
    constexpr int lo = i * 16 / n_, hi = (i + 1) * 16 / n_;
    [&]<int... Ws>(std::integer_sequence<int, Ws...>) {
      (prob(sx, pf, ls, kbc, std::integral_constant<int, lo + Ws>{}), ...);
    }(std::make_integer_sequence<int, hi - lo>{});
  };
  auto prob_all = [&](const f32x16 (&sx)[2], bf16x8 (&pf)[4], float& ls, auto kbc) {
    [&]<int... Ws>(std::integer_sequence<int, Ws...>) {
      (prob(sx, pf, ls, kbc, std::integral_constant<int, Ws>{}), ...);
    }(std::make_integer_sequence<int, 16>{});
  };
  using KB0 = std::integral_constant<int, 0>;
  using KB1 = std::integral_constant<int, 1>;
  // ---- slow path for a tile that failed the test: raise m to the tile's max,
  // rescale the accumulator and row sum, form the tile's probabilities again
  auto redo_tile = [&](const f32x16 (&sx)[2], bf16x8 (&pf)[4], float& ls) {
    const float mnew = fmaxf(m, tile_max(sx));
    if (mnew != m) {                // from m = -inf (no key seen yet): alpha = 0, acc and l are 0
      const float alpha = exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m = mnew;
    }
    mneg = (EMPTY && m == -INFINITY) ? 0.f : -m;
    ls = 0.f;
    prob_all(sx, pf, ls, KB0{});
    prob_all(sx, pf, ls, KB1{});
  };

  // scores of the current tile (sa) and of the next one (sb), probabilities
  // of the current tile (pa) and of the next one (pb), row-sum partials of
  // the first half (lsa) and second half (lsb) of a tile; the loop is
  // unrolled twice so that the two sets swap roles without copies
  f32x16 sa[2], sb[2];
  bf16x8 pa[4], pb[4];
  float lsa = 0.f, lsb = 0.f;
  if (nit > 0) {
    // prologue: K, V of tiles 0 and 1 into buffers 0 and 1, then S^T of
    // tile 0, its mask, its max as m and the probabilities of its first
    // half (a barrier before the loop's first loads, which overwrite K(0))
#pragma unroll
    for (int i = 0; i < NL; ++i) load_piece(i, 0, t0 * BC, 0, t0 * BC);
#pragma unroll
    for (int i = 0; i < NL; ++i) load_piece(i, 1, t1 * BC, 1, t1 * BC);
    wait_global_loads();
    __syncthreads();
    scores(sa, 0, [](auto) {});
    mask_tile(sa, t0);
    m = tile_max(sa);
    mneg = (EMPTY && m == -INFINITY) ? 0.f : -m;
    prob_all(sa, pa, lsa, KB0{});
    __syncthreads();
  }

  // one tile: sc holds its (masked) scores and pc[0..1] the probabilities of
  // its first half (lsa their sum); sn, pn[0..1] and lsa receive the next tile's
  auto iteration = [&](int it, const f32x16 (&sc)[2], f32x16 (&sn)[2], bf16x8 (&pc)[4], bf16x8 (&pn)[4]) {
    const int vb = it & 1;
    const bf16* vt = sm.v[vb];
    // ---- phase A: S^T of tile it+1 with P of the second half of tile it and the next loads
    lsb = 0.f;
    {
      const int jk = t2 * BC, jv = t1 * BC;
      scores(sn, vb ^ 1, [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        progress_priority<i, 2 * KS, 2 * KS + 2 * DB, 2 * KS + 3 * DB>();   // steps 0 .. 2 KS - 1 of the tile
        prob_steps(sc, pc, lsb, KB1{}, ic, std::integral_constant<int, 2 * KS>{});
        constexpr int lo = i * NL / (2 * KS), hi = (i + 1) * NL / (2 * KS);
        [&]<int... Ws>(std::integer_sequence<int, Ws...>) {
          (load_piece(lo + Ws, vb, jk, vb ^ 1, jv), ...);
        }(std::make_integer_sequence<int, hi - lo>{});
      });
    }
    // ---- the test of tile it (every lane's probability sum at most 2^8)
    float ls = lsa + lsb;
    if (__builtin_amdgcn_ballot_w64(ls > 256.f || (EMPTY && m == -INFINITY)) != 0) redo_tile(sc, pc, ls);
    l += ls;
    mask_tile(sn, t1);

    // ---- phase B: O^T += V^T P^T of tile it (V^T by transposing reads;
    // step i = (kq, db)) with P of the first half of tile it+1
    lsa = 0.f;
    lockstep_products<4 * DB, 4>(
        [&](auto ic) {
          constexpr int i = decltype(ic)::value, kq = i / DB, db = i % DB;
          const bf16x4 r0 = lds_read_tr4(vt + rd_t[0] + 16 * kq * ROW + 32 * db);
          const bf16x4 r1 = lds_read_tr4(vt + rd_t[1] + 16 * kq * ROW + 32 * db);
          return bf16x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
        },
        [&](auto ic, bf16x8 a) {
          constexpr int i = decltype(ic)::value, kq = i / DB, db = i % DB;
          acc[db] = mfma32(a, pc[kq], acc[db]);
        },
        [&](auto ic) {
          // the tile's steps 2 KS + i of 2 KS + 4 DB: step-downs at 1/2, 3/4, 7/8
          static_assert(2 * KS == 4 * DB, "the two phases have equal step counts");
          progress_priority<2 * KS + decltype(ic)::value, 2 * KS, 2 * KS + 2 * DB, 2 * KS + 3 * DB>();
          prob_steps(sn, pn, lsa, KB0{}, ic, std::integral_constant<int, 4 * DB>{});
        },
        std::true_type{});
    t1 = t2;
    t2 = t3;
    t3 = list_at(it + 4);
    wait_global_loads();
    __syncthreads();
  };
  for (int it = 0; it < nit; it += 2) {
    iteration(it, sa, sb, pa, pb);
    if (it + 1 < nit) iteration(it + 1, sb, sa, pb, pa);
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2
  const float lt = sum_halves(l);
  if (row < p.Nq) {
    // a row that saw no key (block-sparse) stores o = 0 and lse = -inf
    const float inv = (SPARSE && lt == 0.f) ? 0.f : 1.f / lt;
    const long long ro = (((long long)b * p.N + p.q_start + row) * p.H + h) * D;
    const long long li = ((long long)b * p.H + h) * p.N + p.q_start + row;
    float lse_row = (m + __log2f(lt)) * kLn2;
    // chunk pair: softmax over the union of the earlier key chunks and this
    // block's keys, from the running result (weight wa) and this block's
    // normalised rows (weight wb), the same arithmetic as the merge kernel
    const float* R = p.mrg_o ? p.mrg_o + ro : nullptr;
    float wa = 0.f, wb = 1.f;
    if (R) {
      const float la = p.mrg_lse[li], lb = lse_row;
      const float mm = fmaxf(la, lb);
      wb = 0.f;
      lse_row = -INFINITY;
      if (mm != -INFINITY) {
        const float ea = __expf(la - mm), eb = __expf(lb - mm);
        const float tot = ea + eb;
        lse_row = mm + __logf(tot);
        const float itot = 1.f / tot;
        wa = ea * itot;
        wb = eb * itot;
      }
    }
    TO* O = (TO*)p.o + ro;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      // accumulator rows (r/4)*8 + g*4 + r%4: four runs of 4 columns
#pragma unroll
      for (int run = 0; run < 4; ++run) {
        const int col = db * 32 + run * 8 + g * 4;
        float z[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = acc[db][run * 4 + e] * inv;
        if (R) {
          const f32x4 x = *(const f32x4*)(R + col);
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] = wa * x[e] + wb * z[e];
        }
        if constexpr (sizeof(TO) == 2) {
          bf16x4 y;
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = (bf16)z[e];
          *(bf16x4*)(O + col) = y;
        } else {
          *(f32x4*)(O + col) = f32x4{z[0], z[1], z[2], z[3]};
        }
      }
    }
    if (g == 0) p.lse[li] = lse_row;
  }
}

// NW waves per workgroup (32 query rows each); the block-sparse kernels
// cover one 256-row block row of the mask per workgroup (8 waves)
template <int D, int NW, typename TO>
hipError_t launch_cfg(const Params& p, hipStream_t s) {
  if (p.bs_row_tiles) {
    const dim3 grid = tile_grid(p.H, p.B, (p.Nq + BS_ROWS - 1) / BS_ROWS, p.causal);
    if (p.causal)
      hipLaunchKernelGGL((fwd_mfma_kernel<D, 8, true, TO, false, true>), grid, dim3(8 * 64), 0, s, p);
    else
      hipLaunchKernelGGL((fwd_mfma_kernel<D, 8, false, TO, false, true>), grid, dim3(8 * 64), 0, s, p);
    return hipGetLastError();
  }
  constexpr int BR = NW * 32;
  const dim3 grid = tile_grid(p.H, p.vl_qtiles ? 1 : p.B, p.vl_qtiles ? p.vl_qcap : (p.Nq + BR - 1) / BR, p.causal);
  if (p.causal && p.window > 0)
    hipLaunchKernelGGL((fwd_mfma_kernel<D, NW, true, TO, true>), grid, dim3(NW * 64), 0, s, p);
  else if (p.causal)
    hipLaunchKernelGGL((fwd_mfma_kernel<D, NW, true, TO>), grid, dim3(NW * 64), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<D, NW, false, TO>), grid, dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma(const Params& p, bool out_f32, hipStream_t s) {
  constexpr int W128 = query_waves(128), W64 = query_waves(64);
  // four-wave workgroups at d = 128 for packed batches (kVarlenQueryWaves) and small grids
  if (p.d == 128 && !p.bs_row_tiles && (p.vl_qtiles || small_query_grid(128, p.B, p.H, p.Nq, device_cu_count())))
    return out_f32 ? launch_cfg<128, 4, float>(p, s) : launch_cfg<128, 4, bf16>(p, s);
  if (p.d == 128) return out_f32 ? launch_cfg<128, W128, float>(p, s) : launch_cfg<128, W128, bf16>(p, s);
  return out_f32 ? launch_cfg<64, W64, float>(p, s) : launch_cfg<64, W64, bf16>(p, s);
}

}  // namespace miattn
