// Attention of a few new query rows against a key/value cache (decode and
// chunked prefill), split over key ranges and combined by the logsumexp
// merge.
//
// The operation is the forward pass of exact attention (FlashAttention
// abstract page) applied at inference time (FlashAttention-2 reviews page,
// reviewer 2, strengths: the method serves training and inference alike;
// reviewer 3, point 3), with the key range cut into chunks whose partial
// results are combined (DistFlashAttn reviews page, reviews 1 and 4;
// BurstAttention rebuttal page: partial softmax results are merged).
//
// Work split (MI355X-specific): with one or a few query rows per head the
// work is a stream over the cache, bound by HBM bandwidth, and one
// (batch, K/V head) offers far too little parallelism for 256 CUs. So:
//  * one single-wave workgroup per (key split, K/V head, block of 32 query
//    rows, batch); the 32 rows are the (query, head) pairs of one grouped-
//    query group, so the group's K/V are read from HBM once per split;
//  * the waves stream tiles of K and V straight from global memory into
//    double-buffered LDS (buffer loads with a hardware range check) and run
//    the forward's tile step on them: S^T = K Q^T with K rows in sigma32
//    order so P stays in registers, online softmax with a lazily raised max,
//    O^T += V^T P^T with V^T from transposing LDS reads. Tiles hold 32 keys
//    for one or two waves (decode: the stream is what matters) and 64 keys
//    when four or eight waves share them (chunked prefill: twice the
//    products per barrier and per tile step; eight waves, 256 rows, halve
//    the tile loads per product again);
//  * it writes its normalised partial output (float32) and logsumexp; a
//    second kernel merges the splits of every row.
#include "common.h"
#include "kernels.h"
#include "mfma_common.h"

namespace miattn {

namespace {

constexpr int NBUF = 2;   // tiles in LDS: the one being used and the next one in flight

// K and V tiles of 32 keys, row-major; rows padded to D + 32 elements with
// the 16-byte chunk index XORed by (row / 4) % 4 (the forward's layout).
// NBUF buffers: the stream keeps NBUF - 1 tiles in flight per wave. (Four
// buffers, three tiles in flight, measured no faster on the decode workload
// and slower on chunked prefill, which then fits fewer waves per CU.)
template <int D, int KB>
struct DecSmem {
  static constexpr int ROW = D + 32;
  static constexpr int TILE = 32 * KB * ROW;   // KB blocks of 32 keys
  bf16 k[NBUF][TILE];
  bf16 v[NBUF][TILE];
};

// s_waitcnt immediate for "at most n vector-memory loads outstanding"
// (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt not waited on)
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Balanced splits: the valid keys of all sequences, taken in order, form
// one range of T = sum_b L_b keys per (K/V head, row block); workgroup w of
// P covers keys [T w / P, T (w + 1) / P) of it, so every workgroup streams
// the same number of keys whatever the length mix. Its partial for sequence
// b goes to slot w + b: the pairs (w, b) whose ranges overlap form a
// staircase, so w + b is unique among them.
// floor(n / d) for 0 <= n < 2^53 and 0 < d < 2^53: the correctly rounded
// double quotient is at most one away from it, so one step either way, with
// exact integer products, fixes it (far shorter than a 64-bit division)
__device__ __forceinline__ long long floor_div(long long n, long long d) {
  long long q = (long long)((double)n / (double)d);
  if (q * d > n) --q;
  else if ((q + 1) * d <= n) ++q;
  return q;
}
__device__ __forceinline__ long long range_start(long long T, int w, int P) { return floor_div(T * w, P); }
// valid cache rows of sequence b, clamped to [0, Nk]
__device__ __forceinline__ int valid_len(const SplitParams& p, int b) {
  return p.k_lens ? min(max(p.k_lens[b], 0), p.Nk) : p.Nk;
}
__device__ __forceinline__ long long wave_sum(long long x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// a value every lane holds alike, as a scalar
__device__ __forceinline__ long long uni64(long long x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long long)x >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}
// T = the sum of the valid lengths, taken by one wave 64 sequences a step
__device__ __forceinline__ long long total_len(const SplitParams& p, int lane) {
  long long T = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) T += wave_sum(b0 + lane < p.B ? valid_len(p, b0 + lane) : 0);
  return uni64(T);
}

template <int D, bool CAUSAL, int NW, int KB, bool BAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(KB)))   // KB = 2: two waves per SIMD
void fwd_split_kernel(SplitParams p) {
  constexpr int KS = D / 16;   // k-steps of the QK^T product
  constexpr int DB = D / 32;   // 32-column blocks of O
  constexpr int DBC = 32 * KB; // keys per tile
  constexpr int ROW = DecSmem<D, KB>::ROW, TILE = DecSmem<D, KB>::TILE;
  constexpr int TILE_KB = TILE * 2 / 1024;          // 1 KB direct loads per tensor tile
  static_assert(TILE * 2 % 1024 == 0, "whole 1 KB pieces");
  constexpr int PIECES = 2 * TILE_KB;               // load instructions per tile (K, V)
  static_assert(PIECES % NW == 0, "tile loads split evenly over the waves");
  constexpr int NL = PIECES / NW;                   // per wave
  __shared__ __attribute__((aligned(16))) DecSmem<D, KB> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;
  // grid: (split, head x row-block group, batch); with 64-key tiles (chunked
  // prefill) the first two are swapped, so that the workgroups of one split
  // over all heads and row blocks run side by side (measured faster there,
  // and slower for decode)
  const int split = KB == 2 ? (int)blockIdx.y : (int)blockIdx.x;
  const int hg = KB == 2 ? (int)blockIdx.x : (int)blockIdx.y;
  const int gkv = hg % p.Hkv;
  const int rb = (hg / p.Hkv) * NW + wave;   // this wave's block of 32 rows

  // ---- the wave's 32 columns: row r = 32 rb + n of the group = (query i, head h)
  const int M = p.Nq * p.G;
  const int r = 32 * rb + n;
  const bool valid = r < M;
  const int rc = valid ? r : M - 1;
  const int i = rc / p.G, h = gkv * p.G + rc % p.G;
  const long long qrs = (long long)p.H * D, krs = (long long)p.Hkv * D;

  float c = fabsf(p.scale) * kLog2e;
  float qsign = p.scale < 0.f ? -1.f : 1.f;
  if (p.scale == 0.f) { c = 1.f; qsign = 0.f; }

  // per-lane LDS read offsets (elements), as in the forward kernel
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

  // Direct loads: piece s = wave * NL + j of a tile (K: s < TILE_KB, then V)
  // covers tensor tile bytes [(s % TILE_KB) KB, +1 KB); lane l fills 16 bytes
  // at 16 l: tile row rr, logical chunk ch (padding from chunk 0), read from
  // byte loff[j] = 2 (rr * row stride + 8 ch) past the tile's first key. Keys
  // past the sequence's valid length read as zeros (buffer range check): a
  // cache's rows past its length may hold anything, NaN included, and a
  // masked score's zero weight times such a V row would not be zero. Keys
  // past k_hi are masked.
  uint32_t loff[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int off = ((wave * NL + j) % TILE_KB) * 1024 + 16 * lane;
    const int rr = off / (ROW * 2), pch = (off % (ROW * 2)) / 16;
    const int col = pch < D / 8 ? ((pch ^ ((rr >> 2) & 3)) << 3) : 0;
    loff[j] = (uint32_t)(rr * krs + col) * 2u;
  }

  // Keys [k_lo, k_hi) of sequence b; the partial goes to slot pslot.
  auto run = [&](int b, int k_lo, int k_hi, long long pslot) {
    const int L = p.k_lens ? min(max(p.k_lens[b], 0), p.Nk) : p.Nk;   // valid cache rows
    const int qpos = L - p.Nq + i;                  // position of query i in the sequence
    const bf16* Q = (const bf16*)p.q + ((long long)b * p.Nq) * qrs;
    const bf16* K = (const bf16*)p.k + ((long long)b * p.Nk) * krs + (long long)gkv * D;
    const bf16* V = (const bf16*)p.v + ((long long)b * p.Nk) * krs + (long long)gkv * D;

    // Q^T operand (B of S^T = K Q^T): lane (g, n) holds Q[i][h][16 ks + 8 g .. +8]
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 x = *(const bf16x8*)(Q + (long long)i * qrs + (long long)h * D + ks * 16 + g * 8);
      if (qsign != 1.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (bf16)((float)x[e] * qsign);
      }
      qf[ks] = x;
    }
    wait_global_loads();

    const int ntile = k_hi > k_lo ? (k_hi - k_lo + DBC - 1) / DBC : 0;
    const uint32_t kbytes = L > 0 ? (uint32_t)(((L - 1) * krs + D) * 2) : 0u;   // rows [0, L)
    const u32x4 rk = rsrc_words(K, kbytes), rv = rsrc_words(V, kbytes);
    auto load_tile = [&](int buf, int key0) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int s_ = wave * NL + j;                // wave-uniform
        const bool is_v = s_ >= TILE_KB;
        buffer_load_lds16_async(is_v ? rv : rk, loff[j], (uint32_t)(key0 * krs) * 2u,
                                lds_addr((is_v ? sm.v[buf] : sm.k[buf]) + (s_ % TILE_KB) * 512));
      }
    };

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    float m = -INFINITY, l = 0.f;

    static_assert(NBUF <= 4 && (NBUF - 2) * NL < 64, "vmcnt range");
    for (int t = 0; t < NBUF - 1 && t < ntile; ++t) load_tile(t, k_lo + t * DBC);
    for (int t = 0; t < ntile; ++t) {
      const int buf = t % NBUF;
      const int key0 = k_lo + t * DBC;
      // wait for tile t; the (at most NBUF - 2) tiles issued after it may stay in flight
      const int later = min(NBUF - 2, ntile - 1 - t);
      if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NL));
      else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL));
      else wait_global_loads();
      // every wave's pieces of tile t are in LDS, and every wave is done with
      // the buffer that the next loads overwrite
      __syncthreads();
      if (t + NBUF - 1 < ntile) load_tile((t + NBUF - 1) % NBUF, key0 + (NBUF - 1) * DBC);
      const bf16* kt = sm.k[buf];
      const bf16* vt = sm.v[buf];

      // ---- S^T = K Q^T: register r of block kb of lane (g, n) <-> key key0 + 32 kb + sigma_row(g, r)
      f32x16 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
      pipelined_products<KB * KS, 4>(
          [&](int i) { return lds_read16(kt + rd_s[(i % KS) & 1], (i / KS) * 32 * ROW + ((i % KS) >> 1) * 32); },
          [&](int i, bf16x8 a) { s[i / KS] = mfma32(a, qf[i % KS], s[i / KS]); });

      // ---- mask: keys past k_hi, and (causal) keys after the query's position
      int thr = k_hi - 1 - key0;
      if (CAUSAL) thr = min(thr, qpos - key0);
      if (__builtin_amdgcn_ballot_w64(thr < DBC - 1) != 0) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (32 * kb + sigma_row(g, rr) > thr) s[kb][rr] = -INFINITY;
      }

      // ---- online softmax; rows that have seen no key yet keep m = -inf and p = 0
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[kb][rr]);
      mx = max_halves(mx);
      const float mt = mx * c;
      const bool raise = mt > m + 8.f;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float mnew = raise ? mt : m;
        // rows that keep their max keep alpha = 1: a row that has seen no key
        // yet has m = -inf, and -inf - -inf has no value
        const float alpha = raise ? exp2f(m - mnew) : 1.f;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) acc[db][rr] *= alpha;
        m = mnew;
      }
      const float mneg = m == -INFINITY ? 0.f : -m;
      bf16x8 pf[2 * KB];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 x;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][half * 8 + e], c, mneg));
            lsum += pv;
            x[e] = (bf16)pv;
          }
          pf[2 * kb + half] = x;
        }
      l += lsum;

      // ---- O^T += V^T P^T: step i = (kq, db), kq = 16-key block of the tile
      pipelined_products<2 * KB * DB, 4>(
          [&](int st) {
            const int kq = st / DB, db = st % DB;
            const bf16x4 r0 = lds_read_tr4(vt + rd_t[0] + 16 * kq * ROW + 32 * db);
            const bf16x4 r1 = lds_read_tr4(vt + rd_t[1] + 16 * kq * ROW + 32 * db);
            return bf16x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
          },
          [&](int st, bf16x8 a) { acc[st % DB] = mfma32(a, pf[st / DB], acc[st % DB]); });
    }

    // ---- partial result of this split: normalised O (float32) and logsumexp;
    // a row without visible keys here gives (0, -inf), the merge's identity
    const float lt = sum_halves(l);
    if (valid) {
      const long long row = pslot * p.Nq + i;        // [slot][i]
      float* O = p.o_part + (row * p.H + h) * D;
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int run = 0; run < 4; ++run) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = acc[db][run * 4 + e] * inv;
          *(f32x4*)(O + db * 32 + run * 8 + g * 4) = x;
        }
      if (g == 0)
        p.lse_part[(pslot * p.H + h) * p.Nq + i] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
    }
  };

  if constexpr (!BAL) {
    // this split's keys of the batch entry
    const int b = blockIdx.z;
    const int L = p.k_lens ? min(max(p.k_lens[b], 0), p.Nk) : p.Nk;
    const int k_lo = split * p.chunk;
    run(b, k_lo, min(L, k_lo + p.chunk), (long long)split * p.B + b);
  } else {
    // this workgroup's range [s0, s1) of the joint key range, sequence by
    // sequence; sequence b holds joint keys [start_b, start_b + L_b)
    static_assert(NW == 1, "balanced ranges: one wave per workgroup");
    const long long T = total_len(p, lane);
    const int P = p.nsplit, w = split;
    const long long s0 = range_start(T, w, P), s1 = range_start(T, w + 1, P);
    if (s0 >= s1) return;
    // the first sequence that ends after s0, and its start: an inclusive scan
    // of the lengths, 64 sequences a step
    int b = p.B;
    long long start = 0, base = 0;
    for (int b0 = 0; b0 < p.B; b0 += 64) {
      const long long x = b0 + lane < p.B ? valid_len(p, b0 + lane) : 0;
      long long incl = x;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const long long y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      // lanes past the last sequence hold the step's total, so the first hit is a sequence
      const unsigned long long hit = __ballot(base + incl > s0);
      if (hit) {
        const int l = __ffsll(hit) - 1;
        b = b0 + l;
        start = base + __shfl(incl - x, l);
        break;
      }
      base += __shfl(incl, 63);
    }
    b = uni(b);
    start = uni64(start);
    for (; b < p.B && start < s1; ++b) {
      const int L = valid_len(p, b);
      const long long a = max(s0, start), e = min(s1, start + L);
      if (e > a) {
        __syncthreads();                          // done with the previous sequence's tiles
        run(b, (int)(a - start), (int)(e - start), (long long)w + b);
      }
      start += L;
    }
  }
}

// acc[c] += sum over t < n of weight_t * row_t[lane + 64 c], with weight_t
// held by lane t of w_l and row_t = src(t). U rows' loads are in flight at
// a time; indices past n repeat the last row, and a zero weight (past n, or
// a partial that no workgroup wrote) selects nothing rather than
// multiplying whatever the row holds.
template <int U, int CPL, class SRC>
__device__ __forceinline__ void accumulate_batches(float (&acc)[CPL], float w_l, int n, int lane, SRC src) {
  for (int t = 0; t < n; t += U) {
    float x[U][CPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* r = src(min(t + u, n - 1)) + lane;
#pragma unroll
      for (int c = 0; c < CPL; ++c) x[u][c] = r[64 * c];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wt = t + u < n ? __shfl(w_l, t + u) : 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] += wt != 0.f ? wt * x[u][c] : 0.f;
    }
  }
}
// (rows with at most four partials, as in chunked prefill, take batches of
// four: eight would double their loads with repeats)
template <int CPL, class SRC>
__device__ __forceinline__ void accumulate_partials(float (&acc)[CPL], float w_l, int n, int lane, SRC src) {
  if (n <= 4) accumulate_batches<4>(acc, w_l, n, lane, src);
  else accumulate_batches<8>(acc, w_l, n, lane, src);
}

// Merge of the splits of every (b, query, head) row: with M the largest
// partial logsumexp, lse = M + ln sum_s e^(lse_s - M) and
// o = sum_s e^(lse_s - lse) o_s; a row with no visible key gives o = 0,
// lse = -inf. One wave per row: lane s < nsplit reads split s's logsumexp
// (64 splits per pass), the wave reduces them, and lane t then accumulates
// columns t, t + 64, ... over the splits with the weights broadcast from
// the lane that holds them.
template <int D>
__global__ __launch_bounds__(64) void split_merge_kernel(SplitParams p) {
  const int lane = threadIdx.x;
  const int row = blockIdx.x;                     // (b, i, h), h fastest
  const int h = row % p.H, i = (row / p.H) % p.Nq, b = row / (p.H * p.Nq);
  const long long ps = (long long)p.B * p.Nq * p.H;   // rows per split
  auto lse_at = [&](int s) { return p.lse_part[(((long long)s * p.B + b) * p.H + h) * p.Nq + i]; };
  const float l0 = lane < p.nsplit ? lse_at(lane) : -INFINITY;   // the first 64 splits, read once
  float mx = l0;
  for (int s = lane + 64; s < p.nsplit; s += 64) mx = fmaxf(mx, lse_at(s));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float tot = 0.f;
  if (mx != -INFINITY) {
    tot = expf(l0 - mx);
    for (int s = lane + 64; s < p.nsplit; s += 64) tot += expf(lse_at(s) - mx);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
  const float lse = mx == -INFINITY ? -INFINITY : mx + logf(tot);
  constexpr int CPL = D / 64;                     // columns per lane
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  if (mx != -INFINITY) {
    for (int s0 = 0; s0 < p.nsplit; s0 += 64) {
      const float ls = s0 == 0 ? l0 : (s0 + lane < p.nsplit ? lse_at(s0 + lane) : -INFINITY);
      accumulate_partials(acc, expf(ls - lse), min(64, p.nsplit - s0), lane,
                          [&](int t) { return p.o_part + ((s0 + t) * ps + row) * D; });
    }
  }
  bf16* O = (bf16*)p.o + (((long long)b * p.Nq + i) * p.H + h) * D + lane;
#pragma unroll
  for (int c = 0; c < CPL; ++c) O[64 * c] = (bf16)acc[c];
  if (lane == 0) p.lse[((long long)b * p.H + h) * p.Nq + i] = lse;
}

// Merge for balanced splits: row (b, i, h) combines the partials of the
// workgroups whose ranges overlap sequence b's keys [a, a + L_b) of the
// joint range (slot w + b), as split_merge_kernel does over splits.
template <int D>
__global__ __launch_bounds__(64) void bal_merge_kernel(SplitParams p) {
  const int lane = threadIdx.x;
  const int row = blockIdx.x;                     // (b, i, h), h fastest
  const int h = row % p.H, i = (row / p.H) % p.Nq, b = row / (p.H * p.Nq);
  long long T = 0, a = 0;                         // all lengths; those before sequence b
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int bb = b0 + lane;
    const long long x = bb < p.B ? valid_len(p, bb) : 0;
    T += wave_sum(x);
    a += wave_sum(bb < b ? x : 0);
  }
  T = uni64(T);
  a = uni64(a);
  const long long e = a + valid_len(p, b);
  const int P = p.nsplit;
  // the last range that starts at or before joint key x: range w starts at
  // or before x exactly when T w < (x + 1) P, so no search is needed
  auto last_range = [&](long long x) { return (int)min((long long)P - 1, floor_div((x + 1) * P - 1, T)); };
  const int w0 = a < e ? last_range(a) : 0, nw = a < e ? last_range(e - 1) - w0 + 1 : 0;
  // a workgroup with an empty range (possible only when T < P) wrote nothing
  auto lse_at = [&](int t) {
    const int w = w0 + t;
    if (T < P && range_start(T, w, P) == range_start(T, w + 1, P)) return -INFINITY;
    return p.lse_part[(((long long)w + b) * p.H + h) * p.Nq + i];
  };
  const float l0 = lane < nw ? lse_at(lane) : -INFINITY;   // the first 64 ranges, read once
  float mx = l0;
  for (int t = lane + 64; t < nw; t += 64) mx = fmaxf(mx, lse_at(t));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float tot = 0.f;
  if (mx != -INFINITY) {
    tot = expf(l0 - mx);
    for (int t = lane + 64; t < nw; t += 64) tot += expf(lse_at(t) - mx);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
  const float lse = mx == -INFINITY ? -INFINITY : mx + logf(tot);
  constexpr int CPL = D / 64;                     // columns per lane
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  if (mx != -INFINITY) {
    for (int t0 = 0; t0 < nw; t0 += 64) {
      const float lt = t0 == 0 ? l0 : (t0 + lane < nw ? lse_at(t0 + lane) : -INFINITY);
      const float w_l = expf(lt - lse);           // 0 for lanes past nw and empty ranges
      accumulate_partials(acc, w_l, min(64, nw - t0), lane, [&](int t) {
        return p.o_part + ((((long long)w0 + t0 + t + b) * p.Nq + i) * p.H + h) * D;
      });
    }
  }
  bf16* O = (bf16*)p.o + (((long long)b * p.Nq + i) * p.H + h) * D + lane;
#pragma unroll
  for (int c = 0; c < CPL; ++c) O[64 * c] = (bf16)acc[c];
  if (lane == 0) p.lse[((long long)b * p.H + h) * p.Nq + i] = lse;
}

template <int D, int NW, bool BAL>
void launch_split_nw(const SplitParams& p, hipStream_t s) {
  constexpr int KB = NW >= 4 ? 2 : 1;    // 64-key tiles when four or more waves share them
  const int rbs = (p.Nq * p.G + 31) / 32;
  const unsigned hgs = p.Hkv * ((rbs + NW - 1) / NW);
  const dim3 grid(KB == 2 ? hgs : p.nsplit, KB == 2 ? p.nsplit : hgs, BAL ? 1 : p.B);
  if (p.causal)
    hipLaunchKernelGGL((fwd_split_kernel<D, true, NW, KB, BAL>), grid, dim3(NW * 64), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_split_kernel<D, false, NW, KB, BAL>), grid, dim3(NW * 64), 0, s, p);
}

template <int D>
hipError_t launch_split_d(const SplitParams& p, hipStream_t s) {
  if (p.balanced) {                               // balanced ranges: one block of 32 rows per group
    launch_split_nw<D, 1, true>(p, s);
  } else {                                        // waves per workgroup = blocks of 32 rows sharing each tile
    const int rbs = (p.Nq * p.G + 31) / 32;
    if (rbs >= 8) launch_split_nw<D, 8, false>(p, s);
    else if (rbs >= 4) launch_split_nw<D, 4, false>(p, s);
    else if (rbs >= 2) launch_split_nw<D, 2, false>(p, s);
    else launch_split_nw<D, 1, false>(p, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.balanced)
    hipLaunchKernelGGL((bal_merge_kernel<D>), dim3(p.B * p.Nq * p.H), dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL((split_merge_kernel<D>), dim3(p.B * p.Nq * p.H), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_split(const SplitParams& p, hipStream_t s) {
  return p.d == 128 ? launch_split_d<128>(p, s) : launch_split_d<64>(p, s);
}

}  // namespace miattn
