// Shared pieces of the bf16 matrix-core kernels (gfx950).
//
// v_mfma_f32_32x32x16_bf16 operand layouts (lane l = 32*g + n, g in {0,1}):
//   A (32 x 16): lane holds A[n][8g .. 8g+7]
//   B (16 x 32): lane holds B[8g .. 8g+7][n]
//   C (32 x 32): lane holds C[(r/4)*8 + 4g + r%4][n], r = 0..15
// The contraction index only has to be split the same way in A and B, so
// any consistent assignment of k to (g, element) is valid.
#pragma once

#include <type_traits>
#include <utility>

#include "common.h"

namespace miattn {

constexpr int LDS_PAD = 8;   // bf16 elements (16 bytes) of padding per LDS row

// Row slot -> index inside a 32-row block with bits 2 and 3 swapped. Loading
// A-operand row slot m from row sigma(m) makes C's register r of lane (g, n)
// hold row 8g + r (r < 8) or 16 + 8g + (r - 8) (r >= 8): 8 consecutive rows,
// which is the layout of an A or B operand whose contraction runs over them.
__device__ __forceinline__ int sigma32(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Row of a 32-row block held in register r of lane group g after the sigma32
// permutation.
__device__ __forceinline__ int sigma_row(int g, int r) { return (r < 8) ? (8 * g + r) : (16 + 8 * g + (r - 8)); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_read16(const bf16* base, int elem_off) {
  return *(const bf16x8*)(base + elem_off);
}

__device__ __forceinline__ uint32_t pack2(bf16 lo, bf16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// Stores a block of 4 rows x 8 columns (one bf16x8 per row) transposed: row
// d = col0 + e of `dst` receives the 4 values at [row0, row0 + 4).
__device__ __forceinline__ void store_transposed4x8(bf16* dst, int row_len, int col0, int row0, const bf16x8 (&r)[4]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint2 w = {pack2(r[0][e], r[1][e]), pack2(r[2][e], r[3][e])};
    *(uint2*)(dst + (col0 + e) * row_len + row0) = w;
  }
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane i receives in slot s element (i % 4) of the 8-byte chunk addressed by
// lane 4s + i / 4 of its group. So if lane j of a group addresses row
// r0 + j / 4, columns c0 + 4 (j % 4) .. +3 of a row-major tile, lane i gets
// column c0 + i of rows r0 .. r0 + 3: a transposed operand fragment.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

// LDS reads through 32-bit LDS byte addresses. lds_addr() gives the address
// of a shared-memory object; lds_opaque() hides an address from the
// optimizer, so that reads at constant offsets from it are encoded with the
// instruction's offset field instead of recomputing addresses per read.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ uint32_t lds_opaque(uint32_t a) {
  asm("" : "+v"(a));
  return a;
}
__device__ __forceinline__ bf16x8 lds_read16_at(uint32_t a) {
  return *(const __attribute__((address_space(3))) bf16x8*)a;
}
__device__ __forceinline__ f32x4 lds_read_f32x4_at(uint32_t a) {
  return *(const __attribute__((address_space(3))) f32x4*)a;
}
__device__ __forceinline__ bf16x4 lds_read_tr4_at(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a);
}

// v_mfma_f32_16x16x32_bf16 operand layouts (lane l = 16 q + i, q in 0..3):
//   A (16 x 32): lane holds A[i][8q .. 8q+7]
//   B (32 x 16): lane holds B[8q .. 8q+7][i]
//   C (16 x 16): lane holds C[4q + r][i], r = 0..3
// At the chip's power limit this shape sustains about 12% more bf16 FLOP/s
// than the 32x32x16 one (it moves half as many accumulator bytes per FLOP).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}


// Direct global -> LDS load of 16 bytes per lane: the wave writes 1 KB of
// LDS contiguously, lane l at lds_base + 16 l; lds_base must be the same in
// every lane. Completion is tracked by vmcnt like any global load.
__device__ __forceinline__ void global_load_lds16(const void* g, bf16* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Buffer descriptor for raw loads from the `bytes` bytes at `base`. The
// hardware checks every dword against the range: one at or past `bytes`
// (vector plus scalar offset) reads as zero and touches no memory, so tiles
// that run past the last row need no clamping. Word 3 (0x00020000) selects
// the 32-bit data format that gfx9-family raw loads need for the check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct buffer -> LDS load of 16 bytes per lane from byte offset voff + soff
// (voff per lane, soff wave-uniform): the wave writes 1 KB of LDS
// contiguously, lane l at lds_base + 16 l (lds_base the same in every lane).
// Completion is tracked by vmcnt like any global load.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                                  bf16* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff,
                                           0, 0);
}

// Buffer descriptor as four dwords (for inline assembly): base address,
// stride 0, `bytes` records, and the same range-checked raw format as
// make_rsrc().
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// buffer_load_lds16 issued through inline assembly. The compiler then does
// not know that the load writes LDS; otherwise it makes every later LDS read
// it cannot prove disjoint from the destination (transposing reads, reads
// through computed addresses) wait for all outstanding tile loads. The tile
// being loaded is never read before the caller's wait_global_loads() and
// barrier, so no such wait is needed. lds_base: LDS byte address.
__device__ __forceinline__ void buffer_load_lds16_async(u32x4 rsrc, uint32_t voff, uint32_t soff,
                                                        uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff)
               : "m0");
}

// The same load with the LDS address given as base + offset (both
// wave-uniform), summed straight into M0: one scalar instruction fewer per
// load where the base changes from tile to tile and the offsets do not.
__device__ __forceinline__ void buffer_load_lds16_async(u32x4 rsrc, uint32_t voff, uint32_t soff,
                                                        uint32_t lds_base, uint32_t lds_off) {
  asm volatile("s_add_u32 m0, %0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds"
               :
               : "s"(lds_base), "s"(lds_off), "v"(voff), "s"(rsrc), "s"(soff)
               : "m0", "scc");
}

// acc += A B with the accumulator held in AGPRs (the matrix cores' own
// accumulation registers), for accumulators that live through a whole loop
// and are read only after it: they then take no VGPRs. The compiler does not
// see this product's latency, so agpr_settle() must separate it from any
// other access to the accumulator (see below).
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// 24 wait states tied to two accumulators: covers both the write of their
// initial values before the first mfma32_agpr and the last product's result
// latency before they are read (both below 20 wait states on gfx950).
__device__ __forceinline__ void agpr_settle(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(x), "+a"(y));
}

// The value of lane l ^ 32 combined with lane l's own, through one
// v_permlane32_swap (no LDS round trip): swapping a register with itself
// leaves the lower half's values in result 0 and the upper half's in
// result 1 of every lane (checked on the device by a lane-layout probe).
__device__ __forceinline__ float max_halves(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// A value every lane holds alike, moved to a scalar register (offsets of the
// inline-assembly buffer loads must be scalar).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Waits for every outstanding global load of this wave. Used after the
// loads of loop-invariant matrix operands: without it the compiler cannot
// prove them complete across the loop back-edge and inserts vmcnt waits
// (on the next tile's prefetch) in front of the loop's first products.
// (gfx9 s_waitcnt encoding: vmcnt = 0, expcnt = 7, lgkmcnt = 15, i.e. wait on
// vector memory only.)
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// A chain of N matrix-core products whose A (or B) operands come from LDS:
// rd(i) reads step i's operand, mm(i, x) issues step i's MPS MFMAs. Keeps R
// LDS reads in flight ahead of the MFMAs, and pins that order for the
// scheduler (R reads, then alternating MPS MFMAs / 1 read), so LDS latency
// overlaps the matrix cores instead of stalling each product.
template <int N, int R, class RD, class MM, int MPS = 1>
__device__ __forceinline__ void pipelined_products(RD rd, MM mm) {
  bf16x8 ring[R];
#pragma unroll
  for (int i = 0; i < R; ++i) ring[i] = rd(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bf16x8 a = ring[i % R];
    if (i + R < N) ring[i % R] = rd(i + R);
    mm(i, a);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, R, 0);   // DS reads
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, MPS, 0); // MFMA
    if (i + R < N) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// The same pipeline split in two, so that other work can sit between the
// issue and the scheduling pattern: sched_group_barrier groups are filled
// from instructions that precede them in the block. issue_products() emits
// the reads and MFMAs; products_pattern<N, R, V>() then pins R reads and
// N x {MPS MFMAs, 1 read, V VALU}, pulling independent vector work written
// between the two calls (same basic block: no branches) in between the
// matrix-core products.
template <int N, int R, class RD, class MM>
__device__ __forceinline__ void issue_products(RD rd, MM mm) {
  bf16x8 ring[R];
#pragma unroll
  for (int i = 0; i < R; ++i) ring[i] = rd(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bf16x8 a = ring[i % R];
    if (i + R < N) ring[i % R] = rd(i + R);
    mm(i, a);
  }
}

template <int N, int R, int V, int MPS = 1>
__device__ __forceinline__ void products_pattern() {
  __builtin_amdgcn_sched_group_barrier(0x100, R, 0);     // DS reads
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, MPS, 0); // MFMA
    if (i + R < N) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);   // VALU
  }
}

// Wave priority from a wave's progress through one tile's lock steps, for
// kernels that run two waves per SIMD and meet at a barrier after every
// tile. When both waves of a SIMD can issue, the hardware issues the older
// one, so the older wave runs ahead, then idles at the barrier while the
// younger one finishes the tile alone, without a partner whose work could
// overlap its own (measured: 32% of the older waves' time in the dQ kernel
// at 16K, 2% of the younger ones'). A wave starts each tile at priority 3 and
// steps down at steps C1 < C2 < C3 of the tile: the wave in front then gives
// way to the one behind at every step-down, and the two reach the barrier
// close together. Call at every step I of the tile (the other steps emit
// nothing).
template <int I, int C1, int C2, int C3>
__device__ __forceinline__ void progress_priority() {
  static_assert(0 < C1 && C1 < C2 && C2 < C3, "step-downs in order, after the first step");
  if constexpr (I == 0) __builtin_amdgcn_s_setprio(3);
  else if constexpr (I == C1) __builtin_amdgcn_s_setprio(2);
  else if constexpr (I == C2) __builtin_amdgcn_s_setprio(1);
  else if constexpr (I == C3) __builtin_amdgcn_s_setprio(0);
}

// A chain of N matrix-core products executed in lock step with other work:
// step i issues the LDS read for step i + R, the MFMA(s) of step i and the
// work ex(i), and nothing moves across step boundaries (sched_barrier). Work
// that does not depend on the products in flight (softmax of an earlier
// block, tile stores and loads) thereby runs on the vector units while the
// matrix cores are busy, also with a single wave per SIMD. The steps are
// expanded at compile time: rd, mm and ex receive std::integral_constant
// step indices, so every per-step decision is resolved by `if constexpr`.
//
// PAIRED: at even steps the product also waits for the next step's operand
// (an empty asm statement that reads it). LDS reads complete in order, so
// one wait then covers two products and the odd steps issue none: half the
// s_waitcnt instructions, for kernels whose issue slots are the limit.
template <int I, int N, int R, bool PAIRED, class RD, class MM, class EX>
__device__ __forceinline__ void lockstep_step(bf16x8 (&ring)[R], RD& rd, MM& mm, EX& ex) {
  if constexpr (I < N) {
    const bf16x8 a = ring[I % R];
    if constexpr (PAIRED && I % 2 == 0 && I + 1 < N) asm volatile("" ::"v"(ring[(I + 1) % R]));
    if constexpr (I + R < N) ring[I % R] = rd(std::integral_constant<int, I + R>{});
    mm(std::integral_constant<int, I>{}, a);
    ex(std::integral_constant<int, I>{});
    __builtin_amdgcn_sched_barrier(0);
    lockstep_step<I + 1, N, R, PAIRED>(ring, rd, mm, ex);
  }
}

template <int N, int R, class RD, class MM, class EX, bool PAIRED = false>
__device__ __forceinline__ void lockstep_products(RD rd, MM mm, EX ex, std::bool_constant<PAIRED> = {}) {
  bf16x8 ring[R];
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    ((ring[Is] = rd(std::integral_constant<int, Is>{})), ...);
  }(std::make_integer_sequence<int, R>{});
  lockstep_step<0, N, R, PAIRED>(ring, rd, mm, ex);
}

// Workgroup x index -> head index, so that with H % 8 == 0 all heads that
// share a K/V head run on one XCD (workgroups are dealt round-robin to the 8
// XCDs, and consecutive x indices are consecutive in dispatch order).
__device__ __forceinline__ int xcd_head(int x, int H) {
  return (H & 7) == 0 ? (x & 7) * (H >> 3) + (x >> 3) : x;
}

// Grid order of the matrix-core kernels. Causal: (head, batch, tile) with the
// tile index slowest, so that the heaviest tiles of every (b, h) are
// dispatched first and the light ones fill the end of the run (a batch-major
// order leaves the heavy tiles of the last batch entries to the end).
// Non-causal: (head, tile, batch); every tile weighs the same, and the
// workgroups of one (b, h) run together and share its K/V in the L2.
template <bool CAUSAL>
__device__ __forceinline__ int tile_grid_index() { return CAUSAL ? (int)blockIdx.z : (int)blockIdx.y; }
template <bool CAUSAL>
__device__ __forceinline__ int tile_grid_count() { return CAUSAL ? (int)gridDim.z : (int)gridDim.y; }
template <bool CAUSAL>
__device__ __forceinline__ int batch_grid_index() { return CAUSAL ? (int)blockIdx.y : (int)blockIdx.z; }
inline dim3 tile_grid(int heads, int batch, int tiles, int causal) {
  return causal ? dim3(heads, batch, tiles) : dim3(heads, tiles, batch);
}

}  // namespace miattn
