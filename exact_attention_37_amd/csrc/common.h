// Shared device/host definitions of libmiattn (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One attention call on a rectangular block of the problem: query rows
// [q_start, q_start + Nq) against key rows [k_start, k_start + Nk) of a
// sequence of length N. Every tensor (including chunk scratch buffers) has
// the full-sequence layout, so a row is always addressed by its absolute
// position: q/o/dout/dq row i at q_start + i, k/v/dk/dv row j at k_start + j,
// lse/dsum entry (b, h, q_start + i).
struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;           // forward output; backward: the forward's o (read)
  float* lse;        // [B, H, N]
  const void* dout;  // backward only
  void* dq;
  void* dk;
  void* dv;
  float* dsum;       // backward: rowsum(dout * o), [B, H, N]
  int fuse_dsum;     // backward, bf16: the dQ kernel forms dsum for its rows from o and dout and writes it
  int B, H, Hkv, G;
  int N;             // full sequence length: row strides and [B,H,N] strides
  int Nq, Nk;        // rows of this block
  int q_start, k_start;
  int d;
  int causal;        // mask keys whose absolute position exceeds the query's
  float scale;
  int accumulate;        // backward: add into float32 dq/dk/dv
  // Store modes of the matrix-core backward kernels, for dq (acc_q) and for
  // dk / dv (acc_kv): ACC_STORE writes the input dtype, ACC_ADD adds into
  // float32, ACC_FIRST writes float32 without reading, ACC_LAST adds the
  // float32 running sums q_part / k_part / v_part (same layouts) and writes
  // the input dtype. Chunk pairs use FIRST / ADD / LAST per chunk.
  int acc_q, acc_kv;
  const float* q_part;
  const float* k_part;
  const float* v_part;
  int window;            // > 0 (causal only): key visible iff query position - window < key position
  // Forward (matrix-core kernel) of a chunk pair: merge the block's result
  // into the running result of the same rows over earlier key chunks, float32
  // [B, N, H, d] and [B, H, N] (the attn_merge arithmetic), and store the
  // merged rows to o / lse, which may be these very buffers; null otherwise.
  const float* mrg_o;
  const float* mrg_lse;
  // Packed variable-length batch: sequence z of the grid owns rows
  // [cu_seqlens[z], cu_seqlens[z + 1]) of a B = 1 layout of N rows; null otherwise.
  const int* cu_seqlens;
  // Packed batch, matrix-core kernels: device-built work lists of (sequence,
  // tile) entries, [0] = count, entry e at [2 + 2e], [3 + 2e] (query tiles of
  // the forward / dQ workgroups; key tiles of the dK/dV workgroups), and the
  // grid extent reserved for them; null otherwise.
  const int* vl_qtiles;
  const int* vl_ktiles;
  int vl_qcap, vl_kcap;
  // Block-sparse attention: one mask entry per block of BS_ROWS query rows x
  // BS_COLS keys, shared by every batch and head; null otherwise.
  const uint8_t* bs_mask;   // [ceil(N / BS_ROWS)][bs_nbc], read by the float32 kernels
  int bs_nbc;               // ceil(N / BS_COLS)
  // Tile lists built from the mask for the matrix-core kernels (BS_TILE rows
  // or keys per tile, ascending, cut at the causal diagonal and the last row):
  const int* bs_row_cnt;    // [nbr] key tiles kept for block row r
  const int* bs_row_plain;  // [nbr] how many of them need no causal / ragged-end mask
  const int* bs_row_tiles;  // [nbr][bs_ld]
  const int* bs_col_cnt;    // [nbc] query tiles kept for block column c
  const int* bs_col_tiles;  // [nbc][bs_ld]
  int bs_ld;                // ceil(N / BS_TILE)
};

constexpr int BS_ROWS = 256, BS_COLS = 128, BS_TILE = 64;
constexpr int ACC_STORE = 0, ACC_ADD = 1, ACC_FIRST = 2, ACC_LAST = 3;

// Waves (32 query rows each) of the forward and dQ matrix-core workgroups:
// 8 at d = 128 (one workgroup per CU, two waves per SIMD); 4 at d = 64,
// where two workgroups share a CU so that one's prologue and epilogue
// overlap the other's products. Packed-batch work lists use the same rows.
constexpr int query_waves(int d) { return d == 64 ? 4 : 8; }
// A dense (not packed, not block-sparse) forward or dQ launch at d = 128
// with fewer eight-wave workgroups than two per compute unit takes
// four-wave workgroups (128 rows) instead: twice the workgroups, two per CU
// at a time, and finer pieces for the causal load balance (small batch x
// heads: the FlashAttention-2 reviews page, authors' common response,
// ablation (B), parallelism over the sequence).
// Packed batches (short sequences) take four-wave (128-row) query
// workgroups at both head sizes: half the masked diagonal per workgroup.
constexpr int kVarlenQueryWaves = 4;
inline bool small_query_grid(int d, int B, int H, int Nq, int cus) {
  return d == 128 && (long long)B * H * ((Nq + 255) / 256) < 2LL * cus;
}

// For a packed variable-length batch, narrows p to sequence s (rows
// [cu_seqlens[s], cu_seqlens[s + 1]) of the single B = 1 layout; the offsets
// are clamped to [0, N] so malformed ones cannot move any access out of the
// tensors) and returns false when the workgroup's first row `row0` lies past
// the sequence. A no-op returning true for ordinary batches.
__device__ __forceinline__ bool narrow_to_sequence(Params& p, int s, int row0) {
  if (!p.cu_seqlens) return true;
  const int e = min(max(p.cu_seqlens[s + 1], 0), p.N);
  const int a = min(max(p.cu_seqlens[s], 0), e);
  p.q_start = p.k_start = a;
  p.Nq = p.Nk = e - a;
  return row0 < p.Nq;
}

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

}  // namespace miattn
