// Launchers of the libmiattn kernels (host side). Each returns the HIP error
// of its launch(es); none synchronises.
#pragma once

#include "common.h"

namespace miattn {

// float32 / vector-ALU kernels (dtype 0 = float32, 1 = bf16 inputs).
hipError_t launch_fwd_simt(const Params& p, int dtype, bool out_f32, hipStream_t s);
hipError_t launch_bwd_simt(const Params& p, int dtype, hipStream_t s);

// bf16 matrix-core kernels (gfx950 MFMA).
hipError_t launch_fwd_mfma(const Params& p, bool out_f32, hipStream_t s);
hipError_t launch_bwd_mfma(const Params& p, hipStream_t s);          // dK/dV kernel, then dQ kernel
hipError_t launch_bwd_dkdv_mfma(const Params& p, hipStream_t s);
hipError_t launch_bwd_dq_mfma(const Params& p, hipStream_t s);

// rowsum(dout * o) for query rows [row0, row0 + nrows) of every (b, h).
hipError_t launch_bwd_pre(const void* o, const void* dout, float* dsum, int B, int H, int N,
                          int d, int row0, int nrows, int dtype, hipStream_t s);

// LSE merge over rows [row0, row0 + nrows); all buffers full-sequence layout.
// ta/tb/to: element types of o_a, o_b, o (0 = float32, 1 = bf16).
hipError_t launch_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                        void* o, float* lse, int B, int H, int N, int d, int row0, int nrows,
                        int ta, int tb, int to, hipStream_t s);

// Query rows against a key/value cache, split over key ranges (bf16).
// q, o: [B, Nq, H, d]; k, v: [B, Nk, Hkv, d]; lse: [B, H, Nq]; k_lens: [B]
// valid cache rows per batch entry, or null for Nk. Causal: query i of batch
// b sits at position k_lens[b] - Nq + i. Split s covers keys
// [s * chunk, (s + 1) * chunk); its partial output and logsumexp go to
// o_part [nsplit, B, Nq, H, d] and lse_part [nsplit, B, H, Nq] (float32)
// before the merge writes o and lse.
struct SplitParams {
  const void* q;
  const void* k;
  const void* v;
  const int* k_lens;
  void* o;
  float* lse;
  float* o_part;
  float* lse_part;
  int B, H, Hkv, G, Nq, Nk, d, causal;
  float scale;
  int nsplit, chunk;
  // Nonzero: balanced ranges (one block of <= 32 rows per K/V head group):
  // nsplit = ranges per K/V head of the joint key range, partial slots w + b
  // (nsplit + B of them). Zero: nsplit chunks of `chunk` keys per sequence,
  // partial slots split * B + b.
  int balanced;
};
hipError_t launch_fwd_split(const SplitParams& p, hipStream_t s);

// dst[i] = (bf16 or float) src[i] for n float32 elements.
hipError_t launch_convert(const float* src, void* dst, long long n, int dtype, hipStream_t s);

// dst[i] = value for n float32 elements (a kernel, so it can sit in a graph).
hipError_t launch_fill(float* dst, long long n, float value, hipStream_t s);
int device_cu_count();   // compute units of the current device (cached per device)

// Block-sparse tile lists (the bs_* fields of Params) from a block mask of
// [nbr = ceil(N / BS_ROWS)][nbc = ceil(N / BS_COLS)] bytes. `ints` must hold
// bs_list_ints(N) int32 values; fills p's list pointers into it.
long long bs_list_ints(int N);
hipError_t launch_bs_lists(const uint8_t* mask, int N, int causal, int* ints, Params& p, hipStream_t s);

// Packed batches: entries reserved for the work list of tiles of `rows`
// rows (ceil(total / rows) + nseq), and the one-workgroup kernel that fills
// it from the device offsets (2 + 2 * cap int32 values at `list`).
int varlen_list_cap(int total, int rows, int nseq);
hipError_t launch_varlen_tiles(const int* cu_seqlens, int nseq, int total, int rows, int desc, int* list,
                               hipStream_t s);

}  // namespace miattn
