// C ABI of libmiattn: argument validation, kernel selection, scratch
// management and the chunk-pair driver. No entry point synchronises the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>
#include <map>
#include <mutex>
#include <optional>
#include <utility>
#include <vector>

#include "../../include/miattn.h"
#include "common.h"
#include "kernels.h"

using miattn::Params;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int ok() {
  g_err.clear();
  return MIATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;
};
Range span(const void* p, long long bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, a + (uintptr_t)bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int check_common(int B, int H, int Hkv, int N, int d, int dtype) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1)
    return fail(MIATTN_EINVAL, "B, H, Hkv and N must be >= 1");
  if (H % Hkv != 0) return fail(MIATTN_EINVAL, "H must be a multiple of Hkv");
  if (d != 64 && d != 128) return fail(MIATTN_EUNSUPPORTED, "head dimension d must be 64 or 128");
  if (dtype != MIATTN_F32 && dtype != MIATTN_BF16)
    return fail(MIATTN_EUNSUPPORTED, "dtype must be MIATTN_F32 or MIATTN_BF16");
  if (B > 65535 || H > 65535) return fail(MIATTN_EUNSUPPORTED, "B and H must be <= 65535");
  // [B, H, N] statistics and row positions are indexed with 32-bit ints; the
  // matrix-core kernels address one sequence of a tensor (plus one tile past
  // its end) with 32-bit byte offsets
  if ((long long)B * H * N >= (1LL << 31) || (long long)(N + 64) * H * d >= (1LL << 31))
    return fail(MIATTN_EUNSUPPORTED, "problem too large for 32-bit row indexing");
  return MIATTN_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (p == nullptr) return fail(MIATTN_EINVAL, "null pointer argument");
    if (!aligned16(p)) return fail(MIATTN_EINVAL, "pointer not 16-byte aligned");
  }
  return MIATTN_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MIATTN_OK;
  return fail(MIATTN_ELAUNCH, std::string(what) + ": " + hipGetErrorString(e));
}

size_t esize(int dtype) { return dtype == MIATTN_F32 ? 4 : 2; }

Params make_params(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                   int N, int d, int causal, float scale) {
  Params p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.G = H / Hkv;
  p.N = N;
  p.Nq = N;
  p.Nk = N;
  p.q_start = 0;
  p.k_start = 0;
  p.d = d;
  p.causal = causal;
  p.scale = scale;
  return p;
}

// One forward block (rows and offsets in p). out_f32: o is float32.
hipError_t fwd_block(const Params& p, int dtype, bool out_f32, hipStream_t s) {
  if (dtype == MIATTN_BF16) return miattn::launch_fwd_mfma(p, out_f32, s);
  return miattn::launch_fwd_simt(p, dtype, out_f32, s);
}

// One backward block: p.dsum must hold rowsum(dout * o) of these rows.
hipError_t bwd_block(const Params& p, int dtype, hipStream_t s) {
  if (dtype == MIATTN_BF16) return miattn::launch_bwd_mfma(p, s);
  return miattn::launch_bwd_simt(p, dtype, s);
}

// Scratch memory of one call, carved from a buffer that the library keeps
// per (device, stream). Every use of that buffer is ordered on its stream,
// so consecutive calls on one stream can share it without any allocation:
// a stream-ordered allocation and free cost about 15 us of GPU time per
// call, a tenth of a decode step. A call whose needs exceed the buffer takes
// the rest with hipMallocAsync and afterwards replaces the buffer with one
// of its full size (freeing the old one in stream order), so allocations
// stop after the largest call. A call being captured into a graph uses
// stream-ordered allocations only: the graph then owns its scratch and never
// refers to a buffer that a later call may replace. attn_release_scratch()
// frees a stream's buffer.
struct Arena {
  void* base = nullptr;
  size_t cap = 0;
};
std::mutex arena_mu;
std::map<std::pair<int, hipStream_t>, Arena> arenas;

struct Scratch {
  hipStream_t s;
  int dev = 0;
  bool cached = false;        // false while the stream is being captured
  Arena a;                    // this call's buffer, taken out of the map
  size_t used = 0;            // bytes asked for, rounded to 256
  std::vector<void*> extra;   // stream-ordered allocations beyond the buffer
  explicit Scratch(hipStream_t st) : s(st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipGetDevice(&dev) != hipSuccess || hipStreamIsCapturing(s, &cs) != hipSuccess ||
        cs != hipStreamCaptureStatusNone)
      return;
    cached = true;
    std::lock_guard<std::mutex> g(arena_mu);
    auto it = arenas.find({dev, s});
    if (it != arenas.end()) {
      a = it->second;   // a concurrent call on the same stream finds none and allocates
      arenas.erase(it);
    }
  }
  void* get(size_t bytes) {
    const size_t b = (bytes + 255) & ~(size_t)255;
    if (used + b <= a.cap) {
      void* p = (char*)a.base + used;
      used += b;
      return p;
    }
    used += b;
    void* p = nullptr;
    if (hipMallocAsync(&p, bytes, s) != hipSuccess) return nullptr;
    extra.push_back(p);
    return p;
  }
  ~Scratch() {
    for (void* p : extra) (void)hipFreeAsync(p, s);
    if (!cached) return;
    if (used > a.cap) {   // grow to this call's full size for the next call
      if (a.base) (void)hipFreeAsync(a.base, s);
      a = Arena{};
      if (hipMallocAsync(&a.base, used, s) == hipSuccess) a.cap = used;
      else a.base = nullptr;
    }
    std::lock_guard<std::mutex> g(arena_mu);
    Arena& slot = arenas[{dev, s}];
    if (slot.cap < a.cap) std::swap(slot, a);   // keep the larger, free the other
    if (a.base) (void)hipFreeAsync(a.base, s);
  }
};

// Balanced rounds of causal chunk pairs (i, j), j <= i, for P chunks.
// Round 0: the diagonal pairs and the pairs at distance P/2; round t
// (1 <= t < P/2): the pairs at distance t and at distance P - t. With a
// diagonal pair counted as half a pair, every round holds P pairs of work.
std::vector<std::vector<std::pair<int, int>>> balanced_rounds(int P) {
  std::vector<std::vector<std::pair<int, int>>> rounds;
  if (P == 1) {
    rounds.push_back({{0, 0}});
    return rounds;
  }
  std::vector<std::pair<int, int>> r0;
  for (int i = 0; i < P; ++i) r0.push_back({i, i});
  for (int i = P / 2; i < P; ++i) r0.push_back({i, i - P / 2});
  rounds.push_back(r0);
  for (int t = 1; t < P / 2; ++t) {
    std::vector<std::pair<int, int>> r;
    for (int i = t; i < P; ++i) r.push_back({i, i - t});
    for (int i = P - t; i < P; ++i) r.push_back({i, i - (P - t)});
    rounds.push_back(r);
  }
  return rounds;
}

}  // namespace

extern "C" {

const char* attn_last_error(void) { return g_err.c_str(); }

const char* attn_version(void) { return "libmiattn 0.1 (gfx950)"; }

int attn_release_scratch(void* stream) {
  const hipStream_t s = (hipStream_t)stream;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MIATTN_ELAUNCH, "hipGetDevice failed");
  Arena a;
  {
    std::lock_guard<std::mutex> g(arena_mu);
    auto it = arenas.find({dev, s});
    if (it == arenas.end()) return ok();
    a = it->second;
    arenas.erase(it);
  }
  if (hipFreeAsync(a.base, s) != hipSuccess) return fail(MIATTN_ELAUNCH, "hipFreeAsync failed");
  return ok();
}

int attn_chunk_schedule(int nchunks, int* round_of, int* q_chunk, int* k_chunk, int capacity) {
  if (nchunks < 1 || (nchunks > 1 && nchunks % 2 != 0)) return -1;
  const int npairs = nchunks * (nchunks + 1) / 2;
  if (capacity < npairs || !round_of || !q_chunk || !k_chunk) return -1;
  int n = 0, r = 0;
  for (const auto& round : balanced_rounds(nchunks)) {
    for (const auto& pr : round) {
      round_of[n] = r;
      q_chunk[n] = pr.first;
      k_chunk[n] = pr.second;
      ++n;
    }
    ++r;
  }
  return n;
}

}  // extern "C"

namespace {

// Block-sparse set-up: the float32 kernels read the block mask itself, the
// matrix-core kernels the tile lists built from it (into scratch) on stream s.
int blocksparse_setup(Params& p, const uint8_t* bmask, int dtype, Scratch& scratch, hipStream_t s) {
  if (dtype != MIATTN_BF16) {
    p.bs_mask = bmask;
    p.bs_nbc = (p.N + miattn::BS_COLS - 1) / miattn::BS_COLS;
    return MIATTN_OK;
  }
  int* ints = (int*)scratch.get((size_t)miattn::bs_list_ints(p.N) * 4);
  if (!ints) return fail(MIATTN_ENOMEM, "hipMallocAsync failed for the block-sparse tile lists");
  return launch_status(miattn::launch_bs_lists(bmask, p.N, p.causal, ints, p, s), "block-sparse tile lists");
}

// Packed batch, matrix-core kernels: the work lists of (sequence, tile)
// entries, built on the device from cu_seqlens into scratch: query tiles of
// the forward / dQ workgroups (32 kVarlenQueryWaves rows, heaviest causal tile
// of a sequence first) and, for the backward, key tiles of the dK/dV
// workgroups (128 keys, first tile first). The grids reserve
// ceil(total / rows) + nseq entries.
int varlen_lists(Params& p, Scratch& scratch, bool backward, hipStream_t s) {
  const int total = p.N, nseq = p.B, qrows = 32 * miattn::kVarlenQueryWaves;
  const int qcap = miattn::varlen_list_cap(total, qrows, nseq);
  int* ql = (int*)scratch.get((size_t)(2 + 2 * (long long)qcap) * 4);
  if (!ql) return fail(MIATTN_ENOMEM, "hipMallocAsync failed for the packed-batch work list");
  int st = launch_status(miattn::launch_varlen_tiles(p.cu_seqlens, nseq, total, qrows, 1, ql, s), "work list");
  if (st) return st;
  p.vl_qtiles = ql;
  p.vl_qcap = qcap;
  if (!backward) return MIATTN_OK;
  const int kcap = miattn::varlen_list_cap(total, 128, nseq);
  int* kl = (int*)scratch.get((size_t)(2 + 2 * (long long)kcap) * 4);
  if (!kl) return fail(MIATTN_ENOMEM, "hipMallocAsync failed for the packed-batch work list");
  if ((st = launch_status(miattn::launch_varlen_tiles(p.cu_seqlens, nseq, total, 128, 0, kl, s), "work list")))
    return st;
  p.vl_ktiles = kl;
  p.vl_kcap = kcap;
  return MIATTN_OK;
}

long long bmask_bytes(int N) {
  return (long long)((N + miattn::BS_ROWS - 1) / miattn::BS_ROWS) * ((N + miattn::BS_COLS - 1) / miattn::BS_COLS);
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int d,
             int causal, float scale, void* stream, int dtype, int window, const uint8_t* bmask = nullptr) {
  int st = check_common(B, H, Hkv, N, d, dtype);
  if (st) return st;
  if ((st = check_ptrs({q, k, v, o, lse}))) return st;
  if (causal != 0 && causal != 1) return fail(MIATTN_EINVAL, "causal must be 0 or 1");
  if (!std::isfinite(scale)) return fail(MIATTN_EINVAL, "scale must be finite");
  const long long qb = (long long)B * N * H * d * esize(dtype);
  const long long kb = (long long)B * N * Hkv * d * esize(dtype);
  const Range ro = span(o, qb), rl = span(lse, (long long)B * H * N * 4);
  for (Range r : {span(q, qb), span(k, kb), span(v, kb)})
    if (overlap(ro, r) || overlap(rl, r)) return fail(MIATTN_EINVAL, "o/lse must not alias q, k or v");
  if (overlap(ro, rl)) return fail(MIATTN_EINVAL, "o and lse must not overlap");
  if (bmask && (overlap(ro, span(bmask, bmask_bytes(N))) || overlap(rl, span(bmask, bmask_bytes(N)))))
    return fail(MIATTN_EINVAL, "o/lse must not alias block_mask");
  Params p = make_params(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale);
  p.window = window;
  Scratch scratch((hipStream_t)stream);
  if (bmask && (st = blocksparse_setup(p, bmask, dtype, scratch, (hipStream_t)stream))) return st;
  if ((st = launch_status(fwd_block(p, dtype, dtype == MIATTN_F32, (hipStream_t)stream), "attn_fwd"))) return st;
  return ok();
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
             int d, int causal, float scale, void* stream, int dtype) {
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, stream, dtype, 0);
}

int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                    int N, int d, int window, float scale, void* stream, int dtype) {
  if (window < 1) return fail(MIATTN_EINVAL, "window must be >= 1");
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, 1, scale, stream, dtype, window);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens,
                    int nseq, int max_len, int total, int H, int Hkv, int d, int causal, int window, float scale,
                    void* stream, int dtype) {
  int st = check_common(1, H, Hkv, total, d, dtype);
  if (st) return st;
  if (nseq < 1 || nseq > 65535) return fail(MIATTN_EINVAL, "nseq must be in [1, 65535]");
  if (max_len < 1 || max_len > total) return fail(MIATTN_EINVAL, "max_len must be in [1, total]");
  if ((st = check_ptrs({q, k, v, o, lse}))) return st;
  if (!cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return fail(MIATTN_EINVAL, "cu_seqlens must be a non-null, 4-byte aligned device pointer");
  if (causal != 0 && causal != 1) return fail(MIATTN_EINVAL, "causal must be 0 or 1");
  if (window < 0 || (window > 0 && !causal)) return fail(MIATTN_EINVAL, "window must be 0, or >= 1 with causal");
  if (!std::isfinite(scale)) return fail(MIATTN_EINVAL, "scale must be finite");
  const long long qb = (long long)total * H * d * esize(dtype), kb = (long long)total * Hkv * d * esize(dtype);
  const Range ro = span(o, qb), rl = span(lse, (long long)H * total * 4);
  for (Range r : {span(q, qb), span(k, kb), span(v, kb)})
    if (overlap(ro, r) || overlap(rl, r)) return fail(MIATTN_EINVAL, "o/lse must not alias q, k or v");
  if (overlap(ro, rl)) return fail(MIATTN_EINVAL, "o and lse must not overlap");
  const Range rcu = span(cu_seqlens, (long long)(nseq + 1) * 4);
  if (overlap(ro, rcu) || overlap(rl, rcu)) return fail(MIATTN_EINVAL, "o/lse must not alias cu_seqlens");
  Params p = make_params(q, k, v, o, lse, nseq, H, Hkv, total, d, causal, scale);
  p.Nq = p.Nk = max_len;       // grid extent; each workgroup narrows to its sequence
  p.window = window;
  p.cu_seqlens = cu_seqlens;
  hipStream_t s = (hipStream_t)stream;
  Scratch scratch(s);
  if (dtype == MIATTN_BF16 && (st = varlen_lists(p, scratch, false, s))) return st;
  if ((st = launch_status(fwd_block(p, dtype, dtype == MIATTN_F32, s), "attn_fwd_varlen"))) return st;
  return ok();
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const int* cu_seqlens, int nseq, int max_len, int total, int H, int Hkv, int d, int causal,
                    int window, float scale, void* stream, const void* dout, void* dq, void* dk, void* dv,
                    int dtype, int accumulate) {
  int st = check_common(1, H, Hkv, total, d, dtype);
  if (st) return st;
  if (nseq < 1 || nseq > 65535) return fail(MIATTN_EINVAL, "nseq must be in [1, 65535]");
  if (max_len < 1 || max_len > total) return fail(MIATTN_EINVAL, "max_len must be in [1, total]");
  if ((st = check_ptrs({q, k, v, o, lse, dout, dq, dk, dv}))) return st;
  if (!cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return fail(MIATTN_EINVAL, "cu_seqlens must be a non-null, 4-byte aligned device pointer");
  if (causal != 0 && causal != 1) return fail(MIATTN_EINVAL, "causal must be 0 or 1");
  if (window < 0 || (window > 0 && !causal)) return fail(MIATTN_EINVAL, "window must be 0, or >= 1 with causal");
  if (accumulate != 0 && accumulate != 1) return fail(MIATTN_EINVAL, "accumulate must be 0 or 1");
  if (!std::isfinite(scale)) return fail(MIATTN_EINVAL, "scale must be finite");
  const size_t ge = accumulate ? 4 : esize(dtype);
  const long long qb = (long long)total * H * d * esize(dtype), kb = (long long)total * Hkv * d * esize(dtype);
  const Range rdq = span(dq, (long long)total * H * d * ge), rdk = span(dk, (long long)total * Hkv * d * ge),
              rdv = span(dv, (long long)total * Hkv * d * ge);
  for (Range out : {rdq, rdk, rdv})
    for (Range in : {span(q, qb), span(k, kb), span(v, kb), span(o, qb), span(dout, qb),
                     span(lse, (long long)H * total * 4)})
      if (overlap(out, in)) return fail(MIATTN_EINVAL, "dq/dk/dv must not alias an input");
  if (overlap(rdq, rdk) || overlap(rdq, rdv) || overlap(rdk, rdv))
    return fail(MIATTN_EINVAL, "dq, dk and dv must not overlap");
  const Range rcu = span(cu_seqlens, (long long)(nseq + 1) * 4);
  if (overlap(rdq, rcu) || overlap(rdk, rcu) || overlap(rdv, rcu))
    return fail(MIATTN_EINVAL, "dq/dk/dv must not alias cu_seqlens");
  hipStream_t s = (hipStream_t)stream;
  Scratch scratch(s);
  float* dsum = (float*)scratch.get((size_t)H * total * 4);
  if (!dsum) return fail(MIATTN_ENOMEM, "hipMallocAsync failed for the rowsum vector");
  Params p = make_params(q, k, v, const_cast<void*>(o), const_cast<float*>(lse), nseq, H, Hkv, total, d, causal,
                         scale);
  p.Nq = p.Nk = max_len;
  p.window = window;
  p.cu_seqlens = cu_seqlens;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dsum = dsum;
  p.accumulate = accumulate;
  p.acc_q = p.acc_kv = accumulate;
  if (dtype == MIATTN_BF16) {
    if ((st = varlen_lists(p, scratch, true, s))) return st;
    // D = rowsum(dout * o) formed by the dQ kernel, for every row of a sequence
    p.fuse_dsum = 1;
    if ((st = launch_status(miattn::launch_bwd_dq_mfma(p, s), "attn_bwd_varlen dQ"))) return st;
    if ((st = launch_status(miattn::launch_bwd_dkdv_mfma(p, s), "attn_bwd_varlen dK/dV"))) return st;
    return ok();
  }
  // rowsum(dout * o) is per token: the packed rows as one sequence
  if ((st = launch_status(miattn::launch_bwd_pre(o, dout, dsum, 1, H, total, d, 0, total, dtype, s),
                          "bwd preprocess")))
    return st;
  if ((st = launch_status(bwd_block(p, dtype, s), "attn_bwd_varlen"))) return st;
  return ok();
}

int attn_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, const int* k_lens, void* o,
                     float* lse, int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale, int nsplit,
                     void* stream, int dtype) {
  int st = check_common(B, H, Hkv, Nk, d, dtype);
  if (st) return st;
  if (Nq < 1) return fail(MIATTN_EINVAL, "Nq must be >= 1");
  if ((long long)B * H * Nq >= (1LL << 31) || (long long)(Nq + 64) * H * d >= (1LL << 31))
    return fail(MIATTN_EUNSUPPORTED, "problem too large for 32-bit row indexing");
  if (dtype != MIATTN_BF16) return fail(MIATTN_EUNSUPPORTED, "attn_fwd_kvcache supports MIATTN_BF16 only");
  if ((st = check_ptrs({q, k_cache, v_cache, o, lse}))) return st;
  if (k_lens && (reinterpret_cast<uintptr_t>(k_lens) & 3u)) return fail(MIATTN_EINVAL, "k_lens not 4-byte aligned");
  if (causal != 0 && causal != 1) return fail(MIATTN_EINVAL, "causal must be 0 or 1");
  if (!std::isfinite(scale)) return fail(MIATTN_EINVAL, "scale must be finite");
  if (nsplit < 0 || nsplit > 1024) return fail(MIATTN_EINVAL, "nsplit must be in [0, 1024]");
  const long long qb = (long long)B * Nq * H * d * 2, kb = (long long)B * Nk * Hkv * d * 2;
  const Range ro = span(o, qb), rl = span(lse, (long long)B * H * Nq * 4);
  for (Range r : {span(q, qb), span(k_cache, kb), span(v_cache, kb)})
    if (overlap(ro, r) || overlap(rl, r)) return fail(MIATTN_EINVAL, "o/lse must not alias q, k_cache or v_cache");
  if (overlap(ro, rl)) return fail(MIATTN_EINVAL, "o and lse must not overlap");

  const int G = H / Hkv;
  const int rbs = (Nq * G + 31) / 32;           // blocks of 32 rows per K/V head group
  hipStream_t s = (hipStream_t)stream;
  Scratch scratch(s);
  const long long rows = (long long)B * Nq * H;
  int chunk = 0;
  long long slots;                              // partial results per row
  if (rbs == 1) {
    // Decode-shaped (one block of rows per group): balanced ranges. The
    // valid keys of all sequences form one joint range per K/V head, cut
    // into nsplit equal ranges, so every workgroup streams the same number
    // of keys whatever the length mix; by default one range per resident
    // single-wave workgroup (four per CU), each at least 256 keys.
    if (nsplit == 0) {
      int dev = 0, ncu = 256;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        ncu = 256;
      const long long most = std::max(1LL, (long long)B * Nk / 256);
      nsplit = (int)std::max(1LL, std::min({(long long)4 * ncu / Hkv, most, 1024LL}));
    }
    slots = (long long)nsplit + B;
  } else {
    // Larger groups: nsplit equal chunks of every sequence, enough workgroups
    // to keep every CU busy (about 2048 single-wave equivalents), each chunk
    // at least 256 keys and a multiple of the 32-key tile. (Balanced ranges
    // were measured here too: they even out the split kernel, but ranges that
    // straddle sequences leave each row more partials, and the merge then
    // costs more than the split kernel saves.)
    const long long groups = (long long)B * Hkv * rbs;
    if (nsplit == 0) {
      const long long want = (2048 + groups - 1) / groups;
      const long long most = (Nk + 255) / 256;
      nsplit = (int)std::max(1LL, std::min(want, most));
    }
    chunk = (Nk + nsplit - 1) / nsplit;
    chunk = (chunk + 31) / 32 * 32;
    nsplit = (Nk + chunk - 1) / chunk;     // no empty trailing split
    slots = (long long)nsplit * B;
  }
  float* o_part = (float*)scratch.get((size_t)(slots * rows / B) * d * 4);
  float* lse_part = (float*)scratch.get((size_t)(slots * rows / B) * 4);
  if (!o_part || !lse_part) return fail(MIATTN_ENOMEM, "hipMallocAsync failed for the split partials");
  miattn::SplitParams p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.k_lens = k_lens;
  p.o = o;
  p.lse = lse;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.B = B;
  p.H = H;
  p.Hkv = Hkv;
  p.G = G;
  p.Nq = Nq;
  p.Nk = Nk;
  p.d = d;
  p.causal = causal;
  p.scale = scale;
  p.nsplit = nsplit;
  p.chunk = chunk;
  p.balanced = rbs == 1;
  if ((st = launch_status(miattn::launch_fwd_split(p, s), "attn_fwd_kvcache"))) return st;
  return ok();
}

}  // extern "C"

namespace {

// fixed_dsum: a caller-provided rowsum buffer of at least B * H * N floats;
// then the call takes no scratch from the per-stream buffer and allocates
// nothing (bmask must be null).
int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H, int Hkv,
             int N, int d, int causal, float scale, void* stream, const void* dout, void* dq, void* dk, void* dv,
             int dtype, int accumulate, void* const* marks, int window, const uint8_t* bmask = nullptr,
             float* fixed_dsum = nullptr) {
  int st = check_common(B, H, Hkv, N, d, dtype);
  if (st) return st;
  if ((st = check_ptrs({q, k, v, o, lse, dout, dq, dk, dv}))) return st;
  if (causal != 0 && causal != 1) return fail(MIATTN_EINVAL, "causal must be 0 or 1");
  if (accumulate != 0 && accumulate != 1) return fail(MIATTN_EINVAL, "accumulate must be 0 or 1");
  if (!std::isfinite(scale)) return fail(MIATTN_EINVAL, "scale must be finite");
  const size_t ge = accumulate ? 4 : esize(dtype);
  const long long qb = (long long)B * N * H * d * esize(dtype), kb = (long long)B * N * Hkv * d * esize(dtype);
  const Range rdq = span(dq, (long long)B * N * H * d * ge), rdk = span(dk, (long long)B * N * Hkv * d * ge),
              rdv = span(dv, (long long)B * N * Hkv * d * ge);
  for (Range out : {rdq, rdk, rdv})
    for (Range in : {span(q, qb), span(k, kb), span(v, kb), span(o, qb), span(dout, qb),
                     span(lse, (long long)B * H * N * 4)})
      if (overlap(out, in)) return fail(MIATTN_EINVAL, "dq/dk/dv must not alias an input");
  if (overlap(rdq, rdk) || overlap(rdq, rdv) || overlap(rdk, rdv))
    return fail(MIATTN_EINVAL, "dq, dk and dv must not overlap");
  if (bmask)
    for (Range out : {rdq, rdk, rdv})
      if (overlap(out, span(bmask, bmask_bytes(N)))) return fail(MIATTN_EINVAL, "dq/dk/dv must not alias block_mask");

  hipStream_t s = (hipStream_t)stream;
  std::optional<Scratch> scratch;
  float* dsum = fixed_dsum;
  if (!dsum) {
    scratch.emplace(s);
    dsum = (float*)scratch->get((size_t)B * H * N * 4);
    if (!dsum) return fail(MIATTN_ENOMEM, "hipMallocAsync failed for the rowsum vector");
  }
  Params p = make_params(q, k, v, const_cast<void*>(o), const_cast<float*>(lse), B, H, Hkv, N, d, causal, scale);
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dsum = dsum;
  p.accumulate = accumulate;
  p.acc_q = p.acc_kv = accumulate;
  p.window = window;
  if (bmask && (!scratch || (st = blocksparse_setup(p, bmask, dtype, *scratch, s))))
    return st ? st : fail(MIATTN_EINVAL, "block masks need library scratch");
  if (dtype == MIATTN_BF16) {
    // the dQ kernel also forms D = rowsum(dout * o) of its rows and writes
    // it; the dK/dV kernel, which reads D, runs after it
    p.fuse_dsum = 1;
    if ((st = launch_status(miattn::launch_bwd_dq_mfma(p, s), "attn_bwd dQ"))) return st;
    if (marks && (st = launch_status(hipEventRecord((hipEvent_t)marks[0], s), "timing mark 0"))) return st;
    if ((st = launch_status(miattn::launch_bwd_dkdv_mfma(p, s), "attn_bwd dK/dV"))) return st;
    if (marks && (st = launch_status(hipEventRecord((hipEvent_t)marks[1], s), "timing mark 1"))) return st;
  } else {
    if ((st = launch_status(miattn::launch_bwd_pre(o, dout, dsum, B, H, N, d, 0, N, dtype, s), "bwd preprocess")))
      return st;
    if (marks && (st = launch_status(hipEventRecord((hipEvent_t)marks[0], s), "timing mark 0"))) return st;
    if ((st = launch_status(bwd_block(p, dtype, s), "attn_bwd"))) return st;
    if (marks && (st = launch_status(hipEventRecord((hipEvent_t)marks[1], s), "timing mark 1"))) return st;
  }
  return ok();
}

// ---- attn_bwd_noalloc: the rowsum vector in a fixed device array

// Rows (B * H * N) the fixed array holds: 16 MiB of float32 per device,
// enough for a [B, H, N] rowsum vector of 4M rows (the 64K-row, 32-head
// workload needs 2M).
constexpr long long kNoallocRows = 1LL << 22;

// One copy per device, held from the library's load to the end of the
// process. Host code never uses this name as an address (on the host it is
// only a stand-in for the device symbol): kernels get the device address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[kNoallocRows];

constexpr int kMaxDevices = 64;
std::mutex noalloc_mu;
float* noalloc_addr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) into *out; returns a status.
int noalloc_scratch(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MIATTN_ELAUNCH, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MIATTN_EUNSUPPORTED, "attn_bwd_noalloc supports device indices below 64");
  std::lock_guard<std::mutex> g(noalloc_mu);
  if (!noalloc_addr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(MIATTN_ELAUNCH, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    noalloc_addr[dev] = (float*)ptr;
  }
  *out = noalloc_addr[dev];
  return MIATTN_OK;
}

}  // namespace

extern "C" {

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
                     int Hkv, int N, int d, int causal, float scale, void* stream, const void* dout, void* dq,
                     void* dk, void* dv, int dtype, int accumulate) {
  int st = check_common(B, H, Hkv, N, d, dtype);
  if (st) return st;
  if ((long long)B * H * N > kNoallocRows)
    return fail(MIATTN_EINVAL, "attn_bwd_noalloc: B * H * N = " + std::to_string((long long)B * H * N) +
                                   " exceeds the fixed scratch of " + std::to_string(kNoallocRows) + " rows");
  float* dsum = nullptr;
  if ((st = noalloc_scratch(&dsum))) return st;
  return bwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, stream, dout, dq, dk, dv, dtype, accumulate,
                  nullptr, 0, nullptr, dsum);
}

int attn_bwd_timed(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
                   int Hkv, int N, int d, int causal, float scale, void* stream, const void* dout, void* dq,
                   void* dk, void* dv, int dtype, int accumulate, void* const* marks) {
  return bwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, stream, dout, dq, dk, dv, dtype, accumulate,
                  marks, 0);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
             int Hkv, int N, int d, int causal, float scale, void* stream, const void* dout, void* dq, void* dk,
             void* dv, int dtype, int accumulate) {
  return bwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, stream, dout, dq, dk, dv, dtype, accumulate,
                  nullptr, 0);
}

int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
                    int Hkv, int N, int d, int window, float scale, void* stream, const void* dout, void* dq,
                    void* dk, void* dv, int dtype, int accumulate) {
  if (window < 1) return fail(MIATTN_EINVAL, "window must be >= 1");
  return bwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, 1, scale, stream, dout, dq, dk, dv, dtype, accumulate,
                  nullptr, window);
}

int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                         const unsigned char* block_mask, int B, int H, int Hkv, int N, int d, int causal,
                         float scale, void* stream, int dtype) {
  if (!block_mask) return fail(MIATTN_EINVAL, "block_mask must not be null");
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, stream, dtype, 0, block_mask);
}

int attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const unsigned char* block_mask, int B, int H, int Hkv, int N, int d, int causal,
                         float scale, void* stream, const void* dout, void* dq, void* dk, void* dv, int dtype,
                         int accumulate) {
  if (!block_mask) return fail(MIATTN_EINVAL, "block_mask must not be null");
  return bwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, stream, dout, dq, dk, dv, dtype, accumulate,
                  nullptr, 0, block_mask);
}

int attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o, float* lse, int B,
               int H, int N, int d, int dtype, void* stream) {
  int st = check_common(B, H, H, N, d, dtype);
  if (st) return st;
  if ((st = check_ptrs({o_a, lse_a, o_b, lse_b, o, lse}))) return st;
  // in place means exactly in place: an output may equal an input of its own
  // kind (each element is read before the same thread writes it) but must not
  // overlap any input at another offset, nor the other output
  const long long ob = (long long)B * N * H * d * esize(dtype), lb = (long long)B * H * N * 4;
  const Range ro = span(o, ob), rl = span(lse, lb);
  const Range roa = span(o_a, ob), rob = span(o_b, ob), rla = span(lse_a, lb), rlb = span(lse_b, lb);
  if ((o != o_a && overlap(ro, roa)) || (o != o_b && overlap(ro, rob)) || overlap(ro, rla) || overlap(ro, rlb))
    return fail(MIATTN_EINVAL, "o must equal o_a or o_b or overlap no input");
  if ((lse != lse_a && overlap(rl, rla)) || (lse != lse_b && overlap(rl, rlb)) || overlap(rl, roa) ||
      overlap(rl, rob))
    return fail(MIATTN_EINVAL, "lse must equal lse_a or lse_b or overlap no input");
  if (overlap(ro, rl)) return fail(MIATTN_EINVAL, "o and lse must not overlap");
  const int t = dtype == MIATTN_BF16 ? 1 : 0;
  if ((st = launch_status(miattn::launch_merge(o_a, lse_a, o_b, lse_b, o, lse, B, H, N, d, 0, N, t, t, t,
                                               (hipStream_t)stream),
                          "attn_merge")))
    return st;
  return ok();
}

int attn_fwd_chunked(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
                     int d, float scale, void* stream, int dtype, int nchunks) {
  int st = check_common(B, H, Hkv, N, d, dtype);
  if (st) return st;
  if ((st = check_ptrs({q, k, v, o, lse}))) return st;
  if (!std::isfinite(scale)) return fail(MIATTN_EINVAL, "scale must be finite");
  if (nchunks < 1 || N % nchunks != 0 || (nchunks > 1 && nchunks % 2 != 0))
    return fail(MIATTN_EINVAL, "nchunks must be 1 or an even divisor of N");
  const long long qb = (long long)B * N * H * d * esize(dtype), kb = (long long)B * N * Hkv * d * esize(dtype);
  const Range ro = span(o, qb), rl = span(lse, (long long)B * H * N * 4);
  for (Range r : {span(q, qb), span(k, kb), span(v, kb)})
    if (overlap(ro, r) || overlap(rl, r)) return fail(MIATTN_EINVAL, "o/lse must not alias q, k or v");

  hipStream_t s = (hipStream_t)stream;
  const int R = N / nchunks;
  const long long no = (long long)B * N * H * d, nl = (long long)B * H * N;
  Scratch scratch(s);
  // running (merged-so-far) result per query chunk; the float32 path also
  // keeps one partial per pair for the merge kernel (the bf16 forward kernel
  // merges into the running result in its epilogue)
  const bool fused = dtype == MIATTN_BF16;
  float* run_o = (float*)scratch.get(no * 4);
  float* run_l = (float*)scratch.get(nl * 4);
  float* part_o = fused ? nullptr : (float*)scratch.get(no * 4);
  float* part_l = fused ? nullptr : (float*)scratch.get(nl * 4);
  if (!run_o || !run_l || (!fused && (!part_o || !part_l)))
    return fail(MIATTN_ENOMEM, "hipMallocAsync failed for chunk partials");

  std::vector<int> done(nchunks, 0);   // pairs merged into each query chunk so far
  for (const auto& round : balanced_rounds(nchunks)) {
    for (const auto& pr : round) {
      const int i = pr.first, j = pr.second;
      const bool last = done[i] == i;   // the query chunk's final pair
      Params p = make_params(q, k, v, nullptr, nullptr, B, H, Hkv, N, d, i == j, scale);
      p.Nq = R;
      p.Nk = R;
      p.q_start = i * R;
      p.k_start = j * R;
      if (done[i] == 0 && last) {
        // a single pair (query chunk 0): write the result directly
        p.o = o;
        p.lse = lse;
        if ((st = launch_status(fwd_block(p, dtype, dtype == MIATTN_F32, s), "chunk forward"))) return st;
      } else if (done[i] == 0) {
        p.o = run_o;
        p.lse = run_l;
        if ((st = launch_status(fwd_block(p, dtype, true, s), "chunk forward"))) return st;
      } else if (fused) {
        // this pair merged into the running result by the forward kernel
        p.mrg_o = run_o;
        p.mrg_lse = run_l;
        p.o = last ? o : (void*)run_o;
        p.lse = last ? lse : run_l;
        if ((st = launch_status(miattn::launch_fwd_mfma(p, !last, s), "chunk forward"))) return st;
      } else {
        p.o = part_o;
        p.lse = part_l;
        if ((st = launch_status(fwd_block(p, dtype, true, s), "chunk forward"))) return st;
        const int tout = last ? (dtype == MIATTN_BF16 ? 1 : 0) : 0;
        void* dst_o = last ? o : (void*)run_o;
        float* dst_l = last ? lse : run_l;
        if ((st = launch_status(miattn::launch_merge(run_o, run_l, part_o, part_l, dst_o, dst_l, B, H, N, d, i * R,
                                                     R, 0, 0, tout, s),
                                "chunk merge")))
          return st;
      }
      done[i] += 1;
    }
  }
  return ok();
}

int attn_bwd_chunked(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
                     int Hkv, int N, int d, float scale, void* stream, const void* dout, void* dq, void* dk, void* dv,
                     int dtype, int nchunks) {
  int st = check_common(B, H, Hkv, N, d, dtype);
  if (st) return st;
  if ((st = check_ptrs({q, k, v, o, lse, dout, dq, dk, dv}))) return st;
  if (!std::isfinite(scale)) return fail(MIATTN_EINVAL, "scale must be finite");
  if (nchunks < 1 || N % nchunks != 0 || (nchunks > 1 && nchunks % 2 != 0))
    return fail(MIATTN_EINVAL, "nchunks must be 1 or an even divisor of N");
  const long long qb = (long long)B * N * H * d * esize(dtype), kb = (long long)B * N * Hkv * d * esize(dtype);
  const Range rdq = span(dq, qb), rdk = span(dk, kb), rdv = span(dv, kb);
  for (Range out : {rdq, rdk, rdv})
    for (Range in : {span(q, qb), span(k, kb), span(v, kb), span(o, qb), span(dout, qb),
                     span(lse, (long long)B * H * N * 4)})
      if (overlap(out, in)) return fail(MIATTN_EINVAL, "dq/dk/dv must not alias an input");

  hipStream_t s = (hipStream_t)stream;
  const int R = N / nchunks;
  const long long nq = (long long)B * N * H * d, nk = (long long)B * N * Hkv * d;
  Scratch scratch(s);
  float* dsum = (float*)scratch.get((size_t)B * H * N * 4);
  float* aq = (float*)scratch.get(nq * 4);
  float* ak = (float*)scratch.get(nk * 4);
  float* av = (float*)scratch.get(nk * 4);
  if (!dsum || !aq || !ak || !av) return fail(MIATTN_ENOMEM, "hipMallocAsync failed for gradient accumulators");
  // bf16: the matrix-core kernels keep the per-chunk float32 sums themselves
  // (the first pair of a chunk stores, later ones add, the last one adds and
  // writes the bf16 result); float32: zeroed accumulators, added into by
  // every pair, converted at the end
  const bool fused = dtype == MIATTN_BF16;
  if (!fused) {
    if ((st = launch_status(miattn::launch_fill(aq, nq, 0.f, s), "clear"))) return st;
    if ((st = launch_status(miattn::launch_fill(ak, nk, 0.f, s), "clear"))) return st;
    if ((st = launch_status(miattn::launch_fill(av, nk, 0.f, s), "clear"))) return st;
  }
  if ((st = launch_status(miattn::launch_bwd_pre(o, dout, dsum, B, H, N, d, 0, N, dtype, s), "bwd preprocess")))
    return st;
  // pairs seen so far per query chunk (i + 1 in all) and per key chunk (nchunks - j)
  std::vector<int> seen_q(nchunks, 0), seen_k(nchunks, 0);
  auto mode = [](int seen, int total) {
    return total == 1 ? miattn::ACC_STORE
                      : seen == 0 ? miattn::ACC_FIRST : seen == total - 1 ? miattn::ACC_LAST : miattn::ACC_ADD;
  };
  for (const auto& round : balanced_rounds(nchunks)) {
    for (const auto& pr : round) {
      const int i = pr.first, j = pr.second;
      Params p = make_params(q, k, v, const_cast<void*>(o), const_cast<float*>(lse), B, H, Hkv, N, d, i == j, scale);
      p.Nq = R;
      p.Nk = R;
      p.q_start = i * R;
      p.k_start = j * R;
      p.dout = dout;
      p.dq = aq;
      p.dk = ak;
      p.dv = av;
      p.dsum = dsum;
      p.accumulate = 1;
      if (fused) {
        p.acc_q = mode(seen_q[i]++, i + 1);
        p.acc_kv = mode(seen_k[j]++, nchunks - j);
        p.q_part = aq;
        p.k_part = ak;
        p.v_part = av;
        if (p.acc_q == miattn::ACC_STORE || p.acc_q == miattn::ACC_LAST) p.dq = dq;
        if (p.acc_kv == miattn::ACC_STORE || p.acc_kv == miattn::ACC_LAST) {
          p.dk = dk;
          p.dv = dv;
        }
        if ((st = launch_status(miattn::launch_bwd_mfma(p, s), "chunk backward"))) return st;
      } else {
        p.acc_q = p.acc_kv = miattn::ACC_ADD;
        if ((st = launch_status(bwd_block(p, dtype, s), "chunk backward"))) return st;
      }
    }
  }
  if (!fused) {
    if ((st = launch_status(miattn::launch_convert(aq, dq, nq, dtype, s), "dq convert"))) return st;
    if ((st = launch_status(miattn::launch_convert(ak, dk, nk, dtype, s), "dk convert"))) return st;
    if ((st = launch_status(miattn::launch_convert(av, dv, nk, dtype, s), "dv convert"))) return st;
  }
  return ok();
}

}  // extern "C"
