// Host-side view of the libfa355 kernels: argument blocks and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa355.h"

namespace fa {

// Arguments of the prefill kernel (fixed-length and packed variants).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;              // may be null
  const int32_t* seqlens_k;  // fixed-length: optional per-batch key count
  const int32_t* cu_q;     // varlen: [nseq + 1]
  const int32_t* cu_k;
  const int32_t* sched;    // varlen: schedule written by the schedule kernel
  int nseq;                // varlen: number of sequences
  int B, H, Nq, Nk;        // fixed-length sizes
  int nqb;                 // fixed-length: query blocks per (batch, head)
  int total_q;             // varlen: lse row stride
  float c;                 // scale * log2(e)
  // mask families (16-bit prefill only; zero / null otherwise)
  int prefix;              // with causal: keys [0, prefix) are seen by every query
  const float* alibi;      // [H] slopes: score += -slope_h * |j - (i + Lk - Lq)|
  // attention dropout (16-bit prefill only; drop_t = 0: none)
  uint32_t drop_t;         // a key is dropped when its random byte is below drop_t
  uint32_t seed_lo, seed_hi;
  float drop_scale;        // 256 / (256 - drop_t)
  // set by the launcher: the whole grid is resident at once (one round of
  // workgroups), so waves take priority by their remaining work
  int tail_prio;
};

// Query rows per workgroup of the prefill kernel instance chosen for (dtype, D).
int fwd_block_rows(fa_dtype_t dtype, int D);

// Fixed-length grid: B * H * ceil(Nq / rows); varlen grid: H * max_tiles.
hipError_t launch_fwd(const FwdArgs& a, fa_dtype_t dtype, int D, bool causal, bool varlen,
                      unsigned grid, hipStream_t stream);

// Varlen schedule, written by one small kernel into the caller's workspace:
//   sched[0]                 number of tiles T
//   sched[2 + 4s .. 5 + 4s]  sequence s: first q row, q rows, first k row, k rows
//                            (clamped to [0, total_q] / [0, total_k])
//   sched[2 + 4*nseq + 2t]   tile t: sequence, query block; tiles sequence by
//                            sequence, each sequence's longest first
hipError_t launch_varlen_schedule(const int32_t* cu_q, const int32_t* cu_k, int nseq,
                                  int total_q, int total_k, int rows, int causal, int max_tiles,
                                  int32_t* sched, hipStream_t stream);

// Device address of the static schedule scratch of the current device
// (FA_NOALLOC_SCRATCH_BYTES bytes), looked up once per device.
hipError_t noalloc_scratch(void** ptr);

// Upper bound on the number of (sequence, query block) tiles.
inline long long varlen_max_tiles(int nseq, int total_q, int rows) {
  return ((long long)total_q + rows - 1) / rows + nseq;
}
inline size_t varlen_sched_bytes(int nseq, long long max_tiles) {
  size_t n = 2 + 4 * (size_t)nseq + 2 * (size_t)max_tiles;
  return (n * 4 + 255) / 256 * 256;
}

struct DecodeArgs {
  const void* q;
  const void* kc;
  const void* vc;
  void* o;
  float* lse;
  const int32_t* seqlens_k;
  float* ws_o;     // [B, H, NC, D]
  float* ws_ml;    // [B, H, NC, 2]
  int B, H, Nk_max, NC, chunk;
  float c;
  // paged cache (block_table == nullptr: contiguous [B, Nk_max, H, D] caches)
  const int32_t* block_table;  // [B, max_pages]
  int page_shift, num_pages, max_pages;
};

hipError_t launch_decode(const DecodeArgs& a, fa_dtype_t dtype, int D, hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;        // [B, H, Nq]
  float* delta;            // workspace [B, H, Nq]: -rowsum(dO * O)
  float* lse2;             // workspace, delta's layout: lse * log2 e (+inf: no visible key)
  void* dq;
  void* dk;
  void* dv;
  const int32_t* seqlens_k;
  int B, H, Nq, Nk;
  int nqb;                 // query blocks of bwd_block_rows() rows
  float c;                 // scale * log2(e)
  float scale;
  // attention dropout of the forward being differentiated (drop_t = 0: none)
  uint32_t drop_t;
  uint32_t seed_lo, seed_hi;
  float drop_scale;        // 256 / (256 - drop_t)
  // mask families of the forward being differentiated (zero / null: none)
  int prefix;              // with causal: keys [0, prefix) are seen by every query
  const float* alibi;      // [H] slopes: score += -slope_h * |j - (i + Lk - Lq)|
  // packed variable-length batches (cu_q null: fixed length).  Then B is the
  // number of sequences, Nq / Nk the longest query / key lengths, lse and
  // delta are [H, total_q] and the tensors [total, H, D].
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
};

int bwd_block_rows();
// delta, then dK/dV, then dQ, all on `stream`
hipError_t launch_bwd(const BwdArgs& a, fa_dtype_t dtype, int D, bool causal, hipStream_t stream);

}  // namespace fa
