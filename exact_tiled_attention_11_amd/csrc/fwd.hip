// Prefill kernel of libfa355: exact attention, one workgroup per block of
// query rows, keys and values streamed through LDS in tiles, online softmax.
//
// The method is the tiled computation the Ascend CANN ops-transformer
// FlashAttention explainer lays out in section 原理 (principle): split Q, K
// and V along the sequence (step 1); for each Q block visit the K blocks and
// form scores (step 2); keep a running maximum m and running sum l per row
// while doing so (step 3, online softmax); and accumulate the output block
// from the probabilities and the V block (step 4).  The rescaling of an old
// partial result by exp(m_old - m_new) is the pairwise merge of the CSDN
// primer 轻松读懂FlashAttention 上, section Softmax求解重构.  Fused into one
// kernel, the N x N scores and probabilities live only in registers (the
// primer's section 内存卡点 on kernel fusion).
//
// gfx950 mapping (ours, not the pages'):
//  * Each wave owns QB blocks of 32 query rows.  Scores are computed
//    transposed, S^T = K Q^T, on the 32x32 MFMA: lane l then holds one query
//    (column l%32) and 16 keys per 32-key block, so row maxima and sums are
//    in-lane plus one exchange between the two 32-lane halves.
//  * Q stays in VGPRs as the MFMA B operand for the whole kernel.
//  * K and V tiles of KB*32 keys are double-buffered in LDS with an XOR
//    swizzle over 16-byte chunks; the next tile's global loads are issued
//    before the current tile's math.
//  * The output is accumulated transposed too, O^T += V^T P^T: the
//    probabilities never leave registers (they are the B operand as
//    computed), and V^T fragments come from LDS with the gfx950
//    transposing read ds_read_b64_tr_b16.
//  * Causal tiles wholly above the diagonal are never loaded; a wave whose
//    rows cannot see a tile skips its math; only diagonal and tail tiles
//    evaluate the mask.  Causal query blocks are issued longest first.
//  * exp is taken as exp2 with scale*log2(e) folded into one FMA.

#include <math.h>

#include "fa_device.h"
#include "launch.h"

namespace fa {

template <typename T, int D, int QB, int KB, int NW>
struct FwdCfg {
  static constexpr int kQW = 32 * QB;          // query rows per wave
  static constexpr int kBR = NW * kQW;         // query rows per workgroup
  static constexpr int kBC = 32 * KB;          // keys per tile
  static constexpr int kNT = NW * 64;          // threads per workgroup
  static constexpr int kES = Elem<T>::kBytes;
  static constexpr int kRowB = D * kES;        // bytes of one K or V row
  static constexpr int kCPR = kRowB / 16;      // 16-byte chunks per row
  static constexpr int kTileB = kBC * kRowB;   // bytes of one K or V tile
  static constexpr int kCPT = kBC * kCPR / kNT;  // chunks per thread per tile
  static_assert(kBC * kCPR % kNT == 0, "tile chunks must divide evenly over threads");
  static_assert(kCPR >= 8, "swizzle needs at least 8 chunks per row");
};

// LDS position (in 16-byte chunks) of chunk c of tile row r.  For 16-bit
// types the XOR pattern makes both the 8-row column reads of K and the
// 4-row x 32-byte transposing reads of V conflict-free; for fp32 it spreads
// the 32-row column reads over 16 chunk positions.
template <int CPR, bool F32>
__device__ __forceinline__ int swz(int r, int c) {
  const int f = F32 ? (r & 15) : (((r & 3) << 1) | ((r >> 2) & 1));
  return r * CPR + (c ^ f);
}

template <typename T, int D, int QB, int KB, int NW, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NW * 64, 2) void fwd_kernel(FwdArgs a) {
  using C = FwdCfg<T, D, QB, KB, NW>;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr bool F32 = (E::kBytes == 4);
  constexpr int KS = D / E::kStep;        // MFMA steps over head_dim
  constexpr int DB = D / 32;              // 32-wide blocks of head_dim
  constexpr int TS = 32 / E::kStep;       // MFMA steps over a 32-key block

  __shared__ u32x4_t smem[4 * C::kTileB / 16];   // [buffer][K, V][tile]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int hh = lane >> 5;

  // ---- which (sequence, head, query block) this workgroup computes ----
  int h, qblk, lq, lk;
  long long q_tok0, k_tok0, lse_base;
  if constexpr (!VARLEN) {
    const int nbh = a.B * a.H;
    const int level = blockIdx.x / nbh;
    const int bh = blockIdx.x - level * nbh;
    qblk = CAUSAL ? (a.nqb - 1 - level) : level;
    const int b = bh / a.H;
    h = bh - b * a.H;
    lq = a.Nq;
    lk = a.Nk;
    if (a.seqlens_k) lk = min(max(a.seqlens_k[b], 0), a.Nk);
    q_tok0 = (long long)b * a.Nq;
    k_tok0 = (long long)b * a.Nk;
    lse_base = ((long long)b * a.H + h) * a.Nq;
  } else {
    const int t = blockIdx.x / a.H;
    h = blockIdx.x - t * a.H;
    if (t >= a.sched[0]) return;  // whole workgroup leaves together
    const int* tl = a.sched + 2 + 4 * a.nseq + 2 * t;
    const int s = tl[0];
    qblk = tl[1];
    const int* sq = a.sched + 2 + 4 * s;
    q_tok0 = sq[0];
    lq = sq[1];
    k_tok0 = sq[2];
    lk = sq[3];
    lse_base = (long long)h * a.total_q + q_tok0;
  }

  const int q0 = qblk * C::kBR;
  const int off = lk - lq;  // bottom-right causal alignment
  const int nkt_all = (lk + C::kBC - 1) / C::kBC;
  int nkt = nkt_all;
  if (CAUSAL) {
    const int kmax = min(q0 + C::kBR, lq) - 1 + off;
    nkt = kmax < 0 ? 0 : min(nkt_all, kmax / C::kBC + 1);
  }
  const int wq0 = q0 + wave * C::kQW;
  const int wq_last = min(wq0 + C::kQW, lq) - 1;

  const size_t rs = (size_t)a.H * D;  // elements between consecutive tokens
  const T* qp = (const T*)a.q + (size_t)q_tok0 * rs + (size_t)h * D;
  const char* kp = (const char*)((const T*)a.k + (size_t)k_tok0 * rs + (size_t)h * D);
  const char* vp = (const char*)((const T*)a.v + (size_t)k_tok0 * rs + (size_t)h * D);
  const size_t rsb = rs * sizeof(T);

  // ---- Q block of this wave, held as MFMA B operands ----
  frag qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = wq0 + qb * 32 + col;
    const bool ok = qi < lq;
    const T* row = qp + (size_t)(ok ? qi : 0) * rs;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (F32) {
        qf[qb][ks] = ok ? row[ks * 2 + hh] : 0.f;
      } else {
        frag z = {};
        qf[qb][ks] = ok ? *(const frag*)(row + ks * 16 + hh * 8) : z;
      }
    }
  }

  f32x16_t oacc[DB][QB];
  float mrow[QB], lrow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrow[qb] = -INFINITY;  // running maximum, in units of scale*log2(e)
    lrow[qb] = 0.f;        // running sum over this lane's keys
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db][qb] = f32x16_t{};
  }

  // ---- K/V tile staging: global -> registers -> LDS ----
  u32x4_t kreg[C::kCPT], vreg[C::kCPT];
  auto gload = [&](int j) {
#pragma unroll
    for (int u = 0; u < C::kCPT; ++u) {
      const int id = tid + u * C::kNT;
      const int r = id / C::kCPR, c = id % C::kCPR;
      const int key = j * C::kBC + r;
      if (key < lk) {
        kreg[u] = *(const u32x4_t*)(kp + (size_t)key * rsb + c * 16);
        vreg[u] = *(const u32x4_t*)(vp + (size_t)key * rsb + c * 16);
      } else {
        kreg[u] = u32x4_t{};  // rows past the end are zero: masked scores,
        vreg[u] = u32x4_t{};  // and no 0 * garbage in P V
      }
    }
  };
  auto sstore = [&](int buf) {
    u32x4_t* kt = smem + buf * (2 * C::kTileB / 16);
    u32x4_t* vt = kt + C::kTileB / 16;
#pragma unroll
    for (int u = 0; u < C::kCPT; ++u) {
      const int id = tid + u * C::kNT;
      const int r = id / C::kCPR, c = id % C::kCPR;
      kt[swz<C::kCPR, F32>(r, c)] = kreg[u];
      vt[swz<C::kCPR, F32>(r, c)] = vreg[u];
    }
  };

  if (nkt > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int buf = j & 1;
    if (j + 1 < nkt) gload(j + 1);
    const int k0 = j * C::kBC;
    const bool active = (wq_last >= wq0) && (!CAUSAL || k0 <= wq_last + off);
    if (active) {
      const bool need_mask = (k0 + C::kBC > lk) || (CAUSAL && k0 + C::kBC - 1 > wq0 + off);
      const char* kt = (const char*)(smem + buf * (2 * C::kTileB / 16));
      const int vt_off = buf * 2 * C::kTileB + C::kTileB;  // byte offset of the V tile

      // S^T = K Q^T for KB key blocks x QB query blocks
      f32x16_t sacc[KB][QB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int r = kb * 32 + col;
          frag kf;
          if constexpr (F32) {
            const int d = ks * 2 + hh;
            kf = *(const float*)(kt + swz<C::kCPR, F32>(r, d >> 2) * 16 + (d & 3) * 4);
          } else {
            kf = *(const frag*)(kt + swz<C::kCPR, F32>(r, ks * 2 + hh) * 16);
          }
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = mma(kf, qf[qb][ks], sacc[kb][qb]);
        }
      }

      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int qi = wq0 + qb * 32 + col;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
              if (key >= lk || (CAUSAL && key > qi + off)) sacc[kb][qb][r] = -INFINITY;
            }
          }
      }

      // online softmax: new maximum, rescale, probabilities, running sum
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
        mx = half_max(mx);
        const float tmc = (mx == -INFINITY) ? -INFINITY : mx * a.c;
        const float mnew = fmaxf(mrow[qb], tmc);
        const float ms = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = fast_exp2(mrow[qb] - ms);
        mrow[qb] = mnew;
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float s = sacc[kb][qb][r];
            float p = fast_exp2(__builtin_fmaf(s, a.c, -ms));
            if (need_mask && s == -INFINITY) p = 0.f;
            sacc[kb][qb][r] = p;
            ps += p;
          }
        lrow[qb] = lrow[qb] * alpha + ps;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
      }

      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int t = 0; t < TS; ++t) {
          frag pf[QB];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            if constexpr (F32) {
              pf[qb] = sacc[kb][qb][t];
            } else {
              u32x4_t u;
#pragma unroll
              for (int e = 0; e < 4; ++e)
                u[e] = pack2(sacc[kb][qb][8 * t + 2 * e], sacc[kb][qb][8 * t + 2 * e + 1], (T*)nullptr);
              pf[qb] = __builtin_bit_cast(frag, u);
            }
          }
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            frag vf;
            if constexpr (F32) {
              const int row = kb * 32 + 8 * (t >> 2) + 4 * hh + (t & 3);
              const int d = 32 * db + col;
              vf = *(const float*)((const char*)smem + vt_off +
                                   swz<C::kCPR, F32>(row, d >> 2) * 16 + (d & 3) * 4);
            } else {
              // lane (16g + 4jj + qq) addresses V[row0 + jj][d0 + 4qq .. +3]; the
              // transposing read hands lane (16g + i) the 4 keys at column d0 + i.
              const int g = lane >> 4, ii = lane & 15, jj = ii >> 2, qq = ii & 3;
              const int row = kb * 32 + 16 * t + 4 * hh + jj;
              const int d = 32 * db + 16 * (g & 1) + 4 * qq;
              const int b0 = vt_off + swz<C::kCPR, F32>(row, d >> 3) * 16 + (qq & 1) * 8;
              const int b1 = vt_off + swz<C::kCPR, F32>(row + 8, d >> 3) * 16 + (qq & 1) * 8;
              s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (FA_LDS(s16x4_t)*)((FA_LDS(char)*)smem + b0));
              s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (FA_LDS(s16x4_t)*)((FA_LDS(char)*)smem + b1));
              u32x4_t u = {__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                           __builtin_bit_cast(u32x2_t, hi)[0], __builtin_bit_cast(u32x2_t, hi)[1]};
              vf = __builtin_bit_cast(frag, u);
            }
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = mma(vf, pf[qb], oacc[db][qb]);
          }
        }
      }
    }
    if (j + 1 < nkt) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O / l, lse = m + ln l ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = half_sum(lrow[qb]);
    const int qi = wq0 + qb * 32 + col;
    if (qi < lq) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      T* orow = (T*)a.o + (size_t)(q_tok0 + qi) * rs + (size_t)h * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = 32 * db + 8 * g4 + 4 * hh;
          const float x0 = oacc[db][qb][4 * g4 + 0] * inv, x1 = oacc[db][qb][4 * g4 + 1] * inv;
          const float x2 = oacc[db][qb][4 * g4 + 2] * inv, x3 = oacc[db][qb][4 * g4 + 3] * inv;
          if constexpr (F32) {
            *(float4*)(orow + d) = make_float4(x0, x1, x2, x3);
          } else {
            u32x2_t u = {pack2(x0, x1, (T*)nullptr), pack2(x2, x3, (T*)nullptr)};
            *(u32x2_t*)(orow + d) = u;
          }
        }
      if (hh == 0 && a.lse)
        a.lse[lse_base + qi] = lt > 0.f ? (mrow[qb] + fast_log2(lt)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// Varlen schedule: one workgroup sorts the (sequence, query block) tiles by
// their number of key tiles, longest first (counting sort over LDS bins).
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;
constexpr int kSchedBins = 1024;

__device__ __forceinline__ int tile_keys(int qb, int rows, int key_tile, int lq, int lk, int causal) {
  const int all = (lk + key_tile - 1) / key_tile;
  if (!causal) return all;
  const int kmax = min((qb + 1) * rows, lq) - 1 + (lk - lq);
  return kmax < 0 ? 0 : min(all, kmax / key_tile + 1);
}

__global__ __launch_bounds__(kSchedThreads) void varlen_schedule_kernel(
    const int* cu_q, const int* cu_k, int nseq, int total_q, int total_k, int rows,
    int key_tile, int causal, int max_tiles, int* sched) {
  __shared__ int hist[kSchedBins];
  __shared__ int scan[kSchedBins];
  const int tid = threadIdx.x;
  int* seq = sched + 2;
  int* tiles = sched + 2 + 4 * nseq;
  for (int b = tid; b < kSchedBins; b += kSchedThreads) hist[b] = 0;
  // per-sequence bounds, clamped to the declared totals
  for (int s = tid; s < nseq; s += kSchedThreads) {
    const int q0 = min(max(cu_q[s], 0), total_q), q1 = min(max(cu_q[s + 1], q0), total_q);
    const int k0 = min(max(cu_k[s], 0), total_k), k1 = min(max(cu_k[s + 1], k0), total_k);
    seq[4 * s + 0] = q0;
    seq[4 * s + 1] = q1 - q0;
    seq[4 * s + 2] = k0;
    seq[4 * s + 3] = k1 - k0;
  }
  __syncthreads();
  for (int s = tid; s < nseq; s += kSchedThreads) {
    const int lq = seq[4 * s + 1], lk = seq[4 * s + 3];
    const int nqb = (lq + rows - 1) / rows;
    for (int qb = 0; qb < nqb; ++qb)
      atomicAdd(&hist[min(tile_keys(qb, rows, key_tile, lq, lk, causal), kSchedBins - 1)], 1);
  }
  __syncthreads();
  // exclusive prefix over bins in descending order: start[b] = sum_{b' > b} hist[b']
  for (int b = tid; b < kSchedBins; b += kSchedThreads) scan[b] = hist[kSchedBins - 1 - b];
  __syncthreads();
  for (int st = 1; st < kSchedBins; st <<= 1) {
    int v = 0;
    const int b = tid;
    if (b < kSchedBins && b >= st) v = scan[b - st];
    __syncthreads();
    if (b < kSchedBins) scan[b] += v;
    __syncthreads();
  }
  // scan[i] is now the inclusive sum of the i+1 largest bins
  for (int b = tid; b < kSchedBins; b += kSchedThreads) {
    const int i = kSchedBins - 1 - b;  // position of bin b in descending order
    hist[b] = scan[i] - hist[b];       // start offset of bin b
  }
  __syncthreads();
  for (int s = tid; s < nseq; s += kSchedThreads) {
    const int lq = seq[4 * s + 1], lk = seq[4 * s + 3];
    const int nqb = (lq + rows - 1) / rows;
    for (int qb = 0; qb < nqb; ++qb) {
      const int bin = min(tile_keys(qb, rows, key_tile, lq, lk, causal), kSchedBins - 1);
      const int pos = atomicAdd(&hist[bin], 1);
      if (pos < max_tiles) {
        tiles[2 * pos] = s;
        tiles[2 * pos + 1] = qb;
      }
    }
  }
  if (tid == 0) {
    sched[0] = min(scan[kSchedBins - 1], max_tiles);
    sched[1] = 0;
  }
}

hipError_t launch_varlen_schedule(const int32_t* cu_q, const int32_t* cu_k, int nseq,
                                  int total_q, int total_k, int rows, int key_tile,
                                  int causal, int max_tiles, int32_t* sched,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(varlen_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, cu_q,
                     cu_k, nseq, total_q, total_k, rows, key_tile, causal, max_tiles, sched);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Instances and dispatch
// ---------------------------------------------------------------------------
// (QB, KB, NW) per element type and head_dim.
template <typename T, int D> struct Tile;
template <> struct Tile<__bf16, 64> { static constexpr int QB = 2, KB = 2, NW = 4; };
template <> struct Tile<_Float16, 64> { static constexpr int QB = 2, KB = 2, NW = 4; };
template <> struct Tile<__bf16, 128> { static constexpr int QB = 1, KB = 2, NW = 4; };
template <> struct Tile<_Float16, 128> { static constexpr int QB = 1, KB = 2, NW = 4; };
template <> struct Tile<float, 64> { static constexpr int QB = 1, KB = 2, NW = 4; };
template <> struct Tile<float, 128> { static constexpr int QB = 1, KB = 1, NW = 4; };

template <typename T, int D>
static hipError_t launch_t(const FwdArgs& a, bool causal, bool varlen, unsigned grid,
                           hipStream_t stream) {
  using Tl = Tile<T, D>;
  constexpr int QB = Tl::QB, KB = Tl::KB, NW = Tl::NW;
  dim3 g(grid), blk(NW * 64);
  if (causal) {
    if (varlen) hipLaunchKernelGGL((fwd_kernel<T, D, QB, KB, NW, true, true>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((fwd_kernel<T, D, QB, KB, NW, true, false>), g, blk, 0, stream, a);
  } else {
    if (varlen) hipLaunchKernelGGL((fwd_kernel<T, D, QB, KB, NW, false, true>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((fwd_kernel<T, D, QB, KB, NW, false, false>), g, blk, 0, stream, a);
  }
  return hipGetLastError();
}

template <typename T, int D> static int rows_t() { return Tile<T, D>::NW * 32 * Tile<T, D>::QB; }
template <typename T, int D> static int keys_t() { return 32 * Tile<T, D>::KB; }

int fwd_block_rows(fa_dtype_t dtype, int D) {
  switch (dtype) {
    case FA_BF16: return D == 64 ? rows_t<__bf16, 64>() : rows_t<__bf16, 128>();
    case FA_F16: return D == 64 ? rows_t<_Float16, 64>() : rows_t<_Float16, 128>();
    default: return D == 64 ? rows_t<float, 64>() : rows_t<float, 128>();
  }
}

int fwd_key_tile(fa_dtype_t dtype, int D) {
  switch (dtype) {
    case FA_BF16: return D == 64 ? keys_t<__bf16, 64>() : keys_t<__bf16, 128>();
    case FA_F16: return D == 64 ? keys_t<_Float16, 64>() : keys_t<_Float16, 128>();
    default: return D == 64 ? keys_t<float, 64>() : keys_t<float, 128>();
  }
}

hipError_t launch_fwd(const FwdArgs& a, fa_dtype_t dtype, int D, bool causal, bool varlen,
                      unsigned grid, hipStream_t stream) {
  switch (dtype) {
    case FA_BF16:
      return D == 64 ? launch_t<__bf16, 64>(a, causal, varlen, grid, stream)
                     : launch_t<__bf16, 128>(a, causal, varlen, grid, stream);
    case FA_F16:
      return D == 64 ? launch_t<_Float16, 64>(a, causal, varlen, grid, stream)
                     : launch_t<_Float16, 128>(a, causal, varlen, grid, stream);
    default:
      return D == 64 ? launch_t<float, 64>(a, causal, varlen, grid, stream)
                     : launch_t<float, 128>(a, causal, varlen, grid, stream);
  }
}

}  // namespace fa
