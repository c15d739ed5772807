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
// primer's section 内存卡点 on kernel fusion); the explainer's 关键优化点
// (on-chip buffer reuse, pipelining data movement with compute) become LDS
// staging with several tiles in flight.
//
// gfx950 mapping (ours, not the pages'):
//  * Each wave owns QB blocks of 32 query rows.  Scores are computed
//    transposed, S^T = K Q^T, on the 32x32 MFMA: lane l then holds one query
//    (column l%32) and 16 keys per 32-key block, so row maxima and sums are
//    in-lane plus one exchange between the two 32-lane halves.
//  * Q stays in VGPRs as the MFMA B operand for the whole kernel; one FMA
//    per score forms the exp2 exponent c*s - m (c = scale*log2 e), so a
//    probability costs an FMA and a v_exp_f32.
//  * The running maximum is raised lazily: a tile is first exponentiated
//    with the current offset, and only if a row's tile sum shows a
//    probability that could exceed 2^15 (or the row has not seen a key yet)
//    is the tile maximum taken, the accumulator and sum rescaled and the tile
//    redone.  The result is the same softmax, since the final division uses
//    the same offset as every exponent; the common path needs no maximum.
//  * K and V tiles of KB*32 keys reach LDS through direct buffer loads
//    (buffer_load_dwordx4 ... lds, no VGPR staging), NBUF tiles deep, with
//    an XOR swizzle over 16-byte chunks chosen per lane on the global side.
//    Rows past the end of the sequence are outside the buffer range and
//    arrive as zeros.
//  * The output is accumulated transposed too, O^T += V^T P^T: the
//    probabilities never leave registers (they are the B operand as
//    computed), and V^T fragments come from LDS with the gfx950
//    transposing read ds_read_b64_tr_b16.  Row sums add the fp32
//    probabilities before they are rounded for P V (the log-sum-exp needs
//    that precision on rows with few keys).
//  * Causal tiles wholly above the diagonal are never loaded; a wave whose
//    rows cannot see a tile skips its math; only diagonal and tail tiles
//    evaluate the mask.  Causal query blocks are issued longest first.
//  * fp32 inputs take the plain tiled kernel (fp32 MFMA, no pipelining); at
//    head_dim 64 the four waves of a workgroup share 32 query rows, split
//    every key tile between them and merge their partial (m, l, O) at the
//    end, which shortens the serial chain of the longest causal row block.

#include <math.h>

#include <atomic>
#include <type_traits>

#include "fa_device.h"
#include "launch.h"

namespace fa {

// A tile whose maximum exceeds the running offset by more than kTau (in
// exp2 units) raises the offset once the lazy check has fired.
constexpr float kTau = 8.0f;

template <typename T, int D, int QB, int KB, int NW, int NBUF, bool KSPLIT = false>
struct FwdCfg {
  static constexpr int kQW = 32 * QB;          // query rows per wave
  // query rows per workgroup: with KSPLIT all waves share one row block and
  // wave w takes 32-key block w of every tile (KB == NW)
  static constexpr int kBR = KSPLIT ? kQW : NW * kQW;
  static_assert(!KSPLIT || KB == NW, "one key block of each tile per wave");
  static constexpr int kBC = 32 * KB;          // keys per tile
  static constexpr int kNT = NW * 64;          // threads per workgroup
  static constexpr int kES = Elem<T>::kBytes;
  static constexpr int kRowB = D * kES;        // bytes of one K or V row
  static constexpr int kCPR = kRowB / 16;      // 16-byte chunks per row
  static constexpr int kTileB = kBC * kRowB;   // bytes of one K or V tile
  static constexpr int kStageB = 2 * kTileB;   // K tile + V tile
  static constexpr int kDmaW = kBC * kCPR / (64 * NW);  // DMA loads per wave per tile
  static constexpr int kLdsB = NBUF * kStageB;
  static_assert(kBC * kCPR % (64 * NW) == 0, "tile chunks must divide evenly over waves");
  static_assert(kCPR >= 8, "swizzle needs at least 8 chunks per row");
  static_assert(kLdsB <= 160 * 1024, "LDS per workgroup");
  static_assert(NBUF >= 2, "at least one tile in flight");
};

// LDS position (in 16-byte chunks) of chunk c of tile row r.  For 16-bit
// types the XOR pattern makes both the 8-row column reads of K and the
// 4-row x 32-byte transposing reads of V conflict-free; for fp32 it spreads
// the 32-row column reads over 16 chunk positions.  It is an involution in
// c, so the same function maps an LDS position back to its global chunk.
template <int CPR, bool F32>
__device__ __forceinline__ int swz_f(int r) {
  return F32 ? (r & 15) : (((r & 3) << 1) | ((r >> 2) & 1));
}
template <int CPR, bool F32>
__device__ __forceinline__ int swz(int r, int c) {
  return r * CPR + (c ^ swz_f<CPR, F32>(r));
}

// Row swizzles of the pipelined kernel's K and V slots (16-bit types; CPR =
// 16-byte chunks per row, 8 for head_dim 64, 16 for 128).  LDS has 64 banks
// of 4 bytes.  K rows are read by ds_read_b128 (16 lanes, 16 rows, per
// cycle): the rows of one cycle must fall on distinct 16-byte bank groups.
// V rows are read by the transposing reads (32 lanes, 4 rows x 4 chunks,
// per cycle) through one lane offset for rows r, r+8, r+16 and r+24, so the
// V swizzle depends on bits 0-2 of r only and must separate the 4-chunk
// groups of the 4 rows.  Both are XOR patterns on the chunk index, hence
// involutions.  At head_dim 128 the two differ and each read is
// conflict-free; at head_dim 64 both slots keep the V pattern (its K reads
// then pair rows r and r+8, a 2-way conflict that measured no slower than a
// separate K pattern, which costs the dropout instance registers).
template <int CPR>
__device__ __forceinline__ int swz_k(int r) {
  return CPR == 8 ? (((r & 3) << 1) | ((r >> 2) & 1)) : (r & 15);
}
template <int CPR>
__device__ __forceinline__ int swz_v(int r) {
  return CPR == 8 ? (((r & 3) << 1) | ((r >> 2) & 1))
                  : (((r & 1) << 1) | (((r >> 1) & 1) << 2) | (((r ^ (r >> 2)) & 1) << 3));
}


// The (sequence, head, query block) a workgroup computes.  Fixed-length
// grids take query blocks as levels with (batch, head) fastest, causal ones
// longest first; varlen grids read the sorted tile list of the schedule
// kernel and may hold more workgroups than tiles (then false).
struct WorkItem {
  int b, h, qblk, lq, lk;
  long long q_tok0, k_tok0, lse_base;
};
// packed batches: each XCD walks the tile table one head at a time
constexpr int kXcdGroupVarlen = 1;
template <bool CAUSAL, bool VARLEN>
__device__ __forceinline__ bool work_item(const FwdArgs& a, WorkItem& w) {
  if constexpr (!VARLEN) {
    int level, bh;
    block_coords(a.B * a.H, level, bh);
    w.qblk = CAUSAL ? (a.nqb - 1 - level) : level;
    const int b = bh / a.H;
    w.b = b;
    w.h = bh - b * a.H;
    w.lq = a.Nq;
    w.lk = a.Nk;
    if (a.seqlens_k) w.lk = min(max(a.seqlens_k[b], 0), a.Nk);
    w.q_tok0 = (long long)b * a.Nq;
    w.k_tok0 = (long long)b * a.Nk;
    w.lse_base = ((long long)b * a.H + w.h) * a.Nq;
  } else {
    int t, h;
    block_coords<kXcdGroupVarlen>(a.H, t, h);
    w.h = h;
    if (t >= a.sched[0]) return false;
    const int* tl = a.sched + 2 + 4 * a.nseq + 2 * t;
    const int s = tl[0];
    w.b = s;  // the sequence takes the batch index's place (dropout counters)
    w.qblk = tl[1];
    const int* sq = a.sched + 2 + 4 * s;
    w.q_tok0 = sq[0];
    w.lq = sq[1];
    w.k_tok0 = sq[2];
    w.lk = sq[3];
    w.lse_base = (long long)w.h * a.total_q + w.q_tok0;
  }
  return true;
}

template <typename T, int D, int QB, int KB, int NW, int NBUF, int OCC, bool KSPLIT, bool CAUSAL,
          bool VARLEN>
__global__ __launch_bounds__(NW * 64, OCC) void fwd_kernel(FwdArgs a) {
  using C = FwdCfg<T, D, QB, KB, NW, NBUF, KSPLIT>;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr bool F32 = (E::kBytes == 4);
  constexpr int KS = D / E::kStep;        // MFMA steps over head_dim
  constexpr int DB = D / 32;              // 32-wide blocks of head_dim
  constexpr int TS = 32 / E::kStep;       // MFMA steps over a 32-key block
  constexpr int L = 2 * C::kDmaW;         // DMA loads per wave per tile (K + V)

  extern __shared__ __attribute__((aligned(16))) u32x4_t smem[];  // C::kLdsB bytes

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int hh = lane >> 5;

  // ---- which (sequence, head, query block) this workgroup computes ----
  WorkItem wi;
  if (!work_item<CAUSAL, VARLEN>(a, wi)) return;  // whole workgroup leaves together
  const int h = wi.h, qblk = wi.qblk, lq = wi.lq, lk = wi.lk;
  const long long q_tok0 = wi.q_tok0, k_tok0 = wi.k_tok0, lse_base = wi.lse_base;

  const int q0 = qblk * C::kBR;
  const int off = lk - lq;  // bottom-right causal alignment
  const int nkt_all = (lk + C::kBC - 1) / C::kBC;
  int nkt = nkt_all;
  if (CAUSAL) {
    const int kmax = min(q0 + C::kBR, lq) - 1 + off;
    nkt = kmax < 0 ? 0 : min(nkt_all, kmax / C::kBC + 1);
  }
  const int wq0 = KSPLIT ? q0 : q0 + wave * C::kQW;
  const int wq_last = min(wq0 + C::kQW, lq) - 1;
  // key blocks of a tile this wave computes: all KB, or (KSPLIT) block kbo
  constexpr int KBW = KSPLIT ? 1 : KB;
  const int kbo = KSPLIT ? wave : 0;

  const size_t rs = (size_t)a.H * D;  // elements between consecutive tokens
  const T* qp = (const T*)a.q + (size_t)q_tok0 * rs + (size_t)h * D;
  const char* kp = (const char*)((const T*)a.k + (size_t)k_tok0 * rs + (size_t)h * D);
  const char* vp = (const char*)((const T*)a.v + (size_t)k_tok0 * rs + (size_t)h * D);
  const unsigned rsb = (unsigned)(rs * sizeof(T));

  // ---- tile loads: per-lane global offsets of the chunks this lane moves ----
  unsigned voff[C::kDmaW];
#pragma unroll
  for (int u = 0; u < C::kDmaW; ++u) {
    const int p = (u * NW + wave) * 64 + lane;  // LDS chunk position within the tile
    const int r = p / C::kCPR, pos = p % C::kCPR;
    voff[u] = (unsigned)r * rsb + (unsigned)((pos ^ swz_f<C::kCPR, F32>(r)) * 16);
  }
  const unsigned lds0 = (unsigned)(size_t)(FA_LDS(char)*)smem;
  auto issue = [&](int j) {
    const int buf = j % NBUF;
    const int rows = min(C::kBC, lk - j * C::kBC);
    const u32x4_t rk = make_rsrc(kp + (size_t)j * C::kBC * rsb, (unsigned)rows * rsb);
    const u32x4_t rv = make_rsrc(vp + (size_t)j * C::kBC * rsb, (unsigned)rows * rsb);
    const unsigned kb0 = lds0 + buf * C::kStageB;
#pragma unroll
    for (int u = 0; u < C::kDmaW; ++u) {
      const unsigned m0 = __builtin_amdgcn_readfirstlane(kb0 + (u * NW + wave) * 1024);
      dma16(rk, voff[u], m0);
      dma16(rv, voff[u], m0 + C::kTileB);
    }
  };

  // the first tiles are requested before Q is read, so that their memory
  // latency and Q's overlap
#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p)
    if (p < nkt) issue(p);

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
  // Q (and the first tiles) must be complete before the loop: Q's loads are
  // the only vector-memory reads the compiler tracks, and a pending one would
  // make it wait for all tile loads in flight at the first use inside the loop.
  __builtin_amdgcn_s_waitcnt(0);

  f32x16_t oacc[DB][QB];
  float mrow[QB], lrow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrow[qb] = -INFINITY;  // running maximum (units of scale*log2 e); -inf: no key yet
    lrow[qb] = 0.f;        // running sum over this lane's keys
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db][qb] = f32x16_t{};
  }

  // Lane parts of the LDS read addresses (byte offsets within a tile).  The
  // swizzle term of a row depends only on the row's low bits, which these
  // fix, so every other term of an address is a compile-time constant.
  constexpr int RB = C::kCPR * 16;  // LDS bytes per tile row
  int klane[KS];                    // K fragment of step ks, rows col (+32 kb)
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if constexpr (F32) {
      const int d = ks * 2 + hh;
      klane[ks] = col * RB + ((d >> 2) ^ swz_f<C::kCPR, F32>(col)) * 16 + (d & 3) * 4;
    } else {
      klane[ks] = col * RB + ((ks * 2 + hh) ^ swz_f<C::kCPR, F32>(col)) * 16;
    }
  }
  constexpr int NV = F32 ? 4 : DB;  // distinct lane parts of the V reads
  int vlane[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if constexpr (F32) {
      // row 4*hh + (t&3) (+ multiples of 8), column col of each 32-wide block
      const int rr = 4 * hh + i;
      vlane[i] = rr * RB + (((col >> 2) ^ (rr & 7)) * 16) + (col & 3) * 4;
    } else {
      // lane (16g + 4jj + qq) addresses V[4*hh + jj][32*db + 16*(g&1) + 4*qq .. +3]
      const int g = lane >> 4, ii = lane & 15, jj = ii >> 2, qq = ii & 3;
      const int rr = 4 * hh + jj;
      const int ch = 4 * i + 2 * (g & 1) + (qq >> 1);
      vlane[i] = rr * RB + ((ch ^ swz_f<C::kCPR, F32>(rr)) * 16) + (qq & 1) * 8;
    }
  }
  // this wave's key block within the tile (KSPLIT): 32 rows further on; the
  // swizzles depend on row bits below 5 only, so it is a plain offset
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) klane[ks] += kbo * 32 * RB;
#pragma unroll
  for (int i = 0; i < NV; ++i) vlane[i] += kbo * 32 * RB;

  f32x16_t sacc[KBW][QB];     // scores of the tile being processed

  auto active = [&](int j) -> bool {
    const int k0w = j * C::kBC + kbo * 32;  // first key of this wave's part of tile j
    return j >= 0 && j < nkt && wq_last >= wq0 && k0w < lk &&
           (!CAUSAL || k0w <= wq_last + off);
  };

  auto scores = [&](int j) {
    {
      const int sb = (j % NBUF) * C::kStageB;  // byte offset of this tile's K in LDS
      const char* kt = (const char*)smem + sb;
      // S^T = K Q^T for KB key blocks x QB query blocks
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          const frag kf = *(const frag*)(kt + klane[ks] + kb * 32 * RB);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            sacc[kb][qb] = mma(kf, qf[qb][ks], sacc[kb][qb]);
        }
      }
    }
  };

  auto softmax = [&](int j) {
    const int k0 = j * C::kBC + kbo * 32;  // first key of this wave's part of the tile
    constexpr int kSpan = 32 * KBW;
    const bool need_mask = (k0 + kSpan > lk) || (CAUSAL && k0 + kSpan - 1 > wq0 + off);
    {  // x = c S - m
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float ms = mrow[qb] == -INFINITY ? 0.f : mrow[qb];
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][qb][r] = __builtin_fmaf(sacc[kb][qb][r], a.c, -ms);
      }
    }
    if (need_mask) {
      // A masked score becomes -2^109 or less: exp2 gives 0 and it never wins a
      // maximum.  Key kb*32 + 8*(r>>2) + 4*hh + (r&3) of the tile is visible to
      // query qi iff 8*(r>>2) + (r&3) <= lim, with lim below; the test is one
      // FMA and one min per score (no lane masks).
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qi = wq0 + qb * 32 + col;
        const int last = CAUSAL ? min(qi + off, lk - 1) : lk - 1;  // last visible key
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          const float lim = (float)(last - k0 - kb * 32 - 4 * hh);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float cr = (float)(8 * (r >> 2) + (r & 3));
            sacc[kb][qb][r] = fminf(sacc[kb][qb][r], __builtin_fmaf(lim, 0x1p110f, (0.5f - cr) * 0x1p110f));
          }
        }
      }
    }

    // Key block by key block: probabilities (packed as the P V operand) and
    // row sums over the unrounded fp32 values (the log-sum-exp needs that
    // precision), then that block's P V products.
    const int vt_off = (j % NBUF) * C::kStageB + C::kTileB;
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      frag pk[TS][QB];
      float tsum[QB];
      auto probs = [&]() {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) tsum[qb] = 0.f;
#pragma unroll
        for (int t = 0; t < TS; ++t)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            if constexpr (F32) {
              const float p = fast_exp2(sacc[kb][qb][t]);
              tsum[qb] += p;
              pk[t][qb] = p;
            } else {
              u32x4_t u;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float p0 = fast_exp2(sacc[kb][qb][8 * t + 2 * e]);
                const float p1 = fast_exp2(sacc[kb][qb][8 * t + 2 * e + 1]);
                tsum[qb] += p0;
                tsum[qb] += p1;
                u[e] = pack2(p0, p1, (T*)nullptr);
              }
              pk[t][qb] = __builtin_bit_cast(frag, u);
            }
          }
      };
      probs();

      // Lazy maximum: the offset m stays unless a probability could exceed
      // 2^15 (seen in this lane's block sum) or the row has not seen a key
      // yet; then the block maximum is taken, m raised, the accumulated
      // output and sum rescaled, and the block redone.
      bool need = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) need |= (mrow[qb] == -INFINITY) || !(tsum[qb] <= 0x1p15f);
      if (__any(need)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float m = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, sacc[kb][qb][r]);
          const float mx = half_max(m);
          const bool fresh = mrow[qb] == -INFINITY;
          const bool none = !(mx > -1e30f);  // no visible key in this block
          float delta;
          if (fresh) delta = none ? 0.f : mx;
          else delta = mx > kTau ? mx : 0.f;
          const float mold = fresh ? 0.f : mrow[qb];
          const float alpha = fresh ? 0.f : fast_exp2(-delta);
          mrow[qb] = (fresh && none) ? -INFINITY : mold + delta;
          lrow[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
#pragma unroll
          for (int k2 = kb; k2 < KBW; ++k2)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[k2][qb][r] -= delta;
        }
        probs();
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) lrow[qb] += tsum[qb];

      // O^T += V^T P^T for this key block
#pragma unroll
      for (int t = 0; t < TS; ++t) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          frag vf;
          if constexpr (F32) {
            // key kb*32 + 8*(t>>2) + 4*hh + (t&3); its swizzle adds 8*((t>>2)&1)
            // to the chunk index of column 32*db + col
            const int cx = (32 * db / 4) ^ (8 * ((t >> 2) & 1));
            vf = *(const float*)((const char*)smem + vt_off + vlane[t & 3] +
                                 (kb * 32 + 8 * (t >> 2)) * RB + cx * 16);
          } else {
            // the transposing read hands lane (16g + i) the 4 keys at column d0 + i
            const int base = vt_off + vlane[db] + (kb * 32 + 16 * t) * RB;
            s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (FA_LDS(s16x4_t)*)((FA_LDS(char)*)smem + base));
            s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (FA_LDS(s16x4_t)*)((FA_LDS(char)*)smem + base + 8 * RB));
            const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo);
            const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi);
            const u32x4_t u = {lo2.x, lo2.y, hi2.x, hi2.y};
            vf = __builtin_bit_cast(frag, u);
          }
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = mma(vf, pk[t][qb], oacc[db][qb]);
        }
      }
    }
  };

  for (int j = 0; j < nkt; ++j) {
    // tile j has landed once at most the loads of the later tiles already
    // issued (up to NBUF - 2 of them) are pending
    const int later = min(NBUF - 2, nkt - 1 - j);
    if (later >= 2) vm_wait<2 * L>();
    else if (later == 1) vm_wait<L>();
    else vm_wait<0>();
    __syncthreads();  // every wave's share of tile j is in; tile j-1's buffer is free
    if (j + NBUF - 1 < nkt) issue(j + NBUF - 1);
    if (active(j)) {
      scores(j);
      softmax(j);
    }
  }

  if constexpr (KSPLIT) {
    // ---- merge of the waves' partial results for the shared row block ----
    // Wave w holds (m_w, l_w, O_w) over its key blocks.  With M = max_w m_w
    // the row's result is sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w (the
    // pairwise merge of the online softmax, here over four partials, added
    // in wave order).  The staging buffers are reused for the exchange.
    static_assert(QB == 1 && NW == 4, "one row block; wave w finishes register group w");
    constexpr int kXO = 2 * NW * 32;  // floats before the partial outputs
    static_assert((kXO + NW * DB * 16 * 64) * 4 <= C::kLdsB, "exchange fits the staging buffers");
    float* xm = (float*)smem;  // [NW][32] offsets m_w
    float* xl = xm + NW * 32;  // [NW][32] sums l_w
    float* xo = xm + kXO;      // [NW][DB][16][64] weighted O_w, lane-major
    const float lt = half_sum(lrow[0]);
    __syncthreads();  // every wave is done with the staging buffers
    if (hh == 0) {
      xm[wave * 32 + col] = mrow[0];
      xl[wave * 32 + col] = lt;
    }
    __syncthreads();
    float mw[NW];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = xm[w * 32 + col];
      M = fmaxf(M, mw[w]);
    }
    float wt[NW];  // weights 2^(m_w - M); 0 for a wave that saw no key
#pragma unroll
    for (int w = 0; w < NW; ++w) wt[w] = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - M);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[((wave * DB + db) * 16 + r) * 64 + lane] = oacc[db][0][r] * wt[wave];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) L += wt[w] * xl[w * 32 + col];
    __syncthreads();
    const int qi = wq0 + col;
    if (qi < lq) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      T* orow = (T*)a.o + (size_t)(q_tok0 + qi) * rs + (size_t)h * D;
      const int g4 = wave;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float acc = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) acc += xo[((w * DB + db) * 16 + 4 * g4 + e) * 64 + lane];
          x[e] = acc * inv;
        }
        const int d = 32 * db + 8 * g4 + 4 * hh;
        if constexpr (F32) {
          *(float4*)(orow + d) = make_float4(x[0], x[1], x[2], x[3]);
        } else {
          u32x2_t u = {pack2(x[0], x[1], (T*)nullptr), pack2(x[2], x[3], (T*)nullptr)};
          *(u32x2_t*)(orow + d) = u;
        }
      }
      if (wave == 0 && hh == 0 && a.lse)
        a.lse[lse_base + qi] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
    }
    return;
  }
  // ---- epilogue: O = O / l, lse = m + log2 l (converted to natural log) ----
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
// Software-pipelined prefill for 16-bit types (head_dim 64 and 128).
//
// The three stages of a key block — scores S = K Q^T (MFMA), softmax
// (VALU), P V (MFMA) — depend on each other only within the block, so while
// a wave turns the scores of block u into probabilities, the MFMAs of P V
// for block u-1 and of the scores of block u+1 are issued between its VALU
// instructions.  Blocks are 32 keys, with one score set, one exponent set
// and one probability set per wave, so head_dim 64 (VALU-bound: per score
// the exponent, exp2, sum and pack outweigh the 4*64 MFMA flops) fits four
// waves per SIMD; head_dim 128 (MFMA-bound) runs two.
//
// LDS holds two rings of 32-key slots: K slots for blocks u+1 .. u+PK+1 and
// V slots for blocks u-1 .. u+PK, so each block is requested PK steps
// before its first use.  Every step issues exactly one K and one V load per
// lane (past the last block the buffer range is empty and the load writes
// zeros), which keeps the count of loads a step may leave pending constant;
// the first of those zero loads fills the V slot of "block -1", whose
// probabilities are zero too.
// ---------------------------------------------------------------------------
constexpr int kPipeLA = 2;  // LDS reads issued this many MFMAs ahead in the hot step
// steps between a block's request and its first use: 2 at head_dim 64; 1 at
// head_dim 128, whose steps are twice as long (3 % faster than 2 there)
constexpr int kPipePK64 = 2, kPipePK128 = 1;

template <typename T, int D, int NW, int PK>
struct PipeCfg {
  static constexpr int kBC = 32;                   // keys per block
  static constexpr int kBR = NW * 32;              // query rows per workgroup
  static constexpr int kNT = NW * 64;
  static constexpr int kRowB = D * 2;              // bytes of one K or V row
  static constexpr int kCPR = kRowB / 16;          // 16-byte chunks per row
  static constexpr int kSlotB = kBC * kRowB;       // one K or V block
  // Both rings have kNS slots (K needs PK+1, V needs PK+2), so slot offsets
  // repeat every kNS steps and the step loop, unrolled by kNS, addresses LDS
  // with constant offsets.
  static constexpr int kNS = PK + 2;
  static constexpr int kVBase = kNS * kSlotB;      // byte offset of the V ring
  static constexpr int kLdsB = 2 * kNS * kSlotB;
  // The 16-byte chunks of a K (or V) block are spread over the lanes.  When a
  // block has fewer chunks than the workgroup has lanes, waves 0 .. kKW-1
  // load K and waves kKW .. 2 kKW-1 load V (the rest load nothing);
  // otherwise every wave loads part of both.
  static constexpr int kChunksBlk = kBC * kCPR;
  static constexpr bool kSplitKV = kChunksBlk < 64 * NW;
  static constexpr int kKW = kSplitKV ? kChunksBlk / 64 : NW;  // waves sharing one block
  static constexpr int kLPS = kChunksBlk / (64 * kKW);        // 16-byte loads per lane per block
  static_assert(kChunksBlk % (64 * kKW) == 0 && (!kSplitKV || 2 * kKW <= NW),
                "a block divides evenly over the lanes");
  static_assert(kCPR >= 8, "swizzle needs at least 8 chunks per row");
};

template <int N>
using IC = std::integral_constant<int, N>;

// MODE: bit flags kPipeAlibi (ALiBi bias) and kPipeDrop (attention dropout),
// fixed-length or packed (a packed sequence's index takes the batch index's
// place in the dropout counters); the prefix mask is a runtime value in all.
constexpr int kPipePlain = 0, kPipeAlibi = 1, kPipeDrop = 2;

// Waves per SIMD: four at head_dim 64 (128 VGPRs), three for the ALiBi
// instances (their score bias vector takes 16 more), two at head_dim 128.
template <int D, int MODE>
constexpr int pipe_occupancy() { return D == 64 ? ((MODE & 1) ? 3 : 4) : 2; }

template <typename T, int D, int NW, int PK, bool CAUSAL, bool VARLEN, int MODE>
__global__ __launch_bounds__(NW * 64, (pipe_occupancy<D, MODE>())) void fwd_pipe_kernel(FwdArgs a) {
  constexpr bool ALIBI = (MODE & kPipeAlibi) != 0;
  constexpr bool DROP = (MODE & kPipeDrop) != 0;
  using C = PipeCfg<T, D, NW, PK>;
  using E = Elem<T>;
  using frag = typename E::frag;
  static_assert(E::kBytes == 2 && (D == 64 || D == 128), "16-bit element types, head_dim 64 or 128");
  constexpr int KS = D / E::kStep;  // MFMA steps over head_dim (score MFMAs per block)
  constexpr int DB = D / 32;        // 32-wide blocks of head_dim
  constexpr int TS = 32 / E::kStep; // MFMA steps over a 32-key block (2)
  constexpr int RB = C::kCPR * 16;  // LDS bytes per block row
  constexpr int LA = kPipeLA;
  constexpr int LPS = C::kLPS;
  constexpr int NPV = TS * DB;      // P V MFMAs per block
  constexpr int NCH = NPV + KS;     // MFMAs (chunks) per block
  constexpr int RP = NCH / 8;       // chunks per score pair
  constexpr int ALAG = DB - 1;      // chunks from a pair's exp2 to its add and pack
  static_assert(NCH % 8 == 0, "whole chunks per score pair");

  extern __shared__ __attribute__((aligned(16))) u32x4_t smem[];  // C::kLdsB bytes

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it stay scalar
  const int col = lane & 31;
  const int hh = lane >> 5;

  WorkItem wi;
  if (!work_item<CAUSAL, VARLEN>(a, wi)) return;  // whole workgroup leaves together
  const int lq = wi.lq, lk = wi.lk;
  float slope2 = 0.f;  // ALiBi slope of this head, in exp2 units
  if constexpr (ALIBI) slope2 = a.alibi[wi.h] * kLog2e;
  // ALiBi: the score MFMAs of every block start from slope2 * (8*(r>>2) +
  // (r&3)) / c in register r, the per-register part of the bias (the keys of
  // a block in the registers' order, less the lane half's 4*hh), so that
  // c * s carries it and no score needs an operation of its own for it
  f32x16_t sinit = {};
  if constexpr (ALIBI) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sinit[r] = slope2 * (float)(8 * (r >> 2) + (r & 3)) / a.c;
  }

  const int q0 = wi.qblk * C::kBR;
  const int off = lk - lq;  // bottom-right causal alignment
  // Under the causal mask row i sees keys 0 .. max(i + off, prefix - 1): the
  // prefix keys are seen by every row, so the visible keys stay a prefix.
  const int pre = a.prefix - 1;
  int nst = (lk + C::kBC - 1) / C::kBC;  // key blocks of the workgroup
  if (CAUSAL) {
    const int kmax = max(min(q0 + C::kBR, lq) - 1 + off, pre);
    nst = kmax < 0 ? 0 : min(nst, kmax / C::kBC + 1);
  }
  const int wq0 = q0 + wave * 32;
  const int wq_last = min(wq0 + 32, lq) - 1;
  int nw = 0;  // this wave's blocks: the prefix 0 .. nw-1
  if (wq_last >= wq0) {
    nw = nst;
    if (CAUSAL) {
      const int t = max(wq_last + off, pre);
      nw = t < 0 ? 0 : min(nst, t / C::kBC + 1);
    }
  }

  const size_t rs = (size_t)a.H * D;  // elements between consecutive tokens
  const T* qp = (const T*)a.q + (size_t)wi.q_tok0 * rs + (size_t)wi.h * D;
  const char* kp = (const char*)((const T*)a.k + (size_t)wi.k_tok0 * rs + (size_t)wi.h * D);
  const char* vp = (const char*)((const T*)a.v + (size_t)wi.k_tok0 * rs + (size_t)wi.h * D);
  const unsigned rsb = (unsigned)(rs * sizeof(T));

  // this lane's 16-byte chunk of a block: row r, LDS position pos (global
  // chunk pos ^ swizzle(r))
  constexpr int KW = C::kKW;
  // this wave's part in the block loads: K, V or both (uniform)
  const bool loads_k = !C::kSplitKV || wave < KW;
  const bool loads_v = !C::kSplitKV || (wave >= KW && wave < 2 * KW);
  const int lw = C::kSplitKV ? wave % KW : wave;  // position among the waves loading a block
  unsigned voffk[LPS], voffv[LPS];
#pragma unroll
  for (int l = 0; l < LPS; ++l) {
    const int p = (l * KW + lw) * 64 + lane;
    const int r = p / C::kCPR, pos = p % C::kCPR;
    voffk[l] = (unsigned)r * rsb + (unsigned)((pos ^ swz_k<C::kCPR>(r)) * 16);
    voffv[l] = (unsigned)r * rsb + (unsigned)((pos ^ swz_v<C::kCPR>(r)) * 16);
  }
  const unsigned lds0 = (unsigned)(size_t)(FA_LDS(char)*)smem;
  // slot offsets of the block whose index is congruent to r modulo kNS
  constexpr auto kslot = [](int r) { return ((r % C::kNS + C::kNS) % C::kNS) * C::kSlotB; };
  constexpr auto vslot = [](int r) { return C::kVBase + ((r % C::kNS + C::kNS) % C::kNS) * C::kSlotB; };
  // one block of K or V into its slot (an empty range past the last block)
  auto load = [&](const char* base, const unsigned (&voff)[LPS], int u, int slot)
                  __attribute__((always_inline)) {
    const int rows = (u >= 0 && u < nst) ? min(C::kBC, lk - u * C::kBC) : 0;
    const u32x4_t rsrc = make_rsrc(base + (size_t)(u > 0 ? u : 0) * C::kBC * rsb, (unsigned)rows * rsb);
#pragma unroll
    for (int l = 0; l < LPS; ++l)
      dma16(rsrc, voff[l], __builtin_amdgcn_readfirstlane(lds0 + slot + (l * KW + lw) * 1024));
  };
  // step s (s = r mod kNS) requests K of block s+PK+1, then V of block s+PK
  auto issue = [&](int s, auto rc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    if (loads_k) load(kp, voffk, s + PK + 1, kslot(r + PK + 1));
    if (loads_v) load(vp, voffv, s + PK, vslot(r + PK));
  };

  frag qf[KS];  // Q rows of this wave (B operands), read after the first block requests

  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16_t{};
  float mrow = -INFINITY;  // running offset (units of scale*log2 e); -inf: no key yet
  float lrow = 0.f;        // running sum over this lane's keys
  float negm = 0.f;        // -mrow, 0 while the row has seen no key
  // A block sum above thr settles (-1 while the row is fresh).  The bound
  // keeps every probability representable in the P V operand: 2^15 for fp16
  // (largest finite 65504); bf16 has fp32's exponent range, so 2^60 there,
  // which lets a row's offset lag further behind a growing maximum (ALiBi's
  // bias rises by slope * 32 per block) before the block has to be redone.
  constexpr float kThr = __is_same(T, __bf16) ? 0x1p60f : 0x1p15f;
  // With ALiBi in bf16 a settle also places the offset kLead above the block
  // maximum: the block's probabilities are then at most 2^-48 (far inside
  // bf16's and fp32's range; the offset cancels in O / l and lse), and the
  // growth that a bias rising block by block brings is absorbed for
  // kLead + 60 units instead of 60.  Not with fp16, whose P operand would
  // lose such small values.
  constexpr float kLead = (ALIBI && __is_same(T, __bf16)) ? 48.f : 0.f;
  float thr = -1.f;

  int klane[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    klane[ks] = col * RB + ((ks * 2 + hh) ^ swz_k<C::kCPR>(col)) * 16;
  int vlane[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    const int g = lane >> 4, ii = lane & 15, jj = ii >> 2, qq = ii & 3;
    const int rr = 4 * hh + jj;
    const int ch = 4 * i + 2 * (g & 1) + (qq >> 1);
    vlane[i] = rr * RB + ((ch ^ swz_v<C::kCPR>(rr)) * 16) + (qq & 1) * 8;
  }

  // nw + 1, hidden from the optimizer: relating it to the loop bound makes
  // the compiler restructure the loop in a way that doubles the registers
  // the accumulators take
  int nwp = nw + 1;
  asm volatile("" : "+s"(nwp));
  const int pq1 = nst >> 2, pq2 = nst >> 1, pq3 = nst - (nst >> 2);  // quarters of the blocks
  auto need_mask = [&](int u) __attribute__((always_inline)) {
    const int k0 = u * C::kBC;
    return (k0 + C::kBC > lk) || (CAUSAL && k0 + C::kBC - 1 > max(wq0 + off, pre));
  };

  // Register roles (fixed, so nothing is copied between blocks):
  //   sS  raw scores S^T of the next block to be exponentiated;
  //   sX  exponents c*s - m of the current block (kept for a rescale);
  //   pk  probabilities as P V operands: those of block u-1 until its P V
  //       MFMAs have read them, then those of block u.
  f32x16_t sS, sX;
  frag pk[TS];
#pragma unroll
  for (int t = 0; t < TS; ++t) pk[t] = frag{};

  // fragments of the block in slot r (a compile-time constant)
  auto kfrag = [&](auto rc, int ks) __attribute__((always_inline)) -> frag {
    constexpr int r = decltype(rc)::value;
    return *(const frag*)((const char*)smem + kslot(r) + klane[ks]);
  };
  // lane addresses of the V reads (the LDS base folded in once)
  FA_LDS(char)* vbase[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    vbase[db] = (FA_LDS(char)*)smem + vlane[db];
    asm volatile("" : "+v"(vbase[db]));  // kept whole (split, it is re-added every block)
  }
  auto vfrag = [&](auto rc, int t, int db) __attribute__((always_inline)) -> frag {
    constexpr int r = decltype(rc)::value;
    const int off = vslot(r) + 16 * t * RB;
    s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS(s16x4_t)*)(vbase[db] + off));
    s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS(s16x4_t)*)(vbase[db] + off + 8 * RB));
    const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo);
    const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi);
    const u32x4_t w = {lo2.x, lo2.y, hi2.x, hi2.y};
    return __builtin_bit_cast(frag, w);
  };
  // S^T = K Q^T of block 0 into sS
  auto scores0 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sS = mma(kfrag(IC<0>{}, ks), qf[ks], ks == 0 ? sinit : sS);
  };
  // Dropout: keep words of the current block (word g: registers 4g..4g+3).
  // The row sums take every probability; the P V operand only the kept ones
  // (their 1 / (1 - p) is applied to O at the end).
  uint32_t kw[4] = {0u, 0u, 0u, 0u};
  auto drop2 = [&](int c, float& p0, float& p1) __attribute__((always_inline)) {
    if constexpr (DROP) {
      const uint32_t w = kw[c >> 1];
      p0 = kept(w, 2 * (c & 1), a.drop_t) ? p0 : 0.f;
      p1 = kept(w, 2 * (c & 1) + 1, a.drop_t) ? p1 : 0.f;
    }
  };
  // probabilities exp2(sX) into pk; returns this lane's sum
  auto probs = [&]() __attribute__((always_inline)) -> float {
    float ts = 0.f;
#pragma unroll
    for (int t = 0; t < TS; ++t) {
      u32x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p0 = fast_exp2(sX[8 * t + 2 * e]);
        float p1 = fast_exp2(sX[8 * t + 2 * e + 1]);
        ts += p0;
        ts += p1;
        drop2(4 * t + e, p0, p1);
        w[e] = pack2(p0, p1, (T*)nullptr);
      }
      pk[t] = __builtin_bit_cast(frag, w);
    }
    return ts;
  };
  // lazy offset: raise m only if a probability could exceed the bound above
  // or the row has seen no key yet; then rescale O and l and redo the block
  auto settle = [&](float ts) __attribute__((always_inline)) {
    // thr is -1 while the row has seen no key, so one compare covers both cases
    const uint64_t need = __builtin_amdgcn_ballot_w64(!(ts <= thr));
    if (any_mask(need)) {
      float m = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, sX[r]);
      const float mx = half_max(m);
      const bool fresh = mrow == -INFINITY;
      const bool none = !(mx > -1e30f);  // no visible key in this block
      float delta;
      if (fresh) delta = none ? 0.f : mx + kLead;
      else delta = mx > kTau ? mx + kLead : 0.f;
      const float mold = fresh ? 0.f : mrow;
      const float alpha = fresh ? 0.f : fast_exp2(-delta);
      mrow = (fresh && none) ? -INFINITY : mold + delta;
      negm = (fresh && none) ? 0.f : -mrow;
      thr = (fresh && none) ? -1.f : kThr;
      lrow *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) sX[r] -= delta;
      ts = probs();
    }
    lrow += ts;
  };

  // Block u.  First, for a masked block, the mask on its raw scores; then
  // the exponents c*s - m of its scores.  Then one chunk per MFMA (P V for block u-1, then the scores
  // of block u+1); a chunk also issues the LDS read of a later MFMA and
  // takes its share of the exp2, add and pack work of the score pairs, so
  // the softmax's VALU work runs between MFMAs.  Scheduling fences keep the
  // chunks in order.  One body serves masked and unmasked blocks: two
  // copies of it would not fit the register budget.
  auto step_block = [&](int u, bool masked, auto rc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    if constexpr (DROP) keep_words_rows<D == 64 && !ALIBI>(kw, 2 * u, hh, wq0 + col, wi.h, wi.b, a.seed_lo, a.seed_hi);
    // The mask, on the raw scores: a hidden one becomes -inf (exp2 gives 0 and
    // it never wins a maximum).  Key 8*(e>>2) + 4*hh + (e&3) of the block is
    // visible to query qi iff 8*(e>>2) + (e&3) <= lim.  Written in place: a
    // select into new registers makes the compiler copy sS on the unmasked
    // path of every block.
    if (masked) {
      const int qi = wq0 + col;
      const int last = CAUSAL ? min(max(qi + off, pre), lk - 1) : lk - 1;
      const int lim = last - u * C::kBC - 4 * hh;
      const float ninf = -INFINITY;
#define FA_HIDE(E)                                                         \
  asm volatile("v_cmp_gt_i32 vcc, %2, %1\n\tv_cndmask_b32 %0, %0, %3, vcc" \
               : "+v"(sS[E])                                               \
               : "v"(lim), "n"(8 * ((E) >> 2) + ((E) & 3)), "v"(ninf)     \
               : "vcc");
      FA_HIDE(0) FA_HIDE(1) FA_HIDE(2) FA_HIDE(3) FA_HIDE(4) FA_HIDE(5) FA_HIDE(6) FA_HIDE(7)
      FA_HIDE(8) FA_HIDE(9) FA_HIDE(10) FA_HIDE(11) FA_HIDE(12) FA_HIDE(13) FA_HIDE(14)
      FA_HIDE(15)
#undef FA_HIDE
    }
    float addend = negm;
    // ALiBi: -slope * |key - position| in exp2 units, key 8*(r>>2) + 4*hh +
    // (r&3) of the block, position qi + off.  In a causal block left of the
    // wave's first row every key is at or before the position, so the bias is
    // slope * (key - position): a per-lane part joins the exponent's addend
    // and the per-element part slope * (8*(r>>2) + (r&3)) came with the
    // scores (sinit).  Other blocks take that part back out with the
    // absolute value (two operations per score).
    bool lin = false;
    float dbase = 0.f;
    if constexpr (ALIBI) {
      dbase = (float)(u * C::kBC + 4 * hh - (wq0 + col + off));
      lin = CAUSAL && (u * C::kBC + C::kBC - 1 <= wq0 + off);
      if (lin) addend = __builtin_fmaf(slope2, dbase, addend);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sX[r] = __builtin_fmaf(sS[r], a.c, addend);
    if constexpr (ALIBI) {
      if (!lin) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = (float)(8 * (r >> 2) + (r & 3));
          sX[r] = __builtin_fmaf(-slope2, fabsf(dbase + e) + e, sX[r]);
        }
      }
    }
    frag op[NCH];  // LDS operand of MFMA i: P V (t-major) first, then the scores
    auto read = [&](int i) __attribute__((always_inline)) {
      if (i < NPV) op[i] = vfrag(IC<(r + C::kNS - 1) % C::kNS>{}, i / DB, i % DB);
      else op[i] = kfrag(IC<(r + 1) % C::kNS>{}, i - NPV);
    };
    auto mf = [&](int i) __attribute__((always_inline)) {
      if (i < NPV) oacc[i % DB] = mma(op[i], pk[i / DB], oacc[i % DB]);
      else sS = mma(op[i], qf[i - NPV], i == NPV ? sinit : sS);
    };
    float pe[16];
    auto exp2c = [&](int c) __attribute__((always_inline)) {
      pe[2 * c] = fast_exp2(sX[2 * c]);
      pe[2 * c + 1] = fast_exp2(sX[2 * c + 1]);
    };
    float ts = 0.f;
    auto acc2 = [&](int c) __attribute__((always_inline)) {
      if (c == 0) {
        ts = pe[0] + pe[1];
      } else {
        ts += pe[2 * c];
        ts += pe[2 * c + 1];
      }
      float p0 = pe[2 * c], p1 = pe[2 * c + 1];
      drop2(c, p0, p1);
      // (held: left free, the compiler converts each probability alone and
      // merges the dropped halves with v_perm, 16 more instructions a block)
      if constexpr (DROP) asm volatile("" : "+v"(p0), "+v"(p1));
      u32x4_t w = __builtin_bit_cast(u32x4_t, pk[c >> 2]);
      unsigned pw = pack2(p0, p1, (T*)nullptr);
      // held here: left free, the compiler sinks the packs below the settle
      // test, which keeps the 16 unrounded probabilities live across it (7
      // more VGPRs, and spills in the dropout instance)
      asm volatile("" : "+v"(pw));
      w[c & 3] = pw;
      pk[c >> 2] = __builtin_bit_cast(frag, w);
    };
    // pair p: exp2 in chunk p*RP, add and pack in chunk p*RP + ALAG; the
    // probabilities of block u-1 in pk[t] are read by the P V MFMAs of
    // chunks t*DB .. t*DB+DB-1, never after their replacement is written
    // At head_dim 128 (MFMA-bound, two waves per SIMD) the chunks run at a
    // raised wave priority: while one wave is in its MFMA chunks and the
    // other in its exponent or row-sum work, the arbiter then issues the
    // MFMAs first and the other wave's VALU work fills their cycles.  At
    // head_dim 64 (VALU-bound, four waves) it measured no different.
    constexpr bool kPrio = D == 128;
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < LA; ++i) read(i);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c + LA < NCH) read(c + LA);
      mf(c);
      if (c % RP == 0) exp2c(c / RP);
      if (c >= ALAG && (c - ALAG) % RP == 0) acc2((c - ALAG) / RP);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int p = 0; p < 8; ++p)
      if (p * RP + ALAG >= NCH) acc2(p);
    settle(ts);
  };

  // Step u: blocks u+1 (K) and u-1 (V) must be in; then P V of u-1, scores
  // of u+1 and the softmax of u.  The scores of u+1 on a wave's last block
  // are computed and never used.
  auto step = [&](int u, auto rc) __attribute__((always_inline)) {
    // K u+1 and V u-1 of this wave's part must be in: later requests (V of u
    // and PK-1 steps' worth) may stay pending
    if constexpr (!C::kSplitKV) vm_wait<(2 * PK - 1) * LPS>();
    else if (loads_k) vm_wait<(PK - 1) * LPS>();
    else if (loads_v) vm_wait<PK * LPS>();
    __syncthreads();        // every wave's part is in; the slots of K u and V u-2 are free
    // When every workgroup of the grid is resident at once (one round), the
    // arbiter's oldest-wave-first order would finish the waves sharing a
    // SIMD one after another and leave it to a single wave at the end; the
    // priority of a wave falls instead with its work done (quarters of its
    // blocks), so the waves of a SIMD progress together.  At head_dim 128 the
    // priority is the MFMA chunks' (below).
    if constexpr (D == 64) {
      if (a.tail_prio) {
        if (u < pq1) __builtin_amdgcn_s_setprio(3);
        else if (u < pq2) __builtin_amdgcn_s_setprio(2);
        else if (u < pq3) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
    }
    issue(u, rc);
    // At u = nw every key of the block is hidden from this wave's rows (it
    // lies past the last one they see), so the masked form adds nothing but
    // the last P V.
    if (u < nwp) step_block(u, u == nw || need_mask(u), rc);
  };

  // requests of steps -PK-1 .. -1: K of blocks 0 .. PK, V of blocks -1 .. PK-1
  [&]<int... S>(std::integer_sequence<int, S...>) {
    (issue(S - PK - 1, IC<(S - PK - 1 + 4 * C::kNS) % C::kNS>{}), ...);
  }(std::make_integer_sequence<int, PK + 1>{});
  // Q is read while those requests are in flight (the two memory latencies
  // overlap); it must be complete before any block load is counted: its loads
  // are the only vector-memory reads the compiler tracks
  {
    const int qi = wq0 + col;
    const bool ok = qi < lq;
    const T* row = qp + (size_t)(ok ? qi : 0) * rs;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      frag z = {};
      qf[ks] = ok ? *(const frag*)(row + ks * 16 + hh * 8) : z;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // Q and the first blocks are in
  __syncthreads();                // every wave's part of them too
  if (nw > 0) scores0();
  // steps 0 .. nst, unrolled by kNS so every slot offset is a constant (the
  // steps past nst issue empty requests and compute nothing)
  for (int u0 = 0; u0 <= nst; u0 += C::kNS) {
    [&]<int... R>(std::integer_sequence<int, R...>) {
      (step(u0 + R, IC<R>{}), ...);
    }(std::make_integer_sequence<int, C::kNS>{});
  }

  // ---- epilogue: O = O / l, lse = m + log2 l (converted to natural log) ----
  const float lt = half_sum(lrow);
  const int qi = wq0 + col;
  if (qi < lq) {
    float inv = lt > 0.f ? 1.f / lt : 0.f;
    if constexpr (DROP) inv *= a.drop_scale;
    T* orow = (T*)a.o + (size_t)(wi.q_tok0 + qi) * rs + (size_t)wi.h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * hh;
        const float x0 = oacc[db][4 * g4 + 0] * inv, x1 = oacc[db][4 * g4 + 1] * inv;
        const float x2 = oacc[db][4 * g4 + 2] * inv, x3 = oacc[db][4 * g4 + 3] * inv;
        u32x2_t w = {pack2(x0, x1, (T*)nullptr), pack2(x2, x3, (T*)nullptr)};
        *(u32x2_t*)(orow + d) = w;
      }
    if (hh == 0 && a.lse)
      a.lse[wi.lse_base + qi] = lt > 0.f ? (mrow + fast_log2(lt)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Varlen schedule, written by one workgroup: the (sequence, query block)
// tiles sequence by sequence, each sequence's longest first.  The forward
// grid walks it per head on each XCD, so the workgroups an XCD runs at once
// share the K and V of one or two sequences in its L2.
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;

__global__ __launch_bounds__(kSchedThreads) void varlen_schedule_kernel(
    const int* cu_q, const int* cu_k, int nseq, int total_q, int total_k, int rows, int causal,
    int max_tiles, int* sched) {
  __shared__ int part[kSchedThreads];
  const int tid = threadIdx.x;
  int* seq = sched + 2;
  int* tiles = sched + 2 + 4 * nseq;
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
  // the tiles of sequence 0, then of sequence 1, ...; within a sequence the
  // longest first.  Offsets: an exclusive scan of the tile counts, taken
  // kSchedThreads sequences at a time.
  int carry = 0;  // tiles of the sequences before this chunk (the same in every thread)
  for (int base = 0; base < nseq; base += kSchedThreads) {
    const int s = base + tid;
    const int n = s < nseq ? (seq[4 * s + 1] + rows - 1) / rows : 0;
    part[tid] = n;
    __syncthreads();
    for (int st = 1; st < kSchedThreads; st <<= 1) {
      const int v = tid >= st ? part[tid - st] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    const int first = carry + part[tid] - n;
    for (int i = 0; i < n; ++i) {
      const int pos = first + i;
      if (pos < max_tiles) {
        tiles[2 * pos] = s;
        tiles[2 * pos + 1] = causal ? n - 1 - i : i;  // causal: the last query block sees the most keys
      }
    }
    carry += part[kSchedThreads - 1];
    __syncthreads();  // every thread has read part before the next chunk writes it
  }
  if (tid == 0) {
    sched[0] = min(carry, max_tiles);
    sched[1] = 0;
  }
}

// Schedule scratch of fa_fwd_varlen_noalloc.  In host code `scratch` names
// a host-side stand-in, not device memory: its device address is looked up
// once per device with that device current, and only that address is used.
static __device__ __align__(256) int32_t scratch[FA_NOALLOC_SCRATCH_BYTES / 4];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch[kScratchDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev].store(p, std::memory_order_release);  // racing threads store the same address
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_varlen_schedule(const int32_t* cu_q, const int32_t* cu_k, int nseq,
                                  int total_q, int total_k, int rows, int causal, int max_tiles,
                                  int32_t* sched, hipStream_t stream) {
  hipLaunchKernelGGL(varlen_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, cu_q,
                     cu_k, nseq, total_q, total_k, rows, causal, max_tiles, sched);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Instances and dispatch
// ---------------------------------------------------------------------------
// fp32 tiles (QB, KB, NW, NBUF, OCC, KSPLIT): query blocks of 32 per wave,
// key blocks of 32 per tile, waves per workgroup, tiles in flight, the waves
// per SIMD the register budget is sized for, and the key split.
template <int QB_, int KB_, int NW_, int NBUF_, int OCC_, int KSPLIT_ = 0>
struct TileCfg {
  static constexpr int QB = QB_, KB = KB_, NW = NW_, NBUF = NBUF_, OCC = OCC_;
  static constexpr bool KSPLIT = KSPLIT_ != 0;
};
template <typename T, int D> struct Tile;
// fp32 at head_dim 64: 32-row workgroups whose four waves split each
// 128-key tile (the longest causal row block otherwise walks every key on
// one wave: fp32 MFMAs are 16 times slower per flop than bf16 ones)
template <> struct Tile<float, 64> : TileCfg<1, 4, 4, 2, 2, 1> {};
template <> struct Tile<float, 128> : TileCfg<1, 1, 4, 2, 2> {};

template <typename K>
static hipError_t launch_k(K kern, unsigned grid, int threads, int lds, hipStream_t stream,
                           const FwdArgs& a) {
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, stream, a);
  return hipGetLastError();
}

// 16-bit types take the software-pipelined kernel, fp32 the plain tiled one.
template <typename T, int D>
struct UsePipe {
  static constexpr bool value = sizeof(T) == 2;
};
// waves (of 32 query rows each) per workgroup of the pipelined kernel (eight
// at head_dim 64 halve the K/V traffic into LDS, and the power drawn, but
// couple two waves of a SIMD through the barrier: no faster)
template <int D>
struct PipeNW {
  static constexpr int value = 4;
};

template <typename T, int D>
static hipError_t launch_t(const FwdArgs& a, bool causal, bool varlen, unsigned grid,
                           hipStream_t stream) {
  if constexpr (UsePipe<T, D>::value) {
    constexpr int NW = PipeNW<D>::value, PK = D == 128 ? kPipePK128 : kPipePK64;
    constexpr int lds = PipeCfg<T, D, NW, PK>::kLdsB;
    // one instance per (mode, causal, packed)
    auto go = [&](auto mc) {
      constexpr int M = decltype(mc)::value;
      if (causal) {
        if (varlen) return launch_k(fwd_pipe_kernel<T, D, NW, PK, true, true, M>, grid, NW * 64, lds, stream, a);
        return launch_k(fwd_pipe_kernel<T, D, NW, PK, true, false, M>, grid, NW * 64, lds, stream, a);
      }
      if (varlen) return launch_k(fwd_pipe_kernel<T, D, NW, PK, false, true, M>, grid, NW * 64, lds, stream, a);
      return launch_k(fwd_pipe_kernel<T, D, NW, PK, false, false, M>, grid, NW * 64, lds, stream, a);
    };
    if (a.alibi && a.drop_t) return go(IC<kPipeAlibi | kPipeDrop>{});
    if (a.alibi) return go(IC<kPipeAlibi>{});
    if (a.drop_t) return go(IC<kPipeDrop>{});
    return go(IC<kPipePlain>{});
  } else {
    using Tl = Tile<T, D>;
    constexpr int QB = Tl::QB, KB = Tl::KB, NW = Tl::NW, NB = Tl::NBUF, OC = Tl::OCC;
    constexpr bool KSP = Tl::KSPLIT;
    constexpr int lds = FwdCfg<T, D, QB, KB, NW, NB, KSP>::kLdsB;
    if (causal) {
      if (varlen) return launch_k(fwd_kernel<T, D, QB, KB, NW, NB, OC, KSP, true, true>, grid, NW * 64, lds, stream, a);
      return launch_k(fwd_kernel<T, D, QB, KB, NW, NB, OC, KSP, true, false>, grid, NW * 64, lds, stream, a);
    }
    if (varlen) return launch_k(fwd_kernel<T, D, QB, KB, NW, NB, OC, KSP, false, true>, grid, NW * 64, lds, stream, a);
    return launch_k(fwd_kernel<T, D, QB, KB, NW, NB, OC, KSP, false, false>, grid, NW * 64, lds, stream, a);
  }
}

template <typename T, int D> static int rows_t() {
  if constexpr (UsePipe<T, D>::value) return PipeNW<D>::value * 32;
  else return (Tile<T, D>::KSPLIT ? 1 : Tile<T, D>::NW) * 32 * Tile<T, D>::QB;
}

int fwd_block_rows(fa_dtype_t dtype, int D) {
  switch (dtype) {
    case FA_BF16: return D == 64 ? rows_t<__bf16, 64>() : rows_t<__bf16, 128>();
    case FA_F16: return D == 64 ? rows_t<_Float16, 64>() : rows_t<_Float16, 128>();
    default: return D == 64 ? rows_t<float, 64>() : rows_t<float, 128>();
  }
}

namespace {
// Compute units of the current device, looked up once per device.
constexpr int kCuDevices = 64;
std::atomic<int> g_cus[kCuDevices];
int cu_count() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  int n = dev < kCuDevices ? g_cus[dev].load(std::memory_order_relaxed) : 0;
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev < kCuDevices) g_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace

hipError_t launch_fwd(const FwdArgs& args, fa_dtype_t dtype, int D, bool causal, bool varlen,
                      unsigned grid, hipStream_t stream) {
  FwdArgs a = args;
  // the head_dim-64 pipelined kernel runs four workgroups per compute unit
  // (three with ALiBi): a grid of at most that many is one round
  a.tail_prio = dtype != FA_F32 && D == 64 && (long long)grid <= (a.alibi ? 3LL : 4LL) * cu_count();
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
