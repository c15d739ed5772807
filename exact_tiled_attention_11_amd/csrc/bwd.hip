// Backward pass of libfa355: dQ, dK, dV from Q, K, V, O, lse and dO.
//
// The CSDN primer 轻松读懂FlashAttention 上, section Softmax求解重构, names the
// two techniques of the method, tiling and recompute: because O and the row
// statistics are stored, the backward pass recomputes the probabilities
// block by block instead of keeping the N x N matrix P.  With lse = m + ln l
// a probability is exp(s - lse) directly.  The gradients are the chain rule
// through S = scale Q K^T (masked), P = row softmax of S, O = P V:
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - delta),  delta = rowsum(dO o O),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// gfx950 mapping (ours):
//  * delta: one thread per (batch, query, head) row.
//  * dK/dV: one workgroup per 128 keys of one (batch, head), a wave per 32
//    keys holding its K and V rows in VGPRs as MFMA B operands; 32-row chunks
//    of Q and dO (with lse and delta) stream through LDS, double buffered.
//    Lanes own key columns: S = Q K^T and dP = dO V^T come out of the MFMA
//    with the chunk's queries along the registers, so P and dS are packed in
//    place as the B operand of dV^T += dO^T P and dK^T += Q^T dS, whose A
//    operands are transposing reads (ds_read_b64_tr_b16) of the same LDS tiles.
//    At head_dim 128 a pair of waves shares each 32 keys instead (one computes
//    P and dV, the other dP, dS and dK, a chunk behind; bwd_dkdv_split_kernel).
//  * dQ: one workgroup per 128 query rows (a wave per 32), Q and dO in
//    VGPRs, 32-key blocks of K and V streaming through LDS; lanes own query
//    columns, as in the forward kernel, and dQ^T += K^T dS^T.  At head_dim 64
//    without dropout it is software-pipelined like the forward
//    (bwd_dq_pipe_kernel): the vector work of one key block runs between the
//    MFMAs of its neighbours.
//  * Rows past the end, rows with no visible key (lse = -inf) and padding
//    keys get a probability of exactly 0; padding keys get dK = dV = 0.
//  * Tiles reach LDS through direct buffer loads (buffer_load ... lds) into
//    rings of stages whose waits the kernels count themselves; every result
//    is written once, with no atomics, so the gradients are bit-reproducible.
//  * Dropout (the forward's keep decisions, redrawn from the same Philox
//    counters): with Z = keep / (1 - p), dV = (P o Z)^T dO and
//    dS = P o (dP o Z - delta).  The dQ kernel has the forward's lane layout
//    and draws the words the same way; in the dK/dV kernel lanes are keys,
//    so each lane draws the call of one query row and the bytes are
//    transposed through a small LDS tile of the wave.

#include <math.h>

#include <type_traits>

#include "fa_device.h"
#include "launch.h"

namespace fa {

namespace {

constexpr int kNW = 4;     // waves per workgroup

// MODE of the gradient kernels: bit flags for the ALiBi bias of the forward
// and for its attention dropout (the prefix mask is a runtime value in all)
constexpr int kBwdPlain = 0, kBwdAlibi = 1, kBwdDrop = 2;
constexpr int kRows = 32;  // rows per wave and per streamed tile

// LDS position (16-byte chunks) of chunk c of tile row r: the XOR pattern of
// the forward kernel, conflict-free for the 4-row x 32-byte transposing
// reads (the 16-byte row reads of head_dim 128 and of 16 rows at head_dim 64
// meet 2-way conflicts; conflict-free patterns need a per-lane offset for the
// transposing read 8 rows down and measured slower).
__device__ __forceinline__ int bswz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

template <typename T>
__device__ __forceinline__ float dot8_16(const u32x4_t& x, const u32x4_t& y) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (__is_same(T, __bf16)) {
      s = __builtin_fmaf(lo_bf16(x[e]), lo_bf16(y[e]), s);
      s = __builtin_fmaf(hi_bf16(x[e]), hi_bf16(y[e]), s);
    } else {
      const f16x2_t a = as_f16x2(x[e]), b = as_f16x2(y[e]);
      s = __builtin_fmaf((float)a[0], (float)b[0], s);
      s = __builtin_fmaf((float)a[1], (float)b[1], s);
    }
  }
  return s;
}

// An LDS address held in a VGPR the compiler may not take apart: reads at a
// constant distance from it then carry that distance in their offset field,
// where the compiler would otherwise keep one base register per read and add
// the ring-stage offset to each of them on every step.
__device__ __forceinline__ const FA_LDS(char)* lds_pin(unsigned a) {
  asm volatile("" : "+v"(a));
  return (const FA_LDS(char)*)a;
}

// Lane parts of the two LDS read patterns of a 32-row tile.
template <int D>
struct ReadLanes {
  static constexpr int KS = D / 16, DB = D / 32, RB = D * 2;
  int rowl[KS];  // 8 consecutive columns of row `col` (A operand, rows = MFMA rows)
  int trl[DB];   // transposing read: columns of 32-wide block db, rows in P's order
  __device__ __forceinline__ void init(int lane) {
    const int col = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) rowl[ks] = col * RB + ((ks * 2 + hh) ^ bswz(col)) * 16;
    const int g = lane >> 4, ii = lane & 15, jj = ii >> 2, qq = ii & 3;
    const int rr = 4 * hh + jj;
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      const int ch = 4 * i + 2 * (g & 1) + (qq >> 1);
      trl[i] = rr * RB + ((ch ^ bswz(rr)) * 16) + (qq & 1) * 8;
    }
  }
  // this lane's read addresses in the tile at LDS address `base` (uniform:
  // kept whole in a scalar register, one vector add per address)
  __device__ __forceinline__ void at(unsigned base, const FA_LDS(char)* (&rp)[KS],
                                     const FA_LDS(char)* (&tp)[DB]) const {
asm volatile("" : "+s"(base));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) rp[ks] = lds_pin(base + rowl[ks]);
#pragma unroll
    for (int i = 0; i < DB; ++i) tp[i] = lds_pin(base + trl[i]);
  }
};

template <typename frag>
__device__ __forceinline__ frag row_frag(const FA_LDS(char)* tile, int off) {
  return *(const FA_LDS(frag)*)(tile + off);
}

// Transposing read: A operand whose k index follows the MFMA output row order
// (rows 16t + 4hh + e and 16t + 8 + 4hh + e of the tile).
template <typename frag>
__device__ __forceinline__ frag tr_frag(const FA_LDS(char)* tile, int off, int t, int RB) {
  const int base = off + 16 * t * RB;
  s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS(s16x4_t)*)(tile + base));
  s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS(s16x4_t)*)(tile + base + 8 * RB));
  const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo);
  const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi);
  const u32x4_t u = {lo2.x, lo2.y, hi2.x, hi2.y};
  return __builtin_bit_cast(frag, u);
}

// The (batch or sequence, head, block) of a workgroup: grid index = block
// level * (B * H) + batch * H + head.  For a packed batch, sequence b owns
// rows cu[b] .. cu[b+1] of the packed tensors (clamped to the totals, as in
// the forward).
struct BwdItem {
  int b, h, blk, lq, lk;
  long long q_tok0, k_tok0;  // first token row of the queries / keys
  long long stat0;           // lse / delta index of query row 0
  int kwrite;                // keys whose dK / dV rows this item writes
};
template <bool VARLEN>
__device__ __forceinline__ BwdItem bwd_item(const BwdArgs& a) {
  BwdItem w;
  int bh;
  block_coords(a.B * a.H, w.blk, bh);
  w.b = bh / a.H;
  w.h = bh - w.b * a.H;
  if constexpr (!VARLEN) {
    w.lq = a.Nq;
    w.lk = a.seqlens_k ? min(max(a.seqlens_k[w.b], 0), a.Nk) : a.Nk;
    w.q_tok0 = (long long)w.b * a.Nq;
    w.k_tok0 = (long long)w.b * a.Nk;
    w.stat0 = ((long long)w.b * a.H + w.h) * a.Nq;
    w.kwrite = a.Nk;  // padding keys get zero rows
  } else {
    const int q0 = min(max(a.cu_q[w.b], 0), a.total_q);
    const int q1 = min(max(a.cu_q[w.b + 1], q0), a.total_q);
    const int k0 = min(max(a.cu_k[w.b], 0), a.total_k);
    const int k1 = min(max(a.cu_k[w.b + 1], k0), a.total_k);
    w.lq = q1 - q0;
    w.lk = k1 - k0;
    w.q_tok0 = q0;
    w.k_tok0 = k0;
    w.stat0 = (long long)w.h * a.total_q + q0;
    w.kwrite = w.lk;
  }
  return w;
}

}  // namespace

// ---------------------------------------------------------------------------
// -delta = -rowsum(dO o O) and lse2 = lse * log2 e for every (query row,
// head), in lse's layout (stored negated: the dK/dV kernels start their dP
// products from it, so dP - delta comes out of the matrix cores)
// ---------------------------------------------------------------------------
template <typename T, int D, bool VARLEN>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  const long long row = (long long)blockIdx.x * 256 + threadIdx.x;  // (token, head), head fastest
  const long long ntok = VARLEN ? (long long)a.total_q : (long long)a.B * a.Nq;
  if (row >= ntok * a.H) return;
  const int h = (int)(row % a.H);
  const long long tok = row / a.H;
  const u32x4_t* po = (const u32x4_t*)((const T*)a.o + row * D);
  const u32x4_t* pd = (const u32x4_t*)((const T*)a.dout + row * D);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) s += dot8_16<T>(po[c], pd[c]);
  long long idx;
  if constexpr (VARLEN) {
    idx = (long long)h * a.total_q + tok;
  } else {
    const int i = (int)(tok % a.Nq);
    const int b = (int)(tok / a.Nq);
    idx = ((long long)b * a.H + h) * a.Nq + i;
  }
  a.delta[idx] = -s;
  // the row's exp2 offset for the gradient kernels: probabilities are
  // exp2(c s - lse2); +inf for a row with no visible key (probability 0)
  const float l = a.lse[idx];
  a.lse2[idx] = l == -INFINITY ? INFINITY : l * kLog2e;
}

// ---------------------------------------------------------------------------
// dK, dV: a workgroup per 128 keys of one (batch, head)
// ---------------------------------------------------------------------------
// LDS bytes per wave of the keep-byte transpose: 32 keys x 32 queries, rows
// padded to 36 bytes
constexpr int kTrRow = 36;
constexpr int kTrWave = 32 * kTrRow;

// Keep words of a lane of the dK/dV kernels, where lanes are keys: the lane
// draws the Philox call of query q0 + col for keys kw0 + 16 hh .. +15 and
// stores the bytes at [key][query] in the wave's LDS tile; word g then holds
// the bytes of its own key for the chunk's query rows 8g + 4hh .. +3.
__device__ __forceinline__ void dkdv_keep_words(uint32_t kw[4], FA_LDS(uint8_t)* trb, int kw0,
                                                int q0, int col, int hh, int h, int b,
                                                const BwdArgs& a) {
  const Philox4 x = philox4x32_10((uint32_t)((kw0 >> 4) + hh), (uint32_t)(q0 + col), (uint32_t)h,
                                  (uint32_t)b, a.seed_lo, a.seed_hi);
#pragma unroll
  for (int m = 0; m < 16; ++m)
    trb[(16 * hh + m) * kTrRow + col] = (uint8_t)(x.w[m >> 2] >> (8 * (m & 3)));
#pragma unroll
  for (int g = 0; g < 4; ++g)
    kw[g] = *(const FA_LDS(uint32_t)*)(trb + col * kTrRow + 8 * g + 4 * hh);
}

// exp2 exponents of the 16 (query row, key) pairs of a lane of the dK/dV
// kernels: register r holds row 8(r>>2) + 4hh + (r&3) of the chunk, the key
// is n.  Query row m sees the key iff m >= lim (and the key is real); the
// key's distance to that row's own position is lim - m.  On a masked chunk a
// hidden pair's exponent is clamped to -2^99 or less (probability exactly
// 0): row cr is visible iff cr >= limv, tested as min(x, (cr - limv + 1/2)
// 2^100), exact for |limv| < 2^20.
template <bool CAUSAL, bool ALIBI>
__device__ __forceinline__ void dkdv_exponents(float x[16], const f32x16_t& s, const float lr[16],
                                               const BwdArgs& a, float slope2, bool masked,
                                               int lim, int n, int lk) {
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(s[r], a.c, -lr[r]);
  if constexpr (ALIBI) {  // - slope |key - (row + Lk - Lq)|
    const float fl = (float)lim;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      x[r] = __builtin_fmaf(-slope2, fabsf(fl - (float)(8 * (r >> 2) + (r & 3))), x[r]);
  }
  if (masked) {
    const int limv = n < lk ? (CAUSAL && n >= a.prefix ? lim : -(1 << 20)) : (1 << 20);
    const float base = (0.5f - (float)limv) * 0x1p100f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      x[r] = fminf(x[r], base + (float)(8 * (r >> 2) + (r & 3)) * 0x1p100f);
  }
}

// Waves per SIMD the registers are sized for: three for the head_dim-64
// instances without dropout (167 VGPRs, no spills; 3.7 % faster than two
// without options, as a third workgroup per CU covers the waits of the other
// two), two with dropout (its keep-word state spills at 168).
template <int D, int MODE>
constexpr int dkdv_occupancy() { return D == 64 ? ((MODE & kBwdDrop) == 0 ? 3 : 2) : 1; }

template <typename T, int D, bool CAUSAL, int MODE, bool VARLEN>
__global__ __launch_bounds__(kNW * 64, (dkdv_occupancy<D, MODE>())) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr bool DROP = (MODE & kBwdDrop) != 0, ALIBI = (MODE & kBwdAlibi) != 0;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int KS = D / 16, DB = D / 32, TS = 2, RB = D * 2;
  constexpr int kTileB = kRows * RB;                     // one 32-row tile
  constexpr int kBufB = 2 * kTileB + 2 * kRows * 4;      // a stage: Q, dO, lse2, delta
  constexpr int kStages = 3;                              // chunks c (read), c+1, c+2 (landing)
  constexpr int kCPR = D / 8;                            // 16-byte chunks per row
  constexpr int kLPT = kRows * kCPR / (kNW * 64);        // 16-byte loads per lane per tile
  static_assert(kLPT >= 1 && kRows * kCPR % (kNW * 64) == 0, "a tile divides evenly over the lanes");

  __shared__ __attribute__((aligned(16))) char smem_raw[kStages * kBufB];
  FA_LDS(char)* smem = (FA_LDS(char)*)smem_raw;
  __shared__ __attribute__((aligned(16))) char trbuf_raw[DROP ? kNW * kTrWave : 16];

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  FA_LDS(uint8_t)* trb = (FA_LDS(uint8_t)*)trbuf_raw + (DROP ? wave * kTrWave : 0);

  // key blocks ascending: causal key blocks with most queries first
  const BwdItem wi = bwd_item<VARLEN>(a);
  const int b = wi.b, h = wi.h;
  const int lq = wi.lq, lk = wi.lk;
  const int off = lk - lq;
  const int k0 = wi.blk * kNW * kRows;
  if (VARLEN && k0 >= lk) return;  // past this sequence's keys: nothing to write
  const int kw0 = k0 + wave * kRows;  // this wave's first key
  const int n = kw0 + col;             // this lane's key

  const size_t rs = (size_t)a.H * D;
  const T* qb = (const T*)a.q + (size_t)wi.q_tok0 * rs + (size_t)h * D;
  const T* dob = (const T*)a.dout + (size_t)wi.q_tok0 * rs + (size_t)h * D;
  const float* dlb = a.delta + wi.stat0;

  // K and V rows of this lane's key (B operands, zero past the real keys),
  // read after the first chunk requests
  frag kf[KS], vf[KS];
  f32x16_t dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dka[db] = dva[db] = f32x16_t{};

  // query chunks that see any key of the workgroup (causal: i >= k0 - off)
  const int nch = (lq + kRows - 1) / kRows;
  // (with a prefix mask, keys below it are seen by every row)
  int c_begin = 0, c_wave = 0;
  if (CAUSAL) {
    c_begin = k0 < a.prefix ? 0 : max(0, k0 - off) / kRows;
    c_wave = kw0 < a.prefix ? 0 : max(0, kw0 - off) / kRows;
  }
  const int pre = a.prefix - 1;  // keys 0 .. pre are visible to every causal row
  const float slope2 = ALIBI ? a.alibi[h] * kLog2e : 0.f;  // ALiBi slope in exp2 units
  const bool wave_live = kw0 < lk;

  ReadLanes<D> rl;
  rl.init(lane);
  // Stage of chunk c (32 query rows): Q and dO rows reach LDS through direct
  // buffer loads (rows past the end are outside the buffer range and arrive
  // as zeros), with the XOR swizzle applied on the global side; wave 0 also
  // loads the rows' lse2 (lanes 0-31) and delta (lanes 32-63), zero past the
  // end (such rows then have P = 1 but dO = 0 and delta = 0: they add
  // nothing to dV or dK).
  unsigned voff[kLPT];
#pragma unroll
  for (int l = 0; l < kLPT; ++l) {
    const int p = (l * kNW + wave) * 64 + lane;  // 16-byte position within the tile
    const int r = p / kCPR, pos = p % kCPR;
    voff[l] = (unsigned)r * (unsigned)(rs * sizeof(T)) + (unsigned)((pos ^ bswz(r)) * 16);
  }
  const unsigned lds0 = (unsigned)(size_t)smem;
  const unsigned rsb = (unsigned)(rs * sizeof(T));
  auto issue = [&](int c) {
    const int rows = max(0, min(kRows, lq - c * kRows));
    const unsigned sb = lds0 + (c % kStages) * kBufB;
    const u32x4_t rq = make_rsrc((const char*)(qb + (size_t)c * kRows * rs), (unsigned)rows * rsb);
    const u32x4_t rd = make_rsrc((const char*)(dob + (size_t)c * kRows * rs), (unsigned)rows * rsb);
#pragma unroll
    for (int l = 0; l < kLPT; ++l) {
      const unsigned m0 = __builtin_amdgcn_readfirstlane(sb + (l * kNW + wave) * 1024);
      dma16(rq, voff[l], m0);
      dma16(rd, voff[l], m0 + kTileB);
    }
    if (wave == 0) {
      const unsigned m0 = __builtin_amdgcn_readfirstlane(sb + 2 * kTileB);
      if (lane < kRows)
        dma4(make_rsrc((const char*)(a.lse2 + wi.stat0 + c * kRows), (unsigned)rows * 4),
             (unsigned)lane * 4, m0);
      else
        dma4(make_rsrc((const char*)(dlb + c * kRows), (unsigned)rows * 4),
             (unsigned)(lane - kRows) * 4, m0);
    }
  };

  auto compute = [&](int c, int buf) {
    // Q tile at the stage's start, dO kTileB further, lse2 and delta after both
    unsigned sb = lds0 + buf * kBufB;
    asm volatile("" : "+s"(sb));
    const FA_LDS(char)* rp[KS];
    const FA_LDS(char)* tp[DB];
    rl.at(sb, rp, tp);
    const FA_LDS(float)* tl = (const FA_LDS(float)*)lds_pin(sb + 2 * kTileB + 16 * hh);
    const int q0 = c * kRows;
    // S = Q K^T and dP = dO V^T: rows (queries) along registers, lanes = keys
    // register r holds query row 8*(r>>2) + 4*hh + (r&3) of the chunk; nd:
    // -delta of those rows, where the dP products start (without dropout,
    // whose dS scales dP first)
    float lr[16];
    f32x16_t nd;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      typedef __attribute__((ext_vector_type(4))) float f32x4_t;
      const f32x4_t l4 = *(const FA_LDS(f32x4_t)*)(tl + 8 * g);
      const f32x4_t d4 = *(const FA_LDS(f32x4_t)*)(tl + kRows + 8 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lr[4 * g + e] = l4[e];
        nd[4 * g + e] = d4[e];
      }
    }
    f32x16_t s = {}, dp = DROP ? f32x16_t{} : nd;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mma(row_frag<frag>(rp[ks], 0), kf[ks], s);
      dp = mma(row_frag<frag>(rp[ks], kTileB), vf[ks], dp);
    }
    const bool masked =
        (kw0 + kRows - 1 >= lk) || (CAUSAL && kw0 + kRows - 1 > max(q0 + off, pre));
    const int lim = n - q0 - off - 4 * hh;
    uint32_t kw[4];
    if constexpr (DROP) dkdv_keep_words(kw, trb, kw0, q0, col, hh, h, b, a);
    float x[16];
    dkdv_exponents<CAUSAL, ALIBI>(x, s, lr, a, slope2, masked, lim, n, lk);
    float p[16], pd[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = fast_exp2(x[r]);
      if constexpr (DROP) {
        const bool kp = kept(kw[r >> 2], r & 3, a.drop_t);
        pd[r] = kp ? p[r] : 0.f;
        // (held: left free, the compiler converts each kept probability alone
        // and merges the halves with v_perm)
        asm volatile("" : "+v"(pd[r]));
        ds[r] = p[r] * ((kp ? dp[r] * a.drop_scale : 0.f) + nd[r]);
      } else {
        pd[r] = p[r];
        ds[r] = p[r] * dp[r];  // dp holds dP - delta
      }
    }
    frag pk[TS], dk[TS];
#pragma unroll
    for (int t = 0; t < TS; ++t) {
      u32x4_t up, ud;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        up[e] = pack2(pd[8 * t + 2 * e], pd[8 * t + 2 * e + 1], (T*)nullptr);
        ud[e] = pack2(ds[8 * t + 2 * e], ds[8 * t + 2 * e + 1], (T*)nullptr);
      }
      pk[t] = __builtin_bit_cast(frag, up);
      dk[t] = __builtin_bit_cast(frag, ud);
    }
    // dV^T += dO^T P and dK^T += Q^T dS (queries as the contraction index)
#pragma unroll
    for (int t = 0; t < TS; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dva[db] = mma(tr_frag<frag>(tp[db], kTileB, t, RB), pk[t], dva[db]);
        dka[db] = mma(tr_frag<frag>(tp[db], 0, t, RB), dk[t], dka[db]);
      }
  };

  if (c_begin < nch) issue(c_begin);
  if (c_begin + 1 < nch) issue(c_begin + 1);
  // K and V are read while those requests are in flight (the two memory
  // latencies overlap); complete before any chunk load is counted
  {
    const bool ok = n < lk;
    const T* kr = (const T*)a.k + ((size_t)wi.k_tok0 + (ok ? n : 0)) * rs + (size_t)h * D;
    const T* vr = (const T*)a.v + ((size_t)wi.k_tok0 + (ok ? n : 0)) * rs + (size_t)h * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      frag z = {};
      kf[ks] = ok ? *(const frag*)(kr + ks * 16 + hh * 8) : z;
      vf[ks] = ok ? *(const frag*)(vr + ks * 16 + hh * 8) : z;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  for (int c = c_begin; c < nch; ++c) {
    // this wave's part of chunk c is in once at most the next chunk's loads
    // are pending (wave 0 also issues the two statistics loads, each with
    // half of its lanes)
    if (c + 1 < nch) {
      if (wave == 0) vm_wait<2 * kLPT + 2>();
      else vm_wait<2 * kLPT>();
    } else {
      vm_wait<0>();
    }
    __syncthreads();  // every part of chunk c is in; every wave is done with chunk c-1's stage
    if (c + 2 < nch) issue(c + 2);
    if (wave_live && c >= c_wave) compute(c, c % kStages);
  }

  // dK = scale * dK^T, dV = dV^T (times 1 / (1 - p) with dropout) for keys
  // < Nk (padding keys: zero)
  const float vsc = DROP ? a.drop_scale : 1.f;
  if (n < wi.kwrite) {
    T* dkr = (T*)a.dk + ((size_t)wi.k_tok0 + n) * rs + (size_t)h * D;
    T* dvr = (T*)a.dv + ((size_t)wi.k_tok0 + n) * rs + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * hh;
        const f32x16_t& kk = dka[db];
        const f32x16_t& vv = dva[db];
        u32x2_t wk = {pack2(kk[4 * g4] * a.scale, kk[4 * g4 + 1] * a.scale, (T*)nullptr),
                      pack2(kk[4 * g4 + 2] * a.scale, kk[4 * g4 + 3] * a.scale, (T*)nullptr)};
        u32x2_t wv = {pack2(vv[4 * g4] * vsc, vv[4 * g4 + 1] * vsc, (T*)nullptr),
                      pack2(vv[4 * g4 + 2] * vsc, vv[4 * g4 + 3] * vsc, (T*)nullptr)};
        *(u32x2_t*)(dkr + d) = wk;
        *(u32x2_t*)(dvr + d) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV with each 32-key block shared by two waves (head_dim 128)
// ---------------------------------------------------------------------------
// One wave holding both accumulators of 32 keys at head_dim 128 (dK^T and
// dV^T, 128 fp32 registers) next to its K and V operands does not fit the
// 256 architectural VGPRs, and the accumulators then travel between the VGPR
// and AGPR files on every chunk.  Here a key block belongs to a pair of waves
// with one accumulator set each: the P wave holds K, computes S = Q K^T, the
// probabilities (masks, bias, dropout) and dV^T += dO^T P; the dS wave holds
// V, computes dP = dO V^T, takes P from the P wave through LDS in fp32 and
// computes dS = P o (dP - delta) and dK^T += Q^T dS.  The MFMA work is that
// of one wave doing both, the arithmetic and its order are the same, so the
// results are identical.  Waves 0-3 are the P waves of key blocks 0-3 and
// waves 4-7 the dS waves, so that each SIMD runs one of each kind.  With
// dropout the P wave hands over P with the sign bit set on dropped pairs.
constexpr int kKB = 4;  // key blocks per workgroup (128 keys, as bwd_dkdv_kernel)
constexpr int kSplitNW = 2 * kKB;

template <typename T, int D, bool CAUSAL, int MODE, bool VARLEN>
__global__ __launch_bounds__(kSplitNW * 64, 1) void bwd_dkdv_split_kernel(BwdArgs a) {
  constexpr bool DROP = (MODE & kBwdDrop) != 0, ALIBI = (MODE & kBwdAlibi) != 0;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int KS = D / 16, DB = D / 32, TS = 2, RB = D * 2;
  constexpr int kTileB = kRows * RB;                     // one 32-row tile
  constexpr int kBufB = 2 * kTileB + 2 * kRows * 4;      // a stage: Q, dO, lse2, delta
  typedef __attribute__((ext_vector_type(4))) float f32x4_t;
  // chunk c - 1 (dS waves), c (both), c + 1 and c + 2 (landing)
  constexpr int kStages = 4;
  constexpr int kCPR = D / 8;                            // 16-byte chunks per row
  constexpr int kLPT = kRows * kCPR / (kSplitNW * 64);   // 16-byte loads per lane per tile
  static_assert(kLPT >= 1 && kRows * kCPR % (kSplitNW * 64) == 0, "a tile divides evenly over the lanes");

  __shared__ __attribute__((aligned(16))) char smem_raw[kStages * kBufB];
  FA_LDS(char)* smem = (FA_LDS(char)*)smem_raw;
  // P of each key block, two chunks: 4 x 64 lanes x 16 bytes (lane-major,
  // register group g)
  __shared__ __attribute__((aligned(16))) f32x4_t pbuf_raw[2 * kKB * 4 * 64];
  __shared__ __attribute__((aligned(16))) char trbuf_raw[DROP ? kKB * kTrWave : 16];

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = wave & (kKB - 1);
  const bool pw = wave < kKB;  // P wave (else dS wave)
  FA_LDS(f32x4_t)* pex = (FA_LDS(f32x4_t)*)pbuf_raw + kb * 4 * 64 + lane;  // + parity * kPB
  constexpr int kPB = kKB * 4 * 64;
  FA_LDS(uint8_t)* trb = (FA_LDS(uint8_t)*)trbuf_raw + (DROP ? kb * kTrWave : 0);

  const BwdItem wi = bwd_item<VARLEN>(a);
  const int b = wi.b, h = wi.h;
  const int lq = wi.lq, lk = wi.lk;
  const int off = lk - lq;
  const int k0 = wi.blk * kKB * kRows;
  if (VARLEN && k0 >= lk) return;  // past this sequence's keys: nothing to write
  const int kw0 = k0 + kb * kRows;  // this wave's first key
  const int n = kw0 + col;          // this lane's key

  const size_t rs = (size_t)a.H * D;
  const T* qb = (const T*)a.q + (size_t)wi.q_tok0 * rs + (size_t)h * D;
  const T* dob = (const T*)a.dout + (size_t)wi.q_tok0 * rs + (size_t)h * D;
  const float* dlb = a.delta + wi.stat0;

  // B operand rows of this lane's key: K (P wave) or V (dS wave), zero past
  // the real keys
  frag kv[KS];
  {
    const bool ok = n < lk;
    const T* src = (const T*)(pw ? a.k : a.v) + ((size_t)wi.k_tok0 + (ok ? n : 0)) * rs +
                   (size_t)h * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      frag z = {};
      kv[ks] = ok ? *(const frag*)(src + ks * 16 + hh * 8) : z;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // K or V complete before any tile load is counted
  f32x16_t acc[DB];  // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};

  const int nch = (lq + kRows - 1) / kRows;
  int c_begin = 0, c_wave = 0;
  if (CAUSAL) {
    c_begin = k0 < a.prefix ? 0 : max(0, k0 - off) / kRows;
    c_wave = kw0 < a.prefix ? 0 : max(0, kw0 - off) / kRows;
  }
  const int pre = a.prefix - 1;
  const float slope2 = ALIBI ? a.alibi[h] * kLog2e : 0.f;
  const bool wave_live = kw0 < lk;

  ReadLanes<D> rl;
  rl.init(lane);
  // Stage of chunk c (32 query rows) in stage c % 4: Q and dO rows through
  // direct buffer loads (rows past the end arrive as zeros), swizzled on the
  // global side; wave 0 also loads the rows' lse2 (lanes 0-31) and delta
  // (lanes 32-63), zero past the end.
  const unsigned rsb = (unsigned)(rs * sizeof(T));
  unsigned voff[kLPT];
#pragma unroll
  for (int l = 0; l < kLPT; ++l) {
    const int p = (l * kSplitNW + wave) * 64 + lane;  // 16-byte position within the tile
    const int r = p / kCPR, pos = p % kCPR;
    voff[l] = (unsigned)r * rsb + (unsigned)((pos ^ bswz(r)) * 16);
  }
  const unsigned lds0 = (unsigned)(size_t)smem;
  auto issue = [&](int c) {
    const int rows = max(0, min(kRows, lq - c * kRows));
    const unsigned sb = lds0 + (c % kStages) * kBufB;
    const u32x4_t rq = make_rsrc((const char*)(qb + (size_t)c * kRows * rs), (unsigned)rows * rsb);
    const u32x4_t rd = make_rsrc((const char*)(dob + (size_t)c * kRows * rs), (unsigned)rows * rsb);
#pragma unroll
    for (int l = 0; l < kLPT; ++l) {
      const unsigned m0 = __builtin_amdgcn_readfirstlane(sb + (l * kSplitNW + wave) * 1024);
      dma16(rq, voff[l], m0);
      dma16(rd, voff[l], m0 + kTileB);
    }
    if (wave == 0) {
      const unsigned m0 = __builtin_amdgcn_readfirstlane(sb + 2 * kTileB);
      if (lane < kRows)
        dma4(make_rsrc((const char*)(a.lse2 + wi.stat0 + c * kRows), (unsigned)rows * 4),
             (unsigned)lane * 4, m0);
      else
        dma4(make_rsrc((const char*)(dlb + c * kRows), (unsigned)rows * 4),
             (unsigned)(lane - kRows) * 4, m0);
    }
  };
  // Start of step c: this wave's part of chunk c is in once at most chunk
  // c + 1's loads are pending (wave 0 also issues the two statistics loads,
  // each with half of its lanes); after the barrier every part is in, and
  // chunk c - 2's stage (last read by the dS waves in step c - 1) takes
  // chunk c + 2.
  auto step_begin = [&](int c) {
    if (c + 1 < nch) {
      if (wave == 0) vm_wait<2 * kLPT + 2>();
      else vm_wait<2 * kLPT>();
    } else {
      vm_wait<0>();
    }
    __syncthreads();
    if (c + 2 < nch) issue(c + 2);
  };

  // The dS wave runs one chunk behind its P wave: in step c the P wave
  // handles chunk c and the dS wave finishes chunk c - 1 (with the P that
  // was handed over in step c - 1) and computes dP of chunk c, so one
  // barrier per step orders everything.  P of chunk c sits in half c & 1.
  if (c_begin < nch) issue(c_begin);
  if (c_begin + 1 < nch) issue(c_begin + 1);
  // the two kinds of wave run separate loops with the same barriers
  if (pw) {
    for (int c = c_begin; c <= nch; ++c) {
      step_begin(c);
      if (wave_live && c < nch && c >= c_wave) {
        unsigned sb = lds0 + (c % kStages) * kBufB;
        asm volatile("" : "+s"(sb));
        const FA_LDS(char)* rp[KS];
        const FA_LDS(char)* tp[DB];
        rl.at(sb, rp, tp);
        const FA_LDS(float)* tl = (const FA_LDS(float)*)lds_pin(sb + 2 * kTileB + 16 * hh);
        const int q0 = c * kRows;
        f32x16_t sd = {};  // S: query rows along registers
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sd = mma(row_frag<frag>(rp[ks], 0), kv[ks], sd);
        float lr[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4_t l4 = *(const FA_LDS(f32x4_t)*)(tl + 8 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) lr[4 * g + e] = l4[e];
        }
        const bool masked =
            (kw0 + kRows - 1 >= lk) || (CAUSAL && kw0 + kRows - 1 > max(q0 + off, pre));
        const int lim = n - q0 - off - 4 * hh;
        uint32_t kw[4];
        if constexpr (DROP) dkdv_keep_words(kw, trb, kw0, q0, col, hh, h, b, a);
        float x[16];
        dkdv_exponents<CAUSAL, ALIBI>(x, sd, lr, a, slope2, masked, lim, n, lk);
        float p[16], pd[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(x[r]);
          if constexpr (DROP) {
            const bool kp = kept(kw[r >> 2], r & 3, a.drop_t);
            pd[r] = kp ? p[r] : 0.f;
            p[r] = kp ? p[r] : -p[r];
          } else {
            pd[r] = p[r];
          }
        }
        FA_LDS(f32x4_t)* px = pex + (c & 1) * kPB;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          px[g * 64] = f32x4_t{p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]};
        frag pk[TS];
#pragma unroll
        for (int t = 0; t < TS; ++t) {
          u32x4_t up;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            up[e] = pack2(pd[8 * t + 2 * e], pd[8 * t + 2 * e + 1], (T*)nullptr);
          pk[t] = __builtin_bit_cast(frag, up);
        }
        // dV^T += dO^T P
#pragma unroll
        for (int t = 0; t < TS; ++t)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[db] = mma(tr_frag<frag>(tp[db], kTileB, t, RB), pk[t], acc[db]);
      }
    }
  } else {
    f32x16_t dpp = {};  // dP of the previous chunk
    for (int c = c_begin; c <= nch; ++c) {
      step_begin(c);
      if (wave_live && c > c_begin && c - 1 >= c_wave) {
        // chunk c - 1: dS = P o (dP - delta), dK^T += Q^T dS (without
        // dropout dpp already holds dP - delta)
        unsigned sb = lds0 + ((c - 1) % kStages) * kBufB;
        asm volatile("" : "+s"(sb));
        const FA_LDS(char)* tp[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) tp[db] = lds_pin(sb + rl.trl[db]);
        const FA_LDS(float)* tlp = (const FA_LDS(float)*)lds_pin(sb + 2 * kTileB + 16 * hh);
        const FA_LDS(f32x4_t)* px = pex + ((c - 1) & 1) * kPB;
        float ds[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4_t p4 = px[g * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            if constexpr (DROP) {
              const f32x4_t d4 = *(const FA_LDS(f32x4_t)*)(tlp + kRows + 8 * g);
              const bool kp = !__builtin_signbit(p4[e]);
              ds[r] = fabsf(p4[e]) * ((kp ? dpp[r] * a.drop_scale : 0.f) + d4[e]);
            } else {
              ds[r] = p4[e] * dpp[r];
            }
          }
        }
        frag pk[TS];
#pragma unroll
        for (int t = 0; t < TS; ++t) {
          u32x4_t ud;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            ud[e] = pack2(ds[8 * t + 2 * e], ds[8 * t + 2 * e + 1], (T*)nullptr);
          pk[t] = __builtin_bit_cast(frag, ud);
        }
#pragma unroll
        for (int t = 0; t < TS; ++t)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[db] = mma(tr_frag<frag>(tp[db], 0, t, RB), pk[t], acc[db]);
      }
      if (wave_live && c < nch && c >= c_wave) {
        // chunk c: dP = dO V^T (without dropout: -delta + dO V^T, the
        // products starting from the rows' -delta)
        unsigned sb = lds0 + (c % kStages) * kBufB + kTileB;
        asm volatile("" : "+s"(sb));
        if constexpr (DROP) {
          dpp = f32x16_t{};
        } else {
          const FA_LDS(float)* tln = (const FA_LDS(float)*)lds_pin(sb + kTileB + 16 * hh);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4_t d4 = *(const FA_LDS(f32x4_t)*)(tln + kRows + 8 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) dpp[4 * g + e] = d4[e];
          }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          dpp = mma(row_frag<frag>(lds_pin(sb + rl.rowl[ks]), 0), kv[ks], dpp);
      }
    }
  }

  // dV = dV^T (times 1 / (1 - p) with dropout), dK = scale * dK^T, for keys
  // < Nk (padding keys: zero)
  const float sc = pw ? (DROP ? a.drop_scale : 1.f) : a.scale;
  if (n < wi.kwrite) {
    T* dst = (T*)(pw ? a.dv : a.dk) + ((size_t)wi.k_tok0 + n) * rs + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * hh;
        const f32x16_t& aa = acc[db];
        u32x2_t w = {pack2(aa[4 * g4] * sc, aa[4 * g4 + 1] * sc, (T*)nullptr),
                     pack2(aa[4 * g4 + 2] * sc, aa[4 * g4 + 3] * sc, (T*)nullptr)};
        *(u32x2_t*)(dst + d) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: a workgroup per 128 query rows of one (batch, head)
// ---------------------------------------------------------------------------
// (four waves per SIMD fit the causal head_dim-64 instances without dropout
// with no spills, measured 1 % faster; the others keep the compiler's choice)
template <typename T, int D, bool CAUSAL, int MODE, bool VARLEN>
__global__ __launch_bounds__(kNW * 64, (D == 64 && CAUSAL && (MODE & kBwdDrop) == 0) ? 4 : 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr bool DROP = (MODE & kBwdDrop) != 0, ALIBI = (MODE & kBwdAlibi) != 0;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int KS = D / 16, DB = D / 32, TS = 2, RB = D * 2;
  constexpr int kTileB = kRows * RB;                     // one 32-row tile
  constexpr int kBufB = 2 * kTileB;                      // a stage: K, V
  constexpr int kStages = 3;                              // blocks j (read), j+1, j+2 (landing)
  constexpr int kCPR = D / 8;                            // 16-byte chunks per row
  constexpr int kLPT = kRows * kCPR / (kNW * 64);        // 16-byte loads per lane per tile
  static_assert(kLPT >= 1 && kRows * kCPR % (kNW * 64) == 0, "a tile divides evenly over the lanes");

  __shared__ __attribute__((aligned(16))) char smem_raw[kStages * kBufB];
  FA_LDS(char)* smem = (FA_LDS(char)*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const BwdItem wi = bwd_item<VARLEN>(a);
  const int qblk = CAUSAL ? (a.nqb - 1 - wi.blk) : wi.blk;  // causal: longest first
  const int b = wi.b, h = wi.h;
  const int lq = wi.lq, lk = wi.lk;
  const int off = lk - lq;
  const int q0 = qblk * kNW * kRows;
  if (VARLEN && q0 >= lq) return;  // past this sequence's rows: nothing to write
  const int wq0 = q0 + wave * kRows;
  const int qi = wq0 + col;  // this lane's query row
  const int wq_last = min(wq0 + kRows, lq) - 1;

  const size_t rs = (size_t)a.H * D;
  const T* kb = (const T*)a.k + (size_t)wi.k_tok0 * rs + (size_t)h * D;
  const T* vb = (const T*)a.v + (size_t)wi.k_tok0 * rs + (size_t)h * D;

  // Q and dO rows of this lane's query (B operands), lse and delta
  frag qf[KS], dof[KS];
  float lrow = INFINITY, ndrow = 0.f;  // lse2 and -delta of this lane's row
  {
    const bool ok = qi < lq;
    const size_t ro = ((size_t)wi.q_tok0 + (ok ? qi : 0)) * rs + (size_t)h * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      frag z = {};
      qf[ks] = ok ? *(const frag*)((const T*)a.q + ro + ks * 16 + hh * 8) : z;
      dof[ks] = ok ? *(const frag*)((const T*)a.dout + ro + ks * 16 + hh * 8) : z;
    }
    if (ok) {
      lrow = a.lse2[wi.stat0 + qi];
      ndrow = a.delta[wi.stat0 + qi];
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // Q, dO and the row statistics complete before any tile load
  f32x16_t dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqa[db] = f32x16_t{};

  // key blocks of the workgroup and of this wave (causal: keys <= row + off)
  // (row i sees keys 0 .. max(i + off, prefix - 1) under the causal mask)
  const int pre = a.prefix - 1;
  const float slope2 = ALIBI ? a.alibi[h] * kLog2e : 0.f;  // ALiBi slope in exp2 units
  int nkb = (lk + kRows - 1) / kRows, nkw = nkb;
  if (CAUSAL) {
    const int kmax = max(min(q0 + kNW * kRows, lq) - 1 + off, pre);
    nkb = kmax < 0 ? 0 : min(nkb, kmax / kRows + 1);
    const int t = max(wq_last + off, pre);
    nkw = (wq_last < wq0 || t < 0) ? 0 : min(nkb, t / kRows + 1);
  } else if (wq_last < wq0) {
    nkw = 0;
  }

  ReadLanes<D> rl;
  rl.init(lane);
  // Stage of key block j: K and V rows through direct buffer loads (rows
  // past the end arrive as zeros), swizzled on the global side.
  const unsigned rsb = (unsigned)(rs * sizeof(T));
  unsigned voff[kLPT];
#pragma unroll
  for (int l = 0; l < kLPT; ++l) {
    const int p = (l * kNW + wave) * 64 + lane;
    const int r = p / kCPR, pos = p % kCPR;
    voff[l] = (unsigned)r * rsb + (unsigned)((pos ^ bswz(r)) * 16);
  }
  const unsigned lds0 = (unsigned)(size_t)(FA_LDS(char)*)smem_raw;
  auto issue = [&](int j) {
    const int rows = max(0, min(kRows, lk - j * kRows));
    const unsigned sb = lds0 + (j % kStages) * kBufB;
    const u32x4_t rk = make_rsrc((const char*)(kb + (size_t)j * kRows * rs), (unsigned)rows * rsb);
    const u32x4_t rv = make_rsrc((const char*)(vb + (size_t)j * kRows * rs), (unsigned)rows * rsb);
#pragma unroll
    for (int l = 0; l < kLPT; ++l) {
      const unsigned m0 = __builtin_amdgcn_readfirstlane(sb + (l * kNW + wave) * 1024);
      dma16(rk, voff[l], m0);
      dma16(rv, voff[l], m0 + kTileB);
    }
  };
  auto compute = [&](int j, int buf) {
    // K tile at the stage's start, V kTileB further
    const FA_LDS(char)* rp[KS];
    const FA_LDS(char)* tp[DB];
    rl.at(lds0 + buf * kBufB, rp, tp);
    const int k0 = j * kRows;
    // S^T = K Q^T and dP^T = V dO^T: keys along registers, lanes = queries
    f32x16_t s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mma(row_frag<frag>(rp[ks], 0), qf[ks], s);
      dp = mma(row_frag<frag>(rp[ks], kTileB), dof[ks], dp);
    }
    const bool masked = (k0 + kRows > lk) || (CAUSAL && k0 + kRows - 1 > max(wq0 + off, pre));
    // key 8*(r>>2) + 4*hh + (r&3) of the block is visible iff that offset <= lim
    const int last = CAUSAL ? min(max(qi + off, pre), lk - 1) : lk - 1;
    const int lim = last - k0 - 4 * hh;
    uint32_t kw[4];
    if constexpr (DROP) keep_words_rows(kw, k0 >> 4, hh, qi, h, b, a.seed_lo, a.seed_hi);
    // exponents; on a masked block key offset kr is visible iff kr <= lim,
    // tested as min(x, (lim - kr + 1/2) 2^100) (hidden: exactly 0 after exp2)
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(s[r], a.c, -lrow);
    if constexpr (ALIBI) {  // - slope |key - (qi + Lk - Lq)|, key k0 + 4hh + offset
      const float d0 = (float)(k0 + 4 * hh - qi - off);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        x[r] = __builtin_fmaf(-slope2, fabsf(d0 + (float)(8 * (r >> 2) + (r & 3))), x[r]);
    }
    if (masked) {
      const float base = ((float)lim + 0.5f) * 0x1p100f;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        x[r] = fminf(x[r], base - (float)(8 * (r >> 2) + (r & 3)) * 0x1p100f);
    }
    frag dsk[TS];
#pragma unroll
    for (int t = 0; t < TS; ++t) {
      u32x4_t ud;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pr[2];
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const int r = 8 * t + 2 * e + z;
          const float p = fast_exp2(x[r]);
          if constexpr (DROP)
            pr[z] = p * ((kept(kw[r >> 2], r & 3, a.drop_t) ? dp[r] * a.drop_scale : 0.f) + ndrow);
          else
            pr[z] = p * (dp[r] + ndrow);
        }
        ud[e] = pack2(pr[0], pr[1], (T*)nullptr);
      }
      dsk[t] = __builtin_bit_cast(frag, ud);
    }
    // dQ^T += K^T dS^T (keys as the contraction index).  At head_dim 128 (two
    // waves per SIMD) these MFMAs issue at a raised wave priority, so they
    // start ahead of the other wave's vector work (+1.7 %; no change at 64).
    constexpr bool kPrio = D == 128;
    if constexpr (kPrio) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < TS; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) dqa[db] = mma(tr_frag<frag>(tp[db], 0, t, RB), dsk[t], dqa[db]);
    if constexpr (kPrio) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (nkb > 0) issue(0);
  if (1 < nkb) issue(1);
  for (int j = 0; j < nkb; ++j) {
    // this wave's part of block j is in once at most the next block's loads are pending
    if (j + 1 < nkb) vm_wait<2 * kLPT>();
    else vm_wait<0>();
    __syncthreads();  // every part of block j is in; every wave is done with block j-1's stage
    if (j + 2 < nkb) issue(j + 2);
    if (j < nkw) compute(j, j % kStages);
  }

  if (qi < lq) {
    T* dqr = (T*)a.dq + ((size_t)wi.q_tok0 + qi) * rs + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * hh;
        const f32x16_t& x = dqa[db];
        u32x2_t w = {pack2(x[4 * g4] * a.scale, x[4 * g4 + 1] * a.scale, (T*)nullptr),
                     pack2(x[4 * g4 + 2] * a.scale, x[4 * g4 + 3] * a.scale, (T*)nullptr)};
        *(u32x2_t*)(dqr + d) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ at head_dim 64 without dropout, software-pipelined as the forward is.
// A block's three stages — S and dP (MFMA), the vector work P = exp2(c s -
// lse), dS = P (dP - delta) (VALU), dQ^T += K^T dS^T (MFMA) — depend on each
// other only within the block, so step j interleaves the vector work of
// block j with the dQ products of block j-1 and the S / dP products of block
// j+1, one fenced chunk per MFMA:
//   chunks 0-3   dQ products of block j-1      exp2 of block j (4 per chunk)
//   chunks 4-7   S products of block j+1       dS of block j (4 per chunk, packed)
//   chunks 8-11  dP products of block j+1      exponents of block j+1
// LDS holds two rings of kNS 32-key slots (K for blocks j-1 .. j+PK+1, V for
// j+1 .. j+PK+1, the same period for both so every offset is a constant of
// the step loop unrolled by kNS).  Each step requests block j+PK+1 (past the
// last block the range is empty and the slots fill with zeros).  157 VGPRs,
// three waves per SIMD, no spills; the results are bit-identical to those of
// bwd_dq_kernel (four waves), and the causal N8192 gradients 1.0-1.3 % faster.
// ---------------------------------------------------------------------------
constexpr int kDqPK = 2;  // steps between a block's request and its first use

template <int N>
using IC = std::integral_constant<int, N>;

template <typename T, int D, bool CAUSAL, int MODE, bool VARLEN>
__global__ __launch_bounds__(kNW * 64, 3) void bwd_dq_pipe_kernel(BwdArgs a) {
  constexpr bool ALIBI = (MODE & kBwdAlibi) != 0;
  static_assert(D == 64 && (MODE & kBwdDrop) == 0, "head_dim 64 without dropout");
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int KS = D / 16, DB = D / 32, TS = 2, RB = D * 2;
  constexpr int kTileB = kRows * RB;                // one 32-key K or V block
  constexpr int PK = kDqPK;
  constexpr int kNS = PK + 3;                       // ring slots
  constexpr int kVBase = kNS * kTileB;
  constexpr int kCPR = D / 8;                       // 16-byte chunks per row
  constexpr int kLPT = kRows * kCPR / (kNW * 64);   // 16-byte loads per lane per block
  static_assert(kLPT >= 1 && kRows * kCPR % (kNW * 64) == 0, "a block divides evenly over the lanes");
  constexpr int NDQ = TS * DB;                      // dQ products per block
  constexpr int NCH = NDQ + 2 * KS;                 // chunks per step
  static_assert(NDQ == 4 && KS == 4, "four chunks per group");
  constexpr int LA = 2;                             // LDS reads issued this many chunks ahead

  __shared__ __attribute__((aligned(16))) char smem_raw[2 * kNS * kTileB];

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const BwdItem wi = bwd_item<VARLEN>(a);
  const int qblk = CAUSAL ? (a.nqb - 1 - wi.blk) : wi.blk;  // causal: longest first
  const int h = wi.h;
  const int lq = wi.lq, lk = wi.lk;
  const int off = lk - lq;
  const int q0 = qblk * kNW * kRows;
  if (VARLEN && q0 >= lq) return;  // past this sequence's rows: nothing to write
  const int wq0 = q0 + wave * kRows;
  const int qi = wq0 + col;  // this lane's query row
  const int wq_last = min(wq0 + kRows, lq) - 1;

  const size_t rs = (size_t)a.H * D;
  const T* kb = (const T*)a.k + (size_t)wi.k_tok0 * rs + (size_t)h * D;
  const T* vb = (const T*)a.v + (size_t)wi.k_tok0 * rs + (size_t)h * D;

  for (int i = tid; i < 2 * kNS * kTileB / 16; i += kNW * 64) ((u32x4_t*)smem_raw)[i] = u32x4_t{};

  // Q and dO rows of this lane's query (B operands), lse2 and -delta: read
  // after the first block requests
  frag qf[KS], dof[KS];
  float lrow = INFINITY, ndrow = 0.f;
  f32x16_t dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqa[db] = f32x16_t{};

  const int pre = a.prefix - 1;
  const float slope2 = ALIBI ? a.alibi[h] * kLog2e : 0.f;
  int nkb = (lk + kRows - 1) / kRows, nkw = nkb;
  if (CAUSAL) {
    const int kmax = max(min(q0 + kNW * kRows, lq) - 1 + off, pre);
    nkb = kmax < 0 ? 0 : min(nkb, kmax / kRows + 1);
    const int t = max(wq_last + off, pre);
    nkw = (wq_last < wq0 || t < 0) ? 0 : min(nkb, t / kRows + 1);
  } else if (wq_last < wq0) {
    nkw = 0;
  }
  __syncthreads();  // LDS zeroed before any block lands

  // this lane's 16-byte chunk of a block (swizzled on the global side)
  const unsigned rsb = (unsigned)(rs * sizeof(T));
  unsigned voff[kLPT];
#pragma unroll
  for (int l = 0; l < kLPT; ++l) {
    const int p = (l * kNW + wave) * 64 + lane;
    const int r = p / kCPR, pos = p % kCPR;
    voff[l] = (unsigned)r * rsb + (unsigned)((pos ^ bswz(r)) * 16);
  }
  const unsigned lds0 = (unsigned)(size_t)smem_raw;
  constexpr auto kslot = [](int r) { return ((r % kNS + kNS) % kNS) * kTileB; };
  constexpr auto vslot = [](int r) { return kVBase + ((r % kNS + kNS) % kNS) * kTileB; };
  // block u of K and V into the slots of ring position r (empty range past the last block)
  auto issue = [&](int u, auto rc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    const int rows = (u >= 0 && u < nkb) ? min(kRows, lk - u * kRows) : 0;
    const size_t ob = (size_t)(u > 0 ? u : 0) * kRows * rs;
    const u32x4_t rk = make_rsrc((const char*)(kb + ob), (unsigned)rows * rsb);
    const u32x4_t rv = make_rsrc((const char*)(vb + ob), (unsigned)rows * rsb);
#pragma unroll
    for (int l = 0; l < kLPT; ++l) {
      const unsigned m0 = __builtin_amdgcn_readfirstlane(lds0 + kslot(r) + (l * kNW + wave) * 1024);
      dma16(rk, voff[l], m0);
      dma16(rv, voff[l], m0 + kVBase);
    }
  };

  // lane parts of the read addresses (the LDS base folded in, kept whole)
  ReadLanes<D> rl;
  rl.init(lane);
  const FA_LDS(char)* rp[KS];
  const FA_LDS(char)* tp[DB];
  rl.at(lds0, rp, tp);
  auto krow = [&](auto rc, int ks) __attribute__((always_inline)) -> frag {
    constexpr int r = decltype(rc)::value;
    return row_frag<frag>(rp[ks], kslot(r));
  };
  auto vrow = [&](auto rc, int ks) __attribute__((always_inline)) -> frag {
    constexpr int r = decltype(rc)::value;
    return row_frag<frag>(rp[ks], vslot(r));
  };
  auto ktr = [&](auto rc, int t, int db) __attribute__((always_inline)) -> frag {
    constexpr int r = decltype(rc)::value;
    return tr_frag<frag>(tp[db], kslot(r), t, RB);
  };

  // Register roles: sS, sD the S^T and dP^T products of the next block; sX
  // the exponents of the current block, then its probabilities, then P (dP -
  // delta); dsk its dS^T packed as the B operand of the dQ products, which
  // read the previous block's values in chunks 0-3 before chunks 4-7 rewrite
  // them.
  f32x16_t sS = {}, sD = {}, sX;
  frag dsk[TS];
#pragma unroll
  for (int t = 0; t < TS; ++t) dsk[t] = frag{};

  // exponents c s - lse2 of block u from sS, with the ALiBi bias and, on a
  // diagonal or tail block, the mask: key offset kr is visible iff kr <= lim,
  // tested as min(x, (lim - kr + 1/2) 2^100) (hidden: exactly 0 after exp2)
  auto exps_rest = [&](int u) __attribute__((always_inline)) {
    const int k0 = u * kRows;
    if constexpr (ALIBI) {  // - slope |key - (qi + Lk - Lq)|, key k0 + 4hh + offset
      const float d0 = (float)(k0 + 4 * hh - qi - off);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sX[r] = __builtin_fmaf(-slope2, fabsf(d0 + (float)(8 * (r >> 2) + (r & 3))), sX[r]);
    }
    const bool masked = (k0 + kRows > lk) || (CAUSAL && k0 + kRows - 1 > max(wq0 + off, pre));
    if (masked) {
      const int last = CAUSAL ? min(max(qi + off, pre), lk - 1) : lk - 1;
      const float base = ((float)(last - k0 - 4 * hh) + 0.5f) * 0x1p100f;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sX[r] = fminf(sX[r], base - (float)(8 * (r >> 2) + (r & 3)) * 0x1p100f);
    }
  };

  // Step j: blocks j+1 (K, V) must be in; then the chunks above.  Waves past
  // their last block only keep the barriers and requests going.
  int nkwp = nkw + 1;  // (hidden from the optimizer, as in the forward kernel)
  asm volatile("" : "+s"(nkwp));
  auto step = [&](int j, auto rc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    vm_wait<2 * (PK - 1) * kLPT>();  // this wave's part of block j+1 is in
    __syncthreads();                 // every part is in; slots of block j-2 are free
    issue(j + PK + 1, IC<(r + PK + 1) % kNS>{});
    if (j < nkwp && nkw > 0) {
      frag op[NCH];
      auto read = [&](int i) __attribute__((always_inline)) {
        if (i < NDQ) op[i] = ktr(IC<(r + kNS - 1) % kNS>{}, i >> 1, i & 1);
        else if (i < NDQ + KS) op[i] = krow(IC<(r + 1) % kNS>{}, i - NDQ);
        else op[i] = vrow(IC<(r + 1) % kNS>{}, i - NDQ - KS);
      };
      auto mf = [&](int i) __attribute__((always_inline)) {
        if (i < NDQ) dqa[i & 1] = mma(op[i], dsk[i >> 1], dqa[i & 1]);
        else if (i < NDQ + KS) sS = mma(op[i], qf[i - NDQ], i == NDQ ? f32x16_t{} : sS);
        else sD = mma(op[i], dof[i - NDQ - KS], i == NDQ + KS ? f32x16_t{} : sD);
      };
#pragma unroll
      for (int i = 0; i < LA; ++i) read(i);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (c + LA < NCH) read(c + LA);
        mf(c);
        // (the empty asm statements hold each chunk's results in place:
        // without them the compiler sinks the vector work of block j below
        // the step's MFMAs, to where the next step first reads it)
        if (c < NDQ) {  // probabilities of block j
          float e4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) e4[e] = fast_exp2(sX[4 * c + e]);
          asm volatile("" : "+v"(e4[0]), "+v"(e4[1]), "+v"(e4[2]), "+v"(e4[3]));
#pragma unroll
          for (int e = 0; e < 4; ++e) sX[4 * c + e] = e4[e];
        } else if (c < NDQ + KS) {  // dS = P (dP - delta) of block j, packed
          const int g = c - NDQ;
          u32x4_t w = __builtin_bit_cast(u32x4_t, dsk[g >> 1]);
          unsigned w0 = pack2(sX[4 * g] * (sD[4 * g] + ndrow), sX[4 * g + 1] * (sD[4 * g + 1] + ndrow),
                              (T*)nullptr);
          unsigned w1 = pack2(sX[4 * g + 2] * (sD[4 * g + 2] + ndrow),
                              sX[4 * g + 3] * (sD[4 * g + 3] + ndrow), (T*)nullptr);
          asm volatile("" : "+v"(w0), "+v"(w1));
          w[2 * (g & 1)] = w0;
          w[2 * (g & 1) + 1] = w1;
          dsk[g >> 1] = __builtin_bit_cast(frag, w);
        } else {  // exponents of block j+1 (its S products are complete)
          const int g = c - NDQ - KS;
#pragma unroll
          for (int e = 0; e < 4; ++e) sX[4 * g + e] = __builtin_fmaf(sS[4 * g + e], a.c, -lrow);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      exps_rest(j + 1);
    }
  };

  // requests of blocks 0 .. PK, then S and dP of block 0 and its exponents
  [&]<int... S>(std::integer_sequence<int, S...>) {
    (issue(S, IC<S % kNS>{}), ...);
  }(std::make_integer_sequence<int, PK + 1>{});
  // Q, dO and the row statistics are read while those requests are in flight
  // (the two memory latencies overlap)
  {
    const bool ok = qi < lq;
    const size_t ro = ((size_t)wi.q_tok0 + (ok ? qi : 0)) * rs + (size_t)h * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      frag z = {};
      qf[ks] = ok ? *(const frag*)((const T*)a.q + ro + ks * 16 + hh * 8) : z;
      dof[ks] = ok ? *(const frag*)((const T*)a.dout + ro + ks * 16 + hh * 8) : z;
    }
    if (ok) {
      lrow = a.lse2[wi.stat0 + qi];
      ndrow = a.delta[wi.stat0 + qi];
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // they and the first blocks are in
  __syncthreads();                // every wave's part of the blocks too
  if (nkw > 0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sS = mma(krow(IC<0>{}, ks), qf[ks], sS);
      sD = mma(vrow(IC<0>{}, ks), dof[ks], sD);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sX[r] = __builtin_fmaf(sS[r], a.c, -lrow);
    exps_rest(0);
  }
  // steps 0 .. nkb, unrolled by kNS so every slot offset is a constant (the
  // steps past nkb are not run: the bound is the workgroup's)
  for (int j0 = 0; j0 <= nkb; j0 += kNS) {
    [&]<int... R>(std::integer_sequence<int, R...>) {
      ((j0 + R <= nkb ? step(j0 + R, IC<R>{}) : void()), ...);
    }(std::make_integer_sequence<int, kNS>{});
  }

  if (qi < lq) {
    T* dqr = (T*)a.dq + ((size_t)wi.q_tok0 + qi) * rs + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * hh;
        const f32x16_t& x = dqa[db];
        u32x2_t w = {pack2(x[4 * g4] * a.scale, x[4 * g4 + 1] * a.scale, (T*)nullptr),
                     pack2(x[4 * g4 + 2] * a.scale, x[4 * g4 + 3] * a.scale, (T*)nullptr)};
        *(u32x2_t*)(dqr + d) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t launch_bwd_td(const BwdArgs& a, bool causal, hipStream_t stream) {
  // empty grids (no queries or no keys) are skipped: the other kernel still
  // writes the zero gradients of its side
  const bool varlen = a.cu_q != nullptr;
  const long long rows = (varlen ? (long long)a.total_q : (long long)a.B * a.Nq) * a.H;
  if (rows > 0) {
    const dim3 grid((unsigned)((rows + 255) / 256));
    if (varlen) hipLaunchKernelGGL((bwd_delta_kernel<T, D, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((bwd_delta_kernel<T, D, false>), grid, dim3(256), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nbh = (unsigned)(a.B * a.H);
  static_assert(kKB == kNW, "both dK/dV kernels cover 128 keys per workgroup");
  const unsigned gk = (unsigned)((a.Nk + kNW * kRows - 1) / (kNW * kRows)) * nbh;
  // head_dim 128: key blocks split over wave pairs (accumulators fit the VGPRs)
  constexpr bool kSplit = D == 128;  // the split dK/dV kernel pays at head_dim 128 only
  const unsigned gq = (unsigned)a.nqb * nbh;
  const int mode = (a.drop_t ? kBwdDrop : 0) | (a.alibi ? kBwdAlibi : 0);
  auto launch2 = [&](auto mc, auto vc) {
    constexpr int M = decltype(mc)::value;
    constexpr bool V = decltype(vc)::value;
    if (gk > 0) {
      if constexpr (kSplit) {
        if (causal) hipLaunchKernelGGL((bwd_dkdv_split_kernel<T, D, true, M, V>), dim3(gk), dim3(kSplitNW * 64), 0, stream, a);
        else hipLaunchKernelGGL((bwd_dkdv_split_kernel<T, D, false, M, V>), dim3(gk), dim3(kSplitNW * 64), 0, stream, a);
      } else {
        if (causal) hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true, M, V>), dim3(gk), dim3(kNW * 64), 0, stream, a);
        else hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false, M, V>), dim3(gk), dim3(kNW * 64), 0, stream, a);
      }
      const hipError_t e2 = hipGetLastError();
      if (e2 != hipSuccess) return e2;
    }
    if (gq > 0) {
      if constexpr (D == 64 && (M & kBwdDrop) == 0) {
        if (causal) hipLaunchKernelGGL((bwd_dq_pipe_kernel<T, D, true, M, V>), dim3(gq), dim3(kNW * 64), 0, stream, a);
        else hipLaunchKernelGGL((bwd_dq_pipe_kernel<T, D, false, M, V>), dim3(gq), dim3(kNW * 64), 0, stream, a);
      } else {
        if (causal) hipLaunchKernelGGL((bwd_dq_kernel<T, D, true, M, V>), dim3(gq), dim3(kNW * 64), 0, stream, a);
        else hipLaunchKernelGGL((bwd_dq_kernel<T, D, false, M, V>), dim3(gq), dim3(kNW * 64), 0, stream, a);
      }
    }
    return hipGetLastError();
  };
  using F = std::false_type;
  using Tr = std::true_type;
  constexpr int kBoth = kBwdAlibi | kBwdDrop;
  if (varlen) {
    if (mode == kBoth) return launch2(std::integral_constant<int, kBoth>{}, Tr{});
    if (mode == kBwdDrop) return launch2(std::integral_constant<int, kBwdDrop>{}, Tr{});
    if (mode == kBwdAlibi) return launch2(std::integral_constant<int, kBwdAlibi>{}, Tr{});
    return launch2(std::integral_constant<int, kBwdPlain>{}, Tr{});
  }
  if (mode == kBoth) return launch2(std::integral_constant<int, kBoth>{}, F{});
  if (mode == kBwdDrop) return launch2(std::integral_constant<int, kBwdDrop>{}, F{});
  if (mode == kBwdAlibi) return launch2(std::integral_constant<int, kBwdAlibi>{}, F{});
  return launch2(std::integral_constant<int, kBwdPlain>{}, F{});
}

int bwd_block_rows() { return kNW * kRows; }

hipError_t launch_bwd(const BwdArgs& a, fa_dtype_t dtype, int D, bool causal, hipStream_t stream) {
  if (dtype == FA_BF16)
    return D == 64 ? launch_bwd_td<__bf16, 64>(a, causal, stream) : launch_bwd_td<__bf16, 128>(a, causal, stream);
  return D == 64 ? launch_bwd_td<_Float16, 64>(a, causal, stream) : launch_bwd_td<_Float16, 128>(a, causal, stream);
}

}  // namespace fa
