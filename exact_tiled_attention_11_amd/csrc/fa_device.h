// Device-side helpers shared by the libfa355 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

#define FA_LDS(T) __attribute__((address_space(3))) T

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Matrix-core products. One 32x32 fp32 accumulator block per call.
//  * 16-bit inputs: v_mfma_f32_32x32x16_{bf16,f16}; lane l supplies
//    A[l%32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l%32].
//  * fp32 inputs:   v_mfma_f32_32x32x2_f32; lane l supplies A[l%32][l/32]
//    and B[l/32][l%32].
//  The accumulator holds C[8*(r/4) + 4*(l/32) + r%4][l%32] in element r.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16_t mma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mma(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mma(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Per-element-type facts used by the kernels.
template <typename T> struct Elem;
template <> struct Elem<__bf16> {
  using frag = bf16x8_t;                // one MFMA operand per lane
  static constexpr int kStep = 16;      // contraction depth of one MFMA
  static constexpr int kBytes = 2;
};
template <> struct Elem<_Float16> {
  using frag = f16x8_t;
  static constexpr int kStep = 16;
  static constexpr int kBytes = 2;
};
template <> struct Elem<float> {
  using frag = float;
  static constexpr int kStep = 2;
  static constexpr int kBytes = 4;
};

// Values of the two 32-lane halves of a wave, combined per column: after the
// swap every lane holds its own value and the one 32 lanes away.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Same for lanes 16 apart within each 32-lane half.
__device__ __forceinline__ float quarter_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float quarter_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Is a wave-wide lane mask (from __builtin_amdgcn_ballot_w64 of a compare)
// non-zero?  Tested with a scalar compare: the compiler's own lowering of a
// combined condition round-trips the mask through two vector ops.
__device__ __forceinline__ bool any_mask(uint64_t m) {
  uint32_t r;
  asm volatile("s_cmp_lg_u64 %1, 0\n\ts_cselect_b32 %0, 1, 0" : "=s"(r) : "s"(m) : "scc");
  return r != 0;
}

// (level, batch*head) coordinates of this workgroup in a grid of nlev * nbh
// workgroups, level 0 the longest.  The eight XCDs take workgroups in turn
// (workgroup i goes to XCD i mod 8), each XCD with its own L2.  When the
// (batch, head) pairs divide evenly over the XCDs, XCD x takes the pairs x,
// x+8, ... in groups of kXcdGroup, one group after another, and within a
// group runs level by level over its pairs: an XCD then streams the K and V
// (or Q and dO) of a few heads at a time, which stay in its L2 for the
// workgroups that share them, while the longest blocks of a group still
// start first.  Otherwise level l holds ids l*nbh .. l*nbh + nbh - 1.
constexpr int kXcdGroup = 4;
template <int G = kXcdGroup>
__device__ __forceinline__ void block_coords(int nbh, int& level, int& bh) {
  const int i = blockIdx.x;
  if (G > 0 && (nbh & 7) == 0) {
    constexpr int g = G;
    const int nlev = gridDim.x / nbh;
    const int j = i >> 3;  // position in this XCD's sequence
    const int grp = j / (g * nlev);
    const int r = j - grp * (g * nlev);
    const int gs = min(g, (nbh >> 3) - grp * g);  // pairs in this group (the last may have fewer)
    level = r / gs;
    bh = (grp * g + (r - level * gs)) * 8 + (i & 7);
  } else {
    level = i / nbh;
    bh = i - level * nbh;
  }
}

// One 16-byte direct-to-LDS load per lane: LDS[m0 + 16*lane] <- buffer[voff].
// Written as inline assembly because the compiler's own form makes every
// later LDS read wait for all such loads; the kernels count them themselves.
__device__ __forceinline__ void dma16(const u32x4_t& rsrc, unsigned voff, unsigned m0) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0)
               : "memory");
}

// The same for 4 bytes per lane: LDS[m0 + 4*lane] <- buffer[voff].
__device__ __forceinline__ void dma4(const u32x4_t& rsrc, unsigned voff, unsigned m0) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0)
               : "memory");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Buffer resource for `bytes` bytes from `base` (raw, stride 0: offsets at or
// beyond `bytes` read as zero).
__device__ __forceinline__ u32x4_t make_rsrc(const char* base, unsigned bytes) {
  const unsigned long long p = (unsigned long long)base;
  u32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)p);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even conversions of fp32 pairs to 16-bit types, packed.
__device__ __forceinline__ unsigned pack2(float a, float b, __bf16*) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}
__device__ __forceinline__ unsigned pack2(float a, float b, _Float16*) {
  f16x2_t v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(unsigned, v);
}

// Two packed fp16 values of a 32-bit word.  The word is taken by value: a
// bit cast applied directly to a vector element expression reads element 0.
__device__ __forceinline__ f16x2_t as_f16x2(unsigned w) { return __builtin_bit_cast(f16x2_t, w); }

// 16-bit element -> fp32 (exact).
__device__ __forceinline__ float lo_bf16(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

// ---------------------------------------------------------------------------
// Attention dropout: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// Random Numbers: As Easy as 1, 2, 3", SC 2011).  A round multiplies words 0
// and 2 by the two Philox multipliers; the new words are (hi(M1*x2) ^ x1 ^
// k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1, lo(M0*x0)); the key advances by the two
// Weyl constants after each round.  Ten rounds.
//
// Keep decisions: pair (query i, key j) of batch b and head h takes byte
// (j mod 4) of word ((j / 4) mod 4) of Philox(counter (j / 16, i, h, b), key
// (seed low, seed high)), least significant byte first, and is kept iff the
// byte is >= t = round(256 p).
// ---------------------------------------------------------------------------
struct Philox4 {
  uint32_t w[4];
};
// a ^ b ^ k (k wave-uniform) in one instruction: v_bitop3_b32 with truth
// table 0x96 (its inputs' columns are 0xF0, 0xCC, 0xAA); the compiler's own
// form is two exclusive-ors
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}
// The counter words that are wave-uniform (head and batch) keep parts of the
// first two rounds on the scalar unit, so those rounds stay in plain code;
// from the third round on every state word is per-lane.
// OPAQUE_KEYS: the keys enter opaque, so each call steps them on the scalar
// unit.  Left visible, the compiler hoists all twenty round keys out of the
// caller's loop; in the forward's dropout instance they then no longer fit the
// scalar registers and sit in vector lanes (a v_readlane per use in the loop).
// Measured per caller: +3.7-3.9 % on that instance, 2-3 % slower on the others.
template <bool OPAQUE_KEYS = false>
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
  if constexpr (OPAQUE_KEYS) asm volatile("" : "+s"(k0), "+s"(k1));
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = r < 2 ? (uint32_t)(p1 >> 32) ^ c1 ^ k0 : xor3((uint32_t)(p1 >> 32), c1, k0);
    const uint32_t n2 = r < 2 ? (uint32_t)(p0 >> 32) ^ c3 ^ k1 : xor3((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// The value lane l^32 holds (v_permlane32_swap returns the lane's own value
// in one result and its partner's in the other; equal values are the same
// either way).
__device__ __forceinline__ uint32_t partner32(uint32_t x) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return r[0] == x ? r[1] : r[0];
}

// Keep words of one 32-key block for a lane whose MFMA registers r hold keys
// 8*(r>>2) + 4*hh + (r&3) of the block (lanes = queries, row i): lanes with
// hh = 0 draw the block's first 16-key group, hh = 1 the second, and the
// halves trade the words the other needs.  Word g serves registers 4g..4g+3
// (byte r&3).
template <bool OPAQUE_KEYS = false>
__device__ __forceinline__ void keep_words_rows(uint32_t kw[4], int group0, int hh, int i, int h,
                                                int b, uint32_t s0, uint32_t s1) {
  const Philox4 x =
      philox4x32_10<OPAQUE_KEYS>((uint32_t)(group0 + hh), (uint32_t)i, (uint32_t)h, (uint32_t)b, s0, s1);
  const uint32_t send0 = hh ? x.w[0] : x.w[1];
  const uint32_t send1 = hh ? x.w[2] : x.w[3];
  const uint32_t got0 = partner32(send0), got1 = partner32(send1);
  kw[0] = hh ? got0 : x.w[0];
  kw[1] = hh ? got1 : x.w[2];
  kw[2] = hh ? x.w[1] : got0;
  kw[3] = hh ? x.w[3] : got1;
}

__device__ __forceinline__ bool kept(uint32_t word, int byte, uint32_t t) {
  return ((word >> (8 * byte)) & 0xffu) >= t;
}

}  // namespace fa
