// Split-KV decode kernels of libfa355: one query row per (batch, head)
// against a padded key/value cache.
//
// Decode has a single query row, so the parallel work has to come from the
// keys (the slavadubrov.com page, table row on prefill versus single-token
// decode).  The cache of each (batch, head) is cut into chunks; each chunk
// is summarised by its maximum m_c, its sum l_c and its unnormalised output
// O_c, and the summaries are merged in a fixed order — the block summary and
// pairwise merge of the CSDN primer 轻松读懂FlashAttention 上, section
// Softmax求解重构, and the running (m, l) of the Ascend CANN explainer's
// 原理 step 3.
//
// gfx950 mapping (ours):
//  * partial kernel: one workgroup of chunk/64 waves per (batch, chunk,
//    head) work item, numbered chunk-major with heads fastest so that
//    workgroups dispatched together read the contiguous all-heads stretch
//    of the cache.  Each wave issues every 16-byte K and V load of its 64
//    keys up front (up to 32 KB in flight per wave) — the path is bound by
//    HBM bandwidth, so the VALU work (dot products, exp2, P·V) is kept
//    simple and overlapped by the loads of other waves.
//  * combine kernel: one wave per (batch, head) merges the chunk summaries
//    in chunk order, with the loads of eight chunks in flight together; the
//    result is bit-reproducible.

#include <math.h>

#include <type_traits>

#include "fa_device.h"
#include "launch.h"

namespace fa {

// Reduction of a value over the `width` lanes (8 or 16) of a lane group, via
// DPP within rows of 16 lanes; afterwards every lane of the group holds it.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // xor 1
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));   // xor 2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));  // half-row mirror
  if constexpr (W == 16)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));  // row mirror
  return x;
}

// Lanes 8 apart within a row of 16 (row rotate by 8).
__device__ __forceinline__ float xor8_max(float x) {
  return fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false)));
}
__device__ __forceinline__ float xor8_sum(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}

// Dot product of 8 elements held as 16 bytes, against q in fp32.
__device__ __forceinline__ float dot8(const u32x4_t& k, const float* q, __bf16*) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s = __builtin_fmaf(lo_bf16(k[e]), q[2 * e], s);
    s = __builtin_fmaf(hi_bf16(k[e]), q[2 * e + 1], s);
  }
  return s;
}
__device__ __forceinline__ float dot8(const u32x4_t& k, const float* q, _Float16*) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f16x2_t h = as_f16x2(k[e]);
    s = __builtin_fmaf((float)h[0], q[2 * e], s);
    s = __builtin_fmaf((float)h[1], q[2 * e + 1], s);
  }
  return s;
}
__device__ __forceinline__ float dot8(const u32x4_t& k, const float* q, float*) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s = __builtin_fmaf(__uint_as_float(k[e]), q[e], s);
  return s;
}

// o[0..EPL) += p * v (EPL elements held in 16 bytes).
__device__ __forceinline__ void axpy(float* o, float p, const u32x4_t& v, __bf16*) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[2 * e] = __builtin_fmaf(p, lo_bf16(v[e]), o[2 * e]);
    o[2 * e + 1] = __builtin_fmaf(p, hi_bf16(v[e]), o[2 * e + 1]);
  }
}
__device__ __forceinline__ void axpy(float* o, float p, const u32x4_t& v, _Float16*) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f16x2_t h = as_f16x2(v[e]);
    o[2 * e] = __builtin_fmaf(p, (float)h[0], o[2 * e]);
    o[2 * e + 1] = __builtin_fmaf(p, (float)h[1], o[2 * e + 1]);
  }
}
__device__ __forceinline__ void axpy(float* o, float p, const u32x4_t& v, float*) {
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(p, __uint_as_float(v[e]), o[e]);
}

// Cache rows are read exactly once per call: non-temporal loads keep them
// from displacing reusable lines (measured about 6 % faster than plain loads).
__device__ __forceinline__ u32x4_t stream_load(const u32x4_t* p) {
  return __builtin_nontemporal_load(p);
}

// NW waves of KPW keys each cover one chunk of NW*KPW keys.  PAGED: the
// cache is a pool of pages of 2^page_shift rows and block_table maps a batch
// entry's key t to row t mod 2^page_shift of page block_table[b][t >> shift].
template <typename T, int D, int NW, int KPW, bool PAGED>
__global__ __launch_bounds__(NW * 64) void decode_partial_kernel(DecodeArgs a) {
  constexpr int ES = Elem<T>::kBytes;
  constexpr int EPL = 16 / ES;          // elements per 16-byte slice
  constexpr int LPK = D * ES / 16;      // lanes per key row
  constexpr int KPI = 64 / LPK;         // keys per wave-wide load
  constexpr int NI = KPW / KPI;         // loads per lane for the wave's keys
  static_assert(KPW % KPI == 0, "keys per wave must fill whole loads");
  static_assert(LPK == 8 || LPK == 16 || LPK == 32, "unsupported row width");

  __shared__ float red_m[NW];
  __shared__ float red_l[NW];
  __shared__ float red_o[NW][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kk = lane / LPK;            // key slot within a wave-wide load
  const int dd = lane % LPK;            // 16-byte slice of the row

  const size_t rs = (size_t)a.H * D;    // elements between cache rows
  {
    const int it = blockIdx.x;          // host guarantees NC*B*H < 2^31
    const int cb = it / a.H;
    const int h = it - cb * a.H;
    const int c = cb / a.B;
    const int b = cb - c * a.B;
    const int lk = min(max(a.seqlens_k[b], 0), a.Nk_max);
    if (c * a.chunk >= lk) return;      // uniform over the workgroup

    const int key0 = c * a.chunk + wave * KPW;
    // first row of this batch entry's cache (the page pool for a paged cache)
    const size_t row0 = PAGED ? 0 : (size_t)b * a.Nk_max;
    const char* kb = (const char*)((const T*)a.kc + row0 * rs + (size_t)h * D) + dd * 16;
    const char* vb = (const char*)((const T*)a.vc + row0 * rs + (size_t)h * D) + dd * 16;
    u32x4_t kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int key = key0 + i * KPI + kk;
      size_t row = (size_t)key;
      if constexpr (PAGED) {
        // The KPI keys of one load lie in one aligned group of at most 8 and
        // pages hold at least 16 rows, so the page is the same for the whole
        // wave: one scalar load, only for groups inside the sequence.  An id
        // outside the pool is clamped into it (no read leaves the cache).
        const int kbase = key0 + i * KPI;
        int pg = 0;
        if (kbase < lk) pg = a.block_table[(size_t)b * a.max_pages + (kbase >> a.page_shift)];
        pg = min(max(pg, 0), a.num_pages - 1);
        row = ((size_t)pg << a.page_shift) + (size_t)(key & ((1 << a.page_shift) - 1));
      }
      if (key < lk) {
        kr[i] = stream_load((const u32x4_t*)(kb + row * rs * ES));
        vr[i] = stream_load((const u32x4_t*)(vb + row * rs * ES));
      } else {
        kr[i] = u32x4_t{};
        vr[i] = u32x4_t{};
      }
    }
    // this lane's slice of q, in fp32
    float qv[EPL];
    {
      const u32x4_t qr = *(const u32x4_t*)((const char*)((const T*)a.q + ((size_t)b * a.H + h) * D) + dd * 16);
      if constexpr (ES == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[e] = __uint_as_float(qr[e]);
      } else if constexpr (sizeof(T) == 2 && __is_same(T, __bf16)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) { qv[2 * e] = lo_bf16(qr[e]); qv[2 * e + 1] = hi_bf16(qr[e]); }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f16x2_t hv = as_f16x2(qr[e]);
          qv[2 * e] = (float)hv[0];
          qv[2 * e + 1] = (float)hv[1];
        }
      }
    }
    // scores in units of scale*log2(e)
    float x[NI];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float s = group_sum<(LPK >= 16 ? 16 : 8)>(dot8(kr[i], qv, (T*)nullptr));
      if constexpr (LPK == 32) s = quarter_sum(s);
      x[i] = (key0 + i * KPI + kk < lk) ? s * a.c : -INFINITY;
      mx = fmaxf(mx, x[i]);
    }
    // maximum over the wave's keys (lane groups 16 / 32 apart, and 8 apart for D*ES = 128)
    if constexpr (LPK == 8) mx = xor8_max(mx);
    if constexpr (LPK <= 16) mx = quarter_max(mx);
    mx = half_max(mx);
    if (lane == 0) red_m[wave] = mx;
    __syncthreads();
    float M = red_m[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, red_m[w]);
    const float Ms = (M == -INFINITY) ? 0.f : M;

    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float p = fast_exp2(x[i] - Ms);
      l += p;
      axpy(o, p, vr[i], (T*)nullptr);
    }
    // sum over the key slots of the wave
    if constexpr (LPK == 8) {
      l = xor8_sum(l);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = xor8_sum(o[e]);
    }
    if constexpr (LPK <= 16) {
      l = quarter_sum(l);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = quarter_sum(o[e]);
    }
    l = half_sum(l);
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = half_sum(o[e]);
    if (kk == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_o[wave][dd * EPL + e] = o[e];
      if (dd == 0) red_l[wave] = l;
    }
    __syncthreads();
    const size_t rec = ((size_t)b * a.H + h) * a.NC + c;
    for (int d = tid; d < D; d += NW * 64) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red_o[w][d];
      a.ws_o[rec * D + d] = s;
    }
    if (tid == 0) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red_l[w];
      a.ws_ml[rec * 2 + 0] = M;
      a.ws_ml[rec * 2 + 1] = s;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  constexpr int DPL = D / 64;  // output elements per lane (1 or 2), loaded together
  constexpr int U = 8;         // chunks whose loads are issued together
  using vec = typename std::conditional<DPL == 2, float2, float>::type;
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int lk = min(max(a.seqlens_k[b], 0), a.Nk_max);
  const int nck = (lk + a.chunk - 1) / a.chunk;
  const float2* ml = (const float2*)(a.ws_ml + (size_t)bh * a.NC * 2);
  const vec* po = (const vec*)(a.ws_o + (size_t)bh * a.NC * D) + lane;

  float M = -INFINITY;
  for (int c = lane; c < nck; c += 64) M = fmaxf(M, ml[c].x);
  // wave-wide maximum (order does not matter for max)
  M = fmaxf(M, __shfl_xor(M, 1));
  M = fmaxf(M, __shfl_xor(M, 2));
  M = fmaxf(M, __shfl_xor(M, 4));
  M = fmaxf(M, __shfl_xor(M, 8));
  M = fmaxf(M, __shfl_xor(M, 16));
  M = fmaxf(M, __shfl_xor(M, 32));
  const float Ms = (M == -INFINITY) ? 0.f : M;

  float L = 0.f;
  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  // fixed chunk order; the loads of U chunks are in flight together
  for (int c0 = 0; c0 < nck; c0 += U) {
    float2 mlv[U];
    vec pv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + u, nck - 1);
      mlv[u] = ml[c];
      pv[u] = po[(size_t)c * (D / DPL)];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u < nck) {
        const float w = fast_exp2(mlv[u].x - Ms);
        L = __builtin_fmaf(w, mlv[u].y, L);
        if constexpr (DPL == 2) {
          o[0] = __builtin_fmaf(w, pv[u].x, o[0]);
          o[1] = __builtin_fmaf(w, pv[u].y, o[1]);
        } else {
          o[0] = __builtin_fmaf(w, pv[u], o[0]);
        }
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  T* out = (T*)a.o + (size_t)bh * D + lane * DPL;
#pragma unroll
  for (int e = 0; e < DPL; ++e) out[e] = (T)(o[e] * inv);
  if (lane == 0 && a.lse) a.lse[bh] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
}

constexpr int kDecodeKPW = 64;  // keys per wave of a chunk

template <typename T, int D, int CHUNK, bool PAGED>
static hipError_t launch_chunk(const DecodeArgs& a, hipStream_t stream) {
  constexpr int KPW = CHUNK < kDecodeKPW ? CHUNK : kDecodeKPW;  // keys per wave
  constexpr int NW = CHUNK / KPW;
  // One workgroup per work item: finished workgroups are replaced at once,
  // so the load phase of some overlaps the arithmetic of others.  (A
  // resident grid striding over the items runs its workgroups in step and
  // was measured slower.)
  const unsigned grid = (unsigned)((long long)a.NC * a.B * a.H);
  if (grid > 0)
    hipLaunchKernelGGL((decode_partial_kernel<T, D, NW, KPW, PAGED>), dim3(grid), dim3(NW * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.B * a.H), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, bool PAGED>
static hipError_t launch_tdp(const DecodeArgs& a, hipStream_t stream) {
  switch (a.chunk) {
    case 64: return launch_chunk<T, D, 64, PAGED>(a, stream);
    case 128: return launch_chunk<T, D, 128, PAGED>(a, stream);
    case 256: return launch_chunk<T, D, 256, PAGED>(a, stream);
    default: return launch_chunk<T, D, 512, PAGED>(a, stream);
  }
}

template <typename T, int D>
static hipError_t launch_td(const DecodeArgs& a, hipStream_t stream) {
  return a.block_table ? launch_tdp<T, D, true>(a, stream) : launch_tdp<T, D, false>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, fa_dtype_t dtype, int D, hipStream_t stream) {
  switch (dtype) {
    case FA_BF16: return D == 64 ? launch_td<__bf16, 64>(a, stream) : launch_td<__bf16, 128>(a, stream);
    case FA_F16: return D == 64 ? launch_td<_Float16, 64>(a, stream) : launch_td<_Float16, 128>(a, stream);
    default: return D == 64 ? launch_td<float, 64>(a, stream) : launch_td<float, 128>(a, stream);
  }
}

}  // namespace fa
