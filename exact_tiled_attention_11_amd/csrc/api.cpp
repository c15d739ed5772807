// libfa355 C ABI: argument validation, kernel selection and launch.
//
// Every check runs before the first HIP call, so invalid arguments are
// reported identically on machines without a GPU.  The mapping of the
// Hugging Face Flash-Attention-2 guide's error catalog (section 常见错误排查:
// unsupported dtype, unsupported head_dim, unsupported GPU) onto status
// codes is: dtype and head_dim -> FA_ERR_UNSUPPORTED, device -> FA_ERR_HIP.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "fa355.h"
#include "launch.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = not yet checked, 1 = gfx950, 2 = something else.  A benign cache:
// racing threads compute the same answer.
std::atomic<int> g_dev_ok[kMaxDevices];

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool dtype_ok(fa_dtype_t d) { return d == FA_F32 || d == FA_F16 || d == FA_BF16; }

size_t esize(fa_dtype_t d) { return d == FA_F32 ? 4 : 2; }

// Current device must be a gfx950; checked once per device.
fa_status_t device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_HIP;
  if (dev < kMaxDevices) {
    const int s = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (s == 1) return FA_OK;
    if (s == 2) return FA_ERR_HIP;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_HIP;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FA_OK : FA_ERR_HIP;
}

fa_status_t from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

constexpr float kLog2eF = 1.4426950408889634f;

// Dropout probability -> byte threshold t = round(256 p) (at most 255); the
// kept weights are scaled by 256 / (256 - t).
bool drop_threshold(float p, uint32_t& t, float& scale) {
  if (!(p >= 0.f && p < 1.f)) return false;
  const double x = floor((double)p * 256.0 + 0.5);
  t = x > 255.0 ? 255u : (uint32_t)x;
  scale = (float)(256.0 / (256.0 - (double)t));
  return true;
}

// Fixed-length prefill with the optional mask families and dropout.
fa_status_t fwd_fixed(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Nq, int Nk, int D, float scale, int causal,
                      const int32_t* seqlens_k, int prefix, const float* alibi_slopes,
                      uint32_t drop_t, float drop_scale, uint64_t seed, fa_dtype_t dtype,
                      void* stream) {
  if (!dtype_ok(dtype) || (D != 64 && D != 128)) return FA_ERR_UNSUPPORTED;
  // the mask families and dropout are implemented by the 16-bit kernel only
  if (dtype == FA_F32 && (prefix != 0 || alibi_slopes || drop_t)) return FA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || Nq < 0 || Nk < 0) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  if ((causal != 0 && causal != 1)) return FA_ERR_INVALID_ARG;
  if (prefix < 0 || (prefix > 0 && !causal)) return FA_ERR_INVALID_ARG;
  if (Nq == 0) return FA_OK;
  if (!q || !o || ((!k || !v) && Nk > 0)) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(seqlens_k) || ((uintptr_t)alibi_slopes & 3u) != 0)
    return FA_ERR_INVALID_ARG;
  // element offsets must fit the kernels' 64-bit address math and grid limits
  const int rows = fa::fwd_block_rows(dtype, D);
  const long long nqb = ((long long)Nq + rows - 1) / rows;
  const long long grid = nqb * B * H;
  if (grid > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  if ((long long)B * Nq > 0x7fffffffLL || (long long)B * Nk > 0x7fffffffLL) return FA_ERR_INVALID_ARG;

  fa_status_t st = device_ok();
  if (st != FA_OK) return st;

  fa::FwdArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.seqlens_k = seqlens_k;
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.nqb = (int)nqb;
  a.c = fmaxf(scale * kLog2eF, 1e-30f);  // a zero scale acts as a vanishing one
  a.prefix = prefix;
  a.alibi = alibi_slopes;
  a.drop_t = drop_t;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.drop_scale = drop_scale;
  return from_hip(fa::launch_fwd(a, dtype, D, causal != 0, false, (unsigned)grid,
                                 (hipStream_t)stream));
}

fa_status_t bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
                     int D, float scale, int causal, const int32_t* seqlens_k, int prefix,
                     const float* alibi_slopes, uint32_t drop_t, float drop_scale, uint64_t seed,
                     void* workspace, size_t workspace_bytes, fa_dtype_t dtype, void* stream);
fa_status_t fwd_varlen_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                            int total_q, int total_k, int H, int D, float scale, int causal,
                            int prefix, const float* alibi_slopes, uint32_t drop_t,
                            float drop_scale, uint64_t seed, void* workspace,
                            size_t workspace_bytes, fa_dtype_t dtype, void* stream,
                            bool use_scratch = false);

}  // namespace

extern "C" {

const char* fa_status_string(fa_status_t s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head_dim, dtype or chunk size";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP error or no gfx950 device";
    case FA_ERR_TOO_LARGE: return "problem exceeds the static scratch of the no-allocation call";
    default: return "unknown status";
  }
}

const char* fa_version(void) { return "libfa355 0.1.0 (gfx950)"; }

fa_status_t fa_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int Nq, int Nk, int D, float scale, int causal,
                          const int32_t* seqlens_k, int prefix, const float* alibi_slopes,
                          fa_dtype_t dtype, void* stream) {
  return fwd_fixed(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, seqlens_k, prefix,
                   alibi_slopes, 0u, 1.f, 0u, dtype, stream);
}

fa_status_t fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int D, float scale, int causal,
                           const int32_t* seqlens_k, float dropout_p, uint64_t seed,
                           fa_dtype_t dtype, void* stream) {
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;  // the dropout kernels are 16-bit only
  uint32_t t = 0;
  float sc = 1.f;
  if (!drop_threshold(dropout_p, t, sc)) return FA_ERR_INVALID_ARG;
  return fwd_fixed(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, seqlens_k, 0, nullptr, t, sc,
                   seed, dtype, stream);
}

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int Nq, int Nk, int D, float scale, int causal,
                   const int32_t* seqlens_k, fa_dtype_t dtype, void* stream) {
  return fa_fwd_masked(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, seqlens_k, 0, nullptr,
                       dtype, stream);
}

// Half of the gradient workspace: one float per (batch, head, query row).
static size_t bwd_half_bytes(int B, int H, int Nq) {
  const size_t n = (size_t)B * H * (Nq > 0 ? Nq : 1);
  return (n * 4 + 255) / 256 * 256;
}

size_t fa_bwd_workspace_bytes(int B, int H, int Nq) {
  if (B < 1 || H < 1 || Nq < 0) return 0;
  return 2 * bwd_half_bytes(B, H, Nq);  // rowsum(dO o O), then lse in exp2 units
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
                   int D, float scale, int causal, const int32_t* seqlens_k, void* workspace,
                   size_t workspace_bytes, fa_dtype_t dtype, void* stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, seqlens_k, 0,
                  nullptr, 0u, 1.f, 0u, workspace, workspace_bytes, dtype, stream);
}

fa_status_t fa_bwd_masked(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                          int H, int Nq, int Nk, int D, float scale, int causal,
                          const int32_t* seqlens_k, int prefix, const float* alibi_slopes,
                          void* workspace, size_t workspace_bytes, fa_dtype_t dtype,
                          void* stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, seqlens_k,
                  prefix, alibi_slopes, 0u, 1.f, 0u, workspace, workspace_bytes, dtype, stream);
}

fa_status_t fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int H, int Nq, int Nk, int D, float scale, int causal,
                           const int32_t* seqlens_k, float dropout_p, uint64_t seed,
                           void* workspace, size_t workspace_bytes, fa_dtype_t dtype,
                           void* stream) {
  uint32_t t = 0;
  float sc = 1.f;
  if (!drop_threshold(dropout_p, t, sc)) return FA_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, seqlens_k, 0,
                  nullptr, t, sc, seed, workspace, workspace_bytes, dtype, stream);
}

}  // extern "C"

namespace {

fa_status_t bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
                     int D, float scale, int causal, const int32_t* seqlens_k, int prefix,
                     const float* alibi_slopes, uint32_t drop_t, float drop_scale, uint64_t seed,
                     void* workspace, size_t workspace_bytes, fa_dtype_t dtype, void* stream) {
  if (!dtype_ok(dtype) || (D != 64 && D != 128)) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;  // the backward kernels are 16-bit only
  if (B < 1 || H < 1 || Nq < 0 || Nk < 0) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (prefix < 0 || (prefix > 0 && !causal)) return FA_ERR_INVALID_ARG;
  if (((uintptr_t)alibi_slopes & 3u) != 0) return FA_ERR_INVALID_ARG;
  if (Nq == 0 && Nk == 0) return FA_OK;
  if ((Nq > 0 && (!q || !o || !lse || !dout || !dq)) || (Nk > 0 && (!k || !v || !dk || !dv)))
    return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(lse) ||
      !aligned16(seqlens_k) || !aligned16(workspace))
    return FA_ERR_INVALID_ARG;
  const long long rows = fa::bwd_block_rows();
  const long long nbh = (long long)B * H;
  if (((long long)Nq + rows - 1) / rows * nbh > 0x7fffffffLL ||
      ((long long)Nk + rows - 1) / rows * nbh > 0x7fffffffLL)
    return FA_ERR_INVALID_ARG;
  if ((long long)B * Nq * H > 0x7fffffffLL * 256LL) return FA_ERR_INVALID_ARG;
  if ((long long)B * Nq > 0x7fffffffLL || (long long)B * Nk > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, H, Nq)) return FA_ERR_WORKSPACE;

  fa_status_t st = device_ok();
  if (st != FA_OK) return st;

  fa::BwdArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.delta = (float*)workspace;
  a.lse2 = (float*)((char*)workspace + bwd_half_bytes(B, H, Nq));
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.seqlens_k = seqlens_k;
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.nqb = (int)((Nq + rows - 1) / rows);
  a.c = fmaxf(scale * kLog2eF, 1e-30f);  // the forward's exponent scale
  a.scale = scale;
  a.drop_t = drop_t;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.drop_scale = drop_scale;
  a.prefix = prefix;
  a.alibi = alibi_slopes;
  return from_hip(fa::launch_bwd(a, dtype, D, causal != 0, (hipStream_t)stream));
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

fa_status_t bwd_varlen_impl(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                            int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int H,
                            int D, float scale, int causal, int prefix,
                            const float* alibi_slopes, uint32_t drop_t, float drop_scale,
                            uint64_t seed, void* workspace, size_t workspace_bytes,
                            fa_dtype_t dtype, void* stream) {
  if (!dtype_ok(dtype) || (D != 64 && D != 128)) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;  // the backward kernels are 16-bit only
  if (nseq < 1 || H < 1 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (prefix < 0 || (prefix > 0 && !causal)) return FA_ERR_INVALID_ARG;
  if (((uintptr_t)alibi_slopes & 3u) != 0) return FA_ERR_INVALID_ARG;
  if (!cu_seqlens_q || !cu_seqlens_k || ((uintptr_t)cu_seqlens_q & 3u) != 0 ||
      ((uintptr_t)cu_seqlens_k & 3u) != 0)
    return FA_ERR_INVALID_ARG;
  if (total_q == 0 && total_k == 0) return FA_OK;
  if ((total_q > 0 && (!q || !o || !lse || !dout || !dq)) ||
      (total_k > 0 && (!k || !v || !dk || !dv)))
    return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(lse) ||
      !aligned16(workspace))
    return FA_ERR_INVALID_ARG;
  const long long rows = fa::bwd_block_rows();
  const long long nsh = (long long)nseq * H;
  if (((long long)max_seqlen_q + rows - 1) / rows * nsh > 0x7fffffffLL ||
      ((long long)max_seqlen_k + rows - 1) / rows * nsh > 0x7fffffffLL)
    return FA_ERR_INVALID_ARG;
  if ((long long)total_q * H > 0x7fffffffLL * 256LL) return FA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(1, H, total_q)) return FA_ERR_WORKSPACE;

  fa_status_t st = device_ok();
  if (st != FA_OK) return st;

  fa::BwdArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.delta = (float*)workspace;
  a.lse2 = (float*)((char*)workspace + bwd_half_bytes(1, H, total_q));
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = nseq;
  a.H = H;
  a.Nq = max_seqlen_q;
  a.Nk = max_seqlen_k;
  a.nqb = (int)((max_seqlen_q + rows - 1) / rows);
  a.c = fmaxf(scale * kLog2eF, 1e-30f);
  a.scale = scale;
  a.drop_t = drop_t;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.drop_scale = drop_scale;
  a.prefix = prefix;
  a.alibi = alibi_slopes;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  return from_hip(fa::launch_bwd(a, dtype, D, causal != 0, (hipStream_t)stream));
}

}  // namespace

extern "C" {

fa_status_t fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                          int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int H,
                          int D, float scale, int causal, void* workspace, size_t workspace_bytes,
                          fa_dtype_t dtype, void* stream) {
  return bwd_varlen_impl(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, nseq,
                         total_q, total_k, max_seqlen_q, max_seqlen_k, H, D, scale, causal, 0,
                         nullptr, 0u, 1.f, 0u, workspace, workspace_bytes, dtype, stream);
}

fa_status_t fa_bwd_varlen_masked(const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, const void* dout, void* dq, void* dk,
                                 void* dv, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int nseq, int total_q, int total_k,
                                 int max_seqlen_q, int max_seqlen_k, int H, int D, float scale,
                                 int causal, int prefix, const float* alibi_slopes,
                                 void* workspace, size_t workspace_bytes, fa_dtype_t dtype,
                                 void* stream) {
  return bwd_varlen_impl(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, nseq,
                         total_q, total_k, max_seqlen_q, max_seqlen_k, H, D, scale, causal,
                         prefix, alibi_slopes, 0u, 1.f, 0u, workspace, workspace_bytes, dtype,
                         stream);
}

fa_status_t fa_bwd_varlen_dropout(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout, void* dq, void* dk,
                                  void* dv, const int32_t* cu_seqlens_q,
                                  const int32_t* cu_seqlens_k, int nseq, int total_q,
                                  int total_k, int max_seqlen_q, int max_seqlen_k, int H, int D,
                                  float scale, int causal, float dropout_p, uint64_t seed,
                                  void* workspace, size_t workspace_bytes, fa_dtype_t dtype,
                                  void* stream) {
  uint32_t t = 0;
  float sc = 1.f;
  if (!drop_threshold(dropout_p, t, sc)) return FA_ERR_INVALID_ARG;
  return bwd_varlen_impl(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, nseq,
                         total_q, total_k, max_seqlen_q, max_seqlen_k, H, D, scale, causal, 0,
                         nullptr, t, sc, seed, workspace, workspace_bytes, dtype, stream);
}

// Every option at once (the mask families and dropout together).
fa_status_t fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Nq, int Nk, int D, float scale, int causal,
                      const int32_t* seqlens_k, int prefix, const float* alibi_slopes,
                      float dropout_p, uint64_t seed, fa_dtype_t dtype, void* stream) {
  uint32_t t = 0;
  float sc = 1.f;
  if (!drop_threshold(dropout_p, t, sc)) return FA_ERR_INVALID_ARG;
  return fwd_fixed(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, seqlens_k, prefix,
                   alibi_slopes, t, sc, seed, dtype, stream);
}

fa_status_t fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, int B, int H, int Nq,
                      int Nk, int D, float scale, int causal, const int32_t* seqlens_k,
                      int prefix, const float* alibi_slopes, float dropout_p, uint64_t seed,
                      void* workspace, size_t workspace_bytes, fa_dtype_t dtype, void* stream) {
  uint32_t t = 0;
  float sc = 1.f;
  if (!drop_threshold(dropout_p, t, sc)) return FA_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, seqlens_k,
                  prefix, alibi_slopes, t, sc, seed, workspace, workspace_bytes, dtype, stream);
}

fa_status_t fa_fwd_varlen_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                             int total_q, int total_k, int H, int D, float scale, int causal,
                             int prefix, const float* alibi_slopes, float dropout_p,
                             uint64_t seed, void* workspace, size_t workspace_bytes,
                             fa_dtype_t dtype, void* stream) {
  uint32_t t = 0;
  float sc = 1.f;
  if (!drop_threshold(dropout_p, t, sc)) return FA_ERR_INVALID_ARG;
  return fwd_varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k, H,
                         D, scale, causal, prefix, alibi_slopes, t, sc, seed, workspace,
                         workspace_bytes, dtype, stream);
}

fa_status_t fa_bwd_varlen_ex(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                             int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int H,
                             int D, float scale, int causal, int prefix,
                             const float* alibi_slopes, float dropout_p, uint64_t seed,
                             void* workspace, size_t workspace_bytes, fa_dtype_t dtype,
                             void* stream) {
  uint32_t t = 0;
  float sc = 1.f;
  if (!drop_threshold(dropout_p, t, sc)) return FA_ERR_INVALID_ARG;
  return bwd_varlen_impl(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, nseq,
                         total_q, total_k, max_seqlen_q, max_seqlen_k, H, D, scale, causal,
                         prefix, alibi_slopes, t, sc, seed, workspace, workspace_bytes, dtype,
                         stream);
}

size_t fa_fwd_varlen_workspace_bytes(int nseq, int total_q) {
  if (nseq < 1 || total_q < 0) return 0;
  // the smallest query block of any instance bounds the tile count from above
  int rows = fa::fwd_block_rows(FA_F32, 64);
  const fa_dtype_t dts[3] = {FA_F32, FA_F16, FA_BF16};
  for (fa_dtype_t dt : dts)
    for (int d = 64; d <= 128; d += 64) rows = rows < fa::fwd_block_rows(dt, d) ? rows : fa::fwd_block_rows(dt, d);
  return fa::varlen_sched_bytes(nseq, fa::varlen_max_tiles(nseq, total_q, rows));
}

}  // extern "C"

namespace {

// Packed prefill with the optional mask families and dropout.
fa_status_t fwd_varlen_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                            int total_q, int total_k, int H, int D, float scale, int causal,
                            int prefix, const float* alibi_slopes, uint32_t drop_t,
                            float drop_scale, uint64_t seed, void* workspace,
                            size_t workspace_bytes, fa_dtype_t dtype, void* stream,
                            bool use_scratch) {
  if (!dtype_ok(dtype) || (D != 64 && D != 128)) return FA_ERR_UNSUPPORTED;
  // the mask families and dropout are implemented by the 16-bit kernel only
  if (dtype == FA_F32 && (prefix != 0 || alibi_slopes || drop_t)) return FA_ERR_UNSUPPORTED;
  if (nseq < 1 || H < 1 || total_q < 0 || total_k < 0) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (prefix < 0 || (prefix > 0 && !causal)) return FA_ERR_INVALID_ARG;
  if (!cu_seqlens_q || !cu_seqlens_k) return FA_ERR_INVALID_ARG;
  if (total_q == 0) return FA_OK;
  if (!q || !o || ((!k || !v) && total_k > 0)) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(workspace) || ((uintptr_t)alibi_slopes & 3u) != 0)
    return FA_ERR_INVALID_ARG;
  const int rows = fa::fwd_block_rows(dtype, D);
  const long long max_tiles = fa::varlen_max_tiles(nseq, total_q, rows);
  if (max_tiles * H > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  const size_t need = fa::varlen_sched_bytes(nseq, max_tiles);
  if (use_scratch) {
    if (need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_TOO_LARGE;
  } else if (!workspace || workspace_bytes < need) {
    return FA_ERR_WORKSPACE;
  }

  fa_status_t st = device_ok();
  if (st != FA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (use_scratch && fa::noalloc_scratch(&workspace) != hipSuccess) return FA_ERR_HIP;

  hipError_t e = fa::launch_varlen_schedule(cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k,
                                            rows, causal,
                                            (int)max_tiles, (int32_t*)workspace, s);
  if (e != hipSuccess) return FA_ERR_HIP;
  fa::FwdArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.sched = (const int32_t*)workspace;
  a.nseq = nseq;
  a.H = H;
  a.total_q = total_q;
  a.c = fmaxf(scale * kLog2eF, 1e-30f);  // a zero scale acts as a vanishing one
  a.prefix = prefix;
  a.alibi = alibi_slopes;
  a.drop_t = drop_t;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.drop_scale = drop_scale;
  return from_hip(fa::launch_fwd(a, dtype, D, causal != 0, true, (unsigned)(max_tiles * H), s));
}

}  // namespace

extern "C" {

fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                          int total_q, int total_k, int H, int D, float scale, int causal,
                          void* workspace, size_t workspace_bytes, fa_dtype_t dtype,
                          void* stream) {
  return fwd_varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k, H,
                         D, scale, causal, 0, nullptr, 0u, 1.f, 0u, workspace, workspace_bytes,
                         dtype, stream);
}

fa_status_t fa_fwd_varlen_noalloc(const void* q, const void* k, const void* v, void* o,
                                  float* lse, const int32_t* cu_seqlens_q,
                                  const int32_t* cu_seqlens_k, int nseq, int total_q,
                                  int total_k, int H, int D, float scale, int causal,
                                  fa_dtype_t dtype, void* stream) {
  return fwd_varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k, H,
                         D, scale, causal, 0, nullptr, 0u, 1.f, 0u, nullptr, 0, dtype, stream,
                         true);
}

fa_status_t fa_fwd_varlen_masked(const void* q, const void* k, const void* v, void* o,
                                 float* lse, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int nseq, int total_q, int total_k,
                                 int H, int D, float scale, int causal, int prefix,
                                 const float* alibi_slopes, void* workspace,
                                 size_t workspace_bytes, fa_dtype_t dtype, void* stream) {
  return fwd_varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k, H,
                         D, scale, causal, prefix, alibi_slopes, 0u, 1.f, 0u, workspace,
                         workspace_bytes, dtype, stream);
}

fa_status_t fa_fwd_varlen_dropout(const void* q, const void* k, const void* v, void* o,
                                  float* lse, const int32_t* cu_seqlens_q,
                                  const int32_t* cu_seqlens_k, int nseq, int total_q,
                                  int total_k, int H, int D, float scale, int causal,
                                  float dropout_p, uint64_t seed, void* workspace,
                                  size_t workspace_bytes, fa_dtype_t dtype, void* stream) {
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;  // the dropout kernels are 16-bit only
  uint32_t t = 0;
  float sc = 1.f;
  if (!drop_threshold(dropout_p, t, sc)) return FA_ERR_INVALID_ARG;
  return fwd_varlen_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k, H,
                         D, scale, causal, 0, nullptr, t, sc, seed, workspace, workspace_bytes,
                         dtype, stream);
}

static bool chunk_ok(int chunk) { return chunk == 64 || chunk == 128 || chunk == 256 || chunk == 512; }

size_t fa_decode_workspace_bytes(int B, int H, int Nk_max, int D, int chunk) {
  if (B < 1 || H < 1 || Nk_max < 0 || (D != 64 && D != 128) || !chunk_ok(chunk)) return 0;
  const size_t nc = ((size_t)Nk_max + chunk - 1) / chunk;
  const size_t recs = (size_t)B * H * (nc > 0 ? nc : 1);
  const size_t o_bytes = (recs * D * 4 + 255) / 256 * 256;
  const size_t ml_bytes = (recs * 2 * 4 + 255) / 256 * 256;
  return o_bytes + ml_bytes;
}

// Shared by the contiguous and the paged decode entry points; `a` carries the
// cache pointers and, for a paged cache, the page table fields.
static fa_status_t decode_common(fa::DecodeArgs& a, const void* q, void* o, float* lse,
                                 const int32_t* seqlens_k, int B, int H, int Nk_max, int D,
                                 float scale, int chunk, void* workspace,
                                 size_t workspace_bytes, fa_dtype_t dtype, void* stream) {
  if (!dtype_ok(dtype) || (D != 64 && D != 128) || !chunk_ok(chunk)) return FA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || Nk_max < 0) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  if (!q || !o || !seqlens_k || ((!a.kc || !a.vc) && Nk_max > 0)) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(a.kc) || !aligned16(a.vc) || !aligned16(o) ||
      !aligned16(lse) || !aligned16(workspace))
    return FA_ERR_INVALID_ARG;
  if ((long long)B * H * (((long long)Nk_max + chunk - 1) / chunk + 1) > 0x7fffffffLL)
    return FA_ERR_INVALID_ARG;
  const size_t need = fa_decode_workspace_bytes(B, H, Nk_max, D, chunk);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;

  fa_status_t st = device_ok();
  if (st != FA_OK) return st;

  const int nc = (Nk_max + chunk - 1) / chunk;
  const size_t recs = (size_t)B * H * (nc > 0 ? nc : 1);
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.seqlens_k = seqlens_k;
  a.ws_o = (float*)workspace;
  a.ws_ml = (float*)((char*)workspace + (recs * D * 4 + 255) / 256 * 256);
  a.B = B;
  a.H = H;
  a.Nk_max = Nk_max;
  a.NC = nc;
  a.chunk = chunk;
  a.c = fmaxf(scale * kLog2eF, 1e-30f);  // a zero scale acts as a vanishing one
  return from_hip(fa::launch_decode(a, dtype, D, (hipStream_t)stream));
}

fa_status_t fa_decode_splitkv(const void* q, const void* k_cache, const void* v_cache, void* o,
                              float* lse, const int32_t* seqlens_k, int B, int H, int Nk_max,
                              int D, float scale, int chunk, void* workspace,
                              size_t workspace_bytes, fa_dtype_t dtype, void* stream) {
  fa::DecodeArgs a = {};
  a.kc = k_cache;
  a.vc = v_cache;
  return decode_common(a, q, o, lse, seqlens_k, B, H, Nk_max, D, scale, chunk, workspace,
                       workspace_bytes, dtype, stream);
}

fa_status_t fa_decode_splitkv_paged(const void* q, const void* k_pages, const void* v_pages,
                                    void* o, float* lse, const int32_t* seqlens_k,
                                    const int32_t* block_table, int B, int H, int num_pages,
                                    int page_size, int max_pages, int D, float scale, int chunk,
                                    void* workspace, size_t workspace_bytes, fa_dtype_t dtype,
                                    void* stream) {
  if (!dtype_ok(dtype) || (D != 64 && D != 128) || !chunk_ok(chunk)) return FA_ERR_UNSUPPORTED;
  if (page_size < 16 || page_size > 1024 || (page_size & (page_size - 1)) != 0)
    return FA_ERR_UNSUPPORTED;
  if (num_pages < 1 || max_pages < 0) return FA_ERR_INVALID_ARG;
  if (!block_table || ((uintptr_t)block_table & 3u) != 0) return FA_ERR_INVALID_ARG;
  const long long nk = (long long)max_pages * page_size;
  if (nk > 0x7fffffffLL || (long long)num_pages * page_size > 0x7fffffffLL)
    return FA_ERR_INVALID_ARG;
  fa::DecodeArgs a = {};
  a.kc = k_pages;
  a.vc = v_pages;
  a.block_table = block_table;
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  a.page_shift = 0;
  while ((1 << a.page_shift) < page_size) ++a.page_shift;
  if (!k_pages || !v_pages) return FA_ERR_INVALID_ARG;
  return decode_common(a, q, o, lse, seqlens_k, B, H, (int)nk, D, scale, chunk, workspace,
                       workspace_bytes, dtype, stream);
}

}  // extern "C"
