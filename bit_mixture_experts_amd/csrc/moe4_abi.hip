// C ABI of libmoe4: argument validation (synchronous, before anything is
// enqueued) and dispatch to the kernel launchers. Every refusal names the
// first offending argument; nothing falls back to another computation
// (project page "experts4bit-qlora", "Do not use this when" and "Limitations --
// qlora-fused-moe-experts": counts or loud refusals, never a silent fallback;
// a base whose epilogue differs from the kernel's is refused).
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "internal.hpp"

namespace {

// Scratch of moe4_expert_forward_noalloc: file-scope device memory, one copy
// on every GPU the library runs on, held until the process ends. In host code
// `scratch` names a host-side stand-in: its device address comes from
// hipGetSymbolAddress, once per device (scratch_of_current_device).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static_assert(MOE4_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes, "moe4.h states the size");
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

thread_local char g_err[512] = "";
thread_local int g_variant = 0;
thread_local hipEvent_t const* g_events = nullptr;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MOE4_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE_PTR(p, name)                                            \
  do {                                                                  \
    if ((p) == nullptr) return fail(MOE4_EINVAL, "%s is NULL", name);   \
  } while (0)
#define REQUIRE_ALIGN(p, a, name)                                                   \
  do {                                                                              \
    if ((p) != nullptr && !aligned((p), (a)))                                       \
      return fail(MOE4_EALIGN, "%s is not %d-byte aligned", name, (int)(a));        \
  } while (0)

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(MOE4_EDEVICE, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// Shared checks of a moe4_experts descriptor.
int check_experts(const moe4_experts* ex) {
  if (ex == nullptr) return fail(MOE4_EINVAL, "moe4_experts is NULL");
  if (ex->format != MOE4_FMT_NF4 && ex->format != MOE4_FMT_MXFP4 &&
      ex->format != MOE4_FMT_NF4_DQ)
    return fail(MOE4_EINVAL, "moe4_experts.format %s (%d)", ex->format ? "unknown" : "unset",
                ex->format);
  if (ex->gu_layout != MOE4_GU_HALVES && ex->gu_layout != MOE4_GU_INTERLEAVED)
    return fail(MOE4_EINVAL, "moe4_experts.gu_layout %s (%d)",
                ex->gu_layout ? "unknown" : "unset", ex->gu_layout);
  if (ex->act != MOE4_ACT_SWIGLU && ex->act != MOE4_ACT_SWIGLU_CLAMPED)
    return fail(MOE4_EINVAL, "moe4_experts.act %s (%d)", ex->act ? "unknown" : "unset", ex->act);
  if (ex->variant != MOE4_VARIANT_AUTO && ex->variant != MOE4_VARIANT_SKINNY &&
      ex->variant != MOE4_VARIANT_TILED)
    return fail(MOE4_EINVAL, "moe4_experts.variant unknown (%d)", ex->variant);
  if (ex->E < 1 || ex->E > 1024)
    return fail(MOE4_ESHAPE, "moe4_experts.E = %d outside [1, 1024]", ex->E);
  if (ex->H <= 0 || ex->I <= 0)
    return fail(MOE4_ESHAPE, "moe4_experts.H = %d, I = %d must be positive", ex->H, ex->I);
  const int blk = ex->format == MOE4_FMT_MXFP4 ? 32 : 64;
  if (ex->H % blk)
    return fail(MOE4_ESHAPE, "moe4_experts.H = %d is not a multiple of %d", ex->H, blk);
  if (ex->I % blk)
    return fail(MOE4_ESHAPE, "moe4_experts.I = %d is not a multiple of %d", ex->I, blk);
  if ((int64_t)ex->E * 2 * ex->I * ex->H > ((int64_t)1 << 40))
    return fail(MOE4_ESHAPE, "moe4_experts: stack of %lld weights is beyond the supported 2^40",
                (long long)ex->E * 2 * ex->I * ex->H);
  // the GEMM kernels address one expert's matrix with 32-bit byte offsets
  if ((int64_t)ex->I * ex->H >= ((int64_t)1 << 31) - ((int64_t)1 << 24))
    return fail(MOE4_ESHAPE, "moe4_experts: I*H = %lld; one expert's packed matrix must stay "
                "under 2 GiB", (long long)ex->I * ex->H);
  // the GEMM kernels address an activation tile (up to 320 rows of K = H or
  // 2I bf16 values) and an output tile (up to 320 rows of H fp32 values) with
  // 32-bit byte offsets
  {
    const int64_t kmax = ex->H > 2 * (int64_t)ex->I ? ex->H : 2 * (int64_t)ex->I;
    if (320 * 4 * kmax >= ((int64_t)1 << 31) - ((int64_t)1 << 24))
      return fail(MOE4_ESHAPE, "moe4_experts: max(H, 2I) = %lld; a 320-row fp32 tile "
                  "must stay under 2 GiB", (long long)kmax);
  }
  REQUIRE_PTR(ex->gu_q, "moe4_experts.gu_q");
  REQUIRE_PTR(ex->gu_s, "moe4_experts.gu_s");
  REQUIRE_PTR(ex->dn_q, "moe4_experts.dn_q");
  REQUIRE_PTR(ex->dn_s, "moe4_experts.dn_s");
  REQUIRE_ALIGN(ex->gu_q, 16, "moe4_experts.gu_q");
  REQUIRE_ALIGN(ex->dn_q, 16, "moe4_experts.dn_q");
  if (ex->format == MOE4_FMT_NF4) {
    REQUIRE_ALIGN(ex->gu_s, 4, "moe4_experts.gu_s");
    REQUIRE_ALIGN(ex->dn_s, 4, "moe4_experts.dn_s");
  }
  if (ex->format == MOE4_FMT_NF4_DQ) {
    REQUIRE_PTR(ex->gu_s2, "moe4_experts.gu_s2");
    REQUIRE_PTR(ex->dn_s2, "moe4_experts.dn_s2");
    REQUIRE_PTR(ex->gu_soff, "moe4_experts.gu_soff");
    REQUIRE_PTR(ex->dn_soff, "moe4_experts.dn_soff");
    REQUIRE_PTR(ex->dq_book, "moe4_experts.dq_book");
    REQUIRE_ALIGN(ex->gu_s2, 4, "moe4_experts.gu_s2");
    REQUIRE_ALIGN(ex->dn_s2, 4, "moe4_experts.dn_s2");
    REQUIRE_ALIGN(ex->gu_soff, 4, "moe4_experts.gu_soff");
    REQUIRE_ALIGN(ex->dn_soff, 4, "moe4_experts.dn_soff");
    REQUIRE_ALIGN(ex->dq_book, 4, "moe4_experts.dq_book");
  } else if (ex->gu_s2 || ex->dn_s2 || ex->gu_soff || ex->dn_soff || ex->dq_book) {
    return fail(MOE4_EINVAL, "moe4_experts: double-quantised absmax fields given for format %d",
                ex->format);
  }
  REQUIRE_ALIGN(ex->gu_bias, 2, "moe4_experts.gu_bias");
  REQUIRE_ALIGN(ex->dn_bias, 2, "moe4_experts.dn_bias");
  if (ex->act == MOE4_ACT_SWIGLU_CLAMPED) {
    if (!(ex->act_limit > 0.0f) || !(ex->act_alpha > 0.0f))
      return fail(MOE4_EINVAL,
                  "moe4_experts.act_alpha/act_limit must be positive for the clamped GLU "
                  "(got %g, %g)",
                  (double)ex->act_alpha, (double)ex->act_limit);
  }
  if ((ex->lora_A == nullptr) != (ex->lora_B == nullptr))
    return fail(MOE4_EINVAL, "moe4_experts.lora_A and lora_B must be given together");
  if (ex->lora_A) {
    if (ex->lora_r < 1 || ex->lora_r > 64)
      return fail(MOE4_ESHAPE, "moe4_experts.lora_r = %d outside [1, 64]", ex->lora_r);
    REQUIRE_ALIGN(ex->lora_A, 16, "moe4_experts.lora_A");
    REQUIRE_ALIGN(ex->lora_B, 2, "moe4_experts.lora_B");
    if (ex->H % 8) return fail(MOE4_ESHAPE, "LoRA needs H %% 8 == 0 (H = %d)", ex->H);
  }
  return MOE4_OK;
}

// Device address of `scratch` on the current device, looked up on the first
// call per device (with that device current) and kept.
int scratch_of_current_device(void* stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(MOE4_EDEVICE, "moe4_expert_forward_noalloc: hipGetDevice failed: %s",
                hipGetErrorString(e));
  if (stream != nullptr) {
    int sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess)
      return fail(MOE4_EINVAL, "moe4_expert_forward_noalloc: stream: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(MOE4_EINVAL,
                  "moe4_expert_forward_noalloc: stream is on device %d, the current device is %d",
                  sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE4_EDEVICE, "moe4_expert_forward_noalloc: device %d beyond the %d supported",
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MOE4_EDEVICE, "moe4_expert_forward_noalloc: device %d: scratch address: %s",
                  dev, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE4_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need, const char* fn) {
  if (need == 0) return MOE4_OK;
  if (ws == nullptr || ws_bytes < need)
    return fail(MOE4_EWORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                ws ? ws_bytes : (size_t)0, need);
  if (!aligned(ws, 256)) return fail(MOE4_EALIGN, "%s: ws is not 256-byte aligned", fn);
  return MOE4_OK;
}

}  // namespace

extern "C" {

int moe4_quantize_nf4(const float* w, int64_t n, int32_t blocksize, uint8_t* packed,
                      float* absmax, void* stream) {
  if (blocksize != 64) return fail(MOE4_EUNSUPPORTED, "blocksize = %d; NF4 uses 64", blocksize);
  if (n < 0 || n % 64) return fail(MOE4_ESHAPE, "n = %lld is not a non-negative multiple of 64",
                                   (long long)n);
  if (n == 0) return ok();
  REQUIRE_PTR(w, "w");
  REQUIRE_PTR(packed, "packed");
  REQUIRE_PTR(absmax, "absmax");
  REQUIRE_ALIGN(w, 16, "w");
  REQUIRE_ALIGN(packed, 4, "packed");
  REQUIRE_ALIGN(absmax, 4, "absmax");
  return launched(moe4::launch_quantize_nf4(w, n, packed, absmax, (hipStream_t)stream),
                  "moe4_quantize_nf4");
}

int moe4_decode_mxfp4(const uint8_t* blocks, const uint8_t* scales, int64_t R, int64_t K,
                      uint16_t* out, void* stream) {
  if (R < 0 || K < 0 || K % 32)
    return fail(MOE4_ESHAPE, "R = %lld, K = %lld: need R >= 0 and K a non-negative multiple of 32",
                (long long)R, (long long)K);
  if (R == 0 || K == 0) return ok();
  REQUIRE_PTR(blocks, "blocks");
  REQUIRE_PTR(scales, "scales");
  REQUIRE_PTR(out, "out");
  REQUIRE_ALIGN(blocks, 16, "blocks");
  REQUIRE_ALIGN(out, 16, "out");
  return launched(moe4::launch_decode_mxfp4(blocks, scales, R, K, out, (hipStream_t)stream),
                  "moe4_decode_mxfp4");
}

int moe4_compress_absmax(const float* absmax, int64_t n, const float* book, uint8_t* code,
                         float* absmax2, float* offset, void* ws, size_t ws_bytes,
                         void* stream) {
  if (n < 0) return fail(MOE4_ESHAPE, "n = %lld is negative", (long long)n);
  if (n == 0) return ok();
  REQUIRE_PTR(absmax, "absmax");
  REQUIRE_PTR(book, "book");
  REQUIRE_PTR(code, "code");
  REQUIRE_PTR(absmax2, "absmax2");
  REQUIRE_PTR(offset, "offset");
  REQUIRE_ALIGN(absmax, 4, "absmax");
  REQUIRE_ALIGN(book, 4, "book");
  REQUIRE_ALIGN(code, 4, "code");
  REQUIRE_ALIGN(absmax2, 4, "absmax2");
  REQUIRE_ALIGN(offset, 4, "offset");
  if (ws == nullptr || ws_bytes < (size_t)MOE4_DQ_WS_BYTES)
    return fail(MOE4_EWORKSPACE, "moe4_compress_absmax: workspace of %zu bytes given, %d needed",
                ws ? ws_bytes : (size_t)0, (int)MOE4_DQ_WS_BYTES);
  if (!aligned(ws, 8)) return fail(MOE4_EALIGN, "moe4_compress_absmax: ws is not 8-byte aligned");
  return launched(moe4::launch_dq_compress(absmax, n, book, code, absmax2, offset, ws,
                                           (hipStream_t)stream),
                  "moe4_compress_absmax");
}

int moe4_expand_absmax(const uint8_t* code, const float* absmax2, const float* offset,
                       const float* book, int64_t n, float* out, void* stream) {
  if (n < 0) return fail(MOE4_ESHAPE, "n = %lld is negative", (long long)n);
  if (n == 0) return ok();
  REQUIRE_PTR(code, "code");
  REQUIRE_PTR(absmax2, "absmax2");
  REQUIRE_PTR(offset, "offset");
  REQUIRE_PTR(book, "book");
  REQUIRE_PTR(out, "out");
  REQUIRE_ALIGN(absmax2, 4, "absmax2");
  REQUIRE_ALIGN(offset, 4, "offset");
  REQUIRE_ALIGN(book, 4, "book");
  REQUIRE_ALIGN(out, 4, "out");
  return launched(moe4::launch_dq_expand(code, absmax2, offset, book, n, out,
                                         (hipStream_t)stream),
                  "moe4_expand_absmax");
}

int moe4_convert_mxfp4_nf4(const uint8_t* blocks, const uint8_t* scales, int64_t R, int64_t K,
                           uint8_t* packed, float* absmax, void* stream) {
  if (R < 0 || K < 0 || K % 64)
    return fail(MOE4_ESHAPE, "R = %lld, K = %lld: need R >= 0 and K a non-negative multiple of 64",
                (long long)R, (long long)K);
  if (R == 0 || K == 0) return ok();
  REQUIRE_PTR(blocks, "blocks");
  REQUIRE_PTR(scales, "scales");
  REQUIRE_PTR(packed, "packed");
  REQUIRE_PTR(absmax, "absmax");
  REQUIRE_ALIGN(blocks, 16, "blocks");
  REQUIRE_ALIGN(packed, 16, "packed");
  REQUIRE_ALIGN(absmax, 4, "absmax");
  return launched(
      moe4::launch_convert_mxfp4_nf4(blocks, scales, R, K, packed, absmax, (hipStream_t)stream),
      "moe4_convert_mxfp4_nf4");
}

int moe4_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renormalize,
               int32_t* topk_idx, float* topk_w, void* stream) {
  if (E < 1 || E > 1024) return fail(MOE4_ESHAPE, "E = %d outside [1, 1024]", E);
  if (k < 1 || k > E) return fail(MOE4_ESHAPE, "k = %d outside [1, E = %d]", k, E);
  if (T < 0 || (int64_t)T * k >= ((int64_t)1 << 31))
    return fail(MOE4_ESHAPE, "T = %d: need T >= 0 and T*k < 2^31", T);
  if (T == 0) return ok();
  REQUIRE_PTR(logits, "logits");
  REQUIRE_PTR(topk_idx, "topk_idx");
  REQUIRE_PTR(topk_w, "topk_w");
  REQUIRE_ALIGN(logits, 4, "logits");
  REQUIRE_ALIGN(topk_idx, 4, "topk_idx");
  REQUIRE_ALIGN(topk_w, 4, "topk_w");
  return launched(moe4::launch_route(logits, T, E, k, renormalize != 0, topk_idx, topk_w,
                                     (hipStream_t)stream),
                  "moe4_route");
}

int moe4_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int32_t T,
                       int32_t H, int32_t E, float* logits, void* stream) {
  if (E < 1 || E > 1024) return fail(MOE4_ESHAPE, "E = %d outside [1, 1024]", E);
  if (H <= 0 || H % 8 || H >= (1 << 25))
    return fail(MOE4_ESHAPE, "H = %d must be a positive multiple of 8 below 2^25", H);
  if (T < 0) return fail(MOE4_ESHAPE, "T = %d is negative", T);
  if (T == 0) return ok();
  REQUIRE_PTR(x, "x");
  REQUIRE_PTR(wr, "wr");
  REQUIRE_PTR(logits, "logits");
  REQUIRE_ALIGN(x, 16, "x");
  REQUIRE_ALIGN(wr, 16, "wr");
  REQUIRE_ALIGN(bias, 4, "bias");
  REQUIRE_ALIGN(logits, 4, "logits");
  return launched(moe4::launch_router_logits(x, wr, bias, T, H, E, logits, (hipStream_t)stream),
                  "moe4_router_logits");
}

int moe4_route_backward(const int32_t* topk_idx, const float* topk_w, const float* logits,
                        int32_t renormalize, const uint16_t* dout, const float* y_perm,
                        const int32_t* row_of_slot, int32_t T, int32_t k, int32_t E, int32_t H,
                        float* dw, float* dlogits, void* stream) {
  if (E < 1 || E > 1024) return fail(MOE4_ESHAPE, "E = %d outside [1, 1024]", E);
  if (k < 1 || k > E) return fail(MOE4_ESHAPE, "k = %d outside [1, E = %d]", k, E);
  if (T < 0 || (int64_t)T * k >= ((int64_t)1 << 31))
    return fail(MOE4_ESHAPE, "T = %d: need T >= 0 and T*k < 2^31", T);
  if (H <= 0 || H % 8) return fail(MOE4_ESHAPE, "H = %d must be a positive multiple of 8", H);
  if (!renormalize && T > 0) REQUIRE_PTR(logits, "logits (needed without renormalisation)");
  if (T == 0) return ok();
  REQUIRE_PTR(topk_idx, "topk_idx");
  REQUIRE_PTR(topk_w, "topk_w");
  REQUIRE_PTR(dout, "dout");
  REQUIRE_PTR(y_perm, "y_perm");
  REQUIRE_PTR(row_of_slot, "row_of_slot");
  REQUIRE_PTR(dw, "dw");
  REQUIRE_PTR(dlogits, "dlogits");
  REQUIRE_ALIGN(dout, 16, "dout");
  REQUIRE_ALIGN(y_perm, 16, "y_perm");
  REQUIRE_ALIGN(topk_idx, 4, "topk_idx");
  REQUIRE_ALIGN(topk_w, 4, "topk_w");
  REQUIRE_ALIGN(logits, 4, "logits");
  REQUIRE_ALIGN(row_of_slot, 4, "row_of_slot");
  REQUIRE_ALIGN(dw, 4, "dw");
  REQUIRE_ALIGN(dlogits, 4, "dlogits");
  return launched(moe4::launch_route_backward(topk_idx, topk_w, logits, renormalize != 0, dout,
                                              y_perm, row_of_slot, T, k, E, H, dw, dlogits,
                                              (hipStream_t)stream),
                  "moe4_route_backward");
}

int moe4_permute(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, int32_t* offsets,
                 int32_t* slot_of_row, int32_t* row_of_slot, const uint16_t* x,
                 const float* row_scale, int32_t H, uint16_t* x_perm, void* ws, size_t ws_bytes,
                 void* stream) {
  if (E < 1 || E > 1024) return fail(MOE4_ESHAPE, "E = %d outside [1, 1024]", E);
  if (k < 1 || k > E) return fail(MOE4_ESHAPE, "k = %d outside [1, E = %d]", k, E);
  if (T < 0 || (int64_t)T * k >= ((int64_t)1 << 31))
    return fail(MOE4_ESHAPE, "T = %d: need T >= 0 and T*k < 2^31", T);
  REQUIRE_PTR(offsets, "offsets");
  if (T > 0) {
    REQUIRE_PTR(topk_idx, "topk_idx");
    REQUIRE_PTR(slot_of_row, "slot_of_row");
    REQUIRE_PTR(row_of_slot, "row_of_slot");
  }
  if (x != nullptr) {
    if (H <= 0 || H % 8) return fail(MOE4_ESHAPE, "H = %d must be a positive multiple of 8", H);
    if (T > 0) REQUIRE_PTR(x_perm, "x_perm");
    REQUIRE_ALIGN(x, 16, "x");
    REQUIRE_ALIGN(x_perm, 16, "x_perm");
  } else if (row_scale != nullptr) {
    return fail(MOE4_EINVAL, "row_scale given without x");
  }
  const size_t need = moe4::permute_ws_bytes(T, k, E);
  int rc = check_ws(ws, ws_bytes, need, "moe4_permute");
  if (rc) return rc;
  if (T == 0) {
    // every expert is empty: offsets = 0 (a fill kernel, so the call can be
    // captured into a HIP graph)
    return launched(moe4::launch_zero_i32(offsets, E + 1, (hipStream_t)stream), "moe4_permute");
  }
  return launched(moe4::launch_permute(topk_idx, T, k, E, offsets, slot_of_row, row_of_slot, x,
                                       row_scale, H, x_perm, ws, (hipStream_t)stream),
                  "moe4_permute");
}

int moe4_gather_rows(const uint16_t* x, int32_t T, int32_t k, int32_t H,
                     const int32_t* slot_of_row, const float* row_scale, uint16_t* x_perm,
                     void* stream) {
  if (k < 1 || k > 1024) return fail(MOE4_ESHAPE, "k = %d outside [1, 1024]", k);
  if (T < 0 || (int64_t)T * k >= ((int64_t)1 << 31))
    return fail(MOE4_ESHAPE, "T = %d: need T >= 0 and T*k < 2^31", T);
  if (H <= 0 || H % 8) return fail(MOE4_ESHAPE, "H = %d must be a positive multiple of 8", H);
  if (T > 0) {
    REQUIRE_PTR(x, "x");
    REQUIRE_PTR(slot_of_row, "slot_of_row");
    REQUIRE_PTR(x_perm, "x_perm");
  }
  REQUIRE_ALIGN(x, 16, "x");
  REQUIRE_ALIGN(x_perm, 16, "x_perm");
  REQUIRE_ALIGN(row_scale, 4, "row_scale");
  return launched(moe4::launch_gather(x, T, k, H, slot_of_row, row_scale, x_perm,
                                      (hipStream_t)stream),
                  "moe4_gather_rows");
}

int moe4_route_permute(const float* logits, int32_t T, int32_t E, int32_t k,
                       int32_t renormalize, int32_t* topk_idx, float* topk_w, int32_t* offsets,
                       int32_t* slot_of_row, int32_t* row_of_slot, const uint16_t* x, int32_t H,
                       uint16_t* x_perm, void* ws, size_t ws_bytes, void* stream) {
  if (E < 1 || E > 1024) return fail(MOE4_ESHAPE, "E = %d outside [1, 1024]", E);
  if (k < 1 || k > E) return fail(MOE4_ESHAPE, "k = %d outside [1, E = %d]", k, E);
  if (T < 0 || (int64_t)T * k >= ((int64_t)1 << 31))
    return fail(MOE4_ESHAPE, "T = %d: need T >= 0 and T*k < 2^31", T);
  REQUIRE_PTR(offsets, "offsets");
  if (T > 0) {
    REQUIRE_PTR(logits, "logits");
    REQUIRE_PTR(topk_idx, "topk_idx");
    REQUIRE_PTR(topk_w, "topk_w");
    REQUIRE_PTR(slot_of_row, "slot_of_row");
    REQUIRE_PTR(row_of_slot, "row_of_slot");
    REQUIRE_ALIGN(logits, 4, "logits");
    REQUIRE_ALIGN(topk_idx, 4, "topk_idx");
    REQUIRE_ALIGN(topk_w, 4, "topk_w");
  }
  if (x != nullptr) {
    if (H <= 0 || H % 8) return fail(MOE4_ESHAPE, "H = %d must be a positive multiple of 8", H);
    if (T > 0) REQUIRE_PTR(x_perm, "x_perm");
    REQUIRE_ALIGN(x, 16, "x");
    REQUIRE_ALIGN(x_perm, 16, "x_perm");
  }
  const size_t need = moe4::permute_ws_bytes(T, k, E);
  int rc = check_ws(ws, ws_bytes, need, "moe4_route_permute");
  if (rc) return rc;
  if (T == 0)
    return launched(moe4::launch_zero_i32(offsets, E + 1, (hipStream_t)stream),
                    "moe4_route_permute");
  return launched(moe4::launch_route_permute(logits, T, E, k, renormalize != 0, topk_idx, topk_w,
                                             offsets, slot_of_row, row_of_slot, x, H, x_perm, ws,
                                             (hipStream_t)stream),
                  "moe4_route_permute");
}

}  // extern "C"

namespace {

// Argument checks of the expert forward (both entry points).
int check_forward(const moe4_experts* ex, const uint16_t* x_perm, const int32_t* offsets,
                  int32_t rows, float* y_perm, float* save_gu, float* save_xa) {
  int rc = check_experts(ex);
  if (rc) return rc;
  if (rows < 0) return fail(MOE4_ESHAPE, "rows = %d is negative", rows);
  if (save_xa && !ex->lora_A) return fail(MOE4_EINVAL, "save_xa given without LoRA adapters");
  if (ex->H % 8) return fail(MOE4_ESHAPE, "H = %d must be a multiple of 8", ex->H);
  REQUIRE_PTR(offsets, "offsets");
  if (rows > 0) {
    REQUIRE_PTR(x_perm, "x_perm");
    REQUIRE_PTR(y_perm, "y_perm");
  }
  REQUIRE_ALIGN(x_perm, 16, "x_perm");
  REQUIRE_ALIGN(y_perm, 16, "y_perm");
  REQUIRE_ALIGN(save_gu, 4, "save_gu");
  REQUIRE_ALIGN(save_xa, 4, "save_xa");
  return MOE4_OK;
}

}  // namespace

extern "C" {

int moe4_expert_forward_noalloc(const moe4_experts* ex, const uint16_t* x_perm,
                                const int32_t* offsets, int32_t rows, float* y_perm,
                                float* save_gu, float* save_xa, void* stream) {
  g_variant = 0;
  int rc = check_forward(ex, x_perm, offsets, rows, y_perm, save_gu, save_xa);
  if (rc) return rc;
  const size_t need = moe4::forward_ws_bytes(*ex, rows);
  if (need > kNoAllocScratchBytes)
    return fail(MOE4_EWORKSPACE,
                "moe4_expert_forward_noalloc: this call needs %zu bytes of scratch, beyond the "
                "%zu the library holds per device (moe4_expert_forward takes a workspace)",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  rc = scratch_of_current_device(stream, &ws);
  if (rc) return rc;
  int variant = 0;
  hipError_t e = moe4::launch_expert_forward(*ex, x_perm, offsets, rows, y_perm, save_gu,
                                             save_xa, ws, &variant, moe4::LaunchEvents{g_events},
                                             (hipStream_t)stream);
  rc = launched(e, "moe4_expert_forward_noalloc");
  if (rc == MOE4_OK) g_variant = variant;
  return rc;
}

int moe4_expert_forward(const moe4_experts* ex, const uint16_t* x_perm, const int32_t* offsets,
                        int32_t rows, float* y_perm, float* save_gu, float* save_xa,
                        void* ws, size_t ws_bytes, void* stream) {
  g_variant = 0;
  int rc = check_forward(ex, x_perm, offsets, rows, y_perm, save_gu, save_xa);
  if (rc) return rc;
  rc = check_ws(ws, ws_bytes, moe4::forward_ws_bytes(*ex, rows), "moe4_expert_forward");
  if (rc) return rc;
  int variant = 0;
  hipError_t e = moe4::launch_expert_forward(*ex, x_perm, offsets, rows, y_perm, save_gu,
                                             save_xa, ws, &variant, moe4::LaunchEvents{g_events},
                                             (hipStream_t)stream);
  rc = launched(e, "moe4_expert_forward");
  if (rc == MOE4_OK) g_variant = variant;
  return rc;
}

int moe4_expert_forward_gather(const moe4_experts* ex, const uint16_t* x, int32_t T, int32_t k,
                               const int32_t* slot_of_row, const int32_t* offsets, int32_t rows,
                               float* y_perm, float* save_gu, void* ws, size_t ws_bytes,
                               void* stream) {
  g_variant = 0;
  int rc = check_experts(ex);
  if (rc) return rc;
  if (ex->lora_A)
    return fail(MOE4_EUNSUPPORTED,
                "moe4_expert_forward_gather: the adapter path takes x_perm (moe4_expert_forward)");
  if (k < 1) return fail(MOE4_ESHAPE, "k = %d must be >= 1", k);
  if (T < 0 || (int64_t)T * k >= ((int64_t)1 << 31))
    return fail(MOE4_ESHAPE, "T = %d: need T >= 0 and T*k < 2^31", T);
  if (rows != T * k) return fail(MOE4_ESHAPE, "rows = %d must be T*k = %d", rows, T * k);
  if (ex->H % 8) return fail(MOE4_ESHAPE, "H = %d must be a multiple of 8", ex->H);
  if ((int64_t)T * ex->H * 2 >= ((int64_t)1 << 29))
    return fail(MOE4_ESHAPE, "x of T = %d rows of H = %d exceeds 2^29 bytes (gathered rows are "
                "addressed with 32-bit offsets); use moe4_permute + moe4_expert_forward", T, ex->H);
  REQUIRE_PTR(offsets, "offsets");
  if (rows > 0) {
    REQUIRE_PTR(x, "x");
    REQUIRE_PTR(slot_of_row, "slot_of_row");
    REQUIRE_PTR(y_perm, "y_perm");
  }
  REQUIRE_ALIGN(x, 16, "x");
  REQUIRE_ALIGN(y_perm, 16, "y_perm");
  REQUIRE_ALIGN(save_gu, 4, "save_gu");
  rc = check_ws(ws, ws_bytes, moe4::forward_ws_bytes(*ex, rows), "moe4_expert_forward_gather");
  if (rc) return rc;
  int variant = 0;
  const moe4::GatherRows ga{x, slot_of_row, k, T};
  hipError_t e = moe4::launch_expert_forward(*ex, nullptr, offsets, rows, y_perm, save_gu,
                                             nullptr, ws, &variant, moe4::LaunchEvents{g_events},
                                             (hipStream_t)stream, &ga);
  rc = launched(e, "moe4_expert_forward_gather");
  if (rc == MOE4_OK) g_variant = variant;
  return rc;
}

int moe4_combine(const float* y_perm, const int32_t* row_of_slot, const float* topk_w,
                 int32_t T, int32_t k, int32_t H, void* out, int32_t out_dtype, void* stream) {
  if (out_dtype != MOE4_DTYPE_BF16 && out_dtype != MOE4_DTYPE_F32)
    return fail(MOE4_EINVAL, "out_dtype %s (%d)", out_dtype ? "unknown" : "unset", out_dtype);
  if (k < 1) return fail(MOE4_ESHAPE, "k = %d must be >= 1", k);
  if (T < 0 || (int64_t)T * k >= ((int64_t)1 << 31))
    return fail(MOE4_ESHAPE, "T = %d: need T >= 0 and T*k < 2^31", T);
  if (H <= 0 || H % 8) return fail(MOE4_ESHAPE, "H = %d must be a positive multiple of 8", H);
  if (T == 0) return ok();
  REQUIRE_PTR(y_perm, "y_perm");
  REQUIRE_PTR(row_of_slot, "row_of_slot");
  REQUIRE_PTR(out, "out");
  REQUIRE_ALIGN(y_perm, 16, "y_perm");
  REQUIRE_ALIGN(out, 16, "out");
  REQUIRE_ALIGN(topk_w, 4, "topk_w");
  return launched(moe4::launch_combine(y_perm, row_of_slot, topk_w, T, k, H, out,
                                       out_dtype == MOE4_DTYPE_F32, (hipStream_t)stream),
                  "moe4_combine");
}

int moe4_expert_backward(const moe4_experts* ex, const uint16_t* x_perm, const int32_t* offsets,
                         int32_t rows, const float* save_gu, const float* save_xa,
                         const uint16_t* dy_perm, float* dx_perm, float* dA, float* dB,
                         void* ws, size_t ws_bytes, void* stream) {
  g_variant = 0;
  int rc = check_experts(ex);
  if (rc) return rc;
  if (rows < 0) return fail(MOE4_ESHAPE, "rows = %d is negative", rows);
  REQUIRE_PTR(offsets, "offsets");
  if (rows > 0) {
    REQUIRE_PTR(save_gu, "save_gu");
    REQUIRE_PTR(dy_perm, "dy_perm");
    REQUIRE_PTR(dx_perm, "dx_perm");
  }
  if (ex->lora_A) {
    REQUIRE_PTR(dA, "dA");
    REQUIRE_PTR(dB, "dB");
    if (rows > 0) {
      REQUIRE_PTR(x_perm, "x_perm");
      REQUIRE_PTR(save_xa, "save_xa");
    }
  } else if (dA || dB) {
    return fail(MOE4_EINVAL, "dA/dB given without LoRA adapters");
  }
  REQUIRE_ALIGN(x_perm, 16, "x_perm");
  REQUIRE_ALIGN(dy_perm, 16, "dy_perm");
  REQUIRE_ALIGN(dx_perm, 16, "dx_perm");
  REQUIRE_ALIGN(save_gu, 4, "save_gu");
  REQUIRE_ALIGN(save_xa, 4, "save_xa");
  REQUIRE_ALIGN(dA, 4, "dA");
  REQUIRE_ALIGN(dB, 4, "dB");
  rc = check_ws(ws, ws_bytes, moe4::backward_ws_bytes(*ex, rows), "moe4_expert_backward");
  if (rc) return rc;
  int variant = 0;
  hipError_t e = moe4::launch_expert_backward(*ex, x_perm, offsets, rows, save_gu, save_xa,
                                              dy_perm, dx_perm, dA, dB, ws, &variant,
                                              moe4::LaunchEvents{g_events}, (hipStream_t)stream);
  rc = launched(e, "moe4_expert_backward");
  if (rc == MOE4_OK) g_variant = variant;
  return rc;
}

size_t moe4_workspace_size(const moe4_experts* ex, int32_t T, int32_t k) {
  if (check_experts(ex) != MOE4_OK) return 0;
  if (T < 0 || k < 1 || k > ex->E || (int64_t)T * k >= ((int64_t)1 << 31)) {
    fail(MOE4_ESHAPE, "moe4_workspace_size: T = %d, k = %d invalid", T, k);
    return 0;
  }
  const int rows = T * k;
  size_t need = moe4::permute_ws_bytes(T, k, ex->E);
  const size_t f = moe4::forward_ws_bytes(*ex, rows);
  const size_t b = moe4::backward_ws_bytes(*ex, rows);
  if (f > need) need = f;
  if (b > need) need = b;
  ok();
  return need < 256 ? 256 : need;
}

int moe4_set_timing_events(void* const* events, int32_t n_events) {
  if (events == nullptr || n_events == 0) {
    g_events = nullptr;
    return ok();
  }
  if (n_events < 4) return fail(MOE4_EINVAL, "n_events = %d: need 0 or at least 4", n_events);
  g_events = reinterpret_cast<hipEvent_t const*>(events);
  return ok();
}

const char* moe4_last_error(void) { return g_err; }

int moe4_last_variant(void) { return g_variant; }

}  // extern "C"
