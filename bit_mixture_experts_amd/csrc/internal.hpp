// Internal launcher interface between the C ABI (moe4_abi.hip) and the kernel
// files. Launchers assume validated arguments and return hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe4.h"

namespace moe4 {

// ---- codecs
hipError_t launch_quantize_nf4(const float* w, int64_t n, uint8_t* packed, float* absmax,
                               hipStream_t s);
hipError_t launch_decode_mxfp4(const uint8_t* blocks, const uint8_t* scales, int64_t R,
                               int64_t K, uint16_t* out, hipStream_t s);
hipError_t launch_convert_mxfp4_nf4(const uint8_t* blocks, const uint8_t* scales, int64_t R,
                                    int64_t K, uint8_t* packed, float* absmax, hipStream_t s);

// ---- double-quantised NF4 absmax
constexpr int kDqPartials = 1024;   // float64 partial sums in the workspace (8 KiB)
int dq_partials(int64_t n);
hipError_t launch_dq_compress(const float* absmax, int64_t n, const float* book, uint8_t* code,
                              float* absmax2, float* offset, void* ws, hipStream_t s);
hipError_t launch_dq_expand(const uint8_t* code, const float* absmax2, const float* offset,
                            const float* book, int64_t n, float* out, hipStream_t s);

// Plain-NF4 view of a double-quantised descriptor: both stacks' absmax
// expanded into abs_ws (dq_expand_bytes of it; 0 for other formats).
size_t dq_expand_bytes(const moe4_experts& ex);
hipError_t dq_expand_experts(const moe4_experts& ex, void* abs_ws, moe4_experts* out,
                             hipStream_t s);

// ---- LoRA rank pieces
// out[row][q] = sum_k M[row][k] P[e(row)][q][k] (fp32), M bf16 [rows, K], P bf16 [E, r, K]
hipError_t launch_rank_proj(const uint16_t* M, const int32_t* offsets, int E, int rows, int K,
                            const uint16_t* P, int r, float* out, hipStream_t s);
// BT[e][q][n] = B[e][n][q]
hipError_t launch_transpose_rank(const uint16_t* B, int E, int N, int r, uint16_t* BT,
                                 hipStream_t s);
// out[e][col][q] (or [e][q][col] when transposed) =
//   lscale * sum over e's rows of bf16(vec[row][q]) * mat[row][col]
hipError_t launch_rank_reduce(const uint16_t* mat, int ncols, const float* vec, int r,
                              const int32_t* offsets, int rows, int E, float lscale, float* out,
                              bool transposed, hipStream_t s);

// ---- router step
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int T,
                                int H, int E, float* logits, hipStream_t s);
hipError_t launch_route_backward(const int32_t* idx, const float* tw, const float* lg,
                                 int renorm, const uint16_t* dout, const float* y,
                                 const int32_t* row_of_slot, int T, int k, int E, int H,
                                 float* dw, float* dlog, hipStream_t s);

// ---- routing / permutation / combine
hipError_t launch_route(const float* logits, int T, int E, int k, int renorm, int32_t* idx,
                        float* w, hipStream_t s);
size_t permute_ws_bytes(int T, int k, int E);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* slot_of_row, int32_t* row_of_slot, const uint16_t* x,
                          const float* row_scale, int H, uint16_t* x_perm, void* ws,
                          hipStream_t s);
// route + permute (+ gather): one launch for small batches, else the two above
hipError_t launch_route_permute(const float* logits, int T, int E, int k, int renorm,
                                int32_t* idx, float* w, int32_t* offsets, int32_t* slot_of_row,
                                int32_t* row_of_slot, const uint16_t* x, int H,
                                uint16_t* x_perm, void* ws, hipStream_t s);
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);
hipError_t launch_gather(const uint16_t* x, int T, int k, int H, const int32_t* slot_of_row,
                         const float* row_scale, uint16_t* x_perm, hipStream_t s);
hipError_t launch_combine(const float* y, const int32_t* row_of_slot, const float* w, int T,
                          int k, int H, void* out, bool out_f32, hipStream_t s);

// ---- expert forward / backward
size_t forward_ws_bytes(const moe4_experts& ex, int rows);
size_t backward_ws_bytes(const moe4_experts& ex, int rows);
// Optional events recorded around the two GEMM launches (null = off):
// ev[0]/ev[1] around the first, ev[2]/ev[3] around the second.
struct LaunchEvents {
  hipEvent_t const* ev;
  void before(int i, hipStream_t s) const {
    if (ev) (void)hipEventRecord(ev[2 * i], s);   // timing only
  }
  void after(int i, hipStream_t s) const {
    if (ev) (void)hipEventRecord(ev[2 * i + 1], s);
  }
};

// Activation rows gathered by the gate_up GEMM itself: row r of the grouped
// GEMM is row slot_of_row[r] / k of x [T, H].
struct GatherRows {
  const uint16_t* x;
  const int32_t* slot_of_row;
  int k, T;
};

// returns the kernel family used through *variant; ga (or null) replaces x_perm
// by rows gathered from x (no adapter then)
hipError_t launch_expert_forward(const moe4_experts& ex, const uint16_t* x_perm,
                                 const int32_t* offsets, int rows, float* y_perm,
                                 float* save_gu, float* save_xa, void* ws, int* variant,
                                 const LaunchEvents& le, hipStream_t s,
                                 const GatherRows* ga = nullptr);
hipError_t launch_expert_backward(const moe4_experts& ex, const uint16_t* x_perm,
                                  const int32_t* offsets, int rows, const float* save_gu,
                                  const float* save_xa, const uint16_t* dy_perm,
                                  float* dx_perm, float* dA, float* dB, void* ws,
                                  int* variant, const LaunchEvents& le, hipStream_t s);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe4
