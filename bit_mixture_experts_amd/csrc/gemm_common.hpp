// Arguments and epilogues shared by the grouped expert GEMM kernels.
#pragma once

#include "common.hpp"
#include "../../include/moe4.h"

namespace moe4 {

// One grouped GEMM over a 4-bit stack [E, Nw, K] (Nw = 2I for gate_up, H for
// down) with activations A [rows, K] ordered by expert (offsets [E+1]).
struct GemmArgs {
  const uint8_t* wq;    // packed nibbles, K/2 bytes per weight row
  const void* ws;       // scales: f32 [E, Nw, K/64] (NF4), u8 [E, Nw, K/32] (MXFP4), or
                        // u8 absmax codes [E, Nw, K/64] (double-quantised NF4)
  const float* ws2;     // double-quantised NF4: absmax2, one per 256 absmax of the stack
  const float* dqoff;   // double-quantised NF4: the stack's absmax offset (one fp32)
  const float* dqbook;  // double-quantised NF4: the 256-entry absmax code book
  int K;
  int N_out;            // gate_up: I (gate/up pairs); down: H
  int I;
  int layout, act;
  float alpha, limit;
  const uint16_t* A;
  // gathered activations (gate_up of moe4_expert_forward_gather): row r of the
  // grouped GEMM is row arows[r] / gk of A, which has a_rows rows; null: row r
  const int32_t* arows;
  int gk, a_rows;
  const int32_t* offsets;
  int E, rows;
  const uint16_t* bias; // bf16 [E, Nw] or null
  const float* xa;      // LoRA: fp32 [rows, r] = x A_e^T (gate_up only)
  const uint16_t* loraB;// bf16 [E, 2I, r]
  int r;
  float lscale;
  uint16_t* hout;       // gate_up: h [rows, I] (bf16)
  float* yout;          // down: y [rows, H] (fp32)
  float* save_gu;       // fp32 [rows, 2I] or null
  int ncg;              // column groups per row tile
};

__device__ __forceinline__ int gate_row(int layout, int I, int j) {
  return layout == MOE4_GU_HALVES ? j : 2 * j;
}
__device__ __forceinline__ int up_row(int layout, int I, int j) {
  return layout == MOE4_GU_HALVES ? I + j : 2 * j + 1;
}

__device__ __forceinline__ float act_apply(int act, float g, float u, float alpha, float limit) {
  if (act == MOE4_ACT_SWIGLU) return g * sigmoidf_(g) * u;
  const float gc = fminf(g, limit);
  const float uc = fminf(fmaxf(u, -limit), limit);
  return (uc + 1.0f) * gc * sigmoidf_(alpha * gc);
}

__device__ __forceinline__ float round_bf16(float v) { return bf16_to_f32(f32_to_bf16(v)); }

// lscale * sum_q bf16(xa[row][q]) * B[e][n][q]
__device__ __forceinline__ float lora_term(const GemmArgs& a, int e, int row, int n) {
  const float* xr = a.xa + (int64_t)row * a.r;
  const uint16_t* br = a.loraB + ((int64_t)e * 2 * a.I + n) * a.r;
  float s = 0.0f;
  for (int q = 0; q < a.r; ++q) s += round_bf16(xr[q]) * bf16_to_f32(br[q]);
  return a.lscale * s;
}

__device__ __forceinline__ void gate_up_epilogue(const GemmArgs& a, int e, int row, int j,
                                                 float g, float u) {
  const int ng = gate_row(a.layout, a.I, j), nu = up_row(a.layout, a.I, j);
  const int64_t bb = (int64_t)e * 2 * a.I;
  if (a.bias) {
    g += bf16_to_f32(a.bias[bb + ng]);
    u += bf16_to_f32(a.bias[bb + nu]);
  }
  if (a.r) {
    g += lora_term(a, e, row, ng);
    u += lora_term(a, e, row, nu);
  }
  if (a.save_gu) {
    float* sg = a.save_gu + (int64_t)row * 2 * a.I;
    sg[ng] = g;
    sg[nu] = u;
  }
  a.hout[(int64_t)row * a.I + j] = f32_to_bf16(act_apply(a.act, g, u, a.alpha, a.limit));
}

__device__ __forceinline__ void down_epilogue(const GemmArgs& a, int e, int row, int col, float y) {
  if (a.bias) y += bf16_to_f32(a.bias[(int64_t)e * a.N_out + col]);
  // y rows are read once, by the combine, long after: stream them out
  __builtin_nontemporal_store(y, a.yout + (int64_t)row * a.N_out + col);
}

// expert owning permuted row `row` (largest e with offsets[e] <= row)
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int E, int row) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= row) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

}  // namespace moe4
