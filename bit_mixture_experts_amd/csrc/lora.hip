// Rank-r pieces of the per-expert LoRA adapters (project page
// "experts4bit-qlora", QLoRA entry: a low-rank delta per expert on top of the
// frozen 4-bit base): the projections onto the rank (forward x A_e^T, backward
// dGU B_e) and the adapter gradients (grouped reductions over each expert's
// rows). They move far fewer bytes than the expert GEMMs; the kernels are
// organised to stream their inputs once.
#include "common.hpp"
#include "gemm_common.hpp"
#include "internal.hpp"

namespace moe4 {
namespace {

// out[row][q] = sum_k M[row][k] P[e(row)][q][k] in fp32, M bf16 [rows, K], P bf16
// [E, r, K]. One wave per 32-row tile of one expert: MFMA operand A = 32 rows
// of M, operand B = 32 rank rows of P (zero past r), both read straight from
// memory as 16-byte pieces (rows past the tile and ranks past r read zeros).
__global__ __launch_bounds__(256) void k_rank_proj(const uint16_t* __restrict__ M,
                                                   const int32_t* __restrict__ offsets, int E,
                                                   int rows, int K, const uint16_t* __restrict__ P,
                                                   int r, float* __restrict__ out) {
  const int w = wave_id(), l = lane_id(), n32 = l & 31, h = l >> 5;
  int e, u, unused;
  locate_tile_eq<32>(offsets, E, 1, blockIdx.x * 4 + w, e, u, unused);
  e = __builtin_amdgcn_readfirstlane(e);
  u = __builtin_amdgcn_readfirstlane(u);
  if (e < 0) return;
  const int ebeg = min(offsets[e], rows);
  const int row0 = ebeg + 32 * u;
  const int nrows = min(32, min(offsets[e + 1], rows) - row0);
  const rsrc_t rm = make_rsrc(M + (int64_t)row0 * K, (uint32_t)nrows * K * 2);
  const int moff = (n32 * K + 8 * h) * 2;
  for (int q0 = 0; q0 < r; q0 += 32) {
    const rsrc_t rp = make_rsrc(P + ((int64_t)e * r + q0) * K, (uint32_t)(r - q0) * K * 2);
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    int k0 = 0;
    for (; k0 + 128 <= K; k0 += 128) {
      u32x4 av[8], bv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        av[j] = buf_load_b128(rm, moff + 2 * (k0 + 16 * j));
        bv[j] = buf_load_b128(rp, moff + 2 * (k0 + 16 * j));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[j]),
                                                      __builtin_bit_cast(bf16x8, bv[j]), acc, 0,
                                                      0, 0);
    }
    for (; k0 < K; k0 += 16) {
      const u32x4 av = buf_load_b128(rm, k0 + 8 * h < K ? moff + 2 * k0 : kOob);
      const u32x4 bv = buf_load_b128(rp, k0 + 8 * h < K ? moff + 2 * k0 : kOob);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                    __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    }
    // lane holds rank column q0 + n32 of rows 8 (i / 4) + 4 h + i % 4
    if (q0 + n32 < r) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = 8 * (i >> 2) + 4 * h + (i & 3);
        if (rr < nrows) out[(int64_t)(row0 + rr) * r + q0 + n32] = acc[i];
      }
    }
  }
}

// BT[e][q][n] = B[e][n][q] (bf16 [E, N, r] -> [E, r, N])
__global__ __launch_bounds__(256) void k_transpose_rank(const uint16_t* __restrict__ B, int E,
                                                        int N, int r, uint16_t* __restrict__ BT) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)E * N * r;
  if (i >= total) return;
  const int q = (int)(i % r);
  const int64_t en = i / r;
  const int n = (int)(en % N), e = (int)(en / N);
  BT[((int64_t)e * r + q) * N + n] = B[i];
}

// out[e][col][q] (TRANSPOSED = false) or out[e][q][col] (true) =
//   lscale * sum over the rows of e of bf16(vec[row][q]) * mat[row][col]
// vec fp32 [rows, r], mat bf16 [rows, ncols]. Block = (256 columns, expert);
// wave w takes rows w, w + 4, ..., lane l columns 4 l .. 4 l + 3, up to kQ
// ranks per pass; the four waves' partial sums meet in LDS.
constexpr int kQ = 8;
template <bool TRANSPOSED>
__global__ __launch_bounds__(256) void k_rank_reduce(const uint16_t* __restrict__ mat, int ncols,
                                                     const float* __restrict__ vec, int r,
                                                     const int32_t* __restrict__ offsets,
                                                     int rows, float lscale,
                                                     float* __restrict__ out) {
  __shared__ float red[4][kQ][256];
  const int e = blockIdx.y;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id();
  const int c0 = blockIdx.x * 256;
  const int r0 = min(offsets[e], rows), r1 = min(offsets[e + 1], rows);
  const int col = c0 + 4 * l;
  const bool on = col < ncols;   // ncols is a multiple of 4
  for (int q0 = 0; q0 < r; q0 += kQ) {
    float acc[kQ][4];
#pragma unroll
    for (int q = 0; q < kQ; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[q][c] = 0.0f;
    for (int row = r0 + w; row < r1; row += 16) {
      uint2 mv[4];
      float vv[4][kQ];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rw = row + 4 * j;
        const bool ok = on && rw < r1;
        mv[j] = ok ? *reinterpret_cast<const uint2*>(mat + (int64_t)rw * ncols + col) : make_uint2(0u, 0u);
#pragma unroll
        for (int q = 0; q < kQ; ++q)
          vv[j][q] = (rw < r1 && q0 + q < r) ? round_bf16(vec[(int64_t)rw * r + q0 + q]) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float m0 = bf16lo(mv[j].x), m1 = bf16hi(mv[j].x), m2 = bf16lo(mv[j].y), m3 = bf16hi(mv[j].y);
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          acc[q][0] += vv[j][q] * m0;
          acc[q][1] += vv[j][q] * m1;
          acc[q][2] += vv[j][q] * m2;
          acc[q][3] += vv[j][q] * m3;
        }
      }
    }
    __syncthreads();   // the previous pass's reads of red are done
#pragma unroll
    for (int q = 0; q < kQ; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) red[w][q][4 * l + c] = acc[q][c];
    __syncthreads();
    // thread t: column c0 + t, ranks q0 .. q0 + kQ - 1
    const int t = threadIdx.x, cc = c0 + t;
    if (cc < ncols) {
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (q0 + q < r) {
          const float v = red[0][q][t] + red[1][q][t] + red[2][q][t] + red[3][q][t];
          const int64_t o = TRANSPOSED ? ((int64_t)e * r + q0 + q) * ncols + cc
                                       : ((int64_t)e * ncols + cc) * r + q0 + q;
          out[o] = lscale * v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_rank_proj(const uint16_t* M, const int32_t* offsets, int E, int rows, int K,
                            const uint16_t* P, int r, float* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  // tiles of 32 rows: at most rows / 32 + (one per expert), plus 8 spare ids
  const int ntiles = rows / 32 + min(E, rows) + 8;
  hipLaunchKernelGGL(k_rank_proj, dim3((ntiles + 3) / 4), dim3(256), 0, s, M, offsets, E, rows,
                     K, P, r, out);
  return hipGetLastError();
}

hipError_t launch_transpose_rank(const uint16_t* B, int E, int N, int r, uint16_t* BT,
                                 hipStream_t s) {
  const int64_t total = (int64_t)E * N * r;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_transpose_rank, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, B,
                     E, N, r, BT);
  return hipGetLastError();
}

hipError_t launch_rank_reduce(const uint16_t* mat, int ncols, const float* vec, int r,
                              const int32_t* offsets, int rows, int E, float lscale, float* out,
                              bool transposed, hipStream_t s) {
  const dim3 grid((unsigned)((ncols + 255) / 256), (unsigned)E);
  if (transposed)
    hipLaunchKernelGGL(k_rank_reduce<true>, grid, dim3(256), 0, s, mat, ncols, vec, r, offsets,
                       rows, lscale, out);
  else
    hipLaunchKernelGGL(k_rank_reduce<false>, grid, dim3(256), 0, s, mat, ncols, vec, r, offsets,
                       rows, lscale, out);
  return hipGetLastError();
}

}  // namespace moe4
