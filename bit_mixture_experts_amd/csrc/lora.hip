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
// [E, r, K]. One workgroup per 32-row tile of one expert; its four waves split
// K into four ranges of 16-k MFMA steps and their 32x32 partial products meet
// in LDS. MFMA operand A = 32 rows of M, operand B = 32 rank rows of P (zero
// past r), both read straight from memory as 16-byte pieces (rows past the
// tile, ranks past r and steps past the wave's range read zeros), eight steps
// per batch with the next batch in flight.
__global__ __launch_bounds__(256) void k_rank_proj(const uint16_t* __restrict__ M,
                                                   const int32_t* __restrict__ offsets, int E,
                                                   int rows, int K, const uint16_t* __restrict__ P,
                                                   int r, float* __restrict__ out) {
  __shared__ float red[4][16][kWave];
  const int w = wave_id(), l = lane_id(), n32 = l & 31, h = l >> 5;
  int e, u, unused;
  locate_tile_eq<32>(offsets, E, 1, blockIdx.x, e, u, unused);
  e = __builtin_amdgcn_readfirstlane(e);
  u = __builtin_amdgcn_readfirstlane(u);
  if (e < 0) return;   // the whole workgroup: e is uniform
  const int ebeg = min(offsets[e], rows);
  const int row0 = ebeg + 32 * u;
  const int nrows = min(32, min(offsets[e + 1], rows) - row0);
  const rsrc_t rm = make_rsrc(M + (int64_t)row0 * K, (uint32_t)nrows * K * 2);
  const int moff = (n32 * K + 8 * h) * 2;
  const int nsteps = (K + 15) / 16;
  const int s0 = w * nsteps / 4, s1 = (w + 1) * nsteps / 4;
  for (int q0 = 0; q0 < r; q0 += 32) {
    const rsrc_t rp = make_rsrc(P + ((int64_t)e * r + q0) * K, (uint32_t)(r - q0) * K * 2);
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    u32x4 av[2][8], bv[2][8];
    // steps st .. st + 7 into batch slot b (never skipped: out-of-range steps
    // read zeros, so the count of loads in flight is the same on every path)
    auto load = [&](int b, int st) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int step = st + j;
        const int off = (step < s1 && 16 * step + 8 * h < K) ? moff + 32 * step : kOob;
        av[b][j] = buf_load_b128(rm, off);
        bv[b][j] = buf_load_b128(rp, off);
      }
    };
    auto mul = [&](int b) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[b][j]),
                                                      __builtin_bit_cast(bf16x8, bv[b][j]), acc,
                                                      0, 0, 0);
    };
    load(0, s0);
    for (int st = s0; st < s1; st += 16) {
      load(1, st + 8);
      __builtin_amdgcn_sched_barrier(0);
      mul(0);
      __builtin_amdgcn_sched_barrier(0);
      load(0, st + 16);
      __builtin_amdgcn_sched_barrier(0);
      mul(1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) red[w][i][l] = acc[i];
    __syncthreads();
    // lane holds rank column q0 + n32 of rows 8 (i / 4) + 4 h + i % 4; wave
    // w sums and stores entries i = 4 w .. 4 w + 3
    if (q0 + n32 < r) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 4 * w + ii;
        const int rr = 8 * (i >> 2) + 4 * h + (i & 3);
        if (rr < nrows)
          out[(int64_t)(row0 + rr) * r + q0 + n32] =
              red[0][i][l] + red[1][i][l] + red[2][i][l] + red[3][i][l];
      }
    }
    __syncthreads();   // red is reused by the next rank tile
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
// ranks per pass; the four waves' partial sums meet in LDS. A rank entry past
// r (read from the next row, or as zero past the last) is multiplied by zero:
// the mask makes it 0 before the product, so it never reaches a sum.
// R4: r % 4 == 0, so every 16-byte piece of a row's ranks lies wholly inside
// the window's resource or wholly past its end (then it reads zeros); other
// ranks are read one dword at a time, each checked against the resource on its
// own (a multi-dword load that straddles the end is not relied on).
constexpr int kQ = 8;
template <bool TRANSPOSED, bool R4>
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
    // 32-row windows of the expert through buffer resources: rows past r1
    // read zeros, so every load is issued (eight rows per wave and window,
    // the four waves interleaved by row)
    for (int rb = r0; rb < r1; rb += 32) {
      const int nw = min(32, r1 - rb);
      const rsrc_t rmat = make_rsrc(mat + (int64_t)rb * ncols, (uint32_t)nw * ncols * 2);
      const rsrc_t rvec = make_rsrc(vec + (int64_t)rb * r, (uint32_t)nw * r * 4);
      u32x2 mv[8];
      f32x4 vlo[8], vhi[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int rw = w + 4 * j;
        mv[j] = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(rmat, on ? (rw * ncols + col) * 2 : kOob,
                                                        0, 0));
        // ranks q0 .. q0 + 7 of the row (entries past r are masked below)
        if constexpr (R4) {
          vlo[j] = __builtin_bit_cast(f32x4, buf_load_b128(rvec, (rw * r + q0) * 4));
          vhi[j] = __builtin_bit_cast(f32x4, buf_load_b128(rvec, (rw * r + q0 + 4) * 4));
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            vlo[j][q] = __uint_as_float(buf_load_b32(rvec, (rw * r + q0 + q) * 4));
            vhi[j][q] = __uint_as_float(buf_load_b32(rvec, (rw * r + q0 + 4 + q) * 4));
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float m0 = bf16lo(mv[j][0]), m1 = bf16hi(mv[j][0]), m2 = bf16lo(mv[j][1]),
                    m3 = bf16hi(mv[j][1]);
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          const float raw = q < 4 ? vlo[j][q] : vhi[j][q - 4];
          const float v = q0 + q < r ? round_bf16(raw) : 0.0f;
          acc[q][0] += v * m0;
          acc[q][1] += v * m1;
          acc[q][2] += v * m2;
          acc[q][3] += v * m3;
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
  // tiles of 32 rows: at most rows / 32 + (one per expert), one workgroup
  // each; the XCD-contiguous deal of locate_tile_eq needs 8 ids beyond the
  // tile count (an XCD's share may start past the last id otherwise)
  const int ntiles = rows / 32 + min(E, rows);
  hipLaunchKernelGGL(k_rank_proj, dim3(ntiles + 8), dim3(256), 0, s, M, offsets, E, rows, K, P,
                     r, out);
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
  const bool r4 = r % 4 == 0;
  if (transposed && r4)
    hipLaunchKernelGGL((k_rank_reduce<true, true>), grid, dim3(256), 0, s, mat, ncols, vec, r,
                       offsets, rows, lscale, out);
  else if (transposed)
    hipLaunchKernelGGL((k_rank_reduce<true, false>), grid, dim3(256), 0, s, mat, ncols, vec, r,
                       offsets, rows, lscale, out);
  else if (r4)
    hipLaunchKernelGGL((k_rank_reduce<false, true>), grid, dim3(256), 0, s, mat, ncols, vec, r,
                       offsets, rows, lscale, out);
  else
    hipLaunchKernelGGL((k_rank_reduce<false, false>), grid, dim3(256), 0, s, mat, ncols, vec, r,
                       offsets, rows, lscale, out);
  return hipGetLastError();
}

}  // namespace moe4
