// Backward of the grouped expert path with respect to its input and the
// per-expert LoRA adapters: the input gradient goes through the frozen 4-bit
// weights ("dgrad"; project page "experts4bit-qlora", "Use this when"), the
// adapter gradients are grouped reductions over each expert's rows. The 4-bit
// base and the biases are frozen (the QLoRA setting of the solutions index's
// fused-experts entry) and get no gradient.
//
// The dgrad GEMMs contract over the weight rows, the opposite orientation of
// the forward: a [32 x 128] tile of packed weights (rows along the reduction)
// is dequantised by the whole workgroup into LDS, transposed so that each
// MFMA lane reads 8 consecutive reduction values with one 128-bit LDS load.
#include "common.hpp"
#include "formats.hpp"
#include "gemm_common.hpp"
#include "internal.hpp"

namespace moe4 {
namespace {

constexpr int kDM = 128, kDN = 128, kDK = 32, kDL = kDK + 8;

enum { DGRAD_DOWN = 0, DGRAD_GATEUP = 1 };

struct DgradArgs {
  const uint8_t* wq;   // stack [E, Kw, Nw] (rows = reduction dim), Nw/2 bytes per row
  const void* ws;      // scales per row: Nw/64 f32 (NF4) or Nw/32 u8 (MXFP4)
  int Kw, Nw;
  const uint16_t* A;   // [rows, Kw] bf16
  const int32_t* offsets;
  int E, rows, I, layout, act;
  float alpha, limit;
  const float* save_gu;     // DGRAD_DOWN: pre-activation gu fp32 [rows, 2I]
  uint16_t* dgu;            // DGRAD_DOWN out: [rows, 2I]
  const float* t;           // DGRAD_GATEUP LoRA: [rows, r] = dGU B_e
  const uint16_t* loraA;    // [E, r, H]
  int r;
  float lscale;
  float* dx;                // DGRAD_GATEUP out: fp32 [rows, H]
  int ncg;
};

// d(loss)/d(g), d(loss)/d(u) for h = act(g, u), given dh.
__device__ __forceinline__ void act_backward(int act, float g, float u, float dh, float alpha,
                                             float limit, float& dg, float& du) {
  if (act == MOE4_ACT_SWIGLU) {
    const float s = sigmoidf_(g);
    du = dh * g * s;
    dg = dh * u * s * (1.0f + g * (1.0f - s));
  } else {
    const float gc = fminf(g, limit);
    const float uc = fminf(fmaxf(u, -limit), limit);
    const float sa = sigmoidf_(alpha * gc);
    du = (u >= -limit && u <= limit) ? dh * gc * sa : 0.0f;
    dg = (g <= limit) ? dh * (uc + 1.0f) * (sa + alpha * gc * sa * (1.0f - sa)) : 0.0f;
  }
}

template <int FMT, int MODE>
__global__ __launch_bounds__(256) void k_dgrad(const DgradArgs a) {
  using F = Format<FMT>;
  constexpr int KB = F::kBlock;
  __shared__ float2 lutf[256];
  __shared__ __attribute__((aligned(16))) uint16_t As[kDM * kDL];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kDN * kDL];
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  lutf[tid] = make_float2(F::level(tid & 15), F::level(tid >> 4));
  int e, ut, cg;
  locate_tile_xcd<kDM>(a.offsets, a.E, a.ncg, blockIdx.x, e, ut, cg);
  e = __builtin_amdgcn_readfirstlane(e);
  ut = __builtin_amdgcn_readfirstlane(ut);
  cg = __builtin_amdgcn_readfirstlane(cg);
  __syncthreads();
  if (e < 0) return;
  const int row0 = min(a.offsets[e], a.rows) + ut * kDM;
  const int nrows = min(kDM, min(a.offsets[e + 1], a.rows) - row0);
  const int nb = cg * kDN;
  const int64_t wrow0 = (int64_t)e * a.Kw;
  const int bytes_per_row = a.Nw / 2;
  // B loader role: rows kb + 2*kp, +1; columns nb + 8*no .. +8
  const int kp = tid >> 4, no = tid & 15;
  const int ncol0 = nb + 8 * no;
  const bool bcol_ok = ncol0 < a.Nw;
  const int wm = w >> 1, wn = w & 1, n32 = l & 31, h = l >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int z = 0; z < 16; ++z) acc[i][j][z] = 0.0f;

  for (int kb = 0; kb < a.Kw; kb += kDK) {
    // global -> registers
    u32x4 areg[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + 256 * i, r = id >> 2, cidx = (id & 3) * 8;
      areg[i] = (r < nrows) ? *reinterpret_cast<const u32x4*>(a.A + (int64_t)(row0 + r) * a.Kw +
                                                              kb + cidx)
                            : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t braw[2] = {0u, 0u};
    float bsc[2] = {0.0f, 0.0f};
    if (bcol_ok) {
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int64_t wr = wrow0 + kb + 2 * kp + rr;
        braw[rr] = *reinterpret_cast<const uint32_t*>(a.wq + wr * bytes_per_row + ncol0 / 2);
        bsc[rr] = F::scale(a.ws, wr, a.Nw, ncol0 / KB);
      }
    }
    __syncthreads();   // previous iteration's LDS reads are done
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + 256 * i, r = id >> 2, cidx = (id & 3) * 8;
      *reinterpret_cast<u32x4*>(&As[r * kDL + cidx]) = areg[i];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float2 v0 = lutf[(braw[0] >> (8 * (c >> 1))) & 255u];
      const float2 v1 = lutf[(braw[1] >> (8 * (c >> 1))) & 255u];
      const float w0 = ((c & 1) ? v0.y : v0.x) * bsc[0];
      const float w1 = ((c & 1) ? v1.y : v1.x) * bsc[1];
      *reinterpret_cast<uint32_t*>(&Bs[(8 * no + c) * kDL + 2 * kp]) = pack_bf16x2(w0, w1);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kDK / 16; ++s) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        av[i] = *reinterpret_cast<const bf16x8*>(&As[(wm * 64 + i * 32 + n32) * kDL + 16 * s + 8 * h]);
        bv[i] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * 64 + i * 32 + n32) * kDL + 16 * s + 8 * h]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = nb + wn * 64 + j * 32 + n32;
      if (n >= a.Nw) continue;
#pragma unroll
      for (int z = 0; z < 16; ++z) {
        const int rr = wm * 64 + i * 32 + 8 * (z >> 2) + 4 * h + (z & 3);
        if (rr >= nrows) continue;
        const int row = row0 + rr;
        const float v = acc[i][j][z];
        if (MODE == DGRAD_DOWN) {
          // n indexes the intermediate dimension: dH[row][n]
          const int ng = gate_row(a.layout, a.I, n), nu = up_row(a.layout, a.I, n);
          const float* sg = a.save_gu + (int64_t)row * 2 * a.I;
          float dg, du;
          act_backward(a.act, sg[ng], sg[nu], v, a.alpha, a.limit, dg, du);
          uint16_t* d = a.dgu + (int64_t)row * 2 * a.I;
          d[ng] = f32_to_bf16(dg);
          d[nu] = f32_to_bf16(du);
        } else {
          float x = v;
          if (a.r) {
            const float* tr = a.t + (int64_t)row * a.r;
            const uint16_t* ar = a.loraA + (int64_t)e * a.r * a.Nw + n;
            float s = 0.0f;
            for (int qq = 0; qq < a.r; ++qq) s += round_bf16(tr[qq]) * bf16_to_f32(ar[(int64_t)qq * a.Nw]);
            x += a.lscale * s;
          }
          a.dx[(int64_t)row * a.Nw + n] = x;
        }
      }
    }
}

// t[row][q] = sum_n dGU[row][n] * B[e][n][q] (fp32); one wave per row.
__global__ __launch_bounds__(256) void k_lora_t(const uint16_t* __restrict__ dgu,
                                                const int32_t* __restrict__ offsets, int E,
                                                int rows, int N2, const uint16_t* __restrict__ B,
                                                int r, float* __restrict__ t) {
  const int row = (int)((blockIdx.x * (unsigned)blockDim.x + threadIdx.x) >> 6);
  if (row >= rows) return;
  const int e = expert_of_row(offsets, E, row);
  const int l = lane_id();
  const uint16_t* dr = dgu + (int64_t)row * N2;
  const uint16_t* be = B + (int64_t)e * N2 * r;
  for (int qq = 0; qq < r; ++qq) {
    float p = 0.0f;
    for (int n = l; n < N2; n += kWave) p += bf16_to_f32(dr[n]) * bf16_to_f32(be[(int64_t)n * r + qq]);
    p = wave_sum(p);
    if (l == 0) t[(int64_t)row * r + qq] = p;
  }
}

// out[e][col][q] (TRANSPOSED=false) or out[e][q][col] (true) =
//   lscale * sum_{rows of e} bf16(vec[row][q]) * mat[row][col]
// Thread per column; vec fp32 [rows, r] (rounded to bf16), mat bf16 [rows, ncols].
template <int RMAX, bool TRANSPOSED>
__global__ __launch_bounds__(256) void k_lora_reduce(const uint16_t* __restrict__ mat, int ncols,
                                                     const float* __restrict__ vec, int r,
                                                     const int32_t* __restrict__ offsets,
                                                     int rows, float lscale,
                                                     float* __restrict__ out) {
  const int e = blockIdx.y;
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= ncols) return;
  const int r0 = min(offsets[e], rows), r1 = min(offsets[e + 1], rows);
  float acc[RMAX];
#pragma unroll
  for (int qq = 0; qq < RMAX; ++qq) acc[qq] = 0.0f;
  for (int row = r0; row < r1; ++row) {
    const float m = bf16_to_f32(mat[(int64_t)row * ncols + col]);
    const float* vr = vec + (int64_t)row * r;
#pragma unroll
    for (int qq = 0; qq < RMAX; ++qq)
      if (qq < r) acc[qq] += round_bf16(vr[qq]) * m;
  }
#pragma unroll
  for (int qq = 0; qq < RMAX; ++qq)
    if (qq < r) {
      const int64_t o = TRANSPOSED ? ((int64_t)e * r + qq) * ncols + col
                                   : ((int64_t)e * ncols + col) * r + qq;
      out[o] = lscale * acc[qq];
    }
}

template <bool TRANSPOSED>
hipError_t run_lora_reduce(const uint16_t* mat, int ncols, const float* vec, int r,
                           const int32_t* offsets, int rows, int E, float lscale, float* out,
                           hipStream_t s) {
  const dim3 grid((unsigned)((ncols + 255) / 256), (unsigned)E);
  if (r <= 8)
    hipLaunchKernelGGL((k_lora_reduce<8, TRANSPOSED>), grid, dim3(256), 0, s, mat, ncols, vec, r,
                       offsets, rows, lscale, out);
  else if (r <= 16)
    hipLaunchKernelGGL((k_lora_reduce<16, TRANSPOSED>), grid, dim3(256), 0, s, mat, ncols, vec, r,
                       offsets, rows, lscale, out);
  else if (r <= 32)
    hipLaunchKernelGGL((k_lora_reduce<32, TRANSPOSED>), grid, dim3(256), 0, s, mat, ncols, vec, r,
                       offsets, rows, lscale, out);
  else
    hipLaunchKernelGGL((k_lora_reduce<64, TRANSPOSED>), grid, dim3(256), 0, s, mat, ncols, vec, r,
                       offsets, rows, lscale, out);
  return hipGetLastError();
}

template <int FMT>
hipError_t backward_fmt(const moe4_experts& ex, const uint16_t* x_perm, const int32_t* offsets,
                        int rows, const float* save_gu, const float* save_xa,
                        const uint16_t* dy_perm, float* dx_perm, float* dA, float* dB,
                        uint16_t* dgu, float* tbuf, const LaunchEvents& le, hipStream_t s) {
  const int E = ex.E, H = ex.H, I = ex.I;
  const bool lora = ex.lora_A != nullptr;
  const int touched = min(E, rows);
  const int ntiles = rows / kDM + touched;
  DgradArgs d{};
  d.offsets = offsets;
  d.E = E;
  d.rows = rows;
  d.I = I;
  d.layout = ex.gu_layout;
  d.act = ex.act;
  d.alpha = ex.act_alpha;
  d.limit = ex.act_limit;
  // dH = dy W_d[e]: W_d is [H (reduction), I]
  d.wq = static_cast<const uint8_t*>(ex.dn_q);
  d.ws = ex.dn_s;
  d.Kw = H;
  d.Nw = I;
  d.A = dy_perm;
  d.save_gu = save_gu;
  d.dgu = dgu;
  d.ncg = (I + kDN - 1) / kDN;
  le.before(0, s);
  if (ntiles * d.ncg > 0)
    // 16 spare ids keep every XCD's share of the items within the ids it is dealt
    hipLaunchKernelGGL((k_dgrad<FMT, DGRAD_DOWN>), dim3(ntiles * d.ncg + 16), dim3(256), 0, s, d);
  le.after(0, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (lora && rows > 0) {
    hipLaunchKernelGGL(k_lora_t, dim3((rows + 3) / 4), dim3(256), 0, s, dgu, offsets, E, rows,
                       2 * I, ex.lora_B, ex.lora_r, tbuf);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // dx = dGU W_gu[e] (+ LoRA): W_gu is [2I (reduction), H]
  DgradArgs g = d;
  g.wq = static_cast<const uint8_t*>(ex.gu_q);
  g.ws = ex.gu_s;
  g.Kw = 2 * I;
  g.Nw = H;
  g.A = dgu;
  g.t = tbuf;
  g.loraA = ex.lora_A;
  g.r = lora ? ex.lora_r : 0;
  g.lscale = ex.lora_scale;
  g.dx = dx_perm;
  g.ncg = (H + kDN - 1) / kDN;
  le.before(1, s);
  if (ntiles * g.ncg > 0)
    hipLaunchKernelGGL((k_dgrad<FMT, DGRAD_GATEUP>), dim3(ntiles * g.ncg + 16), dim3(256), 0, s,
                       g);
  le.after(1, s);
  err = hipGetLastError();
  if (err != hipSuccess || !lora) return err;
  // dB[e] = s * dGU^T bf16(xa)  -> [E, 2I, r];  dA[e] = s * bf16(t)^T x -> [E, r, H]
  err = run_lora_reduce<false>(dgu, 2 * I, save_xa, ex.lora_r, offsets, rows, E, ex.lora_scale,
                               dB, s);
  if (err != hipSuccess) return err;
  return run_lora_reduce<true>(x_perm, H, tbuf, ex.lora_r, offsets, rows, E, ex.lora_scale, dA,
                               s);
}

}  // namespace

size_t backward_ws_bytes(const moe4_experts& ex, int rows) {
  size_t b = align_up((size_t)rows * 2 * ex.I * sizeof(uint16_t), 256);
  if (ex.lora_A) b += align_up((size_t)rows * ex.lora_r * sizeof(float), 256);
  return b + dq_expand_bytes(ex);
}

hipError_t launch_expert_backward(const moe4_experts& ex, const uint16_t* x_perm,
                                  const int32_t* offsets, int rows, const float* save_gu,
                                  const float* save_xa, const uint16_t* dy_perm,
                                  float* dx_perm, float* dA, float* dB, void* ws,
                                  int* variant, const LaunchEvents& le, hipStream_t s) {
  *variant = MOE4_VARIANT_TILED;
  char* p = static_cast<char*>(ws);
  uint16_t* dgu = reinterpret_cast<uint16_t*>(p);
  p += align_up((size_t)rows * 2 * ex.I * sizeof(uint16_t), 256);
  float* tbuf = ex.lora_A ? reinterpret_cast<float*>(p) : nullptr;
  if (ex.lora_A) p += align_up((size_t)rows * ex.lora_r * sizeof(float), 256);
  if (rows == 0 && !ex.lora_A) return hipSuccess;
  if (ex.format == MOE4_FMT_NF4_DQ) {
    // expand the double-quantised absmax, then the plain NF4 dgrad
    moe4_experts plain;
    hipError_t err = dq_expand_experts(ex, p, &plain, s);
    if (err != hipSuccess) return err;
    return backward_fmt<MOE4_FMT_NF4>(plain, x_perm, offsets, rows, save_gu, save_xa, dy_perm,
                                      dx_perm, dA, dB, dgu, tbuf, le, s);
  }
  if (ex.format == MOE4_FMT_NF4)
    return backward_fmt<MOE4_FMT_NF4>(ex, x_perm, offsets, rows, save_gu, save_xa, dy_perm,
                                      dx_perm, dA, dB, dgu, tbuf, le, s);
  return backward_fmt<MOE4_FMT_MXFP4>(ex, x_perm, offsets, rows, save_gu, save_xa, dy_perm,
                                      dx_perm, dA, dB, dgu, tbuf, le, s);
}

}  // namespace moe4
