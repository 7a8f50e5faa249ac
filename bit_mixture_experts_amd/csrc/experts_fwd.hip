// Grouped expert forward on 4-bit stacks: gate_up GEMM (+ bias + LoRA delta)
// fused with SwiGLU / clamped GLU, then the down GEMM (+ bias).
//
// The routed expert GEMM runs on packed 4-bit weights with the nibbles decoded
// in registers and fp32 accumulation, never materialising a bf16 expert tensor
// ("MoE Training & Inference Guides", grouped-nf4-gemm entries for the NF4 and
// native MXFP4 grouped GEMMs). gpt-oss adds per-expert biases, interleaved
// gate/up rows and a clamped GLU ("How do I train and serve MoE models
// released in MXFP4", "Why it happens"); the stock epilogue is act(gate)*up
// (project page "experts4bit-qlora", "Limitations -- qlora-fused-moe-experts");
// the LoRA delta is added before the activation (QLoRA fused-experts entry of
// the solutions index).
//
// Two kernel families:
//  * skinny (decode-sized row counts): one workgroup streams 32 weight rows of
//    one expert over all of K, split across its waves; each wave dequantises
//    its nibbles through an LDS byte table and runs 16x16x32 bf16 MFMA, one
//    k-step per 32 weights; waves are reduced through LDS. NF4 weights get
//    their absmax before the MFMA; MXFP4 blocks get their power-of-two scale
//    on the fp32 partial product of the block (exact either way).
//  * tiled (prefill-sized row counts): a 128-row tile of one expert's permuted
//    activations is staged in LDS (double-buffered); each wave owns 64 weight
//    rows, loads their nibbles straight into registers with 128-bit loads,
//    dequantises with the scale folded in, and runs 32x32x16 bf16 MFMA.
#include "common.hpp"
#include "formats.hpp"
#include "internal.hpp"
#include "gemm_common.hpp"

namespace moe4 {
namespace {

// ------------------------------------------------------------ skinny kernel

template <int FMT, bool GATEUP, int MAXR, int U>
__global__ __launch_bounds__(1024) void k_skinny(const GemmArgs a) {
  using F = Format<FMT>;
  constexpr int KB = F::kBlock;
  constexpr int STEPS = KB / 32;
  // NF4: each weight is formed as bf16(level * absmax) before the MFMA (the
  // operand the method defines). MXFP4: e2m1 * 2^(s-127) is exact in bf16, so
  // the power-of-two scale is applied once to each block's fp32 partial sum.
  constexpr bool PRESCALE = FMT == MOE4_FMT_NF4;
  __shared__ uint32_t lut[256];
  __shared__ float2 lutf[256];
  extern __shared__ float red[];
  const int S = blockDim.x >> 6, w = wave_id(), l = lane_id();
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    if (PRESCALE) lutf[i] = make_float2(F::level(i & 15), F::level(i >> 4));
    else lut[i] = lut_bf16x2<FMT>(i);
  }
  const int item = blockIdx.x / a.ncg, cg = blockIdx.x - item * a.ncg;
  int e, unused;
  locate_item(a.offsets, a.E, item, [](int n) { return n > 0 ? 1 : 0; }, e, unused);
  __syncthreads();
  if (e < 0) return;
  const int rbeg = min(a.offsets[e], a.rows);
  const int n_e = min(a.offsets[e + 1], a.rows) - rbeg;
  const int nl = l & 15, g = l >> 4;
  const int Nw = GATEUP ? 2 * a.I : a.N_out;
  int wrow[2];
  if (GATEUP) {
    const int j = cg * 16 + nl;
    wrow[0] = gate_row(a.layout, a.I, j);
    wrow[1] = up_row(a.layout, a.I, j);
  } else {
    wrow[0] = cg * 32 + nl;
    wrow[1] = cg * 32 + 16 + nl;
  }
  const int64_t growbase = (int64_t)e * Nw;
  const uint8_t* qp0 = a.wq + (growbase + wrow[0]) * (int64_t)(a.K / 2) + 4 * g;
  const uint8_t* qp1 = a.wq + (growbase + wrow[1]) * (int64_t)(a.K / 2) + 4 * g;
  const int nblk = a.K / KB;
  const int b0 = (int)((int64_t)w * nblk / S), b1 = (int)((int64_t)(w + 1) * nblk / S);
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  bf16x8 zero8;
#pragma unroll
  for (int i = 0; i < 8; ++i) zero8[i] = (__bf16)0.0f;

  for (int rc = 0; rc < n_e; rc += 16 * MAXR) {
    const int nrows = min(16 * MAXR, n_e - rc);
    const int nrt = (nrows + 15) >> 4;
    f32x4 acc[MAXR][2];
#pragma unroll
    for (int rt = 0; rt < MAXR; ++rt) acc[rt][0] = acc[rt][1] = zero4;
    for (int bb = b0; bb < b1; bb += U) {
      uint32_t wv[U][2][STEPS];
      float sc[U][2];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int b = bb + u;
        if (b < b1) {
#pragma unroll
          for (int st = 0; st < STEPS; ++st) {
            wv[u][0][st] = *reinterpret_cast<const uint32_t*>(qp0 + (int64_t)b * (KB / 2) + st * 16);
            wv[u][1][st] = *reinterpret_cast<const uint32_t*>(qp1 + (int64_t)b * (KB / 2) + st * 16);
          }
          sc[u][0] = F::scale(a.ws, growbase + wrow[0], a.K, b);
          sc[u][1] = F::scale(a.ws, growbase + wrow[1], a.K, b);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int b = bb + u;
        if (b < b1) {
          bf16x8 bq[2][STEPS];
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
              const uint32_t v = wv[u][c][st];
              u32x4 t;
              if (PRESCALE) {
#pragma unroll
                for (int bi = 0; bi < 4; ++bi) {
                  const float2 f = lutf[(v >> (8 * bi)) & 255u];
                  t[bi] = pack_bf16x2(f.x * sc[u][c], f.y * sc[u][c]);
                }
              } else {
                t[0] = lut[v & 255u];
                t[1] = lut[(v >> 8) & 255u];
                t[2] = lut[(v >> 16) & 255u];
                t[3] = lut[v >> 24];
              }
              bq[c][st] = __builtin_bit_cast(bf16x8, t);
            }
#pragma unroll
          for (int rt = 0; rt < MAXR; ++rt) {
            if (rt < nrt) {
              const int m = rc + rt * 16 + nl;
              bf16x8 av[STEPS];
#pragma unroll
              for (int st = 0; st < STEPS; ++st)
                av[st] = (m < n_e)
                             ? *reinterpret_cast<const bf16x8*>(
                                   a.A + (int64_t)(rbeg + m) * a.K + b * KB + st * 32 + 8 * g)
                             : zero8;
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                if (PRESCALE) {
#pragma unroll
                  for (int st = 0; st < STEPS; ++st)
                    acc[rt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[st], bq[c][st],
                                                                         acc[rt][c], 0, 0, 0);
                } else {
                  const f32x4 t =
                      __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[0], bq[c][0], zero4, 0, 0, 0);
                  acc[rt][c] += sc[u][c] * t;
                }
              }
            }
          }
        }
      }
    }
    // reduce the S partial sums through LDS: red[w][rt][c][lane*4 + i]
#pragma unroll
    for (int rt = 0; rt < MAXR; ++rt)
      if (rt < nrt)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          *reinterpret_cast<f32x4*>(red + (((size_t)w * MAXR + rt) * 2 + c) * 256 + l * 4) =
              acc[rt][c];
    __syncthreads();
    if (GATEUP) {
      for (int el = threadIdx.x; el < nrows * 16; el += blockDim.x) {
        const int m = el >> 4, jj = el & 15;
        const int rt = m >> 4, mr = m & 15;
        const int off = (16 * (mr >> 2) + jj) * 4 + (mr & 3);
        float gs = 0.0f, us = 0.0f;
        for (int ww = 0; ww < S; ++ww) {
          const float* p = red + ((size_t)ww * MAXR + rt) * 2 * 256;
          gs += p[off];
          us += p[256 + off];
        }
        gate_up_epilogue(a, e, rbeg + rc + m, cg * 16 + jj, gs, us);
      }
    } else {
      for (int el = threadIdx.x; el < nrows * 32; el += blockDim.x) {
        const int m = el >> 5, cc = el & 31;
        const int rt = m >> 4, mr = m & 15, ct = cc >> 4, jj = cc & 15;
        const int off = (16 * (mr >> 2) + jj) * 4 + (mr & 3);
        float ys = 0.0f;
        for (int ww = 0; ww < S; ++ww) ys += red[(((size_t)ww * MAXR + rt) * 2 + ct) * 256 + off];
        down_epilogue(a, e, rbeg + rc + m, cg * 32 + cc, ys);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------- tiled kernel

constexpr int kBM = 128, kBK = 64, kLDA = kBK + 8;

template <int FMT, bool GATEUP>
__global__ __launch_bounds__(256) void k_tiled(const GemmArgs a) {
  using F = Format<FMT>;
  constexpr int KB = F::kBlock;
  __shared__ float2 lutf[256];
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLDA];
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  lutf[tid] = make_float2(F::level(tid & 15), F::level(tid >> 4));
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int q = logical / a.ncg, cg = logical - q * a.ncg;
  int e, ut;
  locate_item(a.offsets, a.E, q, [](int n) { return (n + kBM - 1) / kBM; }, e, ut);
  __syncthreads();
  if (e < 0) return;
  const int row0 = min(a.offsets[e], a.rows) + ut * kBM;
  const int nrows = min(kBM, min(a.offsets[e + 1], a.rows) - row0);
  const int n32 = l & 31, h = l >> 5;
  const int Nw = GATEUP ? 2 * a.I : a.N_out;
  int wrow[2];
  bool tact[2];
  if (GATEUP) {
    const int jb = cg * 128 + w * 32;
    tact[0] = tact[1] = jb < a.I;
    const int j = tact[0] ? jb + n32 : 0;
    wrow[0] = gate_row(a.layout, a.I, j);
    wrow[1] = up_row(a.layout, a.I, j);
  } else {
    const int c0 = cg * 256 + w * 64;
    tact[0] = c0 < a.N_out;
    tact[1] = c0 + 32 < a.N_out;
    wrow[0] = tact[0] ? c0 + n32 : 0;
    wrow[1] = tact[1] ? c0 + 32 + n32 : 0;
  }
  const int64_t growbase = (int64_t)e * Nw;
  const int K = a.K;
  const uint8_t* qp0 = a.wq + (growbase + wrow[0]) * (int64_t)(K / 2) + 16 * h;
  const uint8_t* qp1 = a.wq + (growbase + wrow[1]) * (int64_t)(K / 2) + 16 * h;
  const int nk = (K + kBK - 1) / kBK;

  u32x4 areg[4];
  auto loadA = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i, r = id >> 3, cidx = (id & 7) * 8;
      areg[i] = (r < nrows && kb + cidx < K)
                    ? *reinterpret_cast<const u32x4*>(a.A + (int64_t)(row0 + r) * K + kb + cidx)
                    : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto storeA = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i, r = id >> 3, cidx = (id & 7) * 8;
      *reinterpret_cast<u32x4*>(&As[buf][r * kLDA + cidx]) = areg[i];
    }
  };
  u32x4 braw[2];
  float bsc[2];
  auto loadB = [&](int kb) {
    const bool inK = kb + 32 * h < K;
    const int blk = (kb + 32 * h) / KB;
    if (tact[0] && inK) {
      braw[0] = *reinterpret_cast<const u32x4*>(qp0 + kb / 2);
      bsc[0] = F::scale(a.ws, growbase + wrow[0], K, blk);
    } else {
      braw[0] = u32x4{0u, 0u, 0u, 0u};
      bsc[0] = 0.0f;
    }
    if (tact[1] && inK) {
      braw[1] = *reinterpret_cast<const u32x4*>(qp1 + kb / 2);
      bsc[1] = F::scale(a.ws, growbase + wrow[1], K, blk);
    } else {
      braw[1] = u32x4{0u, 0u, 0u, 0u};
      bsc[1] = 0.0f;
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rt][c][i] = 0.0f;

  loadA(0);
  loadB(0);
  storeA(0);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    // dequantise this step's 32 nibbles per lane and weight row, scale folded in
    u32x4 bq[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
          const float2 v = lutf[(braw[c][s] >> (8 * bi)) & 255u];
          bq[c][s][bi] = pack_bf16x2(v.x * bsc[c], v.y * bsc[c]);
        }
    if (it + 1 < nk) {
      loadA((it + 1) * kBK);
      loadB((it + 1) * kBK);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const bf16x8 av =
            *reinterpret_cast<const bf16x8*>(&As[cur][(rt * 32 + n32) * kLDA + 32 * h + 8 * s]);
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[rt][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              av, __builtin_bit_cast(bf16x8, bq[c][s]), acc[rt][c], 0, 0, 0);
      }
    if (it + 1 < nk) storeA(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column n32 of each 32x32 tile, rows 8*(i/4) + 4*h + i%4
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rt_row = rt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
      if (rt_row < nrows) {
        const int row = row0 + rt_row;
        if (GATEUP) {
          if (tact[0]) gate_up_epilogue(a, e, row, cg * 128 + w * 32 + n32, acc[rt][0][i], acc[rt][1][i]);
        } else {
          if (tact[0]) down_epilogue(a, e, row, wrow[0], acc[rt][0][i]);
          if (tact[1]) down_epilogue(a, e, row, wrow[1], acc[rt][1][i]);
        }
      }
    }
}

// -------------------------------------------------------------- LoRA x A^T

// xa[row][q] = sum_h x_perm[row][h] * A[e(row)][q][h], fp32; one wave per row.
__global__ __launch_bounds__(256) void k_lora_xa(const uint16_t* __restrict__ x,
                                                 const int32_t* __restrict__ offsets, int E,
                                                 int rows, int H, const uint16_t* __restrict__ A,
                                                 int r, float* __restrict__ xa) {
  const int row = (int)((blockIdx.x * (unsigned)blockDim.x + threadIdx.x) >> 6);
  if (row >= rows) return;
  const int e = expert_of_row(offsets, E, row);
  const int l = lane_id();
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (int64_t)row * H);
  for (int qq = 0; qq < r; ++qq) {
    const u32x4* ar = reinterpret_cast<const u32x4*>(A + ((int64_t)e * r + qq) * H);
    float p = 0.0f;
    for (int c = l; c < H / 8; c += kWave) {
      const u32x4 xv = xr[c], av = ar[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) p += bf16lo(xv[i]) * bf16lo(av[i]) + bf16hi(xv[i]) * bf16hi(av[i]);
    }
    p = wave_sum(p);
    if (l == 0) xa[(int64_t)row * r + qq] = p;
  }
}

template <int FMT, bool GATEUP>
hipError_t run_skinny(const GemmArgs& a, int nitems, int nblk, hipStream_t s) {
  const int nwg = nitems * a.ncg;
  if (nwg == 0) return hipSuccess;
  int S = (4096 + nwg - 1) / nwg;
  S = max(1, min(S, min(16, nblk)));
  constexpr int MAXR = 2;
  const size_t lds = (size_t)S * MAXR * 2 * 256 * sizeof(float);
  hipLaunchKernelGGL((k_skinny<FMT, GATEUP, MAXR, 4>), dim3(nwg), dim3(64 * S), lds, s, a);
  return hipGetLastError();
}

template <int FMT, bool GATEUP>
hipError_t run_tiled(const GemmArgs& a, int ntiles, hipStream_t s) {
  const int nwg = ntiles * a.ncg;
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL((k_tiled<FMT, GATEUP>), dim3(nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t forward_fmt(const moe4_experts& ex, const uint16_t* x_perm, const int32_t* offsets,
                       int rows, float* y_perm, float* save_gu, const float* xa,
                       uint16_t* hbuf, int variant, const LaunchEvents& le, hipStream_t s) {
  const int E = ex.E, H = ex.H, I = ex.I;
  GemmArgs g{};
  g.offsets = offsets;
  g.E = E;
  g.rows = rows;
  g.I = I;
  g.layout = ex.gu_layout;
  g.act = ex.act;
  g.alpha = ex.act_alpha;
  g.limit = ex.act_limit;
  // gate_up: A = x_perm [rows, H], weights [E, 2I, H], output h [rows, I]
  g.wq = static_cast<const uint8_t*>(ex.gu_q);
  g.ws = ex.gu_s;
  g.K = H;
  g.N_out = I;
  g.A = x_perm;
  g.bias = ex.gu_bias;
  g.xa = xa;
  g.loraB = ex.lora_B;
  g.r = ex.lora_A ? ex.lora_r : 0;
  g.lscale = ex.lora_scale;
  g.hout = hbuf;
  g.yout = nullptr;
  g.save_gu = save_gu;
  // down: A = h [rows, I], weights [E, H, I], output y [rows, H]
  GemmArgs d = g;
  d.wq = static_cast<const uint8_t*>(ex.dn_q);
  d.ws = ex.dn_s;
  d.K = I;
  d.N_out = H;
  d.A = hbuf;
  d.bias = ex.dn_bias;
  d.xa = nullptr;
  d.loraB = nullptr;
  d.r = 0;
  d.hout = nullptr;
  d.yout = y_perm;
  d.save_gu = nullptr;
  const int touched = min(E, rows);
  hipError_t err;
  if (variant == MOE4_VARIANT_SKINNY) {
    g.ncg = I / 16;
    d.ncg = H / 32;
    le.before(0, s);
    err = run_skinny<FMT, true>(g, touched, H / Format<FMT>::kBlock, s);
    le.after(0, s);
    if (err != hipSuccess) return err;
    le.before(1, s);
    err = run_skinny<FMT, false>(d, touched, I / Format<FMT>::kBlock, s);
    le.after(1, s);
    return err;
  }
  const int ntiles = rows / kBM + touched;
  g.ncg = (I + 127) / 128;
  d.ncg = (H + 255) / 256;
  le.before(0, s);
  err = run_tiled<FMT, true>(g, ntiles, s);
  le.after(0, s);
  if (err != hipSuccess) return err;
  le.before(1, s);
  err = run_tiled<FMT, false>(d, ntiles, s);
  le.after(1, s);
  return err;
}

}  // namespace

size_t forward_ws_bytes(const moe4_experts& ex, int rows) {
  size_t b = align_up((size_t)rows * ex.I * sizeof(uint16_t), 256);
  if (ex.lora_A) b += align_up((size_t)rows * ex.lora_r * sizeof(float), 256);
  return b;
}

int choose_variant(const moe4_experts& ex, int rows) {
  if (ex.variant == MOE4_VARIANT_SKINNY || ex.variant == MOE4_VARIANT_TILED) return ex.variant;
  const int touched = rows < ex.E ? rows : ex.E;
  // expected rows per touched expert; the skinny kernel covers up to 32 in one pass
  return (touched == 0 || rows <= 16 * touched) ? MOE4_VARIANT_SKINNY : MOE4_VARIANT_TILED;
}

hipError_t launch_expert_forward(const moe4_experts& ex, const uint16_t* x_perm,
                                 const int32_t* offsets, int rows, float* y_perm,
                                 float* save_gu, float* save_xa, void* ws, int* variant,
                                 const LaunchEvents& le, hipStream_t s) {
  *variant = choose_variant(ex, rows);
  if (rows == 0) return hipSuccess;
  char* p = static_cast<char*>(ws);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(p);
  p += align_up((size_t)rows * ex.I * sizeof(uint16_t), 256);
  float* xa = nullptr;
  if (ex.lora_A) {
    xa = save_xa ? save_xa : reinterpret_cast<float*>(p);
    hipLaunchKernelGGL(k_lora_xa, dim3((rows + 3) / 4), dim3(256), 0, s, x_perm, offsets, ex.E,
                       rows, ex.H, ex.lora_A, ex.lora_r, xa);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (ex.format == MOE4_FMT_NF4)
    return forward_fmt<MOE4_FMT_NF4>(ex, x_perm, offsets, rows, y_perm, save_gu, xa, hbuf,
                                     *variant, le, s);
  return forward_fmt<MOE4_FMT_MXFP4>(ex, x_perm, offsets, rows, y_perm, save_gu, xa, hbuf,
                                     *variant, le, s);
}

}  // namespace moe4
