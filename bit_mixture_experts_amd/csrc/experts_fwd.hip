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

// Copies of the byte -> level table in LDS. Lanes look up data-dependent
// entries; with the table stored entry-major and lane l reading copy l % 32,
// the lookups of a wave fall in distinct banks instead of colliding.
constexpr int kLutCopies = 1;

// ------------------------------------------------------------ skinny kernel

// 4x4 transpose of dwords across the four 16-lane rows of a wave: on entry
// row g holds D[g][0..3] in v[0..3]; on exit row g holds D[0..3][g].
// permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; permlane16_swap exchanges the odd 16-lane rows of
// its first operand with the even rows of its second.
__device__ __forceinline__ void transpose4x4_rows(u32x4& v) {
  auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  v[0] = c[0];
  v[1] = c[1];
  v[2] = d[0];
  v[3] = d[1];
}

// K loop of one wave for NRT 16-row tiles of one expert's rows and two
// 16-column weight tiles. Each k-iteration covers 128 k: lane (n = l%16,
// g = l/16) loads 16 bytes (32 k) of its weight row with one 128-bit load, so
// the four lanes of a row read 64 contiguous bytes.
//  NF4: lane g's 32 k lie in one absmax block; each weight becomes
//       bf16(level * absmax) and MFMA step s uses k = kb + 32g + 8s.
//  MXFP4: the 4x4 transpose above makes MFMA step s cover exactly the 32-k
//       block kb/32 + s (k = kb + 32s + 8g), so the block's power-of-two
//       scale multiplies the fp32 partial sum of that step.
template <int FMT, int NRT, int U>
struct SkinnyBatch {
  u32x4 wraw[U][2];
  float sc[U][2][FMT == MOE4_FMT_NF4 ? 1 : 4];
  u32x4 av[U][NRT][4];
};

template <int FMT, int NRT, int U>
__device__ __forceinline__ void skinny_load(SkinnyBatch<FMT, NRT, U>& bt, const GemmArgs& a,
                                            const uint8_t* __restrict__ q0,
                                            const uint8_t* __restrict__ q1, int64_t srow0,
                                            int64_t srow1, const uint16_t* __restrict__ arow0,
                                            int rows_here, int it, int it1) {
  using F = Format<FMT>;
  constexpr bool PRESCALE = FMT == MOE4_FMT_NF4;
  const int l = lane_id(), nl = l & 15, g = l >> 4;
  const int K = a.K;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int kb = (it + u) * 128;
    const bool live = it + u < it1;
    const bool ink = live && kb + 32 * g < K;
    bt.wraw[u][0] = ink ? *reinterpret_cast<const u32x4*>(q0 + kb / 2 + 16 * g) : z4;
    bt.wraw[u][1] = ink ? *reinterpret_cast<const u32x4*>(q1 + kb / 2 + 16 * g) : z4;
    if (PRESCALE) {
      bt.sc[u][0][0] = ink ? F::scale(a.ws, srow0, K, (kb + 32 * g) / 64) : 0.0f;
      bt.sc[u][1][0] = ink ? F::scale(a.ws, srow1, K, (kb + 32 * g) / 64) : 0.0f;
    } else {
#pragma unroll
      for (int st = 0; st < (PRESCALE ? 1 : 4); ++st) {
        const bool inb = live && kb + 32 * st < K;
        bt.sc[u][0][st] = inb ? F::scale(a.ws, srow0, K, kb / 32 + st) : 0.0f;
        bt.sc[u][1][st] = inb ? F::scale(a.ws, srow1, K, kb / 32 + st) : 0.0f;
      }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int m = rt * 16 + nl;
      const uint16_t* ar = arow0 + (int64_t)m * K;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int k = PRESCALE ? kb + 32 * g + 8 * st : kb + 32 * st + 8 * g;
        bt.av[u][rt][st] = (live && m < rows_here && k < K)
                               ? *reinterpret_cast<const u32x4*>(ar + k) : z4;
      }
    }
  }
}

template <int FMT, int NRT, int U>
__device__ __forceinline__ void skinny_compute(const SkinnyBatch<FMT, NRT, U>& bt, int it,
                                               int it1, const float2* lutf, const uint32_t* lut,
                                               f32x4 (&acc)[2][2]) {
  constexpr bool PRESCALE = FMT == MOE4_FMT_NF4;
  // lutf / lut point at this lane's copy of the replicated table (stride kLutCopies)
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (it + u >= it1) break;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (PRESCALE) {
        // 32 nibbles -> 32 bf16 operands bf16(level * absmax)
        u32x4 bq[4];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int bi = 0; bi < 4; ++bi) {
            const float2 f = lutf[((bt.wraw[u][c][st] >> (8 * bi)) & 255u) * kLutCopies];
            bq[st][bi] = pack_bf16x2(f.x * bt.sc[u][c][0], f.y * bt.sc[u][c][0]);
          }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int st = 0; st < 4; ++st)
            acc[rt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, bt.av[u][rt][st]), __builtin_bit_cast(bf16x8, bq[st]),
                acc[rt][c], 0, 0, 0);
      } else {
        u32x4 v = bt.wraw[u][c];
        transpose4x4_rows(v);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          u32x4 t;
          t[0] = lut[(v[st] & 255u) * kLutCopies];
          t[1] = lut[((v[st] >> 8) & 255u) * kLutCopies];
          t[2] = lut[((v[st] >> 16) & 255u) * kLutCopies];
          t[3] = lut[(v[st] >> 24) * kLutCopies];
          const bf16x8 bq = __builtin_bit_cast(bf16x8, t);
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            const f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, bt.av[u][rt][st]), bq, zero4, 0, 0, 0);
            acc[rt][c] += bt.sc[u][c][st] * p;
          }
        }
      }
    }
  }
}

// K loop of one wave for NRT 16-row tiles of one expert's rows and two
// 16-column weight tiles. Each k-iteration covers 128 k: lane (n = l%16,
// g = l/16) loads 16 bytes (32 k) of its weight row with one 128-bit load, so
// the four lanes of a row read 64 contiguous bytes. Batches of U iterations
// are double-buffered: the next batch's loads are in flight while the current
// one is dequantised and multiplied.
//  NF4: lane g's 32 k lie in one absmax block; each weight becomes
//       bf16(level * absmax) and MFMA step s uses k = kb + 32g + 8s.
//  MXFP4: the 4x4 transpose above makes MFMA step s cover exactly the 32-k
//       block kb/32 + s (k = kb + 32s + 8g), so the block's power-of-two
//       scale multiplies the fp32 partial sum of that step.
template <int FMT, int NRT, int U>
__device__ __forceinline__ void skinny_kloop(const GemmArgs& a, const uint8_t* __restrict__ q0,
                                             const uint8_t* __restrict__ q1, int64_t srow0,
                                             int64_t srow1, const uint16_t* __restrict__ arow0,
                                             int rows_here, int it0, int it1,
                                             const float2* lutf, const uint32_t* lut,
                                             f32x4 (&acc)[2][2]) {
  SkinnyBatch<FMT, NRT, U> b0, b1;
  skinny_load(b0, a, q0, q1, srow0, srow1, arow0, rows_here, it0, it1);
  for (int it = it0; it < it1; it += 2 * U) {
    if (it + U < it1) skinny_load(b1, a, q0, q1, srow0, srow1, arow0, rows_here, it + U, it1);
    skinny_compute(b0, it, it1, lutf, lut, acc);
    if (it + U >= it1) break;
    if (it + 2 * U < it1)
      skinny_load(b0, a, q0, q1, srow0, srow1, arow0, rows_here, it + 2 * U, it1);
    skinny_compute(b1, it + U, it1, lutf, lut, acc);
  }
}

template <int FMT, bool GATEUP, int U>
__global__ __launch_bounds__(512) void k_skinny(const GemmArgs a) {
  using F = Format<FMT>;
  constexpr bool PRESCALE = FMT == MOE4_FMT_NF4;
  constexpr int MAXR = 2;
  // dynamic LDS: the byte table replicated kLutCopies times (entry-major, so
  // lanes reading random entries hit distinct banks), then the reduction buffer
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  float2* lutf_all = reinterpret_cast<float2*>(dyn);
  uint32_t* lut_all = reinterpret_cast<uint32_t*>(dyn);
  float* red = dyn + (PRESCALE ? 2 : 1) * 256 * kLutCopies;
  const int S = blockDim.x >> 6, w = wave_id(), l = lane_id();
  for (int i = threadIdx.x; i < 256 * kLutCopies; i += blockDim.x) {
    const int byte = i / kLutCopies;
    if (PRESCALE) lutf_all[i] = make_float2(F::level(byte & 15), F::level(byte >> 4));
    else lut_all[i] = lut_bf16x2<FMT>(byte);
  }
  const float2* lutf = lutf_all + (l & (kLutCopies - 1));
  const uint32_t* lut = lut_all + (l & (kLutCopies - 1));
  const int item = blockIdx.x / a.ncg, cg = blockIdx.x - item * a.ncg;
  int e, unused;
  locate_item(a.offsets, a.E, item, [](int n) { return n > 0 ? 1 : 0; }, e, unused);
  __syncthreads();
  if (e < 0) return;
  const int rbeg = min(a.offsets[e], a.rows);
  const int n_e = min(a.offsets[e + 1], a.rows) - rbeg;
  const int nl = l & 15;
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
  const uint8_t* q0 = a.wq + (growbase + wrow[0]) * (int64_t)(a.K / 2);
  const uint8_t* q1 = a.wq + (growbase + wrow[1]) * (int64_t)(a.K / 2);
  const int nit = (a.K + 127) / 128;
  const int it0 = (int)((int64_t)w * nit / S), it1 = (int)((int64_t)(w + 1) * nit / S);
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int rc = 0; rc < n_e; rc += 16 * MAXR) {
    const int nrows = min(16 * MAXR, n_e - rc);
    const int nrt = (nrows + 15) >> 4;
    f32x4 acc[2][2] = {{zero4, zero4}, {zero4, zero4}};
    const uint16_t* arow0 = a.A + (int64_t)(rbeg + rc) * a.K;
    if (nrt == 1)
      skinny_kloop<FMT, 1, U>(a, q0, q1, growbase + wrow[0], growbase + wrow[1], arow0, nrows,
                              it0, it1, lutf, lut, acc);
    else
      skinny_kloop<FMT, 2, U>(a, q0, q1, growbase + wrow[0], growbase + wrow[1], arow0, nrows,
                              it0, it1, lutf, lut, acc);
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

// Per-wave state of the tiled kernel's K loop.
struct TiledLane {
  const uint8_t* q[2];   // this lane's 16-byte column of each weight row, at k = 32h
  int64_t srow[2];       // scale rows
  bool tact[2];          // weight tile inside the stack
};

// One k-tile of the tiled kernel: dequantise this lane's weight nibbles (scale
// folded in) and run the MFMAs against the A tile in LDS buffer `buf`.
template <int FMT>
__device__ __forceinline__ void tiled_step(const uint16_t* As, const float2* lutf,
                                           const u32x4 (&braw)[2], const float (&bsc)[2],
                                           int nrt, f32x16 (&acc)[4][2]) {
  const int l = lane_id(), n32 = l & 31, h = l >> 5;
  u32x4 bq[2][4];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const float2 v = lutf[((braw[c][s] >> (8 * bi)) & 255u) * kLutCopies];
        bq[c][s][bi] = pack_bf16x2(v.x * bsc[c], v.y * bsc[c]);
      }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    if (rt < nrt) {   // uniform: row tiles past the tile's rows are skipped
      bf16x8 af[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        af[s] = *reinterpret_cast<const bf16x8*>(&As[(rt * 32 + n32) * kLDA + 32 * h + 8 * s]);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[rt][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              af[s], __builtin_bit_cast(bf16x8, bq[c][s]), acc[rt][c], 0, 0, 0);
    }
  }
}

// K loop for NRT 32-row tiles (NRT = ceil(rows / 32) of this tile). The A tile
// (activations) is double-buffered in LDS; both the A tile and each lane's
// weight nibbles are fetched two k-tiles ahead (two register sets, loop
// unrolled by two), so an HBM round trip overlaps two k-tiles of MFMA work.
template <int FMT>
__device__ __forceinline__ void tiled_kloop(const GemmArgs& a, const TiledLane& tl,
                                            uint16_t (*As)[kBM * kLDA], const float2* lutf,
                                            int row0, int nrows, f32x16 (&acc)[4][2]) {
  const int nrt = (nrows + 31) >> 5;
  using F = Format<FMT>;
  constexpr int KB = F::kBlock;
  const int tid = threadIdx.x, l = lane_id();
  const int h = l >> 5;
  const int K = a.K;
  const int nk = (K + kBK - 1) / kBK;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  auto loadA = [&](u32x4 (&r)[4], int kt) {
    const int kb = kt * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i, rr = id >> 3, cidx = (id & 7) * 8;
      r[i] = (kt < nk && rr < nrows && kb + cidx < K)
                 ? *reinterpret_cast<const u32x4*>(a.A + (int64_t)(row0 + rr) * K + kb + cidx)
                 : z4;
    }
  };
  auto storeA = [&](const u32x4 (&r)[4], int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i, rr = id >> 3, cidx = (id & 7) * 8;
      *reinterpret_cast<u32x4*>(&As[buf][rr * kLDA + cidx]) = r[i];
    }
  };
  auto loadB = [&](u32x4 (&br)[2], float (&bs)[2], int kt) {
    const int kb = kt * kBK;
    const bool inK = kt < nk && kb + 32 * h < K;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bool on = tl.tact[c] && inK;
      br[c] = on ? *reinterpret_cast<const u32x4*>(tl.q[c] + kb / 2) : z4;
      bs[c] = on ? F::scale(a.ws, tl.srow[c], K, (kb + 32 * h) / KB) : 0.0f;
    }
  };

  u32x4 r0[4], r1[4], b0[2], b1[2];
  float s0[2], s1[2];
  loadA(r0, 0);
  loadB(b0, s0, 0);
  loadA(r1, 1);
  loadB(b1, s1, 1);
  storeA(r0, 0);
  __syncthreads();
  for (int it = 0; it < nk; it += 2) {
    // k-tile `it` (LDS buffer 0, weights b0); fetch k-tile it+2 into r0/b0
    {
      const u32x4 bc[2] = {b0[0], b0[1]};
      const float sc[2] = {s0[0], s0[1]};
      loadA(r0, it + 2);
      loadB(b0, s0, it + 2);
      tiled_step<FMT>(As[0], lutf, bc, sc, nrt, acc);
      if (it + 1 < nk) storeA(r1, 1);
      __syncthreads();
    }
    if (it + 1 >= nk) break;
    // k-tile `it+1` (LDS buffer 1, weights b1); fetch k-tile it+3 into r1/b1
    {
      const u32x4 bc[2] = {b1[0], b1[1]};
      const float sc[2] = {s1[0], s1[1]};
      loadA(r1, it + 3);
      loadB(b1, s1, it + 3);
      tiled_step<FMT>(As[1], lutf, bc, sc, nrt, acc);
      if (it + 2 < nk) storeA(r0, 0);
      __syncthreads();
    }
  }
}

template <int FMT, bool GATEUP>
__global__ __launch_bounds__(256) void k_tiled(const GemmArgs a) {
  using F = Format<FMT>;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLDA];
  extern __shared__ __attribute__((aligned(16))) float2 lutf_all[];   // [256][kLutCopies]
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  for (int i = tid; i < 256 * kLutCopies; i += 256) {
    const int byte = i / kLutCopies;
    lutf_all[i] = make_float2(F::level(byte & 15), F::level(byte >> 4));
  }
  const float2* lutf = lutf_all + (l & (kLutCopies - 1));
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
  TiledLane tl;
  if (GATEUP) {
    const int jb = cg * 128 + w * 32;
    tl.tact[0] = tl.tact[1] = jb < a.I;
    const int j = tl.tact[0] ? jb + n32 : 0;
    wrow[0] = gate_row(a.layout, a.I, j);
    wrow[1] = up_row(a.layout, a.I, j);
  } else {
    const int c0 = cg * 256 + w * 64;
    tl.tact[0] = c0 < a.N_out;
    tl.tact[1] = c0 + 32 < a.N_out;
    wrow[0] = tl.tact[0] ? c0 + n32 : 0;
    wrow[1] = tl.tact[1] ? c0 + 32 + n32 : 0;
  }
  const int64_t growbase = (int64_t)e * Nw;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    tl.srow[c] = growbase + wrow[c];
    tl.q[c] = a.wq + tl.srow[c] * (int64_t)(a.K / 2) + 16 * h;
  }
  f32x16 acc[4][2];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rt][c][i] = 0.0f;
  tiled_kloop<FMT>(a, tl, As, lutf, row0, nrows, acc);

  // epilogue: lane holds column n32 of each 32x32 tile, rows 8*(i/4) + 4*h + i%4
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rt_row = rt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
      if (rt_row < nrows) {
        const int row = row0 + rt_row;
        if (GATEUP) {
          if (tl.tact[0])
            gate_up_epilogue(a, e, row, cg * 128 + w * 32 + n32, acc[rt][0][i], acc[rt][1][i]);
        } else {
          if (tl.tact[0]) down_epilogue(a, e, row, wrow[0], acc[rt][0][i]);
          if (tl.tact[1]) down_epilogue(a, e, row, wrow[1], acc[rt][1][i]);
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
hipError_t run_skinny(const GemmArgs& a, int nitems, hipStream_t s) {
  const int nwg = nitems * a.ncg;
  if (nwg == 0) return hipSuccess;
  // split K over S waves so that ~6K waves stream the weights (about six per
  // SIMD), each wave keeping at least two 128-k iterations
  const int nit = (a.K + 127) / 128;
  int S = (6144 + nwg - 1) / nwg;
  S = max(1, min(S, min(8, nit / 2)));
  constexpr int MAXR = 2;
  const size_t lut_bytes = (FMT == MOE4_FMT_NF4 ? 8 : 4) * 256 * kLutCopies;
  const size_t lds = lut_bytes + (size_t)S * MAXR * 2 * 256 * sizeof(float);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_skinny<FMT, GATEUP, 1>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)(lut_bytes + 8 * MAXR * 2 * 256 * 4));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_skinny<FMT, GATEUP, 1>), dim3(nwg), dim3(64 * S), lds, s, a);
  return hipGetLastError();
}

template <int FMT, bool GATEUP>
hipError_t run_tiled(const GemmArgs& a, int ntiles, hipStream_t s) {
  const int nwg = ntiles * a.ncg;
  if (nwg == 0) return hipSuccess;
  constexpr size_t lds = (size_t)256 * kLutCopies * sizeof(float2);
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_tiled<FMT, GATEUP>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_tiled<FMT, GATEUP>), dim3(nwg), dim3(256), lds, s, a);
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
    err = run_skinny<FMT, true>(g, touched, s);
    le.after(0, s);
    if (err != hipSuccess) return err;
    le.before(1, s);
    err = run_skinny<FMT, false>(d, touched, s);
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
