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

// Per-wave operands of one 128-k iteration of the skinny kernel.
template <int FMT, int NRT>
struct SkinnyBatch {
  u32x4 wraw[2];
  float sc[2][FMT == MOE4_FMT_NF4 ? 1 : 4];
  u32x4 av[NRT][4];
};

// Buffer resources and lane offsets of one wave of the skinny kernel.
struct SkinnyLane {
  rsrc_t rq, rs, ra;    // this expert's nibbles and scales; this row chunk's activations
  int qoff[2];          // byte offset of the lane's 16-byte column in weight row c, k = 0
  int srow[2];          // weight row index of column tile c (inside the expert)
};

// Each k-iteration covers 128 k: lane (n = l%16, g = l/16) loads 16 bytes
// (32 k) of its weight row with one 128-bit load, so the four lanes of a row
// read 64 contiguous bytes.
//  NF4: lane g's 32 k lie in one absmax block; each weight becomes
//       bf16(level * absmax) and MFMA step s uses k = kb + 32g + 8s.
//  MXFP4: the 4x4 transpose above makes MFMA step s cover exactly the 32-k
//       block kb/32 + s (k = kb + 32s + 8g), so the block's power-of-two
//       scale multiplies the fp32 partial sum of that step.
template <int FMT, int NRT>
__device__ __forceinline__ void skinny_load(SkinnyBatch<FMT, NRT>& bt, const SkinnyLane& sl,
                                            int K, int it, int it1) {
  using F = Format<FMT>;
  constexpr bool PRESCALE = FMT == MOE4_FMT_NF4;
  const int l = lane_id(), nl = l & 15, g = l >> 4;
  const int kb = it * 128;
  const bool live = it < it1;
  const bool ink = live && kb + 32 * g < K;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    bt.wraw[c] = buf_load_b128(sl.rq, ink ? sl.qoff[c] + kb / 2 : kOob);
    if (PRESCALE) {
      const int so = ink ? (sl.srow[c] * (K / 64) + (kb + 32 * g) / 64) * 4 : kOob;
      bt.sc[c][0] = __uint_as_float(buf_load_b32(sl.rs, so));
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bool inb = live && kb + 32 * st < K;
        bt.sc[c][st] = Format<MOE4_FMT_MXFP4>::e8m0(
            buf_load_u8(sl.rs, inb ? sl.srow[c] * (K / 32) + kb / 32 + st : kOob));
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int m = rt * 16 + nl;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int k = PRESCALE ? kb + 32 * g + 8 * st : kb + 32 * st + 8 * g;
      bt.av[rt][st] = buf_load_b128(sl.ra, (live && k < K) ? (m * K + k) * 2 : kOob);
    }
  }
}

template <int FMT, int NRT>
__device__ __forceinline__ void skinny_compute(const SkinnyBatch<FMT, NRT>& bt,
                                               const float2* lutf, const uint32_t* lut,
                                               f32x4 (&acc)[2][2]) {
  constexpr bool PRESCALE = FMT == MOE4_FMT_NF4;
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (PRESCALE) {
      // 32 nibbles -> 32 bf16 operands bf16(level * absmax)
      u32x4 bq[4];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
          const float2 f = lutf[(bt.wraw[c][st] >> (8 * bi)) & 255u];
          bq[st][bi] = pack_bf16x2(f.x * bt.sc[c][0], f.y * bt.sc[c][0]);
        }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int st = 0; st < 4; ++st)
          acc[rt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, bt.av[rt][st]), __builtin_bit_cast(bf16x8, bq[st]),
              acc[rt][c], 0, 0, 0);
    } else {
      u32x4 v = bt.wraw[c];
      transpose4x4_rows(v);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        u32x4 t;
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) t[bi] = lut[(v[st] >> (8 * bi)) & 255u];
        const bf16x8 bq = __builtin_bit_cast(bf16x8, t);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          const f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, bt.av[rt][st]), bq, zero4, 0, 0, 0);
          acc[rt][c] += bt.sc[c][st] * p;
        }
      }
    }
  }
}

// K loop of one wave over iterations [it0, it1) for NRT 16-row tiles; the
// next iteration's loads are in flight while the current one is dequantised
// and multiplied.
template <int FMT, int NRT>
__device__ __forceinline__ void skinny_kloop(const SkinnyLane& sl, int K, int it0, int it1,
                                             const float2* lutf, const uint32_t* lut,
                                             f32x4 (&acc)[2][2]) {
  SkinnyBatch<FMT, NRT> b0, b1;
  skinny_load(b0, sl, K, it0, it1);
  for (int it = it0; it < it1; it += 2) {
    if (it + 1 < it1) skinny_load(b1, sl, K, it + 1, it1);
    skinny_compute(b0, lutf, lut, acc);
    if (it + 1 >= it1) break;
    if (it + 2 < it1) skinny_load(b0, sl, K, it + 2, it1);
    skinny_compute(b1, lutf, lut, acc);
  }
}

// Skinny grouped GEMM: one workgroup = one expert x 32 weight rows (gate_up:
// 16 (gate, up) pairs; down: 32 output columns); its S waves split K and are
// reduced through LDS; the expert's rows are taken 32 at a time.
template <int FMT, bool GATEUP>
__global__ __launch_bounds__(512) void k_skinny(const GemmArgs a) {
  using F = Format<FMT>;
  constexpr bool PRESCALE = FMT == MOE4_FMT_NF4;
  constexpr int MAXR = 2;
  constexpr int KB = F::kBlock;
  // byte -> two levels: fp32 pair (NF4, scaled afterwards) or bf16 pair (MXFP4)
  __shared__ __attribute__((aligned(16))) float2 lutf[PRESCALE ? 256 : 1];
  __shared__ uint32_t lut[PRESCALE ? 1 : 256];
  extern __shared__ __attribute__((aligned(16))) float red[];   // [S][MAXR][2][256]
  const int S = blockDim.x >> 6, w = wave_id(), l = lane_id();
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    if (PRESCALE) lutf[i] = make_float2(F::level(i & 15), F::level(i >> 4));
    else lut[i] = lut_bf16x2<FMT>(i);
  }
  const int item = blockIdx.x / a.ncg, cg = blockIdx.x - item * a.ncg;
  int e, unused;
  locate_item(a.offsets, a.E, item, [](int n) { return n > 0 ? 1 : 0; }, e, unused);
  e = __builtin_amdgcn_readfirstlane(e);
  __syncthreads();
  if (e < 0) return;
  const int K = a.K;
  const int rbeg = min(a.offsets[e], a.rows);
  const int n_e = min(a.offsets[e + 1], a.rows) - rbeg;
  const int nl = l & 15, g = l >> 4;
  const int Nw = GATEUP ? 2 * a.I : a.N_out;
  SkinnyLane sl;
  if (GATEUP) {
    const int j = cg * 16 + nl;
    sl.srow[0] = gate_row(a.layout, a.I, j);
    sl.srow[1] = up_row(a.layout, a.I, j);
  } else {
    sl.srow[0] = cg * 32 + nl;
    sl.srow[1] = cg * 32 + 16 + nl;
  }
  sl.rq = make_rsrc(a.wq + (int64_t)e * Nw * (K / 2), (uint32_t)Nw * (K / 2));
  const int sbytes = PRESCALE ? 4 : 1;
  sl.rs = make_rsrc(static_cast<const uint8_t*>(a.ws) + (int64_t)e * Nw * (K / KB) * sbytes,
                    (uint32_t)Nw * (K / KB) * sbytes);
#pragma unroll
  for (int c = 0; c < 2; ++c) sl.qoff[c] = sl.srow[c] * (K / 2) + 16 * g;
  const int nit = (K + 127) / 128;
  const int it0 = (int)((int64_t)w * nit / S), it1 = (int)((int64_t)(w + 1) * nit / S);
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int rc = 0; rc < n_e; rc += 16 * MAXR) {
    const int nrows = min(16 * MAXR, n_e - rc);
    const int nrt = (nrows + 15) >> 4;
    f32x4 acc[2][2] = {{zero4, zero4}, {zero4, zero4}};
    sl.ra = make_rsrc(a.A + (int64_t)(rbeg + rc) * K, (uint32_t)nrows * K * 2);
    if (nrt == 1) skinny_kloop<FMT, 1>(sl, K, it0, it1, lutf, lut, acc);
    else skinny_kloop<FMT, 2>(sl, K, it0, it1, lutf, lut, acc);
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

// One k-tile of the tiled kernel: dequantise this lane's 32 weight bytes (two
// weight rows x 32 k, scale folded in) and run the MFMAs against the A tile.
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
        const float2 v = lutf[(braw[c][s] >> (8 * bi)) & 255u];
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

// Tiled grouped GEMM: one workgroup = one 128-row tile of one expert's
// permuted rows x 128 output columns (gate_up: 128 (gate, up) pairs, i.e. 256
// weight rows; down: 256 output columns). The A tile goes through LDS
// (double-buffered, one k-tile of 64 ahead); each wave owns 64 weight rows and
// fetches its lanes' nibbles and scales straight into registers one k-tile
// ahead. All loads are raw buffer loads: rows past the tile, k past K and
// weight rows past the stack read as zero.
template <int FMT, bool GATEUP>
__global__ __launch_bounds__(256, 2) void k_tiled(const GemmArgs a) {
  using F = Format<FMT>;
  constexpr int KB = F::kBlock;
  __shared__ __attribute__((aligned(16))) float2 lutf[256];
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLDA];
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  lutf[tid] = make_float2(F::level(tid & 15), F::level(tid >> 4));
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int q = logical / a.ncg, cg = logical - q * a.ncg;
  int e, ut;
  locate_item(a.offsets, a.E, q, [](int n) { return (n + kBM - 1) / kBM; }, e, ut);
  // wave-uniform by construction; make it visible to the compiler so that the
  // buffer resources below live in scalar registers
  e = __builtin_amdgcn_readfirstlane(e);
  ut = __builtin_amdgcn_readfirstlane(ut);
  __syncthreads();
  if (e < 0) return;
  const int K = a.K;
  const int row0 = min(a.offsets[e], a.rows) + ut * kBM;
  const int nrows = min(kBM, min(a.offsets[e + 1], a.rows) - row0);
  const int nrt = (nrows + 31) >> 5;
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
  // buffer resources: this tile's activations, this expert's nibbles and scales
  const rsrc_t ra = make_rsrc(a.A + (int64_t)row0 * K, (uint32_t)nrows * K * 2);
  const rsrc_t rq = make_rsrc(a.wq + (int64_t)e * Nw * (K / 2), (uint32_t)Nw * (K / 2));
  const int sbytes = FMT == MOE4_FMT_NF4 ? 4 : 1;
  const rsrc_t rs = make_rsrc(static_cast<const uint8_t*>(a.ws) + (int64_t)e * Nw * (K / KB) * sbytes,
                              (uint32_t)Nw * (K / KB) * sbytes);
  int aoff[4], acol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    acol[i] = (id & 7) * 8;
    aoff[i] = ((id >> 3) * K + acol[i]) * 2;
  }
  int qoff[2], soff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    qoff[c] = wrow[c] * (K / 2) + 16 * h;
    soff[c] = (wrow[c] * (K / KB)) * sbytes;
  }
  const int nk = (K + kBK - 1) / kBK;
  auto loadA = [&](u32x4 (&r)[4], int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = buf_load_b128(ra, kb + acol[i] < K ? aoff[i] + 2 * kb : kOob);
  };
  auto storeA = [&](const u32x4 (&r)[4], int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      *reinterpret_cast<u32x4*>(&As[buf][(id >> 3) * kLDA + acol[i]]) = r[i];
    }
  };
  auto loadB = [&](u32x4 (&br)[2], float (&bs)[2], int kb) {
    const bool ink = kb + 32 * h < K;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bool on = ink && tact[c];
      br[c] = buf_load_b128(rq, on ? qoff[c] + kb / 2 : kOob);
      const int so = on ? soff[c] + ((kb + 32 * h) / KB) * sbytes : kOob;
      if (FMT == MOE4_FMT_NF4) bs[c] = __uint_as_float(buf_load_b32(rs, so));
      else bs[c] = Format<MOE4_FMT_MXFP4>::e8m0(buf_load_u8(rs, so));
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rt][c][i] = 0.0f;

  u32x4 ra_regs[4], bcur[2], bnext[2];
  float scur[2], snext[2];
  loadA(ra_regs, 0);
  loadB(bcur, scur, 0);
  storeA(ra_regs, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      loadA(ra_regs, (kt + 1) * kBK);
      loadB(bnext, snext, (kt + 1) * kBK);
    }
    tiled_step<FMT>(As[kt & 1], lutf, bcur, scur, nrt, acc);
    if (more) storeA(ra_regs, (kt + 1) & 1);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bcur[c] = bnext[c];
      scur[c] = snext[c];
    }
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
          if (tact[0])
            gate_up_epilogue(a, e, row, cg * 128 + w * 32 + n32, acc[rt][0][i], acc[rt][1][i]);
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
hipError_t run_skinny(const GemmArgs& a, int nitems, hipStream_t s) {
  const int nwg = nitems * a.ncg;
  if (nwg == 0) return hipSuccess;
  // split K over S waves so that ~6K waves stream the weights (about six per
  // SIMD), each wave keeping at least two 128-k iterations
  const int nit = (a.K + 127) / 128;
  int S = (6144 + nwg - 1) / nwg;
  S = max(1, min(S, min(8, nit / 2)));
  constexpr int MAXR = 2;
  const size_t lds = (size_t)S * MAXR * 2 * 256 * sizeof(float);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_skinny<FMT, GATEUP>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)(8 * MAXR * 2 * 256 * sizeof(float)));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_skinny<FMT, GATEUP>), dim3(nwg), dim3(64 * S), lds, s, a);
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
