// Backward of the grouped expert path with respect to its input and the
// per-expert LoRA adapters: the input gradient goes through the frozen 4-bit
// weights ("dgrad"; project page "experts4bit-qlora", "Use this when"), the
// adapter gradients are grouped reductions over each expert's rows. The 4-bit
// base and the biases are frozen (the QLoRA setting of the solutions index's
// fused-experts entry) and get no gradient.
//
// The dgrad GEMMs contract over the weight rows, the opposite orientation of
// the forward: each MFMA lane needs 8 consecutive weight rows of one column,
// which it assembles in registers from one byte of each row (see k_dgrad).
#include <type_traits>

#include "common.hpp"
#include "formats.hpp"
#include "gemm_common.hpp"
#include "internal.hpp"

namespace moe4 {
namespace {

enum { DGRAD_DOWN = 0, DGRAD_GATEUP = 1 };

struct DgradArgs {
  const uint8_t* wq;   // stack [E, Kw, Nw] (rows = reduction dim), Nw/2 bytes per row
  const void* ws;      // scales per row: Nw/64 f32 (NF4), Nw/32 u8 (MXFP4) or
                       // Nw/64 u8 absmax codes (double-quantised NF4)
  const float* ws2;    // double-quantised NF4: absmax2, one per 256 absmax of the stack
  const float* dqoff;  // double-quantised NF4: the stack's absmax offset
  const float* dqbook; // double-quantised NF4: the 256-entry code book
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
template <int ACT>
__device__ __forceinline__ void act_backward_t(float g, float u, float dh, float alpha,
                                               float limit, float& dg, float& du) {
  if constexpr (ACT == MOE4_ACT_SWIGLU) {
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

// One workgroup per CU: eight waves, an expert tile of up to kDM rows and kDN
// output columns, k-tiles of kDK weight rows (the reduction). A k-tile's
// activation rows, packed weights [kDK rows][kDN / 2 B] and scales come to LDS
// by direct loads, two k-tiles ahead; one barrier per k-tile.
//
// Each wave owns 64 output columns as two interleaved 32-wide MFMA column
// tiles: MFMA column c of tile m is output column nb + 64 w + 2 c + m, so that
// one byte of a weight row holds the lane's weight of both tiles (low nibble:
// tile 0). The MFMA wants each lane's B operand along the reduction (8
// consecutive weight rows of one column), which is the opposite of the packed
// order; the lane therefore reads one byte from each of the 8 rows, looks the
// byte up in the table of fp32 NF4 level pairs (MXFP4: the hardware e2m1
// conversion), scales and rounds, and packs the two tiles' operands in
// registers. No transposed copy of the weights is written, and no wave reads
// another wave's dequantised values: the barrier only guards the ring.
constexpr int kDM = 160, kDN = 512, kDK = 64, kDStages = 3;
constexpr int kDMaxRowTiles = kDM / 32;
// Stage: A [kDM rows][128 B] (16-byte chunk c of row r stored at c ^ ((r >> 1)
// & 7), the forward's layout: the 16 rows of an operand read fall in 16
// different bank groups), the packed weights [kDK rows][256 B] (16-byte chunk
// c of row r stored at (c + 2 ((r >> 3) & 1)) % 16: the two halves of a wave,
// which read rows 8 apart, hit disjoint banks), and the scales in 4-byte slots
// 64 b + r (block b of the workgroup's columns, weight row r of the k-tile:
// NF4 the fp32 absmax, MXFP4 the e8m0 byte in the low byte; double-quantised
// NF4 the code byte, and in slot 512 + 64 b + r the group's absmax2).
constexpr int kDStageA = kDM * kDK * 2;
constexpr int kDStageW = kDK * kDN / 2;
constexpr int kDStageS = 4096;
constexpr int kDStage = kDStageA + kDStageW + kDStageS;
constexpr int kDLds = kDStages * kDStage;
static_assert(kDLds + 256 * 8 + 256 * 4 <= 160 * 1024, "dgrad LDS");
static_assert(kDM % 64 == 32, "A loads: two per lane, a third for waves 0..3");

template <int FMT, int MODE>
__global__ __launch_bounds__(512, 1) void k_dgrad(const DgradArgs a) {
  using F = Format<FMT>;
  constexpr bool NF4 = FMT != MOE4_FMT_MXFP4;   // NF4 levels (plain or double-quantised)
  constexpr bool DQ = FMT == MOE4_FMT_NF4_DQ;
  constexpr int KB = F::kBlock;
  // direct loads per lane and batch: A 2 (+1 in waves 0..3), weights 2, scales
  constexpr int kSLoads = FMT == MOE4_FMT_NF4 ? 1 : 2;
  constexpr int kLoads = 4 + kSLoads;
  __shared__ __attribute__((aligned(16))) float2 lutf[NF4 ? 256 : 1];
  __shared__ float dqbook[DQ ? 256 : 1];
  extern __shared__ __attribute__((aligned(16))) uint8_t gmem[];
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id();
  float2 lv0 = make_float2(0.0f, 0.0f);
  float dq0 = 0.0f;
  if (NF4 && tid < 256) lv0 = make_float2(F::level(tid & 15), F::level(tid >> 4));
  if (DQ && tid < 256) dq0 = a.dqbook[tid];
  int e, ut, cg, obeg, oend;
  locate_tile_sorted<kDM>(a.offsets, a.E, a.ncg, blockIdx.x, e, ut, cg, obeg, oend);
  if (NF4 && tid < 256) lutf[tid] = lv0;
  if (DQ && tid < 256) dqbook[tid] = dq0;
  e = __builtin_amdgcn_readfirstlane(e);
  ut = __builtin_amdgcn_readfirstlane(ut);
  cg = __builtin_amdgcn_readfirstlane(cg);
  obeg = __builtin_amdgcn_readfirstlane(obeg);
  oend = __builtin_amdgcn_readfirstlane(oend);
  __syncthreads();
  if (e < 0) return;
  const int Kw = a.Kw, Nw = a.Nw;
  const int ebeg = min(obeg, a.rows);
  const int n_e = min(oend, a.rows) - ebeg;
  const int R = eq_tile_rows<kDM>(n_e);
  const int row0 = ebeg + ut * R;
  const int nrows = min(R, ebeg + n_e - row0);
  const int nrt = (nrows + 31) >> 5;
  const int c32 = l & 31, hk = l >> 5;
  const int nb = cg * kDN;
  // the lane's two output columns (tile 0, tile 1)
  const int n0 = nb + 64 * w + 2 * c32;

  // every resource is wave-uniform by construction, said so to the compiler
  // (else it may keep one in vector registers and loop over its lanes' values)
  const rsrc_t ra = make_rsrc_uniform(a.A + (int64_t)row0 * Kw, (uint32_t)nrows * Kw * 2);
  const rsrc_t rq = make_rsrc_uniform(a.wq + (int64_t)e * Kw * (Nw / 2), (uint32_t)Kw * (Nw / 2));
  constexpr int sbytes = FMT == MOE4_FMT_NF4 ? 4 : 1;
  const rsrc_t rs = make_rsrc_uniform(
      static_cast<const uint8_t*>(a.ws) + (int64_t)e * Kw * (Nw / KB) * sbytes,
      (uint32_t)Kw * (Nw / KB) * sbytes);
  const rsrc_t rs2 =
      DQ ? make_rsrc_uniform(a.ws2, (uint32_t)(((int64_t)a.E * Kw * (Nw / KB) + 255) / 256) * 4)
         : rs;
  auto stage = [&](int st) { return gmem + st * kDStage; };

  // ---- loader roles (lane-contiguous LDS destinations)
  // A: load p of lane (w, l) fills bytes 8192 p + 1024 w + 16 l of the tile =
  //    row 64 p + 8 w + l / 8, physical chunk l % 8 (p = 2: waves 0..3 only)
  const int a_lc = (l & 7) ^ ((4 * w + (l >> 4)) & 7);
  int a_off[3];
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const int r = 64 * p + 8 * w + (l >> 3);
    a_off[p] = r < nrows ? (r * Kw + 8 * a_lc) * 2 : kOob;
  }
  // weights: load q fills bytes 8192 q + 1024 w + 16 l = row 32 q + 4 w + l /
  //    16, physical chunk l % 16
  int w_row[2], w_off[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int rr = 32 * q + 4 * w + (l >> 4);
    const int c = ((l & 15) - 2 * ((rr >> 3) & 1)) & 15;
    w_row[q] = rr;
    w_off[q] = nb + 32 * c < Nw ? rr * (Nw / 2) + nb / 2 + 16 * c : kOob;
  }
  auto issue = [&](int kt) {
    const int kb = kt * kDK;
    uint8_t* base = stage(kt % kDStages);
    const bool kin = (NF4 && KB % kDK == 0) || kb + 8 * a_lc < Kw;
#pragma unroll
    for (int p = 0; p < 3; ++p)
      if (p < 2 || w < 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, MOE4_LDS(base + p * 8192 + w * 1024), 16,
            (kin && a_off[p] != kOob) ? a_off[p] + 2 * kb : kOob, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, MOE4_LDS(base + kDStageA + q * 8192 + w * 1024), 16,
          (w_off[q] != kOob && kb + w_row[q] < Kw) ? w_off[q] + kb * (Nw / 2) : kOob, 0, 0, 0);
    uint8_t* sb = base + kDStageA + kDStageW;
    const bool rin = kb + l < Kw;
    if constexpr (FMT == MOE4_FMT_NF4) {
      // slot 64 w + l: block w of the workgroup's columns, row l
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, MOE4_LDS(sb + w * 256), 4,
          (rin && nb / 64 + w < Nw / 64) ? ((kb + l) * (Nw / 64) + nb / 64 + w) * 4 : kOob, 0, 0,
          0);
    } else if constexpr (DQ) {
      const bool on = rin && nb / 64 + w < Nw / 64;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, MOE4_LDS(sb + w * 256), 1, on ? (kb + l) * (Nw / 64) + nb / 64 + w : kOob, 0, 0, 0);
      // absmax2 of the slot's flat absmax index (in the whole stack)
      const int64_t flat = ((int64_t)e * Kw + kb + l) * (Nw / 64) + nb / 64 + w;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs2, MOE4_LDS(sb + 2048 + w * 256), 4,
                                               on ? (int)(flat >> 8) * 4 : kOob, 0, 0, 0);
    } else {
      // slots 512 q + 64 w + l: block 8 q + w, row l
#pragma unroll
      for (int q = 0; q < 2; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, MOE4_LDS(sb + q * 2048 + w * 256), 1,
            (rin && nb / 32 + 8 * q + w < Nw / 32) ? (kb + l) * (Nw / 32) + nb / 32 + 8 * q + w
                                                   : kOob,
            0, 0, 0);
    }
  };
  // wait until batch kt is in (at most the following batch in flight)
  auto wait_batch = [&](bool more) {
    if (more) {
      if (w < 4) wait_vmcnt<kLoads + 1>();
      else wait_vmcnt<kLoads>();
    } else {
      wait_vmcnt<0>();
    }
  };

  // ---- operand addresses within a stage
  // B bytes: rows 16 s + 8 hk + i, byte 32 w + c32 of the row (its physical
  // chunk is rotated by 2 for rows with bit 3 set, i.e. hk = 1)
  const int b_rd = kDStageA + 8 * hk * 256 + 16 * ((2 * w + (c32 >> 4) + 2 * hk) & 15) + (c32 & 15);
  // scales: NF4 / double-quantised block w, MXFP4 block 2 w + c32 / 16; rows
  // 16 s + 8 hk .. + 7
  const int s_rd = kDStageA + kDStageW + 4 * ((NF4 ? w : 2 * w + (c32 >> 4)) * 64 + 8 * hk);
  // A operand of step s: chunk 2 s + hk of row 32 rt + c32
  int a_rd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) a_rd[s] = c32 * 128 + 16 * ((2 * s + hk) ^ ((c32 >> 1) & 7));
  const float dqo = DQ ? a.dqoff[0] : 0.0f;

  // B operands of step s of the k-tile in stage base (tile 0 and tile 1)
  auto b_operands = [&](const uint8_t* base, int s, u32x4& b0, u32x4& b1) {
    uint32_t by[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) by[i] = base[b_rd + (16 * s + i) * 256];
    const u32x4 s0 = *reinterpret_cast<const u32x4*>(base + s_rd + 64 * s);
    const u32x4 s1 = *reinterpret_cast<const u32x4*>(base + s_rd + 64 * s + 16);
    float sc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t raw = i < 4 ? s0[i] : s1[i - 4];
      if constexpr (FMT == MOE4_FMT_NF4) {
        sc[i] = __uint_as_float(raw);
      } else if constexpr (DQ) {
        const float g2 = *reinterpret_cast<const float*>(base + s_rd + 2048 + 64 * s + 4 * i);
        sc[i] = mul_then_add(dqbook[raw & 255u], g2, dqo);
      } else {
        sc[i] = __uint_as_float((raw & 255u) << 23);
      }
    }
    if constexpr (NF4) {
      f32x2 lv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) lv[i] = reinterpret_cast<const f32x2*>(lutf)[by[i]];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        b0[q] = pack_bf16x2(lv[2 * q].x * sc[2 * q], lv[2 * q + 1].x * sc[2 * q + 1]);
        b1[q] = pack_bf16x2(lv[2 * q].y * sc[2 * q], lv[2 * q + 1].y * sc[2 * q + 1]);
      }
    } else {
      uint32_t p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        p[i] = __builtin_bit_cast(uint32_t,
                                  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(by[i], sc[i], 0));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        b0[q] = __builtin_amdgcn_perm(p[2 * q + 1], p[2 * q], 0x05040100u);
        b1[q] = __builtin_amdgcn_perm(p[2 * q + 1], p[2 * q], 0x07060302u);
      }
    }
  };

  const int nk = (Kw + kDK - 1) / kDK;
  auto kloop = [&](auto nrt_c) {
    constexpr int NRT = decltype(nrt_c)::value;
    f32x16 acc0[NRT], acc1[NRT];
#pragma unroll
    for (int i = 0; i < NRT; ++i)
#pragma unroll
      for (int z = 0; z < 16; ++z) acc0[i][z] = acc1[i][z] = 0.0f;

    issue(0);
    if (nk > 1) issue(1);
    // LoRA delta of dx (gate_up dgrad) while the first batches land: MFMA steps
    // over the rank, A = bf16(t[row][q]), B = A_e[q][n] (bf16 already). They
    // start from zero accumulators, which then hold the fp32 sum scaled once
    // by lora_scale, as dx = dGU W + lora_scale * (bf16(t) A) defines it; the
    // k-tiles accumulate on top.
    if (MODE == DGRAD_GATEUP && a.r) {
      // the lane's two columns are adjacent: one dword of a row of A_e
      const uint32_t* ar = reinterpret_cast<const uint32_t*>(a.loraA + (int64_t)e * a.r * Nw + n0);
      for (int q0 = 0; q0 < a.r; q0 += 16) {
        uint32_t x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int q = q0 + 8 * hk + i;
          x[i] = (n0 < Nw && q < a.r) ? ar[(int64_t)q * (Nw / 2)] : 0u;
        }
        u32x4 pb0, pb1;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          pb0[jj] = __builtin_amdgcn_perm(x[2 * jj + 1], x[2 * jj], 0x05040100u);
          pb1[jj] = __builtin_amdgcn_perm(x[2 * jj + 1], x[2 * jj], 0x07060302u);
        }
#pragma unroll
        for (int i = 0; i < NRT; ++i) {
          const int rr = i * 32 + c32;
          const float* tr = a.t + (int64_t)(row0 + rr) * a.r;
          u32x4 pk;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int q = q0 + 8 * hk + 2 * jj;
            const float x0 = (rr < nrows && q < a.r) ? tr[q] : 0.0f;
            const float x1 = (rr < nrows && q + 1 < a.r) ? tr[q + 1] : 0.0f;
            pk[jj] = pack_bf16x2(x0, x1);
          }
          acc0[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pk),
                                                            __builtin_bit_cast(bf16x8, pb0),
                                                            acc0[i], 0, 0, 0);
          acc1[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pk),
                                                            __builtin_bit_cast(bf16x8, pb1),
                                                            acc1[i], 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < NRT; ++i)
#pragma unroll
        for (int z = 0; z < 16; ++z) {
          acc0[i][z] *= a.lscale;
          acc1[i][z] *= a.lscale;
        }
    }
    for (int kt = 0; kt < nk; ++kt) {
      wait_batch(kt + 1 < nk);
      // batch kt is in LDS everywhere; stage (kt + 2) % 3 is free
      lds_barrier();
      if (kt + 2 < nk) issue(kt + 2);
      const uint8_t* base = stage(kt % kDStages);
#pragma unroll
      for (int s = 0; s < kDK / 16; ++s) {
        u32x4 b0, b1;
        b_operands(base, s, b0, b1);
#pragma unroll
        for (int i = 0; i < NRT; ++i) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(base + a_rd[s] + i * 4096);
          acc0[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, b0),
                                                            acc0[i], 0, 0, 0);
          acc1[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, b1),
                                                            acc1[i], 0, 0, 0);
        }
      }
    }

    // ---- epilogue: lane holds columns n0 (acc0) and n0 + 1 (acc1) of each
    // 32 x 32 row tile, rows 8 (z / 4) + 4 hk + z % 4. Stores go through
    // resources over the tile's rows; a pair past Nw is sent out of range.
    const bool con = n0 < Nw;
    if (MODE == DGRAD_DOWN) {
      // n0 indexes the intermediate dimension: dH[row][n0], dH[row][n0 + 1].
      // The layout and the activation are uniform: one epilogue per pair.
      auto down = [&](auto halves_c, auto act_c) {
        constexpr bool HALVES = decltype(halves_c)::value;
        constexpr int ACT = decltype(act_c)::value;
        const int I = a.I;
        const rsrc_t rg = make_rsrc_uniform(a.save_gu + (int64_t)row0 * 2 * I,
                                            (uint32_t)nrows * 2 * I * 4);
        const rsrc_t rd = make_rsrc_uniform(a.dgu + (int64_t)row0 * 2 * I,
                                            (uint32_t)nrows * 2 * I * 2);
        // byte offsets within a row: HALVES gate pair at n0, up pair at I + n0;
        // INTERLEAVED (g, u, g, u) at 2 n0
        const uint32_t gin = con ? (uint32_t)(HALVES ? n0 : 2 * n0) * 4 : (uint32_t)kOob;
        const uint32_t uin = con ? (uint32_t)(I + n0) * 4 : (uint32_t)kOob;
        const uint32_t gout = con ? (uint32_t)(HALVES ? n0 : 2 * n0) * 2 : (uint32_t)kOob;
        const uint32_t uout = con ? (uint32_t)(I + n0) * 2 : (uint32_t)kOob;
        // group q = entries 4 (q % 4) .. + 3 of row tile q / 4: the saved
        // pre-activations of group q + 1 are loaded while group q is finished
        // (each wait then covers one group's loads, not one element's)
        constexpr int NG = 4 * NRT;
        auto row_of = [&](int q, int zz) {
          const int z = 4 * (q & 3) + zz;
          return (q >> 2) * 32 + 8 * (z >> 2) + 4 * hk + (z & 3);
        };
        auto load_group = [&](int q, u32x4 (&b)[4]) {
#pragma unroll
          for (int zz = 0; zz < 4; ++zz) {
            const uint32_t ro = (uint32_t)row_of(q, zz) * 8 * I;
            if constexpr (HALVES) {
              const u32x2 gg = __builtin_bit_cast(
                  u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, (int)(ro + gin), 0, 0));
              const u32x2 uu = __builtin_bit_cast(
                  u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, (int)(ro + uin), 0, 0));
              b[zz] = u32x4{gg.x, uu.x, gg.y, uu.y};
            } else {
              b[zz] = buf_load_b128(rg, (int)(ro + gin));
            }
          }
        };
        u32x4 bufs[2][4];
        load_group(0, bufs[0]);
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          if (q + 1 < NG) load_group(q + 1, bufs[(q + 1) & 1]);
          const int i = q >> 2;
#pragma unroll
          for (int zz = 0; zz < 4; ++zz) {
            const int z = 4 * (q & 3) + zz;
            const u32x4 v = bufs[q & 1][zz];   // g0, u0, g1, u1
            float dg0, du0, dg1, du1;
            act_backward_t<ACT>(__uint_as_float(v[0]), __uint_as_float(v[1]), acc0[i][z],
                                a.alpha, a.limit, dg0, du0);
            act_backward_t<ACT>(__uint_as_float(v[2]), __uint_as_float(v[3]), acc1[i][z],
                                a.alpha, a.limit, dg1, du1);
            const uint32_t ro = (uint32_t)row_of(q, zz) * 4 * I;
            if constexpr (HALVES) {
              __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(dg0, dg1), rd, (int)(ro + gout),
                                                    0, 0);
              __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(du0, du1), rd, (int)(ro + uout),
                                                    0, 0);
            } else {
              const u32x2 o = {pack_bf16x2(dg0, du0), pack_bf16x2(dg1, du1)};
              __builtin_amdgcn_raw_buffer_store_b64(o, rd, (int)(ro + gout), 0, 0);
            }
          }
        }
      };
      using Sw = std::integral_constant<int, MOE4_ACT_SWIGLU>;
      using Cl = std::integral_constant<int, MOE4_ACT_SWIGLU_CLAMPED>;
      if (a.layout == MOE4_GU_HALVES) {
        if (a.act == MOE4_ACT_SWIGLU) down(std::true_type{}, Sw{});
        else down(std::true_type{}, Cl{});
      } else {
        if (a.act == MOE4_ACT_SWIGLU) down(std::false_type{}, Sw{});
        else down(std::false_type{}, Cl{});
      }
    } else {
      const rsrc_t rx = make_rsrc_uniform(a.dx + (int64_t)row0 * Nw, (uint32_t)nrows * Nw * 4);
      const uint32_t cin = con ? (uint32_t)n0 * 4 : (uint32_t)kOob;
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
#pragma unroll
        for (int z = 0; z < 16; ++z) {
          const int rr = i * 32 + 8 * (z >> 2) + 4 * hk + (z & 3);
          const u32x2 o = {__float_as_uint(acc0[i][z]), __float_as_uint(acc1[i][z])};
          __builtin_amdgcn_raw_buffer_store_b64(o, rx,
                                                (int)(rr * 4 * Nw + cin), 0, 0);
        }
      }
    }
  };
  switch (nrt) {
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    default: kloop(std::integral_constant<int, kDMaxRowTiles>{}); break;
  }
}

template <int FMT>
hipError_t set_dgrad_lds() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dgrad<FMT, DGRAD_DOWN>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kDLds);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dgrad<FMT, DGRAD_GATEUP>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kDLds);
}

template <int FMT>
hipError_t backward_fmt(const moe4_experts& ex, const uint16_t* x_perm, const int32_t* offsets,
                        int rows, const float* save_gu, const float* save_xa,
                        const uint16_t* dy_perm, float* dx_perm, float* dA, float* dB,
                        uint16_t* dgu, float* tbuf, uint16_t* bt_ws, const LaunchEvents& le,
                        hipStream_t s) {
  const int E = ex.E, H = ex.H, I = ex.I;
  const bool lora = ex.lora_A != nullptr;
  const int touched = min(E, rows);
  const int ntiles = rows / kDM + touched;
  static const hipError_t attr = set_dgrad_lds<FMT>();
  if (attr != hipSuccess) return attr;
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
  d.ws2 = ex.dn_s2;
  d.dqoff = ex.dn_soff;
  d.dqbook = ex.dq_book;
  d.Kw = H;
  d.Nw = I;
  d.A = dy_perm;
  d.save_gu = save_gu;
  d.dgu = dgu;
  d.ncg = (I + kDN - 1) / kDN;
  le.before(0, s);
  if (ntiles * d.ncg > 0)
    // ntiles bounds the row tiles; tile j of the largest-first order runs on
    // XCD j % 8, so every XCD needs ceil(tiles / 8) * ncg ids
    hipLaunchKernelGGL((k_dgrad<FMT, DGRAD_DOWN>), dim3((ntiles + 7) * d.ncg), dim3(512), kDLds,
                       s, d);
  le.after(0, s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (lora && rows > 0) {
    // t = dGU B_e as a projection onto the rank against B_e^T
    err = launch_transpose_rank(ex.lora_B, E, 2 * I, ex.lora_r, bt_ws, s);
    if (err != hipSuccess) return err;
    err = launch_rank_proj(dgu, offsets, E, rows, 2 * I, bt_ws, ex.lora_r, tbuf, s);
    if (err != hipSuccess) return err;
  }
  // dx = dGU W_gu[e] (+ LoRA): W_gu is [2I (reduction), H]
  DgradArgs g = d;
  g.wq = static_cast<const uint8_t*>(ex.gu_q);
  g.ws = ex.gu_s;
  g.ws2 = ex.gu_s2;
  g.dqoff = ex.gu_soff;
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
    hipLaunchKernelGGL((k_dgrad<FMT, DGRAD_GATEUP>), dim3((ntiles + 7) * g.ncg), dim3(512),
                       kDLds, s, g);
  le.after(1, s);
  err = hipGetLastError();
  if (err != hipSuccess || !lora) return err;
  // dB[e] = s * dGU^T bf16(xa)  -> [E, 2I, r];  dA[e] = s * bf16(t)^T x -> [E, r, H]
  err = launch_rank_reduce(dgu, 2 * I, save_xa, ex.lora_r, offsets, rows, E, ex.lora_scale, dB,
                           false, s);
  if (err != hipSuccess) return err;
  return launch_rank_reduce(x_perm, H, tbuf, ex.lora_r, offsets, rows, E, ex.lora_scale, dA, true,
                            s);
}

}  // namespace

size_t backward_ws_bytes(const moe4_experts& ex, int rows) {
  size_t b = align_up((size_t)rows * 2 * ex.I * sizeof(uint16_t), 256);
  if (ex.lora_A) {
    b += align_up((size_t)rows * ex.lora_r * sizeof(float), 256);
    b += align_up((size_t)ex.E * ex.lora_r * 2 * ex.I * sizeof(uint16_t), 256);   // B^T
  }
  return b;
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
  uint16_t* bt_ws = ex.lora_A ? reinterpret_cast<uint16_t*>(p) : nullptr;
  if (ex.lora_A) p += align_up((size_t)ex.E * ex.lora_r * 2 * ex.I * sizeof(uint16_t), 256);
  if (rows == 0 && !ex.lora_A) return hipSuccess;
  if (ex.format == MOE4_FMT_NF4_DQ)
    // both absmax levels decoded per k-tile inside the dgrad kernels
    return backward_fmt<MOE4_FMT_NF4_DQ>(ex, x_perm, offsets, rows, save_gu, save_xa, dy_perm,
                                         dx_perm, dA, dB, dgu, tbuf, bt_ws, le, s);
  if (ex.format == MOE4_FMT_NF4)
    return backward_fmt<MOE4_FMT_NF4>(ex, x_perm, offsets, rows, save_gu, save_xa, dy_perm,
                                      dx_perm, dA, dB, dgu, tbuf, bt_ws, le, s);
  return backward_fmt<MOE4_FMT_MXFP4>(ex, x_perm, offsets, rows, save_gu, save_xa, dy_perm,
                                      dx_perm, dA, dB, dgu, tbuf, bt_ws, le, s);
}

}  // namespace moe4
