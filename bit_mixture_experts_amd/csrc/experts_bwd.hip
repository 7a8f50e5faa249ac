// Backward of the grouped expert path with respect to its input and the
// per-expert LoRA adapters: the input gradient goes through the frozen 4-bit
// weights ("dgrad"; project page "experts4bit-qlora", "Use this when"), the
// adapter gradients are grouped reductions over each expert's rows. The 4-bit
// base and the biases are frozen (the QLoRA setting of the solutions index's
// fused-experts entry) and get no gradient.
//
// The dgrad GEMMs contract over the weight rows, the opposite orientation of
// the forward: each k-tile of packed weights (rows along the reduction) is
// dequantised by the whole workgroup into LDS, transposed so that each MFMA
// lane reads 8 consecutive reduction values with one 128-bit LDS load.
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

// One workgroup per CU: eight waves, an expert tile of up to kGM rows and kGN
// output columns, k-tiles of kGK weight rows. A k-tile's packed weights
// [kGK rows][kGN/2 B] and their scales come to LDS by direct loads one k-tile
// ahead of its activation tile; while the MFMAs of k-tile kt run, every thread
// dequantises its share of k-tile kt + 1 (8 weight rows x 2 columns) into a
// transposed bf16 buffer Bt [kGN columns][kGK], which the next k-tile's MFMAs
// read as their B operand. Wave w computes columns 32 w .. +31 of the tile
// against every 32-row tile (the loop is instantiated per count of row tiles,
// so that short expert tiles keep all eight waves busy).
constexpr int kGM = 256, kGN = 256, kGK = 32, kGStages = 4;
// Stage: A [kGM rows][kGK] bf16 (four 16-byte chunks a row, chunk c of row r
// stored at c ^ ((r >> 2) & 3): 16 consecutive rows of one chunk column fall
// in 16 different 16-byte bank groups of the 64-bank LDS), the packed weights
// [kGK rows][kGN / 2 B] (16-byte chunk c of row r stored at c ^ ((r >> 3) & 3),
// so that the dequantising threads' byte reads spread over the banks), and
// the scales in 4-byte slots 32 b + r (block b of weight row r: NF4 the fp32
// absmax, MXFP4 the e8m0 byte; double-quantised NF4 the code byte, and in slot
// 128 + 32 b + r the group's absmax2).
constexpr int kGStageA = kGM * kGK * 2;
constexpr int kGStageB = kGK * kGN / 2;
constexpr int kGStageS = 1024;
constexpr int kGStage = kGStageA + kGStageB + kGStageS;
// Bt [kGN columns][kGK] bf16 at a pitch of 80 bytes: the MFMA operand reads
// of 16 consecutive columns hit 16 different 16-byte bank groups
constexpr int kGBtPitch = kGK * 2 + 16;
constexpr int kGBt = kGN * kGBtPitch;
constexpr int kGLds = kGStages * kGStage + 2 * kGBt;
constexpr int kGLoads = 3;   // direct loads per thread and batch
static_assert(kGLds + 256 * 8 <= 160 * 1024, "dgrad LDS");

template <int FMT, int MODE>
__global__ __launch_bounds__(512, 1) void k_dgrad(const DgradArgs a) {
  using F = Format<FMT>;
  constexpr bool NF4 = FMT != MOE4_FMT_MXFP4;   // NF4 levels (plain or double-quantised)
  constexpr bool DQ = FMT == MOE4_FMT_NF4_DQ;
  constexpr int KB = F::kBlock;
  __shared__ __attribute__((aligned(16))) float2 lutf[256];
  __shared__ float dqbook[DQ ? 256 : 1];
  extern __shared__ __attribute__((aligned(16))) uint8_t gmem[];
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  if (tid < 256) lutf[tid] = make_float2(F::level(tid & 15), F::level(tid >> 4));
  if (DQ && tid < 256) dqbook[tid] = a.dqbook[tid];
  int e, ut, cg;
  locate_tile_eq<kGM>(a.offsets, a.E, a.ncg, blockIdx.x, e, ut, cg);
  e = __builtin_amdgcn_readfirstlane(e);
  ut = __builtin_amdgcn_readfirstlane(ut);
  cg = __builtin_amdgcn_readfirstlane(cg);
  __syncthreads();
  if (e < 0) return;
  const int Kw = a.Kw, Nw = a.Nw;
  const int ebeg = min(a.offsets[e], a.rows);
  const int n_e = min(a.offsets[e + 1], a.rows) - ebeg;
  const int R = eq_tile_rows<kGM>(n_e);
  const int row0 = ebeg + ut * R;
  const int nrows = min(R, ebeg + n_e - row0);
  const int n32 = l & 31, h = l >> 5;
  const int nb = cg * kGN;

  const rsrc_t ra = make_rsrc(a.A + (int64_t)row0 * Kw, (uint32_t)nrows * Kw * 2);
  const rsrc_t rq = make_rsrc(a.wq + (int64_t)e * Kw * (Nw / 2), (uint32_t)Kw * (Nw / 2));
  constexpr int sbytes = FMT == MOE4_FMT_NF4 ? 4 : 1;
  const rsrc_t rs = make_rsrc(static_cast<const uint8_t*>(a.ws) + (int64_t)e * Kw * (Nw / KB) * sbytes,
                              (uint32_t)Kw * (Nw / KB) * sbytes);
  auto stage = [&](int st) { return gmem + st * kGStage; };
  uint8_t* bt = gmem + kGStages * kGStage;

  // ---- loader roles (lane-contiguous LDS destinations)
  // A: load p of thread t fills bytes 8192 p + 16 t of the A tile = row
  //    128 p + t / 4, physical chunk t % 4
  const int arow = tid >> 2;
  const int a_col = 8 * ((tid & 3) ^ ((arow >> 2) & 3));
  const int a_off = (arow * Kw + a_col) * 2;
  // weights (waves 0..3): thread t fills bytes 16 t of the packed tile = row
  //    t / 8, physical chunk t % 8 = logical chunk ^ ((row >> 3) & 3)
  // scales (waves 4..7): thread 256 + i fills slot i = 32 b + r (NF4: slots
  //    past 127 read zeros; double-quantised NF4: slots past 127 hold the
  //    absmax2 of slot i - 128)
  const int bq_row = (tid & 255) >> 3;
  const int bq_byte = 16 * ((tid & 7) ^ ((bq_row >> 3) & 3));
  const bool bq_on = nb / 2 + bq_byte < Nw / 2;
  const int si = tid & 255;
  const int sj = DQ ? si & 127 : si;
  const int s_row = sj & 31, s_blk = sj >> 5;
  const bool s_on = (FMT == MOE4_FMT_NF4 ? si < 128 : true) && (nb / KB + s_blk) < Nw / KB;
  const rsrc_t rs2 = DQ ? make_rsrc(a.ws2, (uint32_t)(((int64_t)a.E * Kw * (Nw / KB) + 255) / 256) * 4)
                        : rs;
  auto issue_w = [&](int kt, int st) {   // weights / scales of k-tile kt
    uint8_t* base = stage(st);
    const int kb = kt * kGK;
    if (w < 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, MOE4_LDS(base + kGStageA + w * 1024), 16,
          (bq_on && kb + bq_row < Kw) ? (kb + bq_row) * (Nw / 2) + nb / 2 + bq_byte : kOob, 0, 0,
          0);
    } else {
      const int soff =
          (s_on && kb + s_row < Kw) ? ((kb + s_row) * (Nw / KB) + nb / KB + s_blk) * sbytes : kOob;
      if constexpr (FMT == MOE4_FMT_NF4) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, MOE4_LDS(base + kGStageA + kGStageB + (w - 4) * 256), 4, soff, 0, 0, 0);
      } else if constexpr (DQ) {
        if (w < 6) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, MOE4_LDS(base + kGStageA + kGStageB + (w - 4) * 256), 1, soff, 0, 0, 0);
        } else {
          // absmax2 of the slot's flat absmax index (in the whole stack)
          const int64_t flat =
              ((int64_t)e * Kw + kb + s_row) * (Nw / KB) + nb / KB + s_blk;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs2, MOE4_LDS(base + kGStageA + kGStageB + (w - 4) * 256), 4,
              (s_on && kb + s_row < Kw) ? (int)(flat >> 8) * 4 : kOob, 0, 0, 0);
        }
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, MOE4_LDS(base + kGStageA + kGStageB + (w - 4) * 256), 1, soff, 0, 0, 0);
      }
    }
  };
  // batch kt: the A tile of k-tile kt (stage kt % 4) and the weights of
  // k-tile kt + 1 (stage (kt + 1) % 4)
  auto issue = [&](int kt) {
    const int kb = kt * kGK;
    const int aoff = kb + a_col < Kw ? a_off + 2 * kb : kOob;
#pragma unroll
    for (int p = 0; p < 2; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, MOE4_LDS(stage(kt % kGStages) + p * 8192 + w * 1024), 16,
          aoff == kOob ? kOob : aoff, p * 128 * Kw * 2, 0, 0);
    issue_w(kt + 1, (kt + 1) % kGStages);
  };
  // dequantise the packed weights of stage st into Bt buffer bi: thread t
  // takes weight rows 8 (t % 4) .. +7 (chunk t % 4 of a Bt column) and byte
  // t / 4 (columns 2 (t / 4), +1). LDS reads go through vector types (the
  // compiler then does not wait for the LDS-DMA loads in flight).
  const int dq_c = tid & 3, dq_j = tid >> 2;
  const int dq_chunk = dq_j >> 4, dq_in = dq_j & 15;
  const int dq_blk = NF4 ? dq_j >> 5 : dq_j >> 4;
  auto dequant_to_bt = [&](int st, int bi) {
    const uint8_t* base = stage(st);
    const uint8_t* qb = base + kGStageA;
    const u32x4* sv = reinterpret_cast<const u32x4*>(base + kGStageA + kGStageB) + 8 * dq_blk + 2 * dq_c;
    const u32x4 s0 = sv[0], s1 = sv[1];   // scale slots of rows 8 dq_c .. +7
    u32x4 g0 = {0u, 0u, 0u, 0u}, g1 = {0u, 0u, 0u, 0u};
    if constexpr (DQ) {
      g0 = sv[32];   // their absmax2 (slots + 128)
      g1 = sv[33];
    }
    const float dqo = DQ ? a.dqoff[0] : 0.0f;
    float v0[8], v1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * dq_c + i;
      // the 8 bytes holding byte dq_in of the row's chunk dq_chunk
      const u32x2 pr = *reinterpret_cast<const u32x2*>(
          qb + row * (kGN / 2) + 16 * (dq_chunk ^ ((row >> 3) & 3)) + 8 * (dq_in >> 3));
      const uint32_t wd = (dq_in & 4) ? pr.y : pr.x;
      const uint32_t byte = (wd >> (8 * (dq_in & 3))) & 255u;
      const uint32_t sraw = i < 4 ? s0[i] : s1[i - 4];
      if constexpr (NF4) {
        // absmax (double-quantised: fp32(fp32(book[code] * absmax2) + offset);
        // a one-byte load fills the low byte of its slot)
        const float sc =
            DQ ? mul_then_add(dqbook[sraw & 255u], __uint_as_float(i < 4 ? g0[i] : g1[i - 4]), dqo)
               : __uint_as_float(sraw);
        const f32x2 lv = reinterpret_cast<const f32x2*>(lutf)[byte];
        v0[i] = lv.x * sc;
        v1[i] = lv.y * sc;
      } else {
        const float sc = __uint_as_float((sraw & 255u) << 23);
        const uint32_t p =
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(byte, sc, 0));
        v0[i] = bf16lo(p);
        v1[i] = bf16hi(p);
      }
    }
    uint8_t* bb = bt + bi * kGBt;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float* v = q ? v1 : v0;
      const u32x4 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                        pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
      *reinterpret_cast<u32x4*>(bb + (2 * dq_j + q) * kGBtPitch + 16 * dq_c) = pk;
    }
  };

  const int nk = (Kw + kGK - 1) / kGK;
  const int nrt = (nrows + 31) >> 5;
  // column of this wave's MFMA B operand and output (wave w: columns
  // nb + 32 w .. +31 against every row tile)
  const int col = 32 * w + n32;
  const int n = nb + col;
  auto kloop = [&](auto nrt_c) {
    constexpr int NRT = decltype(nrt_c)::value;
    f32x16 acc[NRT];
#pragma unroll
    for (int i = 0; i < NRT; ++i)
#pragma unroll
      for (int z = 0; z < 16; ++z) acc[i][z] = 0.0f;

    // prologue: weights of k-tile 0, batches 0 .. 2, then k-tile 0 into Bt 0
    issue_w(0, 0);
#pragma unroll
    for (int j = 0; j < kGStages - 1; ++j)
      if (j < nk) issue(j);
    // LoRA delta of dx (gate_up dgrad) while the first batches land: MFMA steps
    // over the rank, A = bf16(t[row][q]), B = A_e[q][n] (bf16 already). They
    // start from zero accumulators, which then hold the fp32 sum scaled once
    // by lora_scale, as dx = dGU W + lora_scale * (bf16(t) A) defines it; the
    // k-tiles accumulate on top.
    if (MODE == DGRAD_GATEUP && a.r) {
      const uint16_t* ar = a.loraA + ((int64_t)e * a.r) * Nw + n;
      for (int q0 = 0; q0 < a.r; q0 += 16) {
        u32x4 pb;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int q = q0 + 8 * h + 2 * jj;
          const uint32_t x0 = (n < Nw && q < a.r) ? ar[(int64_t)q * Nw] : 0u;
          const uint32_t x1 = (n < Nw && q + 1 < a.r) ? ar[(int64_t)(q + 1) * Nw] : 0u;
          pb[jj] = x0 | (x1 << 16);
        }
#pragma unroll
        for (int i = 0; i < NRT; ++i) {
          const int rr = i * 32 + n32;
          const float* tr = a.t + (int64_t)(row0 + rr) * a.r;
          u32x4 pk;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int q = q0 + 8 * h + 2 * jj;
            const float x0 = (rr < nrows && q < a.r) ? tr[q] : 0.0f;
            const float x1 = (rr < nrows && q + 1 < a.r) ? tr[q + 1] : 0.0f;
            pk[jj] = pack_bf16x2(x0, x1);
          }
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pk),
                                                           __builtin_bit_cast(bf16x8, pb), acc[i],
                                                           0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < NRT; ++i)
#pragma unroll
        for (int z = 0; z < 16; ++z) acc[i][z] *= a.lscale;
    }
    if (nk >= 3) wait_vmcnt<3 * kGLoads>();
    else if (nk == 2) wait_vmcnt<2 * kGLoads>();
    else wait_vmcnt<kGLoads>();
    lds_barrier();   // the weights of k-tile 0 come from every wave's loads
    dequant_to_bt(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      // batch kt landed (for this wave); then everyone's, and every wave's Bt
      // writes of the previous step, behind the barrier
      if (kt + 2 < nk) wait_vmcnt<2 * kGLoads>();
      else if (kt + 1 < nk) wait_vmcnt<kGLoads>();
      else wait_vmcnt<0>();
      wait_lgkm0();
      lds_barrier();
      if (kt + kGStages - 1 < nk) issue(kt + kGStages - 1);
      const uint8_t* As = stage(kt % kGStages);
      const uint8_t* Bs = bt + (kt & 1) * kGBt;
#pragma unroll
      for (int s = 0; s < kGK / 16; ++s) {
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(Bs + col * kGBtPitch + 16 * (2 * s + h));
#pragma unroll
        for (int i = 0; i < NRT; ++i) {
          const int r = i * 32 + n32;
          const bf16x8 av =
              *reinterpret_cast<const bf16x8*>(As + r * 64 + 16 * ((2 * s + h) ^ ((r >> 2) & 3)));
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[i], 0, 0, 0);
        }
      }
      // next k-tile's weights into the other Bt buffer (after the last k-tile
      // the stage holds zeros or stale bytes: decoded and never read)
      dequant_to_bt((kt + 1) % kGStages, (kt + 1) & 1);
    }

    // ---- epilogue: lane holds column n of each 32 x 32 row tile, rows
    // 8 (z / 4) + 4 h + z % 4
    if (n >= Nw) return;
    int ng = 0, nu = 0;
    if (MODE == DGRAD_DOWN) {
      ng = gate_row(a.layout, a.I, n);
      nu = up_row(a.layout, a.I, n);
    }
#pragma unroll
    for (int i = 0; i < NRT; ++i) {
#pragma unroll
      for (int z = 0; z < 16; ++z) {
        const int rr = i * 32 + 8 * (z >> 2) + 4 * h + (z & 3);
        if (rr >= nrows) continue;
        const int row = row0 + rr;
        const float v = acc[i][z];
        if (MODE == DGRAD_DOWN) {
          // n indexes the intermediate dimension: dH[row][n]
          const float* sg = a.save_gu + (int64_t)row * 2 * a.I;
          float dg, du;
          act_backward(a.act, sg[ng], sg[nu], v, a.alpha, a.limit, dg, du);
          uint16_t* d = a.dgu + (int64_t)row * 2 * a.I;
          d[ng] = f32_to_bf16(dg);
          d[nu] = f32_to_bf16(du);
        } else {
          a.dx[(int64_t)row * Nw + n] = v;
        }
      }
    }
  };
  switch (nrt) {
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 5: kloop(std::integral_constant<int, 5>{}); break;
    case 6: kloop(std::integral_constant<int, 6>{}); break;
    case 7: kloop(std::integral_constant<int, 7>{}); break;
    default: kloop(std::integral_constant<int, kGM / 32>{}); break;
  }
}

template <int FMT>
hipError_t set_dgrad_lds() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dgrad<FMT, DGRAD_DOWN>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kGLds);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dgrad<FMT, DGRAD_GATEUP>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kGLds);
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
  const int ntiles = rows / kGM + touched;
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
  d.ncg = (I + kGN - 1) / kGN;
  le.before(0, s);
  if (ntiles * d.ncg > 0)
    // ntiles bounds the row tiles; 8 spare ids keep every XCD's share of the
    // items within the ids it is dealt
    hipLaunchKernelGGL((k_dgrad<FMT, DGRAD_DOWN>), dim3(ntiles * d.ncg + 8), dim3(512), kGLds, s,
                       d);
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
  g.ncg = (H + kGN - 1) / kGN;
  le.before(1, s);
  if (ntiles * g.ncg > 0)
    hipLaunchKernelGGL((k_dgrad<FMT, DGRAD_GATEUP>), dim3(ntiles * g.ncg + 8), dim3(512), kGLds,
                       s, g);
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
