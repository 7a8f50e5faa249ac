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
//    one expert over all of K, split across its waves, with the scales of its
//    rows staged once in LDS; each wave loads 16-byte pieces of nibbles into
//    registers, transposes them across lanes into MFMA order, dequantises them
//    (NF4 through an LDS table of fp32 level pairs, MXFP4 in the hardware
//    conversion) and runs 16x16x32 bf16 MFMA; waves are reduced through LDS.
//  * tiled (prefill-sized row counts): one workgroup of eight waves per work
//    item of up to 320 activation rows x 256 weight rows; activation tiles and
//    packed weights arrive in a three-stage LDS ring by direct loads, every
//    weight is dequantised once per workgroup, and each wave owns one 32-wide
//    column tile on 32x32x16 bf16 MFMA against every row of the item.
#include <type_traits>

#include "common.hpp"
#include "formats.hpp"
#include "internal.hpp"
#include "gemm_common.hpp"

namespace moe4 {
namespace {

// ------------------------------------------------------------ dequantisation

// bf16 operands of 8 weights (one dword of nibbles, even element in the low
// nibble). NF4: fp32 levels of each byte from the LDS table, the absmax
// applied in fp32 and the product rounded once to bf16. MXFP4: the hardware
// e2m1 -> bf16 conversion scaled by the block's power of two (exact; the scale
// operand is the e8m0 byte placed in an fp32 exponent field).
template <int FMT>
__device__ __forceinline__ u32x4 dequant8(uint32_t w, float sc, const float2* lutf) {
  u32x4 r;
  if constexpr (FMT != MOE4_FMT_MXFP4) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      // read through the vector type: the compiler then leaves these reads
      // free of a wait for every LDS-DMA load in flight (the loop's own
      // counted waits and barriers order them)
      const f32x2 v = reinterpret_cast<const f32x2*>(lutf)[(w >> (8 * bi)) & 255u];
      r[bi] = pack_bf16x2(v.x * sc, v.y * sc);
    }
  } else {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  }
  return r;
}

// dequant8 in two parts, so that the table reads can be issued well before
// the arithmetic: fetch8 reads the NF4 levels of the dword's four bytes,
// apply8 scales and rounds them (MXFP4: the hardware conversion of w).
template <int FMT>
__device__ __forceinline__ void fetch8(uint32_t w, const float2* lutf, f32x2 (&v)[4]) {
  if constexpr (FMT != MOE4_FMT_MXFP4) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
      v[bi] = reinterpret_cast<const f32x2*>(lutf)[(w >> (8 * bi)) & 255u];
  }
}
template <int FMT>
__device__ __forceinline__ u32x4 apply8(uint32_t w, const f32x2 (&v)[4], float sc) {
  if constexpr (FMT != MOE4_FMT_MXFP4) {
    u32x4 r;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) r[bi] = pack_bf16x2(v[bi].x * sc, v[bi].y * sc);
    return r;
  } else {
    return dequant8<FMT>(w, sc, nullptr);
  }
}

// scale operand of dequant8 from a raw scale word: NF4 fp32 absmax bits, or an
// e8m0 byte
template <int FMT>
__device__ __forceinline__ float scale_operand(uint32_t raw) {
  return FMT == MOE4_FMT_NF4 ? __uint_as_float(raw) : __uint_as_float((raw & 255u) << 23);
}

// ------------------------------------------------------------ skinny kernel

// 4x4 transpose of dwords across the four 16-lane rows of a wave: on entry
// row g holds D[g][0..3] in v[0..3]; on exit row g holds D[0..3][g]. The
// 32-lane swap trades the upper half of its first operand for the lower half
// of its second; the 16-lane swap trades the odd rows of its first operand for
// the even rows of its second.
__device__ __forceinline__ void transpose4x4_rows(u32x4& v) {
  const auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  v[0] = c[0];
  v[1] = c[1];
  v[2] = d[0];
  v[3] = d[1];
}

// Scale layout of the skinny kernel. The scales of the workgroup's weight
// rows are copied once into LDS by direct loads, a chunk of at most kKc k at a
// time (one chunk for every K up to kKc): row r of the chunk starts in dword
// r * pitch, shifted by the byte offset of the row's first scale within its
// dword. The pitch is odd in dwords, so the 16 rows of a column tile sit in 16
// different banks.
template <int FMT>
struct SkinnyScales {
  static constexpr int kBytes = FMT == MOE4_FMT_NF4 ? 4 : 1;   // per block
  static constexpr int kKb = Format<FMT>::kBlock;
  static constexpr int kKc = FMT == MOE4_FMT_NF4 ? 8192 : 16384;
  // dword pitch of one row for a chunk of kc k: the chunk's bytes, up to
  // three bytes of lead, rounded up, and made odd
  __host__ __device__ static constexpr int pitch(int kc) {
    return (((kc / kKb) * kBytes + 3 + 3) / 4) | 1;
  }
  // the stage of nrow rows, rounded up to whole 64-dword loads
  __host__ __device__ static constexpr int lds_bytes(int K, int nrow) {
    return (nrow * pitch(K < kKc ? K : kKc) * 4 + 255) / 256 * 256;
  }
};

// Column tiles of 16 weight rows per wave of the skinny kernel: every
// activation operand feeds kSkNc MFMAs (four measured slower than two: fewer,
// fatter workgroups and more registers).
constexpr int kSkNc = 2;
static_assert(kSkNc == 2 || kSkNc == 4, "8 kSkNc gate/up pairs must divide I (a multiple of 32)");

// Per-wave operands of one 128-k iteration of the skinny kernel: the nibbles
// of the column tiles and the activation operands of the four MFMA steps.
template <int NRT>
struct SkinnyBatch {
  u32x4 wraw[kSkNc];
  u32x4 av[NRT][4];
};

// Buffer resources and lane offsets of one wave of the skinny kernel.
struct SkinnyLane {
  rsrc_t rq, ra;        // this expert's nibbles; this row chunk's activations
  int qoff[kSkNc];      // byte offset of the lane's 16-byte column in weight row c, k = 0
  int aoff;             // byte offset of the lane's activation operand (its row, k = 8 g)
  int sb[kSkNc];        // LDS byte address of the first staged scale of weight row c
  int a2bnd[kSkNc];     // double-quantised NF4: the first block of weight row c that
                        // lies in the row's second absmax group
};

// Double-quantised NF4 in the skinny kernel: the workgroup's weight rows
// each span at most two groups of 256 absmax (rows of at most 256 blocks);
// a2tab[2 * (16 c + n) + h] holds the group scale of half h of row (c, n).
struct SkinnyDq {
  const float* book;   // LDS: the 256-entry code book
  const float* a2tab;  // LDS: [16 kSkNc rows][2]
  float off;           // the stack's absmax offset
};

// Each k-iteration covers 128 k. Lane (n = l%16, g = l/16) loads 16 bytes
// (32 k) of its weight row with one 128-bit load, so the four lanes of a row
// read 64 contiguous bytes; a 4x4 dword transpose across g then gives lane g,
// for MFMA step s, the 8 k at kb + 32s + 8g. The activation operand of step s
// is loaded in the same order (the four lanes of a row read 64 contiguous
// bytes), and every step lies inside one scale block (64 for NF4, 32 for
// MXFP4).
// FULL: the iteration lies inside K (kb + 128 <= K), so only `live` (an
// iteration of this wave) decides, once per operand set; the four activation
// loads then differ only in their immediate offsets. Otherwise every 32-k piece
// is checked against K.
template <int FMT, int NRT, bool FULL>
__device__ __forceinline__ void skinny_load(SkinnyBatch<NRT>& bt, const SkinnyLane& sl, int K,
                                            int kb, bool live) {
  const int l = lane_id(), nl = l & 15, g = l >> 4;
  const bool ink = live && (FULL || kb + 32 * g < K);
#pragma unroll
  for (int c = 0; c < kSkNc; ++c)
    bt.wraw[c] = buf_load_b128(sl.rq, ink ? sl.qoff[c] + kb / 2 : kOob);
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    if constexpr (FULL) {
      const int base = live ? sl.aoff + (rt * 16 * K + kb) * 2 : kOob;
#pragma unroll
      for (int st = 0; st < 4; ++st) bt.av[rt][st] = buf_load_b128(sl.ra, base + 64 * st);
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int k = kb + 32 * st + 8 * g;
        bt.av[rt][st] =
            buf_load_b128(sl.ra, (live && k < K) ? sl.aoff + (rt * 16 * K + kb + 32 * st) * 2 : kOob);
      }
    }
  }
}

// Multiply one batch: iteration `it` of the chunk (its first block is
// it * 128 / block of the staged row, nblk blocks staged). Blocks past the
// staged ones (an iteration beyond K, whose activations are zero) take the
// last staged scale, so every operand stays finite. Each weight becomes the
// bf16 operand of dequant8 (NF4: bf16(fp32(level * absmax)); MXFP4: the exact
// hardware conversion with the block's power of two).
template <int FMT, int NRT>
__device__ __forceinline__ void skinny_compute(const SkinnyBatch<NRT>& bt, const float2* lutf,
                                               const uint8_t* stage, const SkinnyLane& sl,
                                               const SkinnyDq& dq, int it, int nblk, int gblk0,
                                               f32x4 (&acc)[2][kSkNc]) {
  constexpr int KB = Format<FMT>::kBlock;
  constexpr int NSC = 128 / KB;   // scale blocks per iteration: 2 (NF4) or 4 (MXFP4)
#pragma unroll
  for (int c = 0; c < kSkNc; ++c) {
    float sc[NSC];
#pragma unroll
    for (int j = 0; j < NSC; ++j) {
      const int b = min(it * NSC + j, nblk - 1);
      if constexpr (FMT == MOE4_FMT_NF4) {
        sc[j] = *reinterpret_cast<const float*>(stage + sl.sb[c] + 4 * b);
      } else if constexpr (FMT == MOE4_FMT_MXFP4) {
        sc[j] = scale_operand<FMT>(stage[sl.sb[c] + b]);
      } else {
        // absmax = fp32(fp32(book[code] * absmax2) + offset); absmax2 is the
        // row's first or second group scale
        const float a2 =
            dq.a2tab[2 * (16 * c + (lane_id() & 15)) + (gblk0 + b < sl.a2bnd[c] ? 0 : 1)];
        sc[j] = mul_then_add(dq.book[stage[sl.sb[c] + b]], a2, dq.off);
      }
    }
    u32x4 wq = bt.wraw[c];
    transpose4x4_rows(wq);
    u32x4 bq[4];
    if constexpr (FMT == MOE4_FMT_NF4_DQ) {
      // every table read of the column tile first, then the arithmetic (17%
      // faster here; the plain NF4 loop measured no different)
      f32x2 lv[4][4];
#pragma unroll
      for (int st = 0; st < 4; ++st) fetch8<FMT>(wq[st], lutf, lv[st]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < 4; ++st) bq[st] = apply8<FMT>(wq[st], lv[st], sc[st * NSC / 4]);
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st) bq[st] = dequant8<FMT>(wq[st], sc[st * NSC / 4], lutf);
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int st = 0; st < 4; ++st)
        acc[rt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, bt.av[rt][st]), __builtin_bit_cast(bf16x8, bq[st]),
            acc[rt][c], 0, 0, 0);
  }
}

// K loop of one wave over the iterations [it0, it1) of a chunk starting at k0,
// for NRT 16-row tiles, with two batches in a register ring: while one batch
// is dequantised and multiplied, the loads of the next are in flight.
// Loads are never skipped: an iteration past it1 reads out of bounds (zero
// activations, no memory traffic), which keeps the count of loads in flight
// the same on every path, so the compiler waits for exactly the batch it
// needs. The prologue (the first NB - 1 batches) is a separate call so that
// the first row chunk can issue it before the workgroup's set-up barrier.
// Batches in the register ring (three or four measured slower: spills at three
// waves per SIMD, or fewer waves).
constexpr int kSkNb = 2;

// Iterations [it0, itf) of the wave lie inside K; iteration itf < it1, if the
// wave has it, is the chunk's partial last one.
template <int FMT, int NRT>
__device__ __forceinline__ void skinny_prologue(SkinnyBatch<NRT> (&b)[kSkNb],
                                                const SkinnyLane& sl, int K, int k0, int it0,
                                                int itf, int it1) {
  static_assert(kSkNb == 2, "one batch of prologue");
  if (it0 < itf) skinny_load<FMT, NRT, true>(b[0], sl, K, k0 + 128 * it0, true);
  else skinny_load<FMT, NRT, false>(b[0], sl, K, k0 + 128 * it0, it0 < it1);
}

template <int FMT, int NRT>
__device__ __forceinline__ void skinny_body(SkinnyBatch<NRT> (&b)[kSkNb], const SkinnyLane& sl,
                                            int K, int k0, int it0, int itf, int it1, int nblk,
                                            const float2* lutf, const uint8_t* stage,
                                            const SkinnyDq& dq, f32x4 (&acc)[2][kSkNc]) {
  constexpr int KB = Format<FMT>::kBlock;
  const int gblk0 = k0 / KB;
  for (int it = it0; it < itf; it += 2) {
    skinny_load<FMT, NRT, true>(b[1], sl, K, k0 + 128 * (it + 1), it + 1 < itf);
    __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the arithmetic
    skinny_compute<FMT>(b[0], lutf, stage, sl, dq, it, nblk, gblk0, acc);
    __builtin_amdgcn_sched_barrier(0);
    skinny_load<FMT, NRT, true>(b[0], sl, K, k0 + 128 * (it + 2), it + 2 < itf);
    __builtin_amdgcn_sched_barrier(0);
    skinny_compute<FMT>(b[1], lutf, stage, sl, dq, it + 1, nblk, gblk0, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (itf < it1) {
    // the partial last iteration (the prologue loaded it if it is the wave's only one)
    if (it0 < itf) skinny_load<FMT, NRT, false>(b[0], sl, K, k0 + 128 * itf, true);
    skinny_compute<FMT>(b[0], lutf, stage, sl, dq, itf, nblk, gblk0, acc);
  }
}

// Skinny grouped GEMM: one workgroup = 16 MAXR rows of one expert x 16 kSkNc
// weight rows (gate_up: 8 kSkNc (gate, up) pairs, the first half of the column
// tiles gate rows and the second half the matching up rows; down: 16 kSkNc
// output columns); its S waves split K and are reduced through LDS. An expert
// with more rows than one chunk gets one workgroup per chunk, so a hot expert
// of a skewed batch spreads over as many workgroups (which read its weights
// concurrently, the repeats mostly from the caches) instead of one workgroup
// streaming them once per chunk.
//
// Set-up is arranged so that its memory latencies overlap: the expert and its
// row range come from one pass over the offsets; then the scales of the
// workgroup's weight rows (direct loads into LDS), the NF4 level table and the first
// batch of weights and activations are all issued before a single wait and
// the workgroup barrier.
//
// Three waves per SIMD (four measured the same), and chunks of 16 rows (one
// 16-row MFMA tile: decode-sized experts rarely have more rows, and a second
// accumulator tile would cost the third wave).
constexpr int kSkWavesPerEu = 3;
constexpr int kSkMaxRowTiles = 1;
// GATHER (gate_up only): the activation rows are gathered from a.A through
// a.arows (see GemmArgs) instead of read as consecutive rows.
template <int FMT, bool GATEUP, bool GATHER = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(kSkWavesPerEu)))
void k_skinny(const GemmArgs a) {
  using F = Format<FMT>;
  using SS = SkinnyScales<FMT>;
  constexpr bool NF4 = FMT != MOE4_FMT_MXFP4;
  constexpr bool DQ = FMT == MOE4_FMT_NF4_DQ;
  constexpr int MAXR = kSkMaxRowTiles;
  constexpr int KB = F::kBlock;
  // NF4 byte -> two fp32 levels; the absmax code book of a double-quantised stack
  __shared__ __attribute__((aligned(16))) float2 lutf[NF4 ? 256 : 1];
  __shared__ __attribute__((aligned(16))) float dqbook[DQ ? 256 : 1];
  __shared__ __attribute__((aligned(16))) float a2tab[DQ ? 32 * kSkNc : 1];
  constexpr int NROW = 16 * kSkNc;   // weight rows of the workgroup
  // [NROW rows][pitch] staged scales (rounded up to 256 bytes), then
  // [S][MAXR][kSkNc][256] partial sums
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  const int K = a.K;
  const int pdw = SS::pitch(min(K, SS::kKc));
  uint8_t* stage = dyn;
  float* red = reinterpret_cast<float*>(dyn + SS::lds_bytes(K, NROW));
  const int S = blockDim.x >> 6, w = wave_id(), l = lane_id();
  const int item = blockIdx.x / a.ncg, cg = blockIdx.x - item * a.ncg;
  int e, u, rbeg, rend;
  auto chunks = [](int n) { return (n + 16 * MAXR - 1) / (16 * MAXR); };
  if (a.E <= 128) locate_item_batched<2>(a.offsets, a.E, item, chunks, e, u, rbeg, rend);
  else locate_item(a.offsets, a.E, item, chunks, e, u, rbeg, rend);
  e = __builtin_amdgcn_readfirstlane(e);
  if (e < 0) return;   // the whole workgroup: e is uniform
  rbeg = __builtin_amdgcn_readfirstlane(min(rbeg, a.rows));
  const int n_e = __builtin_amdgcn_readfirstlane(min(rend, a.rows)) - rbeg;
  const int rc0 = __builtin_amdgcn_readfirstlane(16 * MAXR * u);   // this workgroup's chunk
  if (rc0 >= n_e) return;   // rows past `rows` (uniform)
  const int Nw = GATEUP ? 2 * a.I : a.N_out;
  // weight row (inside the expert) of the workgroup's row r = 16 c + n
  auto wrow = [&](int r) {
    constexpr int H2 = kSkNc / 2;
    const int c = r >> 4, n = r & 15;
    return GATEUP ? (c < H2 ? gate_row(a.layout, a.I, cg * 8 * kSkNc + 16 * c + n)
                            : up_row(a.layout, a.I, cg * 8 * kSkNc + 16 * (c - H2) + n))
                  : cg * NROW + r;
  };
  const int rowbytes = (K / KB) * SS::kBytes;
  const rsrc_t rs = make_rsrc(static_cast<const uint8_t*>(a.ws) + (int64_t)e * Nw * rowbytes,
                              (uint32_t)Nw * rowbytes);
  // direct loads of the scales of chunk [k0, k0 + kc) of the rows: dword j
  // of the stage is dword j % pdw of row j / pdw's covering span; the waves
  // take the 64-dword pieces in turn (a piece may cross rows)
  const float inv_pdw = 1.0f / (float)pdw;
  auto stage_issue = [&](int k0) {
    const int c0 = (k0 / KB) * SS::kBytes;
    const int npiece = (NROW * pdw + 63) / 64;
    for (int q = w; q < npiece; q += S) {
      const int j = 64 * q + l;
      // j / pdw for j < 2^16: the rounded quotient of the float product is exact
      const int r = (int)(((float)j + 0.5f) * inv_pdw), d = j - r * pdw;
      const int off = r < NROW ? ((wrow(r) * rowbytes + c0) & ~3) + 4 * d : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MOE4_LDS(stage + 256 * q), 4, off, 0, 0, 0);
    }
  };
  // the NF4 level pairs (2 KiB), by direct loads into LDS as well
  auto lut_issue = [&]() {
    if constexpr (NF4) {
      const rsrc_t rl = make_rsrc(kNf4Pairs.v, sizeof(kNf4Pairs.v));
      for (int q = w; q < 8; q += S)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rl, MOE4_LDS(reinterpret_cast<uint8_t*>(lutf) + 256 * q), 4, 256 * q + 4 * l, 0, 0,
            0);
    }
  };
  // double-quantised NF4: the code book (1 KiB) and the group scales of the
  // workgroup's weight rows, a2tab[2 t + h] = group h of row t = 16 c + n (zero
  // past the last group), by direct loads into LDS as well
  auto dq_issue = [&]() {
    if constexpr (DQ) {
      const rsrc_t rb = make_rsrc(a.dqbook, 256 * sizeof(float));
      for (int q = w; q < 4; q += S)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, MOE4_LDS(reinterpret_cast<uint8_t*>(dqbook) + 256 * q), 4, 256 * q + 4 * l, 0, 0,
            0);
      static_assert((2 * NROW) % 64 == 0, "whole 64-lane loads cover a2tab");
      const int64_t ng = ((int64_t)a.E * Nw * (K / KB) + 255) / 256;
      const rsrc_t r2 = make_rsrc(a.ws2, (uint32_t)(ng * 4));
      for (int q = S - 1 - w; q < 2 * NROW / 64; q += S) {
        const int j = 64 * q + l;   // a2tab entry: group j % 2 of row j / 2
        const int64_t g = ((((int64_t)e * Nw + wrow(j >> 1)) * (K / KB)) >> 8) + (j & 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r2, MOE4_LDS(reinterpret_cast<uint8_t*>(a2tab) + 256 * q),
                                                 4, g < ng ? (int)g * 4 : kOob, 0, 0, 0);
      }
    }
  };
  SkinnyDq dq{dqbook, a2tab, DQ ? a.dqoff[0] : 0.0f};
  const int nl = l & 15, g = l >> 4;
  SkinnyLane sl;
  int srow[kSkNc];
#pragma unroll
  for (int c = 0; c < kSkNc; ++c) srow[c] = wrow(16 * c + nl);
  sl.rq = make_rsrc(a.wq + (int64_t)e * Nw * (K / 2), (uint32_t)Nw * (K / 2));
  if (DQ) {
#pragma unroll
    for (int c = 0; c < kSkNc; ++c)
      sl.a2bnd[c] = 256 - (int)((((int64_t)e * Nw + srow[c]) * (K / KB)) & 255);
  }
#pragma unroll
  for (int c = 0; c < kSkNc; ++c) sl.qoff[c] = srow[c] * (K / 2) + 16 * g;
  const int nchunk = (K + SS::kKc - 1) / SS::kKc;
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  // rows [rc, rc + 16 MAXR) of the expert; FIRST: the first chunk of rows,
  // whose first chunk of K finishes the set-up
  auto run_rows = [&](auto nrt_c, auto first_c, int rc) {
    constexpr int NRT = decltype(nrt_c)::value;
    constexpr bool FIRST = decltype(first_c)::value;
    const int nrows = min(16 * MAXR, n_e - rc);
    f32x4 acc[2][kSkNc];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int c = 0; c < kSkNc; ++c) acc[rt][c] = zero4;
    if constexpr (GATHER) {
      // the lane's row: row arows[.] / gk of A; rows past the chunk read past
      // the resource (A has fewer than 2^29 / K rows, checked by the caller)
      sl.ra = make_rsrc(a.A, (uint32_t)a.a_rows * K * 2);
      sl.aoff = nl < nrows ? ((a.arows[rbeg + rc + nl] / a.gk) * K + 8 * g) * 2 : (1 << 30);
    } else {
      sl.ra = make_rsrc(a.A + (int64_t)(rbeg + rc) * K, (uint32_t)max(nrows, 0) * K * 2);
      sl.aoff = (nl * K + 8 * g) * 2;
    }
    SkinnyBatch<NRT> b[kSkNb];
    // chunk ch of K: its scales in the stage, then the wave's iterations
    auto chunk = [&](int ch, bool setup) {
      const int k0 = ch * SS::kKc, kc = min(SS::kKc, K - k0);
      const int c0 = (k0 / KB) * SS::kBytes;
#pragma unroll
      for (int c = 0; c < kSkNc; ++c)
        sl.sb[c] = (16 * c + nl) * pdw * 4 + ((srow[c] * rowbytes + c0) & 3);
      const int nit = (kc + 127) / 128;
      const int it0 = (int)((int64_t)w * nit / S), it1 = (int)((int64_t)(w + 1) * nit / S);
      const int itf = min(it1, kc / 128);   // end of the wave's whole iterations
      skinny_prologue<FMT>(b, sl, K, k0, it0, itf, it1);
      if (setup) {
        // the scales and level pairs travel together with the first batch
        __builtin_amdgcn_sched_barrier(0);
        stage_issue(0);
        lut_issue();
        dq_issue();
        wait_vmcnt<0>();
        lds_barrier();
      }
      skinny_body<FMT>(b, sl, K, k0, it0, itf, it1, kc / KB, lutf, stage, dq, acc);
    };
    auto restage = [&](int ch) {
      __syncthreads();   // every wave is done with the staged scales
      stage_issue(ch * SS::kKc);
      wait_vmcnt<0>();
      __syncthreads();
    };
    // the first chunk of the first row chunk is straight-line code after the
    // set-up (no merge with a loop's back edge before its prologue)
    if (FIRST) {
      chunk(0, true);
    } else {
      if (nchunk > 1) restage(0);
      chunk(0, false);
    }
    for (int ch = 1; ch < nchunk; ++ch) {
      restage(ch);
      chunk(ch, false);
    }
    // reduce the S partial sums through LDS: red[w][rt][c][lane*4 + i]
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int c = 0; c < kSkNc; ++c)
        *reinterpret_cast<f32x4*>(red + (((size_t)w * MAXR + rt) * kSkNc + c) * 256 + l * 4) =
            acc[rt][c];
    __syncthreads();
    if (GATEUP) {
      // pair jj of the workgroup: gate in column tile jj / 16, up in tile
      // jj / 16 + kSkNc / 2
      for (int el = threadIdx.x; el < nrows * 8 * kSkNc; el += blockDim.x) {
        const int m = el / (8 * kSkNc), jj = el - m * 8 * kSkNc;
        const int rt = m >> 4, mr = m & 15, ct = jj >> 4, n = jj & 15;
        const int off = (16 * (mr >> 2) + n) * 4 + (mr & 3);
        float gs = 0.0f, us = 0.0f;
        for (int ww = 0; ww < S; ++ww) {
          const float* p = red + ((size_t)ww * MAXR + rt) * kSkNc * 256;
          gs += p[ct * 256 + off];
          us += p[(ct + kSkNc / 2) * 256 + off];
        }
        gate_up_epilogue(a, e, rbeg + rc + m, cg * 8 * kSkNc + jj, gs, us);
      }
    } else {
      for (int el = threadIdx.x; el < nrows * NROW; el += blockDim.x) {
        const int m = el / NROW, cc = el - m * NROW;
        const int rt = m >> 4, mr = m & 15, ct = cc >> 4, n = cc & 15;
        const int off = (16 * (mr >> 2) + n) * 4 + (mr & 3);
        float ys = 0.0f;
        for (int ww = 0; ww < S; ++ww)
          ys += red[(((size_t)ww * MAXR + rt) * kSkNc + ct) * 256 + off];
        if (cg * NROW + cc < a.N_out) down_epilogue(a, e, rbeg + rc + m, cg * NROW + cc, ys);
      }
    }
    __syncthreads();
  };
  using One = std::integral_constant<int, 1>;
  using Max = std::integral_constant<int, MAXR>;
  using Yes = std::true_type;
  if (MAXR == 1 || n_e - rc0 <= 16) run_rows(One{}, Yes{}, rc0);
  else run_rows(Max{}, Yes{}, rc0);
}

// ------------------------------------------------------------- tiled kernel

// One workgroup per CU: eight waves, an expert tile of up to kBM rows and 256
// weight rows (gate_up: 128 (gate, up) pairs; down: 256 output columns).
// Wave w owns 32 of the weight rows -- one 32-wide MFMA column tile -- against
// every row of the tile, so each weight is dequantised once per workgroup. An
// expert whose rows fit in kBM takes one tile; larger experts are cut into
// equal tiles (multiples of 32 rows).
constexpr int kBM = 320, kBN = 256, kBK = 64, kStages = 3, kTiledWaves = 8;
constexpr int kMaxRowTiles = kBM / 32;
// One LDS stage holds a k-tile of 64: the A tile [kBM rows][128 B] with the
// 16-byte chunks of row r stored at chunk ^ ((r >> 1) & 7), each wave's packed
// nibbles [32 rows][32 B], and each wave's
// scales in 4-byte slots (NF4: slot n = row n's fp32 absmax; double-quantised
// NF4: slot n = row n's absmax code byte; MXFP4: slot
// 32 h + n = the e8m0 byte of half h of row n; sub-dword loads to LDS advance
// 4 bytes a lane).
// The LDS has 64 four-byte banks: a 16-byte operand read serves 16 lanes
// (rows r .. r+15 of one chunk column) per pass, and rows r and r + 1 share a
// 256-byte bank line, so the swizzle keys on r / 2 to give those 16 rows 16
// different 16-byte bank groups.
constexpr int kStageA = kBM * kBK * 2;
constexpr int kStageB = kTiledWaves * 32 * 32;
constexpr int kStageS = kTiledWaves * 64 * 4;
constexpr int kStageBytes = kStageA + kStageB + kStageS;
constexpr int kTiledLds = kStages * kStageBytes;
static_assert(kTiledLds + 256 * 8 <= 160 * 1024, "tiled kernel LDS");

// An empty asm that takes v in registers at this point: whatever computes v
// stays before it.
__device__ __forceinline__ void pin_regs(const u32x4& v) { asm volatile("" ::"v"(v)); }

// Element column (within the k-tile) of lane l's 16-byte A load in wave w: the
// chunk l % 8 of row 8 w + l / 8, swizzled by (row >> 1) & 7.
__device__ __forceinline__ int a_col_of(int l, int w) {
  return 8 * ((l & 7) ^ (((8 * w + (l >> 3)) >> 1) & 7));
}
// The lane index, recomputed where it is used: the empty asm hides it from the
// compiler, which then cannot keep values derived from it live across the
// k-loop (the loop's registers are full; such values were spilled and every
// reload waited for all loads in flight).
__device__ __forceinline__ int opaque_lane() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t & (kWave - 1);
}

template <int FMT, bool GATEUP, bool GATHER>
__global__ __launch_bounds__(512, 1) void k_tiled(const GemmArgs a) {
  using F = Format<FMT>;
  constexpr bool NF4 = FMT != MOE4_FMT_MXFP4;   // NF4 levels (plain or double-quantised)
  constexpr bool DQ = FMT == MOE4_FMT_NF4_DQ;
  constexpr int KB = F::kBlock;
  constexpr int kLoadsPerTile = kBM / 64 + 1 + 1;
  // NF4 stacks have K (H or I) a multiple of their 64-element block, so every
  // 64-wide k-tile is whole; MXFP4 (32-element blocks) may end in a half tile
  constexpr bool kWholeTiles = NF4 && F::kBlock % kBK == 0;
  __shared__ __attribute__((aligned(16))) float2 lutf[NF4 ? 256 : 1];
  // double-quantised NF4: the absmax code book
  __shared__ float dqbook[DQ ? 256 : 1];
  extern __shared__ __attribute__((aligned(16))) uint8_t stage_mem[];
  // w in a scalar register: every LDS destination derived from it is scalar
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id();
  // the table values are loaded first and stored after the locator, so that
  // their loads and the locator's are in flight together
  float2 lv0 = make_float2(0.0f, 0.0f);
  float dq0 = 0.0f;
  if (NF4 && tid < 256) lv0 = make_float2(F::level(tid & 15), F::level(tid >> 4));
  if (DQ && tid < 256) dq0 = a.dqbook[tid];
  int e, ut, cg, obeg, oend;
  locate_tile_sorted<kBM>(a.offsets, a.E, a.ncg, blockIdx.x, e, ut, cg, obeg, oend);
  if (NF4 && tid < 256) lutf[tid] = lv0;
  if (DQ && tid < 256) dqbook[tid] = dq0;
  // wave-uniform by construction; make it visible to the compiler so that the
  // buffer resources below live in scalar registers
  e = __builtin_amdgcn_readfirstlane(e);
  ut = __builtin_amdgcn_readfirstlane(ut);
  cg = __builtin_amdgcn_readfirstlane(cg);
  obeg = __builtin_amdgcn_readfirstlane(obeg);
  oend = __builtin_amdgcn_readfirstlane(oend);
  __syncthreads();
  if (e < 0) return;
  const int K = a.K;
  const int ebeg = min(obeg, a.rows);
  const int n_e = min(oend, a.rows) - ebeg;
  const int R = eq_tile_rows<kBM>(n_e);
  const int row0 = ebeg + ut * R;
  const int nrows = min(R, ebeg + n_e - row0);
  const int nrt = (nrows + 31) >> 5;
  const int n32 = l & 31, h = l >> 5;
  const int Nw = GATEUP ? 2 * a.I : a.N_out;

  // weight row of MFMA column n of this wave (gate_up: columns 0..15 are the
  // gate rows of pairs j0 .. j0+15, columns 16..31 their up rows)
  const int j0 = cg * 128 + w * 16;
  auto wrow_of = [&](int n, bool& on) {
    if (GATEUP) {
      const int j = j0 + (n & 15);
      on = j < a.I;
      const int jj = on ? j : 0;
      return n < 16 ? gate_row(a.layout, a.I, jj) : up_row(a.layout, a.I, jj);
    }
    const int c = cg * kBN + w * 32 + n;
    on = c < a.N_out;
    return on ? c : 0;
  };

  // (the conditional operator does not take buffer-resource operands)
  rsrc_t ra;
  if constexpr (GATHER) ra = make_rsrc(a.A, (uint32_t)a.a_rows * K * 2);
  else ra = make_rsrc(a.A + (int64_t)row0 * K, (uint32_t)nrows * K * 2);
  const rsrc_t rq = make_rsrc(a.wq + (int64_t)e * Nw * (K / 2), (uint32_t)Nw * (K / 2));
  constexpr int sbytes = FMT == MOE4_FMT_NF4 ? 4 : 1;
  const rsrc_t rs = make_rsrc(static_cast<const uint8_t*>(a.ws) + (int64_t)e * Nw * (K / KB) * sbytes,
                              (uint32_t)Nw * (K / KB) * sbytes);

  // ---- loader roles (lane-contiguous LDS destinations)
  // A: load p of lane (w, l) fills LDS bytes p*8192 + w*1024 + 16*l of the A
  //    tile = row 64p + 8w + l/8, physical chunk l%8 = logical chunk ^ ((row >> 1) & 7)
  //    ((row >> 1) & 7 does not depend on p: load p is load 0 moved down 64
  //    rows, an offset passed in a scalar register)
  const int a_col = a_col_of(l, w);
  const int a_off = ((8 * w + (l >> 3)) * K + a_col) * 2;
  // gathered activations: the byte offset of load p's row (row 64 p + 8 w + l / 8
  // of the tile = row arows[.] / gk of A), or -1 past the tile's rows
  // (a fixed size: an array of template-dependent size captured by the loader
  // lambdas made the host-side instantiation fail silently)
  int a_offg[kBM / 64];
  if constexpr (GATHER) {
#pragma unroll
    for (int p = 0; p < kBM / 64; ++p) {
      const int r = 64 * p + 8 * w + (l >> 3);
      a_offg[p] = r < nrows ? ((a.arows[row0 + r] / a.gk) * K + a_col) * 2 : -1;
    }
  }
  // B: lane l fills [l/2][16 (l%2)] of this wave's nibble block (row n = l/2,
  //    bytes 16 (l%2) of the k-tile's 32)
  bool b_on;
  const int b_off = wrow_of(l >> 1, b_on) * (K / 2) + 16 * (l & 1);
  // scales: NF4 lane l < 32 covers row l; MXFP4 lane l covers half l/32 of row l%32
  bool s_on;
  const int s_row = wrow_of(n32, s_on);
  const int s_off = s_row * (K / KB) * sbytes;
  // double-quantised NF4: absmax = fp32(fp32(book[code] * absmax2) + offset),
  // absmax2 one per 256 absmax of the stack; a row of at most 256 blocks lies
  // in at most two such groups, the second from k-tile a2bnd on (k-tiles are
  // blocks)
  float a2lo = 0.0f, a2hi = 0.0f, dqoff = 0.0f;
  int a2bnd = 0;
  if constexpr (DQ) {
    const int64_t nb = K / KB;
    const int64_t f0 = ((int64_t)e * Nw + s_row) * nb;
    const int64_t ng = ((int64_t)a.E * Nw * nb + 255) / 256;
    const int64_t g0 = f0 >> 8;
    a2bnd = 256 - (int)(f0 & 255);
    a2lo = g0 < ng ? a.ws2[g0] : 0.0f;
    a2hi = g0 + 1 < ng ? a.ws2[g0 + 1] : 0.0f;
    dqoff = a.dqoff[0];
  }

  auto stage = [&](int st) { return stage_mem + st * kStageBytes; };
  // Batch j holds the A tile of k-tile j and the wave's weights of k-tile
  // j + 1, the A tile in stage j % 3 and the weights in stage (j + 1) % 3, so
  // that a k-tile's weights are in LDS one k-tile before its A tile and can be
  // dequantised between the MFMAs of the k-tile before.
  auto issue_b = [&](int kt, int st) {
    uint8_t* base = stage(st);
    const int kb = kt * kBK;
    // a whole k-tile (wave-uniform; every NF4 k-tile, as K is a multiple of
    // the 64-element block) needs no per-lane k check
    const bool kin = kWholeTiles || kb + kBK <= K || kb + 32 * (opaque_lane() & 1) < K;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rq, MOE4_LDS(base + kStageA + w * 1024), 16, (b_on && kin) ? b_off + kb / 2 : kOob, 0, 0,
        0);
    uint8_t* sbase = base + kStageA + kStageB + w * 256;
    if (FMT == MOE4_FMT_NF4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, MOE4_LDS(sbase), 4, (s_on && h == 0 && kb < K) ? s_off + (kb / 64) * 4 : kOob, 0,
          0, 0);
    } else if (DQ) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, MOE4_LDS(sbase), 1, (s_on && h == 0 && kb < K) ? s_off + kb / 64 : kOob, 0, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, MOE4_LDS(sbase), 1, (s_on && kb + 32 * h < K) ? s_off + kb / 32 + h : kOob, 0, 0,
          0);
    }
  };
  // part j of batch kt: A load j (j < kBM / 64), else the weights
  constexpr int kParts = kBM / 64 + 1;
  auto issue_part = [&](int kt, int j) {
    if (j < kBM / 64) {
      const int kb = kt * kBK;
      const bool kin = kWholeTiles || kb + kBK <= K || kb + a_col_of(opaque_lane(), w) < K;
      if constexpr (GATHER) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, MOE4_LDS(stage(kt % kStages) + j * 8192 + w * 1024), 16,
            (kin && a_offg[j] >= 0) ? a_offg[j] + 2 * kb : kOob, 0, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, MOE4_LDS(stage(kt % kStages) + j * 8192 + w * 1024), 16,
            kin ? a_off + 2 * kb : kOob, j * 64 * K * 2, 0, 0);
      }
    } else {
      issue_b(kt + 1, (kt + 1) % kStages);
    }
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int j = 0; j < kParts; ++j) issue_part(kt, j);
  };
  // this lane's raw nibbles (k 32h .. 32h+31 of row n32) and scale of the
  // weights of k-tile kt in stage st (LDS reads through vector types: see
  // dequant8)
  auto read_b = [&](int st, int kt, u32x4& braw, float& sc) {
    const uint8_t* base = stage(st);
    braw = *reinterpret_cast<const u32x4*>(base + kStageA + w * 1024 + n32 * 32 + 16 * h);
    const f32x2* Sw = reinterpret_cast<const f32x2*>(base + kStageA + kStageB + w * 256);
    const int slot = NF4 ? n32 : h * 32 + n32;
    const f32x2 pr = Sw[slot >> 1];
    const float raw = (slot & 1) ? pr.y : pr.x;
    if constexpr (FMT == MOE4_FMT_NF4) {
      sc = raw;
    } else if constexpr (DQ) {
      // a one-byte load fills the low byte of its 4-byte slot
      sc = mul_then_add(dqbook[__float_as_uint(raw) & 255u], kt < a2bnd ? a2lo : a2hi, dqoff);
    } else {
      sc = __uint_as_float((__float_as_uint(raw) & 255u) << 23);
    }
  };

  const int nk = (K + kBK - 1) / kBK;
  bool col_on;
  const int col_row = wrow_of(n32, col_on);
  // the bias of the lane's column is where its accumulators start (after the
  // scaled LoRA sum, when there is one), so the epilogue adds no bias
  const float binit = (a.bias && col_on) ? bf16_to_f32(a.bias[(int64_t)e * Nw + col_row]) : 0.0f;
  auto kloop = [&](auto nrt_c) {
    constexpr int NRT = decltype(nrt_c)::value;
    f32x16 acc[NRT];
    const float a0 = (GATEUP && a.r) ? 0.0f : binit;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rt][i] = a0;
    // A operand f = NRT s + rt of a k-tile: chunk 4h + s of row 32 rt + n32
    // (ten row tiles: a shorter ring keeps the loop within 256 VGPRs)
    constexpr int kN = 4 * NRT, kPre = NRT >= 10 ? 2 : 4;
    auto rd = [&](const uint16_t* As, int f) {
      const int s = f / NRT, rt = f % NRT, row = rt * 32 + n32;
      return *reinterpret_cast<const bf16x8*>(As + row * kBK + (((4 * h + s) ^ ((row >> 1) & 7)) * 8));
    };
    // Piece p of a k-tile's weights = the bf16 operands of step p (dword p of
    // the lane's nibbles). Its table reads (NF4) are issued one block of NRT
    // MFMAs before its arithmetic, which overwrites bq[p] once the MFMAs of
    // step p of the previous k-tile are issued: in block s of k-tile kt the
    // wave finishes piece s - 1 of k-tile kt + 1 (s = 0: piece 3 of kt) and
    // starts the table reads of piece s of kt + 1.
    u32x4 bq[4];
    u32x4 braw, braw_n;
    float sc, sc_n;
    f32x2 lv[4];
    issue_b(0, 0);
    issue(0);
    if (nk > 1) issue(1);
    // LoRA delta while the first batches land: MFMA steps over the rank (the
    // rank index q is their k), operand A = bf16(xa[row][q]), operand B =
    // B[e][n][q] (bf16 already; zero past r and for idle columns). They start
    // from zero accumulators, which then hold the fp32 sum scaled once by
    // lora_scale, as gu = x W^T + lora_scale * (bf16(xa) B^T) defines it; the
    // k-tiles accumulate on top.
    if constexpr (GATEUP) {
      if (a.r) {
        bool on;
        const int wr = wrow_of(n32, on);
        const uint16_t* brow = a.loraB + ((int64_t)e * 2 * a.I + wr) * a.r;
        for (int q0 = 0; q0 < a.r; q0 += 16) {
          u32x4 bl;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int q = q0 + 8 * h + 2 * jj;
            const uint32_t v0 = (on && q < a.r) ? brow[q] : 0u;
            const uint32_t v1 = (on && q + 1 < a.r) ? brow[q + 1] : 0u;
            bl[jj] = v0 | (v1 << 16);
          }
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            const int row = rt * 32 + n32;
            const float* xr = a.xa + (int64_t)(row0 + row) * a.r;
            u32x4 al;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int q = q0 + 8 * h + 2 * jj;
              const float v0 = (row < nrows && q < a.r) ? xr[q] : 0.0f;
              const float v1 = (row < nrows && q + 1 < a.r) ? xr[q + 1] : 0.0f;
              al[jj] = pack_bf16x2(v0, v1);
            }
            acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, al), __builtin_bit_cast(bf16x8, bl), acc[rt], 0, 0, 0);
          }
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[rt][i] = acc[rt][i] * a.lscale + binit;
      }
    }
    if (nk > 1) wait_vmcnt<2 * kLoadsPerTile>();
    else wait_vmcnt<kLoadsPerTile>();
    read_b(0, 0, braw, sc);   // the wave's own loads: no barrier needed
#pragma unroll
    for (int p = 0; p < 3; ++p) bq[p] = dequant8<FMT>(braw[p], sc, lutf);
    fetch8<FMT>(braw[3], lutf, lv);
    uint32_t wpend = braw[3];   // nibbles of the piece whose table reads are in lv
    float scpend = sc;
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) wait_vmcnt<kLoadsPerTile>();
      else wait_vmcnt<0>();
      // batch kt is in LDS everywhere (its weights are k-tile kt + 1's);
      // stage (kt + 2) % 3's A area and stage kt % 3's B area are free
      lds_barrier();
      // batch kt + 2 is issued part by part between the MFMAs below
      const bool more = kt + 2 < nk;
      const uint16_t* As = reinterpret_cast<const uint16_t*>(stage(kt % kStages));
      // after the last k-tile the B area holds zeros or stale nibbles:
      // decoded and never used
      read_b((kt + 1) % kStages, kt + 1, braw_n, sc_n);
      bf16x8 ring[kPre];
#pragma unroll
      for (int f = 0; f < kPre; ++f)
        if (f < kN) ring[f] = rd(As, f);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < kN; ++f) {
        const int s = f / NRT, rt = f % NRT;
        acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            ring[f % kPre], __builtin_bit_cast(bf16x8, bq[s]), acc[rt], 0, 0, 0);
        if (f + kPre < kN) ring[f % kPre] = rd(As, f + kPre);
        if (rt == 0) {
          // finish the pending piece: s = 0 -> piece 3 of k-tile kt, else
          // piece s - 1 of k-tile kt + 1
          bq[(s + 3) & 3] = apply8<FMT>(wpend, lv, scpend);
          // NF4: pieces of k-tile kt + 1 are read only in the next iteration;
          // the compiler would otherwise sink their arithmetic to the end of
          // this one (a burst of VALU work with no MFMAs beside it, and three
          // pieces' table values live at once). MXFP4's piece is one
          // conversion per pair and measured no better pinned.
          if constexpr (NF4) pin_regs(bq[(s + 3) & 3]);
        }
        if (rt == NRT / 2) {
          // table reads of piece s of k-tile kt + 1
          wpend = braw_n[s];
          scpend = sc_n;
          fetch8<FMT>(wpend, lutf, lv);
        }
#pragma unroll
        for (int j = 0; j < kParts; ++j)
          if (f == j * kN / kParts && more) issue_part(kt + 2, j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- epilogue. Lane holds column n32 of each 32x32 tile, rows
    // 8*(i/4) + 4*h + i%4.
    if constexpr (GATEUP) {
      // The gate of pair j0 + n sits in column n, its up in column n + 16 (same
      // rows): a shuffle gives each lane the pair; lanes n32 < 16 finish entries
      // i < 8 and lanes n32 >= 16 entries i >= 8. h is staged through LDS (the
      // stages are free once every wave is past its last k-tile) and written
      // out as whole 16-byte chunks of each row.
      const int jl = n32 & 15, j = j0 + jl;
      const bool jon = j < a.I;
      const int ng = gate_row(a.layout, a.I, jon ? j : 0), nu = up_row(a.layout, a.I, jon ? j : 0);
      const bool gate_lane = n32 < 16;
      // entry (rt, q) of the lane sits in row lrow + rrow(rt, q) of the tile
      const int lrow = (gate_lane ? 0 : 16) + 4 * h;
      auto rrow = [](int rt, int q) { return rt * 32 + 8 * (q >> 2) + (q & 3); };
      // h staged as [kBM][128] bf16; this lane's column of it
      uint16_t* hl = reinterpret_cast<uint16_t*>(stage_mem) + lrow * 128 + w * 16 + jl;
      // the pre-activations g and u saved for the backward pass go through a
      // resource over the tile's rows, so that stores past its last row (or
      // of a pair past I, sent out of range without wrapping: the host keeps
      // a 320-row fp32 tile of 2I values under 2 GiB) are dropped; the test
      // on save_gu is uniform, a scalar branch
      const bool extra = a.save_gu != nullptr;
      const rsrc_t rg = make_rsrc_uniform(extra ? a.save_gu + (int64_t)row0 * 2 * a.I : a.save_gu,
                                          (uint32_t)nrows * 2 * a.I * 4);
      const uint32_t gpitch = (uint32_t)a.I * 8;
      uint32_t cg_off = (jon ? (uint32_t)ng * 4 : (uint32_t)kOob) + lrow * gpitch;
      uint32_t cu_off = (jon ? (uint32_t)nu * 4 : (uint32_t)kOob) + lrow * gpitch;
      asm volatile("" : "+v"(cg_off), "+v"(cu_off));
      // h = g sigma(g) u (SwiGLU) or gc sigma(al gc) (uc + 1) with gc = min(g,
      // lim), uc = clamp(u, -lim, lim) (clamped GLU); sigma(z) = 1 / (1 +
      // 2^(-z log2 e)), the exponent's scale folded into one constant
      auto finish = [&](auto clamped_c) {
        constexpr bool CL = decltype(clamped_c)::value;
        const float ns = (CL ? a.alpha : 1.0f) * -1.4426950408889634f;
        const float lim = a.limit;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          // entry i' < 8 of a gate lane and entry i' + 8 of an up lane are
          // finished by that lane; the partner lane (16 apart) holds the other
          // half of the pair
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            // v_permlane16_swap(lo, hi) swaps rows 1 and 3 of lo with rows 0
            // and 2 of hi (16-lane rows): every lane then holds the gate value
            // of its entry in the first result and the up value in the second
            // (a gate lane keeps its own entries i < 8, an up lane its i >= 8)
            const auto gu = __builtin_amdgcn_permlane16_swap(
                __float_as_uint(acc[rt][q]), __float_as_uint(acc[rt][q + 8]), false, false);
            const float g = __uint_as_float(gu[0]), u = __uint_as_float(gu[1]);
            const uint32_t roff = (uint32_t)rrow(rt, q) * gpitch;
            if (extra) {
              __builtin_amdgcn_raw_buffer_store_b32(gu[0], rg, (int)(roff + cg_off), 0, 0);
              __builtin_amdgcn_raw_buffer_store_b32(gu[1], rg, (int)(roff + cu_off), 0, 0);
            }
            float hv;
            if constexpr (CL) {
              const float gc = fminf(g, lim);
              const float uc = fminf(fmaxf(u, -lim), lim);
              hv = gc * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gc * ns)) * (uc + 1.0f);
            } else {
              hv = g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * ns)) * u;
            }
            // every entry goes to the staging tile (row < kBM): rows past the
            // tile and pairs past I are never copied out
            hl[rrow(rt, q) * 128] = f32_to_bf16(hv);
          }
        }
      };
      __syncthreads();
      if (a.act == MOE4_ACT_SWIGLU_CLAMPED) finish(std::true_type{});
      else finish(std::false_type{});
      __syncthreads();
      const uint16_t* hs = reinterpret_cast<const uint16_t*>(stage_mem);
      const int pbase = cg * 128;
      for (int idx = tid; idx < nrows * 16; idx += 64 * kTiledWaves) {
        const int r = idx >> 4, c = idx & 15;
        if (pbase + 8 * c < a.I)
          __builtin_nontemporal_store(
              *reinterpret_cast<const u32x4*>(hs + r * 128 + 8 * c),
              reinterpret_cast<u32x4*>(a.hout + (int64_t)(row0 + r) * a.I + pbase + 8 * c));
      }
    } else {
      // the tile's rows of y as one buffer resource: a store past its last
      // row (or of a column past N_out, sent out of range) is dropped by the
      // hardware, so no store needs a branch; y rows are read once, by the
      // combine, long after: non-temporal
      const rsrc_t ry =
          make_rsrc_uniform(a.yout + (int64_t)row0 * a.N_out, (uint32_t)nrows * a.N_out * 4);
      const uint32_t pitch = (uint32_t)a.N_out * 4;
      // a lane with no column adds kOob to every offset, which puts them all
      // past the resource without wrapping (the host keeps a 320-row fp32
      // tile under 2 GiB); opaque, so that the choice stays one select
      uint32_t cb = col_on ? (uint32_t)col_row * 4 : (uint32_t)kOob;
      asm volatile("" : "+v"(cb));
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t rt_row = rt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[rt][i]), ry,
                                                (int)(rt_row * pitch + cb), 0, kCpolNt);
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
    case 8: kloop(std::integral_constant<int, 8>{}); break;
    case 9: kloop(std::integral_constant<int, 9>{}); break;
    default: kloop(std::integral_constant<int, 10>{}); break;
  }
}

// nitems: touched experts (sets the K split); nchunks: a bound on the 16-row
// chunks of all experts (sets the grid; the workgroups past the last chunk exit)
template <int FMT, bool GATEUP, bool GATHER = false>
hipError_t run_skinny(const GemmArgs& a, int nitems, int nchunks, hipStream_t s) {
  const int nwg = nitems * a.ncg;
  if (nwg == 0) return hipSuccess;
  // split K over S waves so that ~6K waves stream the weights (about six per
  // SIMD), each wave keeping at least two 128-k iterations (targets of 3K and
  // 4K waves measured no different); gate_up takes at most four (with one row
  // per expert, four waves per workgroup measured 5-15% faster than eight, and
  // no slower elsewhere)
  const int nit = (a.K + 127) / 128;
  int S = (6144 + nwg - 1) / nwg;
  S = max(1, min(S, min(GATEUP ? 4 : 8, nit / 2)));
  constexpr int MAXR = kSkMaxRowTiles;
  using SS = SkinnyScales<FMT>;
  // staged scales, then the partial sums of the S waves
  const size_t lds =
      SS::lds_bytes(a.K, 16 * kSkNc) + (size_t)S * MAXR * kSkNc * 256 * sizeof(float);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_skinny<FMT, GATEUP, GATHER>),
      hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)(SS::lds_bytes(SS::kKc, 16 * kSkNc) + 8 * MAXR * kSkNc * 256 * sizeof(float)));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_skinny<FMT, GATEUP, GATHER>), dim3(nchunks * a.ncg), dim3(64 * S), lds, s,
                     a);
  return hipGetLastError();
}

template <int FMT, bool GATEUP, bool GATHER = false>
hipError_t run_tiled(const GemmArgs& a, int ntiles, hipStream_t s) {
  if (ntiles == 0) return hipSuccess;
  // ntiles bounds the row tiles; tile j of the largest-first order runs on
  // XCD j % 8, so every XCD needs ceil(tiles / 8) * ncg ids
  const int nwg = (ntiles + 7) * a.ncg;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&k_tiled<FMT, GATEUP, GATHER>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kTiledLds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_tiled<FMT, GATEUP, GATHER>), dim3(nwg), dim3(64 * kTiledWaves), kTiledLds,
                     s, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t forward_fmt(const moe4_experts& ex, const uint16_t* x_perm, const int32_t* offsets,
                       int rows, float* y_perm, float* save_gu, const float* xa,
                       uint16_t* hbuf, int variant, const GatherRows* ga,
                       const LaunchEvents& le, hipStream_t s) {
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
  if (ga) {
    // gate_up reads row slot_of_row[r] / k of x for its row r
    g.A = ga->x;
    g.arows = ga->slot_of_row;
    g.gk = ga->k;
    g.a_rows = ga->T;
  }
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
  d.arows = nullptr;
  d.bias = ex.dn_bias;
  d.xa = nullptr;
  d.loraB = nullptr;
  d.r = 0;
  d.hout = nullptr;
  d.yout = y_perm;
  d.save_gu = nullptr;
  // double-quantised NF4: the absmax codes, their per-256 scales and the offset
  g.ws2 = ex.gu_s2;
  g.dqoff = ex.gu_soff;
  g.dqbook = ex.dq_book;
  d.ws2 = ex.dn_s2;
  d.dqoff = ex.dn_soff;
  d.dqbook = ex.dq_book;
  const int touched = min(E, rows);
  hipError_t err;
  if (variant == MOE4_VARIANT_SKINNY) {
    // I is a multiple of 32 (the pairs of a column group); H may end in a
    // partial column group, whose rows past H read as zeros and are not stored
    g.ncg = I / (8 * kSkNc);
    d.ncg = (H + 16 * kSkNc - 1) / (16 * kSkNc);
    // 16-row chunks: at most one per row, and at most rows / 16 plus one per
    // touched expert
    const int nchunks = min(rows, rows / (16 * kSkMaxRowTiles) + touched);
    le.before(0, s);
    err = ga ? run_skinny<FMT, true, true>(g, touched, nchunks, s)
             : run_skinny<FMT, true>(g, touched, nchunks, s);
    le.after(0, s);
    if (err != hipSuccess) return err;
    le.before(1, s);
    err = run_skinny<FMT, false>(d, touched, nchunks, s);
    le.after(1, s);
    return err;
  }
  // row tiles: at most rows / kBM + (one per touched expert)
  const int ntiles = rows / kBM + touched;
  g.ncg = (I + 127) / 128;
  d.ncg = (H + kBN - 1) / kBN;
  le.before(0, s);
  err = ga ? run_tiled<FMT, true, true>(g, ntiles, s) : run_tiled<FMT, true>(g, ntiles, s);
  le.after(0, s);
  if (err != hipSuccess) return err;
  le.before(1, s);
  err = run_tiled<FMT, false>(d, ntiles, s);
  le.after(1, s);
  return err;
}

}  // namespace

// double-quantised absmax decoded inside the kernels: every weight row spans at
// most 256 absmax (two groups of the second level); else expanded first
static bool dq_in_kernel(const moe4_experts& ex) {
  return ex.format == MOE4_FMT_NF4_DQ && ex.H / 64 <= 256 && ex.I / 64 <= 256;
}

size_t forward_ws_bytes(const moe4_experts& ex, int rows) {
  size_t b = align_up((size_t)rows * ex.I * sizeof(uint16_t), 256);
  if (ex.lora_A) b += align_up((size_t)rows * ex.lora_r * sizeof(float), 256);
  return b + (dq_in_kernel(ex) ? 0 : dq_expand_bytes(ex));
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
                                 const LaunchEvents& le, hipStream_t s, const GatherRows* ga) {
  *variant = choose_variant(ex, rows);
  if (rows == 0) return hipSuccess;
  char* p = static_cast<char*>(ws);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(p);
  p += align_up((size_t)rows * ex.I * sizeof(uint16_t), 256);
  float* xa = nullptr;
  char* abs_ws = p + (ex.lora_A ? align_up((size_t)rows * ex.lora_r * sizeof(float), 256) : 0);
  if (ex.lora_A) {
    xa = save_xa ? save_xa : reinterpret_cast<float*>(p);
    hipError_t err = launch_rank_proj(x_perm, offsets, ex.E, rows, ex.H, ex.lora_A, ex.lora_r,
                                      xa, s);
    if (err != hipSuccess) return err;
  }
  if (ex.format == MOE4_FMT_NF4_DQ) {
    // rows of at most 256 absmax (K <= 16384): both absmax levels decoded
    // inside the kernels; otherwise expand the absmax once into the workspace,
    // then the plain NF4 kernels
    if (dq_in_kernel(ex))
      return forward_fmt<MOE4_FMT_NF4_DQ>(ex, x_perm, offsets, rows, y_perm, save_gu, xa, hbuf,
                                          *variant, ga, le, s);
    moe4_experts plain;
    hipError_t err = dq_expand_experts(ex, abs_ws, &plain, s);
    if (err != hipSuccess) return err;
    return forward_fmt<MOE4_FMT_NF4>(plain, x_perm, offsets, rows, y_perm, save_gu, xa, hbuf,
                                     *variant, ga, le, s);
  }
  if (ex.format == MOE4_FMT_NF4)
    return forward_fmt<MOE4_FMT_NF4>(ex, x_perm, offsets, rows, y_perm, save_gu, xa, hbuf,
                                     *variant, ga, le, s);
  return forward_fmt<MOE4_FMT_MXFP4>(ex, x_perm, offsets, rows, y_perm, save_gu, xa, hbuf,
                                     *variant, ga, le, s);
}

}  // namespace moe4
