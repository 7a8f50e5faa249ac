// 4-bit weight formats as seen by the GEMM kernels.
//
// Both formats store a weight row n of a [N, K] stack as K/2 contiguous bytes,
// two values per byte with the even element in the low nibble (an MXFP4 row of
// [K/32, 16] blocks is the same byte sequence). They differ in the per-block
// scale: NF4 keeps one fp32 absmax per 64 values; MXFP4 one e8m0 byte per 32
// values, worth 2^(s - 127). ("How do I train and serve MoE models released in
// MXFP4", "Why it happens"; project page "experts4bit-qlora", "Limitations --
// qlora-fused-moe-experts".)
#pragma once

#include "common.hpp"
#include "../../include/moe4.h"

namespace moe4 {

// NormalFloat4 levels (QLoRA paper, appendix E), exact fp32 values.
__device__ constexpr float kNf4Levels[16] = {
    -1.0f, -0.6961928009986877f, -0.5250730514526367f, -0.39491748809814453f,
    -0.28444138169288635f, -0.18477343022823334f, -0.09105003625154495f, 0.0f,
    0.07958029955625534f, 0.16093020141124725f, 0.24611230194568634f,
    0.33791524171829224f, 0.44070982933044434f, 0.5626170039176941f,
    0.7229568362236023f, 1.0f};

// e2m1 code points (OCP MX v1.0): sign bit 3, then {0, .5, 1, 1.5, 2, 3, 4, 6}.
__device__ constexpr float kE2m1[16] = {0.0f,  0.5f,  1.0f,  1.5f,  2.0f,  3.0f,  4.0f,  6.0f,
                                        -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};

template <int FMT>
struct Format;

template <>
struct Format<MOE4_FMT_NF4> {
  static constexpr int kBlock = 64;
  __device__ static float level(int c) { return kNf4Levels[c]; }
  // scale of block b in row `row` of a stack whose rows hold K values
  __device__ static float scale(const void* s, int64_t row, int K, int b) {
    return static_cast<const float*>(s)[row * (K / 64) + b];
  }
};

template <>
struct Format<MOE4_FMT_MXFP4> {
  static constexpr int kBlock = 32;
  __device__ static float level(int c) { return kE2m1[c]; }
  __device__ static float e8m0(uint32_t s) {
    // 2^(s-127); s = 0 is the fp32 subnormal 2^-127; s = 255 is NaN
    if (s == 0u) return __uint_as_float(0x00400000u);
    if (s == 255u) return __uint_as_float(0x7FC00000u);
    return __uint_as_float(s << 23);
  }
  __device__ static float scale(const void* s, int64_t row, int K, int b) {
    return e8m0(static_cast<const uint8_t*>(s)[row * (K / 32) + b]);
  }
};

// NF4 with double-quantised absmax: the same codes and blocks; the absmax
// arrives as an 8-bit code plus a per-256 scale and a stack offset (decoded by
// the kernels that read it; Format::scale is not used for it)
template <>
struct Format<MOE4_FMT_NF4_DQ> {
  static constexpr int kBlock = 64;
  __device__ static float level(int c) { return kNf4Levels[c]; }
};

// byte -> the fp32 NF4 levels of its two nibbles (low nibble first): a
// 2 KiB table in device memory that kernels copy into LDS
struct Nf4Pairs {
  float v[512];
};
constexpr Nf4Pairs make_nf4_pairs() {
  Nf4Pairs p{};
  for (int i = 0; i < 256; ++i) {
    p.v[2 * i] = kNf4Levels[i & 15];
    p.v[2 * i + 1] = kNf4Levels[i >> 4];
  }
  return p;
}
__device__ constexpr Nf4Pairs kNf4Pairs = make_nf4_pairs();

// byte -> two bf16 levels (low nibble in the low half)
template <int FMT>
__device__ __forceinline__ uint32_t lut_bf16x2(int byte) {
  return pack_bf16x2(Format<FMT>::level(byte & 15), Format<FMT>::level(byte >> 4));
}

}  // namespace moe4
