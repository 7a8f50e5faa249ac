// NF4 quantiser and bit-exact MXFP4 decoder.
//
// NF4: one fp32 absmax per 64 weights (project page "experts4bit-qlora",
// "Limitations -- qlora-fused-moe-experts"); levels = the NormalFloat4 data type
// of the QLoRA paper (appendix E). MXFP4: OCP microscaling FP4, e2m1 nibbles in
// blocks of 32 sharing one e8m0 scale, decoded bit-identically ("How do I train
// and serve MoE models released in MXFP4", sections "Why it happens" and "Two
// fidelity paths").
#include "common.hpp"
#include "internal.hpp"

namespace moe4 {
namespace {

// NormalFloat4 levels (exact fp32 values, QLoRA paper appendix E).
constexpr float kNf4[16] = {
    -1.0f, -0.6961928009986877f, -0.5250730514526367f, -0.39491748809814453f,
    -0.28444138169288635f, -0.18477343022823334f, -0.09105003625154495f, 0.0f,
    0.07958029955625534f, 0.16093020141124725f, 0.24611230194568634f,
    0.33791524171829224f, 0.44070982933044434f, 0.5626170039176941f,
    0.7229568362236023f, 1.0f};

// Decision thresholds: the float64 midpoint of adjacent levels (exact, since
// both are fp32), rounded once to fp32.
constexpr float mid(int i) { return (float)(((double)kNf4[i] + (double)kNf4[i + 1]) * 0.5); }
__constant__ float kMid[15] = {mid(0), mid(1), mid(2),  mid(3),  mid(4),  mid(5),  mid(6), mid(7),
                               mid(8), mid(9), mid(10), mid(11), mid(12), mid(13), mid(14)};

__device__ __forceinline__ uint32_t nf4_code(float x) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) c += (x > kMid[i]) ? 1u : 0u;
  return c;
}

// 8 lanes per 64-element block; each lane owns 8 consecutive elements.
__global__ __launch_bounds__(256) void k_quantize_nf4(const float* __restrict__ w,
                                                      int64_t nblocks,
                                                      uint8_t* __restrict__ packed,
                                                      float* __restrict__ absmax) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gid >> 3;
  const int sub = (int)(gid & 7);
  const bool valid = blk < nblocks;
  float v[8];
  if (valid) {
    const float4* p = reinterpret_cast<const float4*>(w + blk * 64 + sub * 8);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, __shfl_xor(m, 1, kWave));
  m = fmaxf(m, __shfl_xor(m, 2, kWave));
  m = fmaxf(m, __shfl_xor(m, 4, kWave));
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = (m == 0.0f) ? 0.0f : v[i] / m;   // IEEE fp32 division
    word |= nf4_code(x) << (4 * i);
  }
  if (valid) {
    reinterpret_cast<uint32_t*>(packed + blk * 32)[sub] = word;
    if (sub == 0) absmax[blk] = m;
  }
}

// bf16 bits of e2m1(nib) * 2^(s - 127), built with integer arithmetic so that
// subnormal results are exact (no reliance on fp32 denormal handling).
__device__ __forceinline__ uint32_t mx_to_bf16(uint32_t nib, uint32_t s) {
  const uint32_t sign = (nib & 8u) << 12;
  const uint32_t c = nib & 7u;
  if (s == 255u) return 0x7FC0u;
  if (c == 0u) return sign;
  // magnitude = (1 + f/2) * 2^E: c=1 -> 0.5, 2 -> 1, 3 -> 1.5, 4 -> 2, 5 -> 3, 6 -> 4, 7 -> 6
  const int E = (int)(c >> 1) - 1;
  const uint32_t f = (c >= 2u) ? (c & 1u) : 0u;
  const int biased = E + (int)s;
  if (biased >= 255) return sign | 0x7F80u;
  if (biased >= 1) return sign | ((uint32_t)biased << 7) | (f << 6);
  // biased in {-1, 0}: subnormal, mantissa (2 + f) * 2^(biased + 5), exact
  return sign | ((2u + f) << (biased + 5));
}

// one thread per 32-element block: 16 bytes in, 64 bytes out
__global__ __launch_bounds__(256) void k_decode_mxfp4(const uint8_t* __restrict__ blocks,
                                                      const uint8_t* __restrict__ scales,
                                                      int64_t nblk, uint16_t* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  const u32x4 q = *reinterpret_cast<const u32x4*>(blocks + b * 16);
  const uint32_t s = scales[b];
  u32x4* dst = reinterpret_cast<u32x4*>(out + b * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wd = q[i];
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t byte = (wd >> (8 * j)) & 0xFFu;
      o[j] = mx_to_bf16(byte & 15u, s) | (mx_to_bf16(byte >> 4, s) << 16);
    }
    dst[i] = o;
  }
}

}  // namespace

hipError_t launch_quantize_nf4(const float* w, int64_t n, uint8_t* packed, float* absmax,
                               hipStream_t s) {
  const int64_t nblocks = n / 64;
  if (nblocks == 0) return hipSuccess;
  const int64_t threads = nblocks * 8;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(k_quantize_nf4, dim3((unsigned)grid), dim3(256), 0, s, w, nblocks, packed,
                     absmax);
  return hipGetLastError();
}

hipError_t launch_decode_mxfp4(const uint8_t* blocks, const uint8_t* scales, int64_t R,
                               int64_t K, uint16_t* out, hipStream_t s) {
  const int64_t nblk = R * (K / 32);
  if (nblk == 0) return hipSuccess;
  const int64_t grid = (nblk + 255) / 256;
  hipLaunchKernelGGL(k_decode_mxfp4, dim3((unsigned)grid), dim3(256), 0, s, blocks, scales, nblk,
                     out);
  return hipGetLastError();
}

}  // namespace moe4
