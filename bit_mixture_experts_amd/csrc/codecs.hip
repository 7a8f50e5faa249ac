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

// ---------------------------------------------------- MXFP4 -> NF4 re-quantisation
//
// The convenient QLoRA path of the MXFP4 page ("Two fidelity paths"): decode
// the released blocks exactly, then quantise the decoded stack to NF4. Fused
// here into one pass with no floating-point work per element: every decoded
// value is m * 2^(s-127) with m an e2m1 magnitude, so the block's absmax is
// (1 + f/2) * 2^(Emax - 127) (f = 0 or 1) and the quantiser's ratio
// x = fp32(v / absmax) = fp32(m * 2^(s - Emax) / (1 + f/2)) depends only on
// v's nibble, f and the exponent gap d = s - Emax. A lane's 32 values share
// one scale, so one table of 16 codes per (f, d) maps all of them. The
// tables are built at compile time with the quantiser's own rule (IEEE fp32
// division, fp32 midpoints), which makes the codes those of quantising the
// decoded values, subnormal decodes (scale bytes 0 and 1) included.

constexpr float kE2m1Mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
// d = 1, 0, -1, ..., -7 take buckets 0..8; d <= -8 (every |x| < 0.024, code 7)
// and the all-zero block take bucket 9
constexpr int kConvBuckets = 10;

// code of nibble n for bucket b and absmax mantissa 1 + f/2
constexpr uint32_t conv_code(int f, int b, int n) {
  const float mag = kE2m1Mag[n & 7];
  if (mag == 0.0f || b >= kConvBuckets - 1) return 7u;
  float p = mag;   // m * 2^d, exact
  for (int i = 0; i < 1 - b; ++i) p *= 2.0f;
  for (int i = 0; i < b - 1; ++i) p *= 0.5f;
  float x = p / (f ? 1.5f : 1.0f);   // correctly rounded, as in the quantiser
  if (n & 8) x = -x;
  uint32_t c = 0;
  for (int i = 0; i < 15; ++i) c += (x > mid(i)) ? 1u : 0u;
  return c;
}
// four codes as bytes: nibbles 4j .. 4j+3 (j = 0: m 0..3 positive, 1: m 4..7
// positive, 2 and 3: the same magnitudes negative)
constexpr uint32_t conv_word(int f, int b, int j) {
  return conv_code(f, b, 4 * j) | (conv_code(f, b, 4 * j + 1) << 8) |
         (conv_code(f, b, 4 * j + 2) << 16) | (conv_code(f, b, 4 * j + 3) << 24);
}
#define MOE4_CONV_ROW(f, b) \
  conv_word(f, b, 0), conv_word(f, b, 1), conv_word(f, b, 2), conv_word(f, b, 3)
#define MOE4_CONV_F(f)                                                                    \
  MOE4_CONV_ROW(f, 0), MOE4_CONV_ROW(f, 1), MOE4_CONV_ROW(f, 2), MOE4_CONV_ROW(f, 3),     \
      MOE4_CONV_ROW(f, 4), MOE4_CONV_ROW(f, 5), MOE4_CONV_ROW(f, 6), MOE4_CONV_ROW(f, 7), \
      MOE4_CONV_ROW(f, 8), MOE4_CONV_ROW(f, 9)
__constant__ uint32_t kConvLut[2 * kConvBuckets * 4] = {MOE4_CONV_F(0), MOE4_CONV_F(1)};
#undef MOE4_CONV_F
#undef MOE4_CONV_ROW

// 8 nibbles (one dword) -> 8 NF4 codes, through the lane's table t: the byte
// permute looks up four magnitudes at once, the sign picks the table half
__device__ __forceinline__ uint32_t conv_dword(uint32_t w, const u32x4& t) {
  uint32_t out = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t nb = (w >> (4 * h)) & 0x0F0F0F0Fu;   // nibbles h, h+2, h+4, h+6 as bytes
    const uint32_t m = nb & 0x07070707u;
    const uint32_t neg = ((nb >> 3) & 0x01010101u) * 0xFFu;
    const uint32_t cp = __builtin_amdgcn_perm(t[1], t[0], m);
    const uint32_t cn = __builtin_amdgcn_perm(t[3], t[2], m);
    out |= ((cn & neg) | (cp & ~neg)) << (4 * h);
  }
  return out;
}

// Two lanes per NF4 block of 64: lane h of block q owns MXFP4 block 2q + h
// (16 bytes, one scale); codes go to the same 16 bytes of the output.
__global__ __launch_bounds__(256) void k_convert_mxfp4_nf4(const uint8_t* __restrict__ blocks,
                                                           const uint8_t* __restrict__ scales,
                                                           int64_t nmx,
                                                           uint8_t* __restrict__ packed,
                                                           float* __restrict__ absmax) {
  __shared__ u32x4 lut[2 * kConvBuckets];
  if (threadIdx.x < 2 * kConvBuckets)
    lut[threadIdx.x] = u32x4{kConvLut[4 * threadIdx.x], kConvLut[4 * threadIdx.x + 1],
                             kConvLut[4 * threadIdx.x + 2], kConvLut[4 * threadIdx.x + 3]};
  __syncthreads();
  const int64_t mb = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool valid = mb < nmx;   // nmx is even: both lanes of a pair agree
  u32x4 q = {0u, 0u, 0u, 0u};
  uint32_t s = 0;
  if (valid) {
    q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(blocks) + mb);
    s = scales[mb];
  }
  uint32_t mm = 0;   // largest magnitude index among the lane's 32 nibbles
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) mm = max(mm, (q[i] >> (4 * j)) & 7u);
  // key monotone in |value| = (1 + f/2) 2^(E - 127): 2 (E + 2) + f, with
  // E = s + (-1, 0, 0, 1, 1, 2, 2) and f = (0, 0, 1, 0, 1, 0, 1) for m = 1..7;
  // 0 when the lane holds only zeros
  const uint32_t kl = mm ? 2u * s + mm + 2u - (mm == 1u ? 1u : 0u) : 0u;
  const uint32_t key = max(kl, (uint32_t)__shfl_xor((int)kl, 1, kWave));
  const int emax = (int)(key >> 1) - 2, f = (int)(key & 1u);
  const int d = (int)s - emax;
  const int b = key == 0u ? kConvBuckets - 1 : min(max(1 - d, 0), kConvBuckets - 1);
  const u32x4 t = lut[f * kConvBuckets + b];
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = conv_dword(q[i], t);
  // absmax = (1 + f/2) 2^(emax - 127); emax >= -1; subnormal for emax <= 0
  uint32_t abits;
  if (key == 0u) abits = 0u;
  else if (emax >= 255) abits = 0x7F800000u;   // overflow: the decode itself is not finite
  else if (emax >= 1) abits = ((uint32_t)emax << 23) | ((uint32_t)f << 22);
  else abits = (2u + (uint32_t)f) << (emax + 21);
  if (valid) {
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(packed) + mb);
    if ((mb & 1) == 0) absmax[mb >> 1] = __uint_as_float(abits);
  }
}

// ------------------------------------------- double-quantised NF4 absmax
//
// The nested absmax form of a resident NF4 stack (project page
// "experts4bit-qlora", "Limitations -- qlora-fused-moe-experts", the
// double-quantised absmax item): offset = fp32 rounding of the float64 mean of
// all absmax; per 256 consecutive values d = fp32(a - offset), absmax2 =
// max |d|, code = the code-book entry nearest to fp32(d / absmax2) (decided by
// fp32 midpoints formed in float64; a value on a midpoint takes the lower
// code). Decoding: fp32(fp32(book[code] * absmax2) + offset), no fused
// multiply-add.

// float64 partial sums of contiguous chunks, one per workgroup
__global__ __launch_bounds__(256) void k_dq_partial(const float* __restrict__ a, int64_t n,
                                                    double* __restrict__ part) {
  __shared__ double red[256];
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per, b1 = min(n, b0 + per);
  double acc = 0.0;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += blockDim.x) acc += (double)a[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// offset = fp32(sum of the partials / n), partials summed in a fixed order
__global__ __launch_bounds__(256) void k_dq_offset(const double* __restrict__ part, int nparts,
                                                   int64_t n, float* __restrict__ offset) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int i = threadIdx.x; i < nparts; i += blockDim.x) acc += part[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) offset[0] = (float)(red[0] / (double)n);
}

// one wave per group of 256 absmax (4 per lane); the 255 midpoints of the
// code book are formed once per workgroup in LDS and searched by bisection
__global__ __launch_bounds__(256) void k_dq_compress(const float* __restrict__ a, int64_t n,
                                                     const float* __restrict__ book,
                                                     const float* __restrict__ offset,
                                                     uint8_t* __restrict__ code,
                                                     float* __restrict__ absmax2) {
  __shared__ float mids[256];
  if (threadIdx.x < 255)
    mids[threadIdx.x] =
        (float)(((double)book[threadIdx.x] + (double)book[threadIdx.x + 1]) * 0.5);
  __syncthreads();
  const int64_t g = (int64_t)blockIdx.x * 4 + wave_id();
  const int64_t ngroups = (n + 255) / 256;
  if (g >= ngroups) return;
  const float off = offset[0];
  const int l = lane_id();
  float d[4];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t idx = g * 256 + 4 * l + i;
    d[i] = idx < n ? __fsub_rn(a[idx], off) : 0.0f;
    m = fmaxf(m, fabsf(d[i]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x = m == 0.0f ? 0.0f : __fdiv_rn(d[i], m);
    // number of midpoints strictly below x
    int lo = 0, hi = 255;   // answer in [lo, hi]
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int mid = (lo + hi) >> 1;
      if (mids[mid] < x) lo = mid + 1;
      else hi = mid;
    }
    packed |= (uint32_t)lo << (8 * i);
  }
  const int64_t base = g * 256 + 4 * l;
  if (base + 3 < n) {
    *reinterpret_cast<uint32_t*>(code + base) = packed;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (base + i < n) code[base + i] = (uint8_t)(packed >> (8 * i));
  }
  if (l == 0) absmax2[g] = m;
}

// decoded absmax, four per thread
__global__ __launch_bounds__(256) void k_dq_expand(const uint8_t* __restrict__ code,
                                                   const float* __restrict__ absmax2,
                                                   const float* __restrict__ offset,
                                                   const float* __restrict__ book, int64_t n,
                                                   float* __restrict__ out) {
  __shared__ float tb[256];
  tb[threadIdx.x] = book[threadIdx.x];
  __syncthreads();
  const float off = offset[0];
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i0 >= n) return;
  const float s2 = absmax2[i0 >> 8];   // the four share one group (256 % 4 == 0)
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i0 + i < n) out[i0 + i] = mul_then_add(tb[code[i0 + i]], s2, off);
}

}  // namespace

int dq_partials(int64_t n) {
  const int64_t p = (n + 4095) / 4096;
  return (int)(p < kDqPartials ? p : kDqPartials);
}

hipError_t launch_dq_compress(const float* absmax, int64_t n, const float* book, uint8_t* code,
                              float* absmax2, float* offset, void* ws, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int np = dq_partials(n);
  double* part = static_cast<double*>(ws);
  hipLaunchKernelGGL(k_dq_partial, dim3(np), dim3(256), 0, s, absmax, n, part);
  hipLaunchKernelGGL(k_dq_offset, dim3(1), dim3(256), 0, s, part, np, n, offset);
  const int64_t ngroups = (n + 255) / 256;
  hipLaunchKernelGGL(k_dq_compress, dim3((unsigned)((ngroups + 3) / 4)), dim3(256), 0, s, absmax,
                     n, book, offset, code, absmax2);
  return hipGetLastError();
}

hipError_t launch_dq_expand(const uint8_t* code, const float* absmax2, const float* offset,
                            const float* book, int64_t n, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(k_dq_expand, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, code,
                     absmax2, offset, book, n, out);
  return hipGetLastError();
}

size_t dq_expand_bytes(const moe4_experts& ex) {
  if (ex.format != MOE4_FMT_NF4_DQ) return 0;
  const int64_t ngu = (int64_t)ex.E * 2 * ex.I * (ex.H / 64);
  const int64_t ndn = (int64_t)ex.E * ex.H * (ex.I / 64);
  return align_up((size_t)ngu * 4, 256) + align_up((size_t)ndn * 4, 256);
}

hipError_t dq_expand_experts(const moe4_experts& ex, void* abs_ws, moe4_experts* out,
                             hipStream_t s) {
  const int64_t ngu = (int64_t)ex.E * 2 * ex.I * (ex.H / 64);
  const int64_t ndn = (int64_t)ex.E * ex.H * (ex.I / 64);
  float* gu = static_cast<float*>(abs_ws);
  float* dn = reinterpret_cast<float*>(static_cast<char*>(abs_ws) + align_up((size_t)ngu * 4, 256));
  hipError_t e = launch_dq_expand(static_cast<const uint8_t*>(ex.gu_s), ex.gu_s2, ex.gu_soff,
                                  ex.dq_book, ngu, gu, s);
  if (e != hipSuccess) return e;
  e = launch_dq_expand(static_cast<const uint8_t*>(ex.dn_s), ex.dn_s2, ex.dn_soff, ex.dq_book,
                       ndn, dn, s);
  if (e != hipSuccess) return e;
  *out = ex;
  out->format = MOE4_FMT_NF4;
  out->gu_s = gu;
  out->dn_s = dn;
  out->gu_s2 = out->dn_s2 = out->gu_soff = out->dn_soff = out->dq_book = nullptr;
  return hipSuccess;
}

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

hipError_t launch_convert_mxfp4_nf4(const uint8_t* blocks, const uint8_t* scales, int64_t R,
                                    int64_t K, uint8_t* packed, float* absmax, hipStream_t s) {
  const int64_t nmx = R * (K / 32);
  if (nmx == 0) return hipSuccess;
  const int64_t grid = (nmx + 255) / 256;
  hipLaunchKernelGGL(k_convert_mxfp4_nf4, dim3((unsigned)grid), dim3(256), 0, s, blocks, scales,
                     nmx, packed, absmax);
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
