// Device-side helpers shared by the moe4 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(v, d, kWave);
    if (l >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

// Locate work item q when expert e owns units(n_e) consecutive items
// (n_e = offsets[e+1] - offsets[e]). Every lane of the wave gets the same
// answer: e = -1 when q is past the last item, else the expert and the item's
// index inside it. Offsets are read once per lane (a contiguous chunk).
template <typename Units>
__device__ __forceinline__ void locate_item(const int32_t* __restrict__ offsets, int E, int q,
                                            Units units, int& e_out, int& u_out) {
  const int l = lane_id();
  const int per = (E + kWave - 1) / kWave;
  const int e0 = l * per;
  int cnt = 0;
  if (e0 < E) {
    int prev = offsets[e0];
    for (int i = 0; i < per && e0 + i < E; ++i) {
      int nx = offsets[e0 + i + 1];
      cnt += units(nx - prev);
      prev = nx;
    }
  }
  int incl = wave_inclusive_scan(cnt);
  int excl = incl - cnt;
  bool own = (q >= excl) && (q < incl);
  unsigned long long b = __ballot(own);
  if (b == 0ull) {
    e_out = -1;
    u_out = 0;
    return;
  }
  int owner = __ffsll((long long)b) - 1;
  int ef = -1, uf = 0;
  if (own) {
    int acc = excl;
    int prev = offsets[e0];
    for (int i = 0; i < per && e0 + i < E; ++i) {
      int nx = offsets[e0 + i + 1];
      int u = units(nx - prev);
      if (q < acc + u) {
        ef = e0 + i;
        uf = q - acc;
        break;
      }
      acc += u;
      prev = nx;
    }
  }
  e_out = __shfl(ef, owner, kWave);
  u_out = __shfl(uf, owner, kWave);
}

// Remap a linear workgroup id so that consecutive logical ids land on the same
// XCD (the dispatcher deals workgroups round-robin over the 8 XCDs, each with
// its own L2). Bijective for any grid size.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int q = nblocks / kXcd, r = nblocks % kXcd;
  const int xcd = bid % kXcd, local = bid / kXcd;
  // XCDs < r hold q+1 logical ids, the rest hold q
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
}

}  // namespace moe4
