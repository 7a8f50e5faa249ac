// The router step in front of the expert path: fp32 router logits from the
// bf16 tokens and router weights, and the backward of the routing weights
// (the gradient of each slot's weight and, through the routing softmax, of
// the logits). The pages make the logits the place where arithmetically
// equivalent forwards part ways (rounding flips top-k choices), so the logits
// are kept in fp32 (project page "experts4bit-qlora", "Current measured
// position").
#include "common.hpp"
#include "internal.hpp"

namespace moe4 {
namespace {

// ------------------------------------------------------------ router logits
//
// logits[t][e] = sum_h x[t][h] W_r[e][h] (+ bias[e]). One workgroup = 32
// experts x 32 tokens; its four waves split H and their partial 32x32 tiles
// are summed through LDS. The router weights are MFMA operand A (rows =
// experts) and the tokens operand B (columns = tokens), so that each lane ends
// with four consecutive experts of one token.
constexpr int kRtTile = 32;

__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ wr,
                                                       const float* __restrict__ bias, int T,
                                                       int H, int E, float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) float red[4][16][kWave];
  const int w = wave_id(), l = lane_id(), n32 = l & 31, h = l >> 5;
  const int t0 = blockIdx.x * kRtTile, e0 = blockIdx.y * kRtTile;
  const int nt = min(kRtTile, T - t0), ne = min(kRtTile, E - e0);
  // tiles as buffer resources: rows past the tile read as zeros
  const rsrc_t rx = make_rsrc(x + (int64_t)t0 * H, (uint32_t)nt * H * 2);
  const rsrc_t rw = make_rsrc(wr + (int64_t)e0 * H, (uint32_t)ne * H * 2);
  const int nsteps = (H + 15) / 16;
  const int per = (nsteps + 3) / 4;
  const int s0 = w * per, s1 = min(nsteps, s0 + per);
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  const int row_off = n32 * H * 2;
  // eight k-steps per batch: all loads first, then the MFMAs
  constexpr int kB = 8;
  for (int s = s0; s < s1; s += kB) {
    u32x4 av[kB], bv[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int k = (s + u) * 16 + 8 * h;
      const bool in = s + u < s1 && k < H;
      av[u] = buf_load_b128(rw, in ? row_off + 2 * k : kOob);
      bv[u] = buf_load_b128(rx, in ? row_off + 2 * k : kOob);
    }
#pragma unroll
    for (int u = 0; u < kB; ++u)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                    __builtin_bit_cast(bf16x8, bv[u]), acc, 0,
                                                    0, 0);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) red[w][i][l] = acc[i];
  __syncthreads();
  // thread (q, lane) sums acc entries 4q..4q+3 of the four waves: experts
  // e0 + 8q + 4h + (0..3) of token t0 + n32
  const int q = w;
  const int t = t0 + n32;
  if (t >= T) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + 8 * q + 4 * h + i;
    if (e < E) {
      float v = red[0][4 * q + i][l] + red[1][4 * q + i][l] + red[2][4 * q + i][l] +
                red[3][4 * q + i][l];
      if (bias) v += bias[e];
      logits[(int64_t)t * E + e] = v;
    }
  }
}

// --------------------------------------------------------- routing backward
//
// One wave per token t: dw[t][j] = <dOut[t], y[row_of_slot[t*k + j]]> for the
// k slots (fp32 sums over H), then the logit gradient through the routing
// softmax: renormalised weights are the softmax of the chosen logits, so
// dlogits[t][e] = w_e (dw_e - sum_j w_j dw_j) for a chosen e and 0 otherwise;
// plain top-k weights are the full softmax p of the logits, and
// dlogits[t][e] = p_e (g_e - sum_j w_j dw_j) with g_e = dw_j for the chosen e.
constexpr int kRbMaxE = 1024;

__global__ __launch_bounds__(256) void k_route_backward(
    const int32_t* __restrict__ idx, const float* __restrict__ tw,
    const float* __restrict__ lg, int renorm, const uint16_t* __restrict__ dout,
    const float* __restrict__ y, const int32_t* __restrict__ row_of_slot, int T, int k, int E,
    int H, float* __restrict__ dw, float* __restrict__ dlog) {
  __shared__ int sj[4][kRbMaxE];      // slot j of expert e for this wave's token, or -1
  __shared__ float sdw[4][kRbMaxE];   // dw of slot j
  const int w = wave_id(), l = lane_id();
  const int t = blockIdx.x * 4 + w;
  const bool live = t < T;
  for (int e = l; e < E; e += kWave) sj[w][e] = -1;
  __syncthreads();
  if (live)
    for (int j = l; j < k; j += kWave) sj[w][idx[(int64_t)t * k + j]] = j;
  // dot products, eight slots at a time; lane c covers elements 4c .. 4c+3
  if (live) {
    const uint16_t* dr = dout + (int64_t)t * H;
    for (int j0 = 0; j0 < k; j0 += 8) {
      const int nj = min(8, k - j0);
      const float* yr[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        yr[u] = y + (int64_t)row_of_slot[(int64_t)t * k + j0 + min(u, nj - 1)] * H;
      float p[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int c = l; c < H / 4; c += kWave) {
        const uint2 dv = *reinterpret_cast<const uint2*>(dr + 4 * c);
        const float d0 = bf16lo(dv.x), d1 = bf16hi(dv.x), d2 = bf16lo(dv.y), d3 = bf16hi(dv.y);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (u < nj) {
            const f32x4 yv = *reinterpret_cast<const f32x4*>(yr[u] + 4 * c);
            p[u] += d0 * yv[0] + d1 * yv[1] + d2 * yv[2] + d3 * yv[3];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u < nj) {
          const float v = wave_sum(p[u]);
          if (l == u) {
            sdw[w][j0 + u] = v;
            dw[(int64_t)t * k + j0 + u] = v;
          }
        }
      }
    }
  }
  __syncthreads();
  if (!live) return;
  float s = 0.0f;
  for (int j = l; j < k; j += kWave) s += tw[(int64_t)t * k + j] * sdw[w][j];
  s = wave_sum(s);
  float* out = dlog + (int64_t)t * E;
  if (renorm) {
    for (int e = l; e < E; e += kWave) {
      const int j = sj[w][e];
      out[e] = j >= 0 ? tw[(int64_t)t * k + j] * (sdw[w][j] - s) : 0.0f;
    }
  } else {
    const float* lr = lg + (int64_t)t * E;
    float m = __int_as_float((int)0xFF800000u);   // -inf
    for (int e = l; e < E; e += kWave) m = fmaxf(m, lr[e]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    float z = 0.0f;
    for (int e = l; e < E; e += kWave) z += __expf(lr[e] - m);
    z = wave_sum(z);
    const float rz = 1.0f / z;
    for (int e = l; e < E; e += kWave) {
      const int j = sj[w][e];
      const float pe = __expf(lr[e] - m) * rz;
      out[e] = pe * ((j >= 0 ? sdw[w][j] : 0.0f) - s);
    }
  }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int T,
                                int H, int E, float* logits, hipStream_t s) {
  const dim3 grid((T + kRtTile - 1) / kRtTile, (E + kRtTile - 1) / kRtTile);
  hipLaunchKernelGGL(k_router_logits, grid, dim3(256), 0, s, x, wr, bias, T, H, E, logits);
  return hipGetLastError();
}

hipError_t launch_route_backward(const int32_t* idx, const float* tw, const float* lg,
                                 int renorm, const uint16_t* dout, const float* y,
                                 const int32_t* row_of_slot, int T, int k, int E, int H,
                                 float* dw, float* dlog, hipStream_t s) {
  hipLaunchKernelGGL(k_route_backward, dim3((T + 3) / 4), dim3(256), 0, s, idx, tw, lg, renorm,
                     dout, y, row_of_slot, T, k, E, H, dw, dlog);
  return hipGetLastError();
}

}  // namespace moe4
