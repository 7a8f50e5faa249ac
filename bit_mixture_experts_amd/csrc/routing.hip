// Top-k routing, the stable permutation of routed slots by expert, the row
// gather, and the weighted combine.
//
// Each token keeps a small part of the expert set ("How do I offload MoE
// experts to host RAM, or serve and train them from an NVMe arena?", "Why it
// happens"); top-k choices are sensitive to rounding (project page
// "experts4bit-qlora", "Current measured position"), so selection works on the
// given fp32 logits with an exact total order.
#include "common.hpp"
#include "internal.hpp"

namespace moe4 {
namespace {

// ------------------------------------------------------------------ routing

// (value, index) order used for selection: larger value first, then lower index.
__device__ __forceinline__ bool beats(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// One wave per token; lane l holds experts l, l+64, ... (NPL per lane).
template <int NPL>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E,
                                               int k, int renorm, int32_t* __restrict__ idx,
                                               float* __restrict__ wout) {
  const int t = (int)((blockIdx.x * (unsigned)blockDim.x + threadIdx.x) >> 6);
  if (t >= T) return;
  const int l = lane_id();
  const float* row = logits + (int64_t)t * E;
  float v[NPL];
  float selv[NPL];
  uint32_t taken = 0, valid = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = l + kWave * i;
    v[i] = 0.0f;
    selv[i] = 0.0f;
    if (e < E) {
      v[i] = row[e];
      valid |= 1u << i;
    }
  }
  float top = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = l + kWave * i;
      if (((valid & ~taken) >> i) & 1u) {
        if (beats(v[i], e, bv, be)) {
          bv = v[i];
          be = e;
        }
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, kWave);
      const int oe = __shfl_xor(be, m, kWave);
      if (beats(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if (j == 0) top = bv;
    if ((be & (kWave - 1)) == l) taken |= 1u << (be / kWave);
    if ((j & (kWave - 1)) == l) {
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (i == j / kWave) selv[i] = bv;
      idx[(int64_t)t * k + j] = be;
    }
  }
  // weights: exp(v - top) normalised over the selection or over all experts
  float part = 0.0f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    if (renorm) {
      const int j = l + kWave * i;
      if (j < k) part += expf(selv[i] - top);
    } else if ((valid >> i) & 1u) {
      part += expf(v[i] - top);
    }
  }
  const float denom = wave_sum(part);
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = l + kWave * i;
    if (j < k) wout[(int64_t)t * k + j] = expf(selv[i] - top) / denom;
  }
}

// --------------------------------------------------------------- permutation

constexpr int kChunk = 256;        // slots ranked per pass (one per thread)
constexpr int kSmallSlots = 1024;  // single-kernel path up to this many slots
constexpr int kBigChunk = 2048;    // slots per workgroup in the multi-kernel path

// Lanes of this wave whose expert equals mine (match-any emulated with one
// ballot per bit of the expert index). Invalid lanes carry e = -1 (all bits
// set) and are masked out by `valid_mask`.
__device__ __forceinline__ unsigned long long peers(int e, int ebits,
                                                    unsigned long long valid_mask) {
  unsigned long long m = valid_mask;
  for (int b = 0; b < ebits; ++b) {
    const bool bit = (e >> b) & 1;
    const unsigned long long bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

__device__ __forceinline__ unsigned long long lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Stable ranks of one chunk of kChunk slots (blockDim.x == kChunk): returns
// the slot's rank among same-expert slots of the chunk. wcnt is LDS
// [4 waves][E], zeroed by the caller before the call and holding per-wave
// counts after it (a __syncthreads separates the count write from the reads).
__device__ __forceinline__ int chunk_rank(int e, bool ok, int E, int ebits, int* wcnt) {
  const int w = wave_id();
  const unsigned long long valid = __ballot(ok);
  unsigned long long pm = peers(e, ebits, valid);
  if (!ok) pm = 0ull;
  const int rin = __popcll(pm & lanemask_lt());
  if (ok && rin == 0) wcnt[w * E + e] = __popcll(pm);
  __syncthreads();
  int before = 0;
  if (ok)
    for (int ww = 0; ww < w; ++ww) before += wcnt[ww * E + e];
  return before + rin;
}

// Exclusive scan over E counters in LDS by one 256-thread workgroup: cnt[] in,
// out[0..E] (out[E] = total). tmp is LDS of >= 256 ints.
__device__ void block_exclusive_scan(const int* cnt, int E, int* out, int* tmp) {
  const int tid = threadIdx.x;
  const int per = (E + 255) / 256;
  const int e0 = tid * per;
  int s = 0;
  for (int i = 0; i < per; ++i)
    if (e0 + i < E) s += cnt[e0 + i];
  const int incl = wave_inclusive_scan(s);
  if (lane_id() == kWave - 1) tmp[wave_id()] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave_id(); ++w) base += tmp[w];
  int run = base + incl - s;
  for (int i = 0; i < per; ++i)
    if (e0 + i < E) {
      out[e0 + i] = run;
      run += cnt[e0 + i];
    }
  if (tid == 255) out[E] = base + incl;
  __syncthreads();
}

__device__ __forceinline__ int bits_for(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

// Copy (and optionally scale) rows of x into x_perm: one wave per row.
__device__ __forceinline__ void copy_row(const uint16_t* __restrict__ x, int src_row, int H,
                                         const float* __restrict__ row_scale, int slot,
                                         uint16_t* __restrict__ dst) {
  const int l = lane_id();
  const u32x4* s = reinterpret_cast<const u32x4*>(x + (int64_t)src_row * H);
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  const int nv = H / 8;
  const float sc = row_scale ? row_scale[slot] : 1.0f;
  // four 16-byte chunks a lane in flight at once
  for (int c0 = l; c0 < nv; c0 += 4 * kWave) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (c0 + u * kWave < nv) v[u] = s[c0 + u * kWave];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (c0 + u * kWave >= nv) break;
      if (row_scale) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = pack_bf16x2(sc * bf16lo(v[u][i]), sc * bf16hi(v[u][i]));
        __builtin_nontemporal_store(o, d + c0 + u * kWave);
      } else {
        __builtin_nontemporal_store(v[u], d + c0 + u * kWave);
      }
    }
  }
}

// Small problems: every workgroup recomputes the whole permutation in LDS (it
// is at most kSmallSlots slots), workgroup 0 writes the index arrays, and each
// workgroup gathers its share of rows. One launch.
__global__ __launch_bounds__(kChunk) void k_permute_small(
    const int32_t* __restrict__ idx, int S, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_of_row, int32_t* __restrict__ row_of_slot,
    const uint16_t* __restrict__ x, const float* __restrict__ row_scale, int H,
    uint16_t* __restrict__ x_perm, int rows_per_wg) {
  extern __shared__ int lds[];
  int* cnt = lds;                 // [E]
  int* run = cnt + E;             // [E+1]
  int* wcnt = run + E + 1;        // [4][E]
  int* sor = wcnt + 4 * E;        // [kSmallSlots]
  int* tmp = sor + kSmallSlots;   // [256]
  const int tid = threadIdx.x;
  const int ebits = bits_for(E);
  for (int e = tid; e < E; e += kChunk) cnt[e] = 0;
  __syncthreads();
  for (int s = tid; s < S; s += kChunk) {
    const int e = idx[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  block_exclusive_scan(cnt, E, run, tmp);
  if (blockIdx.x == 0)
    for (int e = tid; e <= E; e += kChunk) offsets[e] = run[e];
  for (int c0 = 0; c0 < S; c0 += kChunk) {
    for (int i = tid; i < 4 * E; i += kChunk) wcnt[i] = 0;
    __syncthreads();
    const int s = c0 + tid;
    const int ev = s < S ? idx[s] : -1;
    const bool ok = (unsigned)ev < (unsigned)E;   // out-of-range indices are skipped
    const int e = ok ? ev : -1;
    const int r = chunk_rank(e, ok, E, ebits, wcnt);
    const int row = ok ? run[e] + r : 0;
    __syncthreads();
    if (ok) {
      sor[row] = s;
      if (blockIdx.x == 0) {
        slot_of_row[row] = s;
        row_of_slot[s] = row;
      }
    }
    // advance each expert's running base by this chunk's count
    for (int ee = tid; ee < E; ee += kChunk)
      run[ee] += wcnt[ee] + wcnt[E + ee] + wcnt[2 * E + ee] + wcnt[3 * E + ee];
    __syncthreads();
  }
  if (x == nullptr) return;
  const int r0 = blockIdx.x * rows_per_wg;
  const int r1 = min(S, r0 + rows_per_wg);
  for (int r = r0 + wave_id(); r < r1; r += kChunk / kWave) {
    const int s = sor[r];
    copy_row(x, s / k, H, row_scale, s, x_perm + (int64_t)r * H);
  }
}

// Large problems, pass 1: per-chunk expert counts, counts[c * E + e], one
// workgroup per chunk of kBigChunk slots.
__global__ __launch_bounds__(kChunk) void k_chunk_hist(const int32_t* __restrict__ idx, int S,
                                                       int E, int32_t* __restrict__ counts) {
  extern __shared__ int cnt[];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kChunk) cnt[e] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * kBigChunk;
  const int s1 = min(S, s0 + kBigChunk);
  for (int s = s0 + tid; s < s1; s += kChunk) {
    const int e = idx[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kChunk) counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Pass 2: each workgroup rebuilds the expert offsets and its chunk's starting
// row per expert from all chunk counts (a few KB, cached), then ranks its
// slots in passes of kChunk. Workgroup 0 writes the offsets.
__global__ __launch_bounds__(kChunk) void k_chunk_scatter(const int32_t* __restrict__ idx, int S,
                                                          int E, int nchunks,
                                                          const int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ slot_of_row,
                                                          int32_t* __restrict__ row_of_slot) {
  extern __shared__ int lds[];
  int* tot = lds;            // [E]
  int* run = tot + E;        // [E+1]
  int* before = run + E + 1; // [E]
  int* wcnt = before + E;    // [4][E]
  int* tmp = wcnt + 4 * E;   // [256]
  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  for (int e = tid; e < E; e += kChunk) {
    int all = 0, pre = 0;
    int cc = 0;
    for (; cc + 8 <= nchunks; cc += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = counts[(int64_t)(cc + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        all += v[u];
        pre += (cc + u < c) ? v[u] : 0;
      }
    }
    for (; cc < nchunks; ++cc) {
      const int v = counts[(int64_t)cc * E + e];
      all += v;
      pre += (cc < c) ? v : 0;
    }
    tot[e] = all;
    before[e] = pre;
  }
  __syncthreads();
  block_exclusive_scan(tot, E, run, tmp);
  if (c == 0)
    for (int e = tid; e <= E; e += kChunk) offsets[e] = run[e];
  for (int e = tid; e < E; e += kChunk) run[e] += before[e];
  const int ebits = bits_for(E);
  const int s0 = c * kBigChunk;
  const int s1 = min(S, s0 + kBigChunk);
  for (int p0 = s0; p0 < s1; p0 += kChunk) {
    for (int i = tid; i < 4 * E; i += kChunk) wcnt[i] = 0;
    __syncthreads();
    const int s = p0 + tid;
    const int ev = s < s1 ? idx[s] : -1;
    const bool ok = (unsigned)ev < (unsigned)E;
    const int e = ok ? ev : -1;
    const int r = chunk_rank(e, ok, E, ebits, wcnt);
    if (ok) {
      const int row = run[e] + r;
      slot_of_row[row] = s;
      row_of_slot[s] = row;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kChunk)
      run[ee] += wcnt[ee] + wcnt[E + ee] + wcnt[2 * E + ee] + wcnt[3 * E + ee];
    __syncthreads();
  }
}

// Pass 4: gather rows (one wave per row).
__global__ __launch_bounds__(256) void k_gather(const uint16_t* __restrict__ x, int S, int k,
                                                int H, const int32_t* __restrict__ slot_of_row,
                                                const float* __restrict__ row_scale,
                                                uint16_t* __restrict__ x_perm) {
  const int r = (int)((blockIdx.x * (unsigned)blockDim.x + threadIdx.x) >> 6);
  if (r >= S) return;
  const int s = slot_of_row[r];
  copy_row(x, s / k, H, row_scale, s, x_perm + (int64_t)r * H);
}

// ------------------------------------------------------------------ combine

// One wave per token: out[t] = sum_j w[t,j] * y[row_of_slot[t*k+j]] over fp32
// rows, accumulated in fp32 in ascending j; stored as fp32 or rounded once to
// bf16.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const int32_t* __restrict__ row_of_slot,
                                                 const float* __restrict__ w, int T, int k,
                                                 int H, void* __restrict__ out) {
  const int t = (int)((blockIdx.x * (unsigned)blockDim.x + threadIdx.x) >> 6);
  if (t >= T) return;
  const int l = lane_id();
  // lane l takes the 4-float chunks l, l + 64, ... of the row, so that every
  // load instruction of the wave reads 1 KiB of one y row contiguously; the
  // first kU rows of the token have all their loads in flight together, any
  // further rows (k > kU) follow one at a time
  const int nv = H / 4;
  constexpr int kU = 8;
  const int ku = min(k, kU);
  int rows[kU];
  float wts[kU];
#pragma unroll
  for (int j = 0; j < kU; ++j) {
    if (j < ku) {
      const int64_t s = (int64_t)t * k + j;
      rows[j] = row_of_slot[s];
      wts[j] = w ? w[s] : 1.0f;
    }
  }
  for (int c = l; c < nv; c += kWave) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 v[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j)
      if (j < ku) v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + (int64_t)rows[j] * H) + c);
#pragma unroll
    for (int j = 0; j < kU; ++j)
      if (j < ku) acc += wts[j] * v[j];
    for (int j = kU; j < k; ++j) {
      const int64_t s = (int64_t)t * k + j;
      const float wj = w ? w[s] : 1.0f;
      acc += wj * reinterpret_cast<const f32x4*>(y + (int64_t)row_of_slot[s] * H)[c];
    }
    if (OUT_F32) {
      reinterpret_cast<f32x4*>(static_cast<float*>(out) + (int64_t)t * H)[c] = acc;
    } else {
      const uint2 o = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (int64_t)t * H)[c] = o;
    }
  }
}

__global__ void k_zero_i32(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, int T, int E, int k, int renorm, int32_t* idx,
                        float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(k_route<1>, grid, block, 0, s, logits, T, E, k, renorm, idx, w);
  else if (E <= 128)
    hipLaunchKernelGGL(k_route<2>, grid, block, 0, s, logits, T, E, k, renorm, idx, w);
  else if (E <= 256)
    hipLaunchKernelGGL(k_route<4>, grid, block, 0, s, logits, T, E, k, renorm, idx, w);
  else if (E <= 512)
    hipLaunchKernelGGL(k_route<8>, grid, block, 0, s, logits, T, E, k, renorm, idx, w);
  else
    hipLaunchKernelGGL(k_route<16>, grid, block, 0, s, logits, T, E, k, renorm, idx, w);
  return hipGetLastError();
}

size_t permute_ws_bytes(int T, int k, int E) {
  const int64_t S = (int64_t)T * k;
  if (S <= kSmallSlots) return 0;
  const int64_t nchunks = (S + kBigChunk - 1) / kBigChunk;
  return align_up((size_t)(nchunks * E) * sizeof(int32_t), 256);
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* slot_of_row, int32_t* row_of_slot, const uint16_t* x,
                          const float* row_scale, int H, uint16_t* x_perm, void* ws,
                          hipStream_t s) {
  const int S = T * k;
  if (S <= kSmallSlots) {
    // every workgroup redoes the (tiny) ranking; at most ~256 workgroups gather
    const int rows_per_wg = x ? max(4, (S + 255) / 256) : max(S, 1);
    const int grid = x ? max(1, (S + rows_per_wg - 1) / rows_per_wg) : 1;
    const size_t lds = (size_t)(E + (E + 1) + 4 * E + kSmallSlots + 256) * sizeof(int);
    hipLaunchKernelGGL(k_permute_small, dim3(grid), dim3(kChunk), lds, s, idx, S, k, E, offsets,
                       slot_of_row, row_of_slot, x, row_scale, H, x_perm, rows_per_wg);
    return hipGetLastError();
  }
  const int nchunks = (S + kBigChunk - 1) / kBigChunk;
  int32_t* counts = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(k_chunk_hist, dim3(nchunks), dim3(kChunk), E * sizeof(int), s, idx, S, E,
                     counts);
  hipLaunchKernelGGL(k_chunk_scatter, dim3(nchunks), dim3(kChunk),
                     (size_t)(E + (E + 1) + E + 4 * E + 256) * sizeof(int), s, idx, S, E,
                     nchunks, counts, offsets, slot_of_row, row_of_slot);
  if (x) {
    hipLaunchKernelGGL(k_gather, dim3((S + 3) / 4), dim3(256), 0, s, x, S, k, H, slot_of_row,
                       row_scale, x_perm);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const float* y, const int32_t* row_of_slot, const float* w, int T,
                          int k, int H, void* out, bool out_f32, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (out_f32)
    hipLaunchKernelGGL(k_combine<true>, dim3((T + 3) / 4), dim3(256), 0, s, y, row_of_slot, w, T,
                       k, H, out);
  else
    hipLaunchKernelGGL(k_combine<false>, dim3((T + 3) / 4), dim3(256), 0, s, y, row_of_slot, w,
                       T, k, H, out);
  return hipGetLastError();
}

}  // namespace moe4
