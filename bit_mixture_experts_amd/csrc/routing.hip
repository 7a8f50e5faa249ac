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

// Selection order: larger logit first, then lower expert index; +0 == -0.
// Each candidate becomes one 64-bit key that is unique and ordered the same
// way: the logit's bits mapped to an unsigned order (negative values have all
// bits flipped, the others get the sign bit set; -0 is taken as +0), then the
// inverted expert index. NaN maps to the lowest value (order 0), so the k
// chosen experts are always distinct and in range. Key 0 marks a lane slot
// with no candidate (past E, or already chosen).
__device__ __forceinline__ uint64_t select_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  if (v != v) o = 0u;
  return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)e;
}
// The logit a key was made from (-0 comes back as +0, NaN as a NaN).
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// DPP move of a 64-bit value inside each row of 16 lanes (CTRL as in
// v_mov_b32_dpp: quad_perm, row_half_mirror, row_mirror).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)x, (int)(uint32_t)x, CTRL, 0xF, 0xF,
                                             false);
  const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(x >> 32), (int)(uint32_t)(x >> 32),
                                             CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Maximum over the wave, returned in every lane (the whole wave active):
// lanes xor 1 and 2 by quad permutes, xor 4 and 8 by the half-row and row
// mirrors, then rows pairwise by v_permlane16_swap and halves by
// v_permlane32_swap; no LDS round trip.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = max_u64(x, dpp_u64<0xB1>(x));   // quad_perm [1,0,3,2]
  x = max_u64(x, dpp_u64<0x4E>(x));   // quad_perm [2,3,0,1]
  x = max_u64(x, dpp_u64<0x141>(x));  // row_half_mirror
  x = max_u64(x, dpp_u64<0x140>(x));  // row_mirror
  {
    const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
    const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    x = max_u64(((uint64_t)b[0] << 32) | a[0], ((uint64_t)b[1] << 32) | a[1]);
  }
  {
    const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
    const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    x = max_u64(((uint64_t)b[0] << 32) | a[0], ((uint64_t)b[1] << 32) | a[1]);
  }
  return x;
}

// Sum over the wave, in every lane, by the exchange pattern of wave_max_u64
// (every lane adds the same pairs in the same tree, so all lanes agree bit
// for bit).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  return x;
}

// Routing of one token by one wave (all 64 lanes active); lane l holds
// experts l, l+64, ... (NPL per lane). The k chosen experts and their weights
// go to idx[0..k) and w[0..k) (device or LDS memory). Each of the k picks is
// one wave-wide maximum of the remaining keys; the owner lane then clears the
// chosen key.
template <int NPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k,
                                            int renorm, int32_t* idx, float* wout) {
  const int l = lane_id();
  float v[NPL];
  float selv[NPL];
  uint64_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = l + kWave * i;
    v[i] = 0.0f;
    selv[i] = 0.0f;
    key[i] = 0;
    if (e < E) {
      v[i] = row[e];
      key[i] = select_key(v[i], e);
    }
  }
  float top = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < NPL; ++i) best = max_u64(best, key[i]);
    best = wave_max_u64(best);
    // the same in every lane: take it into scalar registers
    const uint32_t be = ~(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)best);
    const float bv = key_value(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(
                                    (int)(uint32_t)(best >> 32)))
                               << 32);
    if (j == 0) top = bv;
    if ((int)(be & (kWave - 1)) == l) {
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (i == (int)(be / kWave)) key[i] = 0;
    }
    if ((j & (kWave - 1)) == l) {
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (i == j / kWave) selv[i] = bv;
      idx[j] = (int32_t)be;
    }
  }
  // weights: exp(v - top) normalised over the selection or over all experts
  float part = 0.0f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    if (renorm) {
      const int j = l + kWave * i;
      if (j < k) part += expf(selv[i] - top);
    } else if (l + kWave * i < E) {
      part += expf(v[i] - top);
    }
  }
  const float denom = wave_sum_dpp(part);
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = l + kWave * i;
    if (j < k) wout[j] = expf(selv[i] - top) / denom;
  }
}

// One wave per token.
template <int NPL>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E,
                                               int k, int renorm, int32_t* __restrict__ idx,
                                               float* __restrict__ wout) {
  const int t = (int)((blockIdx.x * (unsigned)blockDim.x + threadIdx.x) >> 6);
  if (t >= T) return;
  route_token<NPL>(logits + (int64_t)t * E, E, k, renorm, idx + (int64_t)t * k,
                   wout + (int64_t)t * k);
}

// --------------------------------------------------------------- permutation

constexpr int kChunk = 256;        // slots ranked per pass (one per thread)
constexpr int kSmallSlots = 1024;  // single-kernel path up to this many slots
// slots per workgroup in the multi-kernel path: 512 up to 64K slots (64 or
// more workgroups at the Qwen3 prefill shape; 2048 took 1% longer per layer
// step there), 2048 beyond (every scatter workgroup sums all chunks' counts,
// so the work grows with the square of the chunk count)
__host__ __device__ constexpr int big_chunk(int64_t S) { return S <= 65536 ? 512 : 2048; }

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
// workgroup gathers its share of rows. One launch. `idx` is device or LDS
// memory; `lds` holds (6 E + 1 + kSmallSlots + 256) ints.
__device__ __forceinline__ void permute_small(
    const int32_t* idx, int S, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_of_row, int32_t* __restrict__ row_of_slot,
    const uint16_t* __restrict__ x, const float* __restrict__ row_scale, int H,
    uint16_t* __restrict__ x_perm, int rows_per_wg, int* lds) {
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

__global__ __launch_bounds__(kChunk) void k_permute_small(
    const int32_t* __restrict__ idx, int S, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_of_row, int32_t* __restrict__ row_of_slot,
    const uint16_t* __restrict__ x, const float* __restrict__ row_scale, int H,
    uint16_t* __restrict__ x_perm, int rows_per_wg) {
  extern __shared__ int lds[];
  permute_small(idx, S, k, E, offsets, slot_of_row, row_of_slot, x, row_scale, H, x_perm,
                rows_per_wg, lds);
}

// Routing and permutation of a small batch in one launch: every workgroup
// routes all T tokens into LDS (its waves take the tokens in turn), workgroup
// 0 writes the routing arrays, then the permutation and gather proceed as in
// k_permute_small from the LDS copy of the chosen experts.
// tokens up to which routing is fused: one per wave (with more, each wave
// routes several tokens in turn, and a batch of 16 measured slower fused)
constexpr int kFusedTokens = kChunk / kWave;
template <int NPL>
__global__ __launch_bounds__(kChunk) void k_route_permute_small(
    const float* __restrict__ logits, int T, int E, int k, int renorm,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_of_row, int32_t* __restrict__ row_of_slot,
    const uint16_t* __restrict__ x, int H, uint16_t* __restrict__ x_perm, int rows_per_wg) {
  extern __shared__ int lds[];
  int32_t* sidx = lds;                                        // [kSmallSlots]
  float* sw = reinterpret_cast<float*>(lds + kSmallSlots);    // [kSmallSlots]
  const int S = T * k;
  for (int t = wave_id(); t < T; t += kChunk / kWave)
    route_token<NPL>(logits + (int64_t)t * E, E, k, renorm, sidx + t * k, sw + t * k);
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int s = threadIdx.x; s < S; s += kChunk) {
      idx_out[s] = sidx[s];
      w_out[s] = sw[s];
    }
  }
  permute_small(sidx, S, k, E, offsets, slot_of_row, row_of_slot, x, nullptr, H, x_perm,
                rows_per_wg, lds + 2 * kSmallSlots);
}

// Large problems, pass 1: per-chunk expert counts, counts[c * E + e], one
// workgroup per chunk of big_chunk(S) slots.
__global__ __launch_bounds__(kChunk) void k_chunk_hist(const int32_t* __restrict__ idx, int S,
                                                       int E, int32_t* __restrict__ counts) {
  const int chunk = big_chunk(S);
  extern __shared__ int cnt[];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kChunk) cnt[e] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * chunk;
  const int s1 = min(S, s0 + chunk);
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
  const int s0 = c * big_chunk(S);
  const int s1 = min(S, s0 + big_chunk(S));
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

// Pass 4: gather rows (one wave per row). A slot outside [0, S) (only from a
// caller's slot_of_row) gives a zero row.
__global__ __launch_bounds__(256) void k_gather(const uint16_t* __restrict__ x, int S, int k,
                                                int H, const int32_t* __restrict__ slot_of_row,
                                                const float* __restrict__ row_scale,
                                                uint16_t* __restrict__ x_perm) {
  const int r = (int)((blockIdx.x * (unsigned)blockDim.x + threadIdx.x) >> 6);
  if (r >= S) return;
  const int s = slot_of_row[r];
  if ((unsigned)s >= (unsigned)S) {
    u32x4* d = reinterpret_cast<u32x4*>(x_perm + (int64_t)r * H);
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int c = lane_id(); c < H / 8; c += kWave) d[c] = z;
    return;
  }
  copy_row(x, s / k, H, row_scale, s, x_perm + (int64_t)r * H);
}

// Routing and permutation of at most 64 slots (a decode step of a few tokens)
// without the row gather, by one workgroup and a single barrier: wave t routes
// token t into LDS; then every slot's row is counted directly (slots of a
// smaller expert, plus earlier slots of the same expert) and so is every
// expert's offset (slots of a smaller expert), each thread reading the
// expert list from LDS. No scan, atomics or cleared counters.
constexpr int kTinySlots = 64;
template <int NPL>
__global__ __launch_bounds__(kChunk) void k_route_permute_tiny(
    const float* __restrict__ logits, int T, int E, int k, int renorm,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_of_row, int32_t* __restrict__ row_of_slot) {
  __shared__ int32_t sidx[kTinySlots];
  __shared__ float sw[kTinySlots];
  const int w = wave_id(), tid = threadIdx.x;
  if (w < T) route_token<NPL>(logits + (int64_t)w * E, E, k, renorm, sidx + w * k, sw + w * k);
  __syncthreads();
  const int S = T * k;
  if (tid < S) {
    const int e = sidx[tid];
    int row = 0;
    for (int s = 0; s < S; ++s) {
      const int o = sidx[s];
      row += (o < e) | ((o == e) & (s < tid));
    }
    idx_out[tid] = e;
    w_out[tid] = sw[tid];
    slot_of_row[row] = tid;
    row_of_slot[tid] = row;
  }
  for (int e = tid; e <= E; e += kChunk) {
    int n = 0;
    for (int s = 0; s < S; ++s) n += sidx[s] < e;
    offsets[e] = n;
  }
}

// ------------------------------------------------------------------ combine

// out[t] = sum_j w[t,j] * y[row_of_slot[t*k+j]] over fp32 rows, accumulated
// in fp32 in ascending j; stored as fp32 or rounded once to bf16. wpt waves per
// token; wave q of a token takes the 4-float chunks q * 64 + l, stepping by
// wpt * 64 (lane l), so that every load instruction reads 1 KiB of one y row
// contiguously. A large batch runs one wave per token (each wave walks its
// row); a decode-sized batch spreads a token's row over up to H / 256 waves
// (one wave per token would walk its row in dependent round trips). The first
// kU rows of the token have their loads in flight together; any further rows
// (k > kU) follow one at a time.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const int32_t* __restrict__ row_of_slot,
                                                 const float* __restrict__ w, int T, int k,
                                                 int H, int wpt, void* __restrict__ out) {
  const int gw = (int)((blockIdx.x * (unsigned)blockDim.x + threadIdx.x) >> 6);
  const int t = gw / wpt;
  if (t >= T) return;
  const int q = gw - t * wpt;
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
  for (int c = q * kWave + lane_id(); c < nv; c += wpt * kWave) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 v[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j)
      if (j < ku)
        v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + (int64_t)rows[j] * H) + c);
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
  const int64_t nchunks = (S + big_chunk(S) - 1) / big_chunk(S);
  return align_up((size_t)(nchunks * E) * sizeof(int32_t), 256);
}

hipError_t launch_gather(const uint16_t* x, int T, int k, int H, const int32_t* slot_of_row,
                         const float* row_scale, uint16_t* x_perm, hipStream_t s) {
  const int S = T * k;
  if (S == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather, dim3((S + 3) / 4), dim3(256), 0, s, x, S, k, H, slot_of_row,
                     row_scale, x_perm);
  return hipGetLastError();
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
  const int nchunks = (S + big_chunk(S) - 1) / big_chunk(S);
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

hipError_t launch_route_permute(const float* logits, int T, int E, int k, int renorm,
                                int32_t* idx, float* w, int32_t* offsets, int32_t* slot_of_row,
                                int32_t* row_of_slot, const uint16_t* x, int H,
                                uint16_t* x_perm, void* ws, hipStream_t s) {
  const int S = T * k;
  if (x == nullptr && S <= kTinySlots && T <= kFusedTokens) {
    const dim3 g(1), b(kChunk);
    if (E <= 64)
      hipLaunchKernelGGL(k_route_permute_tiny<1>, g, b, 0, s, logits, T, E, k, renorm, idx, w,
                         offsets, slot_of_row, row_of_slot);
    else if (E <= 128)
      hipLaunchKernelGGL(k_route_permute_tiny<2>, g, b, 0, s, logits, T, E, k, renorm, idx, w,
                         offsets, slot_of_row, row_of_slot);
    else if (E <= 256)
      hipLaunchKernelGGL(k_route_permute_tiny<4>, g, b, 0, s, logits, T, E, k, renorm, idx, w,
                         offsets, slot_of_row, row_of_slot);
    else if (E <= 512)
      hipLaunchKernelGGL(k_route_permute_tiny<8>, g, b, 0, s, logits, T, E, k, renorm, idx, w,
                         offsets, slot_of_row, row_of_slot);
    else
      hipLaunchKernelGGL(k_route_permute_tiny<16>, g, b, 0, s, logits, T, E, k, renorm, idx, w,
                         offsets, slot_of_row, row_of_slot);
    return hipGetLastError();
  }
  if (S > kSmallSlots || T > kFusedTokens) {
    hipError_t err = launch_route(logits, T, E, k, renorm, idx, w, s);
    if (err != hipSuccess) return err;
    return launch_permute(idx, T, k, E, offsets, slot_of_row, row_of_slot, x, nullptr, H, x_perm,
                          ws, s);
  }
  const int rows_per_wg = x ? max(4, (S + 255) / 256) : max(S, 1);
  const int grid = x ? max(1, (S + rows_per_wg - 1) / rows_per_wg) : 1;
  const size_t lds =
      (size_t)(2 * kSmallSlots + E + (E + 1) + 4 * E + kSmallSlots + 256) * sizeof(int);
  const dim3 g(grid), b(kChunk);
  if (E <= 64)
    hipLaunchKernelGGL(k_route_permute_small<1>, g, b, lds, s, logits, T, E, k, renorm, idx, w,
                       offsets, slot_of_row, row_of_slot, x, H, x_perm, rows_per_wg);
  else if (E <= 128)
    hipLaunchKernelGGL(k_route_permute_small<2>, g, b, lds, s, logits, T, E, k, renorm, idx, w,
                       offsets, slot_of_row, row_of_slot, x, H, x_perm, rows_per_wg);
  else if (E <= 256)
    hipLaunchKernelGGL(k_route_permute_small<4>, g, b, lds, s, logits, T, E, k, renorm, idx, w,
                       offsets, slot_of_row, row_of_slot, x, H, x_perm, rows_per_wg);
  else if (E <= 512)
    hipLaunchKernelGGL(k_route_permute_small<8>, g, b, lds, s, logits, T, E, k, renorm, idx, w,
                       offsets, slot_of_row, row_of_slot, x, H, x_perm, rows_per_wg);
  else
    hipLaunchKernelGGL(k_route_permute_small<16>, g, b, lds, s, logits, T, E, k, renorm, idx, w,
                       offsets, slot_of_row, row_of_slot, x, H, x_perm, rows_per_wg);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y, const int32_t* row_of_slot, const float* w, int T,
                          int k, int H, void* out, bool out_f32, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // waves per token: enough waves for about 4096 in all, at most one per 256
  // columns (a batch of 4096 tokens runs one wave per token)
  const int npiece = (H / 4 + kWave - 1) / kWave;
  const int wpt = max(1, min(npiece, 4096 / T));
  const int64_t waves = (int64_t)T * wpt;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (out_f32)
    hipLaunchKernelGGL(k_combine<true>, grid, dim3(256), 0, s, y, row_of_slot, w, T, k, H, wpt,
                       out);
  else
    hipLaunchKernelGGL(k_combine<false>, grid, dim3(256), 0, s, y, row_of_slot, w, T, k, H, wpt,
                       out);
  return hipGetLastError();
}

}  // namespace moe4
