// Device-side helpers shared by the moe4 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Raw buffer resources: a load whose byte offset is at or past the resource's
// size returns zeros, which takes the place of per-lane bounds branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kOob = 0x7FFFFFF0;   // offset past the end of any resource used here
// cache-policy operand of the raw buffer builtins: the non-temporal bit
constexpr int kCpolNt = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: 32-bit data format, no swizzle (gfx9 family)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// make_rsrc for a base and size that are wave-uniform by construction, said so
// to the compiler (else it may keep the resource in vector registers and wrap
// every access in a loop over its distinct values)
__device__ __forceinline__ rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                   __builtin_amdgcn_readfirstlane(bytes));
}
__device__ __forceinline__ u32x4 buf_load_b128(rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load_b32(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_u8(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// two fp32 -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
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

// Integer sum over the wave, in every lane (the whole wave active): lanes
// xor 1 and 2 by quad permutes, xor 4 and 8 by the half-row and row mirrors
// (DPP), then rows pairwise by v_permlane16_swap and halves by
// v_permlane32_swap; no LDS round trip.
__device__ __forceinline__ int wave_sum_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  x = (int)(a[0] + a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return (int)(b[0] + b[1]);
}

// Inclusive prefix sum over the wave (the whole wave active): Hillis-Steele
// steps inside each 16-lane row by DPP row shifts (lanes shifted in from
// outside the row add zero), then the totals of the rows below, read from
// lanes 15, 31 and 47. The same result as wave_inclusive_scan without its
// six LDS permutes.
__device__ __forceinline__ int wave_scan_dpp(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int l = lane_id();
  return x + (l >= 16 ? r0 : 0) + (l >= 32 ? r1 : 0) + (l >= 48 ? r2 : 0);
}

// fp32(fp32(a * b) + c): one rounded product, one rounded sum; the pragma
// keeps the compiler from contracting the pair into a fused multiply-add
__device__ __forceinline__ float mul_then_add(float a, float b, float c) {
#pragma clang fp contract(off)
  return a * b + c;
}

// logistic function; v_exp_f32 and v_rcp_f32 (about 1 ulp each)
__device__ __forceinline__ float sigmoidf_(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Locate work item q when expert e owns units(n_e) consecutive items
// (n_e = offsets[e+1] - offsets[e]). Every lane of the wave gets the same
// answer: e = -1 when q is past the last item, else the expert, the item's
// index inside it and the expert's row range [beg, end) = [offsets[e],
// offsets[e+1]). Offsets are read once per lane (a contiguous chunk).
template <typename Units>
__device__ __forceinline__ void locate_item(const int32_t* __restrict__ offsets, int E, int q,
                                            Units units, int& e_out, int& u_out, int& beg_out,
                                            int& end_out) {
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
  int incl = wave_scan_dpp(cnt);
  int excl = incl - cnt;
  bool own = (q >= excl) && (q < incl);
  unsigned long long b = __ballot(own);
  if (b == 0ull) {
    e_out = -1;
    u_out = 0;
    beg_out = end_out = 0;
    return;
  }
  int owner = __ffsll((long long)b) - 1;
  int ef = -1, uf = 0, bf = 0, nf = 0;
  if (own) {
    int acc = excl;
    int prev = offsets[e0];
    for (int i = 0; i < per && e0 + i < E; ++i) {
      int nx = offsets[e0 + i + 1];
      int u = units(nx - prev);
      if (q < acc + u) {
        ef = e0 + i;
        uf = q - acc;
        bf = prev;
        nf = nx;
        break;
      }
      acc += u;
      prev = nx;
    }
  }
  e_out = __builtin_amdgcn_readlane(ef, owner);
  u_out = __builtin_amdgcn_readlane(uf, owner);
  beg_out = __builtin_amdgcn_readlane(bf, owner);
  end_out = __builtin_amdgcn_readlane(nf, owner);
}
// locate_item for E <= 64 * PER: each lane reads its PER + 1 offsets as one
// batch of loads (no dependent round trips), keeps them in registers for the
// second pass, and the answer is the same.
template <int PER, typename Units>
__device__ __forceinline__ void locate_item_batched(const int32_t* __restrict__ offsets, int E,
                                                    int q, Units units, int& e_out, int& u_out,
                                                    int& beg_out, int& end_out) {
  const int l = lane_id();
  const int e0 = l * PER;
  const rsrc_t ro = make_rsrc(offsets, (uint32_t)(E + 1) * 4);
  int o[PER + 1];
#pragma unroll
  for (int i = 0; i <= PER; ++i) o[i] = (int)buf_load_b32(ro, e0 + i <= E ? 4 * (e0 + i) : kOob);
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (e0 + i < E) cnt += units(o[i + 1] - o[i]);
  const int incl = wave_scan_dpp(cnt);
  const int excl = incl - cnt;
  const bool own = (q >= excl) && (q < incl);
  const unsigned long long b = __ballot(own);
  if (b == 0ull) {
    e_out = -1;
    u_out = 0;
    beg_out = end_out = 0;
    return;
  }
  const int owner = __ffsll((long long)b) - 1;
  int ef = -1, uf = 0, bf = 0, nf = 0;
  if (own) {
    int acc = excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (e0 + i < E) {
        const int u = units(o[i + 1] - o[i]);
        if (ef < 0 && q < acc + u) {
          ef = e0 + i;
          uf = q - acc;
          bf = o[i];
          nf = o[i + 1];
        }
        acc += u;
      }
    }
  }
  e_out = __builtin_amdgcn_readlane(ef, owner);
  u_out = __builtin_amdgcn_readlane(uf, owner);
  beg_out = __builtin_amdgcn_readlane(bf, owner);
  end_out = __builtin_amdgcn_readlane(nf, owner);
}
template <typename Units>
__device__ __forceinline__ void locate_item(const int32_t* __restrict__ offsets, int E, int q,
                                            Units units, int& e_out, int& u_out) {
  int beg, end;
  locate_item(offsets, E, q, units, e_out, u_out, beg, end);
}

// Work item of workgroup b in a grouped GEMM whose experts are cut into BM-row
// tiles, each tile split into ncg column groups. Items are (tile, column
// group) pairs, column group fastest. The dispatcher deals workgroup ids
// round-robin over the 8 XCDs (each with its own L2) and in id order within
// one: XCD x gets a contiguous 1/8 of the full-tile items, then a contiguous
// 1/8 of the partial-tile items (each expert's last, short tile). Items that
// share an activation tile or an expert's weights stay on one XCD, and the
// cheap partial tiles come last everywhere. The grid needs at least
// (full + partial tiles) * ncg + 16 workgroups; the rest get e = -1.
template <int BM>
__device__ __forceinline__ void locate_tile_xcd(const int32_t* __restrict__ offsets, int E,
                                                int ncg, int b, int& e_out, int& u_out,
                                                int& cg_out) {
  constexpr int kXcd = 8;
  const int l = lane_id();
  const int per = (E + kWave - 1) / kWave;
  const int e0 = l * per;
  int nf = 0, nr = 0;
  if (e0 < E) {
    int prev = offsets[e0];
    for (int i = 0; i < per && e0 + i < E; ++i) {
      const int nx = offsets[e0 + i + 1];
      nf += (nx - prev) / BM;
      nr += (nx - prev) % BM ? 1 : 0;
      prev = nx;
    }
  }
  const int NF = wave_sum_i32(nf) * ncg;
  const int NR = wave_sum_i32(nr) * ncg;
  const int x = b % kXcd, i = b / kXcd;
  const int f0 = (int)((int64_t)NF * x / kXcd), f1 = (int)((int64_t)NF * (x + 1) / kXcd);
  const int r0 = (int)((int64_t)NR * x / kXcd), r1 = (int)((int64_t)NR * (x + 1) / kXcd);
  int item, e = -1, u = 0;
  if (i < f1 - f0) {
    item = f0 + i;
    locate_item(offsets, E, item / ncg, [](int n) { return n / BM; }, e, u);
  } else if (i < (f1 - f0) + (r1 - r0)) {
    item = r0 + (i - (f1 - f0));
    int unused;
    locate_item(offsets, E, item / ncg, [](int n) { return n % BM ? 1 : 0; }, e, unused);
    if (e >= 0) u = (offsets[e + 1] - offsets[e]) / BM;
  } else {
    item = 0;
  }
  e_out = e;
  u_out = u;
  cg_out = item % ncg;
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

// ---------------------------------------------------------------- LDS-DMA

#define MOE4_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// wait until at most N vector-memory loads of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// wait for every LDS access of this wave (vector-memory loads untouched)
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}
// workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding LDS-DMA load); compiler-level ordering only
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------ equal-split row tiles

// Row tiles of an expert with n rows: ceil(n / BM) tiles of R rows each (R a
// multiple of 32), the last one shorter.
template <int BM>
__device__ __forceinline__ int eq_tiles(int n) { return (n + BM - 1) / BM; }
template <int BM>
__device__ __forceinline__ int eq_tile_rows(int n) {
  const int nt = eq_tiles<BM>(n);
  return nt ? ((n + nt - 1) / nt + 31) / 32 * 32 : 0;
}

// Work item of workgroup b: (expert e, row tile u, column group cg). Items are
// (tile, column group) pairs, column group fastest, experts in order. The
// dispatcher deals workgroup ids round-robin over the 8 XCDs (each with its
// own L2); XCD x gets a contiguous 1/8 of the items, so the column groups of
// one tile (which share its activation rows) and the tiles of one expert
// (which share its weights) stay on one XCD. The grid needs at least
// items + 8 workgroups; the rest get e = -1.
template <int BM>
__device__ __forceinline__ void locate_tile_eq(const int32_t* __restrict__ offsets, int E,
                                               int ncg, int b, int& e_out, int& u_out,
                                               int& cg_out) {
  constexpr int kXcd = 8;
  const int l = lane_id();
  const int per = (E + kWave - 1) / kWave;
  const int e0 = l * per;
  int nt = 0;
  if (e0 < E) {
    int prev = offsets[e0];
    for (int i = 0; i < per && e0 + i < E; ++i) {
      const int nx = offsets[e0 + i + 1];
      nt += eq_tiles<BM>(nx - prev);
      prev = nx;
    }
  }
  const int N = wave_sum_i32(nt) * ncg;
  const int x = b % kXcd, i = b / kXcd;
  const int f0 = (int)((int64_t)N * x / kXcd), f1 = (int)((int64_t)N * (x + 1) / kXcd);
  int e = -1, u = 0, item = 0;
  if (i < f1 - f0) {
    item = f0 + i;
    locate_item(offsets, E, item / ncg, [](int n) { return eq_tiles<BM>(n); }, e, u);
  }
  e_out = e;
  u_out = u;
  cg_out = item % ncg;
}

// Row-tile count (32-row MFMA tiles) of tile u of an expert with n rows.
template <int BM>
__device__ __forceinline__ int eq_tile_nrt(int n, int u) {
  const int nt = eq_tiles<BM>(n), R = eq_tile_rows<BM>(n);
  const int rows = u < nt - 1 ? R : n - (nt - 1) * R;
  return (rows + 31) >> 5;
}

// As locate_tile_eq, with the tiles dealt largest first: tiles are ordered by
// their count of 32-row MFMA tiles (descending; experts in order within a
// count), tile j of that order goes to XCD j % 8, and each XCD takes its tiles
// in order, column group fastest. The dispatcher starts workgroups in id order,
// so every XCD starts its largest tiles first and fills in with the small ones
// (longest-first list scheduling). The grid needs (tiles + 7) * ncg
// workgroups; the rest get e = -1.
template <int BM, int PER>
__device__ __forceinline__ void locate_tile_sorted_p(const int32_t* __restrict__ offsets, int E,
                                                     int ncg, int b, int& e_out, int& u_out,
                                                     int& cg_out, int& beg_out, int& end_out) {
  constexpr int kXcd = 8, kC = BM / 32;
  const int l = lane_id();
  const int e0 = l * PER;
  // lane l owns experts [e0, e0 + PER): its PER + 1 offsets go out as one
  // batch of loads (a single round trip) and both passes below run on them
  const rsrc_t ro = make_rsrc(offsets, (uint32_t)(E + 1) * 4);
  int o[PER + 1];
#pragma unroll
  for (int i = 0; i <= PER; ++i) o[i] = (int)buf_load_b32(ro, e0 + i <= E ? 4 * (e0 + i) : kOob);
  // per expert: tile count, and the classes (row-tile counts) of its first
  // and last tile; an expert's tiles are all of the first class but the last
  int nt[PER], cf[PER], cl[PER];
  int cnt[kC];
#pragma unroll
  for (int c = 0; c < kC; ++c) cnt[c] = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int n = e0 + i < E ? o[i + 1] - o[i] : 0;
    nt[i] = eq_tiles<BM>(n);
    cf[i] = nt[i] ? eq_tile_nrt<BM>(n, 0) : 0;
    cl[i] = nt[i] ? eq_tile_nrt<BM>(n, nt[i] - 1) : 0;
#pragma unroll
    for (int c = 0; c < kC; ++c) cnt[c] += (cf[i] == c + 1 ? nt[i] - 1 : 0) + (cl[i] == c + 1 ? 1 : 0);
  }
  const int x = b % kXcd, i = b / kXcd;
  const int j = (i / ncg) * kXcd + x;   // position in the largest-first order
  cg_out = i % ncg;
  e_out = -1;
  u_out = 0;
  beg_out = end_out = 0;
  int before = 0;
#pragma unroll
  for (int c = kC - 1; c >= 0; --c) {
    const int tot = wave_sum_i32(cnt[c]);
    if (j >= before && j < before + tot) {
      // the k-th tile of class C, experts in order: find the lane whose
      // experts hold it, then the expert within the lane
      const int k = j - before, C = c + 1;
      const int mine = cnt[c];
      const int incl = wave_scan_dpp(mine), excl = incl - mine;
      const bool own = k >= excl && k < incl;
      const unsigned long long bl = __ballot(own);
      const int owner = __ffsll((long long)bl) - 1;   // bl != 0: k < tot
      int ef = -1, uf = 0, bf = 0, nf = 0, acc = excl;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int nfull = cf[q] == C ? nt[q] - 1 : 0;
        const int u = nfull + (cl[q] == C ? 1 : 0);
        if (ef < 0 && k < acc + u) {
          ef = e0 + q;
          uf = k - acc < nfull ? k - acc : nt[q] - 1;
          bf = o[q];
          nf = o[q + 1];
        }
        acc += u;
      }
      e_out = __builtin_amdgcn_readlane(ef, owner);
      u_out = __builtin_amdgcn_readlane(uf, owner);
      beg_out = __builtin_amdgcn_readlane(bf, owner);
      end_out = __builtin_amdgcn_readlane(nf, owner);
      return;
    }
    before += tot;
  }
}

// beg_out/end_out: offsets[e] and offsets[e + 1] of the expert found (the
// locator holds them already; zero when there is none)
template <int BM>
__device__ __forceinline__ void locate_tile_sorted(const int32_t* __restrict__ offsets, int E,
                                                   int ncg, int b, int& e_out, int& u_out,
                                                   int& cg_out, int& beg_out, int& end_out) {
  // experts per lane, rounded up to a power of two (E <= 1024)
  const int per = (E + kWave - 1) / kWave;
#define MOE4_LOCATE(P) \
  locate_tile_sorted_p<BM, P>(offsets, E, ncg, b, e_out, u_out, cg_out, beg_out, end_out)
  if (per <= 1) MOE4_LOCATE(1);
  else if (per <= 2) MOE4_LOCATE(2);
  else if (per <= 4) MOE4_LOCATE(4);
  else if (per <= 8) MOE4_LOCATE(8);
  else MOE4_LOCATE(16);
#undef MOE4_LOCATE
}

}  // namespace moe4
