// Device helpers shared by the kernels of libstdk (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define STDK_DEV __device__ __forceinline__

namespace stdk {

constexpr int kHeadDim = 128;
constexpr int kMaxRanges = 16;
constexpr int kHistBits = 11;              // first radix digit: bits 31..21 of the key
constexpr int kHistBins = 1 << kHistBits;  // 2048

// Position -> row map for the union of up to kMaxRanges half-open ranges.
// Position p lies in range r when pos0[r] <= p < pos0[r+1]; its row is
// row0[r] + (p - pos0[r]).
struct RangeTab {
  int32_t n;
  int32_t pad_;
  int64_t row0[kMaxRanges];
  int64_t pos0[kMaxRanges + 1];
};

// Every table entry is addressed with a compile-time index, so the table is
// read with uniform (scalar) loads; a per-lane index would turn each access
// into a vector load from the kernel-argument segment.
STDK_DEV int64_t pos_to_row(const RangeTab& t, int64_t p) {
  int64_t row0 = t.row0[0], pos0 = t.pos0[0];
#pragma unroll
  for (int i = 1; i < kMaxRanges; ++i) {
    if (i >= t.n) break;
    if (p >= t.pos0[i]) {
      row0 = t.row0[i];
      pos0 = t.pos0[i];
    }
  }
  return row0 + (p - pos0);
}

// Order-preserving map fp32 -> uint32: a > b (as floats) <=> key(a) > key(b).
// -0 is folded onto +0 so that equal floats give equal keys.
STDK_DEV uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

STDK_DEV float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
STDK_DEV float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// DPP row rotate (within each 16-lane row): lane i reads lane (i + n) mod 16.
template <int N>
STDK_DEV float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the same
// bits (each step adds two values that are equal across the paired lanes).
STDK_DEV float row16_sum(float x) {
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  x += row_ror<1>(x);
  return x;
}

// Sum over aligned groups of LPR lanes (16 or 32); all lanes of a group get
// the same bits.
template <int LPR>
STDK_DEV float group_sum(float x) {
  x = row16_sum(x);
  if constexpr (LPR == 32) x += __shfl_xor(x, 16, 64);
  return x;
}

// Value of lane l (the same l in every lane: a constant or a value derived
// from a ballot) in every lane, through a scalar register.
STDK_DEV uint32_t lane_read(uint32_t x, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)x, l); }
STDK_DEV float lane_read(float x, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); }

// Wave reductions (every lane of the wave active): DPP rotations reduce each
// 16-lane row (all lanes of a row end with the same bits), then the four
// rows' values are read through scalar registers and combined in row order,
// so every lane receives the same bits.
template <typename F>
STDK_DEV float wave_reduce(float x, F op) {
  x = op(x, row_ror<8>(x));
  x = op(x, row_ror<4>(x));
  x = op(x, row_ror<2>(x));
  x = op(x, row_ror<1>(x));
  return op(op(lane_read(x, 0), lane_read(x, 16)), op(lane_read(x, 32), lane_read(x, 48)));
}
template <typename F>
STDK_DEV uint32_t wave_reduce_u32(uint32_t x, F op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false));  // row_ror:8
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, false));  // row_ror:4
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x122, 0xF, 0xF, false));  // row_ror:2
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x121, 0xF, 0xF, false));  // row_ror:1
  return op(op(lane_read(x, 0), lane_read(x, 16)), op(lane_read(x, 32), lane_read(x, 48)));
}

STDK_DEV float wave_max(float x) {
  return wave_reduce(x, [](float a, float b) { return fmaxf(a, b); });
}
STDK_DEV float wave_min(float x) {
  return wave_reduce(x, [](float a, float b) { return fminf(a, b); });
}
STDK_DEV float wave_sum(float x) {
  return wave_reduce(x, [](float a, float b) { return a + b; });
}
STDK_DEV uint32_t wave_max_u32(uint32_t x) {
  return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
STDK_DEV uint32_t wave_min_u32(uint32_t x) {
  return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

// Number of set bits of `mask` below this lane.
STDK_DEV uint32_t lane_rank(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifted adds
// inside each 16-lane row, then row broadcasts across rows.
STDK_DEV uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum over the block (NT threads, NT % 64 == 0). `tmp` is
// LDS of at least NT/64 + 1 words. Returns the exclusive prefix; *total gets
// the block sum. Ends with a barrier, so `tmp` may be reused afterwards.
template <int NT>
STDK_DEV uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  if (w == 0) {
    const uint32_t t = (lane < NW) ? tmp[lane] : 0u;
    const uint32_t s = wave_incl_scan(t);
    if (lane < NW) tmp[lane] = s - t;
    if (lane == NW - 1) tmp[NW] = s;
  }
  __syncthreads();
  const uint32_t res = x - v + tmp[w];
  *total = tmp[NW];
  __syncthreads();
  return res;
}

// Exclusive prefix sums of two values over the block in one pass (NT
// threads; `tmp` is LDS of at least 2*NT/64 + 2 words). Ends with a barrier.
template <int NT>
STDK_DEV void block_excl_scan2(uint32_t v0, uint32_t v1, uint32_t* tmp, uint32_t* ex0, uint32_t* ex1,
                               uint32_t* tot0, uint32_t* tot1) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t x0 = wave_incl_scan(v0), x1 = wave_incl_scan(v1);
  if (lane == 63) {
    tmp[w] = x0;
    tmp[NW + 1 + w] = x1;
  }
  __syncthreads();
  if (w == 0) {
    const uint32_t t0 = (lane < NW) ? tmp[lane] : 0u, t1 = (lane < NW) ? tmp[NW + 1 + lane] : 0u;
    const uint32_t s0 = wave_incl_scan(t0), s1 = wave_incl_scan(t1);
    if (lane < NW) {
      tmp[lane] = s0 - t0;
      tmp[NW + 1 + lane] = s1 - t1;
    }
    if (lane == NW - 1) {
      tmp[NW] = s0;
      tmp[2 * NW + 1] = s1;
    }
  }
  __syncthreads();
  *ex0 = x0 - v0 + tmp[w];
  *ex1 = x1 - v1 + tmp[NW + 1 + w];
  *tot0 = tmp[NW];
  *tot1 = tmp[2 * NW + 1];
  __syncthreads();
}

// Radix-bin search over an LDS histogram of `nb` bins.
// DESC: the bin b where the count of strictly higher bins is < need and the
//       count of bins >= b reaches need (the bin holding the need-th largest).
// ASC : the same from the low end (the bin holding the need-th smallest).
// Result in *bin (-1 if the histogram holds fewer than `need` items) and the
// count strictly beyond it in *beyond. Every thread must call it.
template <int NT, bool DESC>
STDK_DEV void find_bin(const uint32_t* hist, int nb, uint32_t need, uint32_t* tmp, int* bin,
                       uint32_t* beyond) {
  const int t = threadIdx.x;
  const int per = (nb + NT - 1) / NT;
  if (t == 0) {
    *bin = -1;
    *beyond = 0;
  }
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) {
    int j = t * per + i;
    if (j < nb) local += hist[DESC ? (nb - 1 - j) : j];
  }
  uint32_t tot;
  uint32_t before = block_excl_scan<NT>(local, tmp, &tot);
  if (before < need && need <= before + local) {
    uint32_t acc = before;
    for (int i = 0; i < per; ++i) {
      int j = t * per + i;
      if (j >= nb) break;
      int b = DESC ? (nb - 1 - j) : j;
      uint32_t h = hist[b];
      if (acc + h >= need) {
        *bin = b;
        *beyond = acc;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
}

// Radix-bin search over an LDS histogram of NB bins by one wave (all 64
// lanes of the calling wave; no barrier inside). Same result as find_bin.
// Lane l owns the NB/64 bins at search ranks [l*NB/64, (l+1)*NB/64) (rank 0
// = the highest bin when DESC); it sums them reading in a lane-rotated order
// (fewer bank conflicts), a wave scan locates the owning lane, and the wave
// then scans that lane's bins together to find the exact one.
template <int NB, bool DESC>
STDK_DEV void find_bin_wave(const uint32_t* hist, uint32_t need, int* bin, uint32_t* beyond) {
  constexpr int PER = NB / 64;
  static_assert(PER >= 1 && PER <= 64 && (PER & (PER - 1)) == 0, "bins per lane");
  const int lane = threadIdx.x & 63;
  auto bin_of = [](int rank) { return DESC ? NB - 1 - rank : rank; };
  uint32_t local = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) local += hist[bin_of(lane * PER + ((k + lane) & (PER - 1)))];
  const uint32_t incl = wave_incl_scan(local);
  const uint32_t before = incl - local;
  const uint64_t own = __ballot(before < need && need <= incl);
  if (own == 0) {  // fewer than `need` items in the histogram
    if (lane == 0) {
      *bin = -1;
      *beyond = 0;
    }
    return;
  }
  const int L = __ffsll((unsigned long long)own) - 1;
  const uint32_t before_L = lane_read(before, L);
  const uint32_t x = lane < PER ? hist[bin_of(L * PER + lane)] : 0u;
  const uint32_t cum = before_L + wave_incl_scan(x);
  const uint64_t hit = __ballot(lane < PER && cum >= need);
  const int k = __ffsll((unsigned long long)hit) - 1;
  if (lane == k) {
    *bin = bin_of(L * PER + k);
    *beyond = cum - x;
  }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Agent-scope (device-wide) relaxed atomic loads and stores: coherent across
// the XCDs, whose L2 caches are not, without a cache-wide fence. Used for
// what one workgroup hands to another inside a kernel; the writer waits
// until its stores are complete before it signals (an atomic counter), and
// the reader issues its loads only after it has seen the signal.
STDK_DEV void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
STDK_DEV uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Thread 0 counts the workgroup in at `counter` once every wave's memory
// accesses are complete; true in every thread of the workgroup that brings
// the count to `total` (which then resets the counter for the next call).
STDK_DEV bool arrive_last(uint32_t* counter, uint32_t total, uint32_t* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t before = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = before + 1 == total ? 1u : 0u;
    if (before + 1 == total) store_agent(counter, 0u);
  }
  __syncthreads();
  return *s_flag != 0u;
}

STDK_DEV u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
STDK_DEV bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Splits 8 fp32 values into bf16 values (rounded to nearest even by the
// hardware conversion) and bf16 remainders, packed two per word in element
// order (element 2i in the low half of word i). The remainder x - hi is exact
// in fp32, so x = hi + lo + r with |r| <= 2^-17 |x|.
STDK_DEV void split_bf16x8(const float (&x)[8], u32x4& hi, u32x4& lo) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2 * i], x[2 * i + 1]}, bf16x2));
    const float r0 = x[2 * i] - __uint_as_float(hb << 16);
    const float r1 = x[2 * i + 1] - __uint_as_float(hb & 0xFFFF0000u);
    hw[i] = hb;
    lw[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
  }
  hi = u32x4{hw[0], hw[1], hw[2], hw[3]};
  lo = u32x4{lw[0], lw[1], lw[2], lw[3]};
}

// Splits 8 fp32 values into three bf16 parts, x = hi + mid + lo + r: each
// part is the bf16 rounding of what the earlier parts leave (an exact fp32
// difference), so the three carry all 24 bits of an fp32 significand and
// |r| <= 2^-27 |x|.
STDK_DEV void split3_bf16x8(const float (&x)[8], u32x4& hi, u32x4& mid, u32x4& lo) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  uint32_t w[3][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float r0 = x[2 * i], r1 = x[2 * i + 1];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
      w[k][i] = hb;
      r0 -= __uint_as_float(hb << 16);
      r1 -= __uint_as_float(hb & 0xFFFF0000u);
    }
  }
  hi = u32x4{w[0][0], w[0][1], w[0][2], w[0][3]};
  mid = u32x4{w[1][0], w[1][1], w[1][2], w[1][3]};
  lo = u32x4{w[2][0], w[2][1], w[2][2], w[2][3]};
}

}  // namespace stdk
