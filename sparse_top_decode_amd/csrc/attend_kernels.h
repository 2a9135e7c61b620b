// Renormalised softmax . V over a row set, and the log-sum-exp combination.
//
// Both follow the RetrievalAttention review: Eq. 2 ("Approximated Attention
// Formulation": softmax over the chosen subset only) written with a local
// maximum as in "CPU-GPU Co-Execution Architecture" (o_W, o_Omega), and the
// rescaled combination of Eq. 4-5 (gamma_j = e^{lse_j - lse}). Work is split
// over several workgroups per head; each produces (m, s, sum e^{z-m} v) for
// its rows and a combine kernel merges them in a fixed order with the same
// rescaling, so the result does not depend on timing.
#pragma once

#include "device.h"
#include "scan_kernels.h"

namespace stdk {

constexpr int kPartStride = 132;  // m, s, pad, pad, o[128]

// Combines `np` partials (m, s, o) starting at `part` into o_out[128] and
// *lse_out, in partial order. Runs on a block of kHeadDim threads; `sm` and
// `sf` are LDS scratch of np floats each (np <= kMaxPartials).
constexpr int kMaxPartials = 1024;

STDK_DEV void combine_partials(const float* part, int np, float* o_out, float* lse_out, float* sm, float* sf,
                               float* red) {
  const int j = threadIdx.x;
  // this thread's output element of the first partials, requested together
  // with the (m, s) pairs so that one memory round trip serves both
  constexpr int PB = 64;
  float ov[PB];
#pragma unroll
  for (int i = 0; i < PB; ++i) ov[i] = part[(int64_t)min(i, np - 1) * kPartStride + 4 + j];
  for (int i = j; i < np; i += kHeadDim) {
    sm[i] = part[(int64_t)i * kPartStride];
    sf[i] = part[(int64_t)i * kPartStride + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int i = j; i < np; i += kHeadDim) M = fmaxf(M, sm[i]);
  M = wave_max(M);
  if ((j & 63) == 0) red[j >> 6] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  __syncthreads();
  // weights e^{m_i - M} (0 for an empty partial); the sums run in partial
  // order. A NaN score reaches S and O through its partial and propagates.
  for (int i = j; i < np; i += kHeadDim) sm[i] = (sm[i] == -INFINITY) ? 0.f : __expf(sm[i] - M);
  __syncthreads();
  float S = 0.f, O = 0.f;
#pragma unroll
  for (int i = 0; i < PB; ++i) {
    if (i < np) {
      const float f = sm[i];
      S = fmaf(sf[i], f, S);
      O = fmaf(ov[i], f, O);
    }
  }
  for (int i0 = PB; i0 < np; i0 += PB) {
#pragma unroll
    for (int i = 0; i < PB; ++i) ov[i] = part[(int64_t)min(i0 + i, np - 1) * kPartStride + 4 + j];
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      if (i0 + i < np) {
        const float f = sm[i0 + i];
        S = fmaf(sf[i0 + i], f, S);
        O = fmaf(ov[i], f, O);
      }
    }
  }
  if (S == 0.f) {  // no row: o = 0, lse = -inf
    o_out[j] = 0.f;
    if (j == 0) *lse_out = -INFINITY;
  } else {
    o_out[j] = O / S;
    if (j == 0) *lse_out = M + __logf(S);
  }
}

// Combines the per-workgroup partials of every segment (one workgroup per
// segment; the kernel boundary makes the partials visible).
struct CombineArgs {
  const float* part;  // [S][np][kPartStride]
  float* o_out;       // [S][128]
  float* lse_out;     // [S]
  int32_t np;
  int32_t pad_;
  const int32_t* seg_active;  // [S] or null: segments whose partials were not written are skipped
};

__global__ __launch_bounds__(kHeadDim) void combine(CombineArgs a) {
  __shared__ float sm[kMaxPartials], sf[kMaxPartials], red[2];
  const int64_t seg = blockIdx.x;
  if (a.seg_active && a.seg_active[seg] == 0) return;
  combine_partials(a.part + seg * a.np * kPartStride, a.np, a.o_out + seg * kHeadDim, a.lse_out + seg, sm, sf, red);
}

// ---------------------------------------------------------------------------
// dense_attn: softmax . V over every row of the ranges (K >= n), G heads per
// KV head from one read of each K and V row. Tiles of 64 rows with a running
// maximum; one partial per (head, workgroup).
// ---------------------------------------------------------------------------
struct DenseArgs {
  const float* q;
  const char* k;
  const char* v;
  int64_t stride_b_bytes, stride_h_bytes;
  float* part;             // [S][nwg][kPartStride]
  int32_t* idx_out;        // [S][K] or null
  int64_t n_idx;           // positions below this are listed in idx_out; the remaining slots get -1
  int64_t n;
  int64_t rows_per_wg;
  int32_t nwg, Hq, Hkv, K;
  float scale;
  int32_t pad_;
  RangeTab tab;
};

constexpr int kDenseThreads = 256;
constexpr int kDenseTile = 64;   // one row per lane of a wave in the tile reductions
constexpr int kDenseSlice = 32;  // rows per workgroup are a multiple of this

template <typename T, int G>
__global__ __launch_bounds__(kDenseThreads) void dense_attn(DenseArgs a) {
  constexpr int EPL = KvTraits<T>::EPL, LPR = KvTraits<T>::LPR, RPL = KvTraits<T>::RPL, ROWB = KvTraits<T>::ROWB;
  constexpr int NW = kDenseThreads / 64;
  constexpr int U = kDenseTile / (NW * RPL);  // tile rows per wave load group
  __shared__ float zt[G][kDenseTile];
  __shared__ int64_t trow[kDenseTile];
  __shared__ float tmax[G], tsum[G];
  __shared__ float red[NW][G][kHeadDim];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rg = lane / LPR, c = lane % LPR;
  const int group = blockIdx.y;
  const int wg = blockIdx.x;
  const int b = group / a.Hkv, hkv = group % a.Hkv;
  const int64_t seg0 = (int64_t)b * a.Hq + (int64_t)hkv * G;
  float qr[G][EPL];
  load_q_slice<T, G>(a.q, seg0, c, qr);
  const char* kb = a.k + (int64_t)b * a.stride_b_bytes + (int64_t)hkv * a.stride_h_bytes;
  const char* vb = a.v + (int64_t)b * a.stride_b_bytes + (int64_t)hkv * a.stride_h_bytes;

  float m_run[G], s_run[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    s_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const int64_t p0 = (int64_t)wg * a.rows_per_wg;
  const int64_t p1 = min(a.n, p0 + a.rows_per_wg);
  for (int64_t tb = p0; tb < p1; tb += kDenseTile) {
    if (tid < kDenseTile) {
      const int64_t p = tb + tid;
      trow[tid] = p < p1 ? pos_to_row(a.tab, p) : -1;
    }
    __syncthreads();
    // key and value chunks of the tile, all loads issued before the first
    // use (rows past the end read row 0 of the set and are masked)
    u32x4 kwv[U], vwv[U];
    const int64_t r_any = trow[0];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = (w * U + u) * RPL + rg;
      const int64_t r = trow[i] >= 0 ? trow[i] : r_any;
      kwv[u] = load16(kb + r * ROWB + c * 16);
      vwv[u] = load16(vb + r * ROWB + c * 16);
    }
    // scores of the tile
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = (w * U + u) * RPL + rg;
      const int64_t r = trow[i];
      float d[G];
      chunk_dots<T, G>(kwv[u], qr, d);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float s = group_sum<LPR>(d[h]);
        if (c == h) zt[h][i] = (r >= 0) ? s * a.scale : -INFINITY;
      }
    }
    __syncthreads();
    // per-head tile maximum and new running maximum
    for (int h = w; h < G; h += NW) {
      const float mx = wave_max(zt[h][lane]);
      if (lane == 0) tmax[h] = mx;
    }
    __syncthreads();
    float f_old[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(m_run[h], tmax[h]);
      f_old[h] = (m_run[h] == -INFINITY) ? 0.f : __expf(m_run[h] - mn);
      m_run[h] = mn;
    }
    // weights e^{z - m} in place, and their tile sums
    if (tid < kDenseTile) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float zz = zt[h][tid];
        zt[h][tid] = (zz == -INFINITY) ? 0.f : __expf(zz - m_run[h]);
      }
    }
    __syncthreads();
    for (int h = w; h < G; h += NW) {
      const float sm = wave_sum(zt[h][lane]);
      if (lane == 0) tsum[h] = sm;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_run[h] = s_run[h] * f_old[h] + tsum[h];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= f_old[h];
    }
    // value rows of the tile (masked rows have weight 0)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = (w * U + u) * RPL + rg;
      float x[EPL];
      unpack16<T>(vwv[u], x);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float wt = zt[h][i];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(wt, x[e], acc[h][e]);
      }
    }
    __syncthreads();
  }
  // reduce the row groups of each wave, then the waves
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = acc[h][e];
      if constexpr (RPL == 4) {
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
      } else {
        x += __shfl_xor(x, 32, 64);
      }
      acc[h][e] = x;
    }
  if (rg == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[w][h][c * EPL + e] = acc[h][e];
  }
  __syncthreads();
  for (int i = tid; i < G * kHeadDim; i += kDenseThreads) {
    const int h = i / kHeadDim, j = i % kHeadDim;
    float o = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) o += red[ww][h][j];
    a.part[((seg0 + h) * a.nwg + wg) * kPartStride + 4 + j] = o;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (tid == h) {
      float* p = a.part + ((seg0 + h) * a.nwg + wg) * kPartStride;
      p[0] = m_run[h];
      p[1] = s_run[h];
    }
  }
  // the row list of a dense call is every position (ascending), -1 padded
  if (a.idx_out) {
    for (int64_t p = p0 + tid; p < min(p1, a.n_idx); p += kDenseThreads) {
      const int32_t row = (int32_t)pos_to_row(a.tab, p);
#pragma unroll
      for (int h = 0; h < G; ++h) a.idx_out[(seg0 + h) * a.K + p] = row;
    }
    if (wg == 0)
      for (int64_t p = a.n_idx + tid; p < a.K; p += kDenseThreads)
#pragma unroll
        for (int h = 0; h < G; ++h) a.idx_out[(seg0 + h) * a.K + p] = -1;
  }
}

// ---------------------------------------------------------------------------
// attn_merge: o = e^{lse_a - lse} o_a + e^{lse_b - lse} o_b (Eq. 4-5).
// One block row of 128 threads per (o, lse) pair; the lse values are read
// before any thread writes so that the outputs may alias the inputs.
// ---------------------------------------------------------------------------
struct MergeArgs {
  const float *o_a, *lse_a, *o_b, *lse_b;
  float *o_out, *lse_out;
  int64_t rows;
  int32_t d;
  int32_t pad_;
};

constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void attn_merge(MergeArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
  const int t = threadIdx.x & 127;
  float la = -INFINITY, lb = -INFINITY;
  if (row < a.rows) {
    la = a.lse_a[row];
    lb = a.lse_b[row];
  }
  __syncthreads();
  if (row >= a.rows) return;
  const float M = fmaxf(la, lb);
  float ga = 0.f, gb = 0.f, lse = -INFINITY;
  if (M != -INFINITY) {
    const float ea = (la == -INFINITY) ? 0.f : __expf(la - M);
    const float eb = (lb == -INFINITY) ? 0.f : __expf(lb - M);
    const float tot = ea + eb;
    lse = M + __logf(tot);
    ga = ea / tot;
    gb = eb / tot;
  }
  for (int j = t; j < a.d; j += 128) {
    const int64_t i = row * a.d + j;
    const float xa = a.o_a[i], xb = a.o_b[i];
    a.o_out[i] = (ga == 0.f ? 0.f : ga * xa) + (gb == 0.f ? 0.f : gb * xb);
  }
  if (t == 0) a.lse_out[row] = lse;
}

// ---------------------------------------------------------------------------
// small utility kernels
// ---------------------------------------------------------------------------
// Every row of the ranges, ascending, in each of S lists of K (-1 padded).
__global__ __launch_bounds__(256) void fill_rows(int32_t* out, int64_t S, int32_t K, RangeTab tab) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= S * K) return;
  const int64_t p = i % K;
  out[i] = p < tab.pos0[tab.n] ? (int32_t)pos_to_row(tab, p) : -1;
}

// ---------------------------------------------------------------------------
// Empty row set: o = 0, lse = -inf, idx = -1.
__global__ __launch_bounds__(256) void fill_empty(float* o, float* lse, int32_t* idx, int64_t S, int32_t K) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < S * kHeadDim) o[i] = 0.f;
  if (i < S) lse[i] = -INFINITY;
  if (idx && i < S * K) idx[i] = -1;
}

}  // namespace stdk
