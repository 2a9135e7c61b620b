// Multi-query exact top-K: for every query of a block of M queries per query
// head, the index set of its K largest scores over the same key rows.
//
// This is the exact Top-K of the ReTopK review ("Exact Top-K 的隐藏成本":
// TopK over every score) taken for a block of queries at once: the ReTopK
// cache starts from the last prefill queries and their supports ("核心方法"
// 1), and RetrievalAttention's index build starts from the exact nearest keys
// of each prefill query ("Attention-Aware ANNS Index Construction"). Ties go
// to the lowest row, as in the decode select.
//
// With R = G*M queries per KV head the scores of one KV head form the dense
// product of an [R x 128] query matrix and a [128 x n] key matrix, so the
// products run on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16). Every
// element x of scale * q (fp32) is split into a bf16 value and a bf16
// remainder, x = hi + lo + r with |r| <= 2^-17 |x|, and both parts are
// multiplied into the same fp32 accumulator. A bf16 key is exact in that product; an fp32 key
// is split the same way and the three products hi*hi, lo*hi and hi*lo are
// kept. The scores therefore differ from an fp32 dot product by about
// 2^-16 * scale * sum_j |q_j k_j| plus fp32 accumulation rounding.
//
// No score array is written. Two passes compute the same scores with the
// same instructions, so they agree bit for bit:
//  1. mq_blockmax: per query, the largest score of every group of 16
//     positions (the 16 keys one lane holds after a block's products).
//  2. mq_threshold: per query, a key t such that at least K group maxima
//     are >= t (two radix digits of the maxima). Those maxima are K distinct
//     positions, so the K-th largest score is >= t.
//  3. mq_collect: the scores again; the (key, position) pairs with key >= t
//     go to the query's candidate list in position order (one slice per
//     workgroup chunk of positions).
//  4. mq_select finishes each query exactly on its candidates with one wave
//     (three radix digits and an ordered compaction): the K-th largest
//     score is among them, with every score above it.
#pragma once

#include "device.h"
#include "select_kernels.h"

namespace stdk {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float mq_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMqWaves = 4;
constexpr int kMqThreads = 64 * kMqWaves;
constexpr int kMqBlock = 32;            // positions per key block (one MFMA tile edge)
constexpr int kMqThreshThreads = 256;
constexpr int kMqMaxChunks = 4096;      // slices per query (the select keeps their prefix in LDS)

// Query tiles (32 queries each) held in registers by one wave.
template <typename T>
struct MqShape;
template <>
struct MqShape<uint16_t> {
  static constexpr int QT = 2;
  static constexpr int ROWB = 256;
};
template <>
struct MqShape<float> {
  static constexpr int QT = 1;
  static constexpr int ROWB = 512;
};

struct MqArgs {
  const float* q;            // [B][Hq][M][128] fp32
  const char* k;             // key cache base
  int64_t stride_b_bytes, stride_h_bytes;
  int64_t n;                 // positions (rows in the ranges)
  int64_t n_pad;             // candidate-list stride per query
  int32_t M, G, Hq, Hkv;
  int32_t rows;              // G * M queries per KV head
  int32_t chunk;             // positions per workgroup, a multiple of kMqBlock
  int32_t nchunk;            // workgroups along the positions
  int32_t ngrp;              // 16-position groups per query (2 per block)
  float scale;
  int32_t pad_;
  float* bmax;               // mq_blockmax output [S][ngrp]
  const uint32_t* thr;       // mq_collect input [S]: keep keys >= thr
  Cand* list;                // mq_collect: [S][n_pad], slice j starts at j * chunk
  uint32_t* slice_cnt;       // mq_collect: [S][nchunk]
  RangeTab tab;
};

// Splits 8 fp32 values into bf16 high parts and bf16 remainders (split_bf16x8).
STDK_DEV void split8(const mq_f32x4& x0, const mq_f32x4& x1, u32x4& hi, u32x4& lo) {
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  split_bf16x8(x, hi, lo);
}

STDK_DEV int64_t min64(int64_t x, int64_t y) { return x < y ? x : y; }

// One pass over the workgroup's chunk of positions for its waves' query
// tiles.
//
// Operand layout of v_mfma_f32_32x32x16_bf16: the A operand of lane l is row
// l%32, k = 8*(l/32) + i; the B operand is column l%32 with the same k; the
// result register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
// Here A is 32 keys (rows) and B is 32 queries (columns). The head dimension
// is permuted so that a lane's k values over the 8 steps are 64 consecutive
// elements: step s, half h = l/32 uses elements 64h + 8s + i. The dot
// product does not depend on the order; each lane reads its query row as 256
// contiguous bytes and its key row as 16-byte LDS reads 128 bytes apart.
//
// Key blocks (32 positions) are loaded once per workgroup, every thread
// taking 32 (bf16) or 64 (fp32) contiguous bytes of one row, kDepth blocks
// ahead, and written to a two-slot LDS ring as bf16 (an fp32 key as its bf16
// high part and remainder). One barrier per block: a slot is rewritten two
// blocks after it was read, and every wave has passed the previous block's
// barrier by then.
//
// After the 8 steps lane (c = l%32, h) holds the scores of query c of the
// tile against the 16 keys 8*(r/4) + 4h + r%4 of the block.
constexpr int kMqLdsRow = 272;    // bytes per staged key row: 256 + 16 (rows start 4 banks apart)
constexpr int kMqLdsSlot = kMqBlock * kMqLdsRow;
constexpr int kMqMaxBuf = 16;     // blocks whose maxima a workgroup keeps in LDS between writes

template <typename T, bool kCollect, int kDepth>
STDK_DEV void mq_pass(const MqArgs& a) {
  constexpr int QT = MqShape<T>::QT, ROWB = MqShape<T>::ROWB;
  constexpr bool kF32 = sizeof(T) == 4;
  constexpr int NL = kF32 ? 4 : 2;   // 16-byte pieces per thread and block
  constexpr int NP = kF32 ? 2 : 1;   // staged parts per key (high, remainder)
  __shared__ __attribute__((aligned(16))) char ring[2][NP][kMqLdsSlot];
  // collect: one 36-word row per lane pair (query c of the wave's tile);
  // rows 4 banks apart
  __shared__ __attribute__((aligned(16))) uint32_t ckeys[kCollect ? kMqWaves : 1][32][kCollect ? 36 : 4];
  // blockmax: the group maxima of up to kMqMaxBuf blocks per query of the
  // workgroup, written out as contiguous runs (rows 33 words apart)
  __shared__ float mxs[kCollect ? 1 : kMqWaves * QT * 32][kCollect ? 1 : 2 * kMqMaxBuf + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the tile tests below are scalar
  const int c = lane & 31, h = lane >> 5;
  const int grp = blockIdx.y;
  const int b = grp / a.Hkv, hk = grp - b * a.Hkv;
  const int64_t seg0 = ((int64_t)b * a.Hq + (int64_t)hk * a.G) * a.M;  // query row 0 of this KV head
  const char* kbase = a.k + b * a.stride_b_bytes + hk * a.stride_h_bytes;
  const int tile0 = ((int)blockIdx.z * kMqWaves + w) * QT;
  uint32_t* ckrow = ckeys[kCollect ? w : 0][c];

  const int64_t p_begin = (int64_t)blockIdx.x * a.chunk;
  const int64_t p_end = min64(a.n, p_begin + a.chunk);
  const int64_t b_begin = p_begin / kMqBlock;
  const int nb = (int)((p_end + kMqBlock - 1) / kMqBlock - b_begin);  // blocks of this chunk

  // a chunk inside one range maps position p to row p + delta (found once,
  // with scalar loads); a chunk across a range boundary looks every row up
  int64_t delta = 0;
  bool one_range = true;
  {
    const int64_t r_first = pos_to_row(a.tab, p_begin), r_last = pos_to_row(a.tab, p_end - 1);
    delta = r_first - p_begin;
    one_range = r_last - (p_end - 1) == delta;
  }

  // this thread's share of a block: key row lk, bytes [lb, lb + 16*NL)
  const int lk = tid >> 3;
  const int lb = (tid & 7) * 16 * NL;
  auto issue = [&](int i, u32x4 (&rr)[NL]) {
    const int64_t p = min64((b_begin + i) * kMqBlock + lk, a.n - 1);
    const int64_t row = one_range ? p + delta : pos_to_row(a.tab, p);
    const char* src = kbase + row * ROWB + lb;
#pragma unroll
    for (int j = 0; j < NL; ++j) rr[j] = load16(src + 16 * j);
  };
  // the first key blocks are requested before the queries are read and split
  u32x4 rr[kDepth][NL];
#pragma unroll
  for (int j = 0; j < kDepth; ++j) issue(min(j, nb - 1), rr[j]);

  // query operands of this wave's tiles, bf16 high parts and remainders
  u32x4 qh[QT][8], ql[QT][8];
  bool tv[QT], rv[QT];
  int64_t seg[QT];
  uint32_t thr[QT], cnt[QT];
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int r = (tile0 + u) * 32 + c;
    tv[u] = (tile0 + u) * 32 < a.rows;  // uniform over the wave
    rv[u] = r < a.rows;
    seg[u] = seg0 + min(r, a.rows - 1);
    const float* qp = a.q + seg[u] * kHeadDim + 64 * h;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      // the scale is applied to the query, so the products are the scores
      const mq_f32x4 x0 = *reinterpret_cast<const mq_f32x4*>(qp + 8 * s) * a.scale;
      const mq_f32x4 x1 = *reinterpret_cast<const mq_f32x4*>(qp + 8 * s + 4) * a.scale;
      split8(x0, x1, qh[u][s], ql[u][s]);
    }
    thr[u] = 0u;
    if constexpr (kCollect) thr[u] = a.thr[seg[u]];
    cnt[u] = 0u;
  }

  auto stage = [&](int slot, const u32x4 (&rr)[NL]) {
    if constexpr (kF32) {
      // 16 fp32 elements [16*(tid&7), +16) -> 32 bytes of each part
      u32x4 h0, l0, h1, l1;
      split8(__builtin_bit_cast(mq_f32x4, rr[0]), __builtin_bit_cast(mq_f32x4, rr[1]), h0, l0);
      split8(__builtin_bit_cast(mq_f32x4, rr[2]), __builtin_bit_cast(mq_f32x4, rr[3]), h1, l1);
      char* dh = ring[slot][0] + lk * kMqLdsRow + (tid & 7) * 32;
      char* dl = ring[slot][1] + lk * kMqLdsRow + (tid & 7) * 32;
      *reinterpret_cast<u32x4*>(dh) = h0;
      *reinterpret_cast<u32x4*>(dh + 16) = h1;
      *reinterpret_cast<u32x4*>(dl) = l0;
      *reinterpret_cast<u32x4*>(dl + 16) = l1;
    } else {
      char* d = ring[slot][0] + lk * kMqLdsRow + lb;
      *reinterpret_cast<u32x4*>(d) = rr[0];
      *reinterpret_cast<u32x4*>(d + 16) = rr[1];
    }
  };

  auto block = [&](int i, int slot) {
    const int64_t blk = b_begin + i;
    f32x16 acc[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u) acc[u] = f32x16{};
    // all of the block's key fragments first, then the products: the LDS
    // reads overlap, and every tile is multiplied (a tile without queries
    // costs no time, the busiest wave of the SIMD sets the pace), so the
    // products carry no branches
    const char* arow = ring[slot][0] + c * kMqLdsRow + 128 * h;
    u32x4 kf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = *reinterpret_cast<const u32x4*>(arow + 16 * s);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 kh = as_bf16x8(kf[s]);
#pragma unroll
      for (int u = 0; u < QT; ++u) {
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, as_bf16x8(qh[u][s]), acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, as_bf16x8(ql[u][s]), acc[u], 0, 0, 0);
      }
    }
    if constexpr (kF32) {
#pragma unroll
      for (int s = 0; s < 8; ++s) kf[s] = *reinterpret_cast<const u32x4*>(arow + kMqLdsSlot + 16 * s);
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int u = 0; u < QT; ++u)
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[s]), as_bf16x8(qh[u][s]), acc[u], 0, 0, 0);
    }
    const int lim = (int)min64(kMqBlock, a.n - blk * kMqBlock);  // valid keys in the block
    const bool whole = lim == kMqBlock;                             // uniform
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      if (!tv[u]) continue;
      if constexpr (!kCollect) {
        // group h of the block: the lane's 16 keys (-inf if none is valid)
        float mx = acc[u][0];
        if (whole) {
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, acc[u][r]);
        } else {
          mx = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 8 * (r >> 2) + 4 * h + (r & 3);
            if (kk < lim) mx = fmaxf(mx, acc[u][r]);
          }
        }
        mxs[(w * QT + u) * 32 + c][2 * (i % kMqMaxBuf) + h] = mx;
      } else {
        uint32_t mine = 0, kv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 8 * (r >> 2) + 4 * h + (r & 3);
          kv[r] = f2key(acc[u][r]);
          mine |= (uint32_t)(kv[r] >= thr[u]) << kk;
        }
        if (!whole) mine &= lim >= 32 ? ~0u : ((1u << lim) - 1u);
        const uint32_t full = mine | (uint32_t)__shfl_xor((int)mine, 32, 64);
        if (rv[u] && mine != 0u) {
          // the lane's keys go to its own LDS row (key kk at word kk) and
          // only the kept ones are read back, in position order
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<u32x4*>(ckrow + 8 * j + 4 * h) = u32x4{kv[4 * j], kv[4 * j + 1], kv[4 * j + 2], kv[4 * j + 3]};
          Cand* out = a.list + seg[u] * a.n_pad + p_begin + cnt[u];
          for (uint32_t bits = mine; bits != 0u; bits &= bits - 1u) {
            const int kk = __ffs((int)bits) - 1;
            out[__popc(full & ((1u << kk) - 1u))] = Cand{ckrow[kk], (int32_t)(blk * kMqBlock + kk)};
          }
        }
        cnt[u] += (uint32_t)__popc(full);
      }
    }
  };

  // blockmax: the groups of blocks [i_first, i_last] go to the queries' rows
  auto flush = [&](int i_first, int i_last) {
    __syncthreads();
    const int nbuf = 2 * (i_last - i_first + 1);
    constexpr int QW = kMqWaves * QT * 32;  // queries of the workgroup
    const int q0 = (int)blockIdx.z * QW;
    for (int e = tid; e < QW * nbuf; e += kMqThreads) {
      const int ql = e / nbuf, j = e - ql * nbuf;
      if (q0 + ql < a.rows)
        a.bmax[(seg0 + q0 + ql) * a.ngrp + 2 * (b_begin + i_first) + j] = mxs[ql][2 * (i_first % kMqMaxBuf) + j];
    }
    __syncthreads();
  };

  // Every refill is issued, past the end clamped onto the last block (read
  // again, unused): with the same number of loads in flight on every path,
  // the wait before staging a block leaves the later blocks' loads pending.
  for (int i0 = 0; i0 < nb; i0 += kDepth) {
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      const int i = i0 + j;
      if (i < nb) {  // uniform over the workgroup
        stage(i & 1, rr[j]);
        issue(min(i + kDepth, nb - 1), rr[j]);
        __syncthreads();
        block(i, i & 1);
        if constexpr (!kCollect) {
          if (i % kMqMaxBuf == kMqMaxBuf - 1 || i == nb - 1) flush(i - i % kMqMaxBuf, i);
        }
      }
    }
  }
  if constexpr (kCollect) {
#pragma unroll
    for (int u = 0; u < QT; ++u)
      if (h == 0 && rv[u]) a.slice_cnt[seg[u] * a.nchunk + blockIdx.x] = cnt[u];
  }
}

// grid (nchunk, B * Hkv, row packs of kMqWaves * QT * 32 queries)
template <typename T>
__global__ __launch_bounds__(kMqThreads) void mq_blockmax(MqArgs a) {
  mq_pass<T, false, 3>(a);
}

template <typename T>
__global__ __launch_bounds__(kMqThreads) __attribute__((amdgpu_waves_per_eu(2))) void mq_collect(MqArgs a) {
  mq_pass<T, true, 3>(a);
}

// ---------------------------------------------------------------------------
// mq_threshold: one workgroup per query. thr = the 22-bit key prefix of the
// bin (two radix digits) that holds the K-th largest group maximum, so that
// at least K maxima have key >= thr. With fewer than K groups, or n <= K,
// thr = 0 keeps every position. (A group without valid positions has
// maximum -inf; if it is counted, thr is at most the key of -inf and every
// position is kept.)
// ---------------------------------------------------------------------------
struct MqThreshArgs {
  const float* bmax;  // [S][ngrp]
  uint32_t* thr;      // [S]
  int64_t n;
  int32_t ngrp, K;
};

__global__ __launch_bounds__(kMqThreshThreads) void mq_threshold(MqThreshArgs a) {
  __shared__ uint32_t hst[kHistBins];
  __shared__ int s_bin;
  __shared__ uint32_t s_beyond;
  const int64_t seg = blockIdx.x;
  const int tid = threadIdx.x;
  if (a.n <= a.K || a.ngrp < a.K) {
    if (tid == 0) a.thr[seg] = 0u;
    return;
  }
  const float* bm = a.bmax + seg * a.ngrp;
  // f(key) over the maxima, 8 loads per thread in flight
  auto each = [&](auto&& f) {
    constexpr int U = 8;
    for (int i0 = 0; i0 < a.ngrp; i0 += U * kMqThreshThreads) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = bm[min(i0 + u * kMqThreshThreads + tid, a.ngrp - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u * kMqThreshThreads + tid < a.ngrp) f(f2key(v[u]));
    }
  };
  for (int i = tid; i < kHistBins; i += kMqThreshThreads) hst[i] = 0u;
  __syncthreads();
  each([&](uint32_t key) { atomicAdd(&hst[key >> 21], 1u); });
  __syncthreads();
  if (tid < 64) find_bin_wave<kHistBins, true>(hst, (uint32_t)a.K, &s_bin, &s_beyond);
  __syncthreads();
  const int b0 = s_bin;
  const uint32_t need = (uint32_t)a.K - s_beyond;
  for (int i = tid; i < kHistBins; i += kMqThreshThreads) hst[i] = 0u;
  __syncthreads();
  if (b0 >= 0) each([&](uint32_t key) {
    if ((int)(key >> 21) == b0) atomicAdd(&hst[(key >> 10) & 0x7FFu], 1u);
  });
  __syncthreads();
  if (b0 >= 0 && tid < 64) find_bin_wave<kHistBins, true>(hst, need, &s_bin, &s_beyond);
  __syncthreads();
  if (tid == 0) a.thr[seg] = (b0 < 0 || s_bin < 0) ? 0u : (((uint32_t)b0 << 21) | ((uint32_t)s_bin << 10));
}

// ---------------------------------------------------------------------------
// mq_select: one wave per query, on its candidates (every score >= thr, in
// position order, slice j of the list at j * chunk with slice_cnt[j]
// entries). The K-th largest key and every larger one are candidates, so the
// exact selection is three radix digits (bits 31..21, 20..10, 9..0) over the
// candidates, then an ordered compaction: key > T, or key == T among the
// first `need` such candidates in position order (lowest rows first).
// Candidates are copied to the wave's LDS when at most `cap` of them exist;
// otherwise every pass reads them from the list.
// Dynamic LDS per wave: hist[2048] | pre[rup(nchunk + 1, 4)] | cache[cap].
// ---------------------------------------------------------------------------
struct MqSelArgs {
  const Cand* list;           // [S][n_pad]
  const uint32_t* slice_cnt;  // [S][nchunk]
  int32_t* idx_out;           // [S][K]
  float* z_out;               // [S][K] or null
  int64_t S, n, n_pad;
  int32_t chunk, nchunk, K, cap;
  int32_t lds_words;          // dynamic LDS words per wave
  int32_t pad_;
  RangeTab tab;
};

constexpr int kMqSelWaves = 4;

__global__ __launch_bounds__(64 * kMqSelWaves) void mq_select(MqSelArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t mq_dyn[];
  __shared__ int s_bin[kMqSelWaves];
  __shared__ uint32_t s_beyond[kMqSelWaves];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t seg = (int64_t)blockIdx.x * kMqSelWaves + w;
  if (seg >= a.S) return;  // whole wave; no workgroup barrier below
  uint32_t* hist = mq_dyn + (size_t)w * a.lds_words;
  uint32_t* pre = hist + kHistBins;
  Cand* cache = reinterpret_cast<Cand*>(pre + ((a.nchunk + 4) & ~3));
  const Cand* lst = a.list + seg * a.n_pad;
  const int ns = a.nchunk;
  const int K = a.K;
  const bool take_all = a.n <= K;

  // slice prefix, 4 loads per lane in flight
  uint32_t run = 0;
  for (int j0 = 0; j0 < ns; j0 += 256) {
    uint32_t cv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * 64 + lane;
      cv[u] = j < ns ? a.slice_cnt[seg * ns + j] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * 64 + lane;
      const uint32_t incl = wave_incl_scan(cv[u]);
      if (j < ns) pre[j] = run + incl - cv[u];
      run += lane_read(incl, 63);
    }
  }
  const uint32_t m = run;
  if (lane == 0) pre[ns] = m;
  const bool cached = m <= (uint32_t)a.cap;

  // candidate g: its slice is the last j with pre[j] <= g, found by a
  // fixed-step search (the same steps for every lane, so the searches of a
  // round run side by side)
  int top = 1;
  while (top * 2 <= ns) top *= 2;
  auto slice_of = [&](uint32_t g) -> int {
    int lo = 0;
    for (int step = top; step > 0; step >>= 1) {
      const int t = lo + step;
      const uint32_t v = pre[min(t, ns - 1)];
      lo = (t < ns && v <= g) ? t : lo;
    }
    return lo;
  };
  auto fetch = [&](uint32_t g) -> Cand {
    const int lo = slice_of(g);
    return lst[(int64_t)lo * a.chunk + (g - pre[lo])];
  };
  // f(g, cand) over every candidate, kU per lane per round: the rounds' reads
  // (from the list, or from the LDS copy) are all issued before their use
  constexpr int kU = 16;
  auto each = [&](bool from_list, auto&& f) {
    for (uint32_t g0 = 0; g0 < m; g0 += 64 * kU) {
      Cand cv[kU];
      if (from_list) {
        int lo[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) lo[u] = 0;
        for (int step = top; step > 0; step >>= 1) {
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            // unconditional read (clamped) and a select: no branch per step
            const uint32_t g = min(g0 + (uint32_t)(u * 64 + lane), m - 1u);
            const int t = lo[u] + step;
            const uint32_t v = pre[min(t, ns - 1)];
            lo[u] = (t < ns && v <= g) ? t : lo[u];
          }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const uint32_t g = min(g0 + (uint32_t)(u * 64 + lane), m - 1u);
          cv[u] = lst[(int64_t)lo[u] * a.chunk + (g - pre[lo[u]])];
        }
      } else {
#pragma unroll
        for (int u = 0; u < kU; ++u) cv[u] = cache[min(g0 + (uint32_t)(u * 64 + lane), m - 1u)];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t g = g0 + (uint32_t)(u * 64 + lane);
        if (g < m) f(g, cv[u]);
      }
    }
  };

  for (int i = lane; i < kHistBins; i += 64) hist[i] = 0u;
  // copy (when cached) and digit 0: each lane takes whole slices, up to kE
  // entries of each of its kS slices per round, all requested at once
  {
    constexpr int kS = 2, kE = 8;
    for (int j0 = 0; j0 < ns; j0 += 64 * kS) {
      uint32_t cnt[kS], off[kS];
      int64_t src[kS];
      uint32_t most = 0;
#pragma unroll
      for (int v = 0; v < kS; ++v) {
        const int j = min(j0 + v * 64 + lane, ns - 1);
        const bool valid = j0 + v * 64 + lane < ns;
        off[v] = pre[j];
        cnt[v] = valid ? pre[j + 1] - off[v] : 0u;
        src[v] = (int64_t)j * a.chunk;
        most = max(most, cnt[v]);
      }
      most = wave_max_u32(most);
      for (uint32_t e0 = 0; e0 < most; e0 += kE) {
        Cand cv[kS][kE];
#pragma unroll
        for (int v = 0; v < kS; ++v)
#pragma unroll
          for (int e = 0; e < kE; ++e) cv[v][e] = lst[src[v] + min(e0 + e, cnt[v] > 0 ? cnt[v] - 1 : 0u)];
#pragma unroll
        for (int v = 0; v < kS; ++v)
#pragma unroll
          for (int e = 0; e < kE; ++e) {
            if (e0 + e < cnt[v]) {
              if (cached) cache[off[v] + e0 + e] = cv[v][e];
              if (!take_all) atomicAdd(&hist[cv[v][e].key >> 21], 1u);
            }
          }
      }
    }
  }
  uint32_t Tk = 0u, need = (uint32_t)K;
  if (!take_all) {
    find_bin_wave<kHistBins, true>(hist, need, &s_bin[w], &s_beyond[w]);
    const uint32_t b0 = (uint32_t)max(s_bin[w], 0);
    need -= s_beyond[w];
    for (int i = lane; i < kHistBins; i += 64) hist[i] = 0u;
    each(!cached, [&](uint32_t, const Cand& cv) {
      if ((cv.key >> 21) == b0) atomicAdd(&hist[(cv.key >> 10) & 0x7FFu], 1u);
    });
    find_bin_wave<kHistBins, true>(hist, need, &s_bin[w], &s_beyond[w]);
    const uint32_t b1 = (uint32_t)max(s_bin[w], 0);
    need -= s_beyond[w];
    const uint32_t p01 = (b0 << 11) | b1;
    for (int i = lane; i < 1024; i += 64) hist[i] = 0u;
    each(!cached, [&](uint32_t, const Cand& cv) {
      if ((cv.key >> 10) == p01) atomicAdd(&hist[cv.key & 0x3FFu], 1u);
    });
    find_bin_wave<1024, true>(hist, need, &s_bin[w], &s_beyond[w]);
    Tk = (p01 << 10) | (uint32_t)max(s_bin[w], 0);
    need -= s_beyond[w];  // candidates with key == Tk to keep, the first ones in position order
  }

  // ordered compaction, 64 candidates per step in position order; with one
  // range a position's row is a fixed offset away
  const bool one_range = a.tab.n == 1;
  const int64_t delta = a.tab.row0[0] - a.tab.pos0[0];
  int32_t* io = a.idx_out + seg * K;
  float* zo = a.z_out ? a.z_out + seg * K : nullptr;
  uint32_t taken = 0, eq_seen = 0;
  for (uint32_t g0 = 0; g0 < m; g0 += 64) {
    const uint32_t g = g0 + lane;
    const Cand cv = g < m ? (cached ? cache[g] : fetch(g)) : Cand{0u, 0};
    const bool eq = g < m && !take_all && cv.key == Tk;
    const uint64_t eqm = __ballot(eq);
    const bool take = g < m && (take_all || cv.key > Tk || (eq && eq_seen + lane_rank(eqm) < need));
    const uint64_t tm = __ballot(take);
    const uint32_t r = taken + lane_rank(tm);
    if (take && r < (uint32_t)K) {
      io[r] = (int32_t)(one_range ? cv.pos + delta : pos_to_row(a.tab, cv.pos));
      if (zo) zo[r] = key2f(cv.key);
    }
    taken += (uint32_t)__popcll(tm);
    eq_seen += (uint32_t)__popcll(eqm);
  }
  for (uint32_t r = min(taken, (uint32_t)K) + lane; r < (uint32_t)K; r += 64) {
    io[r] = -1;
    if (zo) zo[r] = -INFINITY;
  }
}

// No positions: every index is -1 and every score -inf.
__global__ __launch_bounds__(256) void mq_fill(int32_t* idx, float* z, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) {
    idx[i] = -1;
    if (z) z[i] = -INFINITY;
  }
}

}  // namespace stdk
