// Exact per-head top-K select over the scan's scores.
//
// The index set is TopK over every score of the segment (ReTopK review,
// "Exact Top-K 的隐藏成本": S_t = TopK(e, K) over all L_t scores), with ties
// resolved towards the lowest row (a reading: the pages leave ties open).
//
// Three passes, all exact:
//  1. k_scan has counted the first radix digit (top 11 key bits). Every
//     filter workgroup derives the same threshold bin b* (the bin holding the
//     K-th largest key) and appends the positions whose digit is >= b* to a
//     per-segment list (unordered; integer atomics only).
//  2. One select workgroup per segment finishes the radix select on the list
//     (digits 20..10 and 9..0) to get the exact K-th key T, and, if several
//     rows share T, the position cut-off among them (radix select on the
//     position). Chosen = key > T, or key == T and position <= cut-off.
//  3. Chosen positions are marked in a bitmap of the segment's positions and
//     read back in ascending order, which gives the ascending row list.
#pragma once

#include "device.h"

namespace stdk {

struct FilterArgs {
  const float* scores;      // [S][n_pad]
  const uint32_t* hist;     // [S][2048]
  int32_t* list;            // [S][n_pad] positions, unordered
  uint32_t* list_cnt;       // [S]
  int64_t n, n_pad, chunk;  // positions, row pitch, positions per workgroup
  int32_t K;
  int32_t pad_;
  const int32_t* seg_active;  // [S] or null
};

constexpr int kFilterThreads = 256;

__global__ __launch_bounds__(kFilterThreads) void topk_filter(FilterArgs a) {
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t tmp[kFilterThreads / 64 + 1];
  __shared__ int s_bin;
  __shared__ uint32_t s_beyond;
  const int64_t seg = blockIdx.y;
  if (a.seg_active && a.seg_active[seg] == 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < kHistBins; i += kFilterThreads) h[i] = a.hist[seg * kHistBins + i];
  __syncthreads();
  find_bin<kFilterThreads, true>(h, kHistBins, (uint32_t)a.K, tmp, &s_bin, &s_beyond);
  const int bstar = s_bin < 0 ? 0 : s_bin;
  const float* sc = a.scores + seg * a.n_pad;
  int32_t* lst = a.list + seg * a.n_pad;
  const int64_t p0 = (int64_t)blockIdx.x * a.chunk;
  const int64_t p1 = min(a.n, p0 + a.chunk);
  for (int64_t pb = p0; pb < p1; pb += kFilterThreads) {
    const int64_t p = pb + tid;
    bool take = false;
    if (p < p1) take = (int)(f2key(sc[p]) >> (32 - kHistBits)) >= bstar;
    const uint64_t m = __ballot(take);
    if (m) {
      const int leader = __ffsll((unsigned long long)m) - 1;
      uint32_t base = 0;
      if (lane == leader) base = atomicAdd(&a.list_cnt[seg], (uint32_t)__popcll(m));
      base = __shfl(base, leader, 64);
      if (take) lst[base + lane_rank(m)] = (int32_t)p;
    }
  }
}

struct SelectArgs {
  const float* scores;       // [S][n_pad]
  const uint32_t* hist;      // [S][2048]
  const int32_t* list;       // [S][n_pad]
  const uint32_t* list_cnt;  // [S]
  int64_t n, n_pad;
  int32_t K;
  int32_t bitmap_words;      // ceil(n / 32)
  int32_t* sel_row;          // [S][K] chosen rows, ascending, -1 padded
  float* sel_z;              // [S][K] their scores
  int32_t* idx_out;          // [S][K] or null (copy of sel_row)
  uint32_t* gbitmap;         // [S][bitmap_words] when the bitmap does not fit in LDS
  const int32_t* seg_active; // [S] or null
  RangeTab tab;
};

constexpr int kSelectThreads = 1024;

template <bool kLdsBitmap>
__global__ __launch_bounds__(kSelectThreads) void topk_select(SelectArgs a) {
  extern __shared__ uint32_t dyn[];  // bitmap (kLdsBitmap)
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t tmp[kSelectThreads / 64 + 1];
  __shared__ int s_bin;
  __shared__ uint32_t s_beyond;
  const int64_t seg = blockIdx.x;
  if (a.seg_active && a.seg_active[seg] == 0) return;
  const int tid = threadIdx.x;
  const float* sc = a.scores + seg * a.n_pad;
  const int32_t* lst = a.list + seg * a.n_pad;
  const uint32_t m = a.list_cnt[seg];

  // digit 0 (bits 31..21): from the scan's histogram
  for (int i = tid; i < kHistBins; i += kSelectThreads) h[i] = a.hist[seg * kHistBins + i];
  __syncthreads();
  find_bin<kSelectThreads, true>(h, kHistBins, (uint32_t)a.K, tmp, &s_bin, &s_beyond);
  const uint32_t b0 = (uint32_t)(s_bin < 0 ? 0 : s_bin);
  uint32_t need = (uint32_t)a.K - s_beyond;
  __syncthreads();

  // digit 1 (bits 20..10) among list entries in bin b0
  for (int i = tid; i < kHistBins; i += kSelectThreads) h[i] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < m; i += kSelectThreads) {
    const uint32_t key = f2key(sc[lst[i]]);
    if ((key >> 21) == b0) atomicAdd(&h[(key >> 10) & 0x7FFu], 1u);
  }
  __syncthreads();
  find_bin<kSelectThreads, true>(h, 2048, need, tmp, &s_bin, &s_beyond);
  const uint32_t b1 = (uint32_t)(s_bin < 0 ? 0 : s_bin);
  need -= s_beyond;
  __syncthreads();

  // digit 2 (bits 9..0)
  const uint32_t pre01 = (b0 << 11) | b1;
  for (int i = tid; i < 1024; i += kSelectThreads) h[i] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < m; i += kSelectThreads) {
    const uint32_t key = f2key(sc[lst[i]]);
    if ((key >> 10) == pre01) atomicAdd(&h[key & 0x3FFu], 1u);
  }
  __syncthreads();
  find_bin<kSelectThreads, true>(h, 1024, need, tmp, &s_bin, &s_beyond);
  const uint32_t b2 = (uint32_t)(s_bin < 0 ? 0 : s_bin);
  const uint32_t T = (pre01 << 10) | b2;
  const uint32_t ties = h[b2];
  need -= s_beyond;  // rows with key == T to keep (1..ties)
  __syncthreads();

  // position cut-off among the ties: the need-th smallest position
  int32_t cut = 0x7FFFFFFF;
  if (need < ties) {
    uint32_t prefix = 0;
    const int shifts[3] = {20, 9, 0};
    const int bits[3] = {11, 11, 9};
    uint32_t rem = need;
    for (int d = 0; d < 3; ++d) {
      const int nb = 1 << bits[d];
      for (int i = tid; i < nb; i += kSelectThreads) h[i] = 0u;
      __syncthreads();
      const int hi_shift = shifts[d] + bits[d];
      for (uint32_t i = tid; i < m; i += kSelectThreads) {
        const uint32_t p = (uint32_t)lst[i];
        if (f2key(sc[p]) == T && (d == 0 || (p >> hi_shift) == prefix))
          atomicAdd(&h[(p >> shifts[d]) & (uint32_t)(nb - 1)], 1u);
      }
      __syncthreads();
      find_bin<kSelectThreads, false>(h, nb, rem, tmp, &s_bin, &s_beyond);
      prefix = (prefix << bits[d]) | (uint32_t)(s_bin < 0 ? 0 : s_bin);
      rem -= s_beyond;
      __syncthreads();
    }
    cut = (int32_t)prefix;
  }

  // mark the chosen positions
  const int W = a.bitmap_words;
  uint32_t* bm = kLdsBitmap ? dyn : (a.gbitmap + seg * (int64_t)W);
  for (int i = tid; i < W; i += kSelectThreads) bm[i] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < m; i += kSelectThreads) {
    const int32_t p = lst[i];
    const uint32_t key = f2key(sc[p]);
    if (key > T || (key == T && p <= cut)) atomicOr(&bm[p >> 5], 1u << (p & 31));
  }
  __syncthreads();

  // ascending compaction: thread t owns words [t*per, (t+1)*per)
  const int per = (W + kSelectThreads - 1) / kSelectThreads;
  const int w0 = tid * per, w1 = min(W, w0 + per);
  uint32_t cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __popc(bm[i]);
  uint32_t total;
  uint32_t r = block_excl_scan<kSelectThreads>(cnt, tmp, &total);
  int32_t* srow = a.sel_row + seg * a.K;
  float* sz = a.sel_z + seg * a.K;
  int32_t* io = a.idx_out ? a.idx_out + seg * a.K : nullptr;
  for (int i = w0; i < w1; ++i) {
    uint32_t bits = bm[i];
    while (bits) {
      const int j = __ffs(bits) - 1;
      bits &= bits - 1;
      const int64_t p = (int64_t)i * 32 + j;
      if (r < (uint32_t)a.K) {
        const int32_t row = (int32_t)pos_to_row(a.tab, p);
        srow[r] = row;
        sz[r] = sc[p];
        if (io) io[r] = row;
      }
      ++r;
    }
  }
  for (uint32_t i = total + tid; i < (uint32_t)a.K; i += kSelectThreads) {
    srow[i] = -1;
    sz[i] = -INFINITY;
    if (io) io[i] = -1;
  }
}

}  // namespace stdk
