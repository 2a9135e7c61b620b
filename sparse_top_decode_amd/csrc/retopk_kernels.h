// ReTopK: query-support cache, similar-query recall, candidate union with the
// recent window, exact rerank inside the candidates, and the cache push.
//
// Follows the ReTopK review "Recall Before You Rank: Similarity-Guided Top-K
// Reuse for Efficient Long-Context Attention", sections "核心方法" 1-5:
//  1. each query head keeps a FIFO of C (unit query, support) pairs, filled
//     from the last C prefill queries and pushed after every step on either
//     path;
//  2. the cosine of the current unit query with every cached one, and the R
//     most similar entries;
//  3. the candidate set is the union of their supports and the W newest rows
//     (at most R*K + W rows);
//  4. exact scores of the current query on the candidates, top K of them;
//  5. the exact path runs instead when the best cosine is below tau or on
//     every T_r-th step.
// The candidate union is a bitmap of the visible rows, read back in
// ascending order (no sort).
#pragma once

#include "attend_kernels.h"
#include "device.h"
#include "scan_kernels.h"
#include "select_kernels.h"

namespace stdk {

// q / ||q||_2 in one fixed arithmetic order, used wherever a unit query is
// formed: part j (0..7) covers dims [16j, 16j+16); its squares are summed in
// dim order, and the norm is the square root of the 8 part sums added in part
// order. A zero query gives zeros.
STDK_DEV float sumsq16(const float (&x)[16]) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s = fmaf(x[e], x[e], s);
  return s;
}
STDK_DEV float norm_of_parts(const float* sq) {
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) t += sq[j];
  return sqrtf(t);
}
STDK_DEV void load16f(const float* p, float (&x)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(p + 4 * i);
    x[4 * i] = v.x;
    x[4 * i + 1] = v.y;
    x[4 * i + 2] = v.z;
    x[4 * i + 3] = v.w;
  }
}

struct RtSelArgs {
  const float* q;           // [S][128]
  const float* q_hat;       // [S][C][128]
  const int32_t* support;   // [S][C][K]
  const int32_t* head;      // [S]
  const int32_t* count;     // [S]
  int32_t C, K, R, W;
  float tau;
  int32_t refresh_now;      // this step is a periodic refresh (host decided; unused with `step`)
  int64_t L_t;              // visible rows; with `step`, the most there can be
  int32_t cand_cap;         // R*K + W
  int32_t bitmap_words;     // ceil(L_t / 32)
  const int64_t* step;      // or null: device memory [L_t, t] for this step; L_t is clamped to
                            // [1, L_t above], and the refresh (t % refresh == 0) is decided here
  int32_t refresh, pad_;
  float* qbar;              // [S][128]
  int32_t* path;            // [S]
  int32_t* exact;           // [S]: 1 = this head takes the exact path
  int32_t* cand;            // [S][cand_cap]
  int32_t* n_cand;          // [S]
  int32_t* path_out;        // [S] or null
  int32_t* n_cand_out;      // [S] or null
  int32_t* cand_out;        // [S][cand_cap] or null
  uint32_t* gbitmap;        // [S][bitmap_words] when not in LDS
  int32_t* rec_slot;        // [S][kMaxVote] recalled slots in recall order, or null (no vote)
  float* rec_rho;           // [S][kMaxVote] their cosines
};

constexpr int kRtSelThreads = 256;
constexpr int kMaxCache = 64;
constexpr int kMaxVote = 8;  // recalled entries a confidence vote can weigh (masks fit a byte)

// Shared-memory state of the selector phases of one head.
template <int NT>
struct RtSelLds {
  float qb[kHeadDim];  // the unit query
  uint2 rkey[kMaxCache];
  float rcos[kMaxCache];
  float sq[8];
  int slot_of[kMaxCache];
  uint32_t tmp[NT / 64 + 1];
  int rec_slot[kMaxVote];
  float rec_rho[kMaxVote];
  float best;
  int npick;
};

// What the selector of one head decided (uniform over the workgroup).
struct RtSelOut {
  int path;      // 0 reuse, 1 similarity fallback, 2 refresh
  uint32_t M;    // reuse path: candidates written
  int64_t L_t;   // visible rows this step
};

// The selector of head `seg` with NT threads: the unit query (to ls.qb), the
// cosines with the cached entries, the path, and on the reuse path the union
// of the R most similar supports with the recent window, written in
// ascending row order to cd[0, min(union, cand_cap)) (global or LDS). `hd`
// and `cnt` are the FIFO's head and count as they stood before this step.
// bm: the bitmap of the visible rows, in LDS (kLdsBitmap) or global memory.
// Nothing else goes to global memory here: rt_select_store writes the
// per-head results once the workgroup's loads are done (a store issued
// before a wait on an earlier load makes that wait include the store).
template <int NT, bool kLdsBitmap>
STDK_DEV RtSelOut rt_select_head(const RtSelArgs& a, int64_t seg, int hd, int cnt, RtSelLds<NT>& ls,
                                 uint32_t* bm, int32_t* cd) {
  constexpr int kGroups = NT / 8;  // cache slots per pass
  constexpr int kPass = (kMaxCache + kGroups - 1) / kGroups;
  const int tid = threadIdx.x;
  const int C = a.C, K = a.K;
  const int j = tid & 7, g = tid >> 3;  // part of the 128 dims, cache slot within a pass
  int64_t L_t = a.L_t;
  int refresh_now = a.refresh_now;
  if (a.step) {
    L_t = min(a.L_t, max((int64_t)1, a.step[0]));
    const int64_t t = max((int64_t)0, a.step[1]);
    refresh_now = a.refresh > 0 && t % a.refresh == 0;
  }

  // One memory round trip: every thread requests its 16 query components and
  // the same components of its cache slots (slot g + kGroups * pass).
  float qx[16];
  load16f(a.q + seg * kHeadDim + 16 * j, qx);
  float qh[kPass][16];
#pragma unroll
  for (int ps = 0; ps < kPass; ++ps) {
    const int sl = min(g + kGroups * ps, C - 1);
    load16f(a.q_hat + (seg * C + sl) * kHeadDim + 16 * j, qh[ps]);
  }
  // unit query
  if (tid < 8) ls.sq[j] = sumsq16(qx);
  __syncthreads();
  const float nrm = norm_of_parts(ls.sq);
  float qn[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) qn[e] = nrm > 0.f ? qx[e] / nrm : 0.f;
  if (tid < 8) {
#pragma unroll
    for (int e = 0; e < 16; ++e) ls.qb[16 * j + e] = qn[e];
  }
  // cosines: 16-dim partial dot products; the 8 of a slot sit in 8
  // consecutive lanes and are summed in part order. Entry sl (< kMaxCache)
  // gets its cosine and rank key; the entry of slot s has age (head - s) mod
  // C, and only the `count` newest are valid (invalid: key 0, below every
  // valid key; cosine -inf).
  const int lane = tid & 63;
#pragma unroll
  for (int ps = 0; ps < kPass; ++ps) {
    const int sl = g + kGroups * ps;
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) t = fmaf(qn[e], qh[ps][e], t);
    float r = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) r += __shfl(t, (lane & ~7) | jj, 64);
    if (j == 0 && sl < kMaxCache) {
      int age = hd - sl;
      if (age < 0) age += C;
      const bool valid = sl < C && age < cnt;
      ls.rkey[sl] = valid ? make_uint2(f2key(r), ~(uint32_t)age) : make_uint2(0u, 0u);
      ls.rcos[sl] = valid ? r : -INFINITY;
    }
  }
  const int Wd = a.step ? (int)((L_t + 31) / 32) : a.bitmap_words;
  if (kLdsBitmap)
    for (int i = tid; i < Wd; i += NT) bm[i] = 0u;
  __syncthreads();
  // top R by (cosine descending, age ascending): the rank of entry i is the
  // number of entries with a larger key, counted by TPS threads over E
  // entries each; the picked entries go out in rank order. Wave 0 also
  // forms the best cosine (maximum over the valid entries; NaN ignored).
  {
    constexpr int TPS = NT / kMaxCache, E = kMaxCache / TPS;
    const int i = tid / TPS, sub = tid % TPS;
    const uint2 ki = ls.rkey[i];
    const uint64_t mine = ((uint64_t)ki.x << 32) | ki.y;
    int gt = 0;
#pragma unroll
    for (int f = 0; f < E; ++f) {
      const uint2 kf = ls.rkey[sub * E + f];
      gt += ((((uint64_t)kf.x << 32) | kf.y) > mine) ? 1 : 0;
    }
#pragma unroll
    for (int o = 1; o < TPS; o <<= 1) gt += __shfl_xor(gt, o, 64);
    const bool pk = mine != 0u && gt < a.R;
    if (sub == 0 && pk) {
      ls.slot_of[gt] = i;
      if (gt < kMaxVote) {
        ls.rec_slot[gt] = i;
        ls.rec_rho[gt] = ls.rcos[i];
      }
    }
    if (tid < 64) {
      const float best = wave_max(ls.rcos[tid]);
      if (tid == 0) ls.best = best;
    }
  }
  __syncthreads();
  int path;
  if (refresh_now) path = 2;
  else if (cnt == 0 || ls.best < a.tau) path = 1;
  else path = 0;
  if (path != 0) return RtSelOut{path, 0u, L_t};
  const int npick = min(a.R, min(cnt, C));
  if (tid == 0) ls.npick = npick;
  if (!kLdsBitmap) {
    for (int i = tid; i < Wd; i += NT) bm[i] = 0u;
    __syncthreads();
  }
  // The recent window [Lw, L) holds the largest visible rows: it is appended
  // after the bitmap's rows, which are the picked supports' rows below Lw.
  const int64_t L = L_t;
  const int64_t Lw = max((int64_t)0, L - a.W);
  // union of the picked supports: thread t takes entries f = t + NT * s of
  // the flattened npick x K list, entry e of picked slot p (f = p * K + e,
  // stepped without a division); kU loads per thread are in flight (past
  // the list: clamped to its last entry, no branches) before their bits are set
  {
    constexpr int kU = NT >= 1024 ? 4 : 8;
    const int total = npick * K;
    const int dp = NT / K, de = NT - dp * K;
    int p = tid / K, e = tid - p * K;
    for (int f0 = 0; f0 < total; f0 += NT * kU) {
      int32_t x[kU];
      bool in[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        in[u] = p < npick;
        const int pc = in[u] ? p : npick - 1, ec = in[u] ? e : K - 1;
        x[u] = a.support[(seg * C + ls.slot_of[pc]) * (int64_t)K + ec];
        e += de;
        p += dp;
        if (e >= K) {
          e -= K;
          ++p;
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (in[u] && x[u] >= 0 && x[u] < Lw) atomicOr(&bm[x[u] >> 5], 1u << (x[u] & 31));
    }
  }
  __syncthreads();
  // ascending compaction of the words below Lw: thread t owns the words
  // [t * CH, t * CH + CH); one block scan of the per-thread bit counts gives
  // each its first slot; then the window
  const int Wb = (int)((Lw + 31) / 32);
  const int CH = (Wb + NT - 1) / NT;
  const int w0 = min(Wb, tid * CH), w1 = min(Wb, w0 + CH);
  uint32_t c0 = 0;
  for (int i = w0; i < w1; ++i) c0 += __popc(bm[i]);
  uint32_t total;
  uint32_t pos = block_excl_scan<NT>(c0, ls.tmp, &total);
  for (int i = w0; i < w1; ++i) {
    uint32_t bits = bm[i];
    while (bits) {
      const int jb = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < (uint32_t)a.cand_cap) cd[pos] = i * 32 + jb;
      ++pos;
    }
  }
  const uint32_t nw = (uint32_t)(L - Lw);
  for (uint32_t t = tid; t < nw; t += NT)
    if (total + t < (uint32_t)a.cand_cap) cd[total + t] = (int32_t)(Lw + t);
  return RtSelOut{0, min(total + nw, (uint32_t)a.cand_cap), L_t};
}

// The per-head results of rt_select_head: the unit query, the path and the
// exact flag, the candidate count (L_t on the exact path), the recalled
// entries of a vote, and the optional copies for the caller. cd: the
// candidate list, complete and visible to every thread (after a barrier).
template <int NT>
STDK_DEV void rt_select_store(const RtSelArgs& a, int64_t seg, const RtSelLds<NT>& ls, const RtSelOut& r,
                              const int32_t* cd) {
  const int tid = threadIdx.x;
  for (int e = tid; e < kHeadDim; e += NT) a.qbar[seg * kHeadDim + e] = ls.qb[e];
  const int32_t nc = r.path == 0 ? (int32_t)r.M : (int32_t)r.L_t;
  if (tid == 0) {
    a.path[seg] = r.path;
    a.exact[seg] = r.path != 0;
    a.n_cand[seg] = nc;
    if (a.path_out) a.path_out[seg] = r.path;
    if (a.n_cand_out) a.n_cand_out[seg] = nc;
  }
  if (a.rec_slot && r.path == 0 && tid < min(ls.npick, kMaxVote)) {
    a.rec_slot[seg * kMaxVote + tid] = ls.rec_slot[tid];
    a.rec_rho[seg * kMaxVote + tid] = ls.rec_rho[tid];
  }
  if (a.cand_out)
    for (int i = tid; i < a.cand_cap; i += NT)
      a.cand_out[seg * a.cand_cap + i] = r.path == 0 && i < (int)r.M ? cd[i] : -1;
}

template <bool kLdsBitmap>
__global__ __launch_bounds__(kRtSelThreads) void retopk_select(RtSelArgs a) {
  extern __shared__ uint32_t dyn[];
  __shared__ RtSelLds<kRtSelThreads> ls;
  const int64_t seg = blockIdx.x;
  const int hd = a.head[seg], cnt = a.count[seg];
  uint32_t* bm = kLdsBitmap ? dyn : (a.gbitmap + seg * (int64_t)a.bitmap_words);
  int32_t* cd = a.cand + seg * a.cand_cap;
  const RtSelOut r = rt_select_head<kRtSelThreads, kLdsBitmap>(a, seg, hd, cnt, ls, bm, cd);
  __syncthreads();
  rt_select_store<kRtSelThreads>(a, seg, ls, r, cd);
}

// ---------------------------------------------------------------------------
// retopk_vote: confidence-voted candidates (ReTopK review, "启发 4-5"). The
// access confidence of row i is f(i) = sum over the recalled entries c of
// w_c * [i in S_c], with w_c the entry's cosine, added in fp32 in recall
// order; rows of the union outside the recent window (which is always kept)
// are capped at `budget`, keeping the largest f, ties to the lowest row.
// One workgroup per reuse-path head, on retopk_select's ascending candidate
// list. A row's membership is a byte mask (bit r: in the support of the r-th
// recalled entry), so f takes at most 2^R values: a histogram over the masks
// gives the cut, and an ordered compaction rewrites the list. kRowMasks: the
// masks of all visible rows [0, L_t) fit in LDS and are set directly from
// the supports; otherwise every support row is looked up in the list.
// Dynamic LDS: candidates [cand_cap] int32, masks [cand_cap] bytes, then
// (kRowMasks) row masks [L_t] bytes.
// ---------------------------------------------------------------------------
struct RtVoteArgs {
  const int32_t* exact;     // [S]
  const int32_t* support;   // [S][C][K]
  const int32_t* count;     // [S] valid cache entries (the recalled ones are min(R, count))
  const int32_t* rec_slot;  // [S][kMaxVote]
  const float* rec_rho;     // [S][kMaxVote]
  int32_t* cand;            // [S][cand_cap], rewritten
  int32_t* n_cand;          // [S], rewritten
  int32_t* n_cand_out;      // [S] or null
  int32_t* cand_out;        // [S][cand_cap] or null
  int64_t L_t;              // visible rows; with `step`, the most there can be
  int32_t C, K, R, W, cand_cap, budget;
  const int64_t* step;      // or null: device memory [L_t, t] (L_t clamped to [1, L_t above])
};

constexpr int kVoteThreads = 256;
constexpr int kVoteMaxCand = 16384;  // R*K + W a voting head may hold (LDS)

template <bool kRowMasks>
__global__ __launch_bounds__(kVoteThreads) void retopk_vote(RtVoteArgs a) {
  extern __shared__ __attribute__((aligned(16))) int32_t vdyn[];
  __shared__ uint32_t hist[1 << kMaxVote];
  __shared__ float fm[1 << kMaxVote];
  __shared__ uint32_t tmp[2 * (kVoteThreads / 64) + 2];
  __shared__ int s_mv;
  __shared__ float s_fc;
  __shared__ uint32_t s_need;
  const int64_t seg = blockIdx.x;
  // the head's flags, counts and recall slots are requested together
  const int ex = a.exact[seg];
  const int M = a.n_cand[seg];
  const int cnt = a.count[seg];
  int slot[kMaxVote];
#pragma unroll
  for (int r = 0; r < kMaxVote; ++r) slot[r] = a.rec_slot[seg * kMaxVote + r];
  if (ex) return;
  const int tid = threadIdx.x;
  const int64_t L_t = a.step ? min(a.L_t, max((int64_t)1, a.step[0])) : a.L_t;
  const int64_t lo_recent = L_t - a.W > 0 ? L_t - a.W : 0;
  int32_t* cl = vdyn;
  uint8_t* mk = reinterpret_cast<uint8_t*>(vdyn + a.cand_cap);
  int32_t* cd = a.cand + seg * a.cand_cap;
  {
    // the list, 8 loads per thread in flight
    constexpr int kU = 8;
    for (int i0 = 0; i0 < M; i0 += kVoteThreads * kU) {
      int32_t x[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) x[u] = cd[min(i0 + u * kVoteThreads + tid, M - 1)];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = i0 + u * kVoteThreads + tid;
        if (i < M) {
          cl[i] = x[u];
          mk[i] = 0;
        }
      }
    }
  }
  for (int i = tid; i < (1 << kMaxVote); i += kVoteThreads) hist[i] = 0u;
  __syncthreads();
  // voted rows: the candidates below the recent window (a prefix of the list)
  if (tid == 0) {
    int lo = 0, hi = M;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)cl[mid] < lo_recent) lo = mid + 1;
      else hi = mid;
    }
    s_mv = lo;
  }
  __syncthreads();
  const int Mv = s_mv;
  if (Mv <= a.budget) return;  // nothing to cap: the select's list stands
  const int nrec = min(a.R, cnt);  // R <= kMaxVote, checked on the host
  const int total = nrec * a.K;
  if constexpr (kRowMasks) {
    // masks of the voted rows [0, lo_recent), set straight from the supports
    uint32_t* rm = reinterpret_cast<uint32_t*>(mk + ((a.cand_cap + 15) & ~15));
    const int nw = (int)((lo_recent + 3) >> 2);
    for (int i = tid; i < nw; i += kVoteThreads) rm[i] = 0u;
    __syncthreads();
    constexpr int kU = 8;
    for (int f0 = 0; f0 < total; f0 += kVoteThreads * kU) {
      int32_t x[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int f = min(f0 + u * kVoteThreads + tid, total - 1);
        const int r = f / a.K;
        int sl = slot[0];
#pragma unroll
        for (int j = 1; j < kMaxVote; ++j) sl = r == j ? slot[j] : sl;
        x[u] = a.support[((int64_t)seg * a.C + sl) * a.K + (f - r * a.K)];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int f = f0 + u * kVoteThreads + tid;
        if (f < total && x[u] >= 0 && (int64_t)x[u] < lo_recent)
          atomicOr(&rm[x[u] >> 2], 1u << (8 * (x[u] & 3) + f / a.K));
      }
    }
    __syncthreads();
    for (int i = tid; i < Mv; i += kVoteThreads) mk[i] = (uint8_t)(rm[cl[i] >> 2] >> (8 * (cl[i] & 3)));
  } else {
    // membership: every support row of a recalled entry, found in the list
    int top = 1;
    while (top * 2 <= Mv) top *= 2;
    for (int f = tid; f < total; f += kVoteThreads) {
      const int r = f / a.K, e = f - r * a.K;
      const int32_t x = a.support[((int64_t)seg * a.C + a.rec_slot[seg * kMaxVote + r]) * a.K + e];
      if (x < 0 || (int64_t)x >= lo_recent) continue;
      int lo = 0;  // last index with cl[lo] <= x
      for (int step = top; step > 0; step >>= 1) {
        const int t = lo + step;
        const int32_t v = cl[min(t, Mv - 1)];
        lo = (t < Mv && v <= x) ? t : lo;
      }
      if (cl[lo] == x) atomicOr(reinterpret_cast<uint32_t*>(mk) + (lo >> 2), 1u << (8 * (lo & 3) + r));
    }
  }
  // confidence of each mask, in recall order
  if (tid < (1 << nrec)) {
    float f = 0.f;
    for (int r = 0; r < nrec; ++r)
      if ((tid >> r) & 1) f = f + a.rec_rho[seg * kMaxVote + r];
    fm[tid] = f;
  }
  __syncthreads();
  for (int i = tid; i < Mv; i += kVoteThreads) atomicAdd(&hist[mk[i]], 1u);
  __syncthreads();
  // the cut: the confidence group holding the budget-th row
  if (tid < (1 << nrec) && hist[tid] > 0u) {
    const float f = fm[tid];
    uint32_t above = 0, same = 0;
    for (int m = 0; m < (1 << nrec); ++m) {
      if (fm[m] > f) above += hist[m];
      else if (fm[m] == f) same += hist[m];
    }
    if (above < (uint32_t)a.budget && (uint32_t)a.budget <= above + same) {
      s_fc = f;  // every mask of the group writes the same values
      s_need = (uint32_t)a.budget - above;
    }
  }
  __syncthreads();
  const float fc = s_fc;
  const uint32_t need = s_need;
  // ordered compaction of the voted rows, then the recent window
  const int per = (Mv + kVoteThreads - 1) / kVoteThreads;
  const int i0 = min(Mv, tid * per), i1 = min(Mv, i0 + per);
  uint32_t n_gt = 0, n_eq = 0;
  for (int i = i0; i < i1; ++i) {
    const float f = fm[mk[i]];
    n_gt += f > fc;
    n_eq += f == fc;
  }
  uint32_t gt_before, eq_before, tot_gt, tot_eq;
  block_excl_scan2<kVoteThreads>(n_gt, n_eq, tmp, &gt_before, &eq_before, &tot_gt, &tot_eq);
  uint32_t r = gt_before + min(eq_before, need);
  uint32_t eq_seen = eq_before;
  for (int i = i0; i < i1; ++i) {
    const float f = fm[mk[i]];
    bool take = f > fc;
    if (f == fc) {
      take = eq_seen < need;
      ++eq_seen;
    }
    if (take) cd[r++] = cl[i];
  }
  const int kept = (int)(tot_gt + min(tot_eq, need));
  for (int i = Mv + tid; i < M; i += kVoteThreads) cd[kept + (i - Mv)] = cl[i];
  const int Mn = kept + (M - Mv);
  if (tid == 0) {
    a.n_cand[seg] = Mn;
    if (a.n_cand_out) a.n_cand_out[seg] = Mn;
  }
  if (a.cand_out) {
    __syncthreads();
    for (int i = tid; i < a.cand_cap; i += kVoteThreads) a.cand_out[seg * a.cand_cap + i] = i < Mn ? cd[i] : -1;
  }
}

// Indexed QK over the candidates of reuse-path heads: rows read in place by
// index, no gathered copy.
struct RtRerankArgs {
  const float* q;           // [S][128]
  const char* k;
  int64_t stride_b_bytes, stride_h_bytes;
  const int32_t* exact;     // [S]
  const int32_t* cand;      // [S][cand_cap]
  const int32_t* n_cand;    // [S]
  float* cz;                // [S][cand_cap] scores
  int32_t* sel_row;         // [S][K]
  float* sel_z;             // [S][K]
  int32_t* support_out;     // [S][K]
  int32_t cand_cap, K, Hq, G, nsplit;
  float scale;
  int32_t n_const;          // candidates per head when n_cand is null (exact and n_cand null: every head reranks)
  // Static rows (the int8 recall step with a static window): the rerank
  // also scores the n_static rows of st_tab, into cz_static [S][n_static];
  // they never enter the top-K (softmax . V takes them from there). 0 for
  // ReTopK.
  int32_t n_static;
  int32_t pad_;
  float* cz_static;
  RangeTab st_tab;
};

constexpr int kRerankThreads = 256;
constexpr int kRerankRows = 128;  // candidates per workgroup

template <typename T>
__global__ __launch_bounds__(kRerankThreads) void retopk_rerank(RtRerankArgs a) {
  constexpr int EPL = KvTraits<T>::EPL, LPR = KvTraits<T>::LPR, RPL = KvTraits<T>::RPL, ROWB = KvTraits<T>::ROWB;
  constexpr int NW = kRerankThreads / 64;
  constexpr int GROUPS = NW * RPL;
  const int64_t seg = blockIdx.y;
  if (a.exact && a.exact[seg]) return;
  const int split = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rg = lane / LPR, c = lane % LPR;
  const int b = (int)(seg / a.Hq), hq = (int)(seg % a.Hq), hkv = hq / a.G;
  const int M = a.n_cand ? a.n_cand[seg] : a.n_const;
  const int Mt = M + a.n_static;  // candidates, then the static rows
  const int32_t* cd = a.cand + seg * a.cand_cap;
  float* cz = a.cz + seg * a.cand_cap;
  float* czs = a.cz_static + seg * a.n_static;

  float qr[1][EPL];
  load_q_slice<T, 1>(a.q, seg, c, qr);
  const char* kb = a.k + (int64_t)b * a.stride_b_bytes + (int64_t)hkv * a.stride_h_bytes;
  // row group gid scores candidates j0 + gid + GROUPS*u, u < RU: the indices
  // and then the rows are fetched in one batch each
  constexpr int RU = kRerankRows / GROUPS;
  const int gid = w * RPL + rg;
  const int j0 = split * kRerankRows;
  int32_t row[RU];
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int j = j0 + gid + GROUPS * u;
    row[u] = (j < M) ? cd[j] : (j < Mt ? (int32_t)pos_to_row(a.st_tab, j - M) : -1);
  }
  u32x4 kw[RU];
#pragma unroll
  for (int u = 0; u < RU; ++u) kw[u] = (row[u] >= 0) ? load16(kb + (int64_t)row[u] * ROWB + c * 16) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    float d[1];
    chunk_dots<T, 1>(kw[u], qr, d);
    const float s = group_sum<LPR>(d[0]);
    const int j = j0 + gid + GROUPS * u;
    if (c == 0 && j < M) cz[j] = s * a.scale;
    else if (c == 0 && j < Mt) czs[j - M] = s * a.scale;
  }
}

// Exact top-K among the M candidates of each reuse-path head (ties -> lower
// candidate index, i.e. lower row). One workgroup per head; writes the chosen
// rows (ascending), their scores and the support output.
constexpr int kRerankSelThreads = 256;

__global__ __launch_bounds__(kRerankSelThreads) void retopk_rerank_select(RtRerankArgs a) {
  constexpr int NT = kRerankSelThreads;
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t tmp[NT / 64 + 1];
  __shared__ int s_bin;
  __shared__ uint32_t s_beyond;
  const int64_t seg = blockIdx.x;
  if (a.exact && a.exact[seg]) return;
  const int tid = threadIdx.x;
  const uint32_t M = (uint32_t)(a.n_cand ? a.n_cand[seg] : a.n_const);
  const int32_t* cd = a.cand + seg * a.cand_cap;
  const float* cz = a.cz + seg * a.cand_cap;
  const int K = a.K;
  int32_t* srow = a.sel_row + seg * K;
  float* sz = a.sel_z + seg * K;
  int32_t* so = a.support_out + seg * K;
  const bool take_all = M <= (uint32_t)K;
  constexpr int U = 8;

  uint32_t Tk = 0u, need = (uint32_t)K;
  if (!take_all) {
    uint32_t prefix = 0;
    const int shifts[3] = {21, 10, 0};
    const int bits[3] = {11, 11, 10};
#pragma unroll
    for (int dgt = 0; dgt < 3; ++dgt) {
      const int nb = 1 << bits[dgt];
      for (int i = tid; i < nb; i += NT) h[i] = 0u;
      __syncthreads();
      const int hs = shifts[dgt] + bits[dgt];
      for (uint32_t base = 0; base < M; base += NT * U) {
        uint32_t kv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t j = base + u * NT + tid;
          kv[u] = (j < M) ? f2key(cz[j]) : 0u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t j = base + u * NT + tid;
          if (j < M && (dgt == 0 || (kv[u] >> hs) == prefix))
            atomicAdd(&h[(kv[u] >> shifts[dgt]) & (uint32_t)(nb - 1)], 1u);
        }
      }
      __syncthreads();
      find_bin<NT, true>(h, nb, need, tmp, &s_bin, &s_beyond);
      prefix = (prefix << bits[dgt]) | (uint32_t)(s_bin < 0 ? 0 : s_bin);
      need -= s_beyond;
      __syncthreads();
    }
    Tk = prefix;  // the K-th largest key; keep the first `need` candidates equal to it
  }
  // ordered compaction over candidate index
  const uint32_t per = (M + NT - 1) / NT;
  const uint32_t q0 = min(M, tid * per), q1 = min(M, q0 + per);
  uint32_t n_gt = 0, n_eq = 0;
  for (uint32_t jb = q0; jb < q1; jb += U) {
    uint32_t kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kv[u] = (jb + u < q1) ? f2key(cz[jb + u]) : 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (jb + u < q1) {
        n_gt += take_all || kv[u] > Tk;
        n_eq += !take_all && kv[u] == Tk;
      }
    }
  }
  uint32_t tot_eq, tot_all;
  const uint32_t eq_before = block_excl_scan<NT>(n_eq, tmp, &tot_eq);
  const uint32_t take_eq = min(n_eq, need > eq_before ? need - eq_before : 0u);
  uint32_t r = block_excl_scan<NT>(n_gt + take_eq, tmp, &tot_all);
  uint32_t eq_seen = eq_before;
  for (uint32_t jb = q0; jb < q1; jb += U) {
    float zv[U];
    int32_t rv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (jb + u < q1) {
        zv[u] = cz[jb + u];
        rv[u] = cd[jb + u];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (jb + u >= q1) break;
      const uint32_t key = f2key(zv[u]);
      bool take = take_all || key > Tk;
      if (!take_all && key == Tk) {
        take = eq_seen < need;
        ++eq_seen;
      }
      if (take) {
        if (r < (uint32_t)K) {
          srow[r] = rv[u];
          sz[r] = zv[u];
          so[r] = rv[u];
        }
        ++r;
      }
    }
  }
  for (uint32_t i = tot_all + tid; i < (uint32_t)K; i += NT) {
    srow[i] = -1;
    sz[i] = -INFINITY;
    so[i] = -1;
  }
}

// Staged variant of retopk_rerank_select, same result: the candidate
// scores and rows are read from global memory once, in one batch, into
// dynamic LDS (8 bytes per candidate slot, cand_cap <= kRselStageMax); the
// radix passes, sized to the candidates' key range, and the ordered
// compaction run on that copy. The compaction gives each wave a contiguous
// candidate segment and ranks with ballots.
constexpr int kRselStageMax = 16384;



__global__ __launch_bounds__(kRerankSelThreads) void retopk_rerank_select_lds(RtRerankArgs a) {
  constexpr int NT = kRerankSelThreads, NW = NT / 64;
  extern __shared__ uint32_t rsel_dyn[];
  float* zs = reinterpret_cast<float*>(rsel_dyn);                 // [cand_cap]
  int32_t* rs = reinterpret_cast<int32_t*>(rsel_dyn + a.cand_cap);  // [cand_cap]
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t wc[2][NW];
  __shared__ int s_bin;
  __shared__ uint32_t s_beyond;
  const int64_t seg = blockIdx.x;
  if (a.exact && a.exact[seg]) return;
  const int tid = threadIdx.x;
  const uint32_t M = (uint32_t)(a.n_cand ? a.n_cand[seg] : a.n_const);
  const int32_t* cd = a.cand + seg * a.cand_cap;
  const float* cz = a.cz + seg * a.cand_cap;
  const int K = a.K;
  int32_t* srow = a.sel_row + seg * K;
  float* sz = a.sel_z + seg * K;
  int32_t* so = a.support_out + seg * K;

  // stage: U loads of each array in flight per thread (clamped indices, so
  // the loads carry no condition)
  constexpr int U = 16;
  if (M > 0) {
    for (uint32_t base = 0; base < M; base += NT * U) {
      float zv[U];
      int32_t rv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t j = min(base + u * NT + tid, M - 1);
        zv[u] = cz[j];
        rv[u] = cd[j];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t j = base + u * NT + tid;
        if (j < M) {
          zs[j] = zv[u];
          rs[j] = rv[u];
        }
      }
    }
  }
  __syncthreads();
  const uint32_t tot = lds_topk<NT>(zs, rs, M, K, h, wc, &s_bin, &s_beyond, [&](uint32_t pos, int32_t r, float z) {
    srow[pos] = r;
    sz[pos] = z;
    so[pos] = r;
  });
  for (uint32_t i = tot + tid; i < (uint32_t)K; i += NT) {
    srow[i] = -1;
    sz[i] = -INFINITY;
    so[i] = -1;
  }
}

// ---------------------------------------------------------------------------
// The reuse path of one head after its candidates are known ([RT] 核心方法 1
// and 4): exact scores of the candidates, their top K,
// renormalised softmax . V over them ([RA] Eq. 2) and the push of (q_bar,
// support). Candidate rows and scores stay in LDS from scoring to the
// softmax, so no phase waits on global memory written by another. Scores,
// selection and support equal those of retopk_rerank + retopk_rerank_select
// (same per-lane products and sums); o and lse are summed in this order.
// retopk_attend runs it on retopk_select's candidate list; retopk_reuse
// runs the selector and it in one workgroup, the candidates never leaving LDS.
// ---------------------------------------------------------------------------
struct RtAttendArgs {
  const float* q;          // [S][128]
  const char* k;           // key cache base
  const char* v;           // value cache base (same layout)
  int64_t stride_b_bytes, stride_h_bytes;
  const int32_t* exact;    // [S]: heads on the exact path are skipped
  const int32_t* cand;     // [S][cand_cap] ascending candidate rows
  const int32_t* n_cand;   // [S]
  int32_t* support_out;    // [S][K]
  float* o_out;            // [S][128]
  float* lse_out;          // [S]
  const float* qbar;       // [S][128] unit queries (retopk_select)
  float* q_hat;            // [S][C][128]
  int32_t* support;        // [S][C][K]
  int32_t* head;           // [S]
  int32_t* count;          // [S]
  int32_t cand_cap, K, Hq, G, C;
  float scale;
};

constexpr int kAttThreads = 1024;
constexpr int kAttStaticLds = 42 * 1024;    // static LDS of retopk_attend, rounded up
constexpr int kReuseStaticLds = 46 * 1024;  // static LDS of retopk_reuse, rounded up

// dynamic LDS bytes of retopk_attend: candidate scores and rows, then the
// chosen rows' scores and rows
inline size_t attend_lds_bytes(int cand_cap, int K) { return ((size_t)2 * cand_cap + 2 * (size_t)K) * 4; }

template <typename T, int NT>
struct RtAttLds {
  uint32_t h[kHistBins];
  uint32_t wc[2][NT / 64];
  float red[NT / KvTraits<T>::LPR][kHeadDim];
  float wred[NT / 64];
  float wlo[NT / 64], whi[NT / 64], wsum[NT / 64];
  uint32_t wbad[NT / 64];
  uint32_t lst[kCutList];
  uint32_t s_cut[2];
  uint32_t s_cnt;
  int s_bin;
  uint32_t s_beyond;
};

// rs: the M ascending candidate rows of head seg, in LDS; zs, cz, cr: LDS
// for cand_cap candidate scores, K chosen scores and K chosen rows. qr: this
// thread's query slice (load_q_slice, issued early by the caller). qbar: the
// head's unit query (LDS or global). hd, cnt0: the FIFO's head and count
// before this step.
template <typename T, int NT>
STDK_DEV void rt_attend_head(const RtAttendArgs& a, int64_t seg, const int32_t* rs, uint32_t M, float* zs,
                             float* cz, int32_t* cr, RtAttLds<T, NT>& ls, const float (&qr)[1][KvTraits<T>::EPL],
                             const float* qbar, int hd, int cnt0) {
  constexpr int NW = NT / 64;
  constexpr int EPL = KvTraits<T>::EPL, LPR = KvTraits<T>::LPR, ROWB = KvTraits<T>::ROWB;
  constexpr int NG = NT / LPR;  // row groups: one row per group and load
  constexpr int U = 8;          // value rows per group in flight
  constexpr int UK = 16;        // key rows per group in flight
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int gid = tid / LPR, c = tid % LPR;
  const int b = (int)(seg / a.Hq), hq = (int)(seg % a.Hq), hkv = hq / a.G;
  const int K = a.K;
  for (int i = tid; i < kHistBins; i += NT) ls.h[i] = 0u;  // for lds_cut_linear
  if (tid == 0) ls.s_cnt = 0u;

  // 1. exact scores of the candidates: row group gid takes candidates
  // gid + NG * u, UK rows in flight (loads clamped to the last candidate; a
  // wave skips the products of rows past M). Their minimum and maximum, and
  // whether any is not finite, per wave.
  const int64_t hoff = (int64_t)b * a.stride_b_bytes + (int64_t)hkv * a.stride_h_bytes + c * 16;
  const char* kb = a.k + hoff;
  const uint32_t g0 = (uint32_t)(w * (64 / LPR));  // first row group of this wave
  float lo = INFINITY, hi = -INFINITY;
  bool bad = false;
  for (uint32_t base = 0; base < M; base += NG * UK) {
    u32x4 kw[UK];
#pragma unroll
    for (int u = 0; u < UK; ++u) kw[u] = load16(kb + (int64_t)rs[min(base + gid + NG * u, M - 1)] * ROWB);
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      if (base + g0 + NG * u < M) {  // wave-uniform
        float d[1];
        chunk_dots<T, 1>(kw[u], qr, d);
        const float sc = group_sum<LPR>(d[0]);
        const uint32_t j = base + gid + NG * u;
        if (c == 0 && j < M) {
          const float z = sc * a.scale;
          zs[j] = z;
          lo = fminf(lo, z);
          hi = fmaxf(hi, z);
          bad |= !(fabsf(z) <= __FLT_MAX__);
        }
      }
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  const bool wbad = __ballot(bad) != 0;
  if (lane == 0) {
    ls.wlo[w] = lo;
    ls.whi[w] = hi;
    ls.wbad[w] = wbad;
  }
  __syncthreads();
  bool any_bad = false;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    lo = fminf(lo, ls.wlo[v]);
    hi = fmaxf(hi, ls.whi[v]);
    any_bad |= ls.wbad[v] != 0u;
  }

  const char* vb = a.v + hoff;

  // 2-3. the top K in candidate (= row) order into LDS, with their softmax
  // weights e^{z - m}. Finite scores: m is their maximum (always kept), the
  // cut comes from one histogram pass (lds_cut_linear) and the weights are
  // formed as the rows are emitted. Otherwise (or when that cut gives up):
  // the radix cut, then the maximum of the kept scores, the weights in place
  // (a -inf score weighs 0, a NaN propagates). Each thread sums its weights
  // in emission order; the per-wave sums are added in wave order.
  float m = hi, ps = 0.f;
  uint32_t tot = 0;
  bool weighted = false;
  if (!any_bad && M > 0) {
    TopkCut cut{0u, (uint32_t)K, true};
    bool ok = true;
    if (M > (uint32_t)K)
      ok = hi > lo && 2048.f / (hi - lo) <= __FLT_MAX__ &&
           lds_cut_linear<NT>(zs, M, K, lo, hi, ls.h, ls.lst, &ls.s_cnt, ls.s_cut, &ls.s_bin, &ls.s_beyond, &cut);
    if (ok) {
      tot = lds_emit<NT>(zs, rs, M, K, cut, ls.wc, [&](uint32_t pos, int32_t r, float z) {
        const float wt = __expf(z - m);
        cz[pos] = wt;
        cr[pos] = r;
        ps += wt;
      });
      weighted = true;
    }
  }
  if (!weighted) {
    tot = lds_topk<NT>(zs, rs, M, K, ls.h, ls.wc, &ls.s_bin, &ls.s_beyond, [&](uint32_t pos, int32_t r, float z) {
      cz[pos] = z;
      cr[pos] = r;
    });
  }
  const int nk = (int)min(tot, (uint32_t)K);
  __syncthreads();
  if (!weighted) {
    float zm = -INFINITY;
    for (int i = tid; i < nk; i += NT) zm = fmaxf(zm, cz[i]);
    zm = wave_max(zm);
    if (lane == 0) ls.wred[w] = zm;
    __syncthreads();
    m = ls.wred[0];
#pragma unroll
    for (int v = 1; v < NW; ++v) m = fmaxf(m, ls.wred[v]);
    for (int i = tid; i < nk; i += NT) {
      const float z = cz[i];
      const float wt = z == -INFINITY ? 0.f : __expf(z - m);
      cz[i] = wt;
      ps += wt;
    }
    __syncthreads();
  }
  ps = wave_sum(ps);
  if (lane == 0) ls.wsum[w] = ps;

  // softmax . V over the nk chosen rows, U value rows per row group in flight
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int base = 0; base < nk; base += NG * U) {
    u32x4 vw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) vw[u] = load16(vb + (int64_t)cr[min(base + gid + NG * u, nk - 1)] * ROWB);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + gid + NG * u;
      const float wt = i < nk ? cz[i] : 0.f;
      float x[EPL];
      unpack16<T>(vw[u], x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wt, x[e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) ls.red[gid][c * EPL + e] = acc[e];
  __syncthreads();
  float ssum = 0.f;
#pragma unroll
  for (int v = 0; v < NW; ++v) ssum += ls.wsum[v];
  if (tid < kHeadDim) {
    float o = 0.f;
#pragma unroll 8
    for (int g = 0; g < NG; ++g) o += ls.red[g][tid];
    // ssum == 0: no row (o = 0, lse = -inf); a NaN sum propagates
    a.o_out[seg * kHeadDim + tid] = ssum == 0.f ? 0.f : o / ssum;
    if (tid == 0) a.lse_out[seg] = ssum == 0.f ? -INFINITY : m + __logf(ssum);
  }

  // 4. the support output, and the push of (q_bar, support) into slot
  // (head + 1) mod C; every global store of the head comes after its last load
  const int slot = hd + 1 == a.C ? 0 : hd + 1;
  if (tid < kHeadDim) a.q_hat[(seg * a.C + slot) * kHeadDim + tid] = qbar[tid];
  int32_t* so = a.support_out + seg * K;
  int32_t* dst = a.support + (seg * a.C + slot) * (int64_t)K;
  for (int i = tid; i < K; i += NT) {
    const int32_t r = i < nk ? cr[i] : -1;
    so[i] = r;
    dst[i] = r;
  }
  if (tid == 0) {
    a.head[seg] = slot;
    a.count[seg] = min(cnt0 + 1, a.C);
  }
}

template <typename T>
__global__ __launch_bounds__(kAttThreads) void retopk_attend(RtAttendArgs a) {
  extern __shared__ uint32_t att_dyn[];
  __shared__ RtAttLds<T, kAttThreads> ls;
  const int64_t seg = blockIdx.x;
  if (a.exact[seg]) return;
  float* zs = reinterpret_cast<float*>(att_dyn);                             // [cand_cap]
  int32_t* rs = reinterpret_cast<int32_t*>(att_dyn + a.cand_cap);            // [cand_cap]
  float* cz = reinterpret_cast<float*>(att_dyn + 2 * a.cand_cap);            // [K] chosen scores, then weights
  int32_t* cr = reinterpret_cast<int32_t*>(att_dyn + 2 * a.cand_cap + a.K);  // [K] chosen rows
  const uint32_t M = (uint32_t)a.n_cand[seg];
  const int32_t* cd = a.cand + seg * a.cand_cap;
  const int hd = a.head[seg], cnt0 = a.count[seg];  // read before any barrier; updated at the end
  float qr[1][KvTraits<T>::EPL];
  load_q_slice<T, 1>(a.q, seg, threadIdx.x % KvTraits<T>::LPR, qr);
  for (uint32_t j = threadIdx.x; j < M; j += kAttThreads) rs[j] = cd[j];
  __syncthreads();
  rt_attend_head<T, kAttThreads>(a, seg, rs, M, zs, cz, cr, ls, qr, a.qbar + seg * kHeadDim, hd, cnt0);
}

// ---------------------------------------------------------------------------
// retopk_reuse: one workgroup per head runs the selector and, on the reuse
// path, rt_attend_head on the candidates it leaves in LDS: one launch for
// the whole reuse path, with no candidate list in global memory. Same
// results as retopk_select<true> followed by retopk_attend. Dynamic LDS:
// candidate scores and rows [cand_cap] each, chosen scores and rows [K]
// each, then the bitmap of the visible rows.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kAttThreads) void retopk_reuse(RtSelArgs s, RtAttendArgs a) {
  extern __shared__ uint32_t ru_dyn[];
  __shared__ RtSelLds<kAttThreads> ss;
  __shared__ RtAttLds<T, kAttThreads> ls;
  const int64_t seg = blockIdx.x;
  const int hd = s.head[seg], cnt = s.count[seg];  // read before any barrier; updated at the end
  float* zs = reinterpret_cast<float*>(ru_dyn);
  int32_t* rs = reinterpret_cast<int32_t*>(ru_dyn + a.cand_cap);
  float* cz = reinterpret_cast<float*>(ru_dyn + 2 * a.cand_cap);
  int32_t* cr = reinterpret_cast<int32_t*>(ru_dyn + 2 * a.cand_cap + a.K);
  uint32_t* bm = ru_dyn + 2 * a.cand_cap + 2 * a.K;
  float qr[1][KvTraits<T>::EPL];  // in flight with the selector's loads
  load_q_slice<T, 1>(a.q, seg, threadIdx.x % KvTraits<T>::LPR, qr);
  const RtSelOut r = rt_select_head<kAttThreads, true>(s, seg, hd, cnt, ss, bm, rs);
  __syncthreads();
  if (r.path == 0) rt_attend_head<T, kAttThreads>(a, seg, rs, r.M, zs, cz, cr, ls, qr, ss.qb, hd, cnt);
  rt_select_store<kAttThreads>(s, seg, ss, r, rs);
}

// Fill the FIFO from a history of (query, support) pairs, oldest first.
struct RtInitArgs {
  const float* q_hist;    // [S][n][128]
  const int32_t* s_hist;  // [S][n][K]
  float* q_hat;
  int32_t* support;
  int32_t* head;
  int32_t* count;
  int32_t C, K, n;
  int32_t pad_;
};

__global__ __launch_bounds__(256) void retopk_init(RtInitArgs a) {
  __shared__ float sq[8];
  const int64_t seg = blockIdx.x;
  const int tid = threadIdx.x;
  const int m = min(a.n, a.C);
  for (int s = 0; s < a.C; ++s) {
    float* dq = a.q_hat + (seg * a.C + s) * kHeadDim;
    int32_t* ds = a.support + (seg * a.C + s) * (int64_t)a.K;
    if (s < m) {
      const int64_t src = (int64_t)a.n - m + s;
      // the unit query in the same arithmetic order as retopk_select
      float x[16];
      if (tid < 8) {
        load16f(a.q_hist + (seg * a.n + src) * kHeadDim + 16 * tid, x);
        sq[tid] = sumsq16(x);
      }
      __syncthreads();
      const float nrm = norm_of_parts(sq);
      if (tid < 8) {
#pragma unroll
        for (int e = 0; e < 16; ++e) dq[16 * tid + e] = nrm > 0.f ? x[e] / nrm : 0.f;
      }
      __syncthreads();
      for (int i = tid; i < a.K; i += 256) ds[i] = a.s_hist[(seg * a.n + src) * (int64_t)a.K + i];
    } else {
      if (tid < kHeadDim) dq[tid] = 0.f;
      for (int i = tid; i < a.K; i += 256) ds[i] = -1;
    }
  }
  if (tid == 0) {
    a.head[seg] = m > 0 ? m - 1 : a.C - 1;
    a.count[seg] = m;
  }
}

}  // namespace stdk
