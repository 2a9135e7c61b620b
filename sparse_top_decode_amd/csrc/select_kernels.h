// Exact per-head top-K select over the scan's scores, and the renormalised
// softmax . V over the chosen rows.
//
// The index set is TopK over every score of the segment (ReTopK review,
// "Exact Top-K 的隐藏成本": S_t = TopK(e, K) over all L_t scores), with ties
// resolved towards the lowest row (a reading: the pages leave ties open).
// The output follows Eq. 2 of the RetrievalAttention review ("Approximated
// Attention Formulation"): softmax over the chosen rows only, written with
// the local maximum of "CPU-GPU Co-Execution Architecture".
//
// Steps, all integer work exact:
//  1. k_scan has counted the first radix digit (top 11 bits of the
//     order-preserving key); the bin b* holding the K-th largest key follows.
//  2. topk_filter_select, P workgroups per head: every wave keeps the
//     positions of its slice whose digit is >= b*, in position order, in the
//     slice's own region of the candidate list. A workgroup then counts
//     itself in the head's arrival counter; the one that arrives last (no
//     workgroup ever waits for another) finishes the head:
//  3. radix digits 20..10 and 9..0 on the candidates of bin b* give the exact
//     K-th key T and how many rows with key == T to keep (`need`): chosen =
//     key > T, or key == T among the first `need` such rows in position
//     order. One ordered compaction writes the chosen rows in ascending
//     order. The last workgroup also zeroes the histogram and the counter
//     again, so they need no separate clearing pass per call.
//  4. sparse_sv (many workgroups) computes softmax . V partials over slices
//     of the chosen rows with fp32 accumulation; `combine` merges them.
#pragma once

#include "attend_kernels.h"
#include "device.h"

namespace stdk {

struct Cand {
  uint32_t key;
  int32_t pos;
};

STDK_DEV float key2f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

constexpr int kSelThreads = 1024;
constexpr size_t kSelStaticLds = 14 * 1024;  // static LDS of the select kernel, rounded up

// The first-digit bin that holds the K-th largest key, found by one wave
// straight from the global histogram (no LDS, no barrier): lane l holds the 32
// bins of search ranks [32l, 32l+32) (rank 0 = bin 2047), a wave scan of the
// lane sums finds the owning lane, whose bins the wave then scans together.
// The loads and the search are separate steps so that other loads can be
// issued between them.
STDK_DEV void first_digit_load(const uint32_t* hist, u32x4 (&hv)[8]) {
  const int lane = threadIdx.x & 63;
  // ranks 32l .. 32l+31 are bins 2047-32l down to 2016-32l: 32 consecutive words
  const uint32_t* base = hist + (kHistBins - 32 - 32 * lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) hv[i] = load16(base + 4 * i);
}

// Returns the bin (0 if the histogram holds fewer than `need` items) and, in
// *beyond, the count in the bins above it and in *bin_count the bin's own.
STDK_DEV uint32_t first_digit_search(const u32x4 (&hv)[8], uint32_t need, uint32_t* beyond = nullptr,
                                     uint32_t* bin_count = nullptr) {
  const int lane = threadIdx.x & 63;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) local += hv[i].x + hv[i].y + hv[i].z + hv[i].w;
  const uint32_t incl = wave_incl_scan(local);
  const uint32_t before = incl - local;
  const uint64_t own = __ballot(before < need && need <= incl);
  if (own == 0) {
    if (beyond) *beyond = 0u;
    if (bin_count) *bin_count = 0u;
    return 0u;
  }
  const int L = __ffsll((unsigned long long)own) - 1;
  const uint32_t before_L = lane_read(before, L);
  // lane k < 32 takes rank k of lane L: bin word 31 - k of L's block
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w4[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t t = lane_read(w4[e], L);
      if (lane == 31 - (4 * i + e)) x = t;
    }
  }
  const uint32_t cum = before_L + wave_incl_scan(lane < 32 ? x : 0u);
  const uint64_t hit = __ballot(lane < 32 && cum >= need);
  const int k = __ffsll((unsigned long long)hit) - 1;
  if (beyond) *beyond = lane_read(cum - x, k);
  if (bin_count) *bin_count = lane_read(x, k);
  return (uint32_t)(kHistBins - 1 - (32 * L + k));
}

// ---------------------------------------------------------------------------
// topk_filter_select: P workgroups per segment filter the scores into the
// candidate list; the last of them to arrive selects the head's K rows from
// the candidates. Writes the chosen rows (ascending) and their scores, and
// the index output.
//
// The workgroups of a segment may run on different XCDs, each with its own
// L2. What they hand over (the candidates, the per-workgroup counts and the
// second-digit histogram) is written and read only with agent-scope atomic
// accesses, which are coherent across the XCDs (written through to, and
// read from, the device's coherence point), so no cache-wide write-back or
// invalidate is needed. A workgroup waits until all its accesses are
// complete before it counts itself in; the last workgroup reads only after
// it has seen the full count, so it observes every workgroup's writes.
// ---------------------------------------------------------------------------
struct SelectArgs {
  const float* scores;        // [S][n_pad]
  uint32_t* hist;             // [S][2048] first digit (the scan's counts); zeroed by the last workgroup
  uint32_t* hist1;            // [S][2048] second digit of the candidates in bin b*; zero on entry and exit
  uint32_t* done;             // [S][kCtlWords]: word 0 counts the arrived workgroups; zero on entry and exit
  Cand* list;                 // [S][n_pad]: workgroup x's candidates from position x * nb * 16 * slice on
  uint32_t* wg_cnt;           // [S][P] candidates per workgroup
  Cand* clist;                // [S][n_pad] contiguous copy when it does not fit in LDS
  int64_t n, n_pad;
  int32_t K;
  int32_t slice;              // positions per wave and batch: a multiple of 64, at most 64 * kFselLoads
  int32_t nb;                 // batches per workgroup
  int32_t cache_cap;          // candidates that fit in the LDS copy
  int32_t* sel_row;           // [S][K] chosen rows, ascending, -1 padded
  float* sel_z;               // [S][K] their scores
  int32_t* idx_out;           // [S][K] or null (copy of the chosen rows)
  const int32_t* seg_active;  // [S] or null
  const int64_t* n_dev;       // or null: device memory holding a position count that replaces n when smaller
  RangeTab tab;
  // topk_filter_select_sv only: softmax . V in the last workgroup, over the
  // chosen rows and the n_extra static slots [n, n + n_extra) (rows from the
  // range table, scores from `scores`); o and lse go to o_out and lse_out
  const char* v;              // value cache base
  int64_t stride_b_bytes, stride_h_bytes;
  float* o_out;               // [S][128]
  float* lse_out;             // [S]
  int32_t n_extra, Hq, G, pad_;
  int32_t* ovf;               // topk_filter_lds_sv only: [S] 1 where a head's candidates did not fit, else 0
};

constexpr int kSelectWaves = kSelThreads / 64;
constexpr int kFuseMaxSlots = 4096;   // chosen + static slots a fused softmax . V takes (LDS)
constexpr int kFuseStatic = 4;        // static slots per thread held in registers
static_assert(kSelThreads == 1024, "one thread per bin of the third digit");
constexpr int kFselLoads = 16;  // score loads per lane: a wave's whole slice
constexpr int kCtlWords = 16;   // control words per segment

STDK_DEV void store_agent(Cand* p, Cand c) {
  const uint64_t v = (uint64_t)c.key | ((uint64_t)(uint32_t)c.pos << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
STDK_DEV Cand load_agent(const Cand* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<Cand*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return Cand{(uint32_t)v, (int32_t)(uint32_t)(v >> 32)};
}

// The last workgroup's part after the first two digits: the contiguous
// candidate copy `cl` (in LDS when kLds, else in global memory; separate
// instantiations keep every access in its own address space instead of
// generic accesses, which serialise on both counters), the third digit
// (bits 9..0) over the candidates whose top 22 bits are `pre22`, and the
// ordered compaction. `pre` holds the workgroups' candidate offsets [P + 1];
// `h2` (1024 bins) is zero on entry.
// With kSv the chosen rows and scores also go to crow / czs (LDS) for the
// fused softmax . V. Returns the number of rows taken before the cap at K.
template <bool kLds, bool kSv>
STDK_DEV uint32_t select_tail(const SelectArgs& a, int64_t seg, int P, int64_t span, uint32_t m, uint32_t pre22,
                              uint32_t need, bool take_all, const uint32_t* pre, Cand* cl, uint32_t cap, uint32_t* h2,
                              uint32_t* tmp, int* s_bin, uint32_t* s_beyond, int32_t* crow, float* czs) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int K = a.K;
  const Cand* lst = a.list + seg * a.n_pad;

  // Copy in position order: candidate i lives in the region of the last
  // workgroup r with pre[r] <= i. Candidates whose first two digits lie
  // below the K-th key's (key >> 10 < pre22) cannot be chosen and are
  // dropped. The kept ones keep their order: each wave publishes its ballot
  // count per load slot, wave 0 turns the round's 4 x 16 counts (slot-major,
  // as the positions run) into offsets with one scan, and each lane adds its
  // rank in the ballot. At most `cap` are kept. The third digit is counted
  // for the candidates in the K-th key's second-digit bin. The next round is
  // requested before a round is placed.
  {
    constexpr int CU = 4;
    constexpr uint32_t RND = kSelThreads * CU;  // candidates per round
    __shared__ uint32_t s_cc[CU * kSelectWaves], s_off[CU * kSelectWaves], s_tot;
    uint32_t mk = 0;
    auto load_round = [&](uint32_t base, Cand (&c)[CU]) {
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const uint32_t i = min(base + (uint32_t)(u * kSelThreads + tid), m - 1u);
        int lo = 0, hi = P - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (pre[mid] <= i) lo = mid;
          else hi = mid - 1;
        }
        c[u] = load_agent(lst + (int64_t)lo * span + (i - pre[lo]));
      }
    };
    auto place_round = [&](uint32_t base, const Cand (&c)[CU]) {
      uint64_t km[CU];
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const uint32_t i = base + (uint32_t)(u * kSelThreads + tid);
        km[u] = __ballot(i < m && (take_all || (c[u].key >> 10) >= pre22));
        if (lane == 0) s_cc[u * kSelectWaves + wv] = (uint32_t)__popcll(km[u]);
      }
      __syncthreads();
      if (wv == 0) {
        const uint32_t x = s_cc[lane];
        const uint32_t incl = wave_incl_scan(x);
        s_off[lane] = mk + incl - x;
        if (lane == 63) s_tot = incl;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        if ((km[u] >> lane) & 1ull) {
          const uint32_t j = s_off[u * kSelectWaves + wv] + lane_rank(km[u]);
          if (j < cap) {
            cl[j] = c[u];
            if (!take_all && (c[u].key >> 10) == pre22) atomicAdd(&h2[c[u].key & 0x3FFu], 1u);
          }
        }
      }
      mk += s_tot;
    };
    Cand ca[CU], cb[CU];
    if (m > 0) load_round(0, ca);
    for (uint32_t base = 0; base < m;) {
      if (base + RND < m) load_round(base + RND, cb);
      place_round(base, ca);
      base += RND;
      if (base >= m) break;
      if (base + RND < m) load_round(base + RND, ca);
      place_round(base, cb);
      base += RND;
    }
    m = min(mk, cap);
  }
  __syncthreads();
  uint32_t Tk = 0;
  if (!take_all) {
    if (wv == 0) find_bin_wave<1024, true>(h2, need, s_bin, s_beyond);
    __syncthreads();
    Tk = (pre22 << 10) | (uint32_t)(*s_bin < 0 ? 0 : *s_bin);
    need -= *s_beyond;  // rows with key == Tk to keep, the first ones in position order
  }

  int32_t* srow = a.sel_row + seg * K;
  float* sz = a.sel_z + seg * K;
  int32_t* io = a.idx_out ? a.idx_out + seg * K : nullptr;
  uint32_t tot_all = 0;
  if (m <= 8u * kSelThreads) {
    // Ordered compaction for up to 8 candidates per thread: thread t owns
    // candidates [t*per, (t+1)*per), all read at once. One block scan of
    // (count > Tk, count == Tk) gives each thread its output offset: the
    // rows above Tk before it plus the ties before it that are kept.
    constexpr int U = 8;
    const uint32_t per = (m + kSelThreads - 1) / kSelThreads;
    const uint32_t i0 = min(m, tid * per), i1 = min(m, i0 + per);
    uint32_t n_gt = 0, n_eq = 0;
    for (uint32_t ib = i0; ib < i1; ib += U) {
      uint32_t kv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) kv[u] = cl[min(ib + u, i1 - 1)].key;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (ib + u < i1) {
          n_gt += take_all || kv[u] > Tk;
          n_eq += !take_all && kv[u] == Tk;
        }
      }
    }
    uint32_t gt_before, eq_before, tot_gt, tot_eq;
    block_excl_scan2<kSelThreads>(n_gt, n_eq, tmp, &gt_before, &eq_before, &tot_gt, &tot_eq);
    tot_all = tot_gt + min(tot_eq, need);
    uint32_t r = gt_before + min(eq_before, need);
    uint32_t eq_seen = eq_before;
    for (uint32_t ib = i0; ib < i1; ib += U) {
      Cand cv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) cv[u] = cl[min(ib + u, i1 - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (ib + u < i1) {
          bool take = take_all || cv[u].key > Tk;
          if (!take_all && cv[u].key == Tk) {
            take = eq_seen < need;
            ++eq_seen;
          }
          if (take) {
            if (r < (uint32_t)K) {
              const int32_t row = (int32_t)pos_to_row(a.tab, cv[u].pos);
              srow[r] = row;
              sz[r] = key2f(cv[u].key);
              if (io) io[r] = row;
              if (kSv) {
                crow[r] = row;
                czs[r] = key2f(cv[u].key);
              }
            }
            ++r;
          }
        }
      }
    }
  } else {
    // Ordered compaction for more candidates (contiguous runs per thread
    // would conflict on LDS banks and scatter the stores): wave w owns
    // candidates [w*SEG, (w+1)*SEG), read 64 at a time with consecutive
    // lanes on consecutive candidates. The waves' counts (above Tk, equal to
    // Tk) give each wave its output offset: the rows above Tk before it plus
    // the ties before it that are kept; inside a wave, ballots rank the ties
    // and the taken rows, so consecutive lanes write consecutive slots.
    const uint32_t SEG = ((m + kSelectWaves - 1) / kSelectWaves + 63u) & ~63u;
    const uint32_t s0 = min(m, (uint32_t)wv * SEG), s1 = min(m, s0 + SEG);
    constexpr int CU = 4;  // chunks of 64 whose reads are issued together
    uint32_t cg = 0, ce = 0;
    for (uint32_t jb = s0; jb < s1; jb += 64 * CU) {
      uint32_t kv[CU];
  #pragma unroll
      for (int u = 0; u < CU; ++u) kv[u] = cl[min(jb + 64 * u + lane, s1 - 1)].key;
  #pragma unroll
      for (int u = 0; u < CU; ++u) {
        const bool valid = jb + 64 * u + lane < s1;
        cg += valid && (take_all || kv[u] > Tk);
        ce += valid && !take_all && kv[u] == Tk;
      }
    }
    cg = lane_read(wave_incl_scan(cg), 63);
    ce = lane_read(wave_incl_scan(ce), 63);
    if (lane == 0) {
      tmp[wv] = cg;
      tmp[kSelectWaves + wv] = ce;
    }
    __syncthreads();
    uint32_t out = 0, eq_seen = 0, eq_all = 0;
  #pragma unroll
    for (int v = 0; v < kSelectWaves; ++v) {
      const uint32_t e = tmp[kSelectWaves + v];
      const uint32_t te = min(e, need > eq_all ? need - eq_all : 0u);
      if (v < wv) {
        out += tmp[v] + te;
        eq_seen += e;
      }
      tot_all += tmp[v] + te;
      eq_all += e;
    }
    for (uint32_t jb = s0; jb < s1; jb += 64 * CU) {
      Cand cv[CU];
  #pragma unroll
      for (int u = 0; u < CU; ++u) cv[u] = cl[min(jb + 64 * u + lane, s1 - 1)];
  #pragma unroll
      for (int u = 0; u < CU; ++u) {
        const bool valid = jb + 64 * u + lane < s1;
        const bool gt = valid && (take_all || cv[u].key > Tk);
        const bool eq = valid && !take_all && cv[u].key == Tk;
        const uint64_t em = __ballot(eq);
        const bool take = gt || (eq && eq_seen + lane_rank(em) < need);
        const uint64_t tm = __ballot(take);
        const uint32_t pos = out + lane_rank(tm);
        if (take && pos < (uint32_t)K) {
          const int32_t row = (int32_t)pos_to_row(a.tab, cv[u].pos);
          srow[pos] = row;
          sz[pos] = key2f(cv[u].key);
          if (io) io[pos] = row;
          if (kSv) {
            crow[pos] = row;
            czs[pos] = key2f(cv[u].key);
          }
        }
        out += (uint32_t)__popcll(tm);
        eq_seen += (uint32_t)__popcll(em);
      }
    }
  }
  for (uint32_t i = tot_all + tid; i < (uint32_t)K; i += kSelThreads) {
    srow[i] = -1;
    sz[i] = -INFINITY;
    if (io) io[i] = -1;
  }
  return tot_all;
}

// Grid (P, S), kSelThreads threads: workgroup x of segment s filters the
// positions [x * span, (x + 1) * span), span = nb * 16 * slice; in batch b,
// wave w takes the slice at x * span + (b * 16 + w) * slice.
// Dynamic LDS (last workgroup): pre[P + 1] (the workgroups' candidate
// offsets) then, if the candidates fit, their contiguous copy (position
// order); else the copy goes to clist.
// softmax . V over the T slots in crow / czs (LDS: rows, then scores, which
// become the weights) by the whole workgroup; the finished o and lse of
// segment seg. red (LDS, NG x 128) and wred (kSelectWaves) are scratch.
// Same arithmetic as sparse_sv + combine up to the order of the sums: m is
// the maximum over all slots, the weights e^{z - m} (a -inf score weighs 0,
// a NaN propagates) are summed in a fixed order, and the value rows are
// accumulated per row group, then over the groups in order.
template <typename T, int NT = kSelThreads>
STDK_DEV void tail_softmax_v(const SelectArgs& a, int64_t seg, const int32_t* crow, float* czs, uint32_t Tn,
                             float (*red)[kHeadDim], float* wred) {
  constexpr int EPL = KvTraits<T>::EPL, LPR = KvTraits<T>::LPR, ROWB = KvTraits<T>::ROWB;
  constexpr int NG = NT / LPR;  // row groups
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int gid = tid / LPR, c = tid % LPR;
  const uint32_t g0 = (uint32_t)(wv * (64 / LPR));  // first row group of this wave
  __syncthreads();  // every slot written; the candidate copy (under red) is dead
  float zm = -INFINITY;
  for (uint32_t i = tid; i < Tn; i += NT) zm = fmaxf(zm, czs[i]);
  zm = wave_max(zm);
  if (lane == 0) wred[wv] = zm;
  __syncthreads();
  float m = wred[0];
#pragma unroll
  for (int v = 1; v < NT / 64; ++v) m = fmaxf(m, wred[v]);
  float ps = 0.f;
  for (uint32_t i = tid; i < Tn; i += NT) {
    const float z = czs[i];
    const float wt = z == -INFINITY ? 0.f : __expf(z - m);
    czs[i] = wt;
    ps += wt;
  }
  ps = wave_sum(ps);
  __syncthreads();  // the weights are visible, and every read of m is done
  if (lane == 0) wred[wv] = ps;
  const int b = (int)(seg / a.Hq), hq = (int)(seg % a.Hq), hkv = hq / a.G;
  const char* vb = a.v + (int64_t)b * a.stride_b_bytes + (int64_t)hkv * a.stride_h_bytes + c * 16;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  // U value rows per group in flight, as few as the slot count needs: every
  // load is issued (clamped to the last slot) so that they are all in flight
  // at once, and loads past the slots would only repeat the last row. Each
  // thread adds its rows in the same order whatever U is.
  Tn = (uint32_t)__builtin_amdgcn_readfirstlane((int)Tn);
  auto gather = [&](auto uc, uint32_t base) {
    constexpr int U = decltype(uc)::value;
    u32x4 vw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) vw[u] = load16(vb + (int64_t)crow[min(base + gid + NG * u, Tn - 1)] * ROWB);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + g0 + NG * u < Tn) {  // wave-uniform
        const uint32_t i = base + gid + NG * u;
        const float wt = i < Tn ? czs[i] : 0.f;
        float x[EPL];
        unpack16<T>(vw[u], x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wt, x[e], acc[e]);
      }
    }
  };
  if (Tn == 0) {
    // no slot: nothing is read (o = 0, lse = -inf below)
  } else if (Tn <= 2 * NG) {
    gather(std::integral_constant<int, 2>(), 0u);
  } else if (Tn <= 4 * NG) {
    gather(std::integral_constant<int, 4>(), 0u);
  } else {
    for (uint32_t base = 0; base < Tn; base += NG * 16) gather(std::integral_constant<int, 16>(), base);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) red[gid][c * EPL + e] = acc[e];
  __syncthreads();
  if (tid < kHeadDim) {
    float o = 0.f;
#pragma unroll 8
    for (int g = 0; g < NG; ++g) o += red[g][tid];
    float ssum = 0.f;
#pragma unroll
    for (int v = 0; v < NT / 64; ++v) ssum += wred[v];
    // ssum == 0: no row (o = 0, lse = -inf); a NaN sum propagates
    a.o_out[seg * kHeadDim + tid] = ssum == 0.f ? 0.f : o / ssum;
    if (tid == 0) a.lse_out[seg] = ssum == 0.f ? -INFINITY : m + __logf(ssum);
  }
}

// The exact top-K of the M candidate scores zs (rows rs) staged in LDS,
// ties to the lower candidate index (the candidates ascend by row), in two
// steps: the cut (lds_cut_radix or lds_cut_linear), then an ordered
// compaction (lds_emit) in which wave w owns a contiguous candidate segment
// and ballots rank the taken ones. emit(pos, row, z) receives the chosen
// candidates in ascending order (pos < K); the count before the cap at K is
// returned. NT threads; every thread must call them.
//
// The cut of a top-K selection: keys (f2key of the scores) above Tk are
// taken and, of the keys equal to Tk, the first `need` in candidate order;
// take_all: every candidate (M <= K).
struct TopkCut {
  uint32_t Tk, need;
  bool take_all;
};

// Radix passes over a window of keys [lo, lo + width): the first spans the
// candidates' own key range, each later one exactly the bin that holds the
// K-th key (keys above it were counted in `beyond` already and must not be
// counted again), in 2048 bins of 1 << sh keys; stop at single keys (sh = 0)
// or once that bin is taken whole. The threshold Tk is then the bin's
// smallest key and `need` the number of keys equal to it to take.
template <int NT>
STDK_DEV TopkCut lds_cut_radix(const float* zs, uint32_t M, int K, uint32_t* h, uint32_t (*wc)[NT / 64],
                               int* s_bin_p, uint32_t* s_beyond_p) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (M <= (uint32_t)K) return TopkCut{0u, (uint32_t)K, true};
  int& s_bin = *s_bin_p;
  uint32_t& s_beyond = *s_beyond_p;
  uint32_t need = (uint32_t)K;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (uint32_t j = tid; j < M; j += NT) {
    const uint32_t kv = f2key(zs[j]);
    kmin = min(kmin, kv);
    kmax = max(kmax, kv);
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    wc[0][w] = kmin;
    wc[1][w] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    kmin = min(kmin, wc[0][v]);
    kmax = max(kmax, wc[1][v]);
  }
  __syncthreads();
  uint32_t lo = kmin;
  const uint32_t span = kmax - kmin;
  int sh = span < 2048u ? 0 : (32 - __clz((int)span)) - 11;
  uint64_t width = 2048ull << sh;  // covers [kmin, kmax]
  // at most three passes: sh <= 21 and drops by 11 (to 0) each time
  for (;;) {
    for (int i = tid; i < 2048; i += NT) h[i] = 0u;
    __syncthreads();
    for (uint32_t j = tid; j < M; j += NT) {
      const uint32_t kv = f2key(zs[j]);
      if (kv >= lo && (uint64_t)(kv - lo) < width) atomicAdd(&h[(kv - lo) >> sh], 1u);
    }
    __syncthreads();
    if (w == 0) find_bin_wave<2048, true>(h, need, &s_bin, &s_beyond);
    __syncthreads();
    const int bin = s_bin < 0 ? 0 : s_bin;
    need -= s_beyond;
    lo += (uint32_t)bin << sh;
    width = 1ull << sh;
    if (sh == 0 || h[bin] == need) break;
    sh = sh > 11 ? sh - 11 : 0;
    __syncthreads();
  }
  return TopkCut{lo, need, false};
}

// One histogram pass instead of radix passes when the scores are finite
// with lo < hi (their minimum and maximum): bin(z) = min(2047, (z - lo) *
// 2048 / (hi - lo)) truncated is non-decreasing in z, so every score in a
// higher bin is larger than every score in a lower one. The bin holding the
// K-th largest score is then ranked exactly (its keys, at most kCutList of
// them) to give Tk and the number of keys equal to it to take. h must be
// zero and *s_cnt 0 on entry. Returns false (workgroup-uniform, nothing
// decided) when that bin holds more than kCutList scores.
constexpr int kCutList = 64;
template <int NT>
STDK_DEV bool lds_cut_linear(const float* zs, uint32_t M, int K, float lo, float hi, uint32_t* h,
                             uint32_t* lst, uint32_t* s_cnt, uint32_t* s_cut, int* s_bin, uint32_t* s_beyond,
                             TopkCut* out) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float sc = 2048.f / (hi - lo);
  auto bin_of = [&](float z) { return (int)fminf((z - lo) * sc, 2047.f); };
  for (uint32_t j = tid; j < M; j += NT) atomicAdd(&h[bin_of(zs[j])], 1u);
  __syncthreads();
  if (w == 0) find_bin_wave<2048, true>(h, (uint32_t)K, s_bin, s_beyond);
  __syncthreads();
  const int b = *s_bin;
  const uint32_t need = (uint32_t)K - *s_beyond, cb = h[b];
  if (cb > (uint32_t)kCutList) return false;
  for (uint32_t j = tid; j < M; j += NT) {
    const float z = zs[j];
    if (bin_of(z) == b) lst[atomicAdd(s_cnt, 1u)] = f2key(z);
  }
  __syncthreads();
  if (w == 0) {
    // Tk: the key with fewer than `need` keys above it and at least `need`
    // at or above it
    const uint32_t k = lane < (int)cb ? lst[lane] : 0u;
    uint32_t gt = 0, ge = 0;
    for (uint32_t f = 0; f < cb; ++f) {
      const uint32_t kf = lst[f];
      gt += kf > k;
      ge += kf >= k;
    }
    if (lane < (int)cb && gt < need && need <= ge) {
      s_cut[0] = k;
      s_cut[1] = need - gt;
    }
  }
  __syncthreads();
  *out = TopkCut{s_cut[0], s_cut[1], false};
  return true;
}

// Ordered compaction of the selection: wave w owns candidates [s0, s1);
// emit(pos, row, score) for each taken candidate in candidate order, pos <
// K. Returns the number taken.
template <int NT, typename Emit>
STDK_DEV uint32_t lds_emit(const float* zs, const int32_t* rs, uint32_t M, int K, const TopkCut& cut,
                           uint32_t (*wc)[NT / 64], Emit emit) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool take_all = cut.take_all;
  const uint32_t Tk = cut.Tk, need = cut.need;
  const uint32_t SEG = ((M + NW - 1) / NW + 63u) & ~63u;
  const uint32_t s0 = min(M, (uint32_t)w * SEG), s1 = min(M, s0 + SEG);
  uint32_t cg = 0, ce = 0;
  for (uint32_t j = s0 + lane; j < s1; j += 64) {
    const uint32_t kv = f2key(zs[j]);
    cg += take_all || kv > Tk;
    ce += !take_all && kv == Tk;
  }
  cg = lane_read(wave_incl_scan(cg), 63);
  ce = lane_read(wave_incl_scan(ce), 63);
  if (lane == 0) {
    wc[0][w] = cg;
    wc[1][w] = ce;
  }
  __syncthreads();
  uint32_t out = 0, eq_seen = 0, tot = 0, eq_all = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const uint32_t e = wc[1][v];
    const uint32_t te = min(e, need > eq_all ? need - eq_all : 0u);
    if (v < w) {
      out += wc[0][v] + te;
      eq_seen += e;
    }
    tot += wc[0][v] + te;
    eq_all += e;
  }
  for (uint32_t jb = s0; jb < s1; jb += 64) {
    const uint32_t j = jb + lane;
    const bool valid = j < s1;
    const float z = valid ? zs[j] : 0.f;
    const uint32_t kv = f2key(z);
    const bool gt = valid && (take_all || kv > Tk);
    const bool eq = valid && !take_all && kv == Tk;
    const uint64_t em = __ballot(eq);
    const bool take = gt || (eq && eq_seen + lane_rank(em) < need);
    const uint64_t tm = __ballot(take);
    const uint32_t pos = out + lane_rank(tm);
    if (take && pos < (uint32_t)K) emit(pos, rs[j], z);
    out += (uint32_t)__popcll(tm);
    eq_seen += (uint32_t)__popcll(em);
  }
  return tot;
}


// lds_cut_radix, then lds_emit
template <int NT, typename Emit>
STDK_DEV uint32_t lds_topk(const float* zs, const int32_t* rs, uint32_t M, int K, uint32_t* h,
                           uint32_t (*wc)[NT / 64], int* s_bin_p, uint32_t* s_beyond_p, Emit emit) {
  const TopkCut cut = lds_cut_radix<NT>(zs, M, K, h, wc, s_bin_p, s_beyond_p);
  return lds_emit<NT>(zs, rs, M, K, cut, wc, emit);
}

// The select of a head with one filter workgroup whose candidates fit its
// LDS: the filter left all m of them there (scores zs and positions rs, in
// position order); the exact top K is taken by the one-pass linear-bin cut
// over their range (lds_cut_linear; the radix passes when a score is not
// finite or the K-th score's bin holds more than kCutList), and the chosen
// rows are emitted in order (lds_emit: the key order and lowest-position
// ties of select_tail). Needs no second-digit histogram. `h` (kHistBins
// words) is zero on entry; `scr` holds at least 128 words.
template <bool kSv, int NT = kSelThreads>
STDK_DEV uint32_t select_tail_lds(const SelectArgs& a, int64_t seg, uint32_t m, float* zs, int32_t* rs, uint32_t* h,
                                  uint32_t (*wc)[NT / 64], uint32_t* scr, uint32_t* tmp, int* s_bin,
                                  uint32_t* s_beyond, int32_t* crow, float* czs) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int K = a.K;
  float lo = INFINITY, hi = -INFINITY;
  bool bad = false;
  for (uint32_t i = tid; i < m; i += NT) {
    const float z = zs[i];
    lo = fminf(lo, z);
    hi = fmaxf(hi, z);
    bad |= !__builtin_isfinite(z);
  }
  float* wlo = reinterpret_cast<float*>(scr + kCutList);
  float* whi = wlo + NT / 64;
  uint32_t* s_bad = scr + kCutList + 2 * NT / 64;
  uint32_t* s_cnt = tmp + 2;
  if (tid == 0) {
    *s_bad = 0u;
    *s_cnt = 0u;
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  const bool wbad = __ballot(bad) != 0ull;
  __syncthreads();
  if (lane == 0) {
    wlo[wv] = lo;
    whi[wv] = hi;
    if (wbad) *s_bad = 1u;
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < NT / 64; ++v) {
    lo = fminf(lo, wlo[v]);
    hi = fmaxf(hi, whi[v]);
  }
  TopkCut cut{0u, (uint32_t)K, true};
  if (m > (uint32_t)K) {
    const bool ok = *s_bad == 0u && hi > lo && 2048.f / (hi - lo) <= __FLT_MAX__ &&
                    lds_cut_linear<NT>(zs, m, K, lo, hi, h, scr, s_cnt, tmp, s_bin, s_beyond, &cut);
    if (!ok) cut = lds_cut_radix<NT>(zs, m, K, h, wc, s_bin, s_beyond);
  }
  int32_t* srow = a.sel_row + seg * K;
  float* sz = a.sel_z + seg * K;
  int32_t* io = a.idx_out ? a.idx_out + seg * K : nullptr;
  const uint32_t tot = lds_emit<NT>(zs, rs, m, K, cut, wc, [&](uint32_t pos, int32_t p, float z) {
    const int32_t row = (int32_t)pos_to_row(a.tab, p);
    srow[pos] = row;
    sz[pos] = z;
    if (io) io[pos] = row;
    if (kSv) {
      crow[pos] = row;
      czs[pos] = z;
    }
  });
  for (uint32_t i = min(tot, (uint32_t)K) + tid; i < (uint32_t)K; i += NT) {
    srow[i] = -1;
    sz[i] = -INFINITY;
    if (io) io[i] = -1;
  }
  return tot;
}

template <typename T, bool kSv>
STDK_DEV void fsel_body(const SelectArgs& a) {
  extern __shared__ uint32_t dyn[];
  __shared__ uint32_t h1[kHistBins];  // second digit, this workgroup's candidates in bin b*
  __shared__ uint32_t h2[1024];       // third digit
  __shared__ uint32_t tmp[2 * kSelectWaves + 2];
  __shared__ uint32_t s_wc[2][kSelectWaves];
  __shared__ int s_bin;
  __shared__ uint32_t s_beyond, s_b1, s_beyond1, s_cnt1, s_last, s_ldsm;
  const int64_t seg = blockIdx.y;
  if (a.seg_active && a.seg_active[seg] == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int P = (int)gridDim.x;
  const int K = a.K;
  const int64_t n = a.n_dev ? min(a.n, max((int64_t)0, *a.n_dev)) : a.n;
  const bool take_all = n <= K;
  uint32_t* hg = a.hist + seg * kHistBins;
  uint32_t* h1g = a.hist1 + seg * kHistBins;
  const int64_t span = (int64_t)a.nb * kSelectWaves * a.slice;
  // one workgroup per head whose candidates fit its LDS (decided below from
  // the first-digit histogram): they go straight to its LDS (scores, then
  // positions, after the 2-word prefix slot), no hand-over
  float* lzs = reinterpret_cast<float*>(dyn + 2);
  int32_t* lrs = reinterpret_cast<int32_t*>(dyn + 2 + a.cache_cap);
  uint32_t written = 0;

  // 1. Filter, in nb batches of 16 wave slices. Wave 0 requests the
  // histogram first, then every wave the scores of its first slice; wave 0
  // finds b* (the first digit's bin of the K-th largest key) while they
  // arrive. The candidates (first digit >= b*) go to this workgroup's region
  // in position order: the waves' counts give each wave its offset, ballots
  // rank the lanes. The candidates in bin b* are counted by their second
  // digit (bits 20..10) in LDS; the non-zero bins are then added to the
  // segment's global histogram, after the candidate stores so that those are
  // not queued behind them. A batch's loads are issued after the previous
  // batch's stores: every workgroup of the grid streams at once, which keeps
  // the memory system busy without deeper pipelining inside one (measured:
  // requesting the next batch first changed nothing).
  {
    const float* sc = a.scores + seg * a.n_pad;
    Cand* out = a.list + seg * a.n_pad + (int64_t)blockIdx.x * span;
    // 16-byte loads: chunk u of a wave's slice is positions [256u, 256u +
    // 256), lane l holding 4l .. 4l + 3 (rows start on 64-float boundaries;
    // addresses past the slice stay inside the segment's row and are not used)
    constexpr int NV = kFselLoads / 4;
    float4 v[NV];
    auto load_batch = [&](int bt) {
      const int64_t p0 = (int64_t)blockIdx.x * span + ((int64_t)bt * kSelectWaves + wv) * a.slice;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
      const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sc + min(p0 + 256 * u + 4 * lane, a.n_pad - 4)));
      v[u] = make_float4(x[0], x[1], x[2], x[3]);
    }
    };
    u32x4 hv[8];
    if (wv == 0 && !take_all) first_digit_load(hg, hv);
    load_batch(0);
#pragma unroll
    for (int u = 0; u < kHistBins / kSelThreads; ++u) h1[u * kSelThreads + tid] = 0u;
    if (wv == 0) {
      uint32_t beyond = 0, cnt0 = 0;
      const uint32_t bin = take_all ? 0u : first_digit_search(hv, (uint32_t)K, &beyond, &cnt0);
      if (lane == 0) {
        s_bin = (int)bin;
        s_beyond = beyond;
        // one workgroup per head whose candidates all fit its LDS: it
        // selects there directly and needs no second-digit histogram (with
        // several, reading that histogram overlaps the read of their counts,
        // and the one-pass cut over all candidates costs more than it saves)
        s_ldsm = P == 1 && (take_all ? (uint32_t)n : beyond + cnt0) <= (uint32_t)a.cache_cap ? 1u : 0u;
      }
    }
    __syncthreads();
    const uint32_t b0 = (uint32_t)s_bin;
    const bool lds_mode = s_ldsm != 0u;
    for (int bt = 0;;) {
      const int64_t p0 = (int64_t)blockIdx.x * span + ((int64_t)bt * kSelectWaves + wv) * a.slice;
      const int64_t p1 = min(n, p0 + a.slice);
      // per chunk: each lane's taken positions as 4 bits, their count
      // scanned over the wave (the order is lane, then element)
      uint32_t key[NV][4], bits[NV], ex[NV], ct[NV];
      uint32_t cnt = 0;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        bits[u] = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t p = p0 + 256 * u + 4 * lane + e;
          key[u][e] = f2key(f[e]);
          const uint32_t d0 = key[u][e] >> (32 - kHistBits);
          const bool take = p < p1 && (take_all || d0 >= b0);
          bits[u] |= (take ? 1u : 0u) << e;
          if (take && !take_all && !lds_mode && d0 == b0) atomicAdd(&h1[(key[u][e] >> 10) & 0x7FFu], 1u);
        }
        const uint32_t c = (uint32_t)__popc(bits[u]);
        const uint32_t incl = wave_incl_scan(c);
        ex[u] = incl - c;
        ct[u] = lane_read(incl, 63);
        cnt += ct[u];
      }
      // the counts alternate between two arrays, so one barrier per batch
      // suffices: a batch's array is rewritten two batches later, after
      // every wave has passed the barrier between
      if (lane == 0) s_wc[bt & 1][wv] = cnt;
      __syncthreads();
      uint32_t off = written, tot = 0;
#pragma unroll
      for (int w = 0; w < kSelectWaves; ++w) {
        const uint32_t c = s_wc[bt & 1][w];
        off += w < wv ? c : 0u;
        tot += c;
      }
      if (lds_mode) {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t idx = off + ex[u] + (uint32_t)__popc(bits[u] & ((1u << e) - 1u));
            if (((bits[u] >> e) & 1u) && idx < (uint32_t)a.cache_cap) {
              lzs[idx] = key2f(key[u][e]);
              lrs[idx] = (int32_t)(p0 + 256 * u + 4 * lane + e);
            }
          }
          off += ct[u];
        }
      } else {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if ((bits[u] >> e) & 1u)
              store_agent(out + off + ex[u] + (uint32_t)__popc(bits[u] & ((1u << e) - 1u)),
                          Cand{key[u][e], (int32_t)(p0 + 256 * u + 4 * lane + e)});
          }
          off += ct[u];
        }
      }
      written += tot;
      if (++bt == a.nb) break;
      load_batch(bt);
    }
    if (tid == 0 && !lds_mode) store_agent(a.wg_cnt + seg * P + blockIdx.x, written);
    if (!take_all && !lds_mode) {
#pragma unroll
      for (int u = 0; u < kHistBins / kSelThreads; ++u) {
        const uint32_t c = h1[u * kSelThreads + tid];
        if (c != 0u) atomicAdd(&h1g[u * kSelThreads + tid], c);
      }
    }
  }

  // 2. Arrival: once every wave's writes and histogram adds are complete,
  // thread 0 counts the workgroup in. The workgroup that takes the count to
  // P finishes the segment (and resets the counter); the others are done.
  // (a workgroup that is its head's only one is also its last)
  const bool lds_mode = s_ldsm != 0u;
  if (!lds_mode && !arrive_last(a.done + seg * kCtlWords, (uint32_t)P, &s_last)) return;

  // 3. Select. Wave 0 finds the second digit's bin from the global
  // histogram, then zeroes both histograms for the next call (every
  // workgroup of the segment read the first before it arrived, and its adds
  // to the second are complete); wave 1 builds the workgroups' candidate
  // offsets; every thread clears the third digit's histogram.
  uint32_t* pre = dyn;
  if (wv == 0) {
    if (!take_all && !lds_mode) {
      // 16-byte loads from the device's coherence point (the bins were
      // added there by every workgroup of the segment), all issued before
      // one wait in the same asm statement, so no output register is read
      // or reused while its load is in flight
      const uint32_t* base = h1g + (kHistBins - 32 - 32 * lane);
      u32x4 hv[8];
      __asm__ volatile(
          "global_load_dwordx4 %0, %8, off sc1\n"
          "global_load_dwordx4 %1, %8, off offset:16 sc1\n"
          "global_load_dwordx4 %2, %8, off offset:32 sc1\n"
          "global_load_dwordx4 %3, %8, off offset:48 sc1\n"
          "global_load_dwordx4 %4, %8, off offset:64 sc1\n"
          "global_load_dwordx4 %5, %8, off offset:80 sc1\n"
          "global_load_dwordx4 %6, %8, off offset:96 sc1\n"
          "global_load_dwordx4 %7, %8, off offset:112 sc1\n"
          "s_waitcnt vmcnt(0)"
          : "=&v"(hv[0]), "=&v"(hv[1]), "=&v"(hv[2]), "=&v"(hv[3]), "=&v"(hv[4]), "=&v"(hv[5]), "=&v"(hv[6]),
            "=&v"(hv[7])
          : "v"(base)
          : "memory");
      uint32_t beyond1 = 0, cnt1 = 0;
      const uint32_t b1 = first_digit_search(hv, (uint32_t)K - s_beyond, &beyond1, &cnt1);
      if (lane == 0) {
        s_b1 = b1;
        s_beyond1 = beyond1;
        s_cnt1 = cnt1;
      }
    }
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<u32x4*>(hg + (kHistBins - 32 - 32 * lane) + 4 * i) = z;
      if (!lds_mode) *reinterpret_cast<u32x4*>(h1g + (kHistBins - 32 - 32 * lane) + 4 * i) = z;
    }
  } else if (wv == 1 && !lds_mode) {
    uint32_t run = 0;
    for (int j0 = 0; j0 < P; j0 += 64) {
      const int j = j0 + lane;
      const uint32_t c = j < P ? load_agent(a.wg_cnt + seg * P + j) : 0u;
      const uint32_t incl = wave_incl_scan(c);
      if (j < P) pre[j] = run + incl - c;
      run += lane_read(incl, 63);
    }
    if (lane == 0) pre[P] = run;
  }
  h2[tid] = 0u;
  __syncthreads();
  const uint32_t m = lds_mode ? min(written, (uint32_t)a.cache_cap) : pre[P];
  const uint32_t b0 = take_all || lds_mode ? 0u : (uint32_t)s_bin;
  const uint32_t b1 = take_all || lds_mode ? 0u : s_b1;
  const uint32_t need = take_all || lds_mode ? (uint32_t)K : (uint32_t)K - s_beyond - s_beyond1;
  const uint32_t pre22 = (b0 << 11) | b1;
  // fused softmax . V: the static slots' scores and rows are requested now
  // (clamped loads, kept in registers until the chosen rows are known);
  // chosen and static slots go after the candidate copy, and the softmax's
  // group sums overwrite the copy once it is read
  const int pre_words = (P + 2) & ~1;
  int32_t* crow = nullptr;
  float* czs = nullptr;
  float zst[kFuseStatic];
  int32_t rst[kFuseStatic];
  if (kSv) {
    crow = reinterpret_cast<int32_t*>(dyn + pre_words + 2 * a.cache_cap);
    czs = reinterpret_cast<float*>(crow + (K + a.n_extra));
    if (a.n_extra > 0) {
#pragma unroll
      for (int u = 0; u < kFuseStatic; ++u) {
        const int64_t p = a.n + min(tid + kSelThreads * u, a.n_extra - 1);
        zst[u] = a.scores[seg * a.n_pad + p];
        rst[u] = (int32_t)pos_to_row(a.tab, p);
      }
    }
  }
  // the candidates the copy keeps: those above the K-th key's first-digit
  // bin, and in it those at or above its second-digit bin (both histograms
  // count exactly the candidates); LDS holds them when they fit
  const uint32_t kept = take_all ? m : min(m, s_beyond + s_beyond1 + s_cnt1);
  uint32_t tot;
  if (lds_mode) {
    tot = select_tail_lds<kSv>(a, seg, m, lzs, lrs, h1, s_wc, h2, tmp, &s_bin, &s_beyond, crow, czs);
  } else if (kept <= (uint32_t)a.cache_cap) {
    Cand* cl = reinterpret_cast<Cand*>(dyn + pre_words);
    tot = select_tail<true, kSv>(a, seg, P, span, m, pre22, need, take_all, pre, cl, (uint32_t)a.cache_cap, h2, tmp,
                                 &s_bin, &s_beyond, crow, czs);
  } else {
    tot = select_tail<false, kSv>(a, seg, P, span, m, pre22, need, take_all, pre, a.clist + seg * a.n_pad, m, h2,
                                  tmp, &s_bin, &s_beyond, crow, czs);
  }
  if (kSv) {
    const uint32_t nk = min(tot, (uint32_t)K);
#pragma unroll
    for (int u = 0; u < kFuseStatic; ++u) {
      const int j = tid + kSelThreads * u;
      if (j < a.n_extra) {
        crow[nk + j] = rst[u];
        czs[nk + j] = zst[u];
      }
    }
    tail_softmax_v<T>(a, seg, crow, czs, nk + (uint32_t)a.n_extra,
                      reinterpret_cast<float(*)[kHeadDim]>(dyn + pre_words), reinterpret_cast<float*>(tmp));
  }
}

__global__ __launch_bounds__(kSelThreads) void topk_filter_select(SelectArgs a) { fsel_body<uint16_t, false>(a); }

// topk_filter_select whose last workgroup per segment also forms softmax . V
// over the chosen rows and the static slots (tail_softmax_v): one launch
// instead of three (sparse_sv + combine after the select). Dynamic LDS: as
// topk_filter_select with room for the copy of at least the group sums
// (NG x 128 floats), then K + n_extra rows and as many scores.
template <typename T>
__global__ __launch_bounds__(kSelThreads) void topk_filter_select_sv(SelectArgs a) {
  fsel_body<T, true>(a);
}

// One head per half-size workgroup (kHalfThreads), for heads that each have
// one filter workgroup and are at least twice as many as the CUs (batched
// decode): the head's candidates (first digit >= b*, from the scan's
// histogram) are filtered straight into LDS, cut there (lds_cut_linear, else
// lds_cut_radix, then lds_emit) and followed by softmax . V, as the
// one-workgroup path of topk_filter_select_sv does. Two of these run on a
// CU where one full-size workgroup would, so one head's LDS phases (cut,
// emit, weights) overlap another head's score and value reads, instead of
// every CU taking its heads in two rounds whose phases run in lockstep.
// A head whose candidates exceed cache_cap sets ovf[seg] = 1 and returns
// before it writes anything else (its histogram stays for
// topk_filter_select_sv, launched next with ovf as its head mask); the
// others set ovf[seg] = 0. Dynamic LDS: 2 words, cache_cap scores and rows,
// then K + n_extra rows and scores; the group sums of softmax . V overwrite
// the candidates once they are read (cache_cap >= 64 * NT / LPR).
constexpr int kHalfThreads = 512;
constexpr size_t kHalfStaticLds = 9 * 1024;  // static LDS of topk_filter_lds_sv, rounded up
template <typename T>
__global__ __launch_bounds__(kHalfThreads) __attribute__((amdgpu_waves_per_eu(4))) void topk_filter_lds_sv(
    SelectArgs a) {
  constexpr int NT = kHalfThreads, NW = NT / 64;
  constexpr int NV = kFselLoads / 4;  // a wave's slice of a batch: 4 x 256 positions
  constexpr int SLICE = 64 * kFselLoads;
  extern __shared__ uint32_t dyn[];
  __shared__ uint32_t h[kHistBins];               // the cut's histogram
  __shared__ uint32_t scr[kCutList + 2 * NW + 2];  // the cut's list, wave minima and maxima, flag
  __shared__ uint32_t tmp[2 * NW + 2];
  __shared__ uint32_t s_wc[2][NW];
  __shared__ int s_bin;
  __shared__ uint32_t s_beyond, s_fit;
  const int64_t seg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int K = a.K;
  const uint32_t cap = (uint32_t)a.cache_cap;
  const int64_t n = a.n_dev ? min(a.n, max((int64_t)0, *a.n_dev)) : a.n;
  const bool take_all = n <= K;
  uint32_t* hg = a.hist + seg * kHistBins;
  const float* sc = a.scores + seg * a.n_pad;
  float* lzs = reinterpret_cast<float*>(dyn + 2);
  int32_t* lrs = reinterpret_cast<int32_t*>(dyn + 2 + cap);
  int32_t* crow = reinterpret_cast<int32_t*>(dyn + 2 + 2 * cap);
  float* czs = reinterpret_cast<float*>(crow + (K + a.n_extra));
  const int64_t nbat = max((int64_t)1, (n + NW * SLICE - 1) / (NW * SLICE));

  // 1. Filter. Wave 0 requests the histogram, every wave its first slice
  // (loads clamped inside the segment's row; positions past n are not
  // taken); wave 0 finds b* and whether the candidates fit.
  float4 v[NV];
  auto load_batch = [&](int64_t bt) {
    const int64_t p0 = (bt * NW + wv) * SLICE;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sc + min(p0 + 256 * u + 4 * lane, a.n_pad - 4)));
      v[u] = make_float4(x[0], x[1], x[2], x[3]);
    }
  };
  u32x4 hv[8];
  if (wv == 0 && !take_all) first_digit_load(hg, hv);
  load_batch(0);
  for (int i = tid; i < kHistBins; i += NT) h[i] = 0u;
  if (wv == 0) {
    uint32_t beyond = 0, cnt0 = 0;
    const uint32_t bin = take_all ? 0u : first_digit_search(hv, (uint32_t)K, &beyond, &cnt0);
    if (lane == 0) {
      s_bin = (int)bin;
      s_fit = (take_all ? (uint64_t)n : (uint64_t)beyond + cnt0) <= cap ? 1u : 0u;
    }
  }
  __syncthreads();
  if (s_fit == 0u) {
    if (tid == 0) a.ovf[seg] = 1;
    return;
  }
  if (tid == 0) a.ovf[seg] = 0;
  if (wv == 0) {
    // the histogram is read: zeroed for the next call
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(hg + (kHistBins - 32 - 32 * lane) + 4 * i) = z;
  }
  const uint32_t b0 = (uint32_t)s_bin;
  uint32_t written = 0;
  for (int64_t bt = 0;;) {
    const int64_t p0 = (bt * NW + wv) * SLICE;
    const int64_t p1 = min(n, p0 + SLICE);
    // per chunk: each lane's taken positions as 4 bits, their count scanned
    // over the wave (the order is lane, then element)
    uint32_t key[NV][4], bits[NV], ex[NV], ct[NV];
    uint32_t cnt = 0;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      bits[u] = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t p = p0 + 256 * u + 4 * lane + e;
        key[u][e] = f2key(f[e]);
        const bool take = p < p1 && (take_all || (key[u][e] >> (32 - kHistBits)) >= b0);
        bits[u] |= (take ? 1u : 0u) << e;
      }
      const uint32_t c = (uint32_t)__popc(bits[u]);
      const uint32_t incl = wave_incl_scan(c);
      ex[u] = incl - c;
      ct[u] = lane_read(incl, 63);
      cnt += ct[u];
    }
    // the counts alternate between two arrays: one barrier per batch
    if (lane == 0) s_wc[bt & 1][wv] = cnt;
    __syncthreads();
    uint32_t off = written, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t c = s_wc[bt & 1][w];
      off += w < wv ? c : 0u;
      tot += c;
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t idx = off + ex[u] + (uint32_t)__popc(bits[u] & ((1u << e) - 1u));
        if (((bits[u] >> e) & 1u) && idx < cap) {
          lzs[idx] = key2f(key[u][e]);
          lrs[idx] = (int32_t)(p0 + 256 * u + 4 * lane + e);
        }
      }
      off += ct[u];
    }
    written += tot;
    if (++bt == nbat) break;
    load_batch(bt);
  }

  // 2. Select in LDS, with the static slots' scores and rows requested first
  float zst[kFuseStatic];
  int32_t rst[kFuseStatic];
  if (a.n_extra > 0) {
#pragma unroll
    for (int u = 0; u < kFuseStatic; ++u) {
      const int64_t p = a.n + min(tid + NT * u, a.n_extra - 1);
      zst[u] = sc[p];
      rst[u] = (int32_t)pos_to_row(a.tab, p);
    }
  }
  __syncthreads();  // every candidate is in LDS
  const uint32_t tot = select_tail_lds<true, NT>(a, seg, min(written, cap), lzs, lrs, h, s_wc, scr, tmp, &s_bin,
                                                 &s_beyond, crow, czs);

  // 3. Softmax . V over the chosen rows and the static slots
  const uint32_t nk = min(tot, (uint32_t)K);
#pragma unroll
  for (int u = 0; u < kFuseStatic; ++u) {
    const int j = tid + NT * u;
    if (j < a.n_extra) {
      crow[nk + j] = rst[u];
      czs[nk + j] = zst[u];
    }
  }
  tail_softmax_v<T, NT>(a, seg, crow, czs, nk + (uint32_t)a.n_extra, reinterpret_cast<float(*)[kHeadDim]>(dyn + 2),
                        reinterpret_cast<float*>(tmp));
}



// ---------------------------------------------------------------------------
// topk_select_lds: the select of a short segment (n <= kSelLdsMax positions)
// in one workgroup, without the filter's hand-over between workgroups: all
// n scores to LDS, the exact top K there (the same key order and
// lowest-position ties as topk_filter_select), the chosen rows in ascending
// order. The segment's first-digit histogram (the scan's counts) is zeroed
// for the next call. Dynamic LDS: n scores, then n positions (each array
// rounded up to 64 entries).
//
// topk_select_lds_sv<T> goes on to softmax . V over the chosen rows and the
// n_extra static slots (tail_softmax_v) in the same workgroup; the chosen
// rows go to idx_out only (the workspace's chosen-row arrays are not
// written). Dynamic LDS: the larger of the two arrays above and the
// softmax's group sums, then K + n_extra rows and as many scores.
// ---------------------------------------------------------------------------
constexpr int kSelLdsMax = 8192;
inline __host__ __device__ uint32_t sel_lds_stride(int64_t n) { return (uint32_t)((n + 63) & ~(int64_t)63); }
// bytes in front of the slot arrays of topk_select_lds_sv
template <typename T>
inline __host__ __device__ size_t sel_lds_sv_head(int64_t n) {
  const size_t arrays = (size_t)2 * sel_lds_stride(n) * 4;
  const size_t red = (size_t)(kSelThreads / KvTraits<T>::LPR) * kHeadDim * 4;
  return arrays > red ? arrays : red;
}

template <typename T, bool kSv>
STDK_DEV void sel_lds_body(const SelectArgs& a) {
  extern __shared__ uint32_t sl_dyn[];
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t wc[2][kSelectWaves];
  __shared__ float wlo[kSelectWaves], whi[kSelectWaves];
  __shared__ uint32_t lst[kCutList], s_cut[2], s_cnt, s_bad;
  __shared__ int s_bin;
  __shared__ uint32_t s_beyond;
  const int64_t seg = blockIdx.x;
  if (a.seg_active && a.seg_active[seg] == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int K = a.K;
  const uint32_t n = (uint32_t)(a.n_dev ? min(a.n, max((int64_t)0, *a.n_dev)) : a.n);
  float* zs = reinterpret_cast<float*>(sl_dyn);
  int32_t* rs = reinterpret_cast<int32_t*>(sl_dyn + sel_lds_stride(a.n));
  const float* sc = a.scores + seg * a.n_pad;
  // the static slots' scores and rows, requested first
  float zst[kFuseStatic];
  int32_t rst[kFuseStatic];
  if (kSv && a.n_extra > 0) {
#pragma unroll
    for (int u = 0; u < kFuseStatic; ++u) {
      const int64_t p = a.n + min(tid + kSelThreads * u, a.n_extra - 1);
      zst[u] = sc[p];
      rst[u] = (int32_t)pos_to_row(a.tab, p);
    }
  }
  // scores to LDS, with their range (lo, hi) and whether any is not finite
  constexpr int U = 8;
  float lo = INFINITY, hi = -INFINITY;
  bool bad = false;
  for (uint32_t j0 = 0; j0 < n; j0 += U * kSelThreads) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = sc[min(j0 + (uint32_t)(u * kSelThreads + tid), n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t j = j0 + (uint32_t)(u * kSelThreads + tid);
      if (j < n) {
        zs[j] = v[u];
        rs[j] = (int32_t)j;
        lo = fminf(lo, v[u]);
        hi = fmaxf(hi, v[u]);
        bad |= !__builtin_isfinite(v[u]);
      }
    }
  }
  for (int i = tid; i < kHistBins; i += kSelThreads) h[i] = 0u;
  if (tid == 0) {
    s_cnt = 0u;
    s_bad = 0u;
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  const bool wbad = __ballot(bad) != 0ull;
  __syncthreads();
  if (lane == 0) {
    wlo[w] = lo;
    whi[w] = hi;
    if (wbad) s_bad = 1u;
  }
  uint32_t* hg = a.hist + seg * kHistBins;
  for (int i = tid; i < kHistBins; i += kSelThreads) hg[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int v = 0; v < kSelectWaves; ++v) {
    lo = fminf(lo, wlo[v]);
    hi = fmaxf(hi, whi[v]);
  }
  // the cut: one histogram pass over [lo, hi] (lds_cut_linear) when the
  // scores are finite and spread, else (or when the K-th score's bin is
  // crowded) the radix passes; both give the same exact cut
  TopkCut cut{0u, (uint32_t)K, true};
  if (n > (uint32_t)K) {
    const bool ok = s_bad == 0u && hi > lo && 2048.f / (hi - lo) <= __FLT_MAX__ &&
                    lds_cut_linear<kSelThreads>(zs, n, K, lo, hi, h, lst, &s_cnt, s_cut, &s_bin, &s_beyond, &cut);
    if (!ok) cut = lds_cut_radix<kSelThreads>(zs, n, K, h, wc, &s_bin, &s_beyond);
  }
  int32_t* srow = a.sel_row + seg * K;
  float* sz = a.sel_z + seg * K;
  int32_t* io = a.idx_out ? a.idx_out + seg * K : nullptr;
  int32_t* crow = reinterpret_cast<int32_t*>(sl_dyn + (kSv ? sel_lds_sv_head<T>(a.n) / 4 : 0));
  float* czs = reinterpret_cast<float*>(crow + (K + a.n_extra));
  const uint32_t tot = lds_emit<kSelThreads>(zs, rs, n, K, cut, wc, [&](uint32_t pos, int32_t p, float z) {
    const int32_t row = (int32_t)pos_to_row(a.tab, p);
    if (kSv) {
      crow[pos] = row;
      czs[pos] = z;
    } else {
      srow[pos] = row;
      sz[pos] = z;
    }
    if (io) io[pos] = row;
  });
  const uint32_t nk = min(tot, (uint32_t)K);
  for (uint32_t i = nk + tid; i < (uint32_t)K; i += kSelThreads) {
    if (!kSv) {
      srow[i] = -1;
      sz[i] = -INFINITY;
    }
    if (io) io[i] = -1;
  }
  if (kSv) {
    // the slots' arrays lie beyond the scores read by lds_emit; the group
    // sums that overwrite those are written after tail_softmax_v's barrier
#pragma unroll
    for (int u = 0; u < kFuseStatic; ++u) {
      const int j = tid + kSelThreads * u;
      if (j < a.n_extra) {
        crow[nk + j] = rst[u];
        czs[nk + j] = zst[u];
      }
    }
    tail_softmax_v<T>(a, seg, crow, czs, nk + (uint32_t)a.n_extra, reinterpret_cast<float(*)[kHeadDim]>(sl_dyn),
                      wlo);
  }
}

__global__ __launch_bounds__(kSelThreads) void topk_select_lds(SelectArgs a) { sel_lds_body<uint16_t, false>(a); }

template <typename T>
__global__ __launch_bounds__(kSelThreads) void topk_select_lds_sv(SelectArgs a) {
  sel_lds_body<T, true>(a);
}

// ---------------------------------------------------------------------------
// sparse_sv: gathered-row softmax . V, kSvRows chosen rows per workgroup;
// partial (m, s, o) per workgroup, merged by `combine`.
// ---------------------------------------------------------------------------
// The ReTopK cache push (q_bar and the chosen rows into FIFO slot
// (head + 1) mod C of every head), done by one workgroup per head of the
// softmax . V launch: every thread reads head and count before the kernel's
// barriers, and thread 0 advances them after the last one.
struct SvPush {
  const float* qbar;          // [S][128]
  const int32_t* support_in;  // [S][K]
  float* q_hat;               // [S][C][128]
  int32_t* support;           // [S][C][K]
  int32_t* head;              // [S]
  int32_t* count;             // [S]
  int32_t C, K;
};

template <int NT>
STDK_DEV int sv_push_copy(const SvPush& p, int64_t seg, int* cnt_out) {
  const int tid = threadIdx.x;
  const int hd = p.head[seg];
  *cnt_out = p.count[seg];
  const int slot = hd + 1 == p.C ? 0 : hd + 1;
  if (tid < kHeadDim) p.q_hat[(seg * p.C + slot) * kHeadDim + tid] = p.qbar[seg * kHeadDim + tid];
  for (int i = tid; i < p.K; i += NT) p.support[(seg * p.C + slot) * (int64_t)p.K + i] = p.support_in[seg * p.K + i];
  return slot;
}

struct SvArgs {
  const char* v;              // value cache base
  int64_t stride_b_bytes, stride_h_bytes;
  const int32_t* sel_row;     // [S][k_top], -1 = unused slot
  const float* sel_z;         // [S][k_top]
  float* part;                // [S][nsplit][kPartStride]
  const int32_t* seg_active;  // [S] or null
  int32_t K, nsplit, Hq, G;   // K = row slots per segment: k_top chosen rows, then the static rows
  int32_t k_top, pad_;
  // Row slots k_top .. K-1 are the static positions [n, n + K - k_top),
  // taken whole: their rows come from the range table, their scores from the
  // scan's score array.
  const float* scores;        // [S][n_pad]
  int64_t n, n_pad;
  RangeTab tab;
  // sparse_sv_ds only: the finished outputs and the number of segments
  float* o_out;               // [S][128]
  float* lse_out;             // [S]
  int64_t n_seg;
  int32_t do_push, pad2_;
  SvPush push;
  int64_t* step_adv;          // or null: workgroup 0 adds 1 to both words ([L_t, t]) when it starts (the
                              // launch is the last of its step; nothing in it reads them)
  // sparse_sv_scored only: the queries and the key cache its rows are
  // scored from
  const float* q;             // [S][128]
  const char* kc;             // key cache base (same layout as the values)
  float scale;
  int32_t pad3_;
};

constexpr int kSvThreads = 256;
constexpr int kSvRows = 64;  // chosen rows per workgroup (a multiple of 64)

template <typename T>
__global__ __launch_bounds__(kSvThreads) void sparse_sv(SvArgs a) {
  constexpr int EPL = KvTraits<T>::EPL, LPR = KvTraits<T>::LPR, ROWB = KvTraits<T>::ROWB;
  constexpr int NG = kSvThreads / LPR;  // row groups
  constexpr int RU = kSvRows / NG;      // rows per row group
  __shared__ int32_t rows[kSvRows];
  __shared__ float wts[kSvRows];
  __shared__ float red[NG][kHeadDim];
  __shared__ float s_m;
  const int64_t seg = blockIdx.y;
  if (a.step_adv && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    a.step_adv[0] += 1;
    a.step_adv[1] += 1;
  }
  if (a.seg_active && a.seg_active[seg] == 0) return;
  const int split = blockIdx.x;
  const bool pusher = a.do_push && split == 0;
  int push_slot = 0, push_cnt = 0;
  if (pusher) push_slot = sv_push_copy<kSvThreads>(a.push, seg, &push_cnt);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int gid = tid / LPR, c = tid % LPR;
  const int b = (int)(seg / a.Hq), hq = (int)(seg % a.Hq), hkv = hq / a.G;
  const int j0 = split * kSvRows;
  const int nr = min(kSvRows, a.K - j0);
  // wave 0: the chosen rows of this slice (kSvRows / 64 per lane), their
  // maximum and weights
  if (w == 0) {
    constexpr int PL = kSvRows / 64;
    int32_t r[PL];
    float z[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      r[i] = -1;
      z[i] = -INFINITY;
      const int jj = 64 * i + lane;
      const int j = j0 + jj;
      if (jj < nr) {
        if (j < a.k_top) {
          // row and score requested together; a padding slot (row -1)
          // weighs nothing
          r[i] = a.sel_row[seg * a.k_top + j];
          const float zz = a.sel_z[seg * a.k_top + j];
          z[i] = r[i] >= 0 ? zz : -INFINITY;
        } else {
          const int64_t p = a.n + (j - a.k_top);
          r[i] = (int32_t)pos_to_row(a.tab, p);
          z[i] = a.scores[seg * a.n_pad + p];
        }
      }
    }
    float zm = z[0];
#pragma unroll
    for (int i = 1; i < PL; ++i) zm = fmaxf(zm, z[i]);
    const float m = wave_max(zm);
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      rows[64 * i + lane] = r[i];
      wts[64 * i + lane] = z[i] == -INFINITY ? 0.f : __expf(z[i] - m);  // a NaN score propagates
    }
    if (lane == 0) s_m = m;
  }
  __syncthreads();
  const char* vb = a.v + (int64_t)b * a.stride_b_bytes + (int64_t)hkv * a.stride_h_bytes + c * 16;
  u32x4 vw[RU];
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int32_t r = rows[gid + NG * u];
    vw[u] = (r >= 0) ? load16(vb + (int64_t)r * ROWB) : u32x4{0u, 0u, 0u, 0u};
  }
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const float wt = wts[gid + NG * u];
    float x[EPL];
    unpack16<T>(vw[u], x);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wt, x[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) red[gid][c * EPL + e] = acc[e];
  __syncthreads();
  float* part = a.part + (seg * a.nsplit + split) * kPartStride;
  if (tid < kHeadDim) {
    float o = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) o += red[g][tid];
    part[4 + tid] = o;
  }
  if (w == 0) {
    // the weight sum in a fixed order: lane-strided partial sums, then the
    // wave reduction
    float ws = 0.f;
#pragma unroll
    for (int i = 0; i < kSvRows / 64; ++i) ws += wts[64 * i + lane];
    const float s = wave_sum(ws);
    if (lane == 0) {
      part[0] = s_m;
      part[1] = s;
    }
  }
  if (pusher && tid == 0) {
    a.push.head[seg] = push_slot;
    a.push.count[seg] = min(push_cnt + 1, a.push.C);
  }
}

// ---------------------------------------------------------------------------
// sparse_sv_ds: the same softmax . V with the work split over value
// dimensions instead of rows. Workgroup (head, slice) takes every chosen row
// of its head and the kDsDims value dimensions of its slice, so it finishes
// its part of o by itself: no partials and no combine pass. Each workgroup
// stages the head's rows and scores in LDS (8 bytes per slot) and takes
// their maximum m, requests its slice of the first value rows, and forms
// the sum of the weights e^{z - m} while they arrive (in a fixed order,
// identical in every slice). Used where the heads and their rows are few:
// the gathers of 32 B pieces need more requests per byte than whole rows.
//
// The kDsSlices workgroups of one head are placed on the same XCD (the
// hardware deals consecutive workgroups to the 8 XCDs in turn), so the
// value rows they share are fetched from HBM once, into that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kDsThreads = 256;
constexpr int kDsDims = 16;                      // value dims per workgroup
constexpr int kDsSlices = kHeadDim / kDsDims;    // workgroups per head
constexpr int kDsMaxSlots = 1024;                // rows per head (LDS staging, one batch of loads)
constexpr int kDsMaxHeads = 128;                 // beyond this the row split fills the chip better
constexpr int kDsXcds = 8;

template <typename T>
__global__ __launch_bounds__(kDsThreads) void sparse_sv_ds(SvArgs a) {
  constexpr int EPL = KvTraits<T>::EPL, ROWB = KvTraits<T>::ROWB;
  constexpr int LPS = kDsDims / EPL;         // lanes per row slice (16 B each)
  constexpr int NG = kDsThreads / LPS;       // row groups
  constexpr int NW = kDsThreads / 64;
  constexpr int U = 8;                       // value loads in flight per thread
  extern __shared__ uint32_t ds_dyn[];
  const int KT = a.K;                        // row slots of the head
  int32_t* rows = reinterpret_cast<int32_t*>(ds_dyn);     // [KT]
  float* zs = reinterpret_cast<float*>(ds_dyn + KT);     // [KT] scores, -inf for empty slots
  constexpr int NP = kDsThreads / kDsDims;  // partial sums per value dim
  constexpr int GP = NG / NP;               // row groups per partial sum
  __shared__ float red[NG][kDsDims];
  __shared__ float red2[NP][kDsDims];
  __shared__ float wmax[NW], wsum[NW];
  // XCD-aware placement: block L runs on XCD L % 8; the slices of one head
  // share it
  const int L = blockIdx.x;
  const int xcd = L % kDsXcds, kk = L / kDsXcds;
  const int64_t seg = (int64_t)(kk / kDsSlices) * kDsXcds + xcd;
  const int slice = kk % kDsSlices;
  if (a.step_adv && L == 0 && threadIdx.x == 0) {
    a.step_adv[0] += 1;
    a.step_adv[1] += 1;
  }
  if (seg >= a.n_seg) return;  // the grid covers the segments rounded up to a multiple of 8
  if (a.seg_active && a.seg_active[seg] == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = (int)(seg / a.Hq), hq = (int)(seg % a.Hq), hkv = hq / a.G;
  const bool pusher = a.do_push && slice == 0;
  int push_slot = 0, push_cnt = 0;
  if (pusher) push_slot = sv_push_copy<kDsThreads>(a.push, seg, &push_cnt);

  // 1. rows and scores of every slot, and the maximum: the chosen rows in
  // batches of plain loads, then the static rows (rows from the range table)
  float zm = -INFINITY;
  const int kt = min(a.k_top, KT);
  for (int j0 = 0; j0 < kt; j0 += kDsThreads * 4) {
    int32_t r[4];
    float z[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = min(j0 + u * kDsThreads + tid, kt - 1);
      r[u] = a.sel_row[seg * a.k_top + j];
      z[u] = a.sel_z[seg * a.k_top + j];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * kDsThreads + tid;
      if (j < kt) {
        const float zz = r[u] >= 0 ? z[u] : -INFINITY;
        rows[j] = r[u];
        zs[j] = zz;
        zm = fmaxf(zm, zz);
      }
    }
  }
  const int nst = KT - kt;
  for (int i0 = 0; i0 < nst; i0 += kDsThreads * 2) {
    float z[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) z[u] = a.scores[seg * a.n_pad + a.n + min(i0 + u * kDsThreads + tid, nst - 1)];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = i0 + u * kDsThreads + tid;
      if (i < nst) {
        rows[kt + i] = (int32_t)pos_to_row(a.tab, a.n + i);
        zs[kt + i] = z[u];
        zm = fmaxf(zm, z[u]);
      }
    }
  }
  zm = wave_max(zm);
  if (lane == 0) wmax[w] = zm;
  __syncthreads();
  float m = wmax[0];
#pragma unroll
  for (int v = 1; v < NW; ++v) m = fmaxf(m, wmax[v]);
  auto weight = [&](float z) { return z == -INFINITY ? 0.f : __expf(z - m); };  // a NaN score propagates

  // 2. the slice of every value row, U rows per thread in flight; the first
  // batch is requested before the weight sum is formed
  const int gid = tid / LPS, c = tid % LPS;
  const char* vb = a.v + (int64_t)b * a.stride_b_bytes + (int64_t)hkv * a.stride_h_bytes +
                   slice * kDsDims * (int)sizeof(T) + c * 16;
  auto issue = [&](int j0, u32x4 (&vw)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t r = rows[min(j0 + NG * u, KT - 1)];
      vw[u] = load16(vb + (int64_t)(r >= 0 ? r : 0) * ROWB);
    }
  };
  u32x4 vw[U];
  issue(gid, vw);
  // weight sum: thread-strided partial sums in slot order, the wave
  // butterflies, then the waves in order (the same in every slice)
  float ps = 0.f;
  for (int j = tid; j < KT; j += kDsThreads) ps += weight(zs[j]);
  ps = wave_sum(ps);
  if (lane == 0) wsum[w] = ps;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int j0 = gid;;) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + NG * u;
      const float wt = j < KT ? weight(zs[j]) : 0.f;
      float x[EPL];
      unpack16<T>(vw[u], x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wt, x[e], acc[e]);
    }
    j0 += NG * U;
    if (j0 >= KT) break;
    issue(j0, vw);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) red[gid][c * EPL + e] = acc[e];
  __syncthreads();
  float ssum = 0.f;
#pragma unroll
  for (int v = 0; v < NW; ++v) ssum += wsum[v];
  // 3. sum over the row groups in a fixed order (GP consecutive groups per
  // thread, then the NP partial sums); the slice's outputs
  {
    const int d = tid % kDsDims, pp = tid / kDsDims;
    float o = 0.f;
#pragma unroll
    for (int g = 0; g < GP; ++g) o += red[pp * GP + g][d];
    red2[pp][d] = o;
  }
  __syncthreads();
  if (tid < kDsDims) {
    float o = 0.f;
#pragma unroll
    for (int g = 0; g < NP; ++g) o += red2[g][tid];
    // ssum == 0: no row (o = 0, lse = -inf); a NaN sum propagates
    a.o_out[seg * kHeadDim + slice * kDsDims + tid] = ssum == 0.f ? 0.f : o / ssum;
    if (slice == 0 && tid == 0) a.lse_out[seg] = ssum == 0.f ? -INFINITY : m + __logf(ssum);
  }
  if (pusher && tid == 0) {
    a.push.head[seg] = push_slot;
    a.push.count[seg] = min(push_cnt + 1, a.push.C);
  }
}

// ---------------------------------------------------------------------------
// sparse_sv_scored: sparse_sv for a row list that comes without scores (the
// int8 recall step with recall_k == top_k, whose superset is the answer).
// Each workgroup scores its own kSvRows slots from the key cache, z =
// scale * (q . k) in fp32 (each lane's 16-byte chunk, then the sum over the
// row's lanes, as the rerank does), and forms the partial (m, s, o) of its
// slots as sparse_sv does; `combine` merges them. Slots past the chosen
// rows are the static rows (range table), scored the same way.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kSvThreads) void sparse_sv_scored(SvArgs a) {
  constexpr int EPL = KvTraits<T>::EPL, LPR = KvTraits<T>::LPR, ROWB = KvTraits<T>::ROWB;
  constexpr int NG = kSvThreads / LPR;  // row groups
  constexpr int RU = kSvRows / NG;      // rows per row group
  constexpr int NW = kSvThreads / 64;
  __shared__ float red[NG][kHeadDim];
  __shared__ float wmax[NW], wsum[NW];
  const int64_t seg = blockIdx.y;
  const int split = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int gid = tid / LPR, c = tid % LPR;
  const int b = (int)(seg / a.Hq), hq = (int)(seg % a.Hq), hkv = hq / a.G;
  const int j0 = split * kSvRows;
  const int nr = min(kSvRows, a.K - j0);
  float qr[1][EPL];
  load_q_slice<T, 1>(a.q, seg, c, qr);
  const int64_t hoff = (int64_t)b * a.stride_b_bytes + (int64_t)hkv * a.stride_h_bytes + c * 16;
  // the row of each of this thread's RU slots (-1: padding), then its key
  // and value chunks, all requested together
  int32_t rr[RU];
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int jj = gid + NG * u;
    const int j = j0 + jj;
    rr[u] = -1;
    if (jj < nr) rr[u] = j < a.k_top ? a.sel_row[seg * a.k_top + j] : (int32_t)pos_to_row(a.tab, a.n + (j - a.k_top));
  }
  u32x4 kw[RU], vw[RU];
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int64_t off = hoff + (int64_t)(rr[u] >= 0 ? rr[u] : 0) * ROWB;
    kw[u] = load16(a.kc + off);
    vw[u] = load16(a.v + off);
  }
  float z[RU];
  float zm = -INFINITY;
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    float d[1];
    chunk_dots<T, 1>(kw[u], qr, d);
    const float sdot = group_sum<LPR>(d[0]);
    z[u] = rr[u] >= 0 ? sdot * a.scale : -INFINITY;
    zm = fmaxf(zm, z[u]);
  }
  zm = wave_max(zm);
  if (lane == 0) wmax[w] = zm;
  __syncthreads();
  float m = wmax[0];
#pragma unroll
  for (int v = 1; v < NW; ++v) m = fmaxf(m, wmax[v]);
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float ps = 0.f;  // the weights of the slots, counted once (lane 0 of each row group)
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const float wt = z[u] == -INFINITY ? 0.f : __expf(z[u] - m);
    float x[EPL];
    unpack16<T>(rr[u] >= 0 ? vw[u] : u32x4{0u, 0u, 0u, 0u}, x);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wt, x[e], acc[e]);
    if (c == 0) ps += wt;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) red[gid][c * EPL + e] = acc[e];
  ps = wave_sum(ps);
  if (lane == 0) wsum[w] = ps;
  __syncthreads();
  float* part = a.part + (seg * a.nsplit + split) * kPartStride;
  if (tid < kHeadDim) {
    float o = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) o += red[g][tid];
    part[4 + tid] = o;
  }
  if (tid == 0) {
    float st = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) st += wsum[v];
    part[0] = m;
    part[1] = st;
  }
}

}  // namespace stdk
