// Exact QK scan over a KV cache: one read of every key row serves all G
// query heads of its KV head.
//
// Scores follow decode attention (RetrievalAttention, papercache summary,
// "背景知识", Eq. 1): z_i = scale * q . k_i, here for every row of the scanned
// ranges ("Exact Top-K 的隐藏成本" in the ReTopK review: the exact path scores
// the whole cache before selecting). The kernel also builds the histogram of
// the first radix digit (top 11 bits of the order-preserving key) that the
// top-K select starts from.
#pragma once

#include <type_traits>

#include "device.h"

namespace stdk {

template <typename T>
struct KvTraits;
// bf16 rows: 256 B = 16 lanes x 16 B; a wave load covers 4 rows.
template <>
struct KvTraits<uint16_t> {
  static constexpr int EPL = 8, LPR = 16, RPL = 4, ROWB = 256;
};
// fp32 rows: 512 B = 32 lanes x 16 B; a wave load covers 2 rows.
template <>
struct KvTraits<float> {
  static constexpr int EPL = 4, LPR = 32, RPL = 2, ROWB = 512;
};

template <typename T>
STDK_DEV void unpack16(const u32x4& w, float* x);
template <>
STDK_DEV void unpack16<uint16_t>(const u32x4& w, float* x) {
  x[0] = bf16lo(w.x); x[1] = bf16hi(w.x);
  x[2] = bf16lo(w.y); x[3] = bf16hi(w.y);
  x[4] = bf16lo(w.z); x[5] = bf16hi(w.z);
  x[6] = bf16lo(w.w); x[7] = bf16hi(w.w);
}
template <>
STDK_DEV void unpack16<float>(const u32x4& w, float* x) {
  x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
  x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
}
// int8 key codes (the int8 recall stage): 16 signed bytes
template <>
STDK_DEV void unpack16<int8_t>(const u32x4& w, float* x) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * i + e] = (float)(int32_t)(int8_t)((v[i] >> (8 * e)) & 0xFFu);
}

// Loads into registers the EPL query values this lane multiplies, for the
// G query heads starting at q + seg0*128.
template <typename T, int G>
STDK_DEV void load_q_slice(const float* q, int64_t seg0, int c, float (&qr)[G][KvTraits<T>::EPL]) {
  constexpr int EPL = KvTraits<T>::EPL;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float4* qp = reinterpret_cast<const float4*>(q + (seg0 + h) * kHeadDim + c * EPL);
#pragma unroll
    for (int e = 0; e < EPL / 4; ++e) {
      float4 v = qp[e];
      qr[h][4 * e + 0] = v.x; qr[h][4 * e + 1] = v.y;
      qr[h][4 * e + 2] = v.z; qr[h][4 * e + 3] = v.w;
    }
  }
}

// Per-lane partial dot products of one 16-byte key chunk with G queries.
template <typename T, int G>
STDK_DEV void chunk_dots(const u32x4& kw, const float (&qr)[G][KvTraits<T>::EPL], float* acc) {
  constexpr int EPL = KvTraits<T>::EPL;
  float x[EPL];
  unpack16<T>(kw, x);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float s = qr[h][0] * x[0];
#pragma unroll
    for (int e = 1; e < EPL; ++e) s = fmaf(qr[h][e], x[e], s);
    acc[h] = s;
  }
}

struct ScanArgs {
  const float* q;          // [B][Hq][128]
  const char* k;           // key cache base
  int64_t stride_b_bytes;  // bytes between sequences
  int64_t stride_h_bytes;  // bytes between KV heads
  float* scores;           // [B*Hq][n_pad]
  uint32_t* hist;          // [B*Hq][2048], accumulated (zero on entry; the select kernel re-zeroes it)
  int64_t n, n_pad;        // positions per segment
  int32_t Hq, Hkv;
  int32_t blocks_per_group, pad_;
  int64_t rows_per_block;
  float scale;
  int32_t pad2_;
  const int32_t* head_active;  // [B*Hq] or null; a group with no active head exits
  int64_t n_hist;              // positions below this are counted in the histogram; the rest are scored only
  int32_t stage_stride;        // > 0: scores are staged in LDS (G rows of this stride) and written in chunks
  int32_t stage_rows;          // positions per staged chunk (a multiple of the rows per iteration)
  const float* kscale;         // int8 keys only: per-row scales, element (b, h_kv, row) at
  int64_t kscale_stride_b;     //   b*kscale_stride_b + h_kv*kscale_stride_h + row
  int64_t kscale_stride_h;
  const int64_t* n_dev;        // or null: device memory holding a row count; positions at or past it
                               // are neither scored nor counted (the launch is sized for n)
  RangeTab tab;
};

constexpr int kScanThreads = 512;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Work shape of the scan for row type T and G query heads per KV head.
//  - LPR lanes read one key row (8, or 16 when G > 4 to halve the query
//    registers); lane c of a row owns the 16-byte chunks at byte offsets
//    k*LPR*16 + c*16, i.e. E elements.
//  - GP = G rounded up to a power of two; a lane computes V = UR*GP partial
//    dot products per iteration (UR rows x GP heads), at most 4 chunk loads
//    per row set.
template <typename T, int G>
struct ScanShape {
  static constexpr int GP = G <= 1 ? 1 : (G <= 2 ? 2 : (G <= 4 ? 4 : 8));
  static constexpr int LPR = GP == 8 && sizeof(T) > 1 ? 16 : 8;  // an int8 row is 8 chunks
  static constexpr int ROWB = (int)sizeof(T) * kHeadDim;
  static constexpr int NCH = ROWB / (LPR * 16);
  static constexpr int EPC = 16 / (int)sizeof(T);
  static constexpr int E = NCH * EPC;
  static constexpr int UR0 = LPR / GP < 4 / NCH ? LPR / GP : 4 / NCH;
  static constexpr int UR = UR0 < 1 ? 1 : UR0;
  static constexpr int V = UR * GP;
  static constexpr int NSTEP = LPR == 16 ? 4 : 3;  // lane-exchange steps
  static constexpr int LOGV = V >= 16 ? 4 : (V >= 8 ? 3 : (V >= 4 ? 2 : (V >= 2 ? 1 : 0)));
  static constexpr int NW = kScanThreads / 64;
  static constexpr int RPW = 64 / LPR;  // rows per wave and row slot
  static constexpr int ROWS_ITER = NW * UR * RPW;
  static_assert(V <= LPR, "slots per lane");
};

// Value of lane i ^ M within its row group (M = 15: row mirror, 7: half-row
// mirror, 2 and 1: quad permutations).
template <int M>
STDK_DEV float xlane(float x) {
  constexpr int ctrl = M == 15 ? 0x140 : (M == 7 ? 0x141 : (M == 2 ? 0x4E : 0xB1));
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xF, 0xF, false));
}

// Exchange mask of reduction step k for LPR lanes per row: 15, 7, 2, 1 (the
// first dropped when LPR = 8).
template <int LPR>
constexpr int step_mask(int k) {
  return LPR == 16 ? (k == 0 ? 15 : (k == 1 ? 7 : (k == 2 ? 2 : 1))) : (k == 0 ? 7 : (k == 1 ? 2 : 1));
}

// Reduction of the V slot values of the LPR lanes of a row group. Step k
// pairs lane c with lane c ^ mask_k. While more than one slot remains, a step
// keeps the low half of the slots and adds the partner's high half; the slots
// are laid out so that both partners then hold the same logical value: slot j
// of lane c carries logical value j ^ pi(c), where pi is linear on the lane
// bits and maps mask_k to the half-size V >> (k+1) of its step (to 0 once a
// single slot is left, where the step is a plain all-reduce). Afterwards slot
// 0 of lane c holds the full sum of logical value pi(c).
template <int LPR, int V, int K = 0, int HV = V>
STDK_DEV void reduce_slots(float (&acc)[V]) {
  constexpr int NSTEP = LPR == 16 ? 4 : 3;
  if constexpr (K < NSTEP) {
    constexpr int M = step_mask<LPR>(K);
    if constexpr (HV > 1) {
#pragma unroll
      for (int j = 0; j < HV / 2; ++j) acc[j] += xlane<M>(acc[j + HV / 2]);
      reduce_slots<LPR, V, K + 1, HV / 2>(acc);
    } else {
      acc[0] += xlane<M>(acc[0]);
      reduce_slots<LPR, V, K + 1, 1>(acc);
    }
  }
}

// pi(c) of the reduction above, and whether lane c writes its sum (lanes
// that only repeat a sum after an all-reduce step do not).
template <int LPR, int V>
STDK_DEV int lane_perm(int c, bool* out_lane) {
  constexpr int NSTEP = LPR == 16 ? 4 : 3;
  int x = c, pi = 0, half = V;
  bool out = true;
#pragma unroll
  for (int k = 0; k < NSTEP; ++k) {
    half >>= 1;
    if ((x >> (NSTEP - 1 - k)) & 1) {
      x ^= step_mask<LPR>(k);
      if (half > 0) pi ^= half;
      else out = false;
    }
  }
  *out_lane = out;
  return pi;
}

// Key rows are read with non-temporal 16-byte loads: each row is read once
// per call, and on this part the non-temporal form streams measurably faster
// than the default cache policy.
template <int OFF>
STDK_DEV void load16_nt(u32x4& dst, const char* p, std::integral_constant<int, OFF>) {
  dst = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + OFF));
}
STDK_DEV void load4_nt(float& dst, const float* p) { dst = __builtin_nontemporal_load(p); }

// The scan on the vector ALUs (fp32 rows and int8 codes).
template <typename T, int G>
STDK_DEV void scan_valu_body(const ScanArgs& a) {
  using Sh = ScanShape<T, G>;
  constexpr bool kQ8 = sizeof(T) == 1;  // int8 codes: score = scale * row scale * (q . code)
  constexpr int GP = Sh::GP, LPR = Sh::LPR, NCH = Sh::NCH, EPC = Sh::EPC, E = Sh::E, UR = Sh::UR, V = Sh::V;
  constexpr int RPW = Sh::RPW, ROWB = Sh::ROWB, IT = Sh::ROWS_ITER;
  constexpr int NL = UR * NCH + (kQ8 ? UR : 0);  // loads per register set
  __shared__ __attribute__((aligned(16))) uint32_t lh[G * kHistBins];
  extern __shared__ __attribute__((aligned(16))) float sst[];  // staged scores, when a.stage_stride > 0

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rg = lane / LPR, c = lane % LPR;
  bool out_lane;
  const int pi = lane_perm<LPR, V>(c, &out_lane);
  const int rowperm = pi / GP, headperm = pi % GP;
  const int u_out = pi / GP, h_out = pi % GP;
  const bool writer = out_lane && h_out < G;
  const int group = blockIdx.x / a.blocks_per_group;
  const int blk = blockIdx.x % a.blocks_per_group;
  const int b = group / a.Hkv, hkv = group % a.Hkv;
  const int64_t seg0 = (int64_t)b * a.Hq + (int64_t)hkv * G;
  uint32_t act = (1u << G) - 1u;  // heads of this group that take part
  if (a.head_active) {
    act = 0u;
#pragma unroll
    for (int h = 0; h < G; ++h) act |= (a.head_active[seg0 + h] != 0 ? 1u : 0u) << h;
    if (act == 0u) return;
  }

  const char* kb = a.k + (int64_t)b * a.stride_b_bytes + (int64_t)hkv * a.stride_h_bytes + c * 16;
  const float* ksb = kQ8 ? a.kscale + (int64_t)b * a.kscale_stride_b + (int64_t)hkv * a.kscale_stride_h : nullptr;
  int64_t n_all = a.n, n_hist = a.n_hist;
  if (a.n_dev) {
    const int64_t nd = max((int64_t)0, *a.n_dev);
    n_all = min(n_all, nd);
    n_hist = min(n_hist, nd);
  }
  const int64_t p_beg = (int64_t)blk * a.rows_per_block;
  const int64_t p_end = min(n_all, p_beg + a.rows_per_block);
  if (p_beg >= p_end) return;  // no row of this workgroup's block is in use
  // An iteration covers positions [base, base + IT) of the piece [.., pe) of
  // one range, whose rows are position + ro. Past the block's end `ok` is
  // false: the iteration keeps the last piece (its loads stay clamped to a
  // valid row) and scores nothing.
  struct Iter {
    int64_t base, pe, ro;
    bool ok;
  };
  // the piece that holds position p (p_beg <= p < p_end), from p on; the
  // range table is read with compile-time indices (scalar loads)
  auto piece_at = [&](int64_t p) -> Iter {
    Iter it{p, a.tab.pos0[1], a.tab.row0[0] - a.tab.pos0[0], true};
#pragma unroll
    for (int i = 1; i < kMaxRanges; ++i) {
      if (i >= a.tab.n) break;
      if (p >= a.tab.pos0[i]) {
        it.pe = a.tab.pos0[i + 1];
        it.ro = a.tab.row0[i] - a.tab.pos0[i];
      }
    }
    it.pe = min(it.pe, p_end);
    return it;
  };
  auto advance = [&](const Iter& it) -> Iter {
    const int64_t nb = it.base + IT;
    if (nb < it.pe) return Iter{nb, it.pe, it.ro, it.ok};
    if (it.ok && it.pe < p_end) return piece_at(it.pe);
    return Iter{p_end + IT, it.pe, it.ro, false};
  };
  // row slot s of an iteration holds row (s ^ rowperm); loads past the piece
  // are clamped to its last row and their results dropped, so every load is
  // issued unconditionally
  auto issue = [&](const Iter& it, u32x4 (&kw)[UR][NCH], float (&sc)[UR]) {
#pragma unroll
    for (int s = 0; s < UR; ++s) {
      const int64_t p = min(it.base + (int64_t)(w * UR + (s ^ rowperm)) * RPW + rg, it.pe - 1);
      const char* rp = kb + (p + it.ro) * ROWB;
      load16_nt(kw[s][0], rp, std::integral_constant<int, 0>{});
      if constexpr (NCH > 1) load16_nt(kw[s][1], rp, std::integral_constant<int, LPR * 16>{});
      if constexpr (NCH > 2) load16_nt(kw[s][2], rp, std::integral_constant<int, 2 * LPR * 16>{});
      if constexpr (NCH > 3) load16_nt(kw[s][3], rp, std::integral_constant<int, 3 * LPR * 16>{});
      if constexpr (kQ8) load4_nt(sc[s], ksb + p + it.ro);
    }
  };
  static_assert(NCH <= 4 && NL < 16, "load shape");
  u32x4 kw[2][UR][NCH];
  float ksc[2][UR];

  // query elements of this lane; head slot hs holds head hs ^ headperm (zero
  // when that head does not exist, G < GP)
  float qr[GP][E];
#pragma unroll
  for (int hs = 0; hs < GP; ++hs) {
    const int h = hs ^ headperm;
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
      for (int e4 = 0; e4 < EPC / 4; ++e4) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (h < G) v = *reinterpret_cast<const float4*>(a.q + (seg0 + h) * kHeadDim + (k * LPR + c) * EPC + 4 * e4);
        qr[hs][k * EPC + 4 * e4 + 0] = v.x;
        qr[hs][k * EPC + 4 * e4 + 1] = v.y;
        qr[hs][k * EPC + 4 * e4 + 2] = v.z;
        qr[hs][k * EPC + 4 * e4 + 3] = v.w;
      }
  }
  // both register sets of key rows are requested right after the query
  Iter d0 = piece_at(p_beg);
  Iter d1 = advance(d0);
  issue(d0, kw[0], ksc[0]);
  issue(d1, kw[1], ksc[1]);
  for (int i = tid; i < G * kHistBins; i += kScanThreads) lh[i] = 0u;
  // LDS-only barrier: the key loads stay in flight
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // int8 codes c are read as unsigned bytes u = c + 128 (one conversion per
  // byte); q . c = q . u - 128 * sum(q), the sum taken once per lane and head
  float qsum[GP];
#pragma unroll
  for (int hs = 0; hs < GP; ++hs) {
    qsum[hs] = 0.f;
    if constexpr (kQ8) {
#pragma unroll
      for (int e = 0; e < E; ++e) qsum[hs] += qr[hs][e];
    }
  }
  auto consume = [&](const Iter& it, int64_t cstart, const u32x4 (&kv)[UR][NCH], const float (&sc)[UR]) {
    float acc[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int s = j / GP, hs = j % GP;
      float x[E];
      if constexpr (kQ8) {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
          const uint32_t v4[4] = {kv[s][k].x ^ 0x80808080u, kv[s][k].y ^ 0x80808080u, kv[s][k].z ^ 0x80808080u,
                                  kv[s][k].w ^ 0x80808080u};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[k * EPC + 4 * i + 0] = (float)((v4[i] >> 0) & 0xFFu);
            x[k * EPC + 4 * i + 1] = (float)((v4[i] >> 8) & 0xFFu);
            x[k * EPC + 4 * i + 2] = (float)((v4[i] >> 16) & 0xFFu);
            x[k * EPC + 4 * i + 3] = (float)((v4[i] >> 24) & 0xFFu);
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < NCH; ++k) unpack16<T>(kv[s][k], x + k * EPC);
      }
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) t = fmaf(qr[hs][e], x[e], t);
      if constexpr (kQ8) t = fmaf(-128.f, qsum[hs], t);
      acc[j] = t;
    }
    reduce_slots<LPR, V>(acc);
    const int64_t p = it.base + (int64_t)(w * UR + u_out) * RPW + rg;
    if (writer && p < it.pe) {
      float val = acc[0] * a.scale;
      if constexpr (kQ8) {
        // logical row u_out sits in slot u_out ^ rowperm
        float r = sc[0];
#pragma unroll
        for (int s = 1; s < UR; ++s) r = (u_out ^ rowperm) == s ? sc[s] : r;
        val = acc[0] * r * a.scale;
      }
      if (a.stage_stride > 0) {
        sst[h_out * a.stage_stride + (p - cstart)] = val;
      } else {
        // streaming store: the scores are read once, by the next kernel
        __builtin_nontemporal_store(val, &a.scores[(seg0 + h_out) * a.n_pad + p]);
      }
      if (p < n_hist) atomicAdd(&lh[h_out * kHistBins + (f2key(val) >> (32 - kHistBits))], 1u);
    }
  };
  // Staged scores: a chunk of consecutive positions [c0, c1) goes out once
  // every wave has scored it, as coalesced non-temporal stores; LDS-only
  // barriers around it keep the key loads in flight.
  auto flush = [&](int64_t c0, int64_t c1) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int len = (int)(c1 - c0);
    // rows start on 64-float boundaries, so a chunk that starts on a multiple
    // of 4 positions goes out in 16-byte stores
    const int nvec = (c0 & 3) == 0 ? len / 4 : 0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!((act >> h) & 1u)) continue;
      float* dst = a.scores + (seg0 + h) * a.n_pad + c0;
      const float* srcp = sst + h * a.stage_stride;
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      for (int i = tid; i < nvec; i += kScanThreads)
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(srcp + 4 * i),
                                    reinterpret_cast<f32x4*>(dst + 4 * i));
      for (int i = 4 * nvec + tid; i < len; i += kScanThreads) __builtin_nontemporal_store(srcp[i], dst + i);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  const bool staged = a.stage_stride > 0;
  int64_t cstart = d0.base;
  // after consuming `it`: the staged chunk goes out when the next iteration
  // would not fit beside it, or at the end (with the whole block staged,
  // that is once, after the last iteration)
  auto after = [&](const Iter& it, const Iter& nx) {
    if (staged && it.ok && (!nx.ok || nx.base + IT - cstart > a.stage_rows)) {
      flush(cstart, min(it.base + IT, it.pe));
      cstart = nx.base;
    }
  };
  // Two register sets: each is requested again as soon as it has been
  // consumed, so while one is consumed the other is in flight, and while a
  // wave waits both are. An iteration past the end is issued clamped and
  // scores nothing. Both sets are requested before the exit test, so every
  // path into the loop head has them in the same order and the compiler's
  // wait for one set leaves the other in flight.
  for (;;) {
    consume(d0, cstart, kw[0], ksc[0]);
    after(d0, d1);
    const Iter d2 = advance(d1);
    issue(d2, kw[0], ksc[0]);
    consume(d1, cstart, kw[1], ksc[1]);
    after(d1, d2);
    const Iter d3 = advance(d2);
    issue(d3, kw[1], ksc[1]);
    if (!d2.ok) break;
    d0 = d2;
    d1 = d3;
  }
  __syncthreads();
  // Add the block histogram to the global one: all LDS reads of a thread are
  // issued before the first wait, then one atomic per non-empty bin. Heads
  // that do not take part are skipped, so their global bins stay zero.
  constexpr int NV = G * kHistBins / 4 / kScanThreads;
  u32x4 hv[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) hv[k] = *reinterpret_cast<const u32x4*>(&lh[4 * (k * kScanThreads + tid)]);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const uint32_t vals[4] = {hv[k].x, hv[k].y, hv[k].z, hv[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * (k * kScanThreads + tid) + e;
      const int hh = i / kHistBins;
      if (vals[e] != 0u && ((act >> hh) & 1u)) atomicAdd(&a.hist[(seg0 + hh) * kHistBins + (i % kHistBins)], vals[e]);
    }
  }
}


// bf16 rows on the matrix cores. The G dot products of a key row are a
// 16-row x 128 x 16-column product tile (v_mfma_f32_16x16x32_bf16, four
// steps of 32 along the head dimension): the A operand is 16 key rows, the B
// operand the group's queries (columns past G are zero). Lane l of a wave
// supplies A row l%16 and B column l%16 with k = 8*(l/16) + i of each step;
// result register r of lane l is key row 4*(l/16) + r, query head l%16.
// Step s, lane group g uses head-dimension elements 32*s + 8*g + i (any
// fixed order of the elements gives the same dot product).
//
// Each query is split into three bf16 parts that together hold its fp32
// significand (|q - hi - mid - lo| <= 2^-27 |q|) and every part is
// multiplied (three products per step). Products of bf16 values are exact in
// fp32 and the matrix core accumulates in fp32, so a score matches the fp32
// dot product to fp32 rounding. (Two parts, |q - hi - lo| <= 2^-17 |q|, were
// measured to reorder rows whose scores differ by about 1e-6.)
//
// The key rows are loaded the way a plain read streams them: each load
// instruction of a wave takes 1 KB of consecutive bytes (4 rows, 16 lanes
// per row), which reads HBM faster than handing each lane its own row. The
// wave then transposes its 16-row tile through its own LDS region (rows 272
// bytes apart, so that both the row-wise stores and the column-wise reads
// fall on distinct banks) into the product's operand layout.
constexpr int kMfTiles = 2;                                       // 16-row tiles per wave and register set
constexpr int kMfRowsIter = (kScanThreads / 64) * 16 * kMfTiles;  // rows per workgroup iteration
constexpr int kMfRowStride = 272;                                 // LDS bytes per transposed key row
constexpr int kMfTileLds = (kScanThreads / 64) * 16 * kMfRowStride;

template <int G>
STDK_DEV void scan_mf_body(const ScanArgs& a) {
  static_assert(G >= 1 && G <= 16, "one product tile holds the group's query heads");
  constexpr int IT = kMfRowsIter, ROWB = 256;
  __shared__ __attribute__((aligned(16))) uint32_t lh[G * kHistBins];
  __shared__ __attribute__((aligned(16))) char tl[kMfTileLds];
  extern __shared__ __attribute__((aligned(16))) float sst[];  // staged scores, when a.stage_stride > 0

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lo = lane & 15, hi = lane >> 4;
  const int group = blockIdx.x / a.blocks_per_group;
  const int blk = blockIdx.x % a.blocks_per_group;
  const int b = group / a.Hkv, hkv = group % a.Hkv;
  const int64_t seg0 = (int64_t)b * a.Hq + (int64_t)hkv * G;
  uint32_t act = (1u << G) - 1u;  // heads of this group that take part
  if (a.head_active) {
    act = 0u;
#pragma unroll
    for (int h = 0; h < G; ++h) act |= (a.head_active[seg0 + h] != 0 ? 1u : 0u) << h;
    if (act == 0u) return;
  }
  const char* kb = a.k + (int64_t)b * a.stride_b_bytes + (int64_t)hkv * a.stride_h_bytes + lo * 16;
  int64_t n_all = a.n, n_hist = a.n_hist;
  if (a.n_dev) {
    const int64_t nd = max((int64_t)0, *a.n_dev);
    n_all = min(n_all, nd);
    n_hist = min(n_hist, nd);
  }
  const int64_t p_beg = (int64_t)blk * a.rows_per_block;
  const int64_t p_end = min(n_all, p_beg + a.rows_per_block);
  if (p_beg >= p_end) return;  // no row of this workgroup's block is in use
  // An iteration covers positions [base, base + IT) of the piece [.., pe) of
  // one range, whose rows are position + ro; wave w takes the tiles at
  // base + 16 * (w * kMfTiles + t). Past the block's end `ok` is false: the
  // iteration keeps the last piece (its loads stay clamped to a valid row)
  // and scores nothing.
  struct Iter {
    int64_t base, pe, ro;
    bool ok;
  };
  auto piece_at = [&](int64_t p) -> Iter {
    Iter it{p, a.tab.pos0[1], a.tab.row0[0] - a.tab.pos0[0], true};
#pragma unroll
    for (int i = 1; i < kMaxRanges; ++i) {
      if (i >= a.tab.n) break;
      if (p >= a.tab.pos0[i]) {
        it.pe = a.tab.pos0[i + 1];
        it.ro = a.tab.row0[i] - a.tab.pos0[i];
      }
    }
    it.pe = min(it.pe, p_end);
    return it;
  };
  auto advance = [&](const Iter& it) -> Iter {
    const int64_t nb = it.base + IT;
    if (nb < it.pe) return Iter{nb, it.pe, it.ro, it.ok};
    if (it.ok && it.pe < p_end) return piece_at(it.pe);
    return Iter{p_end + IT, it.pe, it.ro, false};
  };
  // load s of tile t: rows 4s .. 4s + 3 of the tile, lane l taking bytes
  // 16*(l%16) .. + 16 of row 4s + l/16 (loads past the piece are clamped to
  // its last row and their results dropped)
  auto issue = [&](const Iter& it, u32x4 (&kw)[kMfTiles][4]) {
#pragma unroll
    for (int t = 0; t < kMfTiles; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t p = min(it.base + (int64_t)(w * kMfTiles + t) * 16 + 4 * s + hi, it.pe - 1);
        kw[t][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (p + it.ro) * ROWB));
      }
  };
  u32x4 kw[2][kMfTiles][4];

  // B operand: query head lo (zero past G), elements 32*s + 8*hi + i
  u32x4 qh[4], qm[4], ql[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float x[8];
    if (lo < G) {
      const float4* qp = reinterpret_cast<const float4*>(a.q + (seg0 + lo) * kHeadDim + 32 * s + 8 * hi);
      const float4 v0 = qp[0], v1 = qp[1];
      x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
      x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
    split3_bf16x8(x, qh[s], qm[s], ql[s]);
  }
  // both register sets of key rows are requested right after the query
  Iter d0 = piece_at(p_beg);
  Iter d1 = advance(d0);
  issue(d0, kw[0]);
  issue(d1, kw[1]);
  for (int i = tid; i < G * kHistBins; i += kScanThreads) lh[i] = 0u;
  // LDS-only barrier: the key loads stay in flight
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  char* my = tl + w * 16 * kMfRowStride;
  auto consume = [&](const Iter& it, int64_t cstart, const u32x4 (&kv)[kMfTiles][4]) {
#pragma unroll
    for (int t = 0; t < kMfTiles; ++t) {
      // The wave's own region: its LDS operations complete in issue order,
      // so only the compiler has to be kept from moving them across each
      // other (the empty asm statements).
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int s = 0; s < 4; ++s) *reinterpret_cast<u32x4*>(my + (4 * s + hi) * kMfRowStride + 16 * lo) = kv[t][s];
      __asm__ volatile("" ::: "memory");
      u32x4 e[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) e[s] = *reinterpret_cast<const u32x4*>(my + lo * kMfRowStride + (4 * s + hi) * 16);
      __asm__ volatile("" ::: "memory");
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(e[s]), as_bf16x8(ql[s]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(e[s]), as_bf16x8(qm[s]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(e[s]), as_bf16x8(qh[s]), acc, 0, 0, 0);
      }
      if (lo < G) {
        const int64_t p0 = it.base + (int64_t)(w * kMfTiles + t) * 16 + 4 * hi;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t p = p0 + r;
          if (p < it.pe) {
            const float val = acc[r] * a.scale;
            if (a.stage_stride > 0) sst[lo * a.stage_stride + (p - cstart)] = val;
            else __builtin_nontemporal_store(val, &a.scores[(seg0 + lo) * a.n_pad + p]);
            if (p < n_hist) atomicAdd(&lh[lo * kHistBins + (f2key(val) >> (32 - kHistBits))], 1u);
          }
        }
      }
    }
  };
  // Staged scores: a chunk of consecutive positions [c0, c1) goes out once
  // every wave has scored it, as coalesced non-temporal stores; LDS-only
  // barriers around it keep the key loads in flight.
  auto flush = [&](int64_t c0, int64_t c1) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int len = (int)(c1 - c0);
    const int nvec = (c0 & 3) == 0 ? len / 4 : 0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!((act >> h) & 1u)) continue;
      float* dst = a.scores + (seg0 + h) * a.n_pad + c0;
      const float* srcp = sst + h * a.stage_stride;
      for (int i = tid; i < nvec; i += kScanThreads)
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(srcp + 4 * i), reinterpret_cast<f32x4*>(dst + 4 * i));
      for (int i = 4 * nvec + tid; i < len; i += kScanThreads) __builtin_nontemporal_store(srcp[i], dst + i);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  const bool staged = a.stage_stride > 0;
  int64_t cstart = d0.base;
  auto after = [&](const Iter& it, const Iter& nx) {
    if (staged && it.ok && (!nx.ok || nx.base + IT - cstart > a.stage_rows)) {
      flush(cstart, min(it.base + IT, it.pe));
      cstart = nx.base;
    }
  };
  // Two register sets, each requested again as soon as it has been consumed;
  // both are requested before the exit test, so that the compiler's wait for
  // one set leaves the other in flight.
  for (;;) {
    consume(d0, cstart, kw[0]);
    __builtin_amdgcn_sched_barrier(0);
    after(d0, d1);
    const Iter d2 = advance(d1);
    issue(d2, kw[0]);
    __builtin_amdgcn_sched_barrier(0);
    consume(d1, cstart, kw[1]);
    __builtin_amdgcn_sched_barrier(0);
    after(d1, d2);
    const Iter d3 = advance(d2);
    issue(d3, kw[1]);
    __builtin_amdgcn_sched_barrier(0);
    if (!d2.ok) break;
    d0 = d2;
    d1 = d3;
  }
  __syncthreads();
  // Add the block histogram to the global one (one atomic per non-empty bin
  // of a head that takes part).
  constexpr int NV = G * kHistBins / 4 / kScanThreads;
  u32x4 hv[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) hv[k] = *reinterpret_cast<const u32x4*>(&lh[4 * (k * kScanThreads + tid)]);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const uint32_t vals[4] = {hv[k].x, hv[k].y, hv[k].z, hv[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * (k * kScanThreads + tid) + e;
      const int hh = i / kHistBins;
      if (vals[e] != 0u && ((act >> hh) & 1u)) atomicAdd(&a.hist[(seg0 + hh) * kHistBins + (i % kHistBins)], vals[e]);
    }
  }
}

// Rows per workgroup iteration of the scan for row type T and group size G.
template <typename T, int G>
constexpr int scan_iter_rows() {
  return std::is_same<T, uint16_t>::value ? kMfRowsIter : ScanShape<T, G>::ROWS_ITER;
}

template <typename T, int G>
__global__ __launch_bounds__(kScanThreads) void k_scan(ScanArgs a) {
  if constexpr (std::is_same<T, uint16_t>::value) scan_mf_body<G>(a);
  else scan_valu_body<T, G>(a);
}

}  // namespace stdk
