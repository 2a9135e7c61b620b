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
  uint32_t* hist;          // [B*Hq][2048], accumulated (must start at 0)
  int64_t n, n_pad;        // positions per segment
  int32_t Hq, Hkv;
  int32_t blocks_per_group, pad_;
  int64_t rows_per_block;
  float scale;
  int32_t pad2_;
  const int32_t* head_active;  // [B*Hq] or null; a group with no active head exits
  RangeTab tab;
};

// The scan reads each key row with 8 lanes; lane c of the row owns the
// 16-byte chunks c, c+8, ... (byte offsets k*128 + c*16), i.e. 16 elements.
template <typename T>
struct ScanTraits;
template <>
struct ScanTraits<uint16_t> {
  static constexpr int NCH = 2, EPC = 8, ROWB = 256;
};
template <>
struct ScanTraits<float> {
  static constexpr int NCH = 4, EPC = 4, ROWB = 512;
};

constexpr int kScanThreads = 512;
constexpr int kScanLPR = 8;  // lanes per key row

template <typename T, int G>
struct ScanShape {
  static constexpr int UR0 = kScanLPR / G;
  static constexpr int UR = UR0 < 1 ? 1 : (UR0 > 4 ? 4 : UR0);  // rows per row group and iteration
  static constexpr int NW = kScanThreads / 64;
  static constexpr int RPB = 64 / kScanLPR;  // rows per wave and row batch (8)
  static constexpr int ROWS_ITER = NW * UR * RPB;
};

// Sum over aligned groups of 8 lanes with DPP (mirror within half rows, then
// two quad permutations); all 8 lanes end with the same bits.
STDK_DEV float sum8(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  return x;
}

template <typename T, int G>
__global__ __launch_bounds__(kScanThreads) void k_scan(ScanArgs a) {
  using Sh = ScanShape<T, G>;
  using Tr = ScanTraits<T>;
  constexpr int NCH = Tr::NCH, EPC = Tr::EPC, ROWB = Tr::ROWB, UR = Sh::UR, RPB = Sh::RPB;
  constexpr int E = NCH * EPC;  // elements per lane (16)
  static_assert(UR * G <= kScanLPR || UR == 1, "output lanes");
  __shared__ uint32_t lh[G * kHistBins];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rg = lane / kScanLPR, c = lane % kScanLPR;
  const int group = blockIdx.x / a.blocks_per_group;
  const int blk = blockIdx.x % a.blocks_per_group;
  const int b = group / a.Hkv, hkv = group % a.Hkv;
  const int64_t seg0 = (int64_t)b * a.Hq + (int64_t)hkv * G;
  if (a.head_active) {
    bool any = false;
#pragma unroll
    for (int h = 0; h < G; ++h) any |= a.head_active[seg0 + h] != 0;
    if (!any) return;
  }

  // this lane's 16 query elements for each head
  float qr[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const float4* qp = reinterpret_cast<const float4*>(a.q + (seg0 + h) * kHeadDim + k * (kHeadDim / NCH) + c * EPC);
#pragma unroll
      for (int e4 = 0; e4 < EPC / 4; ++e4) {
        const float4 v = qp[e4];
        qr[h][k * EPC + 4 * e4 + 0] = v.x;
        qr[h][k * EPC + 4 * e4 + 1] = v.y;
        qr[h][k * EPC + 4 * e4 + 2] = v.z;
        qr[h][k * EPC + 4 * e4 + 3] = v.w;
      }
    }
  for (int i = tid; i < G * kHistBins; i += kScanThreads) lh[i] = 0u;
  __syncthreads();

  const char* kb = a.k + (int64_t)b * a.stride_b_bytes + (int64_t)hkv * a.stride_h_bytes + c * 16;
  const int64_t p_beg = (int64_t)blk * a.rows_per_block;
  const int64_t p_end = min(a.n, p_beg + a.rows_per_block);
  for (int r = 0; r < a.tab.n; ++r) {
    const int64_t s0 = max(p_beg, a.tab.pos0[r]);
    const int64_t s1 = min(p_end, a.tab.pos0[r + 1]);
    if (s0 >= s1) continue;
    const int64_t rowoff = a.tab.row0[r] - a.tab.pos0[r];
    // rows of row batch u of this lane for the iteration at `base`; loads are
    // clamped to the last row of the piece and the extra results dropped
    auto issue = [&](int64_t base, u32x4 (&kw)[UR][NCH]) {
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        const int64_t p = min(base + (int64_t)(w * UR + u) * RPB + rg, s1 - 1);
        const char* rp = kb + (p + rowoff) * ROWB;
#pragma unroll
        for (int k = 0; k < NCH; ++k) kw[u][k] = load16(rp + k * 128);
      }
    };
    auto consume = [&](int64_t base, const u32x4 (&kw)[UR][NCH]) {
      float acc[UR][G];
#pragma unroll
      for (int u = 0; u < UR; ++u) {
        float x[E];
#pragma unroll
        for (int k = 0; k < NCH; ++k) unpack16<T>(kw[u][k], x + k * EPC);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float s = qr[h][0] * x[0];
#pragma unroll
          for (int e = 1; e < E; ++e) s = fmaf(qr[h][e], x[e], s);
          acc[u][h] = sum8(s);
        }
      }
#pragma unroll
      for (int i0 = 0; i0 < UR * G; i0 += kScanLPR) {
        const int i = i0 + c;
        if (i < UR * G) {
          float val = 0.f;
#pragma unroll
          for (int j = 0; j < UR * G; ++j)
            if (i == j) val = acc[j / G][j % G];
          const int uu = i / G, hh = i % G;
          const int64_t p = base + (int64_t)(w * UR + uu) * RPB + rg;
          if (p < s1) {
            val *= a.scale;
            a.scores[(seg0 + hh) * a.n_pad + p] = val;
            atomicAdd(&lh[hh * kHistBins + (f2key(val) >> (32 - kHistBits))], 1u);
          }
        }
      }
    };
    // two register sets: the loads of the next iteration are in flight while
    // the current one is computed
    u32x4 ka[UR][NCH], kc[UR][NCH];
    int64_t base = s0;
    issue(base, ka);
    while (true) {
      const int64_t nb = base + Sh::ROWS_ITER;
      if (nb < s1) issue(nb, kc);
      consume(base, ka);
      if (nb >= s1) break;
      base = nb;
      const int64_t nb2 = base + Sh::ROWS_ITER;
      if (nb2 < s1) issue(nb2, ka);
      consume(base, kc);
      if (nb2 >= s1) break;
      base = nb2;
    }
  }
  __syncthreads();
  for (int i = tid; i < G * kHistBins; i += kScanThreads) {
    const uint32_t v = lh[i];
    if (v) atomicAdd(&a.hist[(seg0 + i / kHistBins) * kHistBins + (i % kHistBins)], v);
  }
}

}  // namespace stdk
