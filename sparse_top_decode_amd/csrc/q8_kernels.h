// int8 keys for the recall stage. RetrievalAttention's review ("CPU memory
// minimization (Appendix C)") proposes 8-bit scalar quantization of the key
// vectors without fixing a scheme; here every row gets a symmetric int8 code
// with one fp32 scale: s = max_j |k_j| / 127 and c_j = k_j / s rounded to the
// nearest integer (halves to even), each one correctly rounded fp32
// operation, clamped to [-127, 127]; a row of zeros has s = 0 and codes 0.
// The codes only choose a superset of rows; the exact keys decide inside it.
#pragma once

#include "device.h"
#include "scan_kernels.h"

namespace stdk {

struct QuantArgs {
  const char* k;            // key cache base
  int64_t stride_b_bytes, stride_h_bytes;
  int8_t* codes;            // [B][H_kv][max_len][128]
  float* scales;            // [B][H_kv][max_len]
  int64_t max_len;
  int64_t n;                // positions (rows of the ranges)
  int32_t Hkv, pad_;
  RangeTab tab;
};

constexpr int kQuantThreads = 256;

// grid (cdiv(n, rows per workgroup), B * H_kv); a row is read by LPR lanes
// (16 B each) and its maximum taken over those lanes.
template <typename T>
__global__ __launch_bounds__(kQuantThreads) void k_quantize(QuantArgs a) {
  constexpr int EPL = KvTraits<T>::EPL, LPR = KvTraits<T>::LPR, RPL = KvTraits<T>::RPL, ROWB = KvTraits<T>::ROWB;
  constexpr int RPB = (kQuantThreads / 64) * RPL;  // rows per workgroup
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rg = lane / LPR, c = lane % LPR;
  const int grp = blockIdx.y;
  const int b = grp / a.Hkv, hk = grp - b * a.Hkv;
  const int64_t p = (int64_t)blockIdx.x * RPB + w * RPL + rg;
  const bool valid = p < a.n;
  const int64_t row = pos_to_row(a.tab, valid ? p : a.n - 1);
  const u32x4 raw = load16(a.k + (int64_t)b * a.stride_b_bytes + (int64_t)hk * a.stride_h_bytes + row * ROWB + c * 16);
  float x[EPL];
  unpack16<T>(raw, x);
  float mx = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) mx = fmaxf(mx, fabsf(x[e]));
  // the row's maximum over its LPR lanes (DPP row rotations, then the other half-row when LPR = 32)
  mx = fmaxf(mx, row_ror<8>(mx));
  mx = fmaxf(mx, row_ror<4>(mx));
  mx = fmaxf(mx, row_ror<2>(mx));
  mx = fmaxf(mx, row_ror<1>(mx));
  if constexpr (LPR == 32) mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  const float s = __fdiv_rn(mx, 127.0f);
  uint32_t packed[EPL / 4];
#pragma unroll
  for (int i = 0; i < EPL / 4; ++i) packed[i] = 0u;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    float t = s > 0.f ? __builtin_rintf(__fdiv_rn(x[e], s)) : 0.f;
    t = fminf(fmaxf(t, -127.f), 127.f);
    packed[e / 4] |= ((uint32_t)(int32_t)t & 0xFFu) << (8 * (e % 4));
  }
  if (!valid) return;
  const int64_t base = ((int64_t)b * a.Hkv + hk) * a.max_len + row;
  int8_t* dst = a.codes + base * kHeadDim + c * EPL;
  if constexpr (EPL == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
  else *reinterpret_cast<uint32_t*>(dst) = packed[0];
  if (c == 0) a.scales[base] = s;
}

}  // namespace stdk
