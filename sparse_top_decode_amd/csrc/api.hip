// Host side of libstdk: argument validation, workspace layout, kernel
// launches and launch timing. The C entry points are declared in
// include/stdk.h, which documents each operation and its source.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "stdk.h"  // include/ (on the include path)
#include "attend_kernels.h"
#include "device.h"
#include "mq_kernels.h"
#include "q8_kernels.h"
#include "retopk_kernels.h"
#include "scan_kernels.h"
#include "select_kernels.h"

using namespace stdk;

namespace {

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
thread_local std::string g_err;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int32_t ok() {
  g_err.clear();
  return STDK_OK;
}

#define STDK_TRY(x)                 \
  do {                              \
    const int32_t rc_ = (x);        \
    if (rc_ != STDK_OK) return rc_; \
  } while (0)

// ---------------------------------------------------------------------------
// launch timing
// ---------------------------------------------------------------------------
enum KernelId {
  KID_SCAN, KID_SELECT, KID_SV, KID_DENSE, KID_COMBINE, KID_MERGE, KID_FILL,
  KID_RT_SELECT, KID_RT_RERANK, KID_RT_RSEL, KID_RT_INIT, KID_MQ_BLOCKMAX, KID_MQ_THRESH,
  KID_MQ_COLLECT, KID_MQ_SELECT, KID_MQ_FILL, KID_RT_VOTE, KID_Q8_QUANT, KID_READ, KID_RT_ATTEND, KID_RT_REUSE, KID_SELECT_SV, KID_SELECT_LDS, KID_SELECT_LDS_SV, KID_SELECT_HALF_SV, KID_COUNT
};
const char* const kKernelNames[KID_COUNT] = {
    "k_scan",        "topk_filter_select",             "sparse_sv",
    "dense_attn",  "combine",       "attn_merge",    "fill_empty",           "retopk_select",
    "retopk_rerank", "retopk_rerank_select", "retopk_init", "mq_blockmax",
    "mq_threshold",  "mq_collect",    "mq_select",     "mq_fill",       "retopk_vote",   "k_quantize",
    "hbm_read",      "retopk_attend", "retopk_reuse", "topk_filter_select_sv",
    "topk_select_lds", "topk_select_lds_sv", "topk_filter_lds_sv"};

struct Profiler {
  std::mutex mu;
  bool on = false;
  int only = -1;  // record only this kernel family (-1: all)
  std::vector<hipEvent_t> ev;  // 2 per slot
  std::vector<int> kid;
  size_t used = 0;
  double total_ms[KID_COUNT] = {};
  int64_t launches[KID_COUNT] = {};
};
Profiler g_prof;

// Events for the next launch of kernel family `kid` (null if not recorded).
// They are handed to the dispatch itself, so they time the kernel, not the
// queue around it.
long prof_slot(int kid, hipEvent_t* e0, hipEvent_t* e1) {
  *e0 = *e1 = nullptr;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.on || g_prof.used >= g_prof.kid.size()) return -1;
  if (g_prof.only >= 0 && g_prof.only != kid) return -1;
  const size_t slot = g_prof.used++;
  g_prof.kid[slot] = kid;
  *e0 = g_prof.ev[2 * slot];
  *e1 = g_prof.ev[2 * slot + 1];
  return (long)slot;
}

// Testing aid (stdk_inject_launch_failure): the launch with this number,
// counted from the moment it is armed, is not enqueued and reports STDK_EHIP.
std::atomic<int64_t> g_fail_at{-1};
std::atomic<int64_t> g_launch_no{0};

// f(e0, e1) enqueues one kernel with hipExtLaunchKernelGGL(..., e0, e1, 0, ...).
template <typename F>
int32_t launch(int kid, hipStream_t s, F&& f) {
  (void)s;
  const int64_t at = g_fail_at.load();
  if (at >= 0 && g_launch_no.fetch_add(1) == at) {
    g_fail_at.store(-1);
    return fail(STDK_EHIP, "%s launch failed: injected failure", kKernelNames[kid]);
  }
  hipEvent_t e0, e1;
  prof_slot(kid, &e0, &e1);
  f(e0, e1);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(STDK_EHIP, "%s launch failed: %s", kKernelNames[kid], hipGetErrorString(e));
  return STDK_OK;
}

// ---------------------------------------------------------------------------
// workspaces left dirty by a failed call
// ---------------------------------------------------------------------------
// A call chain keeps the counters at the start of its workspace (radix
// histograms and the select's arrival counters) zero between calls: the
// scan and the filter-select add to them, the filter-select clears them. A chain that stops with STDK_EHIP after its scan was enqueued
// leaves them non-zero; the workspace is recorded here with the extent of
// its counter region, and the next call on it clears that region first.
std::mutex g_dirty_mu;
std::vector<std::pair<uintptr_t, size_t>> g_dirty;

void mark_dirty(const void* ws, size_t bytes) {
  if (!ws || bytes == 0) return;
  std::lock_guard<std::mutex> lk(g_dirty_mu);
  for (auto& d : g_dirty)
    if (d.first == (uintptr_t)ws) {
      d.second = std::max(d.second, bytes);
      return;
    }
  g_dirty.emplace_back((uintptr_t)ws, bytes);
}

__global__ __launch_bounds__(256) void clear_words(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// Clears the counter region of `ws` if a failed call left it dirty.
int32_t clean_if_dirty(void* ws, size_t ws_bytes, hipStream_t s) {
  if (!ws) return STDK_OK;
  size_t bytes = 0;
  {
    std::lock_guard<std::mutex> lk(g_dirty_mu);
    if (g_dirty.empty()) return STDK_OK;
    for (auto& d : g_dirty)
      if (d.first == (uintptr_t)ws) bytes = d.second;
  }
  if (bytes == 0) return STDK_OK;
  const int64_t n = (int64_t)(std::min(bytes, ws_bytes) / 4);
  hipLaunchKernelGGL(clear_words, dim3((unsigned)std::min<int64_t>(1024, std::max<int64_t>(1, (n + 255) / 256))),
                     dim3(256), 0, s, (uint32_t*)ws, n);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(STDK_EHIP, "clearing a dirty workspace: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_dirty_mu);
  for (size_t i = 0; i < g_dirty.size(); ++i)
    if (g_dirty[i].first == (uintptr_t)ws) {
      g_dirty.erase(g_dirty.begin() + (long)i);
      break;
    }
  return STDK_OK;
}

// The result of a call chain on workspace `ws` whose counter region is
// `hist_bytes` long: a launch failure marks the workspace dirty.
int32_t finish(int32_t rc, const void* ws, size_t hist_bytes) {
  if (rc == STDK_EHIP) mark_dirty(ws, hist_bytes);
  if (rc != STDK_OK) return rc;
  g_err.clear();
  return STDK_OK;
}

#define STDK_LAUNCH(kernel, grid, block, shmem, stream, ...) \
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, e0, e1, 0, __VA_ARGS__)

// ---------------------------------------------------------------------------
// limits
// ---------------------------------------------------------------------------
constexpr int kMaxTopK = 65536;  // softmax.V partials of one head fit one combine workgroup
constexpr int kDenseMaxWg = 32;  // workgroups per KV head on the dense path

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t rup(int64_t a, int64_t b) { return cdiv(a, b) * b; }
inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }
constexpr int kScanStageMax = 96 * 1024;  // LDS bytes for staged scores

// ---------------------------------------------------------------------------
// device limits (per device, queried once)
// ---------------------------------------------------------------------------
struct DevInfo {
  bool init = false;
  int max_lds = 65536;
  int n_cu = 256;
  int scan_occ[3][STDK_MAX_GROUP + 1] = {};     // resident k_scan workgroups per CU, by (fp32 / bf16 / int8, G)
  int scan_static[3][STDK_MAX_GROUP + 1] = {};  // static LDS bytes of k_scan, same index
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

// Resident workgroups per CU of k_scan<T, G>, and its static LDS bytes; the
// staged scores may use the rest of the CU's LDS (up to kScanStageMax).
template <typename T, int G>
void occ_of(int max_lds, int* occ, int* stat) {
  hipFuncAttributes fa{};
  int st = G * kHistBins * 4;
  if (hipFuncGetAttributes(&fa, (const void*)k_scan<T, G>) == hipSuccess) st = (int)fa.sharedSizeBytes;
  (void)hipFuncSetAttribute((const void*)k_scan<T, G>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            std::max(0, std::min(kScanStageMax, max_lds - st)));
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_scan<T, G>, kScanThreads, 0) != hipSuccess || nb < 1) nb = 1;
  *occ = nb;
  *stat = st;
}

template <typename T>
void occ_row(int max_lds, int* o, int* st) {
  occ_of<T, 1>(max_lds, o + 1, st + 1); occ_of<T, 2>(max_lds, o + 2, st + 2);
  occ_of<T, 3>(max_lds, o + 3, st + 3); occ_of<T, 4>(max_lds, o + 4, st + 4);
  occ_of<T, 5>(max_lds, o + 5, st + 5); occ_of<T, 6>(max_lds, o + 6, st + 6);
  occ_of<T, 7>(max_lds, o + 7, st + 7); occ_of<T, 8>(max_lds, o + 8, st + 8);
}

int32_t dev_info(DevInfo** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(STDK_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(STDK_EUNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo& d = g_dev[dev];
  if (!d.init) {
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return fail(STDK_EHIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    d.max_lds = v;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(STDK_EHIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    d.n_cu = v;
    occ_row<float>(d.max_lds, d.scan_occ[0], d.scan_static[0]);
    occ_row<uint16_t>(d.max_lds, d.scan_occ[1], d.scan_static[1]);
    occ_row<int8_t>(d.max_lds, d.scan_occ[2], d.scan_static[2]);
    const int dyn_max = std::max(0, d.max_lds - (int)kSelStaticLds);
    (void)hipFuncSetAttribute((const void*)topk_filter_select, hipFuncAttributeMaxDynamicSharedMemorySize, dyn_max);
    (void)hipFuncSetAttribute((const void*)topk_filter_select_sv<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              dyn_max);
    (void)hipFuncSetAttribute((const void*)topk_filter_select_sv<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              dyn_max);
    (void)hipFuncSetAttribute((const void*)topk_select_lds, hipFuncAttributeMaxDynamicSharedMemorySize, dyn_max);
    (void)hipFuncSetAttribute((const void*)topk_select_lds_sv<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              dyn_max);
    (void)hipFuncSetAttribute((const void*)topk_select_lds_sv<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              dyn_max);
    const int half_max = std::max(0, d.max_lds / 2 - (int)kHalfStaticLds);
    (void)hipFuncSetAttribute((const void*)topk_filter_lds_sv<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              half_max);
    (void)hipFuncSetAttribute((const void*)topk_filter_lds_sv<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              half_max);
    (void)hipFuncSetAttribute((const void*)retopk_select<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              std::max(0, d.max_lds - 12 * 1024));
    (void)hipFuncSetAttribute((const void*)mq_select, hipFuncAttributeMaxDynamicSharedMemorySize,
                              std::max(0, d.max_lds - 1024));
    (void)hipFuncSetAttribute((const void*)retopk_vote<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              std::max(0, d.max_lds - 4 * 1024));
    (void)hipFuncSetAttribute((const void*)retopk_vote<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              std::max(0, d.max_lds - 4 * 1024));
    (void)hipFuncSetAttribute((const void*)retopk_attend<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              std::max(0, d.max_lds - kAttStaticLds));
    (void)hipFuncSetAttribute((const void*)retopk_attend<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              std::max(0, d.max_lds - kAttStaticLds));
    (void)hipFuncSetAttribute((const void*)retopk_reuse<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              std::max(0, d.max_lds - kReuseStaticLds));
    (void)hipFuncSetAttribute((const void*)retopk_reuse<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              std::max(0, d.max_lds - kReuseStaticLds));
    (void)hipFuncSetAttribute((const void*)retopk_rerank_select_lds, hipFuncAttributeMaxDynamicSharedMemorySize,
                              std::max(0, d.max_lds - 12 * 1024));
    (void)hipFuncSetAttribute((const void*)sparse_sv_ds<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              std::max(0, d.max_lds - 20 * 1024));
    (void)hipFuncSetAttribute((const void*)sparse_sv_ds<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              std::max(0, d.max_lds - 20 * 1024));
    (void)hipGetLastError();
    d.init = true;
  }
  *out = &d;
  return STDK_OK;
}

// ---------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------
int32_t check_layout(const stdk_layout* lay) {
  if (!lay) return fail(STDK_EINVAL, "layout is NULL");
  if (lay->batch < 1 || lay->n_q_heads < 1 || lay->n_kv_heads < 1)
    return fail(STDK_EINVAL, "batch, n_q_heads and n_kv_heads must be >= 1");
  if (lay->n_q_heads % lay->n_kv_heads != 0)
    return fail(STDK_EUNSUPPORTED, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", lay->n_q_heads,
                lay->n_kv_heads);
  const int G = lay->n_q_heads / lay->n_kv_heads;
  if (G > STDK_MAX_GROUP) return fail(STDK_EUNSUPPORTED, "group size %d > %d", G, STDK_MAX_GROUP);
  if (lay->head_dim != kHeadDim) return fail(STDK_EUNSUPPORTED, "head_dim %d (only 128 is supported)", lay->head_dim);
  if (lay->kv_dtype != STDK_F32 && lay->kv_dtype != STDK_BF16)
    return fail(STDK_EUNSUPPORTED, "kv_dtype %d", lay->kv_dtype);
  if (lay->max_len < 1 || lay->max_len > 0x7FFFFFFFLL)
    return fail(STDK_EINVAL, "max_len %lld out of range", (long long)lay->max_len);
  if (lay->stride_h < lay->max_len * kHeadDim) return fail(STDK_EINVAL, "stride_h smaller than max_len * head_dim");
  if (lay->batch > 1 && lay->stride_b < (int64_t)lay->n_kv_heads * lay->stride_h)
    return fail(STDK_EINVAL, "stride_b smaller than n_kv_heads * stride_h");
  const int esz = lay->kv_dtype == STDK_BF16 ? 2 : 4;
  if ((lay->stride_h * esz) % 16 != 0 || (lay->stride_b * esz) % 16 != 0)
    return fail(STDK_EINVAL, "strides must keep rows 16-byte aligned");
  return STDK_OK;
}

int32_t check_ptr(const void* p, const char* what, size_t align) {
  if (!p) return fail(STDK_EINVAL, "%s is NULL", what);
  if (((uintptr_t)p) % align != 0) return fail(STDK_EINVAL, "%s is not %zu-byte aligned", what, align);
  return STDK_OK;
}

struct Geo {
  int B, Hq, Hkv, G;
  int64_t S, groups;
  int64_t sb_bytes, sh_bytes;
  bool bf16;
};

Geo geo_of(const stdk_layout* lay) {
  Geo g{};
  g.B = lay->batch;
  g.Hq = lay->n_q_heads;
  g.Hkv = lay->n_kv_heads;
  g.G = g.Hq / g.Hkv;
  g.S = (int64_t)g.B * g.Hq;
  g.groups = (int64_t)g.B * g.Hkv;
  g.bf16 = lay->kv_dtype == STDK_BF16;
  const int esz = g.bf16 ? 2 : 4;
  g.sb_bytes = lay->stride_b * esz;
  g.sh_bytes = lay->stride_h * esz;
  return g;
}

// ---------------------------------------------------------------------------
// workspace: [counters (zero between calls)] [scores] [candidates] [partials]
// ---------------------------------------------------------------------------
// The counter region: per segment a 2048-bin first-digit histogram, then
// per segment a 2048-bin second-digit histogram, then per segment
// kCtlWords control words (word 0: the select's arrival counter).
inline size_t counter_bytes(int64_t S) { return al256((size_t)S * (2 * kHistBins + kCtlWords) * 4); }

// Filter-select geometry: about one workgroup per CU over the grid, each
// wave's slice (a multiple of 64 positions) loaded whole in one round.
constexpr int64_t kFselTargetWg = 256;

// n positions take part in the top-K; n_extra more (a static row set) are
// scored by the same scan and appended whole to every chosen-row list.
struct TopkWs {
  int64_t S, n, n_extra, n_pad, K, ksel, nsplit, slice, nb, wg;
  size_t hist, hist1, done, counters, scores, list, clist, wg_cnt, sel_row, sel_z, part, ovf, total;
};

TopkWs topk_ws(int64_t S, int64_t n, int64_t K, int64_t n_extra = 0) {
  TopkWs w{};
  w.S = S;
  w.n = n;
  w.n_extra = n_extra;
  const int64_t n1 = std::max<int64_t>(n, 1);
  w.n_pad = rup(std::max<int64_t>(n + n_extra, 1), 64);
  w.K = K;
  w.ksel = K + n_extra;
  w.nsplit = cdiv(w.ksel, kSvRows);
  // filter-select: about one workgroup per CU over the grid (P per
  // segment, each with at least 64 positions per wave), each taking nb
  // batches of 16 wave slices of at most 64 * kFselLoads positions
  constexpr int64_t WV = kSelectWaves;
  constexpr int64_t kMaxSlice = 64 * kFselLoads;
  const int64_t wg = std::max<int64_t>(1, std::min(cdiv(kFselTargetWg, S), cdiv(n1, 64 * WV)));
  w.nb = cdiv(n1, wg * WV * kMaxSlice);
  w.slice = rup(cdiv(n1, wg * WV * w.nb), 64);
  w.wg = cdiv(n1, w.nb * WV * w.slice);
  w.hist = 0;
  w.hist1 = (size_t)S * kHistBins * 4;
  w.done = (size_t)S * 2 * kHistBins * 4;
  w.counters = counter_bytes(S);
  size_t off = w.counters;
  w.scores = off;
  off = al256(off + (size_t)S * w.n_pad * 4);
  w.list = off;
  off = al256(off + (size_t)S * w.n_pad * sizeof(Cand));
  w.clist = off;
  off = al256(off + (size_t)S * w.n_pad * sizeof(Cand));
  w.wg_cnt = off;
  off = al256(off + (size_t)S * w.wg * 4);
  w.sel_row = off;
  off = al256(off + (size_t)S * K * 4);
  w.sel_z = off;
  off = al256(off + (size_t)S * K * 4);
  w.part = off;
  off = al256(off + (size_t)S * std::max<int64_t>(w.nsplit, kDenseMaxWg) * kPartStride * 4);
  w.ovf = off;
  off = al256(off + (size_t)S * 4);
  w.total = off;
  return w;
}

// Dense attention over n rows (K >= n) needs only its softmax.V partials;
// they follow the counter region, which stays untouched (zero).
TopkWs dense_ws(int64_t S, int64_t n) {
  TopkWs w{};
  w.S = S;
  w.n = n;
  w.n_pad = rup(std::max<int64_t>(n, 1), 64);
  w.K = n;
  w.counters = counter_bytes(S);
  w.part = w.counters;
  w.total = al256(w.part + (size_t)S * kDenseMaxWg * kPartStride * 4);
  return w;
}

RangeTab make_tab(const int64_t* ranges, int n_ranges, int64_t* n_total) {
  RangeTab t{};
  t.n = n_ranges;
  int64_t pos = 0;
  for (int r = 0; r < n_ranges; ++r) {
    t.row0[r] = ranges[2 * r];
    t.pos0[r] = pos;
    pos += ranges[2 * r + 1] - ranges[2 * r];
  }
  t.pos0[n_ranges] = pos;
  if (n_ranges == 0) {
    t.n = 1;
    t.row0[0] = 0;
    t.pos0[0] = 0;
    t.pos0[1] = 0;
  }
  *n_total = pos;
  return t;
}

// ---------------------------------------------------------------------------
// kernel dispatch on (dtype, G)
// ---------------------------------------------------------------------------
template <typename T>
int scan_rows_iter(int G) {
  switch (G) {
    case 1: return scan_iter_rows<T, 1>();
    case 2: return scan_iter_rows<T, 2>();
    case 3: return scan_iter_rows<T, 3>();
    case 4: return scan_iter_rows<T, 4>();
    case 5: return scan_iter_rows<T, 5>();
    case 6: return scan_iter_rows<T, 6>();
    case 7: return scan_iter_rows<T, 7>();
    default: return scan_iter_rows<T, 8>();
  }
}

template <typename T>
void launch_scan_t(int G, dim3 grid, hipStream_t s, const ScanArgs& a, hipEvent_t e0, hipEvent_t e1) {
  const size_t lds = a.stage_stride > 0 ? (size_t)G * a.stage_stride * 4 : 0;
  switch (G) {
    case 1: STDK_LAUNCH((k_scan<T, 1>), grid, dim3(kScanThreads), lds, s, a); break;
    case 2: STDK_LAUNCH((k_scan<T, 2>), grid, dim3(kScanThreads), lds, s, a); break;
    case 3: STDK_LAUNCH((k_scan<T, 3>), grid, dim3(kScanThreads), lds, s, a); break;
    case 4: STDK_LAUNCH((k_scan<T, 4>), grid, dim3(kScanThreads), lds, s, a); break;
    case 5: STDK_LAUNCH((k_scan<T, 5>), grid, dim3(kScanThreads), lds, s, a); break;
    case 6: STDK_LAUNCH((k_scan<T, 6>), grid, dim3(kScanThreads), lds, s, a); break;
    case 7: STDK_LAUNCH((k_scan<T, 7>), grid, dim3(kScanThreads), lds, s, a); break;
    default: STDK_LAUNCH((k_scan<T, 8>), grid, dim3(kScanThreads), lds, s, a); break;
  }
}

template <typename T>
void launch_dense_t(int G, dim3 grid, hipStream_t s, const DenseArgs& a, hipEvent_t e0, hipEvent_t e1) {
  switch (G) {
    case 1: STDK_LAUNCH((dense_attn<T, 1>), grid, dim3(kDenseThreads), 0, s, a); break;
    case 2: STDK_LAUNCH((dense_attn<T, 2>), grid, dim3(kDenseThreads), 0, s, a); break;
    case 3: STDK_LAUNCH((dense_attn<T, 3>), grid, dim3(kDenseThreads), 0, s, a); break;
    case 4: STDK_LAUNCH((dense_attn<T, 4>), grid, dim3(kDenseThreads), 0, s, a); break;
    case 5: STDK_LAUNCH((dense_attn<T, 5>), grid, dim3(kDenseThreads), 0, s, a); break;
    case 6: STDK_LAUNCH((dense_attn<T, 6>), grid, dim3(kDenseThreads), 0, s, a); break;
    case 7: STDK_LAUNCH((dense_attn<T, 7>), grid, dim3(kDenseThreads), 0, s, a); break;
    default: STDK_LAUNCH((dense_attn<T, 8>), grid, dim3(kDenseThreads), 0, s, a); break;
  }
}

// The exact select over n positions (any n >= 1; n <= K takes every row):
// scan, then filter-select. The counter region (the first counter_bytes(S)
// of the workspace) is zero on entry and the filter-select leaves it zero.
// Leaves the chosen rows and scores in the workspace. `active` restricts the
// work to the listed segments (ReTopK exact heads); null = all.
// int8 key codes and their row scales (packed: [B][H_kv][max_len][128] and
// [B][H_kv][max_len]), scanned instead of the cache by the int8 recall stage
struct Q8Keys {
  const int8_t* codes;
  const float* scales;
  int64_t max_len;
};

// Softmax . V fused into the select launch, where the caller wants o and
// lse of every head (no per-head mask, no cache push). Long segments
// (topk_filter_select_sv): where the chosen plus static slots fit the last
// workgroup's LDS and there are at least as many heads as CUs; short ones
// (topk_select_lds_sv): fuse_lds_short below. One workgroup reads a head's
// value rows at about one CU's share of HBM bandwidth (~40 GB/s measured),
// so the fusion pays only when the heads' tails cover the whole chip
// (batched decode: 3.47K against 3.42K steps/s on 16 x 32 heads); with 32
// heads the separate softmax . V launch is faster (11.8K against 11.1K
// steps/s on the 128K single-sequence step).
struct SvFuse {
  const void* v_cache;
  float* o_out;
  float* lse_out;
};

// LDS of the fused select: the candidate copy (at least the softmax's group
// sums), then rows and scores of the slots. Returns false when it does not fit.
bool fuse_lds(const Geo& g, const TopkWs& w, const DevInfo* di, size_t* dyn, int32_t* cache_cap) {
  if (w.ksel > kFuseMaxSlots || w.n_extra > (int64_t)kFuseStatic * kSelThreads || w.S < di->n_cu) return false;
  const size_t pre_bytes = (size_t)((w.wg + 2) & ~1LL) * 4;
  const size_t avail = (size_t)di->max_lds - kSelStaticLds;
  const size_t slots = (size_t)w.ksel * 8;
  const size_t red = (size_t)(kSelThreads / (g.bf16 ? KvTraits<uint16_t>::LPR : KvTraits<float>::LPR)) * kHeadDim * 4;
  if (pre_bytes + slots + red > avail) return false;
  const int64_t want = std::min<int64_t>(w.n, std::max<int64_t>(8192, 2 * w.K));
  const int64_t cap = std::min<int64_t>(want, (int64_t)((avail - pre_bytes - slots) / sizeof(Cand)));
  if ((size_t)cap * sizeof(Cand) < red) return false;
  *cache_cap = (int32_t)cap;
  *dyn = pre_bytes + (size_t)cap * sizeof(Cand) + slots;
  return true;
}

// LDS of the fused one-workgroup select of a short segment
// (topk_select_lds_sv). Each head's softmax . V then runs in one workgroup
// at about one CU's share of HBM bandwidth, which pays where the heads cover
// the chip or where a head's value rows are few (K + n_extra rows of at most
// kFuseShortBytes: the separate softmax . V launch costs more than reading
// them); false otherwise or when it does not fit.
constexpr size_t kFuseShortBytes = 64 * 1024;
bool fuse_lds_short(const Geo& g, const TopkWs& w, const DevInfo* di, size_t* dyn) {
  if (w.n > kSelLdsMax || w.n_extra > (int64_t)kFuseStatic * kSelThreads) return false;
  const int rowb = g.bf16 ? KvTraits<uint16_t>::ROWB : KvTraits<float>::ROWB;
  if (w.S < di->n_cu && (size_t)(w.K + w.n_extra) * rowb > kFuseShortBytes) return false;
  const size_t head = g.bf16 ? sel_lds_sv_head<uint16_t>(w.n) : sel_lds_sv_head<float>(w.n);
  const size_t bytes = head + (size_t)(w.K + w.n_extra) * 8;
  if (bytes + kSelStaticLds > (size_t)di->max_lds) return false;
  *dyn = bytes;
  return true;
}

// LDS of topk_filter_lds_sv (two workgroups per CU, each with at most half
// of its LDS): used where every head has one filter workgroup and the heads
// are at least twice as many as the CUs; false otherwise or when the slots
// and the group sums do not fit. The candidate capacity takes the rest, up
// to n.
bool fuse_half(const Geo& g, const TopkWs& w, const DevInfo* di, size_t* dyn, int32_t* cache_cap) {
  if (w.wg != 1 || w.n <= kSelLdsMax || w.S < 2 * (int64_t)di->n_cu || w.ksel > kFuseMaxSlots ||
      w.n_extra > (int64_t)kFuseStatic * kHalfThreads)
    return false;
  const size_t avail = (size_t)di->max_lds / 2 - kHalfStaticLds;
  const size_t slots = (size_t)w.ksel * 8;
  const size_t red = (size_t)(kHalfThreads / (g.bf16 ? KvTraits<uint16_t>::LPR : KvTraits<float>::LPR)) * kHeadDim * 4;
  if (8 + slots + red > avail) return false;
  const int64_t cap = std::min<int64_t>(w.n, (int64_t)((avail - 8 - slots) / sizeof(Cand)));
  if ((size_t)cap * sizeof(Cand) < red) return false;
  *cache_cap = (int32_t)cap;
  *dyn = 8 + (size_t)cap * sizeof(Cand) + slots;
  return true;
}

// Whether run_exact_select can fuse softmax . V into its select launch.
bool can_fuse(const Geo& g, const TopkWs& w, const DevInfo* di) {
  size_t dyn;
  int32_t cap;
  return w.n <= kSelLdsMax ? fuse_lds_short(g, w, di, &dyn) : fuse_lds(g, w, di, &dyn, &cap);
}

int32_t run_exact_select(const Geo& g, const TopkWs& w, char* ws, const float* q, const void* k_cache,
                         const RangeTab& tab, float scale, const int32_t* active, int32_t* idx_out,
                         const DevInfo* di, hipStream_t s, const Q8Keys* q8 = nullptr,
                         const int64_t* n_dev = nullptr, const SvFuse* fuse = nullptr) {
  float* scores = (float*)(ws + w.scores);
  uint32_t* hist = (uint32_t*)(ws + w.hist);
  Cand* list = (Cand*)(ws + w.list);
  {
    ScanArgs a{};
    a.q = q;
    a.k = (const char*)k_cache;
    a.stride_b_bytes = g.sb_bytes;
    a.stride_h_bytes = g.sh_bytes;
    if (q8) {
      a.k = (const char*)q8->codes;
      a.stride_h_bytes = q8->max_len * kHeadDim;
      a.stride_b_bytes = (int64_t)g.Hkv * a.stride_h_bytes;
      a.kscale = q8->scales;
      a.kscale_stride_h = q8->max_len;
      a.kscale_stride_b = (int64_t)g.Hkv * q8->max_len;
    }
    const int ti = q8 ? 2 : (g.bf16 ? 1 : 0);
    a.scores = scores;
    a.hist = hist;
    a.n = w.n + w.n_extra;
    a.n_hist = w.n;
    a.n_pad = w.n_pad;
    a.Hq = g.Hq;
    a.Hkv = g.Hkv;
    a.scale = scale;
    a.head_active = active;
    a.n_dev = n_dev;
    a.tab = tab;
    const int ri = q8 ? scan_rows_iter<int8_t>(g.G) : (g.bf16 ? scan_rows_iter<uint16_t>(g.G) : scan_rows_iter<float>(g.G));
    // one resident wave of workgroups over the whole chip, whole iterations each
    const int64_t target_blocks = (int64_t)di->n_cu * di->scan_occ[ti][g.G];
    const int64_t per_group = std::max<int64_t>(1, cdiv(target_blocks, g.groups));
    const int64_t rpb = std::max<int64_t>(ri, rup(cdiv(a.n, per_group), ri));
    a.rows_per_block = rpb;
    a.blocks_per_group = (int32_t)cdiv(a.n, rpb);
    // stage the scores in LDS, in chunks of whole iterations that fit
    // beside the histogram (row stride padded so that the G rows start on
    // different banks)
    const int occ = di->scan_occ[ti][g.G];
    const int64_t lds_free = std::min<int64_t>(kScanStageMax, (int64_t)di->max_lds / occ - di->scan_static[ti][g.G] - 1024);
    const int64_t chunk = std::min<int64_t>(rpb, (lds_free / (4 * g.G) - 16) / ri * ri);
    if (chunk >= ri) {
      a.stage_rows = (int32_t)chunk;
      a.stage_stride = (int32_t)(rup(chunk, 64) + 16);
    }
    const dim3 grid((unsigned)(g.groups * a.blocks_per_group));
    STDK_TRY(launch(KID_SCAN, s, [&](hipEvent_t e0, hipEvent_t e1) {
      if (q8) launch_scan_t<int8_t>(g.G, grid, s, a, e0, e1);
      else if (g.bf16) launch_scan_t<uint16_t>(g.G, grid, s, a, e0, e1);
      else launch_scan_t<float>(g.G, grid, s, a, e0, e1);
    }));
  }
  {
    SelectArgs a{};
    a.scores = scores;
    a.hist = hist;
    a.hist1 = (uint32_t*)(ws + w.hist1);
    a.done = (uint32_t*)(ws + w.done);
    a.list = list;
    a.wg_cnt = (uint32_t*)(ws + w.wg_cnt);
    a.clist = (Cand*)(ws + w.clist);
    a.n = w.n;
    a.n_pad = w.n_pad;
    a.K = (int32_t)w.K;
    a.slice = (int32_t)w.slice;
    a.nb = (int32_t)w.nb;
    a.sel_row = (int32_t*)(ws + w.sel_row);
    a.sel_z = (float*)(ws + w.sel_z);
    a.idx_out = idx_out;
    a.seg_active = active;
    a.n_dev = n_dev;
    a.tab = tab;
    // LDS for the workgroups' offsets and the candidates (typically under
    // 2K of them): room for max(8192, 2K)
    const size_t pre_bytes = (size_t)((w.wg + 2) & ~1LL) * 4;
    const size_t avail = (size_t)di->max_lds - kSelStaticLds;
    const int64_t want = std::min<int64_t>(w.n, std::max<int64_t>(8192, 2 * w.K));
    size_t dyn = std::min(avail, pre_bytes + (size_t)want * sizeof(Cand));
    a.cache_cap = (int32_t)((dyn - pre_bytes) / sizeof(Cand));
    if (w.n <= kSelLdsMax) {
      // a short segment: the whole select in one workgroup per head
      if (fuse) {
        size_t lds;
        if (!fuse_lds_short(g, w, di, &lds)) return fail(STDK_EUNSUPPORTED, "fused softmax.V does not fit");
        a.v = (const char*)fuse->v_cache;
        a.stride_b_bytes = g.sb_bytes;
        a.stride_h_bytes = g.sh_bytes;
        a.o_out = fuse->o_out;
        a.lse_out = fuse->lse_out;
        a.n_extra = (int32_t)w.n_extra;
        a.Hq = g.Hq;
        a.G = g.G;
        return launch(KID_SELECT_LDS_SV, s, [&](hipEvent_t e0, hipEvent_t e1) {
          if (g.bf16) STDK_LAUNCH(topk_select_lds_sv<uint16_t>, dim3((unsigned)w.S), dim3(kSelThreads), lds, s, a);
          else STDK_LAUNCH(topk_select_lds_sv<float>, dim3((unsigned)w.S), dim3(kSelThreads), lds, s, a);
        });
      }
      const size_t lds = (size_t)2 * sel_lds_stride(w.n) * 4;
      return launch(KID_SELECT_LDS, s, [&](hipEvent_t e0, hipEvent_t e1) {
        STDK_LAUNCH(topk_select_lds, dim3((unsigned)w.S), dim3(kSelThreads), lds, s, a);
      });
    }
    if (w.wg > 65535) return fail(STDK_EUNSUPPORTED, "%lld select workgroups per head", (long long)w.wg);
    const dim3 grid((unsigned)w.wg, (unsigned)w.S);
    if (fuse) {
      if (!fuse_lds(g, w, di, &dyn, &a.cache_cap)) return fail(STDK_EUNSUPPORTED, "fused softmax.V does not fit");
      a.v = (const char*)fuse->v_cache;
      a.stride_b_bytes = g.sb_bytes;
      a.stride_h_bytes = g.sh_bytes;
      a.o_out = fuse->o_out;
      a.lse_out = fuse->lse_out;
      a.n_extra = (int32_t)w.n_extra;
      a.Hq = g.Hq;
      a.G = g.G;
      size_t dyn_h;
      int32_t cap_h;
      if (!active && fuse_half(g, w, di, &dyn_h, &cap_h)) {
        // half-size workgroups, two per CU; the heads whose candidates do not
        // fit their LDS are then taken by topk_filter_select_sv, masked by
        // the flags (all its workgroups exit at once when no head is flagged)
        SelectArgs ah = a;
        ah.cache_cap = cap_h;
        ah.ovf = (int32_t*)(ws + w.ovf);
        STDK_TRY(launch(KID_SELECT_HALF_SV, s, [&](hipEvent_t e0, hipEvent_t e1) {
          if (g.bf16) STDK_LAUNCH(topk_filter_lds_sv<uint16_t>, dim3((unsigned)w.S), dim3(kHalfThreads), dyn_h, s, ah);
          else STDK_LAUNCH(topk_filter_lds_sv<float>, dim3((unsigned)w.S), dim3(kHalfThreads), dyn_h, s, ah);
        }));
        a.seg_active = ah.ovf;
      }
      STDK_TRY(launch(KID_SELECT_SV, s, [&](hipEvent_t e0, hipEvent_t e1) {
        if (g.bf16) STDK_LAUNCH(topk_filter_select_sv<uint16_t>, grid, dim3(kSelThreads), dyn, s, a);
        else STDK_LAUNCH(topk_filter_select_sv<float>, grid, dim3(kSelThreads), dyn, s, a);
      }));
      return STDK_OK;
    }
    STDK_TRY(launch(KID_SELECT, s, [&](hipEvent_t e0, hipEvent_t e1) {
      STDK_LAUNCH(topk_filter_select, grid, dim3(kSelThreads), dyn, s, a);
    }));
  }
  return STDK_OK;
}

int32_t run_combine(const TopkWs& w, char* ws, int32_t np, float* o_out, float* lse_out, hipStream_t s,
                    const int32_t* seg_active = nullptr);

// Softmax . V over the chosen rows left by the select kernels: for few
// heads with few rows (where the combine pass would cost as much as the
// gather), one workgroup per (head, value slice); else slices of kSvRows
// rows and the combine.
int32_t run_sv(const Geo& g, const TopkWs& w, char* ws, const void* v_cache, float* o_out, float* lse_out,
               hipStream_t s, const RangeTab* tab = nullptr, const SvPush* push = nullptr,
               int64_t* step_adv = nullptr, const int32_t* seg_active = nullptr) {
  SvArgs a{};
  if (push) {
    a.do_push = 1;
    a.push = *push;
  }
  a.step_adv = step_adv;
  a.seg_active = seg_active;
  a.k_top = (int32_t)w.K;
  a.scores = (const float*)(ws + w.scores);
  a.n = w.n;
  a.n_pad = w.n_pad;
  if (tab) a.tab = *tab;
  a.v = (const char*)v_cache;
  a.stride_b_bytes = g.sb_bytes;
  a.stride_h_bytes = g.sh_bytes;
  a.sel_row = (const int32_t*)(ws + w.sel_row);
  a.sel_z = (const float*)(ws + w.sel_z);
  a.part = (float*)(ws + w.part);
  a.K = (int32_t)w.ksel;
  a.nsplit = (int32_t)w.nsplit;
  a.Hq = g.Hq;
  a.G = g.G;
  DevInfo* di = nullptr;
  STDK_TRY(dev_info(&di));
  const size_t ds_lds = (size_t)w.ksel * 8;
  if (w.ksel <= kDsMaxSlots && w.S <= kDsMaxHeads && ds_lds + 20 * 1024 <= (size_t)di->max_lds) {
    // one workgroup per (head, value slice): finished outputs, no combine
    a.o_out = o_out;
    a.lse_out = lse_out;
    a.n_seg = w.S;
    const dim3 grid((unsigned)(rup(w.S, kDsXcds) * kDsSlices));
    return launch(KID_SV, s, [&](hipEvent_t e0, hipEvent_t e1) {
      if (g.bf16) STDK_LAUNCH(sparse_sv_ds<uint16_t>, grid, dim3(kDsThreads), ds_lds, s, a);
      else STDK_LAUNCH(sparse_sv_ds<float>, grid, dim3(kDsThreads), ds_lds, s, a);
    });
  }
  if (w.nsplit > kMaxPartials) return fail(STDK_EUNSUPPORTED, "%lld softmax.V partials per head", (long long)w.nsplit);
  const dim3 grid((unsigned)w.nsplit, (unsigned)w.S);
  STDK_TRY(launch(KID_SV, s, [&](hipEvent_t e0, hipEvent_t e1) {
    if (g.bf16) STDK_LAUNCH(sparse_sv<uint16_t>, grid, dim3(kSvThreads), 0, s, a);
    else STDK_LAUNCH(sparse_sv<float>, grid, dim3(kSvThreads), 0, s, a);
  }));
  return run_combine(w, ws, (int32_t)w.nsplit, o_out, lse_out, s, seg_active);
}

int32_t run_combine(const TopkWs& w, char* ws, int32_t np, float* o_out, float* lse_out, hipStream_t s,
                    const int32_t* seg_active) {
  CombineArgs a{(const float*)(ws + w.part), o_out, lse_out, np, 0, seg_active};
  return launch(KID_COMBINE, s, [&](hipEvent_t e0, hipEvent_t e1) { STDK_LAUNCH(combine, dim3((unsigned)w.S), dim3(kHeadDim), 0, s, a); });
}

// Dense attention over all n rows (K >= n): one read of every K and V row
// serves the G query heads of its KV head; partials combined per head.
int32_t run_dense(const Geo& g, const TopkWs& w, char* ws, const float* q, const void* k_cache,
                  const void* v_cache, const RangeTab& tab, float scale, int32_t top_k, int32_t* idx_out,
                  float* o_out, float* lse_out, hipStream_t s, int64_t n_idx = -1) {
  DenseArgs a{};
  a.n_idx = n_idx < 0 ? w.n : n_idx;
  a.q = q;
  a.k = (const char*)k_cache;
  a.v = (const char*)v_cache;
  a.stride_b_bytes = g.sb_bytes;
  a.stride_h_bytes = g.sh_bytes;
  a.part = (float*)(ws + w.part);
  a.idx_out = idx_out;
  a.n = w.n;
  a.Hq = g.Hq;
  a.Hkv = g.Hkv;
  a.K = top_k;
  a.scale = scale;
  a.tab = tab;
  // slices of at least kDenseSlice rows (a workgroup streams little data, so
  // short row sets are spread over more workgroups)
  const int64_t nwg = std::min<int64_t>(kDenseMaxWg, cdiv(w.n, kDenseSlice));
  a.rows_per_wg = rup(cdiv(w.n, nwg), kDenseSlice);
  a.nwg = (int32_t)cdiv(w.n, a.rows_per_wg);
  const dim3 grid((unsigned)a.nwg, (unsigned)g.groups);
  STDK_TRY(launch(KID_DENSE, s, [&](hipEvent_t e0, hipEvent_t e1) {
    if (g.bf16) launch_dense_t<uint16_t>(g.G, grid, s, a, e0, e1);
    else launch_dense_t<float>(g.G, grid, s, a, e0, e1);
  }));
  return run_combine(w, ws, a.nwg, o_out, lse_out, s);
}

// ---------------------------------------------------------------------------
// multi-query exact top-K: workspace and dispatch
// ---------------------------------------------------------------------------
// [block maxima] [thresholds] [candidate lists] [slice counts]; nothing is
// kept between calls
struct MqWs {
  int64_t S, n, n_pad, K, nblk, ngrp, chunk, nchunk, packs;
  size_t bmax, thr, list, slice_cnt, total;
};

constexpr int kMqTargetWg = 512;   // workgroups per pass (2 per CU on 256 CUs)
constexpr int kMqSelCache = 1024;  // candidates per query copied to the select wave's LDS

// The chunking depends on the shapes only, so the workspace size does too.
MqWs mq_ws(const Geo& g, int64_t M, int64_t n, int64_t K) {
  MqWs w{};
  w.S = g.S * M;
  w.n = n;
  w.K = K;
  w.n_pad = rup(std::max<int64_t>(n, 1), 64);
  w.nblk = cdiv(std::max<int64_t>(n, 1), kMqBlock);
  w.ngrp = 2 * w.nblk;
  const int64_t rows_per_pack = (int64_t)kMqWaves * (g.bf16 ? MqShape<uint16_t>::QT : MqShape<float>::QT) * 32;
  w.packs = cdiv((int64_t)g.G * M, rows_per_pack);
  int64_t nchunk = std::max<int64_t>(1, cdiv(kMqTargetWg, g.groups * w.packs));
  nchunk = std::min<int64_t>(nchunk, w.nblk);
  w.chunk = std::max<int64_t>(rup(cdiv(std::max<int64_t>(n, 1), nchunk), kMqBlock), rup(cdiv(std::max<int64_t>(n, 1), kMqMaxChunks), kMqBlock));
  w.nchunk = cdiv(std::max<int64_t>(n, 1), w.chunk);
  // the decode calls' counter region, which is zero between calls, is left
  // untouched, so one buffer may serve both
  size_t off = counter_bytes(g.S);
  w.bmax = off;
  off = al256(off + (size_t)w.S * w.ngrp * 4);
  w.thr = off;
  off = al256(off + (size_t)w.S * 4);
  w.list = off;
  off = al256(off + (size_t)w.S * w.n_pad * sizeof(Cand));
  w.slice_cnt = off;
  off = al256(off + (size_t)w.S * w.nchunk * 4);
  w.total = off;
  return w;
}

int32_t run_multi_query(const Geo& g, const MqWs& w, char* ws, const float* q, int32_t M, const void* k_cache,
                        const RangeTab& tab, float scale, int32_t* idx_out, float* z_out, const DevInfo* di,
                        hipStream_t s) {
  MqArgs a{};
  a.q = q;
  a.k = (const char*)k_cache;
  a.stride_b_bytes = g.sb_bytes;
  a.stride_h_bytes = g.sh_bytes;
  a.n = w.n;
  a.n_pad = w.n_pad;
  a.M = M;
  a.G = g.G;
  a.Hq = g.Hq;
  a.Hkv = g.Hkv;
  a.rows = g.G * M;
  a.chunk = (int32_t)w.chunk;
  a.nchunk = (int32_t)w.nchunk;
  a.ngrp = (int32_t)w.ngrp;
  a.scale = scale;
  a.bmax = (float*)(ws + w.bmax);
  a.thr = (const uint32_t*)(ws + w.thr);
  a.list = (Cand*)(ws + w.list);
  a.slice_cnt = (uint32_t*)(ws + w.slice_cnt);
  a.tab = tab;
  const dim3 grid((unsigned)w.nchunk, (unsigned)g.groups, (unsigned)w.packs);
  STDK_TRY(launch(KID_MQ_BLOCKMAX, s, [&](hipEvent_t e0, hipEvent_t e1) {
    if (g.bf16) STDK_LAUNCH(mq_blockmax<uint16_t>, grid, dim3(kMqThreads), 0, s, a);
    else STDK_LAUNCH(mq_blockmax<float>, grid, dim3(kMqThreads), 0, s, a);
  }));
  {
    MqThreshArgs t{(const float*)(ws + w.bmax), (uint32_t*)(ws + w.thr), w.n, (int32_t)w.ngrp, (int32_t)w.K};
    STDK_TRY(launch(KID_MQ_THRESH, s, [&](hipEvent_t e0, hipEvent_t e1) {
      STDK_LAUNCH(mq_threshold, dim3((unsigned)w.S), dim3(kMqThreshThreads), 0, s, t);
    }));
  }
  STDK_TRY(launch(KID_MQ_COLLECT, s, [&](hipEvent_t e0, hipEvent_t e1) {
    if (g.bf16) STDK_LAUNCH(mq_collect<uint16_t>, grid, dim3(kMqThreads), 0, s, a);
    else STDK_LAUNCH(mq_collect<float>, grid, dim3(kMqThreads), 0, s, a);
  }));
  {
    MqSelArgs sa{};
    sa.list = (const Cand*)(ws + w.list);
    sa.slice_cnt = (const uint32_t*)(ws + w.slice_cnt);
    sa.idx_out = idx_out;
    sa.z_out = z_out;
    sa.S = w.S;
    sa.n = w.n;
    sa.n_pad = w.n_pad;
    sa.chunk = (int32_t)w.chunk;
    sa.nchunk = (int32_t)w.nchunk;
    sa.K = (int32_t)w.K;
    sa.cap = (int32_t)std::min<int64_t>(w.n, kMqSelCache);
    sa.lds_words = (int32_t)(kHistBins + ((w.nchunk + 4) & ~3LL) + 2LL * sa.cap);
    sa.tab = tab;
    const size_t dyn = (size_t)kMqSelWaves * sa.lds_words * 4;
    if (dyn > (size_t)di->max_lds) return fail(STDK_EUNSUPPORTED, "multi-query select needs %zu bytes of LDS", dyn);
    STDK_TRY(launch(KID_MQ_SELECT, s, [&](hipEvent_t e0, hipEvent_t e1) {
      STDK_LAUNCH(mq_select, dim3((unsigned)cdiv(w.S, kMqSelWaves)), dim3(64 * kMqSelWaves), dyn, s, sa);
    }));
  }
  return STDK_OK;
}

// ---------------------------------------------------------------------------
// top-K with the int8 recall stage: workspace
// ---------------------------------------------------------------------------
// [the int8 scan's top-K' workspace] [exact scores of the superset] [exact
// scores of the n_st static rows] [chosen rows, scores and softmax.V
// partials of the final top-K and the static rows]
struct Q8Ws {
  TopkWs t1;  // scan of the codes, top-K' superset
  TopkWs t2;  // view for softmax . V over the final K rows, then the static rows
  size_t cz, czs, total;
};

Q8Ws q8_ws(const Geo& g, int64_t n, int64_t K, int64_t K2, int64_t n_st = 0) {
  Q8Ws w{};
  w.t1 = topk_ws(g.S, n, K2);
  size_t off = w.t1.total;
  w.cz = off;
  off = al256(off + (size_t)g.S * K2 * 4);
  w.czs = off;
  off = al256(off + (size_t)g.S * n_st * 4);
  w.t2 = w.t1;
  w.t2.K = K;
  w.t2.ksel = K + n_st;
  w.t2.nsplit = cdiv(K + n_st, kSvRows);
  // softmax . V reads static slot K + i's score at scores[seg * n_pad + i]
  w.t2.n = 0;
  w.t2.n_extra = n_st;
  w.t2.n_pad = n_st;
  w.t2.scores = w.czs;
  if (K == K2) {
    // the superset is the final set: softmax . V (sparse_sv_scored) reads
    // the superset's rows in place and scores them itself; the score arrays
    // above stay unused
    w.t2.sel_row = w.t1.sel_row;
    w.t2.sel_z = w.cz;
  } else {
    w.t2.sel_row = off;
    off = al256(off + (size_t)g.S * K * 4);
    w.t2.sel_z = off;
    off = al256(off + (size_t)g.S * K * 4);
  }
  w.t2.part = off;
  off = al256(off + (size_t)g.S * w.t2.nsplit * kPartStride * 4);
  w.total = off;
  return w;
}

// Host-side validation of one ascending, disjoint list of [begin, end) ranges.
int32_t check_ranges(const stdk_layout* lay, const int64_t* ranges, int32_t n_ranges, const char* what) {
  if (n_ranges < 0 || n_ranges > STDK_MAX_RANGES)
    return fail(STDK_EINVAL, "%s: count %d outside 0..%d", what, n_ranges, STDK_MAX_RANGES);
  if (n_ranges > 0 && !ranges) return fail(STDK_EINVAL, "%s is NULL", what);
  int64_t prev_end = 0;
  for (int r = 0; r < n_ranges; ++r) {
    const int64_t b = ranges[2 * r], e = ranges[2 * r + 1];
    if (b < 0 || e > lay->max_len || e <= b)
      return fail(STDK_EINVAL, "%s %d [%lld, %lld) invalid", what, r, (long long)b, (long long)e);
    if (r > 0 && b < prev_end) return fail(STDK_EINVAL, "%s must be ascending and disjoint", what);
    prev_end = e;
  }
  return STDK_OK;
}

// A dynamic and a static row set, validated: the position space of `all`
// holds the dynamic ranges first, then the static ones.
struct StaticSplit {
  RangeTab all, dyn, st;
  int64_t n_dyn, n_st;
};

int32_t split_static(const stdk_layout* lay, const int64_t* ranges, int32_t n_ranges, const int64_t* static_ranges,
                     int32_t n_static, StaticSplit* sp) {
  STDK_TRY(check_ranges(lay, ranges, n_ranges, "ranges"));
  STDK_TRY(check_ranges(lay, static_ranges, n_static, "static_ranges"));
  if (n_ranges + n_static > STDK_MAX_RANGES)
    return fail(STDK_EINVAL, "%d ranges in total, at most %d", n_ranges + n_static, STDK_MAX_RANGES);
  for (int i = 0; i < n_ranges; ++i)
    for (int j = 0; j < n_static; ++j)
      if (ranges[2 * i] < static_ranges[2 * j + 1] && static_ranges[2 * j] < ranges[2 * i + 1])
        return fail(STDK_EINVAL, "static range %d overlaps range %d", j, i);
  std::vector<int64_t> all(2 * (size_t)(n_ranges + n_static));
  for (int i = 0; i < 2 * n_ranges; ++i) all[i] = ranges[i];
  for (int i = 0; i < 2 * n_static; ++i) all[2 * n_ranges + i] = static_ranges[i];
  int64_t n_all = 0;
  sp->all = make_tab(all.data(), n_ranges + n_static, &n_all);
  sp->dyn = make_tab(ranges, n_ranges, &sp->n_dyn);
  sp->st = make_tab(static_ranges, n_static, &sp->n_st);
  return STDK_OK;
}

// Exact top-K over the dynamic rows, the static rows whole (validated
// inputs; the workspace holds topk_attn_decode_static's need).
int32_t run_static(const Geo& g, const StaticSplit& sp, char* ws, const float* q, const void* k_cache,
                   const void* v_cache, int32_t top_k, float scale, int32_t* idx_out, float* o_out, float* lse_out,
                   const DevInfo* di, hipStream_t s) {
  const int64_t n_all = sp.n_dyn + sp.n_st;
  if (n_all == 0) {
    const int64_t m = std::max<int64_t>(g.S * kHeadDim, g.S * (int64_t)top_k);
    return launch(KID_FILL, s, [&](hipEvent_t e0, hipEvent_t e1) {
      STDK_LAUNCH(fill_empty, dim3((unsigned)cdiv(m, 256)), dim3(256), 0, s, o_out, lse_out, idx_out, g.S, top_k);
    });
  }
  if (top_k >= sp.n_dyn) {
    // every dynamic row is chosen: dense attention over the union; idx_out
    // lists the dynamic rows, then -1
    return run_dense(g, dense_ws(g.S, n_all), ws, q, k_cache, v_cache, sp.all, scale, top_k, idx_out, o_out,
                     lse_out, s, sp.n_dyn);
  }
  const TopkWs w = topk_ws(g.S, sp.n_dyn, top_k, sp.n_st);
  if (can_fuse(g, w, di)) {
    const SvFuse fz{v_cache, o_out, lse_out};
    return run_exact_select(g, w, ws, q, k_cache, sp.all, scale, nullptr, idx_out, di, s, nullptr, nullptr, &fz);
  }
  STDK_TRY(run_exact_select(g, w, ws, q, k_cache, sp.all, scale, nullptr, idx_out, di, s));
  return run_sv(g, w, ws, v_cache, o_out, lse_out, s, &sp.all);
}

// Validation shared by topk_attn_decode_static and its allocation-free
// variant (everything but the workspace).
int32_t check_static_args(const stdk_layout* lay, const float* q, const void* k_cache, const void* v_cache,
                          const int64_t* ranges, int32_t n_ranges, const int64_t* static_ranges, int32_t n_static,
                          int32_t top_k, float scale, const int32_t* idx_out, const float* o_out,
                          const float* lse_out, StaticSplit* sp) {
  STDK_TRY(check_layout(lay));
  STDK_TRY(check_ptr(q, "q", 16));
  STDK_TRY(check_ptr(k_cache, "k_cache", 16));
  STDK_TRY(check_ptr(v_cache, "v_cache", 16));
  STDK_TRY(check_ptr(o_out, "o_out", 4));
  STDK_TRY(check_ptr(lse_out, "lse_out", 4));
  if (idx_out && ((uintptr_t)idx_out) % 4) return fail(STDK_EINVAL, "idx_out is not 4-byte aligned");
  if (top_k < 1) return fail(STDK_EINVAL, "top_k %d < 1", top_k);
  if (!std::isfinite(scale)) return fail(STDK_EINVAL, "scale is not finite");
  STDK_TRY(split_static(lay, ranges, n_ranges, static_ranges, n_static, sp));
  if (top_k > kMaxTopK && top_k < sp->n_dyn)
    return fail(STDK_EUNSUPPORTED, "top_k %d > %d (below the row count)", top_k, kMaxTopK);
  if (top_k < sp->n_dyn && top_k + sp->n_st > kMaxTopK)
    return fail(STDK_EUNSUPPORTED, "top_k %d + %lld static rows > %d", top_k, (long long)sp->n_st, kMaxTopK);
  return STDK_OK;
}

// ---------------------------------------------------------------------------
// scratch of the allocation-free entry point: one array per GPU, owned by the
// library for the life of the process. Host code never uses the array's name
// as an address (that is a host-side stand-in); the device address comes
// from hipGetSymbolAddress, once per device with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[STDK_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

int32_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(STDK_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(STDK_EUNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(STDK_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return STDK_OK;
}

// The top-K among the reranked candidates: staged in LDS when every
// candidate slot fits there, else read from global memory in each pass.
int32_t run_rerank_select(const RtRerankArgs& a, int64_t S, const DevInfo* di, hipStream_t s) {
  const size_t dyn = (size_t)a.cand_cap * 8;
  const bool staged = a.cand_cap <= kRselStageMax && dyn + 12 * 1024 <= (size_t)di->max_lds;
  return launch(KID_RT_RSEL, s, [&](hipEvent_t e0, hipEvent_t e1) {
    if (staged) STDK_LAUNCH(retopk_rerank_select_lds, dim3((unsigned)S), dim3(kRerankSelThreads), dyn, s, a);
    else STDK_LAUNCH(retopk_rerank_select, dim3((unsigned)S), dim3(kRerankSelThreads), 0, s, a);
  });
}

// The int8 recall step proper (recall_k below the row count of `tab`): the
// top-recall_k superset by the int8 scores, the exact scores of the superset
// and of the n_st rows of `stab`, the top-K inside the superset, then
// softmax . V over the K rows and the static ones in one pass.
int32_t run_int8(const Geo& g, const Q8Ws& w, char* ws, const float* q, const void* k_cache, const void* v_cache,
                 const Q8Keys& keys, const RangeTab& tab, const RangeTab& stab, int64_t n_st, int32_t top_k,
                 int32_t recall_k, float scale, int32_t* idx_out, int32_t* sup_out, float* o_out, float* lse_out,
                 const DevInfo* di, hipStream_t s) {
  // recall_k == top_k: the superset is the answer, and only its exact
  // scores are still needed: the softmax . V workgroups score their own rows
  const bool same = recall_k == top_k;
  int32_t* first = same && idx_out ? idx_out : sup_out;
  STDK_TRY(run_exact_select(g, w.t1, ws, q, nullptr, tab, scale, nullptr, first, di, s, &keys));
  if (same && idx_out && sup_out) {
    const hipError_t e = hipMemcpyAsync(sup_out, idx_out, (size_t)g.S * top_k * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return fail(STDK_EHIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  }
  if (same) {
    SvArgs a{};
    a.k_top = top_k;
    a.K = (int32_t)(top_k + n_st);
    a.nsplit = (int32_t)cdiv(a.K, kSvRows);
    a.sel_row = (const int32_t*)(ws + w.t1.sel_row);
    a.n = 0;
    a.tab = stab;
    a.v = (const char*)v_cache;
    a.kc = (const char*)k_cache;
    a.q = q;
    a.scale = scale;
    a.stride_b_bytes = g.sb_bytes;
    a.stride_h_bytes = g.sh_bytes;
    a.part = (float*)(ws + w.t2.part);
    a.Hq = g.Hq;
    a.G = g.G;
    if (a.nsplit > kMaxPartials) return fail(STDK_EUNSUPPORTED, "%d softmax.V partials per head", a.nsplit);
    const dim3 grid((unsigned)a.nsplit, (unsigned)g.S);
    STDK_TRY(launch(KID_SV, s, [&](hipEvent_t e0, hipEvent_t e1) {
      if (g.bf16) STDK_LAUNCH(sparse_sv_scored<uint16_t>, grid, dim3(kSvThreads), 0, s, a);
      else STDK_LAUNCH(sparse_sv_scored<float>, grid, dim3(kSvThreads), 0, s, a);
    }));
    return run_combine(w.t2, ws, a.nsplit, o_out, lse_out, s);
  }
  RtRerankArgs a{};
  a.q = q;
  a.k = (const char*)k_cache;
  a.stride_b_bytes = g.sb_bytes;
  a.stride_h_bytes = g.sh_bytes;
  a.exact = nullptr;
  a.cand = (const int32_t*)(ws + w.t1.sel_row);
  a.n_cand = nullptr;
  a.n_const = recall_k;
  a.cz = (float*)(ws + w.cz);
  a.sel_row = (int32_t*)(ws + w.t2.sel_row);
  a.sel_z = (float*)(ws + w.t2.sel_z);
  a.support_out = idx_out ? idx_out : (int32_t*)(ws + w.t2.sel_row);
  a.cand_cap = recall_k;
  a.K = top_k;
  a.Hq = g.Hq;
  a.G = g.G;
  a.nsplit = (int32_t)cdiv(recall_k + n_st, kRerankRows);
  a.scale = scale;
  a.n_static = (int32_t)n_st;
  a.cz_static = (float*)(ws + w.czs);
  a.st_tab = stab;
  const dim3 grid((unsigned)a.nsplit, (unsigned)g.S);
  STDK_TRY(launch(KID_RT_RERANK, s, [&](hipEvent_t e0, hipEvent_t e1) {
    if (g.bf16) STDK_LAUNCH(retopk_rerank<uint16_t>, grid, dim3(kRerankThreads), 0, s, a);
    else STDK_LAUNCH(retopk_rerank<float>, grid, dim3(kRerankThreads), 0, s, a);
  }));
  if (!same) STDK_TRY(run_rerank_select(a, g.S, di, s));
  return run_sv(g, w.t2, ws, v_cache, o_out, lse_out, s, &stab);
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* stdk_last_error(void) { return g_err.c_str(); }
int32_t stdk_version(void) { return STDK_VERSION; }

size_t topk_attn_decode_workspace_size(const stdk_layout* lay, int64_t n_scan, int32_t top_k) {
  if (check_layout(lay) != STDK_OK || n_scan < 0 || top_k < 1) return 0;
  const int64_t S = geo_of(lay).S;
  return top_k >= n_scan ? dense_ws(S, n_scan).total : topk_ws(S, n_scan, top_k).total;
}

int32_t topk_attn_decode(const stdk_layout* lay, const float* q, const void* k_cache, const void* v_cache,
                         const int64_t* ranges, int32_t n_ranges, int32_t top_k, float scale, int32_t* idx_out,
                         float* o_out, float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  STDK_TRY(check_layout(lay));
  STDK_TRY(check_ptr(q, "q", 16));
  STDK_TRY(check_ptr(k_cache, "k_cache", 16));
  STDK_TRY(check_ptr(v_cache, "v_cache", 16));
  STDK_TRY(check_ptr(o_out, "o_out", 4));
  STDK_TRY(check_ptr(lse_out, "lse_out", 4));
  if (idx_out && ((uintptr_t)idx_out) % 4) return fail(STDK_EINVAL, "idx_out is not 4-byte aligned");
  if (top_k < 1) return fail(STDK_EINVAL, "top_k %d < 1", top_k);
  if (!std::isfinite(scale)) return fail(STDK_EINVAL, "scale is not finite");
  STDK_TRY(check_ranges(lay, ranges, n_ranges, "ranges"));
  int64_t n = 0;
  const RangeTab tab = make_tab(ranges, n_ranges, &n);
  if (top_k > kMaxTopK && top_k < n)
    return fail(STDK_EUNSUPPORTED, "top_k %d > %d (below the row count)", top_k, kMaxTopK);
  const Geo g = geo_of(lay);
  const TopkWs w = topk_ws(g.S, n, top_k);
  if (n > 0) {
    STDK_TRY(check_ptr(workspace, "workspace", 256));
    const size_t need = topk_attn_decode_workspace_size(lay, n, top_k);
    if (workspace_bytes < need)
      return fail(STDK_EWORKSPACE, "workspace is %zu bytes, %zu needed", workspace_bytes, need);
  }
  hipStream_t s = (hipStream_t)stream;
  DevInfo* di = nullptr;
  STDK_TRY(dev_info(&di));
  char* ws = (char*)workspace;

  if (n == 0) {
    const int64_t m = std::max<int64_t>(g.S * kHeadDim, g.S * (int64_t)top_k);
    STDK_TRY(launch(KID_FILL, s, [&](hipEvent_t e0, hipEvent_t e1) {
      STDK_LAUNCH(fill_empty, dim3((unsigned)cdiv(m, 256)), dim3(256), 0, s, o_out, lse_out, idx_out, g.S,
                         top_k);
    }));
    return ok();
  }
  STDK_TRY(clean_if_dirty(ws, workspace_bytes, s));
  int32_t rc;
  if (top_k >= n) {
    rc = run_dense(g, dense_ws(g.S, n), ws, q, k_cache, v_cache, tab, scale, top_k, idx_out, o_out, lse_out, s);
  } else {
    const SvFuse fz{v_cache, o_out, lse_out};
    if (can_fuse(g, w, di)) {
      rc = run_exact_select(g, w, ws, q, k_cache, tab, scale, nullptr, idx_out, di, s, nullptr, nullptr, &fz);
    } else {
      rc = run_exact_select(g, w, ws, q, k_cache, tab, scale, nullptr, idx_out, di, s);
      if (rc == STDK_OK) rc = run_sv(g, w, ws, v_cache, o_out, lse_out, s, &tab);
    }
  }
  return finish(rc, ws, w.counters);
}

size_t topk_attn_decode_static_workspace_size(const stdk_layout* lay, int64_t n_scan, int64_t n_static,
                                              int32_t top_k) {
  if (check_layout(lay) != STDK_OK || n_scan < 0 || n_static < 0 || top_k < 1) return 0;
  const int64_t S = geo_of(lay).S;
  // the one-pass path, or (every dynamic row chosen) dense attention over
  // the union of both sets
  return top_k >= n_scan ? dense_ws(S, n_scan + n_static).total : topk_ws(S, n_scan, top_k, n_static).total;
}

int32_t topk_attn_decode_static(const stdk_layout* lay, const float* q, const void* k_cache, const void* v_cache,
                                const int64_t* ranges, int32_t n_ranges, const int64_t* static_ranges,
                                int32_t n_static, int32_t top_k, float scale, int32_t* idx_out, float* o_out,
                                float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  StaticSplit sp{};
  STDK_TRY(check_static_args(lay, q, k_cache, v_cache, ranges, n_ranges, static_ranges, n_static, top_k, scale,
                             idx_out, o_out, lse_out, &sp));
  const Geo g = geo_of(lay);
  if (sp.n_dyn + sp.n_st > 0) {
    STDK_TRY(check_ptr(workspace, "workspace", 256));
    const size_t need = topk_attn_decode_static_workspace_size(lay, sp.n_dyn, sp.n_st, top_k);
    if (workspace_bytes < need) return fail(STDK_EWORKSPACE, "workspace is %zu bytes, %zu needed", workspace_bytes, need);
  }
  DevInfo* di = nullptr;
  STDK_TRY(dev_info(&di));
  STDK_TRY(clean_if_dirty(workspace, workspace_bytes, (hipStream_t)stream));
  const int32_t rc = run_static(g, sp, (char*)workspace, q, k_cache, v_cache, top_k, scale, idx_out, o_out, lse_out,
                                di, (hipStream_t)stream);
  return finish(rc, workspace, counter_bytes(g.S));
}

int32_t topk_attn_decode_static_noalloc(const stdk_layout* lay, const float* q, const void* k_cache,
                                        const void* v_cache, const int64_t* ranges, int32_t n_ranges,
                                        const int64_t* static_ranges, int32_t n_static, int32_t top_k, float scale,
                                        int32_t* idx_out, float* o_out, float* lse_out, void* stream) {
  StaticSplit sp{};
  STDK_TRY(check_static_args(lay, q, k_cache, v_cache, ranges, n_ranges, static_ranges, n_static, top_k, scale,
                             idx_out, o_out, lse_out, &sp));
  const Geo g = geo_of(lay);
  hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  const size_t counters = counter_bytes(g.S);
  if (sp.n_dyn + sp.n_st > 0) {
    const size_t need = topk_attn_decode_static_workspace_size(lay, sp.n_dyn, sp.n_st, top_k);
    if (need > (size_t)STDK_NOALLOC_SCRATCH_BYTES)
      return fail(STDK_EWORKSPACE, "this call needs %zu bytes of scratch; the library's array holds %zu", need,
                  (size_t)STDK_NOALLOC_SCRATCH_BYTES);
    STDK_TRY(scratch_ptr(&ws));
    // the array keeps the previous call's contents: the radix counters
    // must start at zero, so they are cleared first (a fill kernel, which
    // is also safe under graph capture)
    const int64_t nw = (int64_t)(counters / 4);
    STDK_TRY(launch(KID_FILL, s, [&](hipEvent_t e0, hipEvent_t e1) {
      STDK_LAUNCH(clear_words, dim3((unsigned)std::min<int64_t>(1024, cdiv(nw, 256))), dim3(256), 0, s,
                  (uint32_t*)ws, nw);
    }));
  }
  DevInfo* di = nullptr;
  STDK_TRY(dev_info(&di));
  return finish(run_static(g, sp, (char*)ws, q, k_cache, v_cache, top_k, scale, idx_out, o_out, lse_out, di, s),
                nullptr, 0);
}

size_t topk_multi_query_workspace_size(const stdk_layout* lay, int32_t n_queries, int64_t n_scan, int32_t top_k) {
  if (check_layout(lay) != STDK_OK || n_queries < 1 || n_scan < 0 || top_k < 1) return 0;
  return mq_ws(geo_of(lay), n_queries, n_scan, top_k).total;
}

int32_t topk_multi_query(const stdk_layout* lay, const float* q, int32_t n_queries, const void* k_cache,
                         const int64_t* ranges, int32_t n_ranges, int32_t top_k, float scale, int32_t* idx_out,
                         float* z_out, void* workspace, size_t workspace_bytes, void* stream) {
  STDK_TRY(check_layout(lay));
  STDK_TRY(check_ptr(q, "q", 16));
  STDK_TRY(check_ptr(k_cache, "k_cache", 16));
  STDK_TRY(check_ptr(idx_out, "idx_out", 4));
  if (z_out && ((uintptr_t)z_out) % 4) return fail(STDK_EINVAL, "z_out is not 4-byte aligned");
  if (n_queries < 1) return fail(STDK_EINVAL, "n_queries %d < 1", n_queries);
  if (top_k < 1) return fail(STDK_EINVAL, "top_k %d < 1", top_k);
  if (!std::isfinite(scale)) return fail(STDK_EINVAL, "scale is not finite");
  STDK_TRY(check_ranges(lay, ranges, n_ranges, "ranges"));
  int64_t n = 0;
  const RangeTab tab = make_tab(ranges, n_ranges, &n);
  if (top_k > kMaxTopK) return fail(STDK_EUNSUPPORTED, "top_k %d > %d", top_k, kMaxTopK);
  const Geo g = geo_of(lay);
  if (g.groups > 65535) return fail(STDK_EUNSUPPORTED, "batch * n_kv_heads = %lld > 65535", (long long)g.groups);
  if ((int64_t)g.G * n_queries > (int64_t)65535 * 128)
    return fail(STDK_EUNSUPPORTED, "%d queries per KV head", g.G * n_queries);
  const MqWs w = mq_ws(g, n_queries, n, top_k);
  hipStream_t s = (hipStream_t)stream;
  if (n == 0) {
    const int64_t cnt = w.S * (int64_t)top_k;
    STDK_TRY(launch(KID_MQ_FILL, s, [&](hipEvent_t e0, hipEvent_t e1) {
      STDK_LAUNCH(mq_fill, dim3((unsigned)cdiv(cnt, 256)), dim3(256), 0, s, idx_out, z_out, cnt);
    }));
    return ok();
  }
  STDK_TRY(check_ptr(workspace, "workspace", 256));
  if (workspace_bytes < w.total)
    return fail(STDK_EWORKSPACE, "workspace is %zu bytes, %zu needed", workspace_bytes, w.total);
  DevInfo* di = nullptr;
  STDK_TRY(dev_info(&di));
  STDK_TRY(run_multi_query(g, w, (char*)workspace, q, n_queries, k_cache, tab, scale, idx_out, z_out, di, s));
  return ok();
}

int32_t quantize_keys_int8(const stdk_layout* lay, const void* k_cache, const int64_t* ranges, int32_t n_ranges,
                           int8_t* codes, float* scales, void* stream) {
  STDK_TRY(check_layout(lay));
  STDK_TRY(check_ptr(k_cache, "k_cache", 16));
  STDK_TRY(check_ptr(codes, "codes", 16));
  STDK_TRY(check_ptr(scales, "scales", 4));
  STDK_TRY(check_ranges(lay, ranges, n_ranges, "ranges"));
  int64_t n = 0;
  const RangeTab tab = make_tab(ranges, n_ranges, &n);
  if (n == 0) return ok();
  const Geo g = geo_of(lay);
  if (g.groups > 65535) return fail(STDK_EUNSUPPORTED, "batch * n_kv_heads = %lld > 65535", (long long)g.groups);
  hipStream_t s = (hipStream_t)stream;
  QuantArgs a{};
  a.k = (const char*)k_cache;
  a.stride_b_bytes = g.sb_bytes;
  a.stride_h_bytes = g.sh_bytes;
  a.codes = codes;
  a.scales = scales;
  a.max_len = lay->max_len;
  a.n = n;
  a.Hkv = g.Hkv;
  a.tab = tab;
  const int rpb = (kQuantThreads / 64) * (g.bf16 ? KvTraits<uint16_t>::RPL : KvTraits<float>::RPL);
  const dim3 grid((unsigned)cdiv(n, rpb), (unsigned)g.groups);
  STDK_TRY(launch(KID_Q8_QUANT, s, [&](hipEvent_t e0, hipEvent_t e1) {
    if (g.bf16) STDK_LAUNCH(k_quantize<uint16_t>, grid, dim3(kQuantThreads), 0, s, a);
    else STDK_LAUNCH(k_quantize<float>, grid, dim3(kQuantThreads), 0, s, a);
  }));
  return ok();
}

size_t topk_attn_decode_int8_workspace_size(const stdk_layout* lay, int64_t n_scan, int32_t top_k, int32_t recall_k) {
  if (check_layout(lay) != STDK_OK || n_scan < 0 || top_k < 1 || recall_k < top_k) return 0;
  const Geo g = geo_of(lay);
  return std::max(q8_ws(g, n_scan, top_k, recall_k).total, topk_ws(g.S, n_scan, top_k).total);
}

int32_t topk_attn_decode_int8(const stdk_layout* lay, const float* q, const void* k_cache, const void* v_cache,
                              const int8_t* codes, const float* scales, const int64_t* ranges, int32_t n_ranges,
                              int32_t top_k, int32_t recall_k, float scale, int32_t* idx_out, int32_t* sup_out,
                              float* o_out, float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  STDK_TRY(check_layout(lay));
  STDK_TRY(check_ptr(q, "q", 16));
  STDK_TRY(check_ptr(k_cache, "k_cache", 16));
  STDK_TRY(check_ptr(v_cache, "v_cache", 16));
  STDK_TRY(check_ptr(codes, "codes", 16));
  STDK_TRY(check_ptr(scales, "scales", 4));
  STDK_TRY(check_ptr(o_out, "o_out", 4));
  STDK_TRY(check_ptr(lse_out, "lse_out", 4));
  if (idx_out && ((uintptr_t)idx_out) % 4) return fail(STDK_EINVAL, "idx_out is not 4-byte aligned");
  if (sup_out && ((uintptr_t)sup_out) % 4) return fail(STDK_EINVAL, "sup_out is not 4-byte aligned");
  if (top_k < 1) return fail(STDK_EINVAL, "top_k %d < 1", top_k);
  if (recall_k < top_k) return fail(STDK_EINVAL, "recall_k %d < top_k %d", recall_k, top_k);
  if (!std::isfinite(scale)) return fail(STDK_EINVAL, "scale is not finite");
  STDK_TRY(check_ranges(lay, ranges, n_ranges, "ranges"));
  int64_t n = 0;
  const RangeTab tab = make_tab(ranges, n_ranges, &n);
  if (recall_k > kMaxTopK && recall_k < n)
    return fail(STDK_EUNSUPPORTED, "recall_k %d > %d (below the row count)", recall_k, kMaxTopK);
  const Geo g = geo_of(lay);
  hipStream_t s = (hipStream_t)stream;
  DevInfo* di = nullptr;
  if (n > 0) {
    STDK_TRY(check_ptr(workspace, "workspace", 256));
    const size_t need = topk_attn_decode_int8_workspace_size(lay, n, top_k, recall_k);
    if (workspace_bytes < need) return fail(STDK_EWORKSPACE, "workspace is %zu bytes, %zu needed", workspace_bytes, need);
    STDK_TRY(dev_info(&di));
  }
  char* ws = (char*)workspace;
  const size_t hb = counter_bytes(g.S);
  if (n > 0) STDK_TRY(clean_if_dirty(ws, workspace_bytes, s));
  if (n == 0 || recall_k >= n) {
    // the superset is every row: exact top-K attention (the superset output
    // lists every row)
    const TopkWs w = topk_ws(g.S, n, top_k);
    int32_t rc = STDK_OK;
    if (n == 0) {
      const int64_t m = std::max<int64_t>(g.S * kHeadDim, g.S * (int64_t)top_k);
      STDK_TRY(launch(KID_FILL, s, [&](hipEvent_t e0, hipEvent_t e1) {
        STDK_LAUNCH(fill_empty, dim3((unsigned)cdiv(m, 256)), dim3(256), 0, s, o_out, lse_out, idx_out, g.S, top_k);
      }));
    } else if (top_k >= n) {
      rc = run_dense(g, dense_ws(g.S, n), ws, q, k_cache, v_cache, tab, scale, top_k, idx_out, o_out, lse_out, s);
    } else {
      rc = run_exact_select(g, w, ws, q, k_cache, tab, scale, nullptr, idx_out, di, s);
      if (rc == STDK_OK) rc = run_sv(g, w, ws, v_cache, o_out, lse_out, s, &tab);
    }
    if (rc == STDK_OK && sup_out) {
      rc = launch(KID_FILL, s, [&](hipEvent_t e0, hipEvent_t e1) {
        STDK_LAUNCH(fill_rows, dim3((unsigned)cdiv(g.S * (int64_t)recall_k, 256)), dim3(256), 0, s, sup_out, g.S,
                    recall_k, tab);
      });
    }
    return finish(rc, ws, hb);
  }
  const Q8Ws w = q8_ws(g, n, top_k, recall_k);
  const Q8Keys keys{codes, scales, lay->max_len};
  const int32_t rc = run_int8(g, w, ws, q, k_cache, v_cache, keys, tab, RangeTab{}, 0, top_k, recall_k, scale,
                              idx_out, sup_out, o_out, lse_out, di, s);
  return finish(rc, ws, hb);
}

size_t topk_attn_decode_int8_static_workspace_size(const stdk_layout* lay, int64_t n_scan, int64_t n_static,
                                                   int32_t top_k, int32_t recall_k) {
  if (check_layout(lay) != STDK_OK || n_scan < 0 || n_static < 0 || top_k < 1 || recall_k < top_k) return 0;
  return std::max(q8_ws(geo_of(lay), n_scan, top_k, recall_k, n_static).total,
                  topk_attn_decode_static_workspace_size(lay, n_scan, n_static, top_k));
}

int32_t topk_attn_decode_int8_static(const stdk_layout* lay, const float* q, const void* k_cache,
                                     const void* v_cache, const int8_t* codes, const float* scales,
                                     const int64_t* ranges, int32_t n_ranges, const int64_t* static_ranges,
                                     int32_t n_static, int32_t top_k, int32_t recall_k, float scale,
                                     int32_t* idx_out, int32_t* sup_out, float* o_out, float* lse_out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  STDK_TRY(check_layout(lay));
  STDK_TRY(check_ptr(q, "q", 16));
  STDK_TRY(check_ptr(k_cache, "k_cache", 16));
  STDK_TRY(check_ptr(v_cache, "v_cache", 16));
  STDK_TRY(check_ptr(codes, "codes", 16));
  STDK_TRY(check_ptr(scales, "scales", 4));
  STDK_TRY(check_ptr(o_out, "o_out", 4));
  STDK_TRY(check_ptr(lse_out, "lse_out", 4));
  if (idx_out && ((uintptr_t)idx_out) % 4) return fail(STDK_EINVAL, "idx_out is not 4-byte aligned");
  if (sup_out && ((uintptr_t)sup_out) % 4) return fail(STDK_EINVAL, "sup_out is not 4-byte aligned");
  if (top_k < 1) return fail(STDK_EINVAL, "top_k %d < 1", top_k);
  if (recall_k < top_k) return fail(STDK_EINVAL, "recall_k %d < top_k %d", recall_k, top_k);
  if (!std::isfinite(scale)) return fail(STDK_EINVAL, "scale is not finite");
  StaticSplit sp{};
  STDK_TRY(split_static(lay, ranges, n_ranges, static_ranges, n_static, &sp));
  if (recall_k > kMaxTopK && recall_k < sp.n_dyn)
    return fail(STDK_EUNSUPPORTED, "recall_k %d > %d (below the row count)", recall_k, kMaxTopK);
  if (top_k < sp.n_dyn && top_k + sp.n_st > kMaxTopK)
    return fail(STDK_EUNSUPPORTED, "top_k %d + %lld static rows > %d", top_k, (long long)sp.n_st, kMaxTopK);
  const Geo g = geo_of(lay);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  DevInfo* di = nullptr;
  if (sp.n_dyn + sp.n_st > 0) {
    STDK_TRY(check_ptr(workspace, "workspace", 256));
    const size_t need = topk_attn_decode_int8_static_workspace_size(lay, sp.n_dyn, sp.n_st, top_k, recall_k);
    if (workspace_bytes < need) return fail(STDK_EWORKSPACE, "workspace is %zu bytes, %zu needed", workspace_bytes, need);
  }
  STDK_TRY(dev_info(&di));
  const size_t hb = counter_bytes(g.S);
  STDK_TRY(clean_if_dirty(ws, workspace_bytes, s));
  if (recall_k >= sp.n_dyn) {
    // the superset is every dynamic row: topk_attn_decode_static's result
    int32_t rc = run_static(g, sp, ws, q, k_cache, v_cache, top_k, scale, idx_out, o_out, lse_out, di, s);
    if (rc == STDK_OK && sup_out) {
      rc = launch(KID_FILL, s, [&](hipEvent_t e0, hipEvent_t e1) {
        STDK_LAUNCH(fill_rows, dim3((unsigned)cdiv(g.S * (int64_t)recall_k, 256)), dim3(256), 0, s, sup_out, g.S,
                    recall_k, sp.dyn);
      });
    }
    return finish(rc, ws, hb);
  }
  const Q8Ws w = q8_ws(g, sp.n_dyn, top_k, recall_k, sp.n_st);
  const Q8Keys keys{codes, scales, lay->max_len};
  const int32_t rc = run_int8(g, w, ws, q, k_cache, v_cache, keys, sp.dyn, sp.st, sp.n_st, top_k, recall_k, scale,
                              idx_out, sup_out, o_out, lse_out, di, s);
  return finish(rc, ws, hb);
}

int32_t attn_merge_lse(int64_t rows, int32_t d, const float* o_a, const float* lse_a, const float* o_b,
                       const float* lse_b, float* o_out, float* lse_out, void* stream) {
  if (rows < 0) return fail(STDK_EINVAL, "rows %lld < 0", (long long)rows);
  if (d < 1 || d > 1024) return fail(STDK_EINVAL, "d %d outside 1..1024", d);
  if (rows == 0) return ok();
  STDK_TRY(check_ptr(o_a, "o_a", 4));
  STDK_TRY(check_ptr(lse_a, "lse_a", 4));
  STDK_TRY(check_ptr(o_b, "o_b", 4));
  STDK_TRY(check_ptr(lse_b, "lse_b", 4));
  STDK_TRY(check_ptr(o_out, "o_out", 4));
  STDK_TRY(check_ptr(lse_out, "lse_out", 4));
  hipStream_t s = (hipStream_t)stream;
  MergeArgs a{o_a, lse_a, o_b, lse_b, o_out, lse_out, rows, d, 0};
  STDK_TRY(launch(KID_MERGE, s, [&](hipEvent_t e0, hipEvent_t e1) {
    STDK_LAUNCH(attn_merge, dim3((unsigned)cdiv(rows, 2)), dim3(kMergeThreads), 0, s, a);
  }));
  return ok();
}

// ---------------------------------------------------------------------------
// ReTopK
// ---------------------------------------------------------------------------
namespace {

int32_t check_retopk(const stdk_layout* lay, const retopk_params* p, const retopk_state* st) {
  STDK_TRY(check_layout(lay));
  if (!p) return fail(STDK_EINVAL, "params is NULL");
  if (!st) return fail(STDK_EINVAL, "state is NULL");
  if (p->top_k < 1) return fail(STDK_EINVAL, "top_k %d < 1", p->top_k);
  if (p->top_k > kMaxTopK) return fail(STDK_EUNSUPPORTED, "top_k %d > %d", p->top_k, kMaxTopK);
  if (p->cache_cap < 1 || p->cache_cap > kMaxCache)
    return fail(STDK_EINVAL, "cache_cap %d outside 1..%d", p->cache_cap, kMaxCache);
  if (p->top_r < 1 || p->top_r > p->cache_cap) return fail(STDK_EINVAL, "top_r %d outside 1..cache_cap", p->top_r);
  if (p->recent < 0) return fail(STDK_EINVAL, "recent %d < 0", p->recent);
  if (p->refresh < 0) return fail(STDK_EINVAL, "refresh %d < 0", p->refresh);
  if (std::isnan(p->tau)) return fail(STDK_EINVAL, "tau is NaN");
  if (!std::isfinite(p->scale)) return fail(STDK_EINVAL, "scale is not finite");
  if ((int64_t)p->top_r * p->top_k + p->recent > 0x7FFFFFFFLL) return fail(STDK_EINVAL, "R*K + W too large");
  if (p->budget < 0) return fail(STDK_EINVAL, "budget %d < 0", p->budget);
  if (p->budget > 0 && p->top_r > kMaxVote)
    return fail(STDK_EUNSUPPORTED, "a candidate budget needs top_r <= %d (got %d)", kMaxVote, p->top_r);
  if (p->budget > 0 && (int64_t)p->top_r * p->top_k + p->recent > kVoteMaxCand)
    return fail(STDK_EUNSUPPORTED, "a candidate budget needs R*K + W <= %d", kVoteMaxCand);
  STDK_TRY(check_ptr(st->q_hat, "state.q_hat", 16));
  STDK_TRY(check_ptr(st->support, "state.support", 4));
  STDK_TRY(check_ptr(st->head, "state.head", 4));
  STDK_TRY(check_ptr(st->count, "state.count", 4));
  return STDK_OK;
}

struct RetopkWs {
  TopkWs t;  // exact path
  int64_t cand_cap, words;
  size_t cand, n_cand, cz, qbar, path, exact, gbitmap, rec_slot, rec_rho, total;
};

RetopkWs retopk_ws(const Geo& g, const retopk_params* p, int64_t L) {
  RetopkWs r{};
  r.t = topk_ws(g.S, L, p->top_k);
  r.cand_cap = (int64_t)p->top_r * p->top_k + p->recent;
  r.words = cdiv(std::max<int64_t>(L, 1), 32);
  size_t off = r.t.total;
  r.cand = off;
  off = al256(off + (size_t)g.S * r.cand_cap * 4);
  r.cz = off;
  off = al256(off + (size_t)g.S * r.cand_cap * 4);
  r.n_cand = off;
  off = al256(off + (size_t)g.S * 4);
  r.qbar = off;
  off = al256(off + (size_t)g.S * kHeadDim * 4);
  r.path = off;
  off = al256(off + (size_t)g.S * 4);
  r.exact = off;
  off = al256(off + (size_t)g.S * 4);
  r.gbitmap = off;
  off = al256(off + (size_t)g.S * r.words * 4);
  r.rec_slot = off;
  off = al256(off + (size_t)g.S * kMaxVote * 4);
  r.rec_rho = off;
  off = al256(off + (size_t)g.S * kMaxVote * 4);
  r.total = off;
  return r;
}

}  // namespace

size_t retopk_state_size(const stdk_layout* lay, const retopk_params* p) {
  if (check_layout(lay) != STDK_OK || !p || p->top_k < 1 || p->cache_cap < 1) return 0;
  const size_t S = (size_t)geo_of(lay).S, C = (size_t)p->cache_cap, K = (size_t)p->top_k;
  return al256(S * C * kHeadDim * 4) + al256(S * C * K * 4) + al256(S * 4) + al256(S * 4);
}

// ---------------------------------------------------------------------------
// plain-read reference: region g of n_groups, workgroup blk of wpg streams
// bytes [blk * share, min(group_bytes, (blk + 1) * share)) of it
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void hbm_read(const char* base, int64_t stride, int64_t group_bytes, int64_t share,
                                                int32_t wpg, uint32_t* sink) {
  const int grp = blockIdx.x / wpg, blk = blockIdx.x % wpg;
  const char* p = base + (int64_t)grp * stride;
  const int64_t b0 = (int64_t)blk * share, b1 = min(group_bytes, b0 + share);
  if (b0 >= b1) return;
  constexpr int64_t kStep = 512 * 16;  // one 16-byte load per thread
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 v[2][4];
  int64_t off = b0 + (int64_t)threadIdx.x * 16;
  // non-temporal loads, as the key scan issues; loads past the share are
  // clamped onto its last 16 bytes
#pragma unroll
  for (int u = 0; u < 4; ++u) v[0][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + min(off + u * kStep, b1 - 16)));
  for (; off < b1; off += 8 * kStep) {
#pragma unroll
    for (int u = 0; u < 4; ++u) v[1][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + min(off + (4 + u) * kStep, b1 - 16)));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[0][u];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) v[0][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + min(off + (8 + u) * kStep, b1 - 16)));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[1][u];
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[0] = acc.x;
}

int32_t stdk_hbm_read(const void* base, int64_t group_stride_bytes, int32_t n_groups, int64_t group_bytes,
                      int32_t wg_per_group, uint32_t* sink, void* stream) {
  STDK_TRY(check_ptr(base, "base", 16));
  STDK_TRY(check_ptr(sink, "sink", 4));
  if (n_groups < 1 || wg_per_group < 1) return fail(STDK_EINVAL, "n_groups %d, wg_per_group %d", n_groups, wg_per_group);
  if ((int64_t)n_groups * wg_per_group > INT32_MAX) return fail(STDK_EINVAL, "too many workgroups");
  if (group_bytes < 16 || group_bytes % 16) return fail(STDK_EINVAL, "group_bytes %lld", (long long)group_bytes);
  if (group_stride_bytes % 16) return fail(STDK_EINVAL, "group_stride_bytes %lld", (long long)group_stride_bytes);
  const int64_t share = rup(cdiv(group_bytes, wg_per_group), 16);
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)(n_groups * wg_per_group));
  STDK_TRY(launch(KID_READ, s, [&](hipEvent_t e0, hipEvent_t e1) {
    STDK_LAUNCH(hbm_read, grid, dim3(512), 0, s, (const char*)base, group_stride_bytes, group_bytes, share,
                wg_per_group, sink);
  }));
  return ok();
}

int32_t stdk_inject_launch_failure(int32_t after_launches) {
  if (after_launches < -1) return fail(STDK_EINVAL, "after_launches %d < -1", after_launches);
  g_launch_no.store(0);
  g_fail_at.store(after_launches);
  return ok();
}

size_t retopk_workspace_size(const stdk_layout* lay, const retopk_params* p, int64_t max_L_t) {
  if (check_layout(lay) != STDK_OK || !p || p->top_k < 1 || p->top_r < 1 || p->recent < 0 || max_L_t < 1) return 0;
  return retopk_ws(geo_of(lay), p, max_L_t).total;
}

int32_t retopk_state_init(const stdk_layout* lay, const retopk_params* p, const retopk_state* st,
                          const float* q_hist, const int32_t* sup_hist, int32_t n_hist, void* stream) {
  STDK_TRY(check_retopk(lay, p, st));
  if (n_hist < 0) return fail(STDK_EINVAL, "n_hist %d < 0", n_hist);
  if (n_hist > 0) {
    STDK_TRY(check_ptr(q_hist, "q_hist", 4));
    STDK_TRY(check_ptr(sup_hist, "sup_hist", 4));
  }
  const Geo g = geo_of(lay);
  hipStream_t s = (hipStream_t)stream;
  RtInitArgs a{q_hist, sup_hist, st->q_hat, st->support, st->head, st->count, p->cache_cap, p->top_k, n_hist, 0};
  STDK_TRY(launch(KID_RT_INIT, s, [&](hipEvent_t e0, hipEvent_t e1) { STDK_LAUNCH(retopk_init, dim3((unsigned)g.S), dim3(256), 0, s, a); }));
  return ok();
}

// One ReTopK step. step_dev == null: L_t and t are the host's. Otherwise
// they are read on the device from step_dev ([L_t, t]) and advanced there at
// the end of the step; every launch is then sized for L_t = max_len (clamped
// on the device), so the same sequence of launches serves every step.
int32_t run_retopk(const stdk_layout* lay, const retopk_params* p, const retopk_state* st, const float* q,
                   const void* k_cache, const void* v_cache, int64_t L_t, int64_t t, int64_t* step_dev,
                   int32_t* support_out, float* o_out, float* lse_out, int32_t* path_out, int32_t* n_cand_out,
                   int32_t* cand_out, void* workspace, size_t workspace_bytes, void* stream) {
  STDK_TRY(check_retopk(lay, p, st));
  STDK_TRY(check_ptr(q, "q", 16));
  STDK_TRY(check_ptr(k_cache, "k_cache", 16));
  STDK_TRY(check_ptr(v_cache, "v_cache", 16));
  STDK_TRY(check_ptr(support_out, "support_out", 4));
  STDK_TRY(check_ptr(o_out, "o_out", 4));
  STDK_TRY(check_ptr(lse_out, "lse_out", 4));
  const bool dev = step_dev != nullptr;
  if (dev) {
    STDK_TRY(check_ptr(step_dev, "step", 8));
    L_t = lay->max_len;
    t = 0;
  }
  if (L_t < 1 || L_t > lay->max_len) return fail(STDK_EINVAL, "L_t %lld outside 1..max_len", (long long)L_t);
  if (L_t > (1 << 20)) return fail(STDK_EUNSUPPORTED, "L_t %lld > 1048576", (long long)L_t);
  if (t < 0) return fail(STDK_EINVAL, "t %lld < 0", (long long)t);
  const Geo g = geo_of(lay);
  const RetopkWs w = retopk_ws(g, p, L_t);
  STDK_TRY(check_ptr(workspace, "workspace", 256));
  if (workspace_bytes < w.total)
    return fail(STDK_EWORKSPACE, "workspace is %zu bytes, %zu needed", workspace_bytes, w.total);
  hipStream_t s = (hipStream_t)stream;
  DevInfo* di = nullptr;
  STDK_TRY(dev_info(&di));
  char* ws = (char*)workspace;
  STDK_TRY(clean_if_dirty(ws, workspace_bytes, s));
  const int32_t rc = [&]() -> int32_t {
    // with device-side steps the refresh is decided by retopk_select, which
    // marks every head exact then; the launches below stay the same
    const bool refresh_now = !dev && p->refresh > 0 && (t % p->refresh) == 0;
    int32_t* exact = (int32_t*)(ws + w.exact);

    // a6: selector (cosine, path, top-R, candidate union); without a vote,
    // and when the bitmap and the reuse path's LDS fit, one workgroup per
    // head also scores the candidates, keeps the top K, forms softmax . V
    // and pushes the cache entry (retopk_reuse); else retopk_select, then
    // (vote,) retopk_attend or the rerank launches below
    const size_t att_dyn = attend_lds_bytes((int)w.cand_cap, p->top_k);
    const size_t bm_bytes = (size_t)w.words * 4;
    const bool one_launch =
        p->budget == 0 && att_dyn + bm_bytes + (size_t)kReuseStaticLds <= (size_t)di->max_lds;
    RtAttendArgs at{};
    at.q = q;
    at.k = (const char*)k_cache;
    at.v = (const char*)v_cache;
    at.stride_b_bytes = g.sb_bytes;
    at.stride_h_bytes = g.sh_bytes;
    at.exact = exact;
    at.cand = (const int32_t*)(ws + w.cand);
    at.n_cand = (const int32_t*)(ws + w.n_cand);
    at.support_out = support_out;
    at.o_out = o_out;
    at.lse_out = lse_out;
    at.qbar = (const float*)(ws + w.qbar);
    at.q_hat = st->q_hat;
    at.support = st->support;
    at.head = st->head;
    at.count = st->count;
    at.cand_cap = (int32_t)w.cand_cap;
    at.K = p->top_k;
    at.Hq = g.Hq;
    at.G = g.G;
    at.C = p->cache_cap;
    at.scale = p->scale;
    {
      RtSelArgs a{};
      a.q = q;
      a.q_hat = st->q_hat;
      a.support = st->support;
      a.head = st->head;
      a.count = st->count;
      a.C = p->cache_cap;
      a.K = p->top_k;
      a.R = p->top_r;
      a.W = p->recent;
      a.tau = p->tau;
      a.refresh_now = refresh_now ? 1 : 0;
      a.L_t = L_t;
      a.step = step_dev;
      a.refresh = p->refresh;
      a.cand_cap = (int32_t)w.cand_cap;
      a.bitmap_words = (int32_t)w.words;
      a.qbar = (float*)(ws + w.qbar);
      a.path = (int32_t*)(ws + w.path);
      a.exact = exact;
      a.cand = (int32_t*)(ws + w.cand);
      a.n_cand = (int32_t*)(ws + w.n_cand);
      a.path_out = path_out;
      a.n_cand_out = n_cand_out;
      a.cand_out = cand_out;
      a.gbitmap = (uint32_t*)(ws + w.gbitmap);
      if (p->budget > 0) {
        a.rec_slot = (int32_t*)(ws + w.rec_slot);
        a.rec_rho = (float*)(ws + w.rec_rho);
      }
      const bool lds = bm_bytes + 12 * 1024 <= (size_t)di->max_lds;
      if (one_launch) {
        STDK_TRY(launch(KID_RT_REUSE, s, [&](hipEvent_t e0, hipEvent_t e1) {
          if (g.bf16) STDK_LAUNCH(retopk_reuse<uint16_t>, dim3((unsigned)g.S), dim3(kAttThreads), att_dyn + bm_bytes, s, a, at);
          else STDK_LAUNCH(retopk_reuse<float>, dim3((unsigned)g.S), dim3(kAttThreads), att_dyn + bm_bytes, s, a, at);
        }));
      } else {
        STDK_TRY(launch(KID_RT_SELECT, s, [&](hipEvent_t e0, hipEvent_t e1) {
          if (lds) STDK_LAUNCH(retopk_select<true>, dim3((unsigned)g.S), dim3(kRtSelThreads), bm_bytes, s, a);
          else STDK_LAUNCH(retopk_select<false>, dim3((unsigned)g.S), dim3(kRtSelThreads), 0, s, a);
        }));
      }
    }
    // confidence vote: cap the candidates of the reuse heads
    if (p->budget > 0 && !refresh_now) {
      RtVoteArgs a{};
      a.exact = exact;
      a.support = st->support;
      a.count = st->count;
      a.rec_slot = (const int32_t*)(ws + w.rec_slot);
      a.rec_rho = (const float*)(ws + w.rec_rho);
      a.cand = (int32_t*)(ws + w.cand);
      a.n_cand = (int32_t*)(ws + w.n_cand);
      a.n_cand_out = n_cand_out;
      a.cand_out = cand_out;
      a.L_t = L_t;
      a.step = step_dev;
      a.C = p->cache_cap;
      a.K = p->top_k;
      a.R = p->top_r;
      a.W = p->recent;
      a.cand_cap = (int32_t)w.cand_cap;
      a.budget = p->budget;
      // candidates and their masks, then (when they fit) the masks of every
      // row below the recent window
      const size_t base = (size_t)w.cand_cap * 4 + (((size_t)w.cand_cap + 15) & ~(size_t)15);
      const size_t with_rows = base + (size_t)rup(std::max<int64_t>(L_t, 1), 4);
      const bool row_masks = with_rows + 4 * 1024 <= (size_t)di->max_lds;
      const size_t dyn = row_masks ? with_rows : base + 16;
      STDK_TRY(launch(KID_RT_VOTE, s, [&](hipEvent_t e0, hipEvent_t e1) {
        if (row_masks) STDK_LAUNCH(retopk_vote<true>, dim3((unsigned)g.S), dim3(kVoteThreads), dyn, s, a);
        else STDK_LAUNCH(retopk_vote<false>, dim3((unsigned)g.S), dim3(kVoteThreads), dyn, s, a);
      }));
    }
    // exact heads: scan + select + softmax.V over [0, L_t)
    const int64_t rng[2] = {0, L_t};
    int64_t n_all = 0;
    const RangeTab tab = make_tab(rng, 1, &n_all);
    const int32_t* active = refresh_now ? nullptr : exact;
    STDK_TRY(run_exact_select(g, w.t, ws, q, k_cache, tab, p->scale, active, support_out, di, s, nullptr, step_dev));
    // reuse heads (not done above): one workgroup per head scores the
    // candidates, keeps the top K, forms softmax . V and pushes the cache
    // entry (retopk_attend), when its LDS holds the candidates; else the
    // rerank, its select and the softmax . V launch below
    const bool fused = one_launch || att_dyn + (size_t)kAttStaticLds <= (size_t)di->max_lds;
    if (!refresh_now && !one_launch && fused) {
      STDK_TRY(launch(KID_RT_ATTEND, s, [&](hipEvent_t e0, hipEvent_t e1) {
        if (g.bf16) STDK_LAUNCH(retopk_attend<uint16_t>, dim3((unsigned)g.S), dim3(kAttThreads), att_dyn, s, at);
        else STDK_LAUNCH(retopk_attend<float>, dim3((unsigned)g.S), dim3(kAttThreads), att_dyn, s, at);
      }));
    } else if (!refresh_now && !fused) {
      RtRerankArgs a{};
      a.q = q;
      a.k = (const char*)k_cache;
      a.stride_b_bytes = g.sb_bytes;
      a.stride_h_bytes = g.sh_bytes;
      a.exact = exact;
      a.cand = (const int32_t*)(ws + w.cand);
      a.n_cand = (const int32_t*)(ws + w.n_cand);
      a.cz = (float*)(ws + w.cz);
      a.sel_row = (int32_t*)(ws + w.t.sel_row);
      a.sel_z = (float*)(ws + w.t.sel_z);
      a.support_out = support_out;
      a.cand_cap = (int32_t)w.cand_cap;
      a.K = p->top_k;
      a.Hq = g.Hq;
      a.G = g.G;
      a.nsplit = (int32_t)cdiv(w.cand_cap, kRerankRows);
      a.scale = p->scale;
      const dim3 grid((unsigned)a.nsplit, (unsigned)g.S);
      STDK_TRY(launch(KID_RT_RERANK, s, [&](hipEvent_t e0, hipEvent_t e1) {
        if (g.bf16) STDK_LAUNCH(retopk_rerank<uint16_t>, grid, dim3(kRerankThreads), 0, s, a);
        else STDK_LAUNCH(retopk_rerank<float>, grid, dim3(kRerankThreads), 0, s, a);
      }));
      STDK_TRY(run_rerank_select(a, g.S, di, s));
    }
    // a8: softmax . V over the chosen rows of the heads not done above (the
    // exact-path heads, or every head without the fused kernel), and the
    // push of (q_bar, support) by one workgroup per head of that launch
    const SvPush push{(const float*)(ws + w.qbar), support_out, st->q_hat, st->support, st->head, st->count,
                      p->cache_cap, p->top_k};
    return run_sv(g, w.t, ws, v_cache, o_out, lse_out, s, nullptr, &push, step_dev, fused ? exact : nullptr);
  }();
  return finish(rc, ws, w.t.counters);
}

int32_t retopk_step(const stdk_layout* lay, const retopk_params* p, const retopk_state* st, const float* q,
                    const void* k_cache, const void* v_cache, int64_t L_t, int64_t t, int32_t* support_out,
                    float* o_out, float* lse_out, int32_t* path_out, int32_t* n_cand_out, int32_t* cand_out,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return run_retopk(lay, p, st, q, k_cache, v_cache, L_t, t, nullptr, support_out, o_out, lse_out, path_out,
                    n_cand_out, cand_out, workspace, workspace_bytes, stream);
}

int32_t retopk_step_device(const stdk_layout* lay, const retopk_params* p, const retopk_state* st, const float* q,
                           const void* k_cache, const void* v_cache, int64_t* step, int32_t* support_out,
                           float* o_out, float* lse_out, int32_t* path_out, int32_t* n_cand_out, int32_t* cand_out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!step) return fail(STDK_EINVAL, "step is NULL");
  return run_retopk(lay, p, st, q, k_cache, v_cache, 0, 0, step, support_out, o_out, lse_out, path_out, n_cand_out,
                    cand_out, workspace, workspace_bytes, stream);
}


// ---------------------------------------------------------------------------
// launch timing
// ---------------------------------------------------------------------------
int32_t stdk_profile_enable(int32_t capacity, const char* only) {
  if (capacity < 1) return fail(STDK_EINVAL, "capacity %d < 1", capacity);
  int only_id = -1;
  if (only) {
    for (int i = 0; i < KID_COUNT; ++i)
      if (std::strcmp(only, kKernelNames[i]) == 0) only_id = i;
    if (only_id < 0) return fail(STDK_EINVAL, "unknown kernel name %s", only);
  }
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.only = only_id;
  const size_t want = (size_t)capacity * 2;
  while (g_prof.ev.size() < want) {
    hipEvent_t e;
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return fail(STDK_EHIP, "hipEventCreate: %s", hipGetErrorString(err));
    g_prof.ev.push_back(e);
  }
  g_prof.kid.assign((size_t)capacity, 0);
  g_prof.used = 0;
  g_prof.on = true;
  return ok();
}

int32_t stdk_profile_disable(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = false;
  return ok();
}

int32_t stdk_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.used = 0;
  for (int i = 0; i < KID_COUNT; ++i) {
    g_prof.total_ms[i] = 0.0;
    g_prof.launches[i] = 0;
  }
  return ok();
}

int32_t stdk_profile_read(const char* name, double* total_ms, int64_t* launches) {
  if (!name || !total_ms || !launches) return fail(STDK_EINVAL, "NULL argument");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (size_t i = 0; i < g_prof.used; ++i) {
    hipError_t e = hipEventSynchronize(g_prof.ev[2 * i + 1]);
    if (e != hipSuccess) return fail(STDK_EHIP, "hipEventSynchronize: %s", hipGetErrorString(e));
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
    if (e != hipSuccess) return fail(STDK_EHIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
    g_prof.total_ms[g_prof.kid[i]] += ms;
    g_prof.launches[g_prof.kid[i]] += 1;
  }
  g_prof.used = 0;
  for (int i = 0; i < KID_COUNT; ++i) {
    if (std::strcmp(name, kKernelNames[i]) == 0) {
      *total_ms = g_prof.total_ms[i];
      *launches = g_prof.launches[i];
      return ok();
    }
  }
  return fail(STDK_EINVAL, "unknown kernel name %s", name);
}

}  // extern "C"
