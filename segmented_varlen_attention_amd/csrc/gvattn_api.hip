// C ABI of gvattn: argument validation, workspace layout, kernel dispatch.
// Every host-checkable problem is rejected before any HIP call, so the
// validation paths run (and are tested) on machines without a GPU.
#include <math.h>

#include <stdio.h>
#include <stdlib.h>

#include <mutex>
#include <unordered_map>

#include "gvattn_internal.h"

namespace gvattn {

int persistent_grid(const void* kernel, int threads, int64_t max_work) {
  if (max_work <= 0) return 0;
  struct Key {
    const void* k;
    int dev;
    bool operator==(const Key& o) const { return k == o.k && dev == o.dev; }
  };
  struct Hash {
    size_t operator()(const Key& k) const {
      return std::hash<const void*>()(k.k) ^ (std::hash<int>()(k.dev) << 1);
    }
  };
  static std::mutex mu;
  static std::unordered_map<Key, int, Hash> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  int slots = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(Key{kernel, dev});
    if (it != cache.end()) {
      slots = it->second;
    } else {
      int per_cu = 0, cus = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
        return -1;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return -1;
      slots = (per_cu > 0 ? per_cu : 1) * cus;
      cache.emplace(Key{kernel, dev}, slots);
    }
  }
  return (int)(max_work < slots ? max_work : slots);
}

int device_cu_count() {
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  cache.emplace(dev, cus);
  return cus;
}

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// GVATTN_ERR_HIP for a failed runtime call; with GVATTN_DEBUG set in the
// environment the HIP error and the step are also printed to stderr.
int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return GVATTN_OK;
  static const bool debug = getenv("GVATTN_DEBUG") != nullptr;
  if (debug) fprintf(stderr, "gvattn: %s: %s (%d)\n", where, hipGetErrorString(e), (int)e);
  return GVATTN_ERR_HIP;
}

bool dtype_ok(int32_t dtype) {
  return dtype == GVATTN_FP32 || dtype == GVATTN_BF16 || dtype == GVATTN_FP16;
}
bool dim_ok(int32_t d) { return d == 64 || d == 128 || d == 256; }
int esize(int32_t dtype) { return dtype == GVATTN_FP32 ? 4 : 2; }

int check_sizes(int32_t dtype, int32_t nseg, int32_t total_q, int32_t total_k, int32_t hq,
                int32_t hkv, int32_t d, int32_t dv, int32_t causal) {
  if (!dtype_ok(dtype)) return GVATTN_ERR_UNSUPPORTED;
  if (nseg < 0 || total_q < 0 || total_k < 0 || hq <= 0 || hkv <= 0) return GVATTN_ERR_INVALID_ARG;
  if (hq % hkv != 0) return GVATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return GVATTN_ERR_INVALID_ARG;
  if (!dim_ok(d) || !dim_ok(dv)) return GVATTN_ERR_UNSUPPORTED;
  // one packed row (all heads) must stay well inside a 32-bit byte offset
  if ((int64_t)hq * (d > dv ? d : dv) * esize(dtype) > (int64_t(1) << 24))
    return GVATTN_ERR_UNSUPPORTED;
  return GVATTN_OK;
}

WsLayout layout_of(int32_t dtype, int32_t nseg, int32_t total_q, int32_t hq, int32_t hkv,
                   int32_t d, int32_t dv) {
  return ws_layout(nseg, total_q, hq, dv, choose_shape(dtype, hq, hkv, d), dtype);
}

int check_workspace(const void* ws, size_t bytes, const WsLayout& L) {
  if (ws == nullptr) return GVATTN_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % GVATTN_WORKSPACE_ALIGN != 0) return GVATTN_ERR_WORKSPACE;
  if (bytes < L.bytes) return GVATTN_ERR_WORKSPACE;
  return GVATTN_OK;
}

// keys per key tile of the forward kernel (split-K chunks are whole tiles)
int key_tile(int32_t d, int32_t dv) { return (d <= 128 && dv <= 128) ? 32 : 64; }

// The plan key of a geometry: the run side recomputes it and refuses a plan
// built for anything else (another head layout, row total or workspace
// layout included).
uint32_t geometry_key(int rows, const Geometry& g, const WsLayout& L, int flags) {
  PlanKeyArgs k;
  k.rows = rows;
  k.causal = g.causal;
  k.nseg = g.nseg;
  k.flags = flags | (g.d << 1) | (g.dv << 10);
  k.hq = g.hq;
  k.hkv = g.hkv;
  k.total_q = g.total_q;
  k.total_k = g.total_k;
  k.splits = L.splits;
  k.max_tiles = L.max_tiles;
  return plan_key(k);
}

Geometry make_geom(const int32_t* cu_q, const int32_t* cu_k, const int32_t* used_q,
                   const int32_t* used_k, int32_t nseg, int32_t total_q, int32_t total_k,
                   int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t causal) {
  Geometry g;
  g.cu_q = cu_q;
  g.cu_k = cu_k;
  g.used_q = used_q;
  g.used_k = used_k;
  g.nseg = nseg;
  g.total_q = total_q;
  g.total_k = total_k;
  g.hq = hq;
  g.hkv = hkv;
  g.d = d;
  g.dv = dv;
  g.causal = causal;
  g.kr_off = nullptr;
  g.kr_start = nullptr;
  g.kr_len = nullptr;
  g.nranges = 0;
  return g;
}

int do_plan(int32_t dtype, const Geometry& g, const WsLayout& L, void* ws, hipStream_t stream) {
  const TileShape t = choose_shape(dtype, g.hq, g.hkv, g.d);
  PlanArgs a;
  a.g = g;
  a.ws = view_workspace(ws, L);
  a.mode = 0;
  a.part_slots = 0;
  a.rows = t.rows;
  a.max_tiles = (int32_t)L.max_tiles;
  a.key_tile = key_tile(g.d, g.dv);
  a.n_head_chunks = g.hq / t.gf;
  a.key = geometry_key(t.rows, g, L, g.kr_off != nullptr ? 1 : 0);
  const int dmax = g.d > g.dv ? g.d : g.dv;
  a.q_row_bytes = (int64_t)g.hq * dmax * esize(dtype);
  a.k_row_bytes = (int64_t)g.hkv * dmax * esize(dtype);
  return hip_status(launch_plan(a, stream), "plan");
}

int do_run(int32_t dtype, const Geometry& g, const WsLayout& L, const void* q, const void* k,
           const void* v, float scale, void* out, float* lse, void* ws, hipStream_t stream) {
  const TileShape t = choose_shape(dtype, g.hq, g.hkv, g.d);
  FwdArgs a;
  a.g = g;
  a.ws = view_workspace(ws, L);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.scale_log2 = scale * kLog2e;
  a.key = geometry_key(t.rows, g, L, g.kr_off != nullptr ? 1 : 0);
  a.n_head_chunks = g.hq / t.gf;
  const int64_t max_work = L.max_tiles * L.splits * a.n_head_chunks;
  bool ok = false;
  hipError_t e = (dtype != GVATTN_FP32) ? launch_fwd_mfma(a, dtype, t, max_work, stream, &ok)
                                        : launch_fwd_fp32(a, t, max_work, stream, &ok);
  if (!ok) return GVATTN_ERR_UNSUPPORTED;
  if (e == hipSuccess && L.splits > 1) e = launch_split_merge(a, dtype, stream);
  return hip_status(e, "forward");
}

int check_fwd_args(int32_t dtype, const void* q, const void* k, const void* v,
                   const int32_t* cu_q, const int32_t* cu_k, const int32_t* used_q,
                   const int32_t* used_k, int32_t nseg, int32_t total_q, int32_t total_k,
                   int32_t hq, int32_t hkv, int32_t d, int32_t dv, float scale,
                   int32_t causal, void* out, float* lse, void* ws, size_t ws_bytes) {
  int rc = check_sizes(dtype, nseg, total_q, total_k, hq, hkv, d, dv, causal);
  if (rc != GVATTN_OK) return rc;
  if (!(scale > 0.f) || !isfinite(scale)) return GVATTN_ERR_INVALID_ARG;
  if (nseg == 0) return GVATTN_OK;
  if (!q || !k || !v || !cu_q || !cu_k || !used_q || !used_k || !out || !lse)
    return GVATTN_ERR_INVALID_ARG;
  return check_workspace(ws, ws_bytes, layout_of(dtype, nseg, total_q, hq, hkv, d, dv));
}

// ---- allocation-free forward -------------------------------------------------

// Device memory of gvattn_fwd_noalloc: the plan and any split-K partials.
// Each device the library runs on holds its own copy until the process
// ends.  Host code never uses this name as an address (on the host it is
// only a stand-in); it uses the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) char scratch[GVATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Address of the current device's scratch array, looked up once per device
// (with that device current).
hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

// Workspace layout that fits the scratch array: the ordinary layout when it
// fits, else the same with fewer split-K chunks.  bytes > the array's size
// when even the plan alone does not fit.
WsLayout noalloc_layout(int32_t dtype, int32_t nseg, int32_t total_q, int32_t hq, int32_t hkv,
                        int32_t d, int32_t dv) {
  const TileShape t = choose_shape(dtype, hq, hkv, d);
  const int64_t cap = (int64_t)GVATTN_NOALLOC_SCRATCH_BYTES;
  const int64_t per_split = (int64_t)total_q * hq * (dv + 1) * 4;
  WsLayout L = ws_layout(nseg, total_q, hq, dv, t, dtype);
  while ((int64_t)L.bytes > cap && L.splits > 1)  // one chunk fewer at a time
    L = ws_layout(nseg, total_q, hq, dv, t, dtype, true, 1, (int64_t)(L.splits - 1) * per_split);
  return L;
}

// ---- backward --------------------------------------------------------------

constexpr int kPlanBwdQ = 1 << 20, kPlanBwdK = 2 << 20;  // plan-key flags

bool bwd_dim_ok(int32_t d) { return d == 64 || d == 128; }

int check_bwd_sizes(int32_t dtype, int32_t nseg, int32_t total_q, int32_t total_k, int32_t hq,
                    int32_t hkv, int32_t d, int32_t dv, int32_t causal) {
  const int rc = check_sizes(dtype, nseg, total_q, total_k, hq, hkv, d, dv, causal);
  if (rc != GVATTN_OK) return rc;
  if (dtype == GVATTN_FP32 || !bwd_dim_ok(d) || !bwd_dim_ok(dv)) return GVATTN_ERR_UNSUPPORTED;
  return GVATTN_OK;
}

BwdLayout bwd_layout_of(int32_t dtype, int32_t nseg, int32_t total_q, int32_t total_k,
                        int32_t hq, int32_t hkv, int32_t d, int32_t dv) {
  return bwd_layout(nseg, total_q, total_k, hq, hkv, d, dv, choose_shape(dtype, hq, hkv, d), dtype);
}

int do_bwd(int32_t dtype, const Geometry& g, const void* q, const void* k, const void* v,
           const void* out, const void* dout, const float* lse, float scale, void* dq,
           void* dk, void* dv, void* ws, hipStream_t stream) {
  const TileShape t = choose_shape(dtype, g.hq, g.hkv, g.d);
  const BwdLayout L = bwd_layout_of(dtype, g.nseg, g.total_q, g.total_k, g.hq, g.hkv, g.d, g.dv);
  char* base = static_cast<char*>(ws);
  const int dmax = g.d > g.dv ? g.d : g.dv;

  PlanArgs pq;
  pq.g = g;
  pq.ws = view_workspace(base, L.q);
  pq.mode = 0;
  pq.part_slots = 0;
  pq.rows = t.rows;
  pq.max_tiles = (int32_t)L.q.max_tiles;
  pq.key_tile = 32;
  pq.n_head_chunks = g.hq / t.gf;
  pq.key = geometry_key(t.rows, g, L.q, kPlanBwdQ);
  pq.q_row_bytes = (int64_t)g.hq * dmax * esize(dtype);
  pq.k_row_bytes = (int64_t)g.hkv * dmax * esize(dtype);
  PlanArgs pk = pq;
  pk.ws = view_workspace(base + L.kplan, L.k);
  pk.mode = 1;
  pk.part_slots = L.part_slots;
  pk.rows = kBwdKeyRows;
  pk.max_tiles = (int32_t)L.k.max_tiles;
  pk.n_head_chunks = g.hkv;
  pk.key = geometry_key(kBwdKeyRows, g, L.k, kPlanBwdK);
  int rc = hip_status(launch_plan(pq, stream), "backward query plan");
  if (rc == GVATTN_OK) rc = hip_status(launch_plan(pk, stream), "backward key plan");
  if (rc != GVATTN_OK) return rc;

  BwdArgs b;
  b.g = g;
  b.qws = pq.ws;
  b.kws = pk.ws;
  b.q = q;
  b.k = k;
  b.v = v;
  b.o = out;
  b.dout = dout;
  b.lse = lse;
  b.stats = reinterpret_cast<float*>(base + L.stats);
  b.kpart = reinterpret_cast<float*>(base + L.kpart);
  b.kpart_slots = L.part_slots;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.scale = scale;
  b.scale_log2 = scale * kLog2e;
  b.qkey = pq.key;
  b.kkey = pk.key;
  b.n_head_chunks = pq.n_head_chunks;
  b.n_cu = 0;
  bool ok = false;
  const hipError_t e = launch_bwd(b, dtype, t, stream, &ok);
  if (!ok) return GVATTN_ERR_UNSUPPORTED;
  return hip_status(e, "backward");
}

}  // namespace
}  // namespace gvattn

using namespace gvattn;

extern "C" {

size_t gvattn_fwd_workspace_size(int32_t nseg, int32_t total_q, int32_t hq, int32_t hkv,
                                 int32_t d, int32_t d_v, int32_t dtype) {
  if (check_sizes(dtype, nseg, total_q, 0, hq, hkv, d, d_v, 0) != GVATTN_OK) return 0;
  return layout_of(dtype, nseg, total_q, hq, hkv, d, d_v).bytes;
}

int gvattn_fwd_plan(int32_t dtype, const int32_t* cu_q, const int32_t* cu_k,
                    const int32_t* used_q, const int32_t* used_k, int32_t nseg,
                    int32_t total_q, int32_t total_k, int32_t hq, int32_t hkv, int32_t d,
                    int32_t d_v, int32_t causal, void* workspace, size_t workspace_bytes_,
                    void* hip_stream) {
  int rc = check_sizes(dtype, nseg, total_q, total_k, hq, hkv, d, d_v, causal);
  if (rc != GVATTN_OK) return rc;
  if (nseg == 0) return GVATTN_OK;
  if (!cu_q || !cu_k || !used_q || !used_k) return GVATTN_ERR_INVALID_ARG;
  rc = check_workspace(workspace, workspace_bytes_,
                       layout_of(dtype, nseg, total_q, hq, hkv, d, d_v));
  if (rc != GVATTN_OK) return rc;
  const Geometry g =
      make_geom(cu_q, cu_k, used_q, used_k, nseg, total_q, total_k, hq, hkv, d, d_v, causal);
  return do_plan(dtype, g, layout_of(dtype, nseg, total_q, hq, hkv, d, d_v), workspace,
                 static_cast<hipStream_t>(hip_stream));
}

int gvattn_fwd_run(int32_t dtype, const void* q, const void* k, const void* v,
                   const int32_t* cu_q, const int32_t* cu_k, const int32_t* used_q,
                   const int32_t* used_k, int32_t nseg, int32_t total_q, int32_t total_k,
                   int32_t hq, int32_t hkv, int32_t d, int32_t d_v, float softmax_scale,
                   int32_t causal,
                   void* out, float* lse, void* workspace, size_t workspace_bytes_,
                   void* hip_stream) {
  int rc = check_fwd_args(dtype, q, k, v, cu_q, cu_k, used_q, used_k, nseg, total_q, total_k,
                          hq, hkv, d, d_v, softmax_scale, causal, out, lse, workspace,
                          workspace_bytes_);
  if (rc != GVATTN_OK || nseg == 0) return rc;
  const Geometry g =
      make_geom(cu_q, cu_k, used_q, used_k, nseg, total_q, total_k, hq, hkv, d, d_v, causal);
  return do_run(dtype, g, layout_of(dtype, nseg, total_q, hq, hkv, d, d_v), q, k, v,
                softmax_scale, out, lse, workspace, static_cast<hipStream_t>(hip_stream));
}

int gvattn_fwd(int32_t dtype, const void* q, const void* k, const void* v,
               const int32_t* cu_q, const int32_t* cu_k, const int32_t* used_q,
               const int32_t* used_k, int32_t nseg, int32_t total_q, int32_t total_k,
               int32_t hq, int32_t hkv, int32_t d, int32_t d_v, float softmax_scale,
               int32_t causal,
               void* out, float* lse, void* workspace, size_t workspace_bytes_,
               void* hip_stream) {
  int rc = check_fwd_args(dtype, q, k, v, cu_q, cu_k, used_q, used_k, nseg, total_q, total_k,
                          hq, hkv, d, d_v, softmax_scale, causal, out, lse, workspace,
                          workspace_bytes_);
  if (rc != GVATTN_OK || nseg == 0) return rc;
  const Geometry g =
      make_geom(cu_q, cu_k, used_q, used_k, nseg, total_q, total_k, hq, hkv, d, d_v, causal);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const WsLayout L = layout_of(dtype, nseg, total_q, hq, hkv, d, d_v);
  rc = do_plan(dtype, g, L, workspace, s);
  if (rc != GVATTN_OK) return rc;
  return do_run(dtype, g, L, q, k, v, softmax_scale, out, lse, workspace, s);
}

int gvattn_fwd_ranges(int32_t dtype, const void* q, const void* k, const void* v,
                      const int32_t* cu_q, const int32_t* used_q, const int32_t* kr_off,
                      const int32_t* kr_start, const int32_t* kr_len, int32_t nseg,
                      int32_t nranges, int32_t total_q, int32_t total_k, int32_t hq,
                      int32_t hkv, int32_t d, int32_t d_v, float softmax_scale,
                      int32_t causal, void* out, float* lse, void* workspace,
                      size_t workspace_bytes_, void* hip_stream) {
  int rc = check_sizes(dtype, nseg, total_q, total_k, hq, hkv, d, d_v, causal);
  if (rc != GVATTN_OK) return rc;
  if (nranges < 0) return GVATTN_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return GVATTN_ERR_INVALID_ARG;
  if (nseg == 0) return GVATTN_OK;
  if (!q || !k || !v || !cu_q || !used_q || !kr_off || !out || !lse) return GVATTN_ERR_INVALID_ARG;
  if (nranges > 0 && (!kr_start || !kr_len)) return GVATTN_ERR_INVALID_ARG;
  rc = check_workspace(workspace, workspace_bytes_,
                       layout_of(dtype, nseg, total_q, hq, hkv, d, d_v));
  if (rc != GVATTN_OK) return rc;
  Geometry g = make_geom(cu_q, nullptr, used_q, nullptr, nseg, total_q, total_k, hq, hkv, d,
                         d_v, causal);
  g.kr_off = kr_off;
  g.kr_start = kr_start;
  g.kr_len = kr_len;
  g.nranges = nranges;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const WsLayout L = layout_of(dtype, nseg, total_q, hq, hkv, d, d_v);
  rc = do_plan(dtype, g, L, workspace, s);
  if (rc != GVATTN_OK) return rc;
  return do_run(dtype, g, L, q, k, v, softmax_scale, out, lse, workspace, s);
}

int gvattn_fwd_noalloc(int32_t dtype, const void* q, const void* k, const void* v,
                       const int32_t* cu_q, const int32_t* cu_k, const int32_t* used_q,
                       const int32_t* used_k, int32_t nseg, int32_t total_q, int32_t total_k,
                       int32_t hq, int32_t hkv, int32_t d, int32_t d_v, float softmax_scale,
                       int32_t causal, void* out, float* lse, void* hip_stream) {
  int rc = check_sizes(dtype, nseg, total_q, total_k, hq, hkv, d, d_v, causal);
  if (rc != GVATTN_OK) return rc;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return GVATTN_ERR_INVALID_ARG;
  if (nseg == 0) return GVATTN_OK;
  if (!q || !k || !v || !cu_q || !cu_k || !used_q || !used_k || !out || !lse)
    return GVATTN_ERR_INVALID_ARG;
  const WsLayout L = noalloc_layout(dtype, nseg, total_q, hq, hkv, d, d_v);
  if (L.bytes > (size_t)GVATTN_NOALLOC_SCRATCH_BYTES) return GVATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  rc = hip_status(scratch_address(&ws), "scratch address");
  if (rc != GVATTN_OK) return rc;
  const Geometry g =
      make_geom(cu_q, cu_k, used_q, used_k, nseg, total_q, total_k, hq, hkv, d, d_v, causal);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  rc = do_plan(dtype, g, L, ws, s);
  if (rc != GVATTN_OK) return rc;
  return do_run(dtype, g, L, q, k, v, softmax_scale, out, lse, ws, s);
}

int gvattn_lse_merge(int32_t nparts, const void* const* part_out, const float* const* part_lse,
                     int32_t part_dtype, int32_t out_dtype, const int32_t* cu_q,
                     const int32_t* used_q, int32_t nseg, int32_t total_q, int32_t hq,
                     int32_t d, void* out, float* lse, int32_t* device_error,
                     void* hip_stream) {
  if (!dtype_ok(part_dtype) || !dtype_ok(out_dtype)) return GVATTN_ERR_UNSUPPORTED;
  if (nparts < 1) return GVATTN_ERR_INVALID_ARG;
  if (nparts > GVATTN_MAX_PARTS) return GVATTN_ERR_UNSUPPORTED;
  if (nseg < 0 || total_q < 0 || hq <= 0) return GVATTN_ERR_INVALID_ARG;
  if (!dim_ok(d)) return GVATTN_ERR_UNSUPPORTED;
  if (nseg == 0 || total_q == 0) return GVATTN_OK;
  if (!part_out || !part_lse || !cu_q || !used_q || !out || !lse) return GVATTN_ERR_INVALID_ARG;
  MergeArgs a;
  for (int p = 0; p < GVATTN_MAX_PARTS; ++p) {
    a.part_out[p] = nullptr;
    a.part_lse[p] = nullptr;
  }
  for (int p = 0; p < nparts; ++p) {
    if (!part_out[p] || !part_lse[p]) return GVATTN_ERR_INVALID_ARG;
    a.part_out[p] = part_out[p];
    a.part_lse[p] = part_lse[p];
  }
  if (out == part_out[0] && out_dtype != part_dtype) return GVATTN_ERR_INVALID_ARG;
  a.nparts = nparts;
  a.cu_q = cu_q;
  a.used_q = used_q;
  a.nseg = nseg;
  a.total_q = total_q;
  a.hq = hq;
  a.d = d;
  a.out = out;
  a.lse = lse;
  a.err = device_error;
  bool ok = false;
  hipError_t e = launch_merge(a, part_dtype, out_dtype, static_cast<hipStream_t>(hip_stream), &ok);
  if (!ok) return GVATTN_ERR_UNSUPPORTED;
  return hip_status(e, "merge");
}

size_t gvattn_bwd_workspace_size(int32_t nseg, int32_t total_q, int32_t total_k, int32_t hq,
                                 int32_t hkv, int32_t d, int32_t d_v, int32_t dtype) {
  if (check_bwd_sizes(dtype, nseg, total_q, total_k, hq, hkv, d, d_v, 0) != GVATTN_OK) return 0;
  return bwd_layout_of(dtype, nseg, total_q, total_k, hq, hkv, d, d_v).bytes;
}

int gvattn_bwd(int32_t dtype, const void* q, const void* k, const void* v, const void* out,
               const void* dout, const float* lse, const int32_t* cu_q, const int32_t* cu_k,
               const int32_t* used_q, const int32_t* used_k, int32_t nseg, int32_t total_q,
               int32_t total_k, int32_t hq, int32_t hkv, int32_t d, int32_t d_v,
               float softmax_scale, int32_t causal, void* dq, void* dk, void* dv,
               void* workspace, size_t workspace_bytes_, void* hip_stream) {
  int rc = check_bwd_sizes(dtype, nseg, total_q, total_k, hq, hkv, d, d_v, causal);
  if (rc != GVATTN_OK) return rc;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return GVATTN_ERR_INVALID_ARG;
  if (nseg == 0) return GVATTN_OK;
  if (!q || !k || !v || !out || !dout || !lse || !cu_q || !cu_k || !used_q || !used_k || !dq ||
      !dk || !dv)
    return GVATTN_ERR_INVALID_ARG;
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % GVATTN_WORKSPACE_ALIGN != 0 ||
      workspace_bytes_ < bwd_layout_of(dtype, nseg, total_q, total_k, hq, hkv, d, d_v).bytes)
    return GVATTN_ERR_WORKSPACE;
  const Geometry g =
      make_geom(cu_q, cu_k, used_q, used_k, nseg, total_q, total_k, hq, hkv, d, d_v, causal);
  return do_bwd(dtype, g, q, k, v, out, dout, lse, softmax_scale, dq, dk, dv, workspace,
                static_cast<hipStream_t>(hip_stream));
}

const char* gvattn_status_string(int status) {
  switch (status) {
    case GVATTN_OK: return "GVATTN_OK";
    case GVATTN_ERR_INVALID_ARG: return "GVATTN_ERR_INVALID_ARG: invalid argument";
    case GVATTN_ERR_UNSUPPORTED: return "GVATTN_ERR_UNSUPPORTED: head dim, dtype or partition count not supported";
    case GVATTN_ERR_WORKSPACE: return "GVATTN_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case GVATTN_ERR_HIP: return "GVATTN_ERR_HIP: HIP runtime error";
    default: return "unknown gvattn status";
  }
}

int gvattn_read_device_error(const void* workspace, void* hip_stream, int32_t* err_out) {
  if (!workspace || !err_out) return GVATTN_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const PlanHeader* h = static_cast<const PlanHeader*>(workspace);
  int32_t v = 0;
  if (hipStreamSynchronize(s) != hipSuccess) return GVATTN_ERR_HIP;
  if (hipMemcpy(&v, &h->err, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return GVATTN_ERR_HIP;
  *err_out = v;
  return GVATTN_OK;
}

int gvattn_version(void) { return 100; }

}  // extern "C"
