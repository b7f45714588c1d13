// Internal definitions shared by the gvattn HIP sources: workspace layout,
// tile shapes, kernel argument blocks and small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gvattn.h"

namespace gvattn {

// ---------------------------------------------------------------------------
// Workspace: [PlanHeader (256 B)]
//            [work list: int4 x max_tiles * splits]
//            [per-segment work offsets: int32 x (nseg + 1)]
//            [per-segment key count: int32 x (nseg + 1)] (key-range form)
//            [per-segment split count: int32 x (nseg + 1)]
//            [split partials, only when splits > 1:
//               O fp32 [splits][total_q][hq][d_v], LSE fp32 [splits][hq][total_q]]
// A work entry is (segment, first row, first key tile, end key tile * 32 +
// split index * 2 + partial flag): one query tile, or one key chunk of it
// when the problem has too few query tiles to fill the GPU.  The list is
// sorted by decreasing number of key tiles so that the persistent kernel
// takes the longest work first.
// ---------------------------------------------------------------------------
struct PlanHeader {
  int32_t n_tiles;        // work entries
  int32_t err;
  uint32_t key;
  int32_t rows_per_tile;
  int32_t max_split;      // most chunks any query tile was split into
  int32_t reserved[59];
};
static_assert(sizeof(PlanHeader) == 256, "plan header is 256 bytes");

constexpr int kCostBuckets = 2048;    // sort buckets (key tiles per entry)

// Split-K: a launch with fewer than kSplitBelow work items (query tiles x
// head chunks) may split long key ranges into up to `splits` chunks of at
// least kMinSplitTiles key tiles, aiming at about kSplitAim items; the
// chunks write FP32 partials that a merge pass combines.
constexpr int kSplitBelow = 512;
constexpr int kSplitAim = 2048;
constexpr int kMaxSplits = 16;
constexpr int kMinSplitTiles = 8;
constexpr int64_t kSplitBytes = int64_t(64) << 20;  // partials at most

// Tile shape of one forward variant.
struct TileShape {
  int rows;   // query rows per tile (per head)
  int gf;     // query heads folded into one workgroup (divides hq / hkv)
  int waves;  // waves per workgroup
};

// Folding: the workgroup owns `gf` consecutive query heads of one KV group
// and 32 * rb query rows of each, one wave per (head, 32-row block).
inline TileShape choose_shape(int dtype, int hq, int hkv, int d) {
  (void)d;
  TileShape t{};
  if (dtype == GVATTN_FP32) {
    t.rows = 16;
    t.gf = 1;
    t.waves = 4;
    return t;
  }
  const int g = hq / hkv;
  int gf = 1;
  if (g % 4 == 0) gf = 4;
  else if (g % 3 == 0) gf = 3;
  else if (g % 2 == 0) gf = 2;
  const int rb = (gf == 3) ? 1 : 4 / gf;
  t.rows = 32 * rb;
  t.gf = gf;
  t.waves = gf * rb;
  return t;
}

// Binds a plan to everything the run side derives from host sizes: tile
// shape, causal flag, segment count, variant flags (key ranges, head dims,
// backward plan kind), head counts, row totals and the workspace layout
// (split capacity and list length).  A run whose key differs from the one
// the plan stored refuses to read the plan.
struct PlanKeyArgs {
  int rows, causal, nseg, flags, hq, hkv, total_q, total_k, splits;
  int64_t max_tiles;
};

inline uint32_t plan_key(const PlanKeyArgs& k) {
  uint32_t h = 2166136261u;
  auto mix = [&h](uint32_t x) {
    for (int i = 0; i < 4; ++i) h = (h ^ ((x >> (8 * i)) & 0xffu)) * 16777619u;
  };
  mix((uint32_t)k.rows);
  mix((uint32_t)k.causal);
  mix((uint32_t)k.nseg);
  mix((uint32_t)k.flags);
  mix((uint32_t)k.hq);
  mix((uint32_t)k.hkv);
  mix((uint32_t)k.total_q);
  mix((uint32_t)k.total_k);
  mix((uint32_t)k.splits);
  mix((uint32_t)k.max_tiles);
  mix((uint32_t)(k.max_tiles >> 32));
  return h | 1u;  // never 0, so a zeroed workspace never matches
}

inline int64_t max_tiles(int64_t nseg, int64_t total_q, int rows) {
  return total_q / rows + nseg + 1;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Byte layout of the workspace; a function of host-known sizes only.
struct WsLayout {
  int64_t max_tiles;  // query tiles at most
  int32_t splits;     // key chunks per query tile at most (1: no split-K)
  size_t tiles, seg_off, seg_keys, seg_split, part_o, part_lse, bytes;
};

// allow_split = false: a plan-only region (the backward's plans), whose work
// list holds list_splits entries per tile (chunks whose partials live
// elsewhere).
// split_bytes caps the split-K partials (a caller with a fixed-size buffer
// passes what is left of it after the plan).
inline WsLayout ws_layout(int64_t nseg, int64_t total_q, int hq, int dv, const TileShape& t,
                          int dtype, bool allow_split = true, int list_splits = 1,
                          int64_t split_bytes = kSplitBytes) {
  WsLayout L{};
  L.max_tiles = max_tiles(nseg, total_q, t.rows);
  const int64_t items = L.max_tiles * (hq / t.gf);
  L.splits = allow_split ? 1 : list_splits;
  if (allow_split && dtype != GVATTN_FP32 && items < kSplitBelow) {
    int64_t s = (kSplitAim + items - 1) / items;
    const int64_t per_split = (int64_t)total_q * hq * (dv + 1) * 4;
    if (per_split > 0 && s * per_split > split_bytes) s = split_bytes / per_split;
    L.splits = (int32_t)(s < 1 ? 1 : (s < kMaxSplits ? s : kMaxSplits));
  }
  size_t b = sizeof(PlanHeader);
  L.tiles = b;
  b += align_up((size_t)L.max_tiles * L.splits * 16, 256);
  L.seg_off = b;
  b += align_up((size_t)(nseg + 1) * 4, 256);
  L.seg_keys = b;
  b += align_up((size_t)(nseg + 1) * 4, 256);
  L.seg_split = b;
  b += align_up((size_t)(nseg + 1) * 4, 256);
  L.part_o = L.part_lse = 0;
  if (allow_split && L.splits > 1) {
    L.part_o = b;
    b += align_up((size_t)L.splits * total_q * hq * dv * 4, 256);
    L.part_lse = b;
    b += align_up((size_t)L.splits * hq * total_q * 4, 256);
  }
  L.bytes = b;
  return L;
}

struct WorkspaceView {
  PlanHeader* header;
  int4* tiles;
  int32_t* seg_tile_off;
  int32_t* seg_keys;   // key-range form: total key count of each segment
  int32_t* seg_split;  // key chunks each query tile of the segment is split into
  float* part_o;       // split partials (null without split-K)
  float* part_lse;
  int32_t splits;      // capacity: most chunks per query tile
};

inline WorkspaceView view_workspace(void* ws, const WsLayout& L) {
  WorkspaceView v;
  char* p = static_cast<char*>(ws);
  v.header = reinterpret_cast<PlanHeader*>(p);
  v.tiles = reinterpret_cast<int4*>(p + L.tiles);
  v.seg_tile_off = reinterpret_cast<int32_t*>(p + L.seg_off);
  v.seg_keys = reinterpret_cast<int32_t*>(p + L.seg_keys);
  v.seg_split = reinterpret_cast<int32_t*>(p + L.seg_split);
  v.part_o = L.part_o ? reinterpret_cast<float*>(p + L.part_o) : nullptr;
  v.part_lse = L.part_lse ? reinterpret_cast<float*>(p + L.part_lse) : nullptr;
  v.splits = L.splits;
  return v;
}

// Geometry shared by plan and forward kernels.  Keys come either as a used
// prefix per segment (cu_k, used_k) or, in the key-range form (kr_off not
// null), as the ranges kr_start[i] .. + kr_len[i], i in [kr_off[s],
// kr_off[s + 1]), concatenated in order.
struct Geometry {
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* used_q;
  const int32_t* used_k;
  const int32_t* kr_off;
  const int32_t* kr_start;
  const int32_t* kr_len;
  int32_t nranges;
  int32_t nseg;
  int32_t total_q;
  int32_t total_k;
  int32_t hq;
  int32_t hkv;
  int32_t d;   // head dim of Q and K
  int32_t dv;  // head dim of V and O
  int32_t causal;
};

struct PlanArgs {
  Geometry g;
  WorkspaceView ws;
  int32_t mode;        // 0: query tiles (forward, dQ); 1: key tiles (dK / dV)
  int32_t part_slots;  // mode 1: (entry, KV head) partials available for splits
  int32_t rows;        // rows per tile
  int32_t max_tiles;   // query tiles at most (the list holds max_tiles * splits)
  int32_t key_tile;    // keys per key tile of the forward kernel
  int32_t n_head_chunks;
  uint32_t key;
  int64_t q_row_bytes;  // bytes of one packed Q/O row (all heads)
  int64_t k_row_bytes;  // bytes of one packed K or V row, the larger (all heads)
};

struct FwdArgs {
  Geometry g;
  WorkspaceView ws;
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  float scale_log2;     // softmax_scale * log2(e)
  uint32_t key;
  int32_t n_head_chunks;  // hq / gf
  int32_t n_cu;           // compute units of the device (set by the launcher)
};

// Backward: the forward's query-tile plan drives the dQ kernel, a key-tile
// plan (entries: segment, first key row, first query row that sees those
// keys) drives the dK / dV kernel.  The dQ kernel also writes the per-row
// statistics the dK / dV kernel reads: (LSE * log2 e, D = rowsum(dO * O))
// per (head, row), +inf in place of LSE * log2 e for a row without keys.
struct BwdArgs {
  Geometry g;
  WorkspaceView qws;
  WorkspaceView kws;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* stats;         // [hq, total_q] x 2 floats
  float* kpart;         // split dK / dV partials: [slot][hkv][64 keys][d + d_v] fp32
  int32_t kpart_slots;  // (slot, KV head) pairs kpart holds
  void* dq;
  void* dk;
  void* dv;
  float scale;
  float scale_log2;     // scale * log2(e)
  uint32_t qkey, kkey;
  int32_t n_head_chunks;  // hq / gf (dQ kernel)
  int32_t n_cu;
};

// Workspace of the backward: [query-tile plan][key-tile plan][row stats]
// [dK / dV partials].  A launch with fewer than kBwdSplitBelow dK / dV items
// (key tiles x KV heads) splits each item's (query head, query tile) loop
// into up to kMaxSplits chunks of at least kBwdMinChunk iterations, aiming
// at kBwdSplitAim items; each chunk writes FP32 partials into one of
// part_slots (entry, KV head) slots and a reduce pass sums them.
constexpr int kBwdKeyRows = 64;    // keys per dK / dV work item (2 wave pairs x 32)
constexpr int kBwdSplitBelow = 384;
constexpr int kBwdSplitAim = 1536;
constexpr int kBwdMinChunk = 8;
constexpr int kBwdPartSlots = 1024;
struct BwdLayout {
  WsLayout q, k;
  int32_t part_slots;
  size_t kplan, stats, kpart, bytes;
};
inline BwdLayout bwd_layout(int64_t nseg, int64_t total_q, int64_t total_k, int hq, int hkv,
                            int d, int dv, const TileShape& t, int dtype) {
  BwdLayout B;
  B.q = ws_layout(nseg, total_q, hq, dv, t, dtype, false);
  TileShape tk = t;
  tk.rows = kBwdKeyRows;
  tk.gf = 1;
  B.k = ws_layout(nseg, total_k, hq, dv, tk, dtype, false, kMaxSplits);
  const int64_t slots = B.k.max_tiles * hkv * kMaxSplits;
  B.part_slots = (int32_t)(slots < kBwdPartSlots ? slots : kBwdPartSlots);
  B.kplan = align_up(B.q.bytes, 256);
  B.stats = B.kplan + align_up(B.k.bytes, 256);
  B.kpart = B.stats + align_up((size_t)hq * total_q * 8, 256);
  B.bytes = B.kpart + align_up((size_t)B.part_slots * kBwdKeyRows * (d + dv) * 4, 256);
  return B;
}

struct MergeArgs {
  const void* part_out[GVATTN_MAX_PARTS];
  const float* part_lse[GVATTN_MAX_PARTS];
  int32_t nparts;
  const int32_t* cu_q;
  const int32_t* used_q;
  int32_t nseg;
  int32_t total_q;
  int32_t hq;
  int32_t d;
  void* out;
  float* lse;
  int32_t* err;
};

// Launches `kern` and returns the status of this launch itself, never an
// error some earlier runtime call of other code left in this thread's
// last-error slot (hipLaunchKernelGGL + hipGetLastError would report that).
template <typename T> struct NoDeduce { using type = T; };
template <typename... P>
inline hipError_t launch_kernel(void (*kern)(P...), dim3 grid, dim3 block, hipStream_t s,
                                typename NoDeduce<P>::type... args) {
  void* ptrs[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, 0, s);
}

// Host-side launchers (one translation unit each).
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
// Combines the split-K partials of the segments the plan split (dtype of
// the output: GVATTN_BF16 or GVATTN_FP16).
hipError_t launch_split_merge(const FwdArgs& a, int dtype, hipStream_t s);
// Backward: dQ (and the row statistics), then dK / dV (dtype GVATTN_BF16 or
// GVATTN_FP16; d and d_v 64 or 128).  The two plans must have been built.
hipError_t launch_bwd(const BwdArgs& a, int dtype, const TileShape& t, hipStream_t s,
                      bool* supported);
// Matrix-core forward for 16-bit inputs (dtype GVATTN_BF16 or GVATTN_FP16);
// the key-range form when a.g.kr_off is set.
hipError_t launch_fwd_mfma(const FwdArgs& a, int dtype, const TileShape& t, int64_t max_work,
                           hipStream_t s, bool* supported);
hipError_t launch_fwd_fp32(const FwdArgs& a, const TileShape& t, int64_t max_work,
                           hipStream_t s, bool* supported);
hipError_t launch_merge(const MergeArgs& a, int part_dtype, int out_dtype, hipStream_t s,
                        bool* supported);

// Persistent grid size for a kernel: resident blocks per CU x CUs, capped by
// the work available.
int persistent_grid(const void* kernel, int threads, int64_t max_work);

// Compute units of the current device (cached), or -1 on a HIP error.
int device_cu_count();

}  // namespace gvattn

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#if defined(__HIPCC__)
namespace gvattn {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource: loads at byte offsets >= num_bytes return zero and
// stores there are dropped, which is how ragged tiles, gap rows and the
// ends of buffers are guarded.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)num_bytes, 0x00020000);
}

__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

__device__ inline void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

// The same with the non-temporal policy (gfx950 cache-policy bit `nt`), for
// output nothing in the kernel reads again: its lines then leave the L2
// early instead of displacing K/V that later tiles still read.
__device__ inline void buf_store16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 2);
}

__device__ inline float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

__device__ inline void buf_store_f32(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (lane ^ 32).
__device__ inline float swap_halves(float x) { return __shfl_xor(x, 32); }

}  // namespace dev
}  // namespace gvattn
#endif
