// Plan kernel: builds the work list of the forward on the device, so the
// host never reads segment lengths (the PR #302 review objects to host
// syncs that read them back).
//
// One workgroup of 1024 threads:
//   1. validates every segment and counts its query tiles, ceil(used_q/R);
//      an invalid segment gets no tiles and sets a device error bit; in the
//      key-range form it also sums the segment's range lengths (its key
//      count) into the workspace;
//   2. when the launch has few query tiles, splits long key ranges into
//      chunks (split-K: up to the workspace's capacity, chunks of at least
//      kMinSplitTiles key tiles) and prefix-sums the work entries into
//      per-segment offsets;
//   3. histograms the entries by cost = number of key tiles they cover
//      (under bottom-right causal the last row of a tile sees the most);
//   4. scatters the entries into cost-descending order, so the persistent
//      forward kernel starts the longest work first.
// The order inside one cost bucket depends on atomics, but each tile's
// result does not depend on the order, so outputs are deterministic.
// Segment lengths, splits and offsets stay in LDS for launches of up to
// kPlanLdsSegs segments (the tile loops then read no global memory), and the
// prefix sums are wave shuffles plus one exchange of wave totals.
#include "gvattn_internal.h"

namespace gvattn {
namespace {

constexpr int kPlanThreads = 1024;

constexpr int kPlanWaves = kPlanThreads / 64;
// Forward entries are ordered by cost in groups of 2^kGroupShift key tiles,
// then by segment.
constexpr int kGroupShift = 3;
constexpr int kExactCost = 16;  // a multiple of 2^kGroupShift
// Segments whose lengths, splits and entry offsets the plan keeps in LDS;
// a launch with more segments reads them from global memory instead.
constexpr int kPlanLdsSegs = 2048;
// Entries the LDS entry -> segment map holds (larger lists search offsets).
constexpr int kSegMapMax = 24576;

// Exclusive prefix sum over the workgroup: an inclusive scan inside each
// wave (shuffles), then the wave totals from LDS.  *total gets the sum of
// all x.  `wsum` holds kPlanWaves values.
template <typename T>
__device__ T block_exclusive_scan(T x, T* wsum, T* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  T v = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  T base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kPlanWaves; ++i) {
    const T t = wsum[i];
    base += (i < w) ? t : T(0);
    tot += t;
  }
  *total = tot;
  __syncthreads();  // wsum is reused by the next scan
  return base + v - x;
}

// Key-range form: checks segment s's ranges and returns their total length
// in *keys (error bits, or 0).
__device__ int range_error(const PlanArgs& a, int s, int* keys) {
  const Geometry& g = a.g;
  const int r0 = g.kr_off[s], r1 = g.kr_off[s + 1];
  *keys = 0;
  if (r0 < 0 || r1 < r0 || r1 > g.nranges) return GVATTN_DEVERR_KRANGES;
  int64_t total = 0;
  for (int i = r0; i < r1; ++i) {
    const int st = g.kr_start[i], len = g.kr_len[i];
    if (st < 0 || len < 0 || (int64_t)st + len > g.total_k) return GVATTN_DEVERR_KRANGES;
    // a range's rows plus a tile of overrun stay below a 2^31-byte offset
    if ((int64_t)(len + 256) * a.k_row_bytes >= (int64_t(1) << 31)) return GVATTN_DEVERR_RANGE;
    total += len;
  }
  if (total >= (int64_t(1) << 31)) return GVATTN_DEVERR_KRANGES;
  *keys = (int)total;
  return 0;
}

// Validates segment s and returns its error bits (0: valid).  *uq and *uk
// get its used query rows and key count.  The prefix form's six loads are
// issued together, before any test, so they cost one memory latency.
__device__ int segment_error(const PlanArgs& a, int s, int* uq_out, int* uk_out) {
  const Geometry& g = a.g;
  const bool kr = g.kr_off != nullptr;
  const int cq0 = g.cu_q[s], cq1 = g.cu_q[s + 1];
  const int uq = g.used_q[s];
  const int ck0 = kr ? 0 : g.cu_k[s], ck1 = kr ? 0 : g.cu_k[s + 1];
  const int uk_p = kr ? 0 : g.used_k[s];
  *uq_out = uq;
  *uk_out = 0;
  if (cq0 < 0 || cq1 < cq0 || cq1 > g.total_q) return GVATTN_DEVERR_OFFSETS;
  int err = 0;
  if (uq < 0 || uq > cq1 - cq0) err |= GVATTN_DEVERR_USED_Q;
  // Tiles may run up to 256 rows past a segment's capacity before the
  // bounds-checked loads reject them; keep every such offset below 2^31.
  if ((int64_t)(cq1 - cq0 + 256) * a.q_row_bytes >= (int64_t(1) << 31)) err |= GVATTN_DEVERR_RANGE;
  if (kr) {
    int keys;
    err |= range_error(a, s, &keys);
    a.ws.seg_keys[s] = err ? 0 : keys;
    *uk_out = keys;
    return err;
  }
  if (ck0 < 0 || ck1 < ck0 || ck1 > g.total_k) return err | GVATTN_DEVERR_OFFSETS;
  if (uk_p < 0 || uk_p > ck1 - ck0) err |= GVATTN_DEVERR_USED_K;
  if ((int64_t)(ck1 - ck0 + 256) * a.k_row_bytes >= (int64_t(1) << 31)) err |= GVATTN_DEVERR_RANGE;
  *uk_out = uk_p;
  return err;
}

// Per-segment values the tile loops read: in LDS when the launch has at most
// kPlanLdsSegs segments, else the workspace / argument arrays.
struct SegView {
  const int32_t* uq;   // used query rows
  const int32_t* uk;   // key count (0 for a segment the plan rejected)
  int32_t* split;      // key chunks per query tile (query tiles until step 2)
  int32_t* off;        // first entry of each segment, [nseg + 1]
};

// Largest s with off[s] <= t (t < off[nseg]).
__device__ int find_segment(const int32_t* off, int nseg, int t) {
  int lo = 0, hi = nseg;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Key tiles the query tile at row0 of segment s sees (under bottom-right
// causal its last row sees the most).
__device__ int tile_key_tiles(const PlanArgs& a, const SegView& v, int s, int row0) {
  const int uq = v.uq[s];
  const int uk = v.uk[s];
  int kend = uk;
  if (a.g.causal) {
    const int r_last = min(row0 + a.rows, uq) - 1;
    kend = max(0, min(uk, r_last + uk - uq + 1));
  }
  return (kend + a.key_tile - 1) / a.key_tile;
}

// Work entry e (its segment s, first entry of s at e0): query tile
// (e - e0) / S and key chunk (e - e0) % S of the segment's S = split[s]
// chunks; the chunk covers key tiles [kt0, kt1) of that query tile.
__device__ int4 make_entry(const PlanArgs& a, const SegView& v, int s, int e0, int e, int* cost) {
  const int S = v.split[s];
  const int local = e - e0;
  if (a.mode == 1) {
    // key tile of `rows` keys: the query rows that see any of its keys
    // start at r_first (bottom-right causal); its loop runs over (query
    // head, 32-row query tile), split into S chunks when S > 1 (chunk j of
    // key tile kt is entry e0 + kt * S + j, and e names its partial slot)
    const int kt = local / S, j = local - kt * S;
    const int uq = v.uq[s], uk = v.uk[s];
    const int k_row0 = kt * a.rows;
    const int r_first = a.g.causal ? max(0, min(uq, k_row0 + uq - uk)) : 0;
    const int n_it = (a.g.hq / a.g.hkv) * ((uq + 31) / 32 - r_first / 32);
    int it0 = 0, it1 = n_it;
    if (S > 1) {
      const int chunk = (n_it + S - 1) / S;
      it0 = min(j * chunk, n_it);
      it1 = min(it0 + chunk, n_it);
    }
    *cost = min(it1 - it0, kCostBuckets - 1);
    return make_int4(s, k_row0, r_first, (e << 5) | (j << 1) | (S > 1 ? 1 : 0));
  }
  const int qt = local / S, j = local - qt * S;
  const int row0 = qt * a.rows;
  const int nkt = tile_key_tiles(a, v, s, row0);
  const int chunk = (nkt + S - 1) / S;
  const int kt0 = min(j * chunk, nkt);
  const int kt1 = min(kt0 + chunk, nkt);
  *cost = min(kt1 - kt0, kCostBuckets - 1);
  return make_int4(s, row0, kt0, (kt1 << 5) | (j << 1) | (S > 1 ? 1 : 0));
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ long long wsum64[kPlanWaves];
  __shared__ int wsum[kPlanWaves];
  __shared__ int hist[kCostBuckets];
  __shared__ int32_t l_uq[kPlanLdsSegs], l_uk[kPlanLdsSegs], l_split[kPlanLdsSegs];
  __shared__ int32_t l_off[kPlanLdsSegs + 1];
  __shared__ uint16_t seg_of[kSegMapMax];
  __shared__ int s_err;
  __shared__ int s_max_split;
  __shared__ int s_max_kt;
  const int tid = threadIdx.x;
  const int nseg = a.g.nseg;
  const bool in_lds = nseg <= kPlanLdsSegs;
  SegView v;
  v.uq = in_lds ? l_uq : a.g.used_q;
  v.uk = in_lds ? l_uk : (a.g.kr_off != nullptr ? a.ws.seg_keys : a.g.used_k);
  v.split = in_lds ? l_split : a.ws.seg_split;
  v.off = in_lds ? l_off : a.ws.seg_tile_off;
  // Without split capacity every segment has one chunk per tile: the entry
  // offsets are the tile-count prefix sums of step 1 and step 2 is skipped.
  const bool direct = a.ws.splits == 1;
  const long long cap = (long long)a.max_tiles * a.ws.splits;

  for (int b = tid; b < kCostBuckets; b += kPlanThreads) hist[b] = 0;
  if (tid == 0) {
    s_err = 0;
    s_max_split = 1;
    s_max_kt = 0;
  }
  __syncthreads();

  // 1. validation and query tiles per segment (an invalid segment: none).
  //    split holds the segment's tile count until step 2 (or 1 when direct;
  //    the per-segment tables the kernels read go to the workspace as they
  //    are computed).
  long long n_qtiles = 0;
  for (int base = 0; base < nseg; base += kPlanThreads) {
    const int s = base + tid;
    long long cnt = 0;
    if (s < nseg) {
      int uq, uk;
      const int err = segment_error(a, s, &uq, &uk);
      if (err) {
        atomicOr(&s_err, err);
        uk = 0;
      } else {
        cnt = ((a.mode == 1 ? uk : uq) + a.rows - 1) / a.rows;
        if (uq > 0) atomicMax(&s_max_kt, (uk + a.key_tile - 1) / a.key_tile);
      }
      if (in_lds) {
        l_uq[s] = uq;
        l_uk[s] = uk;
      }
      v.split[s] = direct ? 1 : (int32_t)cnt;
      if (direct && in_lds) a.ws.seg_split[s] = 1;
    }
    long long tot;
    const long long excl = block_exclusive_scan<long long>(cnt, wsum64, &tot);
    if (direct && s < nseg) {
      const int32_t o = (int32_t)min(n_qtiles + excl, cap);
      v.off[s] = o;
      if (in_lds) a.ws.seg_tile_off[s] = o;
    }
    n_qtiles += tot;
  }
  __threadfence_block();
  __syncthreads();

  long long carry = n_qtiles;
  if (!direct) {
    // 2. split-K decision, then entry counts and their offsets.  Segments
    // whose capacities overlap can claim more entries than the list holds;
    // the whole plan is then rejected (no entries) rather than written past
    // the workspace.
    const long long items = n_qtiles * a.n_head_chunks;
    const bool split_on =
        a.mode == 0 ? (a.g.kr_off == nullptr && items > 0 && items < kSplitBelow)
                    : (items > 0 && items < kBwdSplitBelow && a.part_slots >= 2 * items);
    int s_aim = 1;
    if (split_on && a.mode == 0)
      s_aim = (int)min((long long)a.ws.splits, (kSplitAim + items - 1) / items);
    else if (split_on)  // every (entry, KV head) chunk needs a partial slot
      s_aim = (int)min(min((long long)a.ws.splits, (kBwdSplitAim + items - 1) / items),
                       (long long)a.part_slots / items);
    carry = 0;
    for (int base = 0; base < nseg; base += kPlanThreads) {
      const int s = base + tid;
      long long cnt = 0;
      if (s < nseg) {
        const int qt = v.split[s];
        int S = 1;
        if (split_on && qt > 0) {
          if (a.mode == 0) {
            const int kt = (v.uk[s] + a.key_tile - 1) / a.key_tile;
            S = max(1, min(s_aim, kt / kMinSplitTiles));
          } else {  // chunks of at least kBwdMinChunk (head, query tile) steps
            const int steps = (a.g.hq / a.g.hkv) * ((v.uq[s] + 31) / 32);
            S = max(1, min(s_aim, steps / kBwdMinChunk));
          }
        }
        v.split[s] = S;
        if (in_lds) a.ws.seg_split[s] = S;
        if (S > 1) atomicMax(&s_max_split, S);
        cnt = (long long)qt * S;
      }
      long long tot;
      const long long excl = block_exclusive_scan<long long>(cnt, wsum64, &tot);
      if (s < nseg) {
        const int32_t o = (int32_t)min(carry + excl, cap);
        v.off[s] = o;
        if (in_lds) a.ws.seg_tile_off[s] = o;
      }
      carry += tot;
    }
  }
  int n_tiles = (int)min(carry, cap);
  if (carry > cap) {
    n_tiles = 0;
    if (tid == 0) s_err |= GVATTN_DEVERR_OFFSETS;
  }
  if (tid == 0) {
    v.off[nseg] = n_tiles;
    if (in_lds) a.ws.seg_tile_off[nseg] = n_tiles;
  }
  __threadfence_block();
  __syncthreads();

  // Entry -> segment map (LDS), so that the two passes over the entries
  // below look their segment up in one read instead of a binary search.
  const bool use_map = in_lds && n_tiles <= kSegMapMax;
  if (use_map) {
    for (int s = tid; s < nseg; s += kPlanThreads) {
      const int e1 = v.off[s + 1];
      for (int e = v.off[s]; e < e1; ++e) seg_of[e] = (uint16_t)s;
    }
    __syncthreads();
  }
  auto seg_of_entry = [&](int t) { return use_map ? (int)seg_of[t] : find_segment(v.off, nseg, t); };

  // 3. histogram of the sort keys.  Forward entries sort by their cost
  // coarsened to 2^kGroupShift key tiles, then by segment, when that key
  // fits the buckets: the static schedule runs consecutive entries at the
  // same time on one XCD, so grouping them by segment keeps fewer
  // segments' K/V in its L2 while the order stays longest first to within
  // the coarsening.  Otherwise (and for the key-tile plan) the key is the
  // cost.
  // Entries below kExactCost key tiles (the last rounds of the schedule)
  // keep their exact cost order, which keeps the end of the launch even.
  const int max_kt = min(s_max_kt, kCostBuckets - 1);
  const bool grouped =
      a.mode == 0 && max_kt >= kExactCost &&
      kExactCost + ((long long)(max_kt >> kGroupShift) - (kExactCost >> kGroupShift) + 1) * nseg <=
          kCostBuckets;
  auto sort_key = [&](int cost, int s) {
    if (!grouped || cost < kExactCost) return cost;
    return kExactCost + ((cost >> kGroupShift) - (kExactCost >> kGroupShift)) * nseg + (nseg - 1 - s);
  };
  for (int t = tid; t < n_tiles; t += kPlanThreads) {
    const int s = seg_of_entry(t);
    int cost;
    make_entry(a, v, s, v.off[s], t, &cost);
    atomicAdd(&hist[sort_key(cost, s)], 1);
  }
  __syncthreads();

  // bucket start positions, most expensive bucket first
  static_assert(kCostBuckets == 2 * kPlanThreads, "two buckets per thread");
  const int b_hi = kCostBuckets - 1 - 2 * tid;  // visited first
  const int b_lo = b_hi - 1;
  const int c_hi = hist[b_hi], c_lo = hist[b_lo];
  int tot;
  const int excl = block_exclusive_scan<int>(c_hi + c_lo, wsum, &tot);
  hist[b_hi] = excl;
  hist[b_lo] = excl + c_hi;
  __syncthreads();

  // 4. scatter
  for (int t = tid; t < n_tiles; t += kPlanThreads) {
    const int s = seg_of_entry(t);
    int cost;
    const int4 e = make_entry(a, v, s, v.off[s], t, &cost);
    const int pos = atomicAdd(&hist[sort_key(cost, s)], 1);
    a.ws.tiles[pos] = e;
  }
  __syncthreads();

  if (tid == 0) {
    a.ws.header->n_tiles = n_tiles;
    a.ws.header->err = s_err;
    a.ws.header->key = a.key;
    a.ws.header->rows_per_tile = a.rows;
    a.ws.header->max_split = s_max_split;
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  return launch_kernel(plan_kernel, dim3(1), dim3(kPlanThreads), s, a);
}

}  // namespace gvattn
