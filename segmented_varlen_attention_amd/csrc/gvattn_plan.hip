// Plan kernel: builds the work list of the forward on the device, so the
// host never reads segment lengths (the PR #302 review objects to host
// syncs that read them back).
//
// One workgroup of 512 threads:
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
// prefix sums and reductions move values between the lanes of a wave with
// DPP, in registers, plus one exchange of wave totals (up to 64 segments or
// 512 buckets, one wave alone and no exchange).  The kernel is
// latency-bound: one memory round trip, a few barriers and the LDS
// atomics.  Each thread takes a contiguous run of entries (one segment
// lookup for all of them), and the atomics of a wave are aggregated over
// neighbouring lanes with equal keys.
#include <climits>
#include <type_traits>

#include "gvattn_internal.h"

namespace gvattn {
namespace {

constexpr int kPlanThreads = 512;

constexpr int kPlanWaves = kPlanThreads / 64;
// Forward entries are ordered by cost in groups of 2^kGroupShift key tiles,
// then by segment.
constexpr int kGroupShift = 3;
constexpr int kExactCost = 16;  // a multiple of 2^kGroupShift
// Segments whose lengths, splits and entry offsets the plan keeps in LDS;
// a launch with more segments reads them from global memory instead.
constexpr int kPlanLdsSegs = 2048;

// Cross-lane steps on DPP (the data-parallel-primitive operand modifier of
// gfx9 vector instructions), which move values between lanes in registers
// instead of a round trip through the LDS crossbar (ds_bpermute):
// row_shr:n reads the lane n below inside each row of 16 lanes, row_bcast:15
// hands lane 15 of each row to the row above it, row_bcast:31 hands lane 31
// to rows 2 and 3.  A lane whose source is outside its row, or whose row the
// row mask leaves out, gets `id`.
constexpr int kDppRowShr = 0x110;  // + n
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_int(int v, int id) {
  return __builtin_amdgcn_update_dpp(id, v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ long long dpp_int(long long v, long long id) {
  const int lo = __builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(id >> 32), (int)(v >> 32), CTRL, ROWS, 0xf, false);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// Inclusive scan of op over the 64 lanes of a wave (every lane takes part):
// shifts of 1, 2, 4 and 8 lanes inside each row, then every row combines
// the totals of the rows below it.
template <typename T, typename Op>
__device__ __forceinline__ T wave_inclusive(T v, T id, Op op) {
  v = op(v, dpp_int<kDppRowShr + 1, 0xf>(v, id));
  v = op(v, dpp_int<kDppRowShr + 2, 0xf>(v, id));
  v = op(v, dpp_int<kDppRowShr + 4, 0xf>(v, id));
  v = op(v, dpp_int<kDppRowShr + 8, 0xf>(v, id));
  v = op(v, dpp_int<kDppRowBcast15, 0xa>(v, id));
  v = op(v, dpp_int<kDppRowBcast31, 0xc>(v, id));
  return v;
}

template <typename T>
__device__ __forceinline__ T lane63(T v) {
  if constexpr (sizeof(T) == 8) {
    const unsigned lo = __builtin_amdgcn_readlane((int)v, 63);
    const unsigned hi = __builtin_amdgcn_readlane((int)((long long)v >> 32), 63);
    return (T)(((unsigned long long)hi << 32) | lo);
  } else {
    return (T)__builtin_amdgcn_readlane((int)v, 63);
  }
}

struct AddOp {
  template <typename T> __device__ T operator()(T a, T b) const { return a + b; }
};

// Exclusive prefix sum over the workgroup: an inclusive scan inside each
// wave, then the wave totals from LDS.  *total gets the sum of all x.
// `wsum` holds kPlanWaves values.
template <typename T>
__device__ T block_exclusive_scan(T x, T* wsum, T* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const T v = wave_inclusive<T>(x, T(0), AddOp{});
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

// Wave reductions (every lane of the wave takes part; uniform result).
__device__ __forceinline__ int wave_max(int x) {
  return lane63(wave_inclusive<int>(x, INT_MIN, [](int a, int b) { return max(a, b); }));
}
__device__ __forceinline__ int wave_or(int x) {
  return lane63(wave_inclusive<int>(x, 0, [](int a, int b) { return a | b; }));
}

// Exclusive prefix sum over the 64 lanes of one wave; *total gets the sum.
template <typename T>
__device__ __forceinline__ T wave_exclusive_scan(T x, T* total) {
  const T v = wave_inclusive<T>(x, T(0), AddOp{});
  *total = lane63(v);
  return v - x;
}

// Wave-aggregated counter update: every lane with `on` takes one slot of
// cnt[key] and gets its position.  Lanes are grouped into runs of
// neighbours with equal keys (neighbouring lanes visit neighbouring
// entries, which mostly share a key); the first lane of a run adds the
// run's length with one LDS atomic, and lane i of the run takes position
// old value + i.  Same-address atomics of one instruction are serialised,
// so this turns up to 64 of them into one.  Every lane of the wave takes
// part.
__device__ __forceinline__ int wave_reserve(int* cnt, int key, bool on) {
  const int lane = threadIdx.x & 63;
  const int prev_key = __shfl_up(key, 1, 64);
  const int prev_on = __shfl_up(on ? 1 : 0, 1, 64);
  const bool head = on && (lane == 0 || prev_on == 0 || prev_key != key);
  const unsigned long long heads = __ballot(head);
  const unsigned long long ends = heads | ~__ballot(on);  // a run stops at either
  const unsigned long long upto = (lane == 63) ? ~0ull : ((1ull << (lane + 1)) - 1ull);
  const unsigned long long after = ends & ~upto;
  const int next = after ? __builtin_ctzll(after) : 64;  // first lane past my run
  int base = 0;
  if (head) base = atomicAdd(&cnt[key], next - lane);
  const unsigned long long mine = heads & upto;
  const int first = (on && mine) ? 63 - __builtin_clzll(mine) : lane;  // my run's head
  base = __shfl(base, first, 64);
  return on ? base + (lane - first) : -1;
}

// x / d for d > 0; d is uniform and almost always a power of two (tile rows,
// key tile, split count 1), which then costs a shift instead of a division.
__device__ __forceinline__ int udiv(int x, int d) {
  return (d & (d - 1)) == 0 ? (int)((unsigned)x >> __builtin_ctz((unsigned)d)) : x / d;
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

// The six per-segment values the validation reads (the prefix form; the
// key-range form reads cu_q and used_q only).
struct SegLoad {
  int cq0, cq1, uq, ck0, ck1, uk;
};

__device__ __forceinline__ SegLoad load_segment(const PlanArgs& a, int s) {
  const Geometry& g = a.g;
  const bool kr = g.kr_off != nullptr;
  SegLoad L;
  L.cq0 = g.cu_q[s];
  L.cq1 = g.cu_q[s + 1];
  L.uq = g.used_q[s];
  L.ck0 = kr ? 0 : g.cu_k[s];
  L.ck1 = kr ? 0 : g.cu_k[s + 1];
  L.uk = kr ? 0 : g.used_k[s];
  return L;
}

// Validates segment s from its loaded values and returns its error bits (0:
// valid).  *uq and *uk get its used query rows and key count.
__device__ int segment_error(const PlanArgs& a, int s, const SegLoad& L, int* uq_out,
                             int* uk_out) {
  const Geometry& g = a.g;
  const bool kr = g.kr_off != nullptr;
  const int cq0 = L.cq0, cq1 = L.cq1, uq = L.uq;
  const int ck0 = L.ck0, ck1 = L.ck1, uk_p = L.uk;
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
__device__ __forceinline__ int find_segment(const int32_t* off, int nseg, int t) {
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
__device__ __forceinline__ int tile_key_tiles(const PlanArgs& a, const SegView& v, int s, int row0) {
  const int uq = v.uq[s];
  const int uk = v.uk[s];
  int kend = uk;
  if (a.g.causal) {
    const int r_last = min(row0 + a.rows, uq) - 1;
    kend = max(0, min(uk, r_last + uk - uq + 1));
  }
  return udiv(kend + a.key_tile - 1, a.key_tile);
}

// Work entry e (its segment s, first entry of s at e0): query tile
// (e - e0) / S and key chunk (e - e0) % S of the segment's S = split[s]
// chunks; the chunk covers key tiles [kt0, kt1) of that query tile.
__device__ __forceinline__ int4 make_entry(const PlanArgs& a, const SegView& v, int s, int e0, int e,
                                           int* cost) {
  const int S = v.split[s];
  const int local = e - e0;
  if (a.mode == 1) {
    // key tile of `rows` keys: the query rows that see any of its keys
    // start at r_first (bottom-right causal); its loop runs over (query
    // head, 32-row query tile), split into S chunks when S > 1 (chunk j of
    // key tile kt is entry e0 + kt * S + j, and e names its partial slot)
    const int kt = udiv(local, S), j = local - kt * S;
    const int uq = v.uq[s], uk = v.uk[s];
    const int k_row0 = kt * a.rows;
    const int r_first = a.g.causal ? max(0, min(uq, k_row0 + uq - uk)) : 0;
    const int n_it = (a.g.hq / a.g.hkv) * ((uq + 31) / 32 - r_first / 32);
    int it0 = 0, it1 = n_it;
    if (S > 1) {
      const int chunk = udiv(n_it + S - 1, S);
      it0 = min(j * chunk, n_it);
      it1 = min(it0 + chunk, n_it);
    }
    *cost = min(it1 - it0, kCostBuckets - 1);
    return make_int4(s, k_row0, r_first, (e << 5) | (j << 1) | (S > 1 ? 1 : 0));
  }
  const int qt = udiv(local, S), j = local - qt * S;
  const int row0 = qt * a.rows;
  const int nkt = tile_key_tiles(a, v, s, row0);
  const int chunk = udiv(nkt + S - 1, S);
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
  __shared__ int s_err;
  __shared__ int s_max_split;
  __shared__ int s_max_kt;
  __shared__ long long s_nq;
  const int tid = threadIdx.x;
  const int nseg = a.g.nseg;
  const bool in_lds = nseg <= kPlanLdsSegs;
  // Without split capacity every segment has one chunk per tile: the entry
  // offsets are the tile-count prefix sums of step 1 and step 2 is skipped.
  const bool direct = a.ws.splits == 1;
  const long long cap = (long long)a.max_tiles * a.ws.splits;

  // The first segment of each thread is loaded before the LDS set-up, so
  // that the set-up and its barrier overlap the memory latency.
  SegLoad first{};
  if (tid < nseg) first = load_segment(a, tid);

  for (int b = tid; b < kCostBuckets; b += kPlanThreads) hist[b] = 0;
  if (tid == 0) {
    s_err = 0;
    s_max_split = 1;
    s_max_kt = 0;
  }
  // Up to 64 segments, step 1 runs in wave 0 alone, which wrote the
  // scalars above itself; the histogram is first used after step 1's
  // barrier.  More segments: every wave updates the scalars in step 1.
  const bool one_wave = nseg <= 64;
  if (!one_wave) __syncthreads();

  // The steps below run with the per-segment tables either all in LDS or
  // all in the workspace; each form is compiled on its own, so that the LDS
  // form reads LDS directly (a pointer that may be either would make every
  // table read wait for all outstanding global stores as well).
  auto body = [&](const SegView v) __attribute__((always_inline)) {

  // 1. validation and query tiles per segment (an invalid segment: none).
  //    split holds the segment's tile count until step 2 (or 1 when direct).
  // Up to 64 segments: wave 0 alone, with a wave scan (no block barriers).
  long long n_qtiles = 0;
  for (int base = 0; base < nseg && (!one_wave || tid < 64); base += kPlanThreads) {
    const int s = base + tid;
    long long cnt = 0;
    int err = 0, kt_max = 0;
    if (s < nseg) {
      int uq, uk;
      err = segment_error(a, s, base == 0 ? first : load_segment(a, s), &uq, &uk);
      if (err) {
        uk = 0;
      } else {
        cnt = udiv((a.mode == 1 ? uk : uq) + a.rows - 1, a.rows);
        if (uq > 0) kt_max = udiv(uk + a.key_tile - 1, a.key_tile);
      }
      if (in_lds) {  // (the workspace form reads the argument arrays)
        l_uq[s] = uq;
        l_uk[s] = uk;
      }
      v.split[s] = direct ? 1 : (int32_t)cnt;
    }
    // one LDS atomic per wave (the lanes' own atomics would serialise)
    err = wave_or(err);
    kt_max = wave_max(kt_max);
    if ((tid & 63) == 0) {
      if (err) atomicOr(&s_err, err);
      if (kt_max > 0) atomicMax(&s_max_kt, kt_max);
    }
    long long tot;
    const long long excl = one_wave ? wave_exclusive_scan<long long>(cnt, &tot)
                                    : block_exclusive_scan<long long>(cnt, wsum64, &tot);
    if (direct && s < nseg) {
      const int32_t o = (int32_t)min(n_qtiles + excl, cap);
      v.off[s] = o;
    }
    n_qtiles += tot;
  }
  if (one_wave && tid == 0) s_nq = n_qtiles;
  __threadfence_block();
  __syncthreads();
  if (one_wave) n_qtiles = s_nq;

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
      int s_wave = 1;
      if (s < nseg) {
        const int qt = v.split[s];
        int S = 1;
        if (split_on && qt > 0) {
          if (a.mode == 0) {
            const int kt = udiv(v.uk[s] + a.key_tile - 1, a.key_tile);
            S = max(1, min(s_aim, kt / kMinSplitTiles));
          } else {  // chunks of at least kBwdMinChunk (head, query tile) steps
            const int steps = (a.g.hq / a.g.hkv) * ((v.uq[s] + 31) / 32);
            S = max(1, min(s_aim, steps / kBwdMinChunk));
          }
        }
        v.split[s] = S;
        cnt = (long long)qt * S;
        s_wave = S;
      }
      s_wave = wave_max(s_wave);
      if ((tid & 63) == 0 && s_wave > 1) atomicMax(&s_max_split, s_wave);
      long long tot;
      const long long excl = block_exclusive_scan<long long>(cnt, wsum64, &tot);
      if (s < nseg) {
        const int32_t o = (int32_t)min(carry + excl, cap);
        v.off[s] = o;
      }
      carry += tot;
    }
  }
  int n_tiles = (int)min(carry, cap);
  if (carry > cap) {
    n_tiles = 0;
    if (tid == 0) s_err |= GVATTN_DEVERR_OFFSETS;
  }
  if (tid == 0) v.off[nseg] = n_tiles;
  __threadfence_block();
  __syncthreads();

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
  // Each thread takes a contiguous run of entries, so that one segment
  // lookup serves all of them.
  const int per = (n_tiles + kPlanThreads - 1) / kPlanThreads;
  const int e_begin = min(tid * per, n_tiles);
  const int e_end = min(e_begin + per, n_tiles);
  // Step i of the walk visits entry e_begin + i of every thread (the same
  // trip count in every lane, so that the counter updates of a step can be
  // aggregated over the wave).  steps_c: a compile-time step count (the
  // loop unrolls and step i is a constant), or 0 for `per` steps.
  auto walk = [&](auto steps_c, auto&& visit) {
    constexpr int N = decltype(steps_c)::value;
    int s = 0, e0 = 0, e1 = 0;
    if (e_begin < e_end) {
      s = find_segment(v.off, nseg, e_begin);
      e0 = v.off[s];
      e1 = v.off[s + 1];
    }
    const int n = N > 0 ? N : per;
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const int t = e_begin + i;
      const bool on = i < per && t < e_end;
      int4 e = make_int4(0, 0, 0, 0);
      int key = 0;
      if (on) {
        while (t >= e1 && s + 1 < nseg) {  // segments without entries are passed over
          ++s;
          e0 = e1;
          e1 = v.off[s + 1];
        }
        int cost;
        e = make_entry(a, v, s, e0, t, &cost);
        key = sort_key(cost, s);
      }
      visit(i, e, key, on);
    }
  };
  // Up to four entries per thread, the scatter reuses the entries, keys and
  // in-bucket ranks of the histogram pass from registers.
  constexpr int kCached = 4;
  const bool cached = per <= kCached;
  int4 c_ent[kCached];
  int c_key[kCached], c_rank[kCached];
  bool c_on[kCached];
  if (cached) {
    walk(std::integral_constant<int, kCached>{}, [&](int i, const int4& e, int key, bool on) {
      c_ent[i] = e;
      c_key[i] = key;
      c_on[i] = on;
      c_rank[i] = wave_reserve(hist, key, on);
    });
  } else {
    walk(std::integral_constant<int, 0>{},
         [&](int, const int4&, int key, bool on) { wave_reserve(hist, key, on); });
  }
  __syncthreads();

  // bucket start positions, most expensive bucket first.  Forward keys
  // stay below n_keys; up to 512 buckets, wave 0 scans them alone (eight
  // per lane), else every thread takes two.
  const int n_keys =
      a.mode != 0 ? kCostBuckets
                  : (grouped ? kExactCost + ((max_kt >> kGroupShift) - (kExactCost >> kGroupShift) + 1) * nseg
                             : max_kt + 1);
  if (n_keys <= 512) {
    if (tid < 64) {
      int c[8], sum = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int b = n_keys - 1 - (8 * tid + j);
        c[j] = b >= 0 ? hist[b] : 0;
        sum += c[j];
      }
      int tot;
      int run = wave_exclusive_scan<int>(sum, &tot);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int b = n_keys - 1 - (8 * tid + j);
        if (b >= 0) hist[b] = run;
        run += c[j];
      }
    }
  } else {
    constexpr int kPer = kCostBuckets / kPlanThreads;  // buckets per thread
    static_assert(kCostBuckets == kPer * kPlanThreads, "buckets split evenly");
    int c[kPer], sum = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      c[j] = hist[kCostBuckets - 1 - (kPer * tid + j)];  // visited first: the highest
      sum += c[j];
    }
    int tot;
    int run = block_exclusive_scan<int>(sum, wsum, &tot);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      hist[kCostBuckets - 1 - (kPer * tid + j)] = run;
      run += c[j];
    }
  }
  __syncthreads();

  // 4. scatter (the header below takes nothing from it: no barrier).  The
  // positions are below n_tiles by construction; the checks keep every
  // store inside the list whatever the counts.
  if (cached) {  // hist holds the bucket starts now
#pragma unroll
    for (int i = 0; i < kCached; ++i)
      if (c_on[i]) {
        const int pos = hist[c_key[i]] + c_rank[i];
        if ((unsigned)pos < (unsigned)n_tiles) a.ws.tiles[pos] = c_ent[i];
      }
  } else {
    walk(std::integral_constant<int, 0>{}, [&](int, const int4& e, int key, bool on) {
      const int pos = wave_reserve(hist, key, on);
      if (on && (unsigned)pos < (unsigned)n_tiles) a.ws.tiles[pos] = e;
    });
  }

  if (tid == 0) {
    a.ws.header->n_tiles = n_tiles;
    a.ws.header->err = s_err;
    a.ws.header->key = a.key;
    a.ws.header->rows_per_tile = a.rows;
    a.ws.header->max_split = s_max_split;
  }
  // The LDS form's tables go to the workspace last (they are final since
  // step 2), with no barrier after them.
  if (in_lds) {
    for (int i = tid; i < nseg; i += kPlanThreads) {
      a.ws.seg_split[i] = v.split[i];
      a.ws.seg_tile_off[i] = v.off[i];
    }
    if (tid == 0) a.ws.seg_tile_off[nseg] = v.off[nseg];
  }
  };
  if (in_lds) {
    body(SegView{l_uq, l_uk, l_split, l_off});
  } else {
    body(SegView{a.g.used_q, a.g.kr_off != nullptr ? a.ws.seg_keys : a.g.used_k, a.ws.seg_split,
                 a.ws.seg_tile_off});
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  return launch_kernel(plan_kernel, dim3(1), dim3(kPlanThreads), s, a);
}

}  // namespace gvattn
