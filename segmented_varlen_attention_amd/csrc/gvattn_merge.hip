// FP32 LSE merge of partial attention results over key partitions
// (cosmos-framework PR #312, "Problem and behavior": visibility partitions
// are computed separately and combined by an FP32 LSE merge).
//
// For each used row and head, in FP32:
//   m = max_p LSE_p;  m = -inf -> O = 0, LSE = -inf;
//   else w_p = exp(LSE_p - m), W = sum_p w_p, LSE = m + ln W,
//        O = sum_p (w_p / W) O_p.
// The kernel is HBM-bound: D/32 lanes own one (row, head), 32 elements each,
// moved with 16-byte vector loads/stores; the per-row work (segment lookup,
// LSE loads, weights) is shared by few lanes.  With two partials (the
// common case) every load of the lane is issued before the dependent
// segment and LSE reads.  Pairs are taken in row-major
// order (all heads of a row, then the next row), which is the memory order
// of O, so a block streams one contiguous piece of every partial and of the
// output.
// Gap rows are skipped (left untouched).  Each (row, head) is fully read before it is
// written by the same lanes, so `out` may alias part_out[0].
#include <math.h>

#include "gvattn_internal.h"

namespace gvattn {
namespace {

using namespace dev;

constexpr int kThreads = 256;
// LSE merge: elements of one (row, head) per lane, held in runs of 8 spread
// over the row so that each 16-byte load instruction of the D/kMergeElems
// lanes of a pair reads one contiguous piece of it
constexpr int kMergeElems = 16;

// 8 elements of type T: 16-byte loads into raw registers, unpacking to
// FP32, and packing / storing FP32 back as T (round to nearest even).  The
// stores are non-temporal: nothing here reads the output again, and
// streaming it past the L2 leaves more of it for the partials' reads.
template <typename T> struct Vec8;
template <> struct Vec8<__bf16> {
  static constexpr int kRaw = 1;  // 16-byte registers per 8 elements
  static __device__ __forceinline__ void unpack(const u32x4* r, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __builtin_bit_cast(float, r[0][i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, r[0][i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(void* p, const float* f) {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (__bf16)f[i];
    __builtin_nontemporal_store(o, reinterpret_cast<bf16x8*>(p));
  }
};
template <> struct Vec8<_Float16> {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  static constexpr int kRaw = 1;
  static __device__ __forceinline__ void unpack(const u32x4* r, float* f) {
    const f16x8 v = __builtin_bit_cast(f16x8, r[0]);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
  }
  static __device__ __forceinline__ void store(void* p, const float* f) {
    f16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (_Float16)f[i];
    __builtin_nontemporal_store(o, reinterpret_cast<f16x8*>(p));
  }
};
template <> struct Vec8<float> {
  static constexpr int kRaw = 2;
  static __device__ __forceinline__ void unpack(const u32x4* r, float* f) {
    // whole-vector casts: a bit cast of one element of a vector lvalue
    // (r[0][i]) compiles to a read of element 0
    const f32x4 a = __builtin_bit_cast(f32x4, r[0]);
    const f32x4 b = __builtin_bit_cast(f32x4, r[1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = a[i];
      f[4 + i] = b[i];
    }
  }
  static __device__ __forceinline__ void store(void* p, const float* f) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = f[i];
      b[i] = f[4 + i];
    }
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p) + 1);
  }
};

// E elements of one lane, in runs of 8 contiguous elements STRIDE elements
// apart, as raw 16-byte registers; and the store of such runs.
template <typename T, int E, int STRIDE>
struct LaneRaw {
  static constexpr int RUNS = E / 8;
  static constexpr int K = Vec8<T>::kRaw;
  u32x4 r[RUNS * K];
  __device__ __forceinline__ void load(const T* src) {
#pragma unroll
    for (int j = 0; j < RUNS; ++j)
#pragma unroll
      for (int k = 0; k < K; ++k) r[j * K + k] = reinterpret_cast<const u32x4*>(src + j * STRIDE)[k];
  }
  __device__ __forceinline__ void unpack(float* f) const {
#pragma unroll
    for (int j = 0; j < RUNS; ++j) Vec8<T>::unpack(r + j * K, f + 8 * j);
  }
};

template <typename T, int E, int STRIDE>
__device__ __forceinline__ void store_runs(T* dst, const float* f) {
#pragma unroll
  for (int j = 0; j < E / 8; ++j) Vec8<T>::store(dst + j * STRIDE, f + 8 * j);
}

// Largest s in [0, nseg) with cu[s] <= row (cu assumed non-decreasing;
// callers re-check membership).
__device__ __forceinline__ int find_segment(const int32_t* cu, int nseg, int row) {
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= row) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Merges the pair first + slot (its D/32 lanes; this lane holds part `sub`).
// NP > 0: exactly NP partials, whose loads are all issued before the row's
// segment and LSEs are looked up, so that they overlap those dependent
// reads; NP == 0: any count, one partial at a time.
template <typename TIn, typename TOut, int D, int NP>
__device__ __forceinline__ void merge_pair(const MergeArgs& a, int64_t first, int slot, int sub,
                                            int64_t npairs) {
  if (first + slot >= npairs) return;
  const int64_t row_first = first / a.hq;  // uniform
  const int t = (int)(first - row_first * a.hq) + slot;
  const int row = (int)(row_first + t / a.hq);
  const int head = t % a.hq;
  constexpr int E = kMergeElems, RS = D * 8 / E;  // run stride
  const int64_t eoff = ((int64_t)row * a.hq + head) * D + sub * 8;

  // row < total_q: every partial holds the row, used or not
  LaneRaw<TIn, E, RS> raw[NP > 0 ? NP : 1];
  if constexpr (NP > 0) {
#pragma unroll
    for (int p = 0; p < NP; ++p) raw[p].load(static_cast<const TIn*>(a.part_out[p]) + eoff);
  }
  {
    const int s = find_segment(a.cu_q, a.nseg, row);
    const int c0 = a.cu_q[s], c1 = a.cu_q[s + 1], us = a.used_q[s];
    if (c0 < 0 || c1 < c0 || c1 > a.total_q || us < 0 || us > c1 - c0) return;
    if (row < c0 || row >= c0 + us) return;  // gap row: untouched
  }

  const int64_t lidx = (int64_t)head * a.total_q + row;
  const int np = NP > 0 ? NP : a.nparts;
  float lp[NP > 0 ? NP : 1];
  float m = -INFINITY;
  bool nan = false;
  if constexpr (NP > 0) {
#pragma unroll
    for (int p = 0; p < NP; ++p) lp[p] = a.part_lse[p][lidx];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      nan |= (lp[p] != lp[p]);
      m = fmaxf(m, lp[p]);
    }
  } else {
    for (int p = 0; p < np; ++p) {
      const float L = a.part_lse[p][lidx];
      nan |= (L != L);
      m = fmaxf(m, L);
    }
  }
  float acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.f;
  float lse_out;
  if (nan) {
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] = NAN;
    lse_out = NAN;
  } else if (m == -INFINITY) {
    lse_out = -INFINITY;
  } else {
    constexpr float kLog2e = 1.4426950408889634f;
    float wsum = 0.f;
    auto add = [&](float L, const LaneRaw<TIn, E, RS>& r) {
      const float w = __builtin_amdgcn_exp2f((L - m) * kLog2e);
      float f[E];
      r.unpack(f);
      wsum += w;
#pragma unroll
      for (int i = 0; i < E; ++i) acc[i] = __builtin_fmaf(w, f[i], acc[i]);
    };
    if constexpr (NP > 0) {
#pragma unroll
      for (int p = 0; p < NP; ++p) add(lp[p], raw[p]);
    } else {
      for (int p = 0; p < np; ++p) {
        raw[0].load(static_cast<const TIn*>(a.part_out[p]) + eoff);
        add(a.part_lse[p][lidx], raw[0]);
      }
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] *= inv;
    lse_out = m + logf(wsum);
  }
  store_runs<TOut, E, RS>(static_cast<TOut*>(a.out) + eoff, acc);
  if (sub == 0) a.lse[lidx] = lse_out;
}

template <typename TIn, typename TOut, int D, int NP>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  constexpr int LPP = D / kMergeElems;     // lanes per (row, head)
  constexpr int PPB = kThreads / LPP;      // pairs per block
  const int sub = threadIdx.x % LPP;
  const int slot = threadIdx.x / LPP;
  const int64_t npairs = (int64_t)a.hq * a.total_q;

  // segment validation (block 0): report, the per-row checks below skip
  if (blockIdx.x == 0 && a.err != nullptr) {
    for (int s = threadIdx.x; s < a.nseg; s += kThreads) {
      const int c0 = a.cu_q[s], c1 = a.cu_q[s + 1], u = a.used_q[s];
      int e = 0;
      if (c0 < 0 || c1 < c0 || c1 > a.total_q) e |= GVATTN_DEVERR_OFFSETS;
      else if (u < 0 || u > c1 - c0) e |= GVATTN_DEVERR_USED_Q;
      if (e) atomicOr(a.err, e);
    }
  }

  // pair = row * hq + head: the block's pairs are contiguous in O
  merge_pair<TIn, TOut, D, NP>(a, (int64_t)blockIdx.x * PPB, slot, sub, npairs);
}

template <typename TIn, typename TOut, int D>
hipError_t launch_np(const MergeArgs& a, int grid, hipStream_t s) {
  if (a.nparts == 2)
    return launch_kernel(merge_kernel<TIn, TOut, D, 2>, dim3(grid), dim3(kThreads), s, a);
  return launch_kernel(merge_kernel<TIn, TOut, D, 0>, dim3(grid), dim3(kThreads), s, a);
}

template <typename TIn, typename TOut>
hipError_t launch_t(const MergeArgs& a, hipStream_t s, bool* ok) {
  if (a.d != 64 && a.d != 128 && a.d != 256) {
    *ok = false;
    return hipSuccess;
  }
  *ok = true;
  const int per_block = kThreads / (a.d / kMergeElems);
  const int64_t blocks = ((int64_t)a.hq * a.total_q + per_block - 1) / per_block;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int grid = (int)blocks;
  switch (a.d) {
    case 64: return launch_np<TIn, TOut, 64>(a, grid, s);
    case 128: return launch_np<TIn, TOut, 128>(a, grid, s);
    default: return launch_np<TIn, TOut, 256>(a, grid, s);
  }
}

// Split-K merge over the plan's entries.  A block takes RPB rows of one
// head of a split query tile (the entry of the tile's chunk 0) and combines
// the chunks' FP32 partials of those rows (O over the chunk, LSE of the
// chunk) as the LSE merge combines partitions.  The entry names the rows,
// so there is no segment lookup and no gap row.  Each lane holds 8
// elements of a row; the loads of all chunks go out together (every chunk's
// LSE at once, the partial rows four chunks at a time; chunks past S read
// chunk S - 1 again and are left out) and the sums run in chunk order.
template <typename TOut, int D>
__global__ __launch_bounds__(kThreads) void split_merge_kernel(FwdArgs a) {
  constexpr int LPR = D / 8;           // lanes per row
  constexpr int RPB = kThreads / LPR;  // rows per block
  const PlanHeader* hdr = a.ws.header;
  if (hdr->key != a.key || hdr->n_tiles == 0 || hdr->max_split <= 1) return;
  const int hq = a.g.hq, total_q = a.g.total_q;
  const int rows = hdr->rows_per_tile;
  const int nsub = (rows + RPB - 1) / RPB;
  const int64_t n_units = (int64_t)hdr->n_tiles * hq * nsub;
  const int lr = threadIdx.x / LPR, c = (threadIdx.x % LPR) * 8;
  for (int64_t v = blockIdx.x; v < n_units; v += gridDim.x) {
    const int sub = (int)(v % nsub);
    const int64_t th = v / nsub;
    const int head = (int)(th % hq);
    const int t = (int)(th / hq);
    const int4 tile = a.ws.tiles[t];
    if (!(tile.w & 1) || ((tile.w >> 1) & 15) != 0) continue;  // chunk 0 of a split tile
    const int seg = tile.x;
    const int rl = sub * RPB + lr;  // row within the tile
    const int r = tile.y + rl;      // row within the segment
    if (rl >= rows || r >= a.g.used_q[seg]) continue;
    const int S = max(1, min(a.ws.seg_split[seg], kMaxSplits));
    const int64_t grow = (int64_t)a.g.cu_q[seg] + r;

    float L[kMaxSplits];
#pragma unroll
    for (int j = 0; j < kMaxSplits; ++j)
      L[j] = a.ws.part_lse[((int64_t)min(j, S - 1) * hq + head) * total_q + grow];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxSplits; ++j)
      if (j < S) m = fmaxf(m, L[j]);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    float lse_out = -INFINITY;
    if (m != -INFINITY) {
      constexpr float kLog2e = 1.4426950408889634f;
      constexpr int kBatch = 4;
      float wsum = 0.f;
#pragma unroll
      for (int j0 = 0; j0 < kMaxSplits; j0 += kBatch) {
        if (j0 < S) {
          LaneRaw<float, 8, 8> raw[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u)
            raw[u].load(a.ws.part_o + (((int64_t)min(j0 + u, S - 1) * total_q + grow) * hq + head) * D + c);
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            if (j0 + u < S) {
              const float w = __builtin_amdgcn_exp2f((L[j0 + u] - m) * kLog2e);
              float f[8];
              raw[u].unpack(f);
              wsum += w;
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(w, f[i], acc[i]);
            }
          }
        }
      }
      const float inv = 1.f / wsum;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= inv;
      lse_out = m + logf(wsum);
    }
    Vec8<TOut>::store(static_cast<TOut*>(a.out) + (grow * hq + head) * D + c, acc);
    if (c == 0) a.lse[(int64_t)head * total_q + grow] = lse_out;
  }
}

template <typename TOut>
hipError_t launch_split_t(const FwdArgs& a, hipStream_t s) {
  // one unit per (entry, head, block of rows), counted on the device; the
  // blocks stride over them (units of entries that are not a split tile's
  // chunk 0 are passed over)
  const dim3 grid(8192), block(kThreads);
  switch (a.g.dv) {
    case 64: return launch_kernel(split_merge_kernel<TOut, 64>, grid, block, s, a);
    case 128: return launch_kernel(split_merge_kernel<TOut, 128>, grid, block, s, a);
    case 256: return launch_kernel(split_merge_kernel<TOut, 256>, grid, block, s, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int part_dtype, int out_dtype, hipStream_t s,
                        bool* supported) {
  switch (part_dtype * 3 + out_dtype) {
    case GVATTN_BF16 * 3 + GVATTN_BF16: return launch_t<__bf16, __bf16>(a, s, supported);
    case GVATTN_BF16 * 3 + GVATTN_FP16: return launch_t<__bf16, _Float16>(a, s, supported);
    case GVATTN_BF16 * 3 + GVATTN_FP32: return launch_t<__bf16, float>(a, s, supported);
    case GVATTN_FP16 * 3 + GVATTN_BF16: return launch_t<_Float16, __bf16>(a, s, supported);
    case GVATTN_FP16 * 3 + GVATTN_FP16: return launch_t<_Float16, _Float16>(a, s, supported);
    case GVATTN_FP16 * 3 + GVATTN_FP32: return launch_t<_Float16, float>(a, s, supported);
    case GVATTN_FP32 * 3 + GVATTN_BF16: return launch_t<float, __bf16>(a, s, supported);
    case GVATTN_FP32 * 3 + GVATTN_FP16: return launch_t<float, _Float16>(a, s, supported);
    case GVATTN_FP32 * 3 + GVATTN_FP32: return launch_t<float, float>(a, s, supported);
    default: break;
  }
  *supported = false;
  return hipSuccess;
}

hipError_t launch_split_merge(const FwdArgs& a, int dtype, hipStream_t s) {
  if (dtype == GVATTN_BF16) return launch_split_t<__bf16>(a, s);
  if (dtype == GVATTN_FP16) return launch_split_t<_Float16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace gvattn
