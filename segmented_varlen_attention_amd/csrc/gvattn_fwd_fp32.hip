// FP32 segmented varlen attention forward (SIMT).
//
// Same operation and conventions as the BF16 matrix-core path (PR #302,
// "What"; issue #18687, "actual behavior"; PR #312, "Problem and
// behavior"), for FP32 inputs and outputs.  One wave handles one
// (query row, head) at a time with the head dimension spread over its
// lanes; each key's score is reduced across the wave and folded into an
// online softmax in the exp2 domain.  This variant exists for FP32 callers
// and small problems; it does not use the matrix cores.
#include <math.h>

#include "gvattn_internal.h"

namespace gvattn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

template <int DQ, int DV>
__global__ __launch_bounds__(kThreads) void fwd_fp32_kernel(FwdArgs a, int rows_per_tile) {
  constexpr int E = DQ / 64;   // Q/K elements per lane
  constexpr int EV = DV / 64;  // V/O elements per lane
  const PlanHeader* hdr = a.ws.header;
  if (hdr->key != a.key) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(&a.ws.header->err, GVATTN_DEVERR_PLAN);
    return;
  }
  const int hq = a.g.hq;
  const int64_t n_work = (int64_t)hdr->n_tiles * hq;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = hq / a.g.hkv;
  const float c = a.scale_log2;
  const float* Q = static_cast<const float*>(a.q);
  const float* K = static_cast<const float*>(a.k);
  const float* V = static_cast<const float*>(a.v);
  float* O = static_cast<float*>(a.out);

  for (int64_t w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int t = (int)(w / hq);
    const int head = (int)(w - (int64_t)t * hq);
    const int kvh = head / G;
    const int4 tile = a.ws.tiles[t];  // never split: all key tiles
    const int seg = tile.x, row0 = tile.y;
    // keys: the used prefix at k0, or the segment's ranges concatenated
    const bool kr = a.g.kr_off != nullptr;
    const int q0 = a.g.cu_q[seg], k0 = kr ? 0 : a.g.cu_k[seg];
    const int uq = a.g.used_q[seg], uk = kr ? a.ws.seg_keys[seg] : a.g.used_k[seg];
    const int r_beg = kr ? a.g.kr_off[seg] : 0, r_end = kr ? a.g.kr_off[seg + 1] : 1;
    for (int row = row0 + wave; row < min(row0 + rows_per_tile, uq); row += kThreads / 64) {
      const int64_t qoff = ((int64_t)(q0 + row) * hq + head) * DQ;
      const int64_t ooff = ((int64_t)(q0 + row) * hq + head) * DV;
      float qv[E], ov[EV];
#pragma unroll
      for (int e = 0; e < E; ++e) qv[e] = Q[qoff + lane + 64 * e];
#pragma unroll
      for (int e = 0; e < EV; ++e) ov[e] = 0.f;
      const int lim = a.g.causal ? max(0, min(uk, row + uk - uq + 1)) : uk;
      float m = -INFINITY, l = 0.f;
      for (int ri = r_beg, pos = 0; ri < r_end && pos < lim; ++ri) {
        const int first = kr ? a.g.kr_start[ri] : k0;
        const int len = kr ? a.g.kr_len[ri] : uk;
        const int n = min(len, lim - pos);
        for (int j = 0; j < n; ++j) {
          const int64_t koff = ((int64_t)(first + j) * a.g.hkv + kvh) * DQ;
          const int64_t voff = ((int64_t)(first + j) * a.g.hkv + kvh) * DV;
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) part = __builtin_fmaf(qv[e], K[koff + lane + 64 * e], part);
          const float sc = wave_sum(part) * c;
          const float m_new = fmaxf(m, sc);
          const float alpha = __builtin_amdgcn_exp2f(m - m_new);
          const float p = __builtin_amdgcn_exp2f(sc - m_new);
          l = l * alpha + p;
#pragma unroll
          for (int e = 0; e < EV; ++e) ov[e] = __builtin_fmaf(p, V[voff + lane + 64 * e], ov[e] * alpha);
          m = m_new;
        }
        pos += len;
      }
      const bool dead = (lim == 0);
      const float inv = dead ? 0.f : 1.f / l;
#pragma unroll
      for (int e = 0; e < EV; ++e) O[ooff + lane + 64 * e] = dead ? 0.f : ov[e] * inv;
      if (lane == 0)
        a.lse[(int64_t)head * a.g.total_q + q0 + row] =
            dead ? -INFINITY : (m + log2f(l)) * 0.69314718055994530942f;
    }
  }
}

template <int DQ, int DV>
hipError_t launch_d(const FwdArgs& a, const TileShape& t, int64_t max_work, hipStream_t s) {
  auto kern = fwd_fp32_kernel<DQ, DV>;
  const int grid = persistent_grid(reinterpret_cast<const void*>(kern), kThreads, max_work);
  if (grid <= 0) return hipSuccess;
  return launch_kernel(kern, dim3(grid), dim3(kThreads), s, a, t.rows);
}

template <int DQ>
hipError_t launch_dq(const FwdArgs& a, const TileShape& t, int64_t max_work, hipStream_t s,
                     bool* supported) {
  switch (a.g.dv) {
    case 64: return launch_d<DQ, 64>(a, t, max_work, s);
    case 128: return launch_d<DQ, 128>(a, t, max_work, s);
    case 256: return launch_d<DQ, 256>(a, t, max_work, s);
    default: *supported = false; return hipSuccess;
  }
}

}  // namespace

hipError_t launch_fwd_fp32(const FwdArgs& a, const TileShape& t, int64_t max_work,
                           hipStream_t s, bool* supported) {
  *supported = true;
  switch (a.g.d) {
    case 64: return launch_dq<64>(a, t, max_work, s, supported);
    case 128: return launch_dq<128>(a, t, max_work, s, supported);
    case 256: return launch_dq<256>(a, t, max_work, s, supported);
    default: *supported = false; return hipSuccess;
  }
}

}  // namespace gvattn
