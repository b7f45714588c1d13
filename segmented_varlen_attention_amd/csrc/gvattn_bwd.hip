// BF16 / FP16 gradients of the segmented varlen attention forward on gfx950
// matrix cores.
//
// The pages' path is forward-only (cosmos-framework PR #302, review: the
// backward raises).  These kernels compute the plain calculus of the
// forward they define (PR #302, "What": used prefixes, untouched gap rows;
// PR #312, "Problem and behavior": GQA folding, FP32 LSE).  With
// P = exp(scale * Q K^T - LSE) taken from the forward's LSE:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
// the query heads of a KV group adding into one dK / dV.
//
// Two kernels, no atomics, deterministic:
//   * dQ: one work item = (query tile, chunk of GF query heads of one KV
//     group), the forward's plan and static schedule.  A wave owns 32 query
//     rows of one head with Q and dO in registers; K / V tiles of 32 keys
//     move HBM -> LDS by buffer_load ... lds, double-buffered.  S^T = K Q^T
//     and dP^T = V dO^T on the matrix cores leave one query row per lane
//     column, so dS^T is formed in registers and dQ^T += K^T dS^T takes it
//     as the B operand, K^T read transposed (ds_read_b64_tr_b16) from the
//     row-major K tile.  The kernel also forms D from O and dO and writes
//     (LSE * log2 e, D) per (head, row) for the second kernel.
//   * dK / dV: one work item = (64 keys of one segment, KV head) from a
//     key-tile plan.  The group's query heads and the query tiles that see
//     those keys stream through LDS (Q, dO and the row statistics).  Two
//     waves share each 32 keys: one holds K and computes S = Q K^T, P and
//     dV^T += dO^T P; the other holds V and computes dP = dO V^T, takes P
//     through LDS, forms dS and dK^T += Q^T dS.  Scores leave one key per
//     lane column, so P and dS are the B operands straight from registers,
//     and Q^T, dO^T are read transposed from the row-major tiles.
// Offsets that must be bounds-checked go in the per-lane offset operand of
// the buffer instructions: loads past a segment's used rows or keys return
// zero and stores there are dropped, so gap rows of dQ, dK and dV are never
// written.  Rows past the used length and invisible keys are also masked
// explicitly, so no value read from outside the used rows can reach a sum.
#include <math.h>

#include <type_traits>

#include "gvattn_internal.h"
#include "gvattn_mfma.h"

namespace gvattn {
namespace {

using namespace dev;
using namespace mfma;

constexpr float kLog2e = 1.4426950408889634f;

template <int D, int DV>
struct BwdCfg {
  static constexpr int CHK = D / 8;    // 16-byte chunks per Q / K row
  static constexpr int CHV = DV / 8;   // 16-byte chunks per V / O / dO row
  static constexpr int KK = D / 16;    // MFMA k-steps over d
  static constexpr int KV = DV / 16;   // MFMA k-steps over d_v
  static constexpr int DBK = D / 32;   // 32-wide blocks of d
  static constexpr int DBV = DV / 32;  // 32-wide blocks of d_v
  static constexpr int KP = D + 8;     // staging row pitches (elements)
  static constexpr int VP = DV + 8;
};

// Static persistent schedule (the forward's): item w lives in queue w % 8
// at position w / 8, so with 8 head chunks or KV heads one XCD's L2 serves
// one KV head; the workgroups of a queue take its items in rounds, forward
// in even rounds and backward in odd ones (the plan sorts items by
// decreasing cost), and the wave priority rotates so that workgroups
// dispatched in later slots of a compute unit are not starved.
struct Schedule {
  int q, qi, n_q, n_slots, slot;
  __device__ __forceinline__ explicit Schedule(int n_cu) {
    q = blockIdx.x & 7;
    qi = blockIdx.x >> 3;
    n_q = ((int)gridDim.x - q + 7) >> 3;
    n_slots = min(4, ((int)gridDim.x + n_cu - 1) / n_cu);
    slot = (int)blockIdx.x / n_cu;
  }
  __device__ __forceinline__ int item(int r) const {
    const int j = r * n_q + ((r & 1) ? n_q - 1 - qi : qi);
    return j * 8 + q;
  }
  __device__ __forceinline__ void priority(int r) const {
    switch ((r + slot) % n_slots) {
      case 0: __builtin_amdgcn_s_setprio(0); break;
      case 1: __builtin_amdgcn_s_setprio(1); break;
      case 2: __builtin_amdgcn_s_setprio(2); break;
      default: __builtin_amdgcn_s_setprio(3); break;
    }
  }
};

template <int R>
struct RoleC {
  static constexpr int value = R;
};

__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, char* lds_dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 4, voff, 0, 0, 0);
}

// XOR swizzle of the 16-byte chunk index of a tile row (W 16-bit elements
// per row) for tiles read both ways: as rows (16 bytes per lane, 16
// consecutive rows at one logical chunk per clock) and transposed
// (ds_read_b64_tr_b16: 4 consecutive rows x 4 chunks per 32 lanes).  Rows
// need 16 distinct slots of the 256-byte bank window across 16 consecutive
// rows; transposed reads need the four rows of an aligned group of four in
// distinct 64-byte quarters of it.  At W = 128 the swizzle is a bijection
// of (row mod 16) whose bits 2-3 come from row bits 0-1; at W = 64 (two
// rows per window) the same holds for each row parity.
template <int W>
__device__ __forceinline__ int swz_kt(int row) {
  return (W == 64) ? ((((row >> 1) & 1) << 2) | ((row >> 2) & 3)) : (((row & 3) << 2) | ((row >> 2) & 3));
}

// 32 x 32 block of the A operand transposed: lane (r32, hh) receives
// column `col0 + r32` of rows {16 * a2 + 8 * (j / 4) + 4 * hh + j % 4}, j < 8,
// of a row-major tile with W 16-bit elements per row and swizzle swz_kt<W>.
template <int W, typename v8>
__device__ __forceinline__ v8 read_a_transposed(const char* tile, int a2, int col0, int trow,
                                                int tcol) {
  const int dcol = col0 + tcol;
  const int ch = dcol >> 3, within = (dcol & 7) * 2;
  const int r_lo = a2 * 16 + trow, r_hi = r_lo + 8;
  const i16x4 lo = read_tr(tile + r_lo * (W * 2) + ((ch ^ swz_kt<W>(r_lo)) << 4) + within);
  const i16x4 hi = read_tr(tile + r_hi * (W * 2) + ((ch ^ swz_kt<W>(r_hi)) << 4) + within);
  return __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row r32, k-step kk of a row-major tile with W elements per row, swizzle
// swz_kt<W>: the A operand of a product whose k index runs over the row.
template <int W, typename v8>
__device__ __forceinline__ v8 read_a_rows(const char* tile, int r32, int hh, int kk) {
  return *reinterpret_cast<const v8*>(tile + r32 * (W * 2) + (((2 * kk + hh) ^ swz_kt<W>(r32)) << 4));
}

// ---------------------------------------------------------------------------
// dQ (and the per-row statistics of the dK / dV kernel)
// ---------------------------------------------------------------------------
template <typename T, int D, int DV, int GF, int RB>
__global__ __launch_bounds__(64 * GF * RB, 2) void bwd_dq_kernel(BwdArgs a) {
  using C = BwdCfg<D, DV>;
  using E = Elem<T>;
  using v8 = typename E::v8;
  using v4 = typename E::v4;
  constexpr int NW = GF * RB;
  constexpr int K_TILE = 32 * D * 2, V_TILE = 32 * DV * 2;
  constexpr int STAGE = K_TILE + V_TILE;
  constexpr int DMA_K = K_TILE / 1024, DMA_V = V_TILE / 1024;
  constexpr int NDMA_K = (DMA_K + NW - 1) / NW, NDMA_V = (DMA_V + NW - 1) / NW;
  constexpr int S_BYTES = NW * 32 * C::KP * 2;
  constexpr int LDS_BYTES = (2 * STAGE > S_BYTES) ? 2 * STAGE : S_BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

  const PlanHeader* hdr = a.qws.header;
  if (hdr->key != a.qkey) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(&a.qws.header->err, GVATTN_DEVERR_PLAN);
    return;
  }
  const int n_hc = a.n_head_chunks;
  const int n_work = hdr->n_tiles * n_hc;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hh = lane >> 5;
  const int hf = wave % GF, rb = wave / GF;
  const int G = a.g.hq / a.g.hkv;
  const uint32_t qstride = (uint32_t)a.g.hq * D * 2;
  const uint32_t kstride = (uint32_t)a.g.hkv * D * 2;
  const uint32_t vstride = (uint32_t)a.g.hkv * DV * 2;
  const uint32_t ostride = (uint32_t)a.g.hq * DV * 2;
  const float c = a.scale_log2;

  // DMA slot s of a K (V) tile: row s / CHK (CHV), chunk (s % CH) ^ swizzle
  uint32_t koff[NDMA_K], voff[NDMA_V];
#pragma unroll
  for (int i = 0; i < NDMA_K; ++i) {
    const int s = (wave + i * NW) * 64 + lane;
    const int row = s / C::CHK, pc = s % C::CHK;
    koff[i] = (uint32_t)row * kstride + (uint32_t)((pc ^ swz_kt<D>(row)) * 16);
  }
#pragma unroll
  for (int i = 0; i < NDMA_V; ++i) {
    const int s = (wave + i * NW) * 64 + lane;
    const int row = s / C::CHV, pc = s % C::CHV;
    voff[i] = (uint32_t)row * vstride + (uint32_t)((pc ^ swz_kt<DV>(row)) * 16);
  }
  // transposed-read addressing (see read_a_transposed)
  const int il = lane & 15;
  const int trow = 4 * hh + (il >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (il & 3);

  const Schedule sch(a.n_cu);
  for (int r = 0;; ++r) {
    const int w = sch.item(r);
    if (w >= n_work) break;
    sch.priority(r);
    const int t = (int)((uint32_t)w / (uint32_t)n_hc);
    const int hc = w - t * n_hc;
    const int4 tile = a.qws.tiles[t];
    const int seg = __builtin_amdgcn_readfirstlane(tile.x);
    const int row0 = __builtin_amdgcn_readfirstlane(tile.y);
    const int head0 = hc * GF;
    const int head = head0 + hf;
    const int kvh = head0 / G;
    const int q0 = __builtin_amdgcn_readfirstlane(a.g.cu_q[seg]);
    const int uq = __builtin_amdgcn_readfirstlane(a.g.used_q[seg]);
    const int k0 = __builtin_amdgcn_readfirstlane(a.g.cu_k[seg]);
    const int uk = __builtin_amdgcn_readfirstlane(a.g.used_k[seg]);
    const int wr0 = row0 + rb * 32;
    const int r_last = min(row0 + 32 * RB, uq) - 1;
    int kend = uk;
    if (a.g.causal) kend = max(0, min(uk, r_last + uk - uq + 1));
    const int n_kt = (kend + 31) / 32;

    const uint32_t qbytes = uq > 0 ? (uint32_t)(uq - 1) * qstride + D * 2 : 0u;
    const uint32_t obytes = uq > 0 ? (uint32_t)(uq - 1) * ostride + DV * 2 : 0u;
    const auto qr = make_rsrc(static_cast<const T*>(a.q) + ((int64_t)q0 * a.g.hq + head) * D, qbytes);
    const auto dor = make_rsrc(static_cast<const T*>(a.dout) + ((int64_t)q0 * a.g.hq + head) * DV, obytes);
    const auto orr = make_rsrc(static_cast<const T*>(a.o) + ((int64_t)q0 * a.g.hq + head) * DV, obytes);
    const auto kr = make_rsrc(static_cast<const T*>(a.k) + ((int64_t)k0 * a.g.hkv + kvh) * D,
                              uk > 0 ? (uint32_t)(uk - 1) * kstride + D * 2 : 0u);
    const auto vr = make_rsrc(static_cast<const T*>(a.v) + ((int64_t)k0 * a.g.hkv + kvh) * DV,
                              uk > 0 ? (uint32_t)(uk - 1) * vstride + DV * 2 : 0u);

    // tile kt goes to stage `stage` (the parity of kt, a constant below)
    auto issue_tile = [&](int kt, int stage) {
      char* st = lds + stage * STAGE;
      const uint32_t ok = (uint32_t)kt * 32 * kstride, ov = (uint32_t)kt * 32 * vstride;
#pragma unroll
      for (int i = 0; i < NDMA_K; ++i) {
        const int inst = wave + i * NW;
        if (inst < DMA_K) dma16(kr, st + inst * 1024, koff[i] + ok, 0);
      }
#pragma unroll
      for (int i = 0; i < NDMA_V; ++i) {
        const int inst = wave + i * NW;
        if (inst < DMA_V) dma16(vr, st + K_TILE + inst * 1024, voff[i] + ov, 0);
      }
    };
    if (n_kt > 0) issue_tile(0, 0);

    // this lane's query row: Q and dO fragments, D = rowsum(dO * O)
    const int row = wr0 + r32;
    v8 qf[C::KK], df[C::KV];
    {
      const uint32_t roff = (uint32_t)row * qstride + hh * 16;
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk)
        qf[kk] = __builtin_bit_cast(v8, buf_load16(qr, roff + kk * 32));
    }
    float dsum = 0.f;
    {
      const uint32_t roff = (uint32_t)row * ostride + hh * 16;
#pragma unroll
      for (int kk = 0; kk < C::KV; ++kk) {
        df[kk] = __builtin_bit_cast(v8, buf_load16(dor, roff + kk * 32));
        const v8 of = __builtin_bit_cast(v8, buf_load16(orr, roff + kk * 32));
#pragma unroll
        for (int j = 0; j < 8; ++j) dsum = __builtin_fmaf((float)df[kk][j], (float)of[j], dsum);
      }
    }
    dsum = sum_across_halves(dsum);
    const bool used = row < uq;
    const float lse = used ? a.lse[(int64_t)head * a.g.total_q + q0 + row] : -INFINITY;
    // a row without keys (LSE -inf) or past the used rows: P = 0
    const float lse2 = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
    if (hh == 0 && used) {
      float2 st;
      st.x = lse2;
      st.y = dsum;
      reinterpret_cast<float2*>(a.stats)[(int64_t)head * a.g.total_q + q0 + row] = st;
    }

    f32x16 dq[C::DBK];
#pragma unroll
    for (int i = 0; i < C::DBK; ++i) dq[i] = f32x16{};
    const int lim = a.g.causal ? min(uk, row + uk - uq + 1) : uk;
    const int lim_w = a.g.causal ? min(uk, wr0 + uk - uq + 1) : uk;

    // One key tile in stage ST (the next one is loaded into 1 - ST).  The
    // loop is unrolled by two so that ST is a constant and the LDS operand
    // addresses are per-lane registers plus immediate offsets.
    auto tile_step = [&](int kt, auto stage_c) __attribute__((always_inline)) {
      const int ST = stage_c;
      wait_vmem();
      __syncthreads();
      if (kt + 1 < n_kt) issue_tile(kt + 1, 1 - ST);
      const char* Ks = lds + ST * STAGE;
      const char* Vs = Ks + K_TILE;

      // S^T = K Q^T and dP^T = V dO^T: lane (r32, hh) holds query row r32
      // and keys 8 * (v / 4) + 4 * hh + v % 4 of the tile
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) s = E::mfma(read_a_rows<D, v8>(Ks, r32, hh, kk), qf[kk], s);
#pragma unroll
      for (int kk = 0; kk < C::KV; ++kk) dp = E::mfma(read_a_rows<DV, v8>(Vs, r32, hh, kk), df[kk], dp);

      const int kbase = kt * 32;
      if (kbase + 32 > lim_w) {
        int nv = lim - kbase - 4 * hh;
        asm volatile("" : "+v"(nv));
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (8 * (v >> 2) + (v & 3) >= nv) s[v] = -INFINITY;
      }

      // dS^T = P^T * (dP^T - D) as 16-bit B operands
      v8 dsb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = exp2_fast(__builtin_fmaf(s[v], c, -lse2));
        dsb[v >> 3][v & 7] = (T)(p * (dp[v] - dsum));
      }

      // dQ^T += K^T dS^T
#pragma unroll
      for (int db = 0; db < C::DBK; ++db)
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2)
          dq[db] = E::mfma(read_a_transposed<D, v8>(Ks, a2, db * 32, trow, tcol), dsb[a2], dq[db]);
    };
    for (int kt = 0; kt < n_kt; kt += 2) {
      tile_step(kt, std::integral_constant<int, 0>{});
      if (kt + 1 < n_kt) tile_step(kt + 1, std::integral_constant<int, 1>{});
    }

    // epilogue: scale, stage through LDS, full-row stores of the used rows
    __syncthreads();
    T* Ss = reinterpret_cast<T*>(lds) + wave * 32 * C::KP;
#pragma unroll
    for (int db = 0; db < C::DBK; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        v4 ov;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) ov[cc] = (T)(dq[db][4 * a4 + cc] * a.scale);
        *reinterpret_cast<v4*>(Ss + r32 * C::KP + db * 32 + 8 * a4 + 4 * hh) = ov;
      }
    __syncthreads();
    {
      const auto dqr = make_rsrc(static_cast<T*>(a.dq) + ((int64_t)q0 * a.g.hq + head) * D, qbytes);
#pragma unroll
      for (int it = 0; it < D / 16; ++it) {
        const int idx = it * 64 + lane;
        const int rr = idx / C::CHK, ch = idx % C::CHK;
        const u32x4 val = *reinterpret_cast<const u32x4*>(Ss + rr * C::KP + 8 * ch);
        buf_store16_nt(dqr, (uint32_t)(wr0 + rr) * qstride + ch * 16, val);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
// One work item = 64 keys of one segment and KV head.  The 4 waves form two
// pairs, one pair per 32 keys.  In each pair the "P" wave (role 0) holds K
// and computes S = Q K^T, P and dV^T += dO^T P; the "dS" wave (role 1) holds
// V and computes dP = dO V^T, takes P from the P wave through LDS, forms
// dS = P * (dP - D) and dK^T += Q^T dS.  Each wave holds one fragment set
// and one accumulator set (two waves per SIMD; the kernel holding both took
// every register of one).
template <typename T, int D, int DV>
__global__ __launch_bounds__(256, 3) void bwd_dkv_kernel(BwdArgs a) {
  using C = BwdCfg<D, DV>;
  using E = Elem<T>;
  using v8 = typename E::v8;
  using v4 = typename E::v4;
  constexpr int NW = 4;
  constexpr int Q_TILE = 32 * D * 2, O_TILE = 32 * DV * 2, ST_TILE = 32 * 8;
  constexpr int STAGE = Q_TILE + O_TILE + ST_TILE;
  constexpr int NDMA_Q = Q_TILE / 1024 / NW, NDMA_O = O_TILE / 1024 / NW;
  static_assert(NDMA_Q * NW * 1024 == Q_TILE && NDMA_O * NW * 1024 == O_TILE, "DMA split");
  constexpr int P_BYTES = 64 * 16 * 4;  // one pair's P: 64 lanes x 16 floats
  constexpr int P_OFF = 2 * STAGE;
  constexpr int PMAX = C::KP > C::VP ? C::KP : C::VP;
  constexpr int S_BYTES = NW * 32 * PMAX * 2;
  constexpr int MAIN_BYTES = P_OFF + 2 * P_BYTES;
  constexpr int LDS_BYTES = (MAIN_BYTES > S_BYTES) ? MAIN_BYTES : S_BYTES;
  constexpr int NF = C::KK > C::KV ? C::KK : C::KV;       // fragment k-steps
  constexpr int NA = C::DBK > C::DBV ? C::DBK : C::DBV;   // accumulator blocks
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

  const PlanHeader* hdr = a.kws.header;
  if (hdr->key != a.kkey) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(&a.kws.header->err, GVATTN_DEVERR_PLAN);
    return;
  }
  const int hkv = a.g.hkv;
  const int n_work = hdr->n_tiles * hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave >> 1, role = wave & 1;
  const int r32 = lane & 31, hh = lane >> 5;
  const int G = a.g.hq / hkv;
  const uint32_t qstride = (uint32_t)a.g.hq * D * 2;
  const uint32_t kstride = (uint32_t)hkv * D * 2;
  const uint32_t vstride = (uint32_t)hkv * DV * 2;
  const uint32_t ostride = (uint32_t)a.g.hq * DV * 2;
  const float c = a.scale_log2;
  // P of the pair: float4 i of lane l at (i * 64 + l) * 16 bytes, so that
  // the 64 lanes of one access fill consecutive 16-byte slots
  float* Px = reinterpret_cast<float*>(lds + P_OFF + pair * P_BYTES) + lane * 4;

  uint32_t qoff[NDMA_Q], ooff[NDMA_O];
#pragma unroll
  for (int i = 0; i < NDMA_Q; ++i) {
    const int s = (wave + i * NW) * 64 + lane;
    const int row = s / C::CHK, pc = s % C::CHK;
    qoff[i] = (uint32_t)row * qstride + (uint32_t)((pc ^ swz_kt<D>(row)) * 16);
  }
#pragma unroll
  for (int i = 0; i < NDMA_O; ++i) {
    const int s = (wave + i * NW) * 64 + lane;
    const int row = s / C::CHV, pc = s % C::CHV;
    ooff[i] = (uint32_t)row * ostride + (uint32_t)((pc ^ swz_kt<DV>(row)) * 16);
  }
  const int il = lane & 15;
  const int trow = 4 * hh + (il >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (il & 3);

  const Schedule sch(a.n_cu);
  for (int r = 0;; ++r) {
    const int w = sch.item(r);
    if (w >= n_work) break;
    sch.priority(r);
    const int t = (int)((uint32_t)w / (uint32_t)hkv);
    const int kvh = w - t * hkv;
    const int4 tile = a.kws.tiles[t];
    const int seg = __builtin_amdgcn_readfirstlane(tile.x);
    const int k_row0 = __builtin_amdgcn_readfirstlane(tile.y);
    const int r_first = __builtin_amdgcn_readfirstlane(tile.z);
    const int q0 = __builtin_amdgcn_readfirstlane(a.g.cu_q[seg]);
    const int uq = __builtin_amdgcn_readfirstlane(a.g.used_q[seg]);
    const int k0 = __builtin_amdgcn_readfirstlane(a.g.cu_k[seg]);
    const int uk = __builtin_amdgcn_readfirstlane(a.g.used_k[seg]);
    const int wk0 = k_row0 + 32 * pair;  // this pair's first key
    const int key = wk0 + r32;           // this lane's key (column)
    const uint32_t kbytes = uk > 0 ? (uint32_t)(uk - 1) * kstride + D * 2 : 0u;
    const uint32_t vbytes = uk > 0 ? (uint32_t)(uk - 1) * vstride + DV * 2 : 0u;

    const int qt_first = r_first / 32;
    const int qt_end = (uq + 31) / 32;
    const int n_qt = qt_end - qt_first;
    // steps [it0, it0 + n_it) of the (query head, query tile) loop: all of
    // them, or chunk j of a split item, whose sums go to partial slot
    // `slot` (the reduce pass adds the chunks)
    const int wfield = __builtin_amdgcn_readfirstlane(tile.w);
    const bool partial = wfield & 1;
    const int slot = (int)((uint32_t)wfield >> 5);
    int it0 = 0, n_it = G * n_qt;
    if (partial) {
      const int n_all = n_it;
      const int S = __builtin_amdgcn_readfirstlane(a.kws.seg_split[seg]);
      const int chunk = (n_all + S - 1) / S;
      it0 = min(((wfield >> 1) & 15) * chunk, n_all);
      n_it = min(it0 + chunk, n_all) - it0;
    }
    const uint32_t qbytes = uq > 0 ? (uint32_t)(uq - 1) * qstride + D * 2 : 0u;
    const uint32_t obytes = uq > 0 ? (uint32_t)(uq - 1) * ostride + DV * 2 : 0u;
    // next (head, query tile) to load
    int ld_h = n_qt > 0 ? it0 / n_qt : 0;
    int ld_qt = qt_first + (it0 - ld_h * n_qt);
    const int qt_start = ld_qt;
    auto issue_next = [&](int stage) {
      const int head = kvh * G + ld_h;
      char* st = lds + stage * STAGE;
      const auto qrs = make_rsrc(static_cast<const T*>(a.q) + ((int64_t)q0 * a.g.hq + head) * D, qbytes);
      const auto ors = make_rsrc(static_cast<const T*>(a.dout) + ((int64_t)q0 * a.g.hq + head) * DV, obytes);
      const auto srs = make_rsrc(a.stats + ((int64_t)head * a.g.total_q + q0) * 2, (uint32_t)uq * 8u);
      const uint32_t oq = (uint32_t)ld_qt * 32 * qstride, oo = (uint32_t)ld_qt * 32 * ostride;
      // The row statistics first, with the lane index recomputed here (not
      // kept, where it was spilled): a wait for a spill reload after the tile
      // loads would also wait for those loads, one memory latency per step
      // for wave 0 and, through the barriers, for the workgroup.
      if (wave == 0) {
        // In asm so that it is not merged with the spilled copy of the index.
        uint32_t l;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
        dma4(srs, st + Q_TILE + O_TILE, (uint32_t)ld_qt * 256u + l * 4u);
      }
#pragma unroll
      for (int i = 0; i < NDMA_Q; ++i) dma16(qrs, st + (wave + i * NW) * 1024, qoff[i] + oq, 0);
#pragma unroll
      for (int i = 0; i < NDMA_O; ++i) dma16(ors, st + Q_TILE + (wave + i * NW) * 1024, ooff[i] + oo, 0);
      if (++ld_qt == qt_end) {
        ld_qt = qt_first;
        ++ld_h;
      }
    };
    if (n_it > 0) issue_next(0);

    // role 0: K fragments of this lane's key; role 1: V fragments
    v8 kvf[NF];
    {
      const auto kr = make_rsrc(static_cast<const T*>(a.k) + ((int64_t)k0 * hkv + kvh) * D, kbytes);
      const auto vr = make_rsrc(static_cast<const T*>(a.v) + ((int64_t)k0 * hkv + kvh) * DV, vbytes);
      if (role == 0) {
        const uint32_t ko = (uint32_t)key * kstride + hh * 16;
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) kvf[kk] = __builtin_bit_cast(v8, buf_load16(kr, ko + kk * 32));
      } else {
        const uint32_t vo = (uint32_t)key * vstride + hh * 16;
#pragma unroll
        for (int kk = 0; kk < C::KV; ++kk) kvf[kk] = __builtin_bit_cast(v8, buf_load16(vr, vo + kk * 32));
      }
    }
    f32x16 acc[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) acc[i] = f32x16{};

    // one copy of the loop per role, so that each is register-allocated on
    // its own
    auto iterate = [&](auto role_c) {
      constexpr int R = decltype(role_c)::value;
      int qt = qt_start;
      for (int it = 0; it < n_it; ++it) {
        wait_vmem();
        __syncthreads();
        if (it + 1 < n_it) issue_next((it + 1) & 1);
        const char* Qs = lds + (it & 1) * STAGE;
        const char* Os = Qs + Q_TILE;
        const float* Ss = reinterpret_cast<const float*>(Os + O_TILE);
        const int qt0 = qt * 32;
        if (++qt == qt_end) qt = qt_first;
        // no key of this pair is used, or no row of the tile sees any of them
        const bool skip = wk0 >= uk || (a.g.causal && qt0 + 31 < wk0 + uq - uk);
        // masked: key past the used keys, row past the used rows, or (causal)
        // key after the row's last visible key
        const bool edge = wk0 + 32 > uk || qt0 + 32 > uq || (a.g.causal && wk0 + 31 > qt0 + uk - uq);

        // lane (r32, hh) holds key `key` and query rows
        // qt0 + 8 * (v / 4) + 4 * hh + v % 4 of the tile
        v8 opb[2];
        if (!skip) {
          if constexpr (R == 0) {
            f32x16 s = f32x16{};
  #pragma unroll
            for (int kk = 0; kk < C::KK; ++kk) s = E::mfma(read_a_rows<D, v8>(Qs, r32, hh, kk), kvf[kk], s);
  #pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
              const f32x4 x0 = *reinterpret_cast<const f32x4*>(Ss + 2 * (8 * a4 + 4 * hh));
              const f32x4 x1 = *reinterpret_cast<const f32x4*>(Ss + 2 * (8 * a4 + 4 * hh) + 4);
              s[4 * a4 + 0] = exp2_fast(__builtin_fmaf(s[4 * a4 + 0], c, -x0[0]));
              s[4 * a4 + 1] = exp2_fast(__builtin_fmaf(s[4 * a4 + 1], c, -x0[2]));
              s[4 * a4 + 2] = exp2_fast(__builtin_fmaf(s[4 * a4 + 2], c, -x1[0]));
              s[4 * a4 + 3] = exp2_fast(__builtin_fmaf(s[4 * a4 + 3], c, -x1[2]));
            }
            if (edge) {
              int lo = a.g.causal ? key - uk + uq - qt0 - 4 * hh : -64;
              int hi = (key < uk) ? uq - qt0 - 4 * hh : -64;
              asm volatile("" : "+v"(lo), "+v"(hi));
  #pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int cv = 8 * (v >> 2) + (v & 3);
                if (cv < lo || cv >= hi) s[v] = 0.f;
              }
            }
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              f32x4 x;
  #pragma unroll
              for (int j = 0; j < 4; ++j) x[j] = s[4 * i + j];
              *reinterpret_cast<f32x4*>(Px + 256 * i) = x;
            }
  #pragma unroll
            for (int v = 0; v < 16; ++v) opb[v >> 3][v & 7] = (T)s[v];
          } else {
            f32x16 dp = f32x16{};
  #pragma unroll
            for (int kk = 0; kk < C::KV; ++kk) dp = E::mfma(read_a_rows<DV, v8>(Os, r32, hh, kk), kvf[kk], dp);
  #pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
              const f32x4 x0 = *reinterpret_cast<const f32x4*>(Ss + 2 * (8 * a4 + 4 * hh));
              const f32x4 x1 = *reinterpret_cast<const f32x4*>(Ss + 2 * (8 * a4 + 4 * hh) + 4);
              dp[4 * a4 + 0] -= x0[1];
              dp[4 * a4 + 1] -= x0[3];
              dp[4 * a4 + 2] -= x1[1];
              dp[4 * a4 + 3] -= x1[3];
            }
            __syncthreads();  // P of this tile is in LDS
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x4 x = *reinterpret_cast<const f32x4*>(Px + 256 * i);
  #pragma unroll
              for (int j = 0; j < 4; ++j) dp[4 * i + j] *= x[j];
            }
            if (edge) {
              int lo = a.g.causal ? key - uk + uq - qt0 - 4 * hh : -64;
              int hi = (key < uk) ? uq - qt0 - 4 * hh : -64;
              asm volatile("" : "+v"(lo), "+v"(hi));
  #pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int cv = 8 * (v >> 2) + (v & 3);
                if (cv < lo || cv >= hi) dp[v] = 0.f;
              }
            }
  #pragma unroll
            for (int v = 0; v < 16; ++v) opb[v >> 3][v & 7] = (T)dp[v];
          }
        }
        if (R == 0 || skip) __syncthreads();  // pairs with the dS wave's wait
        // a skipped tile adds zero products: the accumulators then stay in
        // place instead of being merged from two paths
        if (skip) opb[0] = opb[1] = v8{};

        // role 0: dV^T += dO^T P;  role 1: dK^T += Q^T dS
        if constexpr (R == 0) {
  #pragma unroll
          for (int db = 0; db < C::DBV; ++db)
  #pragma unroll
            for (int a2 = 0; a2 < 2; ++a2)
              acc[db] = E::mfma(read_a_transposed<DV, v8>(Os, a2, db * 32, trow, tcol), opb[a2], acc[db]);
        } else {
  #pragma unroll
          for (int db = 0; db < C::DBK; ++db)
  #pragma unroll
            for (int a2 = 0; a2 < 2; ++a2)
              acc[db] = E::mfma(read_a_transposed<D, v8>(Qs, a2, db * 32, trow, tcol), opb[a2], acc[db]);
        }
      }
    };
    if (role == 0) iterate(RoleC<0>{});
    else iterate(RoleC<1>{});

    if (partial) {
      // FP32 sums of this chunk: [64 keys][d + d_v] per (slot, KV head),
      // dK (unscaled) in columns [0, d), dV in [d, d + d_v)
      float* pp = a.kpart + ((int64_t)slot * hkv + kvh) * (kBwdKeyRows * (D + DV)) +
                  (pair * 32 + r32) * (D + DV) + (role == 0 ? D : 0);
      const int width = role == 0 ? DV : D;
#pragma unroll
      for (int db = 0; db < NA; ++db)
        if (db * 32 < width)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            f32x4 x;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) x[cc] = acc[db][4 * a4 + cc];
            *reinterpret_cast<f32x4*>(pp + db * 32 + 8 * a4 + 4 * hh) = x;
          }
      __syncthreads();  // the next item's loads reuse the stages
      continue;
    }

    // epilogue: role 0 writes dV, role 1 writes dK (scaled), rows of used
    // keys, staged through LDS
    T* Ws = reinterpret_cast<T*>(lds) + wave * 32 * PMAX;
    __syncthreads();
    const int width = role == 0 ? DV : D;
    const float f = role == 0 ? 1.f : a.scale;
#pragma unroll
    for (int db = 0; db < NA; ++db)
      if (db * 32 < width)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          v4 ov;
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) ov[cc] = (T)(acc[db][4 * a4 + cc] * f);
          *reinterpret_cast<v4*>(Ws + r32 * PMAX + db * 32 + 8 * a4 + 4 * hh) = ov;
        }
    __syncthreads();
    {
      const uint32_t stride = role == 0 ? vstride : kstride;
      const auto orr = (role == 0)
          ? make_rsrc(static_cast<T*>(a.dv) + ((int64_t)k0 * hkv + kvh) * DV, vbytes)
          : make_rsrc(static_cast<T*>(a.dk) + ((int64_t)k0 * hkv + kvh) * D, kbytes);
      const int ch_row = width / 8;
#pragma unroll
      for (int it = 0; it < (D > DV ? D : DV) / 16; ++it) {
        const int idx = it * 64 + lane;
        const int rr = idx / ch_row, ch = idx % ch_row;
        if (rr < 32) {
          const u32x4 val = *reinterpret_cast<const u32x4*>(Ws + rr * PMAX + 8 * ch);
          buf_store16_nt(orr, (uint32_t)(wk0 + rr) * stride + ch * 16, val);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// dK / dV of split items: sum of the chunks' FP32 partials
// ---------------------------------------------------------------------------
// A block takes one slab of kRedRows key rows of a split item; each of its
// threads issues the loads of all S partials of a 16-byte column before
// adding them, in chunk order, so that the loads of one column are in
// flight together instead of one after another.
constexpr int kRedRows = 16;
template <typename T, int D, int DV>
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(BwdArgs a) {
  const PlanHeader* hdr = a.kws.header;
  // a plan of another geometry: the dK / dV kernel reported it; no split
  // item: nothing to reduce
  if (hdr->key != a.kkey || hdr->max_split <= 1) return;
  const int hkv = a.g.hkv;
  const int n_work = hdr->n_tiles * hkv;
  constexpr int W = D + DV;
  constexpr int C4 = W / 4;  // float4 columns per key row
  constexpr int NSLAB = kBwdKeyRows / kRedRows;
  const int64_t jstride = (int64_t)hkv * kBwdKeyRows * C4;  // between chunks, in float4
  for (int v = blockIdx.x; v < n_work * NSLAB; v += gridDim.x) {
    const int w = v / NSLAB, slab = v - w * NSLAB;
    const int t = w / hkv, kvh = w - t * hkv;
    const int4 tile = a.kws.tiles[t];
    // chunk 0 of a split item reduces it; its slot is the first of S
    if (!(tile.w & 1) || ((tile.w >> 1) & 15) != 0) continue;
    const int seg = tile.x, k_row0 = tile.y;
    const int slot0 = (int)((uint32_t)tile.w >> 5);
    const int S = max(1, min(a.kws.seg_split[seg], kMaxSplits));
    const int k0 = a.g.cu_k[seg], uk = a.g.used_k[seg];
    const f32x4* part = reinterpret_cast<const f32x4*>(a.kpart) +
                        ((int64_t)slot0 * hkv + kvh) * kBwdKeyRows * C4;
    for (int i = threadIdx.x; i < kRedRows * C4; i += blockDim.x) {
      const int kr = slab * kRedRows + i / C4, c4 = i % C4;
      if (k_row0 + kr >= uk) continue;
      const f32x4* p = part + kr * C4 + c4;
      // every load unconditional (chunks past S read chunk S - 1 again), so
      // that they form one block and issue back to back
      f32x4 pj[kMaxSplits];
#pragma unroll
      for (int j = 0; j < kMaxSplits; ++j) pj[j] = p[min(j, S - 1) * jstride];
      f32x4 sum = f32x4{};
#pragma unroll
      for (int j = 0; j < kMaxSplits; ++j)
        if (j < S) sum += pj[j];
      const int64_t row = (int64_t)(k0 + k_row0 + kr) * hkv + kvh;
      typename Elem<T>::v4 o;
      if (4 * c4 < D) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) o[cc] = (T)(sum[cc] * a.scale);
        *reinterpret_cast<typename Elem<T>::v4*>(static_cast<T*>(a.dk) + row * D + 4 * c4) = o;
      } else {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) o[cc] = (T)sum[cc];
        *reinterpret_cast<typename Elem<T>::v4*>(static_cast<T*>(a.dv) + row * DV + 4 * c4 - D) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename K>
hipError_t launch_persistent(K kern, int threads, int64_t max_work, const BwdArgs& a,
                             hipStream_t s) {
  const int grid = persistent_grid(reinterpret_cast<const void*>(kern), threads, max_work);
  if (grid <= 0) return grid == 0 ? hipSuccess : hipErrorInvalidValue;
  return launch_kernel(kern, dim3(grid), dim3(threads), s, a);
}

template <typename T, int D, int DV>
hipError_t launch_dims(const BwdArgs& a, const TileShape& t, hipStream_t s, bool* ok) {
  *ok = true;
  const int64_t q_work = (int64_t)(a.g.total_q / t.rows + a.g.nseg + 1) * a.n_head_chunks;
  hipError_t e;
  switch (t.gf) {
    case 4: e = launch_persistent(bwd_dq_kernel<T, D, DV, 4, 1>, 256, q_work, a, s); break;
    case 3: e = launch_persistent(bwd_dq_kernel<T, D, DV, 3, 1>, 192, q_work, a, s); break;
    case 2: e = launch_persistent(bwd_dq_kernel<T, D, DV, 2, 2>, 256, q_work, a, s); break;
    case 1: e = launch_persistent(bwd_dq_kernel<T, D, DV, 1, 4>, 256, q_work, a, s); break;
    default: *ok = false; return hipSuccess;
  }
  if (e != hipSuccess) return e;
  const int64_t k_work =
      (int64_t)(a.g.total_k / kBwdKeyRows + a.g.nseg + 1) * a.g.hkv * kMaxSplits;
  e = launch_persistent(bwd_dkv_kernel<T, D, DV>, 256, k_work, a, s);
  if (e != hipSuccess) return e;
  // walks the work list and reduces the split items (none: it only scans)
  const int64_t r_work = a.kpart_slots > 0 ? k_work : 0;
  const int grid = (int)(r_work < 2048 ? r_work : 2048);
  if (grid > 0) {
    auto reduce = bwd_kv_reduce_kernel<T, D, DV>;
    e = launch_kernel(reduce, dim3(grid), dim3(256), s, a);
  }
  return e;
}

template <typename T>
hipError_t launch_bwd_t(const BwdArgs& a, const TileShape& t, hipStream_t s, bool* ok) {
  const int dd = a.g.d, dv = a.g.dv;
  if (dd == 64 && dv == 64) return launch_dims<T, 64, 64>(a, t, s, ok);
  if (dd == 64 && dv == 128) return launch_dims<T, 64, 128>(a, t, s, ok);
  if (dd == 128 && dv == 64) return launch_dims<T, 128, 64>(a, t, s, ok);
  if (dd == 128 && dv == 128) return launch_dims<T, 128, 128>(a, t, s, ok);
  *ok = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int dtype, const TileShape& t, hipStream_t s,
                      bool* supported) {
  BwdArgs args = a;
  args.n_cu = device_cu_count();
  if (args.n_cu <= 0) return hipErrorInvalidValue;
  if (dtype == GVATTN_BF16) return launch_bwd_t<__bf16>(args, t, s, supported);
  if (dtype == GVATTN_FP16) return launch_bwd_t<_Float16>(args, t, s, supported);
  *supported = false;
  return hipSuccess;
}

}  // namespace gvattn
