// BF16 / FP16 segmented varlen attention forward on gfx950 matrix cores.
//
// What it computes: cosmos-framework PR #302, "What" (used prefixes of each
// segment, untouched gap rows, zero output / -inf LSE without keys);
// TensorRT-LLM issue #18687, "actual behavior" (keys past the used length
// are masked, never attended as zeros); PR #312, "Problem and behavior"
// (GQA folding, FP32 LSE).
//
// Design (gfx950):
//   * A persistent grid walks the plan's tile list (segment, first row);
//     work item = (tile, chunk of GF query heads sharing one KV head).  One
//     wave owns 32 query rows of one head, so the K/V tiles in LDS serve
//     all GF heads of the group.
//   * K and V tiles (32 keys for d <= 128, which fits three workgroups per
//     compute unit; 64 keys for d = 256) move HBM -> LDS with
//     buffer_load ... lds (no register staging), double-buffered: the loads
//     of tile t+1 are issued between the score MFMAs of tile t, one barrier
//     per tile.  The LDS rows are XOR swizzled at 16-byte granularity so
//     that the matrix-core operand reads avoid bank conflicts.
//   * Scores are computed transposed, S^T = K . Q^T, with
//     v_mfma_f32_32x32x16_bf16 (or _f16); Q stays in registers.  Each lane
//     then holds half of the tile's keys for one query row: one cross-lane
//     exchange per tile for the row max, none for the row sum until the end.
//   * O^T += V^T . P^T takes P straight from the score registers; V^T is
//     read from the row-major V tile with ds_read_b64_tr_b16 (a 4x16
//     transpose per 16 lanes), so V is never transposed in memory.
//   * Online softmax in the exp2 domain with FP32 max/sum.  The running max
//     is only raised (and O rescaled) when a row's max grows by more than
//     2^8, which keeps the rescale off the common path.  Two row sums are
//     kept: the sum of the FP32 weights gives the LSE, the sum of the
//     weights as rounded for the P.V product normalises O, so that O is a
//     weighted mean of V whose weights' rounding largely cancels (a key that
//     dominates a row then costs no rounding error; with the max held back,
//     its weight is not exactly 1).
//   * Rows that see at most one tile of keys add the rounding remainder of
//     P as a second product on that tile.
//   * O rows leave through LDS staging as full-row stores with the
//     non-temporal policy (nothing reads them again; K/V keeps the L2).
//   * Buffer resources end at the segment's last used row: loads past it
//     return zero (ragged key tiles, gap rows, buffer ends) and stores past
//     it are dropped (gap rows of O stay bit-exact).  Key-padding and causal
//     masks set scores to -inf on boundary tiles only.
#include <math.h>

#include <type_traits>

#include "gvattn_internal.h"
#include "gvattn_mfma.h"

namespace gvattn {
namespace {

using namespace dev;
using namespace mfma;

// DQ: head dim of Q and K; DV: head dim of V and O.
template <int DQ, int DV, int GF, int RB, int NKB>
struct Cfg {
  static constexpr int NW = GF * RB;          // waves per workgroup
  static constexpr int NT = 64 * NW;          // threads
  static constexpr int NKB_ = NKB;            // 32-key blocks per tile (1 or 2)
  static constexpr int BN = 32 * NKB;         // keys per tile
  static constexpr int CHK = DQ / 8;          // 16-byte chunks per K row
  static constexpr int CHV = DV / 8;          // 16-byte chunks per V / O row
  static constexpr int K_TILE_BYTES = BN * DQ * 2;
  static constexpr int V_TILE_BYTES = BN * DV * 2;
  static constexpr int STAGE_BYTES = K_TILE_BYTES + V_TILE_BYTES;
  static constexpr int DMA_K = K_TILE_BYTES / 1024;  // 1 KB per wave instruction
  static constexpr int DMA_V = V_TILE_BYTES / 1024;
  static constexpr int OP = DV + 8;           // O staging row pitch (elements)
  static constexpr int O_BYTES = NW * 32 * OP * 2;
  static constexpr int LDS_BYTES = (2 * STAGE_BYTES > O_BYTES) ? 2 * STAGE_BYTES : O_BYTES;
  static constexpr int KK = DQ / 16;          // k-steps of the score MFMA
  static constexpr int DB = DV / 32;          // 32-wide d blocks of O
  static constexpr int MIN_BLOCKS = (DQ <= 128 && DV <= 128) ? (NKB == 1 ? 3 : 2) : 1;
  static constexpr int NDMA_K = (DMA_K + NW - 1) / NW;  // DMA instructions per wave
  static constexpr int NDMA_V = (DMA_V + NW - 1) / NW;
};

// Position of a key-range cursor: range i (rows row0 .. row0 + len - 1 of
// K/V, keys pos .. pos + len - 1 of the segment's concatenated sequence),
// local tile lt of its nt tiles.  nt == 0: no tiles left.
struct KeyCursor {
  int i, row0, len, pos, lt, nt;
};

template <typename T, int DQ, int DV, int GF, int RB, int NKB, bool KR>
__global__ __launch_bounds__((Cfg<DQ, DV, GF, RB, NKB>::NT),
                             (Cfg<DQ, DV, GF, RB, NKB>::MIN_BLOCKS))
void fwd_mfma_kernel(FwdArgs a) {
  using C = Cfg<DQ, DV, GF, RB, NKB>;
  using E = Elem<T>;
  using v8 = typename E::v8;
  using v4 = typename E::v4;
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];

  const PlanHeader* hdr = a.ws.header;
  if (hdr->key != a.key) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(&a.ws.header->err, GVATTN_DEVERR_PLAN);
    return;
  }
  const int n_tiles = hdr->n_tiles;
  const int n_hc = a.n_head_chunks;
  const int n_work = n_tiles * n_hc;  // < 2^31: tiles <= total_q / 32 + nseg

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hh = lane >> 5;
  const int hf = wave % GF, rb = wave / GF;
  const int G = a.g.hq / a.g.hkv;
  // bytes between consecutive rows of Q, K, V and O
  const uint32_t qstride = (uint32_t)a.g.hq * DQ * 2;
  const uint32_t kstride = (uint32_t)a.g.hkv * DQ * 2;
  const uint32_t vstride = (uint32_t)a.g.hkv * DV * 2;
  const uint32_t ostride = (uint32_t)a.g.hq * DV * 2;
  const float c = a.scale_log2;

  // Per-lane global offsets of this wave's K/V DMA instructions: slot s of
  // a tile (1 KB per instruction, 16 B per lane) holds row s / CH, chunk
  // (s % CH) ^ swizzle(row).
  uint32_t koff[C::NDMA_K], voff[C::NDMA_V];
#pragma unroll
  for (int i = 0; i < C::NDMA_K; ++i) {
    const int s = (wave + i * C::NW) * 64 + lane;
    const int row = s / C::CHK, pc = s % C::CHK;
    koff[i] = (uint32_t)row * kstride + (uint32_t)((pc ^ swz_k<DQ>(row)) * 16);
  }
#pragma unroll
  for (int i = 0; i < C::NDMA_V; ++i) {
    const int s = (wave + i * C::NW) * 64 + lane;
    const int row = s / C::CHV, pc = s % C::CHV;
    voff[i] = (uint32_t)row * vstride + (uint32_t)((pc ^ swz_v<DV>(row)) * 16);
  }

  // ds_read_b64_tr_b16 addressing inside each 16-lane group: local lane
  // i = lane % 16 addresses row 4*hh + i/4 of a 16-key block and the 8 bytes
  // at element 16*((lane >> 4) & 1) + 4*(i % 4) of a 32-wide d block; lane
  // i then receives column i (d = db*32 + r32) of those 4 rows.
  const int il = lane & 15;
  const int vrow_l = 4 * hh + (il >> 2);
  const int vd_l = 16 * ((lane >> 4) & 1) + 4 * (il & 3);

  // Static schedule.  Work item w lives in queue w % 8 at position w / 8
  // (with 8 head chunks, queue = head chunk = KV head, and workgroup b runs
  // on XCD b % 8 under round-robin dispatch, so one XCD's L2 serves one KV
  // head).  The n_q workgroups of queue q take its items in rounds, forward
  // in even rounds and backward in odd ones: with the tile list sorted by
  // decreasing cost, every workgroup alternates long and short items.
  //
  // Workgroups sharing a compute unit are dispatched in slots (slot =
  // blockIdx / compute units) and wave arbitration favours the older ones,
  // so with equal work the last slot would finish well after the first.
  // The wave priority therefore rotates with every item: each workgroup
  // holds the top priority for 1 / slots of its items.
  const int q = blockIdx.x & 7, qi = blockIdx.x >> 3;
  const int n_q = ((int)gridDim.x - q + 7) >> 3;
  const int n_slots = min(4, ((int)gridDim.x + a.n_cu - 1) / a.n_cu);
  const int slot = (int)blockIdx.x / a.n_cu;
  for (int r = 0;; ++r) {
    const int j = r * n_q + ((r & 1) ? n_q - 1 - qi : qi);
    const int w = j * 8 + q;
    if (w >= n_work) break;
    switch ((r + slot) % n_slots) {
      case 0: __builtin_amdgcn_s_setprio(0); break;
      case 1: __builtin_amdgcn_s_setprio(1); break;
      case 2: __builtin_amdgcn_s_setprio(2); break;
      default: __builtin_amdgcn_s_setprio(3); break;
    }
    const int t = (int)((uint32_t)w / (uint32_t)n_hc);
    const int hc = w - t * n_hc;
    // Work-item geometry is wave-uniform: keep it in scalar registers so
    // the buffer resources built from it need no per-lane loops.
    const int4 tile = a.ws.tiles[t];
    const int seg = __builtin_amdgcn_readfirstlane(tile.x);
    const int row0 = __builtin_amdgcn_readfirstlane(tile.y);
    const int head0 = hc * GF;
    const int head = head0 + hf;
    const int kvh = head0 / G;
    const int q0 = __builtin_amdgcn_readfirstlane(a.g.cu_q[seg]);
    const int uq = __builtin_amdgcn_readfirstlane(a.g.used_q[seg]);
    // keys: the used prefix at k0, or (KR) the concatenation of the
    // segment's ranges, whose total length the plan stored
    const int k0 = KR ? 0 : __builtin_amdgcn_readfirstlane(a.g.cu_k[seg]);
    const int uk = __builtin_amdgcn_readfirstlane(KR ? a.ws.seg_keys[seg] : a.g.used_k[seg]);
    const int wr0 = row0 + rb * 32;                  // first row of this wave
    const int r_last = min(row0 + 32 * RB, uq) - 1;  // last used row of the tile
    int kend = uk;
    if (a.g.causal) kend = max(0, min(uk, r_last + uk - uq + 1));

    // Key-range form: tiles never straddle two ranges; cursor `cur` is the
    // tile being computed, `nx` the one being loaded.
    const int kr_end = KR ? __builtin_amdgcn_readfirstlane(a.g.kr_off[seg + 1]) : 0;
    auto settle = [&](KeyCursor& c) {  // first range from c.i on with a tile below kend
      c.nt = 0;
      while (c.i < kr_end && c.pos < kend) {
        c.row0 = __builtin_amdgcn_readfirstlane(a.g.kr_start[c.i]);
        c.len = __builtin_amdgcn_readfirstlane(a.g.kr_len[c.i]);
        const int n = min(c.len, kend - c.pos);
        c.lt = 0;
        c.nt = n > 0 ? (n + C::BN - 1) / C::BN : 0;
        if (c.nt > 0) return;
        c.pos += c.len;
        ++c.i;
      }
      c.nt = 0;
    };
    auto advance = [&](KeyCursor& c) {
      if (c.lt + 1 < c.nt) {
        ++c.lt;
      } else {
        c.pos += c.len;
        ++c.i;
        settle(c);
      }
    };
    KeyCursor cur{0, 0, 0, 0, 0, 0};
    int n_kt;
    if constexpr (KR) {
      cur.i = __builtin_amdgcn_readfirstlane(a.g.kr_off[seg]);
      settle(cur);
      n_kt = 0;
      for (KeyCursor c = cur; c.nt > 0; c.pos += c.len, ++c.i, settle(c)) n_kt += c.nt;
    } else {
      n_kt = (kend + C::BN - 1) / C::BN;
    }
    // key tiles of this entry: all of them, or one split-K chunk
    // [tile.z, tile.w >> 5) whose result goes to the FP32 partials
    const bool partial = !KR && (tile.w & 1);
    const int split_j = (tile.w >> 1) & 15;
    const int kt_begin = KR ? 0 : min(__builtin_amdgcn_readfirstlane(tile.z), n_kt);
    const int kt_end = KR ? n_kt : min(__builtin_amdgcn_readfirstlane(tile.w) >> 5, n_kt);

    const T* qbase = static_cast<const T*>(a.q) + ((int64_t)q0 * a.g.hq + head) * DQ;
    const uint32_t qbytes = uq > 0 ? (uint32_t)(uq - 1) * qstride + DQ * 2 : 0u;
    const auto qr = make_rsrc(qbase, qbytes);
    // K and V rows [first, first + n) of this KV head as bounded resources
    auto k_rsrc = [&](int first, int n) {
      return make_rsrc(static_cast<const T*>(a.k) + ((int64_t)first * a.g.hkv + kvh) * DQ,
                       n > 0 ? (uint32_t)(n - 1) * kstride + DQ * 2 : 0u);
    };
    auto v_rsrc = [&](int first, int n) {
      return make_rsrc(static_cast<const T*>(a.v) + ((int64_t)first * a.g.hkv + kvh) * DV,
                       n > 0 ? (uint32_t)(n - 1) * vstride + DV * 2 : 0u);
    };
    const int kfirst = KR ? cur.row0 : k0, klen = KR ? cur.len : uk;
    const auto kr = k_rsrc(kfirst, klen);
    const auto vr = v_rsrc(kfirst, klen);

    // the first tile of the item goes to stage 0 (the stage of a tile is
    // its parity counted from kt_begin, a compile-time constant below)
    auto issue_tile = [&](int kt) {
      char* st = lds;
      const uint32_t soffk = (uint32_t)kt * C::BN * kstride;
      const uint32_t soffv = (uint32_t)kt * C::BN * vstride;
#pragma unroll
      for (int i = 0; i < C::NDMA_K; ++i) {
        const int inst = wave + i * C::NW;
        if (inst < C::DMA_K) dma16(kr, st + inst * 1024, koff[i], soffk);
      }
#pragma unroll
      for (int i = 0; i < C::NDMA_V; ++i) {
        const int inst = wave + i * C::NW;
        if (inst < C::DMA_V) dma16(vr, st + C::K_TILE_BYTES + inst * 1024, voff[i], soffv);
      }
    };

    if (kt_begin < kt_end) issue_tile(kt_begin);

    // Q fragment: lane holds Q[wr0 + r32][16*kk + 8*hh .. +7]
    v8 qf[C::KK];
    {
      const uint32_t roff = (uint32_t)(wr0 + r32) * qstride + hh * 16;
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk)
        qf[kk] = __builtin_bit_cast(v8, buf_load16(qr, roff + kk * 32));
    }

    f32x16 o[C::DB];
#pragma unroll
    for (int i = 0; i < C::DB; ++i) o[i] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    float lh_run = 0.f;  // sum of the rounded weights (normalises O)

    const int row = wr0 + r32;                       // this lane's query row
    const int lim = a.g.causal ? min(uk, row + uk - uq + 1) : uk;
    const int lim_w = a.g.causal ? min(uk, wr0 + uk - uq + 1) : uk;  // wave minimum

    KeyCursor nx = cur;
    // One tile: stage ST holds it, the loads of the next tile go to stage
    // 1 - ST.  With the stage a constant (std::integral_constant) every LDS
    // operand address is a per-lane register plus an immediate offset.
    auto tile_step = [&](int kt, auto stage_c) __attribute__((always_inline)) {
      const int ST = stage_c;
      wait_vmem();
      __syncthreads();
      const char* Ks = lds + ST * C::STAGE_BYTES;
      const char* Vs = Ks + C::K_TILE_BYTES;
      if constexpr (KR) advance(nx);

      // The loads of tile kt + 1 are spread between the score MFMAs, so
      // their issue overlaps matrix-core work.  Without a next tile they go
      // through zero-size buffer resources (every load returns zero into the
      // stage nobody reads any more), which keeps the phase branch-free.
      const int nlen = (kt + 1 < kt_end) ? (KR ? nx.len : uk) : 0;
      const int nfirst = KR ? nx.row0 : k0;
      const auto krn = k_rsrc(nfirst, nlen);
      const auto vrn = v_rsrc(nfirst, nlen);
      char* stn = lds + (1 - ST) * C::STAGE_BYTES;
      const uint32_t ntile = (uint32_t)(KR ? nx.lt : kt + 1) * C::BN;
      const uint32_t soffkn = ntile * kstride, soffvn = ntile * vstride;
      // j < NDMA_K: K instruction j of this wave, then the V instructions
      auto issue_one = [&](int j) {
        if (j < C::NDMA_K) {
          const int inst = wave + j * C::NW;
          if (j + 1 < C::NDMA_K || inst < C::DMA_K) dma16(krn, stn + inst * 1024, koff[j], soffkn);
        } else {
          const int i = j - C::NDMA_K;
          const int inst = wave + i * C::NW;
          if (i + 1 < C::NDMA_V || inst < C::DMA_V)
            dma16(vrn, stn + C::K_TILE_BYTES + inst * 1024, voff[i], soffvn);
        }
      };

      // S^T = K . Q^T for two 32-key blocks
      f32x16 s[C::NKB_];
#pragma unroll
      for (int kb = 0; kb < C::NKB_; ++kb) {
        s[kb] = f32x16{};
        const int krow = kb * 32 + r32;
        const char* kp = Ks + krow * (DQ * 2);
        const int sw = swz_k<DQ>(krow);
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) {
          const v8 ka = *reinterpret_cast<const v8*>(kp + (((2 * kk + hh) ^ sw) << 4));
          s[kb] = E::mfma(ka, qf[kk], s[kb]);
          const int step = kb * C::KK + kk;
          constexpr int NJ = C::NDMA_K + C::NDMA_V;
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            if ((j * C::NKB_ * C::KK) / NJ == step) issue_one(j);
        }
      }

      // key-padding / causal mask on boundary tiles (in the key-range form
      // keys past the end of the tile's range are masked as well)
      const int kbase = KR ? cur.pos + cur.lt * C::BN : kt * C::BN;
      const int lim_t = KR ? min(lim, cur.pos + cur.len) : lim;
      const int lim_wt = KR ? min(lim_w, cur.pos + cur.len) : lim_w;
      if constexpr (C::MIN_BLOCKS == 1) {
        // one workgroup per CU (d = 256): mask, then the exact step below
        // only (a second softmax path cost these variants more registers
        // than it saved)
        if (kbase + C::BN > lim_wt) {
          int nv = lim_t - kbase - 4 * hh;
          asm volatile("" : "+v"(nv));
#pragma unroll
          for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (kb * 32 + 8 * (v >> 2) + (v & 3) >= nv) s[kb][v] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
        mx = fmaxf(mx, max_across_halves(mx));
        const float cand = mx * c;
        if (__any(cand > m_run + 8.f)) {
          keep_branch();
          const float m_new = fmaxf(m_run, cand);
          const float alpha = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
          lh_run *= alpha;
#pragma unroll
          for (int i = 0; i < C::DB; ++i) o[i] *= alpha;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float p = exp2_fast(__builtin_fmaf(s[kb][v], c, -m_use));
            s[kb][v] = p;
            rs += p;
          }
        l_run += rs;
      } else {
        auto mask_scores = [&]() __attribute__((always_inline)) {
          if (kbase + C::BN > lim_wt) {
            // score (kb, v) is key kbase + kb*32 + 8*(v/4) + 4*hh + v%4: it is
            // masked when its compile-time offset reaches lim_t - kbase - 4*hh
            int nv = lim_t - kbase - 4 * hh;
            asm volatile("" : "+v"(nv));  // defined here: the compares stay in the branch
#pragma unroll
            for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
              for (int v = 0; v < 16; ++v)
                if (kb * 32 + 8 * (v >> 2) + (v & 3) >= nv) s[kb][v] = -INFINITY;
          }
        };
        mask_scores();

        // Online softmax in the exp2 domain.  P = exp2(S*c - m) with m the
        // running max as it stands: P then exceeds 1 by the factor the row's
        // max has grown since m was set.  The exact step (tile row max; m
        // raised and O rescaled when it grew by more than 2^8) runs when a
        // row with keys in this tile has no m yet, or when some lane's
        // partial row sum leaves [0, 2^15] (its scores are then recomputed
        // from the K tile), so that every weight stays within fp16 range.
        float rs = 0.f;
        bool exact = __any(m_run == -INFINITY && kbase < lim_t);
        if (!exact) {
          // rows without m have no key in this tile: their scores are -inf
          const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
          for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float p = exp2_fast(__builtin_fmaf(s[kb][v], c, -m_use));
              s[kb][v] = p;
              rs += p;
            }
          exact = __any(!(rs <= 0x1p15f));  // every weight <= 2^15: fp16 holds it
          if (exact) {
            keep_branch();
#pragma unroll
            for (int kb = 0; kb < C::NKB_; ++kb) {
              s[kb] = f32x16{};
              const int krow = kb * 32 + r32;
              const char* kp = Ks + krow * (DQ * 2);
              const int sw = swz_k<DQ>(krow);
#pragma unroll
              for (int kk = 0; kk < C::KK; ++kk)
                s[kb] = E::mfma(*reinterpret_cast<const v8*>(kp + (((2 * kk + hh) ^ sw) << 4)), qf[kk], s[kb]);
            }
            mask_scores();
          }
        }
        if (exact) {
          keep_branch();
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
          mx = fmaxf(mx, max_across_halves(mx));
          const float cand = mx * c;
          if (__any(cand > m_run + 8.f)) {
            keep_branch();
            const float m_new = fmaxf(m_run, cand);
            const float alpha = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
            lh_run *= alpha;
#pragma unroll
            for (int i = 0; i < C::DB; ++i) o[i] *= alpha;
          }
          const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
          rs = 0.f;
#pragma unroll
          for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float p = exp2_fast(__builtin_fmaf(s[kb][v], c, -m_use));
              s[kb][v] = p;
              rs += p;
            }
        }
        l_run += rs;
      }

      // P^T as 16-bit MFMA operands straight from the score registers
      v8 pb[C::NKB_][2];
#pragma unroll
      for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[kb][a2][j] = (T)s[kb][8 * a2 + j];
#pragma unroll
      for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) lh_run = E::sum8(pb[kb][a2], lh_run);

      // O^T += V^T . P^T, V^T read transposed from the row-major V tile
      auto pv = [&](const v8 (&p)[C::NKB_][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int dcol = db * 32 + vd_l;
          const int ch = dcol >> 3, within = (dcol & 7) * 2;
#pragma unroll
          for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2) {
              const int r_lo = kb * 32 + a2 * 16 + vrow_l;
              const int r_hi = r_lo + 8;
              const i16x4 lo = read_tr(Vs + r_lo * (DV * 2) + ((ch ^ swz_v<DV>(r_lo)) << 4) + within);
              const i16x4 hi = read_tr(Vs + r_hi * (DV * 2) + ((ch ^ swz_v<DV>(r_hi)) << 4) + within);
              const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
              const v8 va = __builtin_bit_cast(v8, both);
              o[db] = E::mfma(va, p[kb][a2], o[db]);
            }
        }
      };
      // Rows that see at most one tile of keys in all: the rounding of their
      // few large weights to 16 bits would dominate their error, so the
      // tiles holding their keys also add the rounding remainder of P,
      // P - round(P), as a second product (P is then exact to about 2^-17).
      if (kbase < C::BN && lim_wt <= C::BN) {
        keep_branch();
        v8 pl[C::NKB_][2];
#pragma unroll
        for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
          for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
            for (int j = 0; j < 8; ++j)
              pl[kb][a2][j] = (T)(s[kb][8 * a2 + j] - (float)pb[kb][a2][j]);
#pragma unroll
        for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
          for (int a2 = 0; a2 < 2; ++a2) lh_run = E::sum8(pl[kb][a2], lh_run);
        pv(pl);
      }
      pv(pb);
      if constexpr (KR) cur = nx;
    };
    if constexpr (C::MIN_BLOCKS > 1) {
      // unrolled by two: constant stages (about 15 fewer VALU instructions
      // per tile)
      for (int kt = kt_begin; kt < kt_end; kt += 2) {
        tile_step(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < kt_end) tile_step(kt + 1, std::integral_constant<int, 1>{});
      }
    } else if constexpr (!KR) {
      // One workgroup per CU (d > 128), so one wave per SIMD: no other wave
      // fills the matrix cores while this one runs its softmax.  The loop is
      // software-pipelined instead, with K one tile ahead of V.  Step t
      // computes the scores of tile t + 1 interleaved with the exponentials
      // and 16-bit conversion of tile t, then P.V of tile t interleaved with
      // the row max of tile t + 1, then (rarely) raises the running max and
      // rescales O before the weights of tile t + 1.  K(t) and V(t) sit in
      // stage (t - kt_begin) & 1 as in the loop above; step t loads K(t + 2)
      // into the stage K(t) leaves and V(t + 1) into the one V(t - 1) left.
      // Past the last tile the loads go through zero-size resources (zeros
      // into stages nobody reads), so the scores of the tile after the last
      // one are computed, from zeros, and dropped.
      auto stage_of = [&](int kt) __attribute__((always_inline)) {
        return lds + ((kt - kt_begin) & 1) * C::STAGE_BYTES;
      };
      auto score_mfma = [&](const char* Ks, f32x16 (&sv)[C::NKB_], int kk, int kb)
                            __attribute__((always_inline)) {
        const int krow = kb * 32 + r32;
        const v8 ka = *reinterpret_cast<const v8*>(Ks + krow * (DQ * 2) +
                                                   (((2 * kk + hh) ^ swz_k<DQ>(krow)) << 4));
        sv[kb] = E::mfma(ka, qf[kk], sv[kb]);
      };
      // P.V with each V^T operand read PD - 1 products ahead of its use (one
      // wave per SIMD: no other wave hides the LDS latency), consecutive
      // products accumulating into different O blocks
      constexpr int PD = 3;
      auto pv_tile = [&](const char* Vs, const v8 (&p)[C::NKB_][2], auto&& work)
                         __attribute__((always_inline)) {
        auto v_operand = [&](int idx) __attribute__((always_inline)) {
          const int db = idx % C::DB, ka = idx / C::DB;
          const int dcol = db * 32 + vd_l;
          const int ch = dcol >> 3, within = (dcol & 7) * 2;
          const int r_lo = (ka >> 1) * 32 + (ka & 1) * 16 + vrow_l;
          const int r_hi = r_lo + 8;
          const i16x4 lo = read_tr(Vs + r_lo * (DV * 2) + ((ch ^ swz_v<DV>(r_lo)) << 4) + within);
          const i16x4 hi = read_tr(Vs + r_hi * (DV * 2) + ((ch ^ swz_v<DV>(r_hi)) << 4) + within);
          return __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        constexpr int NPV = C::DB * C::NKB_ * 2;
        v8 ring[PD];
#pragma unroll
        for (int i = 0; i < PD - 1; ++i) ring[i] = v_operand(i);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
          if (i + PD - 1 < NPV) ring[(i + PD - 1) % PD] = v_operand(i + PD - 1);
          asm volatile("" ::: "memory");  // the reads stay here, ahead of their use
          const int db = i % C::DB, ka = i / C::DB;
          o[db] = E::mfma(ring[i % PD], p[ka >> 1][ka & 1], o[db]);
          work(i);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // key-padding / causal mask of a score tile starting at key kbase
      auto mask_tile = [&](f32x16 (&sv)[C::NKB_], int kbase) __attribute__((always_inline)) {
        if (kbase + C::BN > lim_w) {
          int nv = lim - kbase - 4 * hh;
          asm volatile("" : "+v"(nv));
#pragma unroll
          for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (kb * 32 + 8 * (v >> 2) + (v & 3) >= nv) sv[kb][v] = -INFINITY;
        }
      };
      // Row max of a score tile (lane max mx, both halves) against the
      // running max: raise it and rescale O when it grew by more than 2^8.
      // Returns the max the weights of that tile are taken against.
      auto settle_max = [&](float mx, bool valid) __attribute__((always_inline)) {
        mx = fmaxf(mx, max_across_halves(mx));
        const float cand = valid ? mx * c : -INFINITY;
        if (__any(cand > m_run + 8.f)) {
          keep_branch();
          const float m_new = fmaxf(m_run, cand);
          const float alpha = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
          lh_run *= alpha;
#pragma unroll
          for (int i = 0; i < C::DB; ++i) o[i] *= alpha;
        }
        return (m_run == -INFINITY) ? 0.f : m_run;
      };

      f32x16 sc[C::NKB_];
#pragma unroll
      for (int kb = 0; kb < C::NKB_; ++kb) sc[kb] = f32x16{};
      if (kt_begin < kt_end) {
        wait_vmem();
        __syncthreads();
        // K of the second tile into stage 1, then the scores of the first
        const int kn = kt_begin + 1;
        const auto krn = k_rsrc(k0, kn < kt_end ? uk : 0);
        char* st = lds + C::STAGE_BYTES;
        const uint32_t soff = (uint32_t)kn * C::BN * kstride;
#pragma unroll
        for (int i = 0; i < C::NDMA_K; ++i) {
          const int inst = wave + i * C::NW;
          if (C::DMA_K % C::NW == 0 || i + 1 < C::NDMA_K || inst < C::DMA_K)
            dma16(krn, st + inst * 1024, koff[i], soff);
        }
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
          for (int kb = 0; kb < C::NKB_; ++kb) score_mfma(lds, sc, kk, kb);
      }
      float m_use = 0.f;
      if (kt_begin < kt_end) {
        mask_tile(sc, kt_begin * C::BN);
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kb][v]);
        m_use = settle_max(mx, true);
      }
      for (int kt = kt_begin; kt < kt_end; ++kt) {
        // Q is only a matrix-core operand: keep it in AGPRs, which leaves
        // the VGPRs to O and the two score tiles
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) asm volatile("" : "+a"(qf[kk]));
        wait_vmem();
        __syncthreads();  // K(kt + 1) and V(kt) are in; K(kt), V(kt - 1) are free
        const char* Vs = stage_of(kt) + C::K_TILE_BYTES;
        const char* Kn = stage_of(kt + 1);
        const auto krn = k_rsrc(k0, kt + 2 < kt_end ? uk : 0);
        const auto vrn = v_rsrc(k0, kt + 1 < kt_end ? uk : 0);
        char* stk = stage_of(kt);
        char* stv = stage_of(kt + 1) + C::K_TILE_BYTES;
        const uint32_t soffk = (uint32_t)(kt + 2) * C::BN * kstride;
        const uint32_t soffv = (uint32_t)(kt + 1) * C::BN * vstride;
        // (the range test is a branch only when the waves do not share the
        // instructions evenly)
        auto issue_one = [&](int j) __attribute__((always_inline)) {
          if (j < C::NDMA_K) {
            const int inst = wave + j * C::NW;
            if (C::DMA_K % C::NW == 0 || j + 1 < C::NDMA_K || inst < C::DMA_K)
              dma16(krn, stk + inst * 1024, koff[j], soffk);
          } else {
            const int i = j - C::NDMA_K;
            const int inst = wave + i * C::NW;
            if (C::DMA_V % C::NW == 0 || i + 1 < C::NDMA_V || inst < C::DMA_V)
              dma16(vrn, stv + inst * 1024, voff[i], soffv);
          }
        };

        const int kbase = kt * C::BN;

        // Scores of tile kt + 1 (and the loads of step kt) with the weights
        // of tile kt, written out as NS chunks that the compiler may not
        // reorder across (sched_barrier): chunk i reads the K operand of
        // MFMA i + PD - 1, issues MFMA i, takes the exponential of score i of
        // tile kt and, as they complete, converts pairs of weights to 16 bits
        // and adds groups of eight to the rounded-weight sum.  The vector
        // instructions of a chunk then issue while its MFMA runs.  The loads
        // of step kt go out over the first half of the chunks: the P.V reads
        // below wait for them (the transposed-read builtin carries no alias
        // information, so the compiler waits for every LDS-DMA in flight).
        constexpr int NS = C::KK * C::NKB_;
        constexpr int NSC = 16 * C::NKB_;            // scores per lane
        constexpr int SPC = (NSC + NS - 1) / NS;      // scores per chunk
        constexpr int NJ = C::NDMA_K + C::NDMA_V;
        f32x16 sn[C::NKB_];
#pragma unroll
        for (int kb = 0; kb < C::NKB_; ++kb) sn[kb] = f32x16{};
        auto k_operand = [&](int i) __attribute__((always_inline)) {
          const int kk = i / C::NKB_, kb = i % C::NKB_;
          const int krow = kb * 32 + r32;
          return *reinterpret_cast<const v8*>(Kn + krow * (DQ * 2) +
                                              (((2 * kk + hh) ^ swz_k<DQ>(krow)) << 4));
        };
        v8 pb[C::NKB_][2];
        float rs = 0.f;
        v8 kring[PD];
#pragma unroll
        for (int i = 0; i < PD - 1; ++i) kring[i] = k_operand(i);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          if (i + PD - 1 < NS) kring[(i + PD - 1) % PD] = k_operand(i + PD - 1);
          asm volatile("" ::: "memory");
          sn[i % C::NKB_] = E::mfma(kring[i % PD], qf[i / C::NKB_], sn[i % C::NKB_]);
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            if ((j * ((NS + 1) / 2)) / NJ == i) issue_one(j);
#pragma unroll
          for (int u = 0; u < SPC; ++u) {
            const int sidx = i * SPC + u;
            if (sidx < NSC) {
              const int kb = sidx / 16, v = sidx % 16;
              const float pw = exp2_fast(__builtin_fmaf(sc[kb][v], c, -m_use));
              sc[kb][v] = pw;
              rs += pw;
              if (v & 1) {
                pb[kb][v >> 3][(v & 7) - 1] = (T)sc[kb][v - 1];
                pb[kb][v >> 3][v & 7] = (T)pw;
              }
              if ((v & 7) == 7) lh_run = E::sum8(pb[kb][v >> 3], lh_run);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        l_run += rs;

        // P.V of tile kt; rows that see at most one tile of keys also add
        // the rounding remainder of P (as in the loop above)
        if (kbase < C::BN && lim_w <= C::BN) {
          keep_branch();
          v8 pl[C::NKB_][2];
#pragma unroll
          for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
              for (int j = 0; j < 8; ++j)
                pl[kb][a2][j] = (T)(sc[kb][8 * a2 + j] - (float)pb[kb][a2][j]);
#pragma unroll
          for (int kb = 0; kb < C::NKB_; ++kb)
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2) lh_run = E::sum8(pl[kb][a2], lh_run);
          pv_tile(Vs, pl, [](int) {});
        }
        // P.V of tile kt with the row max of tile kt + 1 (one score per
        // product); then the rescale, if any, before the weights of kt + 1
        mask_tile(sn, kbase + C::BN);
        float mx = -INFINITY;
        pv_tile(Vs, pb, [&](int i) __attribute__((always_inline)) {
          constexpr int NSC = 16 * C::NKB_;
          constexpr int NPV = C::DB * C::NKB_ * 2;
          constexpr int SPP = (NSC + NPV - 1) / NPV;
#pragma unroll
          for (int u = 0; u < SPP; ++u)
            if (i * SPP + u < NSC) mx = fmaxf(mx, sn[(i * SPP + u) / 16][(i * SPP + u) % 16]);
        });
        m_use = settle_max(mx, kt + 1 < kt_end);
#pragma unroll
        for (int kb = 0; kb < C::NKB_; ++kb) sc[kb] = sn[kb];
      }
    } else {
      // key-range form with one workgroup per CU: the plain loop
      for (int kt = kt_begin; kt < kt_end; ++kt) tile_step(kt, (kt - kt_begin) & 1);
    }

    // epilogue: normalise, LSE, stage O through LDS, full-row stores
    const float l_tot = sum_across_halves(l_run);
    const float lh_tot = sum_across_halves(lh_run);
    const bool dead = (l_tot == 0.f);
    const float inv = dead ? 0.f : 1.f / lh_tot;
    const float lse = dead ? -INFINITY : (m_run + log2f(l_tot)) * 0.69314718055994530942f;
    if (partial) {
      // split-K chunk: FP32 O (normalised over the chunk) and LSE of chunk
      // split_j, straight from the registers
      if (row < uq) {
        float* po = a.ws.part_o +
                    (((int64_t)split_j * a.g.total_q + q0 + row) * a.g.hq + head) * DV;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            f32x4 ov;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) ov[cc] = o[db][4 * a4 + cc] * inv;
            *reinterpret_cast<f32x4*>(po + db * 32 + 8 * a4 + 4 * hh) = ov;
          }
        if (hh == 0)
          a.ws.part_lse[((int64_t)split_j * a.g.hq + head) * a.g.total_q + q0 + row] = lse;
      }
      wait_vmem();      // loads past the last tile still write their stage
      __syncthreads();  // the next item's K/V loads reuse the stages
      continue;
    }
    __syncthreads();  // every wave is done with the K/V stages
    T* Os = reinterpret_cast<T*>(lds) + wave * 32 * C::OP;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        v4 ov;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) ov[cc] = (T)(o[db][4 * a4 + cc] * inv);
        *reinterpret_cast<v4*>(Os + r32 * C::OP + db * 32 + 8 * a4 + 4 * hh) = ov;
      }
    // The LSE store follows the staging writes: the wait that orders those
    // writes after the last tile's LDS-DMA then does not wait for it.
    if (hh == 0 && row < uq) a.lse[(int64_t)head * a.g.total_q + q0 + row] = lse;
    __syncthreads();
    {
      T* obase = static_cast<T*>(a.out) + ((int64_t)q0 * a.g.hq + head) * DV;
      const auto orr = make_rsrc(obase, uq > 0 ? (uint32_t)(uq - 1) * ostride + DV * 2 : 0u);
#pragma unroll
      for (int it = 0; it < DV / 16; ++it) {
        const int idx = it * 64 + lane;
        const int r = idx / C::CHV, ch = idx % C::CHV;
        const u32x4 val = *reinterpret_cast<const u32x4*>(Os + r * C::OP + 8 * ch);
        buf_store16_nt(orr, (uint32_t)(wr0 + r) * ostride + ch * 16, val);
      }
    }
    __syncthreads();  // staging area is reused by the next item's K/V loads
  }
}

template <typename T, int DQ, int DV, int GF, int RB>
hipError_t launch_one(const FwdArgs& a, int64_t max_work, hipStream_t s) {
  constexpr int NKB = (DQ <= 128 && DV <= 128) ? 1 : 2;
  using C = Cfg<DQ, DV, GF, RB, NKB>;
  auto kern = (a.g.kr_off != nullptr) ? fwd_mfma_kernel<T, DQ, DV, GF, RB, NKB, true>
                                      : fwd_mfma_kernel<T, DQ, DV, GF, RB, NKB, false>;
  const int grid = persistent_grid(reinterpret_cast<const void*>(kern), C::NT, max_work);
  if (grid <= 0) return grid == 0 ? hipSuccess : hipErrorInvalidValue;
  FwdArgs args = a;
  args.n_cu = device_cu_count();
  if (args.n_cu <= 0) return hipErrorInvalidValue;
  return launch_kernel(kern, dim3(grid), dim3(C::NT), s, args);
}

template <typename T, int DQ, int DV>
hipError_t launch_d(const FwdArgs& a, const TileShape& t, int64_t max_work, hipStream_t s,
                    bool* ok) {
  *ok = true;
  switch (t.gf) {
    case 4: return launch_one<T, DQ, DV, 4, 1>(a, max_work, s);
    case 3: return launch_one<T, DQ, DV, 3, 1>(a, max_work, s);
    case 2: return launch_one<T, DQ, DV, 2, 2>(a, max_work, s);
    case 1: return launch_one<T, DQ, DV, 1, 4>(a, max_work, s);
    default: *ok = false; return hipSuccess;
  }
}

template <typename T, int DQ>
hipError_t launch_dq(const FwdArgs& a, const TileShape& t, int64_t max_work, hipStream_t s,
                     bool* supported) {
  switch (a.g.dv) {
    case 64: return launch_d<T, DQ, 64>(a, t, max_work, s, supported);
    case 128: return launch_d<T, DQ, 128>(a, t, max_work, s, supported);
    case 256: return launch_d<T, DQ, 256>(a, t, max_work, s, supported);
    default: *supported = false; return hipSuccess;
  }
}

template <typename T>
hipError_t launch_t(const FwdArgs& a, const TileShape& t, int64_t max_work, hipStream_t s,
                    bool* supported) {
  switch (a.g.d) {
    case 64: return launch_dq<T, 64>(a, t, max_work, s, supported);
    case 128: return launch_dq<T, 128>(a, t, max_work, s, supported);
    case 256: return launch_dq<T, 256>(a, t, max_work, s, supported);
    default: *supported = false; return hipSuccess;
  }
}

}  // namespace

hipError_t launch_fwd_mfma(const FwdArgs& a, int dtype, const TileShape& t, int64_t max_work,
                           hipStream_t s, bool* supported) {
  if (dtype == GVATTN_BF16) return launch_t<__bf16>(a, t, max_work, s, supported);
  if (dtype == GVATTN_FP16) return launch_t<_Float16>(a, t, max_work, s, supported);
  *supported = false;
  return hipSuccess;
}

}  // namespace gvattn
