// BF16 segmented varlen attention forward on gfx950 matrix cores.
//
// What it computes: cosmos-framework PR #302, "What" (used prefixes of each
// segment, untouched gap rows, zero output / -inf LSE without keys);
// TensorRT-LLM issue #18687, "actual behavior" (keys past the used length
// are masked, never attended as zeros); PR #312, "Problem and behavior"
// (GQA folding, FP32 LSE).
//
// Design (gfx950):
//   * A persistent grid walks the plan's tile list (segment, first row),
//     longest first; work item = (tile, chunk of GF query heads that share
//     one KV head).  One wave owns 32 query rows of one head.
//   * Scores are computed transposed, S^T = K . Q^T, with
//     v_mfma_f32_32x32x16_bf16: K comes from LDS (row-major), Q stays in
//     registers for the whole tile.  Each lane then holds 32 of the 64 keys
//     of one query row, so the row max needs a single cross-lane exchange
//     and the row sum none until the end.
//   * The probabilities feed O^T += V^T . P^T directly from the score
//     registers (no shuffle): V is written to LDS transposed with its keys
//     permuted inside each 16-key block so every lane reads its 8 keys with
//     one 16-byte LDS load.
//   * Online softmax in the exp2 domain, FP32 row max / sum, FP32 LSE.
//   * Every global access goes through a buffer resource whose size ends
//     at the segment's last used row: loads past it return zero (ragged key
//     tiles, gap rows, buffer ends) and stores past it are dropped (gap rows
//     of O stay bit-exact).  Key-padding and causal masks are applied to the
//     scores as -inf on boundary tiles only.
//   * The next K/V tile is prefetched into registers while the current one
//     is computed; O leaves through LDS so global stores are full rows.
#include <math.h>

#include "gvattn_internal.h"

namespace gvattn {
namespace {

using namespace dev;

template <int D, int GF, int RB>
struct Cfg {
  static constexpr int NW = GF * RB;          // waves per workgroup
  static constexpr int NT = 64 * NW;          // threads
  static constexpr int BN = kKeyTile;         // keys per tile
  static constexpr int KP = D + 8;            // K row pitch in LDS (elements)
  static constexpr int VP = BN + 8;           // V^T row pitch in LDS
  static constexpr int OP = D + 8;            // O staging row pitch
  static constexpr int LDS_KV = BN * KP + D * VP;
  static constexpr int LDS_O = NW * 32 * OP;
  static constexpr int LDS = LDS_KV > LDS_O ? LDS_KV : LDS_O;
  static constexpr int CH = D / 8;            // 16-byte chunks per row
  static constexpr int UNITS = (BN / 4) * CH; // (key quad, chunk) per tile
  static constexpr int UPT = (UNITS + NT - 1) / NT;
  static constexpr int KK = D / 16;           // k-steps of the score MFMA
  static constexpr int DB = D / 32;           // 32-wide d blocks of O
};

// Position of key kappa (0..63) inside the V^T row: inside each 16-key
// block the 4-key quads are stored in the order 0, 2, 1, 3.
__device__ __forceinline__ int vt_pos(int kappa) {
  const int blk = kappa >> 4, qd = (kappa >> 2) & 3;
  const int pq = ((qd & 1) << 1) | (qd >> 1);
  return (blk << 4) | (pq << 2) | (kappa & 3);
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo_src, uint32_t hi_src, int upper) {
  const uint32_t a = upper ? (lo_src >> 16) : (lo_src & 0xffffu);
  const uint32_t b = upper ? (hi_src & 0xffff0000u) : (hi_src << 16);
  return a | b;
}

template <int D, int GF, int RB>
__global__ __launch_bounds__((Cfg<D, GF, RB>::NT)) void fwd_bf16_kernel(FwdArgs a) {
  using C = Cfg<D, GF, RB>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[C::LDS];
  __bf16* Ks = lds;
  __bf16* Vt = lds + C::BN * C::KP;

  const PlanHeader* hdr = a.ws.header;
  if (hdr->key != a.key) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(&a.ws.header->err, GVATTN_DEVERR_PLAN);
    return;
  }
  const int n_tiles = hdr->n_tiles;
  const int n_hc = a.n_head_chunks;
  const int64_t n_work = (int64_t)n_tiles * n_hc;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r32 = lane & 31, hh = lane >> 5;
  const int hf = wave % GF, rb = wave / GF;
  const int G = a.g.hq / a.g.hkv;
  const uint32_t qstride = (uint32_t)a.g.hq * D * 2;    // bytes between rows
  const uint32_t kstride = (uint32_t)a.g.hkv * D * 2;
  const float c = a.scale_log2;

  for (int64_t w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int t = (int)(w / n_hc);
    const int hc = (int)(w - (int64_t)t * n_hc);
    const int2 tile = a.ws.tiles[t];
    const int seg = tile.x, row0 = tile.y;
    const int head0 = hc * GF;
    const int head = head0 + hf;
    const int kvh = head0 / G;
    const int q0 = a.g.cu_q[seg], k0 = a.g.cu_k[seg];
    const int uq = a.g.used_q[seg], uk = a.g.used_k[seg];
    const int wr0 = row0 + rb * 32;                 // first row of this wave
    const int r_last = min(row0 + 32 * RB, uq) - 1;  // last used row of the tile
    int kend = uk;
    if (a.g.causal) kend = max(0, min(uk, r_last + uk - uq + 1));
    const int n_kt = (kend + C::BN - 1) / C::BN;

    // buffer resources limited to the used rows of this segment/head
    const __bf16* qbase = static_cast<const __bf16*>(a.q) + ((int64_t)q0 * a.g.hq + head) * D;
    const uint32_t qbytes = uq > 0 ? (uint32_t)(uq - 1) * qstride + D * 2 : 0u;
    const auto qr = make_rsrc(qbase, qbytes);
    const int64_t kvoff = ((int64_t)k0 * a.g.hkv + kvh) * D;
    const uint32_t kbytes = uk > 0 ? (uint32_t)(uk - 1) * kstride + D * 2 : 0u;
    const auto kr = make_rsrc(static_cast<const __bf16*>(a.k) + kvoff, kbytes);
    const auto vr = make_rsrc(static_cast<const __bf16*>(a.v) + kvoff, kbytes);

    // Q fragment: lane holds Q[wr0 + r32][16*kk + 8*hh .. +7]
    bf16x8 qf[C::KK];
    {
      const uint32_t roff = (uint32_t)(wr0 + r32) * qstride + hh * 16;
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk)
        qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(qr, roff + kk * 32));
    }

    f32x16 o[C::DB];
#pragma unroll
    for (int i = 0; i < C::DB; ++i) o[i] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    const int row = wr0 + r32;                       // this lane's query row
    const int lim = a.g.causal ? min(uk, row + uk - uq + 1) : uk;
    const int lim_w = a.g.causal ? min(uk, wr0 + uk - uq + 1) : uk;  // wave minimum

    u32x4 kreg[C::UPT][4], vreg[C::UPT][4];
    auto gload = [&](int kt) {
#pragma unroll
      for (int u = 0; u < C::UPT; ++u) {
        const int unit = tid + u * C::NT;
        if (unit < C::UNITS) {
          const int p = unit / C::CH, ch = unit % C::CH;
          const uint32_t off = (uint32_t)(kt * C::BN + 4 * p) * kstride + ch * 16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            kreg[u][r] = buf_load16(kr, off + r * kstride);
            vreg[u][r] = buf_load16(vr, off + r * kstride);
          }
        }
      }
    };
    auto lstore = [&]() {
#pragma unroll
      for (int u = 0; u < C::UPT; ++u) {
        const int unit = tid + u * C::NT;
        if (unit < C::UNITS) {
          const int p = unit / C::CH, ch = unit % C::CH;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            *reinterpret_cast<u32x4*>(Ks + (4 * p + r) * C::KP + 8 * ch) = kreg[u][r];
          const int pos = vt_pos(4 * p);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int dw = j >> 1, up = j & 1;
            u32x2 pr;
            pr[0] = pack2(vreg[u][0][dw], vreg[u][1][dw], up);
            pr[1] = pack2(vreg[u][2][dw], vreg[u][3][dw], up);
            *reinterpret_cast<u32x2*>(Vt + (8 * ch + j) * C::VP + pos) = pr;
          }
        }
      }
    };

    if (n_kt > 0) gload(0);
    for (int kt = 0; kt < n_kt; ++kt) {
      __syncthreads();
      lstore();
      __syncthreads();
      if (kt + 1 < n_kt) gload(kt + 1);

      // S^T = K . Q^T for two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const __bf16* kp = Ks + (kb * 32 + r32) * C::KP + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kp + 16 * kk);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[kb], 0, 0, 0);
        }
      }

      // key-padding / causal mask on boundary tiles
      const int kbase = kt * C::BN;
      if (kbase + C::BN > lim_w) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kbase + kb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
            if (key >= lim) s[kb][v] = -INFINITY;
          }
      }

      // online softmax (exp2 domain)
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx * c);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = exp2_fast(__builtin_fmaf(s[kb][v], c, -m_use));
          s[kb][v] = p;
          rs += p;
        }
      l_run = l_run * alpha + rs;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < C::DB; ++i) o[i] *= alpha;
      }

      // P^T as bf16 MFMA operands straight from the score registers
      bf16x8 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[kb][a2][j] = (__bf16)s[kb][8 * a2 + j];

      // O^T += V^T . P^T
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const __bf16* vp = Vt + (db * 32 + r32) * C::VP + 8 * hh;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int a2 = 0; a2 < 2; ++a2) {
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(vp + kb * 32 + a2 * 16);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb][a2], o[db], 0, 0, 0);
          }
      }
    }

    // epilogue: normalise, LSE, stage O through LDS, full-row stores
    const float l_tot = l_run + swap_halves(l_run);
    const bool dead = (l_tot == 0.f);
    const float inv = dead ? 0.f : 1.f / l_tot;
    if (hh == 0 && row < uq) {
      const float lse = dead ? -INFINITY : (m_run + log2f(l_tot)) * 0.69314718055994530942f;
      a.lse[(int64_t)head * a.g.total_q + q0 + row] = lse;
    }
    __syncthreads();
    __bf16* Os = lds + wave * 32 * C::OP;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 ov;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) ov[cc] = (__bf16)(dead ? 0.f : o[db][4 * a4 + cc] * inv);
        *reinterpret_cast<bf16x4*>(Os + r32 * C::OP + db * 32 + 8 * a4 + 4 * hh) = ov;
      }
    __syncthreads();
    {
      __bf16* obase = static_cast<__bf16*>(a.out) + ((int64_t)q0 * a.g.hq + head) * D;
      const auto orr = make_rsrc(obase, qbytes);
#pragma unroll
      for (int it = 0; it < D / 16; ++it) {
        const int idx = it * 64 + lane;
        const int r = idx / C::CH, ch = idx % C::CH;
        const u32x4 val = *reinterpret_cast<const u32x4*>(Os + r * C::OP + 8 * ch);
        buf_store16(orr, (uint32_t)(wr0 + r) * qstride + ch * 16, val);
      }
    }
    __syncthreads();
  }
}

template <int D, int GF, int RB>
hipError_t launch_one(const FwdArgs& a, int64_t max_work, hipStream_t s) {
  using C = Cfg<D, GF, RB>;
  auto kern = fwd_bf16_kernel<D, GF, RB>;
  const int grid = persistent_grid(reinterpret_cast<const void*>(kern), C::NT, max_work);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, const TileShape& t, int64_t max_work, hipStream_t s,
                    bool* ok) {
  *ok = true;
  switch (t.gf) {
    case 4: return launch_one<D, 4, 1>(a, max_work, s);
    case 3: return launch_one<D, 3, 1>(a, max_work, s);
    case 2: return launch_one<D, 2, 2>(a, max_work, s);
    case 1: return launch_one<D, 1, 4>(a, max_work, s);
    default: *ok = false; return hipSuccess;
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, const TileShape& t, int64_t max_work,
                           hipStream_t s, bool* supported) {
  switch (a.g.d) {
    case 64: return launch_d<64>(a, t, max_work, s, supported);
    case 128: return launch_d<128>(a, t, max_work, s, supported);
    case 256: return launch_d<256>(a, t, max_work, s, supported);
    default: *supported = false; return hipSuccess;
  }
}

}  // namespace gvattn
