"""Seeded synthetic inputs for segmented ("gapped") varlen attention.

This module only draws inputs: segment geometry, Q/K/V values and the
sentinel-prefilled output buffers.  It holds none of the attention
arithmetic, so both the HIP path and the FP64 oracle can consume what it
produces without sharing any code of the method.

Recipe (one seed per workload):
  * ``numpy.random.default_rng(seed)`` draws the segment lengths first;
  * Q, then K, then V are drawn as float32 normals in fixed chunks of
    ``CHUNK`` elements; chunk ``c`` of tensor ``t`` uses its own generator
    ``default_rng([seed, t, c])`` so the values do not depend on how many
    threads fill the tensor;
  * bf16 and fp16 workloads round the float32 draws to that type with
    round-to-nearest-even (the values kept in float32 are then exactly
    representable in it);
  * output and LSE buffers are prefilled with the sentinel 7.0 so untouched
    gap rows can be checked bit for bit.

Shapes follow the workloads the pages describe: Cosmos3 text cross-attention
with right-padded text whose pad slots are exactly zero (TensorRT-LLM issue
#18687, "Reproduction" step 3), causal gapped replay and multiview joint
attention with visibility partitions (cosmos-framework PR #312, "Problem and
behavior"; PR #302, "What").
"""

from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

SENTINEL = 7.0
CHUNK = 1 << 22

FP32 = "fp32"
BF16 = "bf16"
FP16 = "fp16"


def _pool_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32.

    NaN and infinities are not expected in the draws; they pass through the
    integer arithmetic unchanged in class (a NaN stays NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    bits = (bits + 0x7FFF + lsb) >> 16
    out = (bits.astype(np.uint32) << 16).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def round_to_fp16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest IEEE binary16 value (ties to even, overflow to
    infinity), returned as float32."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_to(dtype: str, x: np.ndarray) -> np.ndarray:
    """Round float32 values to the element type ``dtype`` (returned as float32)."""
    if dtype == BF16:
        return round_to_bf16(x)
    if dtype == FP16:
        return round_to_fp16(x)
    return np.asarray(x, dtype=np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are exactly bf16 (no rounding)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def normal_tensor(seed: int, tensor_id: int, shape, std: float = 1.0,
                  dtype: str = BF16, threads: int | None = None) -> np.ndarray:
    """Chunked, thread-count independent N(0, std^2) float32 draw.

    Each chunk of ``CHUNK`` elements comes from ``default_rng([seed,
    tensor_id, chunk])``; every value is then rounded to ``dtype``."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.default_rng([seed, tensor_id, c])
        vals = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            vals *= np.float32(std)
        out[lo:hi] = round_to(dtype, vals)

    threads = threads or _pool_threads()
    if nchunks <= 1 or threads == 1:
        for c in range(nchunks):
            fill(c)
    else:
        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


@dataclasses.dataclass
class Geometry:
    """Packed-segment description, as the kernels take it.

    ``cu_q``/``cu_k`` are the segment start offsets (int32, nseg+1 entries;
    the capacity of segment s is ``cu[s+1]-cu[s]``), ``used_q``/``used_k`` the
    used prefix of each segment (seqused_q / seqused_k)."""
    cu_q: np.ndarray
    cu_k: np.ndarray
    used_q: np.ndarray
    used_k: np.ndarray
    hq: int
    hkv: int
    d: int
    dv: int
    causal: bool
    dtype: str
    total_q: int
    total_k: int

    @property
    def nseg(self) -> int:
        return int(self.used_q.shape[0])

    @property
    def scale(self) -> np.float32:
        """1/sqrt(d) rounded to float32, the value both sides use."""
        return np.float32(1.0) / np.sqrt(np.float32(self.d))

    def with_keys(self, cu_k: np.ndarray, used_k: np.ndarray) -> "Geometry":
        return dataclasses.replace(self, cu_k=np.asarray(cu_k, np.int32),
                                   used_k=np.asarray(used_k, np.int32))


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    geom: Geometry
    q: np.ndarray  # [total_q, hq, d] float32 (bf16-exact for bf16)
    k: np.ndarray  # [total_k, hkv, d]
    v: np.ndarray  # [total_k, hkv, dv]
    partitions: list | None = None  # list of (cu_k, used_k) key partitions
    note: str = ""
    # key-range form: (kr_off [nseg+1], kr_start [n], kr_len [n]) int32
    key_ranges: tuple | None = None

    def out_init(self) -> np.ndarray:
        g = self.geom
        return np.full((g.total_q, g.hq, g.dv), SENTINEL, dtype=np.float32)

    def lse_init(self) -> np.ndarray:
        g = self.geom
        return np.full((g.hq, g.total_q), SENTINEL, dtype=np.float32)


def _offsets(caps) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(caps, np.int64))]).astype(np.int32)


def make_geometry(caps_q, caps_k, used_q, used_k, hq, hkv, d, causal,
                  dtype=BF16, dv=None) -> Geometry:
    cu_q, cu_k = _offsets(caps_q), _offsets(caps_k)
    return Geometry(cu_q=cu_q, cu_k=cu_k,
                    used_q=np.asarray(used_q, np.int32),
                    used_k=np.asarray(used_k, np.int32),
                    hq=hq, hkv=hkv, d=d, dv=dv or d, causal=bool(causal),
                    dtype=dtype, total_q=int(cu_q[-1]), total_k=int(cu_k[-1]))


def fill_qkv(geom: Geometry, seed: int, std: float = 1.0, threads=None):
    dt = geom.dtype
    q = normal_tensor(seed, 0, (geom.total_q, geom.hq, geom.d), std, dt, threads)
    k = normal_tensor(seed, 1, (geom.total_k, geom.hkv, geom.d), std, dt, threads)
    v = normal_tensor(seed, 2, (geom.total_k, geom.hkv, geom.dv), std, dt, threads)
    return q, k, v


# --- the five workloads -----------------------------------------------------

def fp32_three_segments() -> Workload:
    """FP32, 3 segments of capacity 64; used q {40,64,13}, used k {50,0,64};
    8 q heads / 2 KV heads, d=64; the middle segment has no keys."""
    seed = 1  # lengths are fixed; only Q/K/V are drawn
    g = make_geometry([64] * 3, [64] * 3, [40, 64, 13], [50, 0, 64], 8, 2, 64,
                      causal=False, dtype=FP32)
    q, k, v = fill_qkv(g, seed)
    return Workload("fp32_gapped_3seg_d64", seed, g, q, k, v,
                    note="segment index 1 has zero keys")


def cfg_cross_attention() -> Workload:
    """BF16 CFG cross-attention, batch 2: 4096 video queries per sample attend
    right-padded text K/V of capacity 4096 with real lengths 24 and 700; pad
    K/V slots are exactly zero; 32 q heads / 8 KV heads, d=128."""
    seed = 2
    text_lens = [24, 700]
    g = make_geometry([4096, 4096], [4096, 4096], [4096, 4096], text_lens,
                      32, 8, 128, causal=False)
    q, k, v = fill_qkv(g, seed)
    for s, L in enumerate(text_lens):
        k0 = int(g.cu_k[s])
        k[k0 + L:k0 + 4096] = 0.0
        v[k0 + L:k0 + 4096] = 0.0
    return Workload("bf16_cfg_cross_attn_b2", seed, g, q, k, v,
                    note="pad-slot K/V exactly zero (text LLM zeroes pad rows)")


def causal_replay_lengths(seed: int = 3, nseg: int = 64, cap: int = 2048):
    rng = np.random.default_rng(seed)
    uq = rng.integers(0, cap, size=nseg, endpoint=True).astype(np.int32)
    uk = rng.integers(0, cap, size=nseg, endpoint=True).astype(np.int32)
    empty = rng.choice(nseg, size=4, replace=False)
    uk[empty] = 0
    return uq, uk


def causal_replay() -> Workload:
    """BF16 causal gapped replay: 64 segments of capacity 2048, used q and k
    lengths uniform in [0, 2048] with 4 segments forced to zero keys; causal
    mask aligned bottom-right in each segment; 32 q heads / 8 KV heads, d=128."""
    seed = 3
    uq, uk = causal_replay_lengths(seed)
    g = make_geometry([2048] * 64, [2048] * 64, uq, uk, 32, 8, 128, causal=True)
    q, k, v = fill_qkv(g, seed)
    return Workload("bf16_causal_replay_64x2048", seed, g, q, k, v)


def multiview_partitions() -> Workload:
    """BF16 multiview joint attention: 8 segments (7 camera views + 1 LiDAR
    stream) with 8190 used query rows and 32760 keys each, keys split into
    visibility partition A (first 16380) and B (the rest); 24 q heads / 8 KV
    heads, d=128.  ``geom`` describes the single pass over all keys."""
    seed = 4
    nseg, nq, nk, half = 8, 8190, 32760, 16380
    g = make_geometry([nq] * nseg, [nk] * nseg, [nq] * nseg, [nk] * nseg,
                      24, 8, 128, causal=False)
    q, k, v = fill_qkv(g, seed)
    starts = np.arange(nseg, dtype=np.int64) * nk
    cu_a = np.concatenate([starts, [nseg * nk]]).astype(np.int32)
    cu_b = np.concatenate([starts + half, [nseg * nk]]).astype(np.int32)
    used = np.full(nseg, half, np.int32)
    return Workload("bf16_multiview_2part_8x8190", seed, g, q, k, v,
                    partitions=[(cu_a, used), (cu_b, used.copy())])


def large_head_lengths(seed: int = 5, nseg: int = 16, cap: int = 16384):
    rng = np.random.default_rng(seed)
    uq = rng.integers(cap // 2, cap, size=nseg, endpoint=True).astype(np.int32)
    uk = rng.integers(0, cap, size=nseg, endpoint=True).astype(np.int32)
    return uq, uk


def large_head_d256() -> Workload:
    """BF16 large-head gapped varlen attention, non-causal: 16 segments of
    capacity 16384, used q uniform in [8192, 16384], used k uniform in
    [0, 16384]; 16 q heads / 4 KV heads, d=256; values N(0, 0.5^2)."""
    seed = 5
    uq, uk = large_head_lengths(seed)
    g = make_geometry([16384] * 16, [16384] * 16, uq, uk, 16, 4, 256, causal=False)
    q, k, v = fill_qkv(g, seed, std=0.5)
    return Workload("bf16_d256_gapped_16x16384", seed, g, q, k, v)


WORKLOADS = {"fp32_three_segments": fp32_three_segments, "cfg_cross_attention": cfg_cross_attention,
             "causal_replay": causal_replay, "multiview_partitions": multiview_partitions,
             "large_head_d256": large_head_d256}


def ulysses_joint(seed: int = 6, ranks: int = 2, text_cap: int = 4096, video: int = 4096,
                  text_lens=(24, 700), nq: int = 4096, hq: int = 32, hkv: int = 8,
                  d: int = 128, dtype: str = BF16) -> Workload:
    """CFG batch of 2 under Ulysses sequence parallelism (issue #18687,
    "additional notes", possible fix 1): each sample's keys arrive rank-major, rank r
    holding text rows [r*T/R, (r+1)*T/R) of the padded text and video rows
    [r*V/R, (r+1)*V/R).  The valid keys of sample b are, per rank, the real
    text rows of that chunk (text_lens[b] in total, pad slots exactly zero)
    and the whole video chunk: 2*ranks key ranges per sample.  ``nq`` video
    queries per sample attend them (non-causal)."""
    tr, vr = text_cap // ranks, video // ranks
    chunk = tr + vr
    per_sample = ranks * chunk
    nseg = len(text_lens)
    g = make_geometry([nq] * nseg, [per_sample] * nseg, [nq] * nseg, [0] * nseg, hq, hkv, d,
                      causal=False, dtype=dtype)
    q, k, v = fill_qkv(g, seed)
    starts, lens, off = [], [], [0]
    for b, L in enumerate(text_lens):
        base = b * per_sample
        for r in range(ranks):
            c0 = base + r * chunk
            real = max(0, min(tr, L - r * tr))
            k[c0 + real:c0 + tr] = 0.0
            v[c0 + real:c0 + tr] = 0.0
            starts += [c0, c0 + tr]
            lens += [real, vr]
        off.append(len(starts))
    ranges = (np.asarray(off, np.int32), np.asarray(starts, np.int32),
              np.asarray(lens, np.int32))
    name = f"{dtype}_ulysses{ranks}_joint_b{nseg}_{nq}q_text{text_cap}_video{video}"
    return Workload(name, seed, g, q, k, v, key_ranges=ranges,
                    note="rank-major keys; pad-slot K/V exactly zero")


def decode_batch(seed: int = 7, batch: int = 32, new_tokens: int = 4, k_lo: int = 4096,
                 k_hi: int = 16384, hq: int = 32, hkv: int = 8, d: int = 128,
                 dtype: str = BF16) -> Workload:
    """Decode-like launch (few query rows, long keys): ``batch`` segments of
    ``new_tokens`` query rows each attend their cache of U{k_lo..k_hi} keys,
    bottom-right causal.  Too few query tiles to fill the GPU: the plan
    splits the key ranges (split-K)."""
    rng = np.random.default_rng(seed)
    uk = rng.integers(k_lo, k_hi, size=batch, endpoint=True)
    g = make_geometry([new_tokens] * batch, uk, [new_tokens] * batch, uk, hq, hkv, d,
                      causal=True, dtype=dtype)
    q, k, v = fill_qkv(g, seed)
    return Workload(f"{dtype}_decode_b{batch}x{new_tokens}_k{k_lo}_{k_hi}", seed, g, q, k, v)


def random_ranges(rng, nseg: int, total_k: int, max_ranges: int = 4, max_len: int = 80):
    """Seeded key ranges for parity sweeps: 0..max_ranges ranges per segment,
    lengths 0..max_len (some empty), starts anywhere in [0, total_k - len];
    ranges may overlap and come in any order."""
    counts = rng.integers(0, max_ranges + 1, size=nseg)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n = int(off[-1])
    lens = rng.integers(0, max_len + 1, size=n)
    lens[rng.random(n) < 0.15] = 0
    lens = np.minimum(lens, total_k)
    starts = np.array([rng.integers(0, total_k - L + 1) for L in lens], dtype=np.int64)
    return off, starts.astype(np.int32), lens.astype(np.int32)


def random_small(seed: int, nseg: int, cap_q: int, cap_k: int, hq: int, hkv: int,
                 d: int, causal: bool, dtype: str = BF16, lengths=None,
                 std: float = 1.0, dv: int | None = None) -> Workload:
    """Small seeded geometry for parity sweeps.  ``lengths`` may fix
    (used_q, used_k); otherwise both are uniform in [0, cap].  ``dv`` is the
    V/O head dim (default d)."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        uq = rng.integers(0, cap_q, size=nseg, endpoint=True)
        uk = rng.integers(0, cap_k, size=nseg, endpoint=True)
    else:
        uq, uk = lengths
    g = make_geometry([cap_q] * nseg, [cap_k] * nseg, uq, uk, hq, hkv, d,
                      causal=causal, dtype=dtype, dv=dv)
    q, k, v = fill_qkv(g, seed + 1000, std=std)
    return Workload(f"small_s{seed}", seed, g, q, k, v)
