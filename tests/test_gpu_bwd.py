"""GPU parity of the backward (gvattn_bwd) against the FP64 oracle's
gradients, through the C ABI.

Inputs: Q, K, V and dO seeded and rounded to the element type; O and LSE
are the oracle forward's (O rounded to the element type, LSE to fp32), so
nothing the checker sees comes from the HIP path.  Gap rows of Q, K, V, O,
dO and LSE hold NaN: they must never be read into a result.

Tolerance (derived, per element): the kernels round P (for dV), dS (for
dQ, dK) and O (inside D = rowsum(dO * O)) to the element type and
accumulate in FP32, so each gradient is within u * (|exact| + A) of the
exact one, A = oracle.attention_bwd_magnitudes (the absolute-value sums of
the rounded terms), u = 2^-8 for bf16 and 2^-11 for fp16; rounding the
result to the element type adds at most u * |result|.  The test allows
2u (|exact| + A) plus 1e-5 * max(A) for the FP32 terms.  Gap rows of dQ, dK
and dV stay bit-exact; rows that see no key and keys no row sees get 0.
"""

import numpy as np
import pytest

import oracle
from segmented_varlen_attention_amd import binding as B
from segmented_varlen_attention_amd import workloads as W

from gpu_util import DIMS_BWD, i32, random_geometry, say, to_np, torch, upload

pytestmark = pytest.mark.gpu

U = {W.BF16: 2.0 ** -8, W.FP16: 2.0 ** -11}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()
    yield


def used_mask(cu, used, total):
    m = np.zeros(total, dtype=bool)
    for s in range(len(used)):
        m[cu[s]:cu[s] + used[s]] = True
    return m


def make_inputs(wl, seed):
    """dO, and the oracle forward's O / LSE, with NaN in every gap row."""
    g = wl.geom
    o, l = oracle.attention_fwd(wl.q, wl.k, wl.v, g.cu_q, g.cu_k, g.used_q, g.used_k,
                                float(g.scale), g.causal, workers=8)
    o = W.round_to(g.dtype, o.astype(np.float32))
    l = l.astype(np.float32)
    do = W.normal_tensor(seed, 7, (g.total_q, g.hq, g.dv), 1.0, g.dtype)
    mq = used_mask(g.cu_q, g.used_q, g.total_q)
    mk = used_mask(g.cu_k, g.used_k, g.total_k)
    q, k, v = wl.q.copy(), wl.k.copy(), wl.v.copy()
    for x in (q, o, do):
        x[~mq] = np.nan
    l[:, ~mq] = np.nan
    k[~mk] = np.nan
    v[~mk] = np.nan
    return q, k, v, o, l, do, mq, mk


def run_bwd(wl, q, k, v, o, l, do):
    t = torch()
    g = wl.geom
    q_, k_, v_ = upload(q, g), upload(k, g), upload(v, g)
    o_, do_ = upload(o, g), upload(do, g)
    l_ = t.from_numpy(np.ascontiguousarray(l)).to("cuda")
    dq = t.full_like(q_, W.SENTINEL)
    dk = t.full_like(k_, W.SENTINEL)
    dv = t.full_like(v_, W.SENTINEL)
    ws = B.gvattn_bwd(q_, k_, v_, o_, do_, l_, i32(g.cu_q), i32(g.cu_k), i32(g.used_q),
                      i32(g.used_k), dq, dk, dv, float(g.scale), g.causal)
    assert B.gvattn_read_device_error(ws) == 0
    return dq, dk, dv


def gap_untouched(x, mask):
    t = torch()
    gap = t.from_numpy(~mask).to("cuda")
    sent = t.tensor(W.SENTINEL, dtype=x.dtype, device="cuda").view(t.int16)
    return bool((x[gap].view(t.int16) == sent).all().item())


def check_grad(got, want, mag, mask, dtype, name):
    got = got[mask].astype(np.float64)
    want, mag = want[mask], mag[mask]
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - want)
    bound = 2 * U[dtype] * (np.abs(want) + mag) + 1e-5 * float(mag.max(initial=0.0))
    ratio = float(np.max(err / np.maximum(bound, 1e-30), initial=0.0))
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(want), 1e-30))
    st = {"max_err": float(err.max(initial=0.0)), "bound_ratio": ratio, "rel_fro": rel}
    assert np.all(err <= bound), f"{name}: error beyond the derived bound {st}"
    return st


def check_case(wl, seed, where):
    g = wl.geom
    q, k, v, o, l, do, mq, mk = make_inputs(wl, seed)
    dq, dk, dv = run_bwd(wl, q, k, v, o, l, do)
    assert gap_untouched(dq, mq), f"{where}: gap rows of dQ changed"
    assert gap_untouched(dk, mk), f"{where}: gap rows of dK changed"
    assert gap_untouched(dv, mk), f"{where}: gap rows of dV changed"
    args = (wl.q, wl.k, wl.v, do, g.cu_q, g.cu_k, g.used_q, g.used_k, float(g.scale), g.causal)
    rq, rk, rv = oracle.attention_bwd(*args)
    aq, ak, av = oracle.attention_bwd_magnitudes(*args)
    st = {}
    for name, got, want, mag, m in (("dq", dq, rq, aq, mq), ("dk", dk, rk, ak, mk),
                                    ("dv", dv, rv, av, mk)):
        st[name] = check_grad(to_np(got), want, mag, m, g.dtype, f"{where} {name}")
    # rows without keys and keys without rows: exact zeros
    gq, gk = to_np(dq), to_np(dk)
    for s in range(g.nseg):
        q0, k0, uq, uk = int(g.cu_q[s]), int(g.cu_k[s]), int(g.used_q[s]), int(g.used_k[s])
        lim = oracle.visible_limit(np.arange(uq), uq, uk, g.causal)
        dead = q0 + np.nonzero(lim == 0)[0]
        assert np.all(gq[dead] == 0.0), f"{where}: dQ of rows without keys not zero"
        if uq == 0 and uk > 0:
            assert np.all(gk[k0:k0 + uk] == 0.0), f"{where}: dK of unseen keys not zero"
    say(f"[{where}]", st)
    return st


@pytest.mark.parametrize("dtype", [W.BF16, W.FP16])
@pytest.mark.parametrize("d,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_random(dtype, d, dv, causal):
    seed = 900 + d + dv // 2 + 7 * causal + (11 if dtype == W.FP16 else 0)
    rng = np.random.default_rng(seed)
    nseg = 5
    uq = rng.integers(0, 161, nseg)
    uk = rng.integers(0, 301, nseg)
    uq[1], uk[1] = 37, 0      # rows without keys
    uq[2], uk[2] = 0, 45      # keys without rows
    wl = W.random_small(seed, nseg, 160, 300, 8, 2, d, causal, dtype, lengths=(uq, uk), dv=dv)
    check_case(wl, seed, f"bwd {dtype} d{d} dv{dv} c{int(causal)}")


@pytest.mark.parametrize("seed", range(960, 972))
def test_bwd_random_geometries(seed):
    """Seeded random geometries: segment counts, independent query and key
    capacities (gaps, empty segments), GQA layouts, head dims, bf16 / fp16,
    causal or not, input spreads 0.5-2; every gradient element against the
    oracle."""
    wl, std = random_geometry(seed, DIMS_BWD, (W.BF16, W.FP16))
    g = wl.geom
    say(f"[bwd random] seed={seed} {g.dtype} d={g.d} dv={g.dv} hq={g.hq} hkv={g.hkv} "
        f"causal={g.causal} std={std} uq={g.used_q.tolist()} uk={g.used_k.tolist()}")
    check_case(wl, seed, f"bwd random seed {seed}")


@pytest.mark.parametrize("hq,hkv", [(4, 4), (6, 2), (12, 4), (8, 1)])
def test_bwd_head_folds(hq, hkv):
    """Every GQA fold of the dQ kernel (4, 3, 2 or 1 heads per workgroup) and
    dK / dV sums over groups of 1 to 8 query heads."""
    seed = 950 + hq + hkv
    rng = np.random.default_rng(seed)
    wl = W.random_small(seed, 4, 130, 200, hq, hkv, 128, True, W.BF16,
                        lengths=(rng.integers(1, 131, 4), rng.integers(1, 201, 4)))
    check_case(wl, seed, f"bwd heads {hq}/{hkv}")


def test_bwd_ragged_edges():
    """Lengths at and next to the tile sizes: 1, 31, 32, 33, 127, 128, 129
    rows and keys, used_k above and below used_q under bottom-right causal."""
    uq = np.array([1, 31, 32, 33, 127, 128, 129, 64])
    uk = np.array([129, 128, 33, 32, 31, 1, 127, 64])
    wl = W.random_small(960, len(uq), 129, 129, 8, 2, 128, True, W.BF16, lengths=(uq, uk))
    check_case(wl, 960, "bwd ragged causal")
    wl = W.random_small(961, len(uq), 129, 129, 8, 2, 64, False, W.FP16, lengths=(uq, uk))
    check_case(wl, 961, "bwd ragged noncausal")


@pytest.mark.parametrize("nseg", [600, 2500])
def test_bwd_many_segments(nseg):
    """Many short segments (capacity <= 40): with 2500 the plans read the
    segment table from global memory instead of LDS."""
    seed = 980 + nseg
    rng = np.random.default_rng(seed)
    cq, ck = rng.integers(0, 41, nseg), rng.integers(0, 41, nseg)
    uq = np.array([rng.integers(0, c + 1) for c in cq])
    uk = np.array([rng.integers(0, c + 1) for c in ck])
    g = W.make_geometry(cq, ck, uq, uk, 4, 2, 64, causal=True)
    q, k, v = W.fill_qkv(g, seed)
    check_case(W.Workload(f"bwd_many_{nseg}", seed, g, q, k, v), seed, f"bwd many {nseg}")


def test_bwd_deterministic():
    wl = W.random_small(970, 4, 100, 150, 8, 2, 128, True, W.BF16)
    q, k, v, o, l, do, _, _ = make_inputs(wl, 970)
    a = run_bwd(wl, q, k, v, o, l, do)
    b = run_bwd(wl, q, k, v, o, l, do)
    t = torch()
    for x, y in zip(a, b):
        assert t.equal(x.view(t.int16), y.view(t.int16))


def test_bwd_causal_replay_full_size_sampled():
    """The causal replay workload at full size (64 segments of capacity
    2048, 32 / 8 heads, d 128): the whole backward runs on the GPU; three
    segments (the longest, a short one and one with used_k < used_q) are
    checked against the oracle in full.  O / LSE of the checked segments are
    the oracle's; the rest come from the GPU forward (they only feed their
    own segments' gradients)."""
    t = torch()
    wl = W.causal_replay()
    g = wl.geom
    used = np.nonzero((g.used_q > 0) & (g.used_k > 0))[0]
    s_long = int(used[np.argmax(g.used_q[used] + g.used_k[used])])
    s_short = int(used[np.argmin(g.used_q[used])])
    below = used[g.used_k[used] < g.used_q[used]]
    picks = sorted({s_long, s_short} | ({int(below[0])} if len(below) else set()))
    say(f"[bwd causal_replay] segments {picks}: used_q {g.used_q[picks].tolist()} "
        f"used_k {g.used_k[picks].tolist()}")
    q_, k_, v_ = upload(wl.q, g), upload(wl.k, g), upload(wl.v, g)
    out = t.zeros((g.total_q, g.hq, g.dv), dtype=t.bfloat16, device="cuda")
    lse = t.zeros((g.hq, g.total_q), dtype=t.float32, device="cuda")
    cu_q, cu_k, used_q, used_k = i32(g.cu_q), i32(g.cu_k), i32(g.used_q), i32(g.used_k)
    B.gvattn_fwd(q_, k_, v_, cu_q, cu_k, used_q, used_k, out, lse, float(g.scale), True)
    do = W.normal_tensor(980, 7, (g.total_q, g.hq, g.dv), 1.0, W.BF16)
    subs = {}
    for s in picks:
        q0, k0, uq, uk = int(g.cu_q[s]), int(g.cu_k[s]), int(g.used_q[s]), int(g.used_k[s])
        sub = (wl.q[q0:q0 + uq], wl.k[k0:k0 + uk], wl.v[k0:k0 + uk], do[q0:q0 + uq])
        cu1, ck1 = np.array([0, uq]), np.array([0, uk])
        o_s, l_s = oracle.attention_fwd(sub[0], sub[1], sub[2], cu1, ck1, [uq], [uk],
                                        float(g.scale), True, workers=8)
        out[q0:q0 + uq] = t.from_numpy(o_s.astype(np.float32)).to("cuda").to(t.bfloat16)
        lse[:, q0:q0 + uq] = t.from_numpy(l_s.astype(np.float32)).to("cuda")
        subs[s] = (sub, cu1, ck1, uq, uk)
    dq = t.full_like(q_, W.SENTINEL)
    dk = t.full_like(k_, W.SENTINEL)
    dv = t.full_like(v_, W.SENTINEL)
    ws = B.gvattn_bwd(q_, k_, v_, out, upload(do, g), lse, cu_q, cu_k, used_q, used_k, dq, dk,
                      dv, float(g.scale), True)
    assert B.gvattn_read_device_error(ws) == 0
    assert gap_untouched(dq, used_mask(g.cu_q, g.used_q, g.total_q))
    mk = used_mask(g.cu_k, g.used_k, g.total_k)
    assert gap_untouched(dk, mk) and gap_untouched(dv, mk)
    for s, (sub, cu1, ck1, uq, uk) in subs.items():
        q0, k0 = int(g.cu_q[s]), int(g.cu_k[s])
        args = (*sub, cu1, ck1, [uq], [uk], float(g.scale), True)
        rq, rk, rv = oracle.attention_bwd(*args)
        aq, ak, av = oracle.attention_bwd_magnitudes(*args)
        st = {}
        for name, got, want, mag in (("dq", dq[q0:q0 + uq], rq, aq), ("dk", dk[k0:k0 + uk], rk, ak),
                                     ("dv", dv[k0:k0 + uk], rv, av)):
            m = np.ones(want.shape[0], dtype=bool)
            st[name] = check_grad(to_np(got), want, mag, m, W.BF16, f"causal_replay seg {s} {name}")
        say(f"[bwd causal_replay] seg {s}", st)


def test_bwd_cross_attention_split():
    """The CFG cross-attention workload at full size (2 x 4096 queries, text
    keys 24 and 700 of capacity 4096, 32 / 8 heads, d 128): few 64-key
    tiles, so the dK / dV loop of every tile is split into chunks whose FP32
    partials a reduce pass sums.  Every used row and key against the
    oracle; pad keys keep their sentinel."""
    wl = W.cfg_cross_attention()
    check_case(wl, 990, "bwd cross-attention split")
