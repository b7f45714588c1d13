"""GPU parity: the HIP path through the C ABI against the FP64 oracle.

Small seeded geometries are compared element by element on every used row;
the full-size workloads are compared on sampled segments / rows that the
oracle computes one by one, plus whole-buffer properties (gap rows bit-exact,
-inf / zero rows, finiteness).
"""

import numpy as np
import pytest

import oracle
from segmented_varlen_attention_amd import binding as B
from segmented_varlen_attention_amd import workloads as W

from gpu_util import (DIMS_FWD, DeviceCase, check_gap_rows, compare, compare_full,
                      compare_sampled, i32, oracle_abs, random_decode_geometry, random_geometry,
                      say, tile_rows, to_np, torch, used_row_mask)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()
    yield


# --- small sweeps: every used row ---------------------------------------------

EDGE_Q = [0, 1, 31, 32, 33, 70, 96]
EDGE_K = [0, 1, 63, 64, 65, 129, 160]


def small_case(seed, g, d, causal, dtype, hkv=2, dv=None):
    rng = np.random.default_rng(seed)
    nseg = 7
    uq = rng.permutation(EDGE_Q)[:nseg]
    uk = rng.permutation(EDGE_K)[:nseg]
    return W.random_small(seed, nseg, 96, 160, g * hkv, hkv, d, causal, dtype,
                          lengths=(uq, uk), dv=dv)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("g", [1, 2, 3, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_small_bf16(d, g, causal):
    wl = small_case(100 + d + g, g, d, causal, W.BF16)
    say(f"[small bf16] d={d} g={g} causal={causal} uq={wl.geom.used_q} uk={wl.geom.used_k}")
    dc = DeviceCase(wl)
    out, lse, _ = dc.fwd()
    st = compare_full(out, lse, wl, where=f"bf16 d{d} g{g} c{int(causal)}", derived=True)
    say("   ", st)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("g", [1, 2, 3, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_small_fp16(d, g, causal):
    """Same geometries as the bf16 sweep (other values), fp16 matrix cores."""
    wl = small_case(150 + d + g, g, d, causal, W.FP16)
    say(f"[small fp16] d={d} g={g} causal={causal} uq={wl.geom.used_q} uk={wl.geom.used_k}")
    dc = DeviceCase(wl)
    out, lse, _ = dc.fwd()
    st = compare_full(out, lse, wl, where=f"fp16 d{d} g{g} c{int(causal)}", derived=True)
    say("   ", st)


@pytest.mark.parametrize("d,dv", [(128, 64), (64, 128), (256, 128), (128, 256), (64, 256),
                                  (256, 64)])
@pytest.mark.parametrize("dtype", [W.BF16, W.FP32])
@pytest.mark.parametrize("causal", [False, True])
def test_small_dv(d, dv, dtype, causal):
    """V/O head dim different from the Q/K one (the pages' FA2 path takes
    equal dims only; the rest goes to their FP32 fallback)."""
    wl = small_case(170 + d + dv, 4, d, causal, dtype, dv=dv)
    say(f"[small dv] {dtype} d={d} dv={dv} causal={causal}")
    out, lse, _ = DeviceCase(wl).fwd()
    st = compare_full(out, lse, wl, where=f"{dtype} d{d} dv{dv} c{int(causal)}", derived=True)
    say("   ", st)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_small_fp32(d, causal):
    wl = small_case(200 + d, 3, d, causal, W.FP32)
    say(f"[small fp32] d={d} causal={causal}")
    dc = DeviceCase(wl)
    out, lse, _ = dc.fwd()
    say("   ", compare_full(out, lse, wl, where=f"fp32 d{d} c{int(causal)}"))


# --- seeded random geometries: every used row -----------------------------------

@pytest.mark.parametrize("seed", range(900, 924))
def test_random_geometries(seed):
    wl, std = random_geometry(seed, DIMS_FWD, (W.BF16, W.FP16, W.FP32))
    g = wl.geom
    say(f"[random] seed={seed} {g.dtype} d={g.d} dv={g.dv} hq={g.hq} hkv={g.hkv} "
        f"causal={g.causal} std={std} caps_q={np.diff(g.cu_q).tolist()} uq={g.used_q.tolist()} "
        f"caps_k={np.diff(g.cu_k).tolist()} uk={g.used_k.tolist()}")
    out, lse, _ = DeviceCase(wl).fwd()
    st = compare_full(out, lse, wl, where=f"random seed {seed}", derived=True)
    say("   ", st)


@pytest.mark.parametrize("nseg", [1000, 3000])
def test_many_segments_tiny_lengths(nseg):
    """Segments of capacity <= 5: many empty and one-row tiles.  The plan
    keeps up to 2048 segments in LDS and reads more from global memory, so
    the two counts take both paths."""
    rng = np.random.default_rng(7 + nseg)
    caps_q = rng.integers(0, 6, nseg)
    caps_k = rng.integers(0, 6, nseg)
    uq = np.array([rng.integers(0, c + 1) for c in caps_q])
    uk = np.array([rng.integers(0, c + 1) for c in caps_k])
    g = W.make_geometry(caps_q, caps_k, uq, uk, 8, 2, 128, causal=True)
    q, k, v = W.fill_qkv(g, 8)
    wl = W.Workload("tiny_many", 7, g, q, k, v)
    out, lse, _ = DeviceCase(wl).fwd()
    say(f"[many tiny {nseg}]", compare_full(out, lse, wl, where=f"many tiny {nseg}",
                                            derived=True))


@pytest.mark.parametrize("dtype", [W.BF16, W.FP16])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_score_jumps_across_key_tiles(dtype, d, causal):
    """Key tiles whose scores are 32x larger (or smaller) than the previous
    tile's: the running max a tile's softmax starts from is then about 2^20
    below the tile's largest weight, the row sums overflow the bound the
    kernel accepts (2^15, which keeps fp16 weights finite) and the tile is
    redone by the exact step (scores recomputed, max raised, O rescaled);
    tiles far below the max underflow to zero weight."""
    seed = 1200 + d + 7 * causal + (3 if dtype == W.FP16 else 0)
    uq, uk = [96, 70, 40, 33], [260, 200, 97, 65]
    wl = W.random_small(seed, 4, 96, 260, 8, 2, d, causal, dtype, lengths=(uq, uk))
    g = wl.geom
    factors = np.array([0.25, 8.0, 0.25, 1.0, 8.0, 0.5, 0.25, 8.0, 2.0])
    k = wl.k.copy()
    for seg in range(g.nseg):
        k0 = int(g.cu_k[seg])
        j = np.arange(int(g.cu_k[seg + 1]) - k0)
        k[k0 + j] *= factors[(j // 32) % len(factors)][:, None, None]
    wl.k = W.round_to(dtype, k)
    out, lse, _ = DeviceCase(wl).fwd()
    say(f"[score jumps {dtype} d{d} c{int(causal)}]",
        compare_full(out, lse, wl, where=f"score jumps {dtype} d{d} c{int(causal)}", derived=True))


@pytest.mark.parametrize("d,dv", [(256, 256), (128, 256), (256, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_score_jumps_long_keys_large_heads(d, dv, causal):
    """The large-head kernels take a tile's row max, and raise the running
    max and rescale O, after the previous tile's P.V and before the tile's
    own weights.  Eleven 64-key tiles whose key scale jumps by up to 32x
    every 32 keys (growth and decay of the row max in the middle of the key
    sequence, several times per row), in bf16 against the oracle."""
    seed = 1300 + d + dv + 7 * causal
    uq, uk = [96, 64, 33], [700, 690, 650]
    wl = W.random_small(seed, 3, 96, 700, 8, 2, d, causal, W.BF16, lengths=(uq, uk), dv=dv)
    g = wl.geom
    factors = np.array([0.25, 8.0, 0.25, 1.0, 8.0, 0.5, 0.25, 8.0, 2.0, 0.125, 4.0])
    k = wl.k.copy()
    for seg in range(g.nseg):
        k0 = int(g.cu_k[seg])
        j = np.arange(int(g.cu_k[seg + 1]) - k0)
        k[k0 + j] *= factors[(j // 32) % len(factors)][:, None, None]
    wl.k = W.round_to(W.BF16, k)
    out, lse, _ = DeviceCase(wl).fwd()
    say(f"[score jumps, long keys, d{d} dv{dv} c{int(causal)}]",
        compare_full(out, lse, wl, where=f"score jumps long d{d} dv{dv} c{int(causal)}",
                     derived=True))


# --- the five workloads -------------------------------------------------------------

def test_fp32_three_segments():
    wl = W.fp32_three_segments()
    out, lse, _ = DeviceCase(wl).fwd()
    st = compare_full(out, lse, wl, where="fp32_three_segments")
    say("[fp32_three_segments]", st)
    lse_np = to_np(lse)
    g = wl.geom
    rows = slice(g.cu_q[1], g.cu_q[1] + g.used_q[1])  # the segment with no keys
    assert np.all(np.isneginf(lse_np[:, rows])) and np.all(to_np(out)[rows] == 0.0)


def test_cfg_cross_attention():
    wl = W.cfg_cross_attention()
    g = wl.geom
    dc = DeviceCase(wl)
    out, lse, _ = dc.fwd()
    o_ref, l_ref = oracle.attention_fwd(wl.q, wl.k, wl.v, g.cu_q, g.cu_k, g.used_q, g.used_k,
                                        float(g.scale), False, workers=16)
    st = compare_full(out, lse, wl, o_ref=o_ref, l_ref=l_ref, where="cfg_cross_attention")
    say("[cfg_cross_attention]", st)
    # equals attention over the text trimmed per sample, not the unmasked form
    lens = [int(x) for x in g.used_k]
    keep = np.concatenate([np.arange(g.cu_k[s], g.cu_k[s] + L) for s, L in enumerate(lens)])
    cu_t = np.array([0, lens[0], lens[0] + lens[1]])
    o_t, l_t = oracle.attention_fwd(wl.q, wl.k[keep], wl.v[keep], g.cu_q, cu_t, g.used_q, lens,
                                    float(g.scale), False, workers=16)
    o_gpu, l_gpu = to_np(out), to_np(lse)
    compare(o_gpu, l_gpu, o_t, l_t, W.BF16, "cfg_cross_attention vs trimmed")
    # the unmasked (buggy) result differs measurably for the short sample
    gb = g.with_keys(g.cu_k, [4096, 4096])
    ob, lb = oracle.attention_fwd(wl.q[:4096], wl.k[:4096], wl.v[:4096], g.cu_q[:2],
                                  g.cu_k[:2], g.used_q[:1], gb.used_k[:1], float(g.scale), False,
                                  workers=16)
    assert np.max(np.abs(l_gpu[:, :4096] - lb)) > 1.0


def test_causal_replay_64x2048():
    """Every used row of all 64 segments against the full oracle, plus the
    rows with no visible key checked on the device."""
    wl = W.causal_replay()
    g = wl.geom
    out, lse, ws = DeviceCase(wl).fwd()
    assert B.gvattn_read_device_error(ws) == 0
    st = compare_full(out, lse, wl, where="causal_replay")
    say("[causal_replay] all used rows", st)
    # any size: all used rows finite; rows with no visible key exactly (0, -inf)
    m = used_row_mask(g)
    t = torch()
    mt = t.from_numpy(m).to("cuda")
    assert t.isfinite(out[mt]).all().item()
    for s in range(g.nseg):
        uq, uk = int(g.used_q[s]), int(g.used_k[s])
        n_dead = uq if uk == 0 else max(0, uq - uk)
        if n_dead:
            r0 = int(g.cu_q[s])
            blk = lse[:, r0:r0 + n_dead]
            assert t.isneginf(blk).all().item(), s
            assert (out[r0:r0 + n_dead] == 0).all().item(), s


def test_multiview_partitions_merge():
    """Both partitions, their merge and the single pass, each on whole
    32-row tiles at the start, middle and end of every segment against the
    oracle.  On the device, the merged result is compared with the single
    pass on every row: each of the two is within the output-rounding floor
    plus 5e-3 of the exact result, so they differ by at most twice that
    (|O| < 4 here, so the floor is at most 2^-7)."""
    wl = W.multiview_partitions()
    g = wl.geom
    dc = DeviceCase(wl)
    (cu_a, used_a), (cu_b, used_b) = wl.partitions
    ga, gb = g.with_keys(cu_a, used_a), g.with_keys(cu_b, used_b)
    out_a, lse_a, _ = dc.fwd(ga)
    out_b, lse_b, _ = dc.fwd(gb)
    out_s, lse_s, _ = dc.fwd(g)  # single pass over all keys
    out_m, lse_m = dc.new_out()
    err = i32([0])
    B.gvattn_lse_merge([out_a, out_b], [lse_a, lse_b], dc.cu_q, dc.used_q, out_m, lse_m,
                       device_error=err)
    torch().cuda.synchronize()
    assert int(err.item()) == 0
    samples = [(s, tile_rows(int(g.used_q[s]))) for s in range(g.nseg)]
    st_m = compare_sampled(out_m, lse_m, wl, samples, where="multiview_partitions merged")
    st_s = compare_sampled(out_s, lse_s, wl, samples, where="multiview_partitions single")
    say("[multiview_partitions] merged", st_m, "single", st_s)
    st_a = compare_sampled(out_a, lse_a, wl, samples, geom=ga, where="multiview_partitions A")
    st_b = compare_sampled(out_b, lse_b, wl, samples, geom=gb, where="multiview_partitions B")
    say("[multiview_partitions] A", st_a, "B", st_b)
    d_lse = (lse_m - lse_s).abs().max().item()
    d_out = (out_m.float() - out_s.float()).abs().max().item()
    say(f"[multiview_partitions] merged-vs-single max |dLSE|={d_lse:.3g} max |dO|={d_out:.3g}")
    assert d_lse <= 2e-5 and d_out <= 2 * (2.0 ** -7 + 5e-3)


def test_large_head_d256():
    """Whole 32-row tiles at the start, middle and end of all 16 segments."""
    wl = W.large_head_d256()
    g = wl.geom
    out, lse, ws = DeviceCase(wl).fwd()
    assert B.gvattn_read_device_error(ws) == 0
    samples = [(s, tile_rows(int(g.used_q[s]))) for s in range(g.nseg)]
    st = compare_sampled(out, lse, wl, samples, where="large_head_d256")
    say("[large_head_d256]", st)


# --- robustness ---------------------------------------------------------------------

def test_nan_gap_rows_and_segment_isolation():
    wl = small_case(300, 4, 128, True, W.BF16)
    g = wl.geom
    out0, lse0, _ = DeviceCase(wl).fwd()
    q, k, v = wl.q.copy(), wl.k.copy(), wl.v.copy()
    for s in range(g.nseg):
        q[g.cu_q[s] + g.used_q[s]:g.cu_q[s + 1]] = np.nan
        k[g.cu_k[s] + g.used_k[s]:g.cu_k[s + 1]] = np.nan
        v[g.cu_k[s] + g.used_k[s]:g.cu_k[s + 1]] = np.nan
    s0 = int(np.argmax(g.used_q))
    q[g.cu_q[s0]:g.cu_q[s0] + g.used_q[s0]] *= 2.0  # perturb one segment
    out1, lse1, _ = DeviceCase(wl, q=q, k=k, v=v).fwd()
    check_gap_rows(out1, lse1, g)
    t = torch()
    m = used_row_mask(g)
    m[g.cu_q[s0]:g.cu_q[s0 + 1]] = False
    mt = t.from_numpy(m).to("cuda")
    assert t.equal(out0[mt].view(t.int16), out1[mt].view(t.int16))
    assert t.equal(lse0[:, mt].view(t.int32), lse1[:, mt].view(t.int32))


def test_deterministic():
    wl = small_case(301, 4, 128, True, W.BF16)
    dc = DeviceCase(wl)
    t = torch()
    a, la, _ = dc.fwd()
    b, lb, _ = dc.fwd()
    assert t.equal(a.view(t.int16), b.view(t.int16)) and t.equal(la.view(t.int32), lb.view(t.int32))


def test_plan_then_run_and_plan_mismatch():
    wl = small_case(302, 4, 128, True, W.BF16)
    g = wl.geom
    dc = DeviceCase(wl)
    ws = B.gvattn_fwd_plan(B.GVATTN_BF16, dc.cu_q, i32(g.cu_k), dc.used_q, i32(g.used_k),
                           g.total_q, g.total_k, g.hq, g.hkv, g.d, g.causal)
    out1, lse1, _ = dc.fwd(fn=B.gvattn_fwd_run, workspace=ws)
    out2, lse2, _ = dc.fwd(fn=B.gvattn_fwd_run, workspace=ws)
    t = torch()
    assert t.equal(out1.view(t.int16), out2.view(t.int16))
    compare_full(out1, lse1, wl, where="plan+run")
    assert B.gvattn_read_device_error(ws) == 0
    # a plan built for the non-causal problem does not match a causal run
    ws2 = B.gvattn_fwd_plan(B.GVATTN_BF16, dc.cu_q, i32(g.cu_k), dc.used_q, i32(g.used_k),
                            g.total_q, g.total_k, g.hq, g.hkv, g.d, False)
    out3, lse3, _ = dc.fwd(fn=B.gvattn_fwd_run, workspace=ws2)
    assert B.gvattn_read_device_error(ws2) & B.GVATTN_DEVERR_PLAN
    assert (out3.float() == W.SENTINEL).all().item() and (lse3 == W.SENTINEL).all().item()


def test_device_errors_skip_bad_segments():
    wl = small_case(303, 2, 64, False, W.BF16)
    g = wl.geom
    dc = DeviceCase(wl)
    bad = int(np.argmax(g.used_q))
    used_q = g.used_q.copy()
    used_q[bad] = (g.cu_q[bad + 1] - g.cu_q[bad]) + 5  # beyond its capacity
    dc.used_q = i32(used_q)
    out, lse, ws = dc.fwd()
    assert B.gvattn_read_device_error(ws) == B.GVATTN_DEVERR_USED_Q
    rows = slice(g.cu_q[bad], g.cu_q[bad + 1])
    assert (out[rows].float() == W.SENTINEL).all().item()
    dc.used_q = i32(g.used_q)
    good = [s for s in range(g.nseg) if s != bad]
    compare_sampled(out, lse, wl, [(s, np.arange(g.used_q[s])) for s in good], where="errs")
    # overlapping capacities reject the whole plan
    cu_q = g.cu_q.copy()
    cu_q[2] = cu_q[1] - 10
    dc.cu_q = i32(cu_q)
    _, _, ws = dc.fwd()
    assert B.gvattn_read_device_error(ws) & B.GVATTN_DEVERR_OFFSETS


@pytest.mark.parametrize("nparts", [2, 3])
@pytest.mark.parametrize("pdt,odt", [("bf16", "bf16"), ("fp32", "fp32"), ("fp32", "bf16"),
                                     ("fp16", "fp16"), ("fp16", "fp32"), ("bf16", "fp16")])
def test_merge_small(pdt, odt, nparts):
    """Two or three key partitions (some empty for some segments) merged on
    the device.  The merge kernel itself is held to FP32 accuracy against
    the oracle merge of the very partials it was given; end to end, the
    merged result matches the single-pass oracle within the derived bound of
    the forward's element type, doubled (the partials were rounded once
    more).  The output may alias partial 0.  fp32 partials are the bf16
    forward's outputs widened."""
    t = torch()
    fw = W.FP16 if pdt == "fp16" else W.BF16
    wl = W.random_small(400, 5, 48, 90, 8, 2, 128, False, fw,
                        lengths=([48, 0, 17, 33, 48], [90, 40, 0, 7, 61]))
    g = wl.geom
    dc = DeviceCase(wl)
    cuts = []
    for frac in ((0.0, 0.3, 0.7, 1.0) if nparts == 3 else (0.0, 0.45, 1.0)):
        cuts.append([int(round(frac * u)) for u in g.used_k])
    outs, lses = [], []
    for p in range(nparts):
        cu = np.array([g.cu_k[s] + cuts[p][s] for s in range(g.nseg)] + [g.total_k], np.int32)
        used = np.array([cuts[p + 1][s] - cuts[p][s] for s in range(g.nseg)], np.int32)
        o, l, _ = dc.fwd(g.with_keys(cu, used))
        outs.append(o.float() if pdt == "fp32" else o)
        lses.append(l)
    part_o = [to_np(o).astype(np.float64) for o in outs]
    part_l = [to_np(l).astype(np.float64) for l in lses]
    om_ref, lm_ref = oracle.lse_merge(part_o, part_l, g.cu_q, g.used_q)
    o_ref, l_ref = oracle.attention_fwd(wl.q, wl.k, wl.v, g.cu_q, g.cu_k, g.used_q, g.used_k,
                                        float(g.scale), False)
    if odt == pdt:
        out, lse = outs[0], lses[0]  # in place
    else:
        odt_t = {"bf16": t.bfloat16, "fp16": t.float16, "fp32": t.float32}[odt]
        out = t.full_like(outs[0], W.SENTINEL, dtype=odt_t)
        lse = t.full_like(lses[0], W.SENTINEL)
    B.gvattn_lse_merge(outs, lses, dc.cu_q, dc.used_q, out, lse)
    m = used_row_mask(g)
    o_gpu, l_gpu = to_np(out), to_np(lse)
    st = compare(o_gpu[m], l_gpu[:, m], om_ref[m], lm_ref[:, m], odt,
                 f"merge kernel {pdt}->{odt} x{nparts}", tol_out=1e-5)
    say(f"[merge kernel {pdt}->{odt} x{nparts}]", st)
    o_abs = oracle_abs(wl)[m]
    st2 = compare(o_gpu[m], l_gpu[:, m], o_ref[m], l_ref[:, m], fw,
                  f"merge end-to-end {pdt}->{odt}", o_abs=2 * o_abs)
    say(f"[merge end-to-end {pdt}->{odt}]", st2)
    check_gap_rows(out, lse, g)


def test_merge_nan_lse_rows():
    """A NaN LSE in one partial (PR #312's FP32 LSE merge, with NaN
    propagation as the convention): exactly those (row, head) pairs come out
    NaN in O and LSE, whichever partial holds the NaN; every other used pair
    is bit-identical to the merge of the same partials without the NaN, and
    gap rows keep the sentinel."""
    t = torch()
    wl = W.random_small(410, 4, 40, 70, 8, 2, 128, False, W.BF16,
                        lengths=([40, 0, 23, 31], [70, 30, 9, 0]))
    g = wl.geom
    dc = DeviceCase(wl)
    half = [u // 2 for u in g.used_k]
    parts = []
    for cu, used in ((g.cu_k, half),
                     (np.array([g.cu_k[s] + half[s] for s in range(g.nseg)] + [g.total_k]),
                      [int(g.used_k[s]) - half[s] for s in range(g.nseg)])):
        o, l, _ = dc.fwd(g.with_keys(cu, used))
        parts.append((o, l))
    clean_o, clean_l = dc.new_out()
    B.gvattn_lse_merge([p[0] for p in parts], [p[1] for p in parts], dc.cu_q, dc.used_q,
                       clean_o, clean_l)
    # (row, head) pairs: used rows of segments 0 and 2, one head each
    nan_at = [(int(g.cu_q[0]) + 3, 1), (int(g.cu_q[0]) + 39, 6), (int(g.cu_q[2]) + 5, 0)]
    for holder in (0, 1):
        lses = [p[1].clone() for p in parts]
        for r, h in nan_at:
            lses[holder][h, r] = float("nan")
        out, lse = dc.new_out()
        B.gvattn_lse_merge([p[0] for p in parts], lses, dc.cu_q, dc.used_q, out, lse)
        t.cuda.synchronize()
        check_gap_rows(out, lse, g)
        o_np, l_np = to_np(out), to_np(lse)
        mask = np.zeros((g.total_q, g.hq), bool)
        for r, h in nan_at:
            mask[r, h] = True
            assert np.isnan(o_np[r, h]).all() and np.isnan(l_np[h, r]), (holder, r, h)
        used = used_row_mask(g)
        keep = used[:, None] & ~mask
        assert not np.isnan(o_np[keep]).any() and not np.isnan(l_np.T[keep]).any()
        assert np.array_equal(out.view(t.int16).cpu().numpy()[keep],
                              clean_o.view(t.int16).cpu().numpy()[keep])
        assert np.array_equal(lse.view(t.int32).cpu().numpy().T[keep],
                              clean_l.view(t.int32).cpu().numpy().T[keep])
    say("[merge NaN LSE] NaN rows", nan_at, "isolated in both partial positions")


def test_plan_from_another_geometry_is_refused():
    """A plan carries a key of its host-side geometry: a run with other head
    counts that give the same tile shape (8/2 against 32/8 heads, both four
    query heads per KV head) or another row total refuses it, writes
    nothing and sets the plan error bit.  Neither geometry splits its keys,
    so no run could write partials even if it accepted the plan."""
    t = torch()
    rng = np.random.default_rng(620)
    nseg = 40
    uq = rng.integers(0, 257, nseg)
    uk = rng.integers(0, 257, nseg)
    g_small = W.make_geometry([256] * nseg, [256] * nseg, uq, uk, 8, 2, 128, True,
                              dtype=W.BF16)
    g_big = W.make_geometry([256] * nseg, [256] * nseg, uq, uk, 32, 8, 128, True,
                            dtype=W.BF16)
    q, k, v = W.fill_qkv(g_big, 621)
    wl = W.Workload("plan_key", 621, g_big, q, k, v)
    dc = DeviceCase(wl)
    n_ws = max(B.gvattn_fwd_workspace_size(nseg, g.total_q, g.hq, g.hkv, 128, B.GVATTN_BF16)
               for g in (g_small, g_big))
    ws = t.zeros(n_ws + 4096, dtype=t.uint8, device="cuda")
    B.gvattn_fwd_plan(B.GVATTN_BF16, dc.cu_q, i32(g_small.cu_k), dc.used_q, i32(g_small.used_k),
                      g_small.total_q, g_small.total_k, g_small.hq, g_small.hkv, 128, True,
                      workspace=ws)
    out, lse, _ = dc.fwd(fn=B.gvattn_fwd_run, workspace=ws)
    assert B.gvattn_read_device_error(ws) & B.GVATTN_DEVERR_PLAN
    assert max_split(ws) == 1
    assert (out.float() == W.SENTINEL).all().item() and (lse == W.SENTINEL).all().item()
    # same heads, one more block of gap rows at the end of Q / O: another total_q
    B.gvattn_fwd_plan(B.GVATTN_BF16, dc.cu_q, i32(g_big.cu_k), dc.used_q, i32(g_big.used_k),
                      g_big.total_q, g_big.total_k, g_big.hq, g_big.hkv, 128, True, workspace=ws)
    q2 = t.cat([dc.q, dc.q[:64]])
    out2 = t.full((g_big.total_q + 64, g_big.hq, 128), W.SENTINEL, dtype=t.bfloat16,
                  device="cuda")
    lse2 = t.full((g_big.hq, g_big.total_q + 64), W.SENTINEL, dtype=t.float32, device="cuda")
    B.gvattn_fwd_run(q2, dc.k, dc.v, dc.cu_q, i32(g_big.cu_k), dc.used_q, i32(g_big.used_k),
                     out2, lse2, float(g_big.scale), True, ws)
    assert B.gvattn_read_device_error(ws) & B.GVATTN_DEVERR_PLAN
    assert (out2.float() == W.SENTINEL).all().item() and (lse2 == W.SENTINEL).all().item()
    # the matching plan still runs
    out3, lse3, _ = dc.fwd(fn=B.gvattn_fwd_run, workspace=ws)
    torch().cuda.synchronize()
    assert not (out3.float() == W.SENTINEL).all().item()


# --- split-K (few query tiles, long keys) ----------------------------------------

def max_split(ws) -> int:
    """Most key chunks the plan split a query tile into (plan header)."""
    return int(ws[16:20].cpu().numpy().view(np.int32)[0])


@pytest.mark.parametrize("dtype", [W.BF16, W.FP16])
@pytest.mark.parametrize("d,dv", [(128, 128), (64, 64), (256, 256), (128, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_split_k_decode(dtype, d, dv, causal):
    """Decode-like launch: six segments with 0-40 used query rows and up to
    3000 keys (one empty, one without keys).  Too few query tiles to fill
    the GPU, so the plan splits the key ranges; every used row against the
    oracle, a second run on the same plan is bit-identical."""
    uq = [1, 7, 40, 0, 3, 33]
    uk = [3000, 2500, 1200, 900, 0, 1999]
    g = W.make_geometry([u + 5 for u in uq], [u + 7 for u in uk], uq, uk, 8, 2, d, causal,
                        dtype=dtype, dv=dv)
    q, k, v = W.fill_qkv(g, 600 + d + dv)
    wl = W.Workload("decode", 600, g, q, k, v)
    dc = DeviceCase(wl)
    out, lse, ws = dc.fwd()
    assert B.gvattn_read_device_error(ws) == 0
    assert max_split(ws) > 1
    st = compare_full(out, lse, wl, where=f"split {dtype} d{d} dv{dv} c{int(causal)}",
                      derived=True)
    say(f"[split-K] {dtype} d={d} dv={dv} causal={causal} max split {max_split(ws)}", st)
    out2, lse2, _ = dc.fwd(fn=B.gvattn_fwd_run, workspace=ws)
    t = torch()
    assert t.equal(out.view(t.int16), out2.view(t.int16))
    assert t.equal(lse.view(t.int32), lse2.view(t.int32))


@pytest.mark.parametrize("seed", range(700, 712))
def test_split_k_random_decode(seed):
    """Seeded decode-like launches (few query rows, up to 6000 keys, random
    GQA layout, head dims, dtype and mask): every used row against the
    oracle, and the same plan run twice gives bit-identical results."""
    wl = random_decode_geometry(seed, DIMS_FWD, (W.BF16, W.FP16))
    g = wl.geom
    dc = DeviceCase(wl)
    out, lse, ws = dc.fwd()
    assert B.gvattn_read_device_error(ws) == 0
    say(f"[split-K random] seed={seed} {g.dtype} d={g.d} dv={g.dv} hq={g.hq} hkv={g.hkv} "
        f"causal={g.causal} uq={g.used_q.tolist()} max split {max_split(ws)}")
    st = compare_full(out, lse, wl, where=f"split random seed {seed}", derived=True)
    say("   ", st)
    out2, lse2, _ = dc.fwd(fn=B.gvattn_fwd_run, workspace=ws)
    t = torch()
    assert t.equal(out.view(t.int16), out2.view(t.int16))
    assert t.equal(lse.view(t.int32), lse2.view(t.int32))


def test_no_split_when_the_gpu_is_full():
    """Enough query tiles: the plan does not split."""
    wl = W.random_small(610, 40, 256, 300, 32, 8, 128, True, W.BF16)
    out, lse, ws = DeviceCase(wl).fwd()
    assert max_split(ws) == 1
    compare_full(out, lse, wl, where="no split", derived=True)
