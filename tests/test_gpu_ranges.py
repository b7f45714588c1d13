"""GPU parity of the key-range forward (gvattn_fwd_ranges) against the FP64
oracle's range form, through the C ABI.

Segment keys given as ordered lists of K/V row ranges: the rank-major key
order after a Ulysses all-to-all (TensorRT-LLM issue #18687, "additional
notes", possible fix 1), random ranges (empty, overlapping, out of order, none), one range
per segment (must equal the prefix form bit for bit) and the two visibility
partitions of the multiview workload fused into one launch.
"""

import numpy as np
import pytest

import oracle
from segmented_varlen_attention_amd import binding as B
from segmented_varlen_attention_amd import workloads as W

from gpu_util import (DeviceCase, check_gap_rows, compare, i32, say, to_np, torch,
                      used_row_mask)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()
    yield


def run_ranges(dc: DeviceCase, ranges, causal=None, out=None, lse=None):
    g = dc.wl.geom
    if out is None:
        out, lse = dc.new_out()
    off, st, ln = ranges
    ws = B.gvattn_fwd_ranges(dc.q, dc.k, dc.v, dc.cu_q, dc.used_q, i32(off), i32(st), i32(ln),
                             out, lse, float(g.scale), g.causal if causal is None else causal)
    return out, lse, ws


def oracle_ranges(wl, ranges, causal=None):
    g = wl.geom
    off, st, ln = ranges
    return oracle.attention_fwd_ranges(wl.q, wl.k, wl.v, g.cu_q, g.used_q, off, st, ln,
                                       float(g.scale), g.causal if causal is None else causal,
                                       workers=8)


def o_abs_ranges(wl, ranges):
    g = wl.geom
    off, st, ln = ranges
    o, _ = oracle.attention_fwd_ranges(wl.q, wl.k, np.abs(wl.v), g.cu_q, g.used_q, off, st, ln,
                                       float(g.scale), g.causal, workers=8)
    return o


def check_all_rows(out, lse, wl, ranges, where, derived=True):
    g = wl.geom
    o_ref, l_ref = oracle_ranges(wl, ranges)
    check_gap_rows(out, lse, g)
    m = used_row_mask(g)
    o_abs = o_abs_ranges(wl, ranges)[m] if (derived and g.dtype != W.FP32) else None
    return compare(to_np(out)[m], to_np(lse)[:, m], o_ref[m], l_ref[:, m], g.dtype, where,
                   o_abs=o_abs)


@pytest.mark.parametrize("dtype", [W.BF16, W.FP16, W.FP32])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_random_ranges(dtype, d, causal):
    rng = np.random.default_rng(500 + d + 7 * causal)
    nseg = 6
    wl = W.random_small(510 + d, nseg, 70, 300, 8, 2, d, causal, dtype,
                        lengths=(rng.integers(0, 71, nseg), np.zeros(nseg, int)))
    ranges = W.random_ranges(rng, nseg, wl.geom.total_k, max_ranges=4, max_len=90)
    say(f"[ranges {dtype} d={d} causal={causal}] per segment "
        f"{np.diff(ranges[0]).tolist()} lens {ranges[2].tolist()}")
    dc = DeviceCase(wl)
    out, lse, ws = run_ranges(dc, ranges)
    assert B.gvattn_read_device_error(ws) == 0
    say("   ", check_all_rows(out, lse, wl, ranges, f"ranges {dtype} d{d} c{int(causal)}"))


@pytest.mark.parametrize("dtype", [W.BF16, W.FP32])
def test_single_range_equals_prefix_form(dtype):
    """(cu_k[s], used_k[s]) as one range per segment: the same tiles in the
    same order as gvattn_fwd, so the outputs are equal bit for bit."""
    rng = np.random.default_rng(520)
    wl = W.random_small(521, 7, 96, 160, 8, 2, 128, True, dtype,
                        lengths=(rng.integers(0, 97, 7), rng.integers(0, 161, 7)))
    g = wl.geom
    dc = DeviceCase(wl)
    o1, l1, _ = dc.fwd()
    ranges = (np.arange(g.nseg + 1, dtype=np.int32), g.cu_k[:-1].astype(np.int32),
              g.used_k.astype(np.int32))
    o2, l2, _ = run_ranges(dc, ranges)
    t = torch()
    iv = t.int16 if dtype == W.BF16 else t.int32
    assert t.equal(o1.view(iv), o2.view(iv)) and t.equal(l1.view(t.int32), l2.view(t.int32))


def test_ulysses_rank_major_joint():
    """The issue's scenario at full size: 2 CFG samples, 4096 video queries,
    text capacity 4096 with real lengths 24 and 700, 4096 video keys, Ulysses
    size 2 (four key ranges per sample).  Every used row against the oracle;
    the result also equals attention over the trimmed keys and differs from
    the unmasked form that attends the zero pad slots."""
    wl = W.ulysses_joint()
    g = wl.geom
    dc = DeviceCase(wl)
    out, lse, ws = run_ranges(dc, wl.key_ranges)
    assert B.gvattn_read_device_error(ws) == 0
    st = check_all_rows(out, lse, wl, wl.key_ranges, "ulysses joint", derived=False)
    say("[ulysses joint]", st)
    # trimmed: gather each sample's valid keys into one prefix and use the
    # prefix form on the device
    off, starts, lens = wl.key_ranges
    keep = [oracle.segment_key_rows(off, starts, lens, s) for s in range(g.nseg)]
    kt = np.concatenate([wl.k[r] for r in keep])
    vt = np.concatenate([wl.v[r] for r in keep])
    nk = [len(r) for r in keep]
    gt = W.make_geometry([4096, 4096], nk, [4096, 4096], nk, g.hq, g.hkv, g.d, False)
    wt = W.Workload("trimmed", 0, gt, wl.q, kt, vt)
    o_t, l_t, _ = DeviceCase(wt).fwd()
    d_o = (o_t.float() - out.float()).abs().max().item()
    d_l = (l_t - lse).abs().max().item()
    say(f"[ulysses joint] vs trimmed prefix form: max |dO| {d_o:.3g} max |dLSE| {d_l:.3g}")
    assert d_l <= 2e-5 and d_o <= 1.6e-2
    # unmasked: every key of the rank-major buffer, pads included
    full = (np.array([0, 1, 2], np.int32), np.array([0, 8192], np.int32),
            np.array([8192, 8192], np.int32))
    o_u, l_u, _ = run_ranges(dc, full)
    assert (l_u - lse).abs().max().item() > 0.1


def test_fused_partitions_single_launch():
    """The multiview workload's two visibility partitions as two key ranges
    per segment: one launch, no merge.  Sampled rows against the oracle."""
    wl = W.multiview_partitions()
    g = wl.geom
    (cu_a, used_a), (cu_b, used_b) = wl.partitions
    starts = np.stack([cu_a[:-1], cu_b[:-1]], axis=1).reshape(-1).astype(np.int32)
    lens = np.stack([used_a, used_b], axis=1).reshape(-1).astype(np.int32)
    off = np.arange(0, 2 * g.nseg + 1, 2, dtype=np.int32)
    dc = DeviceCase(wl)
    out, lse, ws = run_ranges(dc, (off, starts, lens))
    assert B.gvattn_read_device_error(ws) == 0
    check_gap_rows(out, lse, g)
    rng = np.random.default_rng(530)
    rows = [np.sort(rng.choice(int(g.used_q[s]), 6, replace=False)) for s in (0, 3, 7)]
    for s, r in zip((0, 3, 7), rows):
        keys = oracle.segment_key_rows(off, starts, lens, s)
        o_ref, l_ref = oracle.attention_fwd(wl.q[g.cu_q[s] + r], wl.k[keys], wl.v[keys],
                                            np.array([0, len(r)]), np.array([0, len(keys)]),
                                            np.array([len(r)]), np.array([len(keys)]),
                                            float(g.scale), False, workers=8)
        gi = torch().from_numpy(g.cu_q[s] + r).to("cuda")
        st = compare(to_np(out.index_select(0, gi)), to_np(lse.index_select(1, gi)), o_ref,
                     l_ref, W.BF16, f"fused seg {s}")
        say(f"[fused partitions] seg {s}", st)


def test_range_errors_skip_segment():
    """A range past total_k: that segment is skipped (rows untouched), the
    error bit is set, the other segments are computed."""
    wl = W.random_small(540, 4, 40, 64, 4, 2, 64, False, W.BF16,
                        lengths=([40, 17, 33, 8], [0, 0, 0, 0]))
    g = wl.geom
    off = np.array([0, 1, 3, 4, 5], np.int32)
    starts = np.array([0, 70, 100, g.total_k - 10, 5], np.int32)
    lens = np.array([60, 20, 30, 11, 50], np.int32)   # segment 2's range overruns
    dc = DeviceCase(wl)
    out, lse, ws = run_ranges(dc, (off, starts, lens))
    assert B.gvattn_read_device_error(ws) == B.GVATTN_DEVERR_KRANGES
    bad = slice(int(g.cu_q[2]), int(g.cu_q[3]))
    assert (out[bad].float() == W.SENTINEL).all().item()
    assert (lse[:, bad] == W.SENTINEL).all().item()
    lens_ok = lens.copy()
    lens_ok[3] = 10
    o_ref, l_ref = oracle_ranges(wl, (off, starts, lens_ok))
    m = used_row_mask(g)
    m[bad] = False
    compare(to_np(out)[m], to_np(lse)[:, m], o_ref[m], l_ref[:, m], W.BF16, "range errors")


@pytest.mark.parametrize("d,dv", [(128, 64), (64, 256)])
def test_random_ranges_dv(d, dv):
    """Key ranges with a V/O head dim different from the Q/K one."""
    rng = np.random.default_rng(550 + d + dv)
    nseg = 5
    wl = W.random_small(551 + dv, nseg, 70, 300, 8, 2, d, True, W.BF16,
                        lengths=(rng.integers(0, 71, nseg), np.zeros(nseg, int)), dv=dv)
    ranges = W.random_ranges(rng, nseg, wl.geom.total_k, max_ranges=3, max_len=90)
    dc = DeviceCase(wl)
    out, lse, ws = run_ranges(dc, ranges)
    assert B.gvattn_read_device_error(ws) == 0
    say(f"[ranges dv] d={d} dv={dv}", check_all_rows(out, lse, wl, ranges, f"ranges d{d} dv{dv}"))
