"""The allocation-free forward (gvattn_fwd_noalloc) against gvattn_fwd and
the FP64 oracle, through the C ABI: calls in a row on one device share the
library's static scratch array, so each case runs after a different one.

Cases, in order: a decode-like launch that splits its keys (the ordinary
layout fits the scratch: bit-identical to gvattn_fwd), a smaller causal
launch without splits (it must not read the first call's plan), a launch
whose ordinary split-K partials do not fit (fewer chunks: checked against
the oracle at the stated bar), and the first case again."""

import numpy as np
import pytest

from segmented_varlen_attention_amd import binding as B
from segmented_varlen_attention_amd import workloads as W

from gpu_util import DeviceCase, compare_full, compare_sampled, i32, say, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()
    yield


def _decode_case():
    uq = [1, 7, 40, 0, 3, 33]
    uk = [3000, 2500, 1200, 900, 0, 1999]
    g = W.make_geometry([u + 5 for u in uq], [u + 7 for u in uk], uq, uk, 8, 2, 128, True)
    q, k, v = W.fill_qkv(g, 700)
    return W.Workload("decode_noalloc", 700, g, q, k, v)


def _noalloc(dc, geom=None):
    g = geom or dc.wl.geom
    out, lse = dc.new_out()
    B.gvattn_fwd_noalloc(dc.q, dc.k, dc.v, dc.cu_q, i32(g.cu_k), dc.used_q, i32(g.used_k), out,
                         lse, float(g.scale), g.causal)
    return out, lse


def _same_bits(a, b, la, lb):
    t = torch()
    return t.equal(a.view(t.int16), b.view(t.int16)) and t.equal(la.view(t.int32),
                                                                lb.view(t.int32))


def test_noalloc_matches_gvattn_fwd_on_calls_in_a_row():
    t = torch()
    wl1 = _decode_case()
    dc1 = DeviceCase(wl1)
    ref1, lref1, ws1 = dc1.fwd()
    t.cuda.synchronize()
    assert int(ws1[16:20].cpu().numpy().view(np.int32)[0]) > 1  # the plan split the keys
    say("[noalloc] call 1: decode-like, split-K")
    o1, l1 = _noalloc(dc1)
    t.cuda.synchronize()
    assert _same_bits(o1, ref1, l1, lref1)
    say("   ", compare_full(o1, l1, wl1, where="noalloc decode", derived=True))

    # a smaller launch after it: the scratch still holds call 1's plan
    wl2 = W.random_small(701, 4, 64, 96, 8, 2, 128, True, W.BF16,
                         lengths=([64, 17, 0, 40], [96, 5, 30, 0]))
    dc2 = DeviceCase(wl2)
    say("[noalloc] call 2: smaller causal launch")
    o2, l2 = _noalloc(dc2)
    ref2, lref2, _ = dc2.fwd()
    t.cuda.synchronize()
    assert _same_bits(o2, ref2, l2, lref2)
    say("   ", compare_full(o2, l2, wl2, where="noalloc small", derived=True))

    # ordinary partials would need 3 chunks of 17 MB: the scratch takes fewer
    uq = [512, 480, 0]
    uk = [6000, 3000, 100]
    g3 = W.make_geometry([512, 512, 8], [6000, 3000, 100], uq, uk, 32, 8, 128, False)
    q, k, v = W.fill_qkv(g3, 702)
    wl3 = W.Workload("noalloc_capped", 702, g3, q, k, v)
    need = B.gvattn_fwd_workspace_size(g3.nseg, g3.total_q, 32, 8, 128, B.GVATTN_BF16)
    assert need > B.GVATTN_NOALLOC_SCRATCH_BYTES
    dc3 = DeviceCase(wl3)
    say("[noalloc] call 3: split partials capped to the scratch")
    o3, l3 = _noalloc(dc3)
    t.cuda.synchronize()
    rng = np.random.default_rng(703)
    samples = [(s, np.unique(np.concatenate([[0, uq[s] - 1], rng.choice(uq[s], 14, replace=False)])))
               for s in range(2)]
    say("   ", compare_sampled(o3, l3, wl3, samples, where="noalloc capped"))

    # call 1 again, after the others
    say("[noalloc] call 4: decode-like again")
    o4, l4 = _noalloc(dc1)
    t.cuda.synchronize()
    assert _same_bits(o4, ref1, l4, lref1)
