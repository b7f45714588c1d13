"""GPU: the device plan's work list against its specification.

The attention tests check the plan only through the results it leads to.
Here the tile list is read back from the workspace and compared with the
entries the plan must produce, written out in Python from the same rules:
one entry per (segment, query tile) whose key tiles run to the last key the
tile's last row sees (bottom-right causal), ordered by cost = key tiles,
longest first, coarsened to groups of 8 key tiles and then ordered by
segment when the launch's largest cost reaches 16 (cosmos-framework PR #302,
review: the segment geometry is read on the device, with no host sync).

The cases cover each code path of the plan kernel:
* up to 64 segments (validation in one wave);
* 1000 segments (every wave validates, tables in LDS);
* 3000 segments (tables in the workspace);
* more than four entries per thread (entries recomputed, not cached);
* split-K chunks;
* rejected segments.
"""

import numpy as np
import pytest

from segmented_varlen_attention_amd import binding as B
from segmented_varlen_attention_amd import workloads as W

from gpu_util import i32, torch

pytestmark = pytest.mark.gpu

COST_BUCKETS = 2048
EXACT_COST = 16
GROUP_SHIFT = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()
    yield


def tile_rows(hq, hkv):
    """Query rows per tile of the 16-bit forward: heads of a KV group folded
    4, 3, 2 or 1 at a time into a workgroup of 4 waves (3 for a fold of 3)."""
    g = hq // hkv
    gf = 4 if g % 4 == 0 else 3 if g % 3 == 0 else 2 if g % 2 == 0 else 1
    rb = 1 if gf == 3 else 4 // gf
    return 32 * rb


def key_tile(d, dv):
    return 32 if d <= 128 and dv <= 128 else 64


def plan_of(g, dtype=B.GVATTN_BF16):
    t = torch()
    dev = lambda x: t.from_numpy(np.ascontiguousarray(x, np.int32)).cuda()
    ws = B.gvattn_fwd_plan(dtype, dev(g.cu_q), dev(g.cu_k), dev(g.used_q), dev(g.used_k),
                           g.total_q, g.total_k, g.hq, g.hkv, g.d, g.causal, d_v=g.dv)
    t.cuda.synchronize()
    hdr = ws[:256].cpu().numpy().view(np.int32)
    n = int(hdr[0])
    tiles = ws[256:256 + 16 * n].cpu().numpy().view(np.int32).reshape(n, 4)
    return hdr, tiles, ws


def valid(g, s):
    cap_q = g.cu_q[s + 1] - g.cu_q[s]
    cap_k = g.cu_k[s + 1] - g.cu_k[s]
    return 0 <= g.used_q[s] <= cap_q and 0 <= g.used_k[s] <= cap_k


def key_tiles(g, rows, kt, s, row0):
    uq, uk = int(g.used_q[s]), int(g.used_k[s])
    kend = uk
    if g.causal:
        r_last = min(row0 + rows, uq) - 1
        kend = max(0, min(uk, r_last + uk - uq + 1))
    return -(-kend // kt)


def expected_entries(g):
    """(entries, sort key of each) of an unsplit plan."""
    rows, kt = tile_rows(g.hq, g.hkv), key_tile(g.d, g.dv)
    nseg = g.nseg
    max_kt = max([-(-int(g.used_k[s]) // kt) for s in range(nseg)
                  if valid(g, s) and g.used_q[s] > 0] or [0])
    max_kt = min(max_kt, COST_BUCKETS - 1)
    grouped = (max_kt >= EXACT_COST and
               EXACT_COST + ((max_kt >> GROUP_SHIFT) - (EXACT_COST >> GROUP_SHIFT) + 1) * nseg
               <= COST_BUCKETS)

    def sort_key(cost, s):
        if not grouped or cost < EXACT_COST:
            return cost
        return (EXACT_COST + ((cost >> GROUP_SHIFT) - (EXACT_COST >> GROUP_SHIFT)) * nseg
                + (nseg - 1 - s))

    ents, keys = [], []
    for s in range(nseg):
        if not valid(g, s):
            continue
        for qt in range(-(-int(g.used_q[s]) // rows)):
            nkt = key_tiles(g, rows, kt, s, qt * rows)
            ents.append((s, qt * rows, 0, nkt << 5))
            keys.append(sort_key(min(nkt, COST_BUCKETS - 1), s))
    return ents, keys, grouped


def check_unsplit(g, expect_err=0):
    hdr, tiles, _ = plan_of(g)
    assert int(hdr[1]) == expect_err
    assert int(hdr[3]) == tile_rows(g.hq, g.hkv)   # rows per tile
    assert int(hdr[4]) == 1                        # no split
    ents, keys, grouped = expected_entries(g)
    got = [tuple(int(x) for x in r) for r in tiles]
    assert len(got) == len(ents)
    assert sorted(got) == sorted(ents)
    # the list runs in non-increasing sort key (ties in any order)
    key_of = {}
    for e, k in zip(ents, keys):
        key_of[e] = k
    seq = [key_of[e] for e in got]
    assert all(a >= b for a, b in zip(seq, seq[1:]))
    return len(got), grouped


def test_plan_causal_replay():
    uq, uk = W.causal_replay_lengths(3)
    g = W.make_geometry([2048] * 64, [2048] * 64, uq, uk, 32, 8, 128, causal=True)
    n, grouped = check_unsplit(g)
    assert n == 1924 and grouped


def test_plan_cfg_cross_attention():
    g = W.make_geometry([4096, 4096], [4096, 4096], [4096, 4096], [24, 700], 32, 8, 128,
                        causal=False)
    n, grouped = check_unsplit(g)
    assert n == 256 and grouped


@pytest.mark.parametrize("g_fold,causal", [(1, True), (2, False), (3, True), (4, False)])
def test_plan_head_folds(g_fold, causal):
    """Each fold of the query heads gives its own rows per tile."""
    rng = np.random.default_rng(40 + g_fold)
    nseg = 50
    uq = rng.integers(0, 700, nseg, endpoint=True)
    uk = rng.integers(0, 900, nseg, endpoint=True)
    g = W.make_geometry([700] * nseg, [900] * nseg, uq, uk, 2 * g_fold, 2, 128, causal)
    check_unsplit(g)


@pytest.mark.parametrize("nseg", [1000, 3000])
def test_plan_many_segments(nseg):
    """Tiny segments: every wave validates (over 64 segments); 3000 segments
    keep their tables in the workspace instead of LDS."""
    rng = np.random.default_rng(7 + nseg)
    caps_q = rng.integers(0, 40, nseg)
    caps_k = rng.integers(0, 80, nseg)
    uq = np.array([rng.integers(0, c + 1) for c in caps_q])
    uk = np.array([rng.integers(0, c + 1) for c in caps_k])
    g = W.make_geometry(caps_q, caps_k, uq, uk, 8, 2, 128, causal=True)
    check_unsplit(g)


def test_plan_many_entries_per_thread():
    """d = 256, 16 segments of up to 16384 rows: thousands of entries, more
    than the histogram pass keeps in registers per thread."""
    uq, uk = W.large_head_lengths(5)
    g = W.make_geometry([16384] * 16, [16384] * 16, uq, uk, 16, 4, 256, causal=False)
    n, _ = check_unsplit(g)
    assert n > 4 * 512


def test_plan_skips_rejected_segments():
    """A segment whose used rows pass its capacity gets no entries and sets
    its error bit; the others are planned as usual."""
    uq = [30, 50, 10, 64]
    uk = [40, 20, 90, 64]
    g = W.make_geometry([32, 40, 16, 64], [48, 32, 96, 64], uq, uk, 8, 2, 128, causal=True)
    assert not valid(g, 1)
    check_unsplit(g, expect_err=B.GVATTN_DEVERR_USED_Q)


def test_plan_split_chunks_partition_each_tile():
    """Decode-like launch (few query tiles): every query tile's key tiles are
    split into contiguous chunks that cover them exactly once."""
    uq = [1, 7, 40, 0, 3, 33]
    uk = [3000, 2500, 1200, 900, 0, 1999]
    g = W.make_geometry([u + 5 for u in uq], [u + 7 for u in uk], uq, uk, 8, 2, 128, True)
    hdr, tiles, _ = plan_of(g)
    rows, kt = tile_rows(g.hq, g.hkv), key_tile(g.d, g.dv)
    max_split = int(hdr[4])
    assert int(hdr[1]) == 0 and max_split > 1
    chunks = {}
    for s, row0, kt0, w in (tuple(int(x) for x in r) for r in tiles):
        chunks.setdefault((s, row0), []).append((kt0, w >> 5, (w >> 1) & 15, w & 1))
    expect = {(s, qt * rows) for s in range(g.nseg) for qt in range(-(-int(g.used_q[s]) // rows))}
    assert set(chunks) == expect
    for (s, row0), cs in chunks.items():
        nkt = key_tiles(g, rows, kt, s, row0)
        cs.sort()
        n = len(cs)
        assert 1 <= n <= max_split
        assert [c[2] for c in cs] == list(range(n))          # chunk indices 0..n-1
        assert all(c[3] == (1 if n > 1 else 0) for c in cs)  # partial flag iff split
        assert cs[0][0] == 0 and cs[-1][1] == nkt
        assert all(a[1] == b[0] for a, b in zip(cs, cs[1:]))  # contiguous, disjoint
