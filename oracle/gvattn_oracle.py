"""FP64 CPU oracle for segmented ("gapped") varlen attention and its LSE merge.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously correct
definition that the HIP path is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product package never does, and the two share no code.

What it computes (the sources are the pages' own statements of the method):

* cosmos-framework PR #302, "What": every segment has a row capacity and a
  used prefix (seqused_q / seqused_k); the used query rows of a segment attend
  the used keys/values of the same segment only; rows past a segment's used
  length are left as they are; a segment with no keys gets a zero output and
  a -inf log-sum-exp.  PR #302, "Tests": the forward is checked against a
  per-segment FP64 reference -- this module is that reference.
* TensorRT-LLM issue #18687, "actual behavior" and "additional notes": keys
  past the used length must be masked, not merely zero, because a zero key
  has logit 0 and would add exp(0) = 1 to the softmax denominator.
* cosmos-framework PR #312, "Problem and behavior": GQA folding (several query
  heads share one KV head) and an FP32 LSE merge of the partial results of
  visibility partitions.
* The gradients (``attention_bwd``): the pages' path is forward-only (PR
  #302 makes the backward raise); the backward here is the calculus of the
  forward above, written out.
* TensorRT-LLM issue #18687, "additional notes", possible fix 1: after the Ulysses
  all-to-all the keys arrive rank-major, so a sample's valid keys are several
  runs of rows rather than one prefix.  ``attention_fwd_ranges`` takes each
  segment's keys as an ordered list of row ranges.

Readings taken where the pages leave a step open:

* query head h uses KV head ``h // (Hq // Hkv)`` (GQA folding, groups of
  consecutive heads);
* causal masks are aligned bottom-right inside each segment: row i (0-based
  in the segment) sees key j iff ``j <= i + used_k - used_q``;
* a row with no visible key (an empty segment, or a causal row above the
  diagonal when used_k < used_q) gets O = +0 and LSE = -inf;
* LSE is the natural log of sum_j exp(scale * q.k_j), scale included;
* layouts: Q [Tq, Hq, D], K [Tk, Hkv, D], V [Tk, Hkv, Dv], O [Tq, Hq, Dv],
  LSE [Hq, Tq] (the [H, total_q] layout named in the PR #302 review);
* the merge works on used rows only and leaves gap rows untouched.

Everything is computed in float64 from the exact input values (float32 arrays
whose values are bf16-exact for bf16 workloads; ``scale`` is the float32 value
the kernel uses, widened).
"""

from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

try:  # BLAS threads would oversubscribe the worker pool
    from threadpoolctl import threadpool_limits as _threadpool_limits
except Exception:  # pragma: no cover
    _threadpool_limits = None

# Row-block byte budget for the [rows, used_k] float64 score block.  The
# block's row count is max(1, budget // (used_k * 8)), the sizing rule the
# PR #302 review asks of the FP32 per-segment matmul path.
SCORE_BUDGET_BYTES = 64 << 20


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def visible_limit(i: np.ndarray, uq: int, uk: int, causal: bool) -> np.ndarray:
    """Number of keys row i of a segment may see (bottom-right causal)."""
    i = np.asarray(i, dtype=np.int64)
    if not causal:
        return np.full(i.shape, uk, dtype=np.int64)
    return np.clip(i + uk - uq + 1, 0, uk)


def segment_head_rows(q, k, v, q0: int, k0: int, uq: int, uk: int, h: int,
                      hkv_of_h: int, scale: float, causal: bool,
                      rows: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Attention of the given segment rows (indices in [0, uq)) for one query
    head.  Returns (O [n, Dv] float64, LSE [n] float64)."""
    rows = np.asarray(rows, dtype=np.int64)
    dv = v.shape[2]
    n = rows.shape[0]
    o = np.zeros((n, dv), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    if n == 0 or uk == 0:
        return o, lse
    qs = np.asarray(q[q0 + rows, h, :], dtype=np.float64)            # [n, D]
    ks = np.asarray(k[k0:k0 + uk, hkv_of_h, :], dtype=np.float64)    # [uk, D]
    vs = np.asarray(v[k0:k0 + uk, hkv_of_h, :], dtype=np.float64)    # [uk, Dv]
    s = float(scale) * (qs @ ks.T)                                   # [n, uk]
    if causal:
        lim = visible_limit(rows, uq, uk, True)                      # [n]
        cols = np.arange(uk, dtype=np.int64)
        s = np.where(cols[None, :] < lim[:, None], s, -np.inf)
    m = s.max(axis=1)                                                # [n]
    live = m > -np.inf
    if not live.any():
        return o, lse
    sl, ml = s[live], m[live]
    p = np.exp(sl - ml[:, None])
    l = p.sum(axis=1)
    o[live] = (p @ vs) / l[:, None]
    lse[live] = ml + np.log(l)
    # NaN inputs inside the used rows propagate (max ignores nothing here).
    nan_rows = np.isnan(m)
    if nan_rows.any():
        o[nan_rows] = np.nan
        lse[nan_rows] = np.nan
    return o, lse


def _work_items(cu_q, cu_k, used_q, used_k, hq, hkv):
    g = hq // hkv
    for s in range(len(used_q)):
        uq, uk = int(used_q[s]), int(used_k[s])
        if uq == 0:
            continue
        for h in range(hq):
            yield s, h, h // g, int(cu_q[s]), int(cu_k[s]), uq, uk


def attention_fwd(q, k, v, cu_q, cu_k, used_q, used_k, scale, causal,
                  out_init=None, lse_init=None, workers: int | None = None,
                  segments=None):
    """Whole-launch oracle.  Returns (O [Tq, Hq, Dv] float64,
    LSE [Hq, Tq] float64); rows not written keep ``out_init``/``lse_init``
    (zeros when not given).  ``segments`` restricts the work to a subset of
    segments (their rows only are written)."""
    tq, hq, _ = q.shape
    hkv, dv = k.shape[1], v.shape[2]
    if hq % hkv:
        raise ValueError(f"hq={hq} is not a multiple of hkv={hkv}")
    out = (np.zeros((tq, hq, dv)) if out_init is None
           else np.array(out_init, dtype=np.float64, copy=True))
    lse = (np.zeros((hq, tq)) if lse_init is None
           else np.array(lse_init, dtype=np.float64, copy=True))
    items = list(_work_items(cu_q, cu_k, used_q, used_k, hq, hkv))
    if segments is not None:
        keep = set(int(s) for s in segments)
        items = [it for it in items if it[0] in keep]

    def run(item):
        s, h, g, q0, k0, uq, uk = item
        step = max(1, SCORE_BUDGET_BYTES // (max(uk, 1) * 8))
        for r0 in range(0, uq, step):
            rows = np.arange(r0, min(uq, r0 + step))
            o, l = segment_head_rows(q, k, v, q0, k0, uq, uk, h, g, scale,
                                     causal, rows)
            out[q0 + rows, h, :] = o
            lse[h, q0 + rows] = l

    workers = workers or host_cores()
    if workers <= 1 or len(items) <= 1:
        for it in items:
            run(it)
    else:
        ctx = (_threadpool_limits(limits=1) if _threadpool_limits is not None
               else _NullCtx())
        with ctx, _cf.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(run, items))
    return out, lse


def segment_key_rows(kr_off, kr_start, kr_len, s: int) -> np.ndarray:
    """Row indices of segment s's keys: the concatenation, in list order, of
    its ranges [kr_start[i], kr_start[i] + kr_len[i]) for i in
    [kr_off[s], kr_off[s + 1])."""
    parts = [np.arange(int(kr_start[i]), int(kr_start[i]) + int(kr_len[i]), dtype=np.int64)
             for i in range(int(kr_off[s]), int(kr_off[s + 1]))]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def attention_fwd_ranges(q, k, v, cu_q, used_q, kr_off, kr_start, kr_len, scale, causal,
                         out_init=None, lse_init=None, workers: int | None = None):
    """Whole-launch oracle when every segment's keys are a list of row ranges
    (issue #18687, "additional notes", possible fix 1).  The segment's key sequence is the
    concatenation of its ranges; with it gathered, the computation is the one
    of ``attention_fwd`` with used_k = the total length (causal alignment is
    bottom-right over that sequence)."""
    tq, hq, _ = q.shape
    hkv, dv = k.shape[1], v.shape[2]
    if hq % hkv:
        raise ValueError(f"hq={hq} is not a multiple of hkv={hkv}")
    out = (np.zeros((tq, hq, dv)) if out_init is None
           else np.array(out_init, dtype=np.float64, copy=True))
    lse = (np.zeros((hq, tq)) if lse_init is None
           else np.array(lse_init, dtype=np.float64, copy=True))
    g = hq // hkv
    items = []
    for s in range(len(used_q)):
        uq = int(used_q[s])
        if uq == 0:
            continue
        keys = segment_key_rows(kr_off, kr_start, kr_len, s)
        for h in range(hq):
            items.append((s, h, keys))

    def run(item):
        s, h, keys = item
        q0, uq, uk = int(cu_q[s]), int(used_q[s]), len(keys)
        ks, vs = k[keys], v[keys]                        # gathered [uk, Hkv, *]
        step = max(1, SCORE_BUDGET_BYTES // (max(uk, 1) * 8))
        for r0 in range(0, uq, step):
            rows = np.arange(r0, min(uq, r0 + step))
            o, l = segment_head_rows(q, ks, vs, q0, 0, uq, uk, h, h // g, scale, causal, rows)
            out[q0 + rows, h, :] = o
            lse[h, q0 + rows] = l

    workers = workers or host_cores()
    if workers <= 1 or len(items) <= 1:
        for it in items:
            run(it)
    else:
        ctx = (_threadpool_limits(limits=1) if _threadpool_limits is not None
               else _NullCtx())
        with ctx, _cf.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(run, items))
    return out, lse


def attention_bwd(q, k, v, do, cu_q, cu_k, used_q, used_k, scale, causal,
                  dq_init=None, dk_init=None, dv_init=None):
    """Gradients of the segmented forward, from its definition, in float64.

    For every segment and query head h (KV head g = h // (Hq/Hkv)), with
    S = scale * Q K^T over the used rows and keys (masked entries -inf),
    P = softmax(S) row by row (a row with no visible key has P = 0) and
    O = P V:  dV_g += P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dP * P)),
    dQ = scale * dS K,  dK_g += scale * dS^T Q.  The heads of a KV group add
    into one dK / dV.  Rows outside the used prefixes keep the initial
    values (zeros when not given); used keys that no row sees get 0.
    The pages' path is forward-only; this is the plain calculus of the
    forward they define."""
    tq, hq, d = q.shape
    tk, hkv, dv = v.shape
    grp = hq // hkv
    dq = np.zeros((tq, hq, d)) if dq_init is None else np.array(dq_init, np.float64, copy=True)
    dk = np.zeros((tk, hkv, d)) if dk_init is None else np.array(dk_init, np.float64, copy=True)
    dvo = np.zeros((tk, hkv, dv)) if dv_init is None else np.array(dv_init, np.float64, copy=True)
    for s in range(len(used_q)):
        q0, k0 = int(cu_q[s]), int(cu_k[s])
        uq, uk = int(used_q[s]), int(used_k[s])
        if uq > 0:
            dq[q0:q0 + uq] = 0.0
        if uk > 0:
            dk[k0:k0 + uk] = 0.0
            dvo[k0:k0 + uk] = 0.0
        if uq == 0 or uk == 0:
            continue
        lim = visible_limit(np.arange(uq), uq, uk, causal)
        vis = np.arange(uk)[None, :] < lim[:, None]                  # [uq, uk]
        live = lim > 0
        for h in range(hq):
            g = h // grp
            qs = np.asarray(q[q0:q0 + uq, h], np.float64)
            ks = np.asarray(k[k0:k0 + uk, g], np.float64)
            vs = np.asarray(v[k0:k0 + uk, g], np.float64)
            dos = np.asarray(do[q0:q0 + uq, h], np.float64)
            sc = float(scale) * (qs @ ks.T)
            sc = np.where(vis, sc, -np.inf)
            p = np.zeros_like(sc)
            m = sc[live].max(axis=1, keepdims=True)
            e = np.exp(sc[live] - m)
            p[live] = e / e.sum(axis=1, keepdims=True)
            dvo[k0:k0 + uk, g] += p.T @ dos
            dp = dos @ vs.T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            dq[q0:q0 + uq, h] = float(scale) * (ds @ ks)
            dk[k0:k0 + uk, g] += float(scale) * (ds.T @ qs)
    return dq, dk, dvo


def attention_bwd_magnitudes(q, k, v, do, cu_q, cu_k, used_q, used_k, scale, causal):
    """Absolute-value sums that bound the rounding error of a backward that
    rounds P, dS and O to a 16-bit type (used by the tests to state their
    tolerance; not a result of the method).  With P and dS as in
    ``attention_bwd``, O = P V and Dabs_i = sum_e |dO_ie| |O_ie|:

        A_dv[j] = sum_h sum_i P_ij |dO_i|
        A_dq[i] = scale * sum_j (|dS_ij| + P_ij * Dabs_i) |K_j|
        A_dk[j] = scale * sum_h sum_i (|dS_ij| + P_ij * Dabs_i) |Q_i|

    Rounding P (for dV), dS (for dQ, dK) and O (in D = rowsum(dO * O)) with
    unit roundoff u, and accumulating in FP32, leaves each gradient within
    about u * (|exact| + A) of the exact one.  Returns (A_dq, A_dk, A_dv)
    with the shapes of the gradients; zero outside the used rows."""
    tq, hq, d = q.shape
    tk, hkv, dv = v.shape
    grp = hq // hkv
    a_dq = np.zeros((tq, hq, d))
    a_dk = np.zeros((tk, hkv, d))
    a_dv = np.zeros((tk, hkv, dv))
    for s in range(len(used_q)):
        q0, k0 = int(cu_q[s]), int(cu_k[s])
        uq, uk = int(used_q[s]), int(used_k[s])
        if uq == 0 or uk == 0:
            continue
        lim = visible_limit(np.arange(uq), uq, uk, causal)
        vis = np.arange(uk)[None, :] < lim[:, None]
        live = lim > 0
        for h in range(hq):
            g = h // grp
            qs = np.asarray(q[q0:q0 + uq, h], np.float64)
            ks = np.asarray(k[k0:k0 + uk, g], np.float64)
            vs = np.asarray(v[k0:k0 + uk, g], np.float64)
            dos = np.asarray(do[q0:q0 + uq, h], np.float64)
            sc = np.where(vis, float(scale) * (qs @ ks.T), -np.inf)
            p = np.zeros_like(sc)
            m = sc[live].max(axis=1, keepdims=True)
            e = np.exp(sc[live] - m)
            p[live] = e / e.sum(axis=1, keepdims=True)
            dp = dos @ vs.T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            dabs = (np.abs(dos) * np.abs(p @ vs)).sum(axis=1, keepdims=True)
            w = np.abs(ds) + p * dabs
            a_dv[k0:k0 + uk, g] += p.T @ np.abs(dos)
            a_dq[q0:q0 + uq, h] = float(scale) * (w @ np.abs(ks))
            a_dk[k0:k0 + uk, g] += float(scale) * (w.T @ np.abs(qs))
    return a_dq, a_dk, a_dv


class _NullCtx:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def lse_merge(part_out, part_lse, cu_q, used_q, out_init=None, lse_init=None):
    """Merge the (O_p, LSE_p) partials of several key partitions, row by row
    and head by head, in float64 (cosmos-framework PR #312, "Problem and
    behavior": visibility partitions combined by an FP32 LSE merge).

    For each used row and head: m = max_p LSE_p; if m = -inf the result is
    O = 0, LSE = -inf; otherwise w_p = exp(LSE_p - m), W = sum_p w_p,
    LSE = m + ln W and O = sum_p (w_p / W) O_p.  Gap rows keep the initial
    values."""
    tq, hq, dv = part_out[0].shape
    out = (np.zeros((tq, hq, dv)) if out_init is None
           else np.array(out_init, dtype=np.float64, copy=True))
    lse = (np.zeros((hq, tq)) if lse_init is None
           else np.array(lse_init, dtype=np.float64, copy=True))
    for s in range(len(used_q)):
        q0, uq = int(cu_q[s]), int(used_q[s])
        if uq == 0:
            continue
        rows = slice(q0, q0 + uq)
        L = np.stack([np.asarray(pl[:, rows], np.float64) for pl in part_lse])  # [P, Hq, uq]
        O = np.stack([np.asarray(po[rows], np.float64) for po in part_out])     # [P, uq, Hq, Dv]
        m = L.max(axis=0)                                                        # [Hq, uq]
        dead = m == -np.inf
        m_safe = np.where(dead, 0.0, m)
        w = np.exp(L - m_safe[None])                                             # [P, Hq, uq]
        W = w.sum(axis=0)
        with np.errstate(divide="ignore", invalid="ignore"):
            merged_lse = np.where(dead, -np.inf, m_safe + np.log(W))
            frac = np.where(dead[None], 0.0, w / W[None])                        # [P, Hq, uq]
        frac_t = np.transpose(frac, (0, 2, 1))[..., None]                        # [P, uq, Hq, 1]
        merged = (frac_t * O).sum(axis=0)
        merged[np.transpose(dead)] = 0.0
        out[rows] = merged
        lse[:, rows] = merged_lse
    return out, lse


def attention_flops(used_q, used_k, hq: int, d: int, dv: int, causal: bool) -> int:
    """Algorithmic FLOPs of one forward over used rows: every visible
    (query, key) pair costs 2*d (scores) + 2*dv (P.V) per query head."""
    pairs = 0
    for uq, uk in zip(used_q, used_k):
        uq, uk = int(uq), int(uk)
        if uq == 0 or uk == 0:
            continue
        if not causal:
            pairs += uq * uk
        else:
            pairs += int(visible_limit(np.arange(uq), uq, uk, True).sum())
    return pairs * hq * (2 * d + 2 * dv)


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    """Bitwise equality of two float32 arrays (used for gap-row checks)."""
    a = np.ascontiguousarray(a, np.float32).view(np.uint32)
    b = np.ascontiguousarray(b, np.float32).view(np.uint32)
    return bool(np.array_equal(a, b))


__all__ = [
    "attention_fwd", "attention_fwd_ranges", "attention_bwd", "segment_key_rows", "lse_merge", "segment_head_rows", "visible_limit",
    "attention_flops", "host_cores", "bits_equal", "SCORE_BUDGET_BYTES",
]
