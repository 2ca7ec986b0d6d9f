"""Shared GPU-vs-oracle harness for the parity tests (test helper).

The output check: every element within MAX_ABS of the oracle's, after the
oracle's own list of decisions that may go either way is taken into account.
A decision (a P code, a block scale, an fp16 rounding) whose exact input lies
within the device's evaluation error of its rounding boundary has two valid
outcomes; the oracle lists each with the exact change of its output row if
the other outcome is taken.  A row that misses MAX_ABS must be matched within
MAX_ABS by the oracle's row with some set of its listed decisions flipped
(resolve_row); the report counts the elements beyond MAX_ABS and the
decisions the match needed.  Nothing else widens the bound.
"""
from __future__ import annotations

import itertools
import sys

import numpy as np

from fp16_attention_amd import workloads as W

MAX_ABS = 2e-3  # element-wise bound on the fp32 output against the oracle
REL_L2 = 1e-3   # relative L2 bound on the whole compared output
SMALL = 1e-6    # decisions moving a row by at most this much are summed, not searched
MAX_FLIPS = 3   # decisions one row may need flipped at once
MAX_CAND = 24   # candidates searched per row (ranked by how well each alone explains the error)


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(d, w, fmt, topk_count, topk_bp, no_fp16=False, fused=False, p_fmt=None):
    """The path on the GPU: separate selection and quantisation calls, or
    (fused) Q and K each read once for means and codes, as the benchmark runs it."""
    import torch

    from fp16_attention_amd import api

    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(np.ascontiguousarray(d[n])).to(dev) for n in ("q", "k", "v"))
    if fused:
        q4, qbar = api.thrift_quantize_fp4_means(q, fmt, w.bq)
        k4, kbar = api.thrift_quantize_fp4_means(k, fmt, w.bk)
        idx, cnt = api.thrift_select_blocks_means(qbar, kbar, w.S, w.S, w.bq, w.bk, w.causal, topk_count,
                                                  topk_bp)
    else:
        idx, cnt = api.thrift_select_blocks(q, k, w.bq, w.bk, w.causal, topk_count, topk_bp)
        q4 = api.thrift_quantize_fp4(q, api.THRIFT_GROUP_D, fmt)
        k4 = api.thrift_quantize_fp4(k, api.THRIFT_GROUP_D, fmt)
    v4 = api.thrift_quantize_fp4(v, api.THRIFT_GROUP_S, fmt)
    args = (None, None, None) if no_fp16 else (q, k, v)
    o, lse = api.thrift_attention_fwd(*args, q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal,
                                      out_fp32=True, with_lse=True, p_fmt=p_fmt)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.cpu().numpy()  # noqa: E731
    return dict(idx=cpu(idx), cnt=cpu(cnt), q4=q4, k4=k4, v4=v4, o=cpu(o).astype(np.float64),
                lse=cpu(lse).astype(np.float64), tensors=(q, k, v, idx, cnt))


def same_fp4(g, r):
    from fp16_attention_amd import api

    codes, scales = api.fp4_transposed(g)  # the oracle keeps V^T in plain transposed order
    assert np.array_equal(codes.cpu().numpy(), r.codes), "FP4 codes differ"
    assert np.array_equal(scales.cpu().numpy(), r.scales), "FP4 block scales differ"
    if r.tensor_scale is not None:
        assert np.array_equal(g.tensor_scale.cpu().numpy(), r.tensor_scale), "slice scales differ"


def resolve_row(err, deltas, tol=MAX_ABS):
    """Match one output row's error err [D] (device minus oracle) by flipping
    decisions of the oracle's list for that row (deltas [k, D], the change of
    the row per decision).  Decisions whose effect is at most SMALL are not
    searched: the sum of their magnitudes is added to the tolerance (any set
    of them moves the row by no more).  The others are searched in sets of up
    to MAX_FLIPS among the MAX_CAND that best explain err alone.  Returns
    (residual beyond tol, flips used, allowance): residual <= 0 is a match."""
    deltas = np.asarray(deltas, np.float64).reshape(-1, err.shape[-1])
    big = np.abs(deltas).max(1) > SMALL
    allow = np.abs(deltas[~big]).sum(0)
    cand = deltas[big]
    best = (np.max(np.abs(err) - allow) - tol, 0)
    if best[0] <= 0 or len(cand) == 0:
        return best[0], 0, float(allow.max(initial=0.0))
    # rank by how much each decision alone reduces the worst element
    alone = np.max(np.abs(err[None, :] - cand) - allow[None, :], axis=1)
    order = np.argsort(alone)[:MAX_CAND]
    cand = cand[order]
    for size in range(1, min(MAX_FLIPS, len(cand)) + 1):
        for comb in itertools.combinations(range(len(cand)), size):
            r = np.max(np.abs(err - cand[list(comb)].sum(0)) - allow) - tol
            if r < best[0]:
                best = (r, size)
        if best[0] <= 0:
            break
    return best[0], best[1], float(allow.max(initial=0.0))


def compare_out(go, ro, gl, rl, amb, rows=None):
    """Output within MAX_ABS of the oracle's once the oracle's decisions that
    may go either way are resolved (resolve_row), and within REL_L2; LSE
    within 1e-3 + 1e-5 |LSE|.  rows selects (b, hq, row-slice) items; amb is
    the oracle's Ambiguity list of the compared forward."""
    B, Hq, S, D = go.shape
    if rows is None:
        rows = [(b, h, slice(0, S)) for b in range(B) for h in range(Hq)]
    sel = [(b, h, np.arange(S)[sl]) for b, h, sl in rows]
    G = np.concatenate([go[b, h, rr] for b, h, rr in sel])
    R = np.concatenate([ro[b, h, rr] for b, h, rr in sel])
    GL = np.concatenate([gl[b, h, rr] for b, h, rr in sel])
    RL = np.concatenate([rl[b, h, rr] for b, h, rr in sel])
    flat = np.concatenate([(b * Hq + h) * S + rr for b, h, rr in sel])
    assert np.all(np.isfinite(G)), "non-finite output"
    err = G - R
    rel = np.linalg.norm(err) / max(np.linalg.norm(R), 1e-30)
    lerr = np.abs(GL - RL)
    over = np.abs(err) > MAX_ABS
    bad_rows = np.nonzero(over.any(1))[0]
    n_listed = int(np.isin(amb.rows, flat).sum())
    worst, used, max_allow, unresolved = -np.inf, 0, 0.0, []
    order = np.argsort(amb.rows, kind="stable")
    srows = amb.rows[order]
    for k in bad_rows:
        lo, hi = np.searchsorted(srows, flat[k]), np.searchsorted(srows, flat[k], side="right")
        res, nf, al = resolve_row(err[k], amb.delta[order[lo:hi]])
        worst, used, max_allow = max(worst, res), max(used, nf), max(max_allow, al)
        if res > 0:
            unresolved.append((int(flat[k]), float(np.abs(err[k]).max()), hi - lo, float(res)))
    note(f"    max-abs {np.abs(err).max():.3e}  rel-L2 {rel:.3e}  lse max-abs {lerr.max():.3e}  |  "
         f"elements beyond {MAX_ABS:g}: {int(over.sum())} in {len(bad_rows)} rows (of {len(flat)}), "
         f"matched by flipping up to {used} listed decisions per row (residual {worst if len(bad_rows) else 0:.2e}, "
         f"summed allowance {max_allow:.1e}); decisions listed for the compared rows: {n_listed}")
    assert not unresolved, f"rows beyond {MAX_ABS} not explained by listed decisions (row, max err, listed, " \
                           f"residual): {unresolved[:8]}"
    assert rel <= REL_L2, f"rel-L2 {rel:.3e}"
    assert np.all(lerr <= 1e-3 + 1e-5 * np.abs(RL)), f"lse max-abs {lerr.max():.3e}"
    return float(np.abs(err).max()), rel


def workload(name, **kw):
    return W.WORKLOADS[name].with_(**kw)
