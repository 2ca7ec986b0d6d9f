"""Shared GPU-vs-oracle harness for the parity tests (test helper)."""
from __future__ import annotations

import sys

import numpy as np

from fp16_attention_amd import workloads as W

MAX_ABS = 2e-3  # element-wise bound on the fp32 output against the oracle
REL_L2 = 1e-3   # relative L2 bound on the whole compared output


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


def compare_out(go, ro, gl, rl, u, rows=None):
    """Output within MAX_ABS (plus the oracle's decision uncertainty u, the
    most that rounding decisions lying within fp32 evaluation error of their
    boundary can move an element) and REL_L2; rows selects (b, hq, row-slice)
    items."""
    if rows is not None:
        go = np.concatenate([go[b, h, sl].ravel() for b, h, sl in rows])
        ro = np.concatenate([ro[b, h, sl].ravel() for b, h, sl in rows])
        gl = np.concatenate([gl[b, h, sl].ravel() for b, h, sl in rows])
        rl = np.concatenate([rl[b, h, sl].ravel() for b, h, sl in rows])
        u = np.concatenate([u[b, h, sl].ravel() for b, h, sl in rows])
    assert np.all(np.isfinite(go)), "non-finite output"
    err = np.abs(go - ro)
    rel = np.linalg.norm(go - ro) / max(np.linalg.norm(ro), 1e-30)
    lerr = np.abs(gl - rl)
    excess = err - u
    note(f"    max-abs {err.max():.3e} (beyond u: {excess.max():.3e}, elements with u > 2e-3: "
         f"{np.mean(u > MAX_ABS):.2e})  rel-L2 {rel:.3e}  lse max-abs {lerr.max():.3e}")
    assert excess.max() <= MAX_ABS, f"max-abs beyond decision uncertainty {excess.max():.3e}"
    assert rel <= REL_L2, f"rel-L2 {rel:.3e}"
    assert np.mean(u > MAX_ABS) < 0.05, "decision uncertainty covers too many elements"
    assert np.all(lerr <= 1e-3 + 1e-5 * np.abs(rl)), f"lse max-abs {lerr.max():.3e}"
    return err.max(), rel


def workload(name, **kw):
    return W.WORKLOADS[name].with_(**kw)
