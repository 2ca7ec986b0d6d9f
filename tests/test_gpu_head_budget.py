"""GPU parity of the per-head budget variant (thrift_select_blocks_head):
one top-k over all valid block pairs of a query head, against the oracle,
bit-exact on idx and cnt; then the mixed forward driven by that selection
against the oracle's forward on the same selection (the bounds of the other
forward parity tests).  Cases: causal and not, GQA, queries at the end of a
longer key sequence, the budget extremes, an absolute count, all scores
equal (every tie decided by position), and the long workload at full size.
"""
import numpy as np
import pytest

from fp16_attention_amd import workloads as W
from tests.gpu_harness import compare_out, note

pytestmark = pytest.mark.gpu

CASES = {
    # name: (B, Hq, Hkv, Sq, Sk, D, causal, bq, topk_count, bp)
    "causal_gqa": (1, 4, 2, 1000, 1000, 64, True, 128, -1, 1000),
    "noncausal_b2": (2, 4, 2, 700, 700, 64, False, 64, -1, 500),
    "end_aligned": (1, 2, 2, 300, 1300, 128, True, 128, -1, 2500),
    "none": (1, 2, 1, 900, 900, 128, True, 128, -1, 0),
    "all": (1, 2, 1, 900, 900, 128, True, 128, -1, 10000),
    "absolute": (1, 2, 1, 900, 900, 128, True, 128, 37, 0),
    "long_rows": (1, 2, 1, 8192, 8192, 64, True, 128, -1, 300),
}


def _inputs(B, Hq, Hkv, Sq, Sk, D, seed):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, Hq, Sq, D)) * 0.7).astype(np.float16)
    k = (rng.standard_normal((B, Hkv, Sk, D)) * 0.7).astype(np.float16)
    v = rng.standard_t(3, size=(B, Hkv, Sk, D)).astype(np.float16)
    k[:, :, :64] *= 3
    return q, k, v


def _gpu_select(q, k, bq, causal, tc, bp):
    import torch

    from fp16_attention_amd import api

    qd, kd = torch.from_numpy(q).to("cuda:0"), torch.from_numpy(k).to("cuda:0")
    _, qbar = api.thrift_quantize_fp4_means(qd, api.THRIFT_MXFP4, bq)
    _, kbar = api.thrift_quantize_fp4_means(kd, api.THRIFT_MXFP4, 64)
    idx, cnt = api.thrift_select_blocks_head(qbar, kbar, q.shape[2], k.shape[2], bq, 64, causal, tc, bp)
    torch.cuda.synchronize()
    return idx, cnt


@pytest.mark.parametrize("name", list(CASES))
def test_head_budget_selection(oracle, name):
    B, Hq, Hkv, Sq, Sk, D, causal, bq, tc, bp = CASES[name]
    note(f"[head] {name}: B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} D{D} causal{int(causal)} bq{bq} topk({tc},{bp})")
    q, k, _ = _inputs(B, Hq, Hkv, Sq, Sk, D, len(name))
    idx, cnt = _gpu_select(q, k, bq, causal, tc, bp)
    ridx, rcnt = oracle.select_head(q, k, bq, 64, causal, tc, bp, kmax_=idx.shape[-1])
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(idx.cpu().numpy(), ridx)


def test_head_budget_all_ties(oracle):
    q, k, _ = _inputs(1, 2, 1, 1000, 1000, 64, 5)
    q[:] = 0  # every score 0: the kept pairs are the first K in (query block, key block) order
    note("[head] all scores equal")
    idx, cnt = _gpu_select(q, k, 128, True, -1, 1500)
    ridx, rcnt = oracle.select_head(q, k, 128, 64, True, -1, 1500, kmax_=idx.shape[-1])
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(idx.cpu().numpy(), ridx)


def test_head_budget_forward(oracle):
    import torch

    from fp16_attention_amd import api

    q, k, v = _inputs(1, 4, 2, 1500, 1500, 128, 6)
    note("[head] forward: B1 Hq4 Hkv2 S1500 D128 causal, 5% per head, MX")
    dev = torch.device("cuda:0")
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o, lse = api.thrift_forward(qd, kd, vd, api.THRIFT_MXFP4, 128, 64, True, -1, 500, out_fp32=True,
                                with_lse=True, budget="head")
    torch.cuda.synchronize()
    ridx, rcnt = oracle.select_head(q, k, 128, 64, True, -1, 500)
    q4, k4 = oracle.quantize(q, oracle.AXIS_D, oracle.MX), oracle.quantize(k, oracle.AXIS_D, oracle.MX)
    v4 = oracle.quantize(v, oracle.AXIS_S, oracle.MX)
    ro, rl, amb = oracle.attention(q, k, v, q4, k4, v4, ridx, rcnt, 128, 64, True, with_amb=True)
    compare_out(o.cpu().numpy().astype(np.float64), ro, lse.cpu().numpy().astype(np.float64), rl, amb)


@pytest.mark.slow
def test_head_budget_long_full_size(oracle):
    w = W.WORKLOADS["long"]
    note(f"[head] full size: {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S} 5% per head")
    d = W.generate(w)
    idx, cnt = _gpu_select(d["q"], d["k"], w.bq, w.causal, -1, w.topk_bp)
    ridx, rcnt = oracle.select_head(d["q"], d["k"], w.bq, w.bk, w.causal, -1, w.topk_bp, kmax_=idx.shape[-1])
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    for b, hq, i, j, *_ in d["planted"]:
        assert j in idx[b, hq, i, : cnt[b, hq, i]].cpu().numpy(), f"planted pair {(b, hq, i, j)} not kept"
