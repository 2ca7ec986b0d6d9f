"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (same entry points: Q and K each read once for block means
and FP4 codes, selection from the means; same block sizes and budgets).

Bit-exact over the whole tensors: selected block indices and counts, FP4
codes, block scales and slice scales.  The output is compared on sampled
query blocks that the oracle computes one by one (first, last, random, GQA
sibling heads, a planted pair's query block), to the same bounds as the
small-size parity tests.  The sweep covers both formats at every budget of
its workload (0, 1, 5, 25 and 100%).  Planted high-similarity pairs must be selected.
"""
import numpy as np
import pytest

from fp16_attention_amd import workloads as W
from tests.gpu_harness import compare_out, note, run_gpu, same_fp4

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

# name: (workload, fmt, topk_count, topk_bp)
CASES = {
    "prefill_mx_5pct": ("prefill", 1, -1, 500),
    "prefill_nvfp4_5pct": ("prefill", 0, -1, 500),
    "sweep_mx_0pct": ("sweep", 1, -1, 0),
    "sweep_mx_1pct": ("sweep", 1, -1, 100),
    "sweep_mx_5pct": ("sweep", 1, -1, 500),
    "sweep_mx_25pct": ("sweep", 1, -1, 2500),
    "sweep_mx_100pct": ("sweep", 1, -1, 10000),
    "sweep_nvfp4_0pct": ("sweep", 0, -1, 0),
    "sweep_nvfp4_1pct": ("sweep", 0, -1, 100),
    "sweep_nvfp4_5pct": ("sweep", 0, -1, 500),
    "sweep_nvfp4_25pct": ("sweep", 0, -1, 2500),
    "sweep_nvfp4_100pct": ("sweep", 0, -1, 10000),
    "long_mx_5pct": ("long", 1, -1, 500),
    "long_nvfp4_5pct": ("long", 0, -1, 500),
    "verylong_mx_2pct": ("verylong", 1, -1, 200),
    "dit_mx_5pct": ("dit", 1, -1, 500),
    "dit_nvfp4_5pct": ("dit", 0, -1, 500),
}

_inputs = {}
_quant = {}


def _data(name):
    if name not in _inputs:
        _inputs.clear()  # keep one full-size input set in host memory at a time
        _quant.clear()
        _inputs[name] = W.generate(W.WORKLOADS[name])
    return _inputs[name]


def _oracle_fp4(oracle, name, d, fmt):
    key = (name, fmt)
    if key not in _quant:
        _quant[key] = (oracle.quantize(d["q"], oracle.AXIS_D, fmt), oracle.quantize(d["k"], oracle.AXIS_D, fmt),
                       oracle.quantize(d["v"], oracle.AXIS_S, fmt))
    return _quant[key]


def _work_items(w, d, nq, seed):
    rng = np.random.default_rng(seed)
    items = [(0, 0, 0), (w.B - 1, w.Hq - 1, nq - 1)]
    b, h, i = int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(nq))
    items.append((b, h, i))
    G = w.Hq // w.Hkv
    if G > 1:  # a sibling head on the same KV head, same query block
        items.append((b, h + 1 if (h % G) + 1 < G else h - 1, i))
    if d["planted"]:
        pb, ph, pi = d["planted"][0][:3]
        items.append((pb, ph, pi))
    return sorted(set(items))


@pytest.mark.parametrize("name", list(CASES))
def test_fullsize_parity(oracle, name):
    wname, fmt, tc, bp = CASES[name]
    w = W.WORKLOADS[wname].with_(topk_count=tc, topk_bp=bp)
    note(f"[fullsize] {name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S} D{w.D} causal{int(w.causal)} "
         f"bq{w.bq} bk{w.bk} fmt{fmt} topk({tc},{bp})")
    d = _data(wname)
    g = run_gpu(d, w, fmt, tc, bp, fused=True)
    idx, cnt, _ = oracle.select(d["q"], d["k"], w.bq, w.bk, w.causal, tc, bp)
    assert np.array_equal(g["cnt"], cnt), "cnt differs"
    km = idx.shape[-1]
    assert np.array_equal(g["idx"][..., :km], idx), "idx differs"
    assert np.all(g["idx"][..., km:] == -1)
    for b, hq, i, j, *_ in d["planted"]:
        if bp > 0:
            assert j in g["idx"][b, hq, i, : g["cnt"][b, hq, i]], f"planted pair {(b, hq, i, j)} not selected"
    q4, k4, v4 = _oracle_fp4(oracle, wname, d, fmt)
    same_fp4(g["q4"], q4)
    same_fp4(g["k4"], k4)
    same_fp4(g["v4"], v4)
    nq = idx.shape[2]
    work = _work_items(w, d, nq, seed=len(name))
    note(f"    sampled query blocks (b, hq, i): {work}")
    o, lse, amb = oracle.attention(d["q"], d["k"], d["v"], q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal,
                                 work=work, with_amb=True)
    rows = [(b, h, slice(i * w.bq, min(w.S, (i + 1) * w.bq))) for b, h, i in work]
    compare_out(g["o"], o, g["lse"], lse, amb, rows=rows)
