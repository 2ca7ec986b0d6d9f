"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: selected block indices and counts, FP4 codes, block scales and
slice scales.  Output: fp32 O within max-abs 2e-3 and rel-L2 1e-3 of the
oracle's result, log-sum-exp within 1e-3 (+1e-5 relative).  The max-abs
bound is widened, element by element, by the oracle's decision uncertainty u:
where a rounding decision of P (fp16 rounding, E2M1 code, block scale) has
its input within fp32 evaluation error of the boundary, either outcome is a
valid result of the method, and u is the most such flips can move O.  Sizes here are
small enough for the oracle to finish in seconds while spanning several
tiles, ragged tails, GQA, both formats and the budget extremes.
"""
import numpy as np
import pytest

from fp16_attention_amd import workloads as W
from tests.gpu_harness import compare_out, note, run_gpu, same_fp4, workload

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, fmt, topk_count, topk_bp)
    "tiny_nvfp4": (workload("tiny"), 0, 2, 0),
    "tiny_mx": (workload("tiny"), 1, 2, 0),
    "prefill_mx": (workload("prefill", Hq=4, Hkv=4, S=1000), 1, -1, 500),
    "prefill_nvfp4": (workload("prefill", Hq=4, Hkv=4, S=1000), 0, -1, 500),
    "gqa_ragged_mx": (workload("sweep", B=2, Hq=4, Hkv=2, S=700), 1, -1, 2500),
    "gqa_ragged_nvfp4": (workload("sweep", B=2, Hq=4, Hkv=2, S=700), 0, -1, 2500),
    "long_sink_planted_mx": (workload("long", Hq=4, Hkv=2, S=2048, planted=2), 1, -1, 500),
    "dit_ragged_mx": (workload("dit", Hq=2, Hkv=2, S=1000), 1, -1, 500),
    "dit_ragged_nvfp4": (workload("dit", Hq=2, Hkv=2, S=1000), 0, -1, 500),
    "bq64_mx": (workload("prefill", Hq=2, Hkv=2, S=513, bq=64), 1, -1, 1000),
    "all_fp16": (workload("prefill", Hq=2, Hkv=1, S=640), 1, -1, 10000),
    "none_fp16_mx": (workload("prefill", Hq=2, Hkv=1, S=640), 1, -1, 0),
    "none_fp16_nvfp4": (workload("prefill", Hq=2, Hkv=1, S=640), 0, -1, 0),
    "single_block": (workload("tiny", S=64), 1, 1, 0),
    "short_tail": (workload("prefill", Hq=1, Hkv=1, S=37), 1, -1, 500),
    "short_tail_nvfp4": (workload("prefill", Hq=1, Hkv=1, S=37), 0, -1, 500),
    "bq64_nvfp4": (workload("prefill", Hq=2, Hkv=2, S=513, bq=64), 0, -1, 1000),
    "single_block_nvfp4": (workload("tiny", S=64), 0, 1, 0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_parity(oracle, name):
    w, fmt, tc, bp = CASES[name]
    note(f"[parity] {name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S} D{w.D} causal{int(w.causal)} "
         f"bq{w.bq} fmt{fmt} topk({tc},{bp})")
    d = W.generate(w)
    g = run_gpu(d, w, fmt, tc, bp, no_fp16=(bp == 0 and tc <= 0))
    r = oracle.pipeline(d["q"], d["k"], d["v"], fmt, w.bq, w.bk, w.causal, tc, bp)
    assert np.array_equal(g["cnt"], r["cnt"]), "cnt differs"
    km = r["idx"].shape[-1]  # the GPU row may be longer (kmax >= 1): -1 beyond
    assert np.array_equal(g["idx"][..., :km], r["idx"]), "idx differs"
    assert np.all(g["idx"][..., km:] == -1)
    same_fp4(g["q4"], r["q4"])
    same_fp4(g["k4"], r["k4"])
    same_fp4(g["v4"], r["v4"])
    compare_out(g["o"], r["o"], g["lse"], r["lse"], r["amb"])


VARIANT_CASES = {
    # NVFP4 Q, K, V with P quantised MX-style (THRIFT_NVFP4_MXP)
    "prefill": (workload("prefill", Hq=4, Hkv=4, S=1000), -1, 500),
    "gqa_ragged": (workload("sweep", B=2, Hq=4, Hkv=2, S=700), -1, 2500),
    "none_fp16": (workload("prefill", Hq=2, Hkv=1, S=640), -1, 0),
    "bq64_d64": (workload("dit", Hq=2, Hkv=2, S=513, bq=64), -1, 1000),
}


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ties", ["groups", "all"])
def test_selection_ties(oracle, causal, ties):
    """Key blocks holding the same data score exactly alike.  For every
    budget k the GPU selection equals the oracle's bit for bit: the k-th
    largest score is found exactly (the search may stop early, once exactly
    k scores lie at or above a prefix), and of the blocks tied at it the
    lower-indexed ones are taken."""
    import torch

    from fp16_attention_amd import api

    w = workload("prefill", Hq=2, Hkv=1, S=1024)  # 16 key blocks of 64, 8 query blocks of 128
    note(f"[selection ties] {ties} causal{int(causal)}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S}")
    d = W.generate(w)
    k = d["k"].copy()
    if ties == "groups":  # blocks 3, 5, 8, 12 alike, and 1, 9
        for j in (5, 8, 12):
            k[:, :, j * 64:(j + 1) * 64] = k[:, :, 3 * 64:4 * 64]
        k[:, :, 9 * 64:10 * 64] = k[:, :, 64:128]
    else:  # every block alike
        for j in range(1, 16):
            k[:, :, j * 64:(j + 1) * 64] = k[:, :, :64]
    dev = torch.device("cuda:0")
    qd, kd = torch.from_numpy(d["q"]).to(dev), torch.from_numpy(k).to(dev)
    for tc in range(0, 17):
        idx, cnt = api.thrift_select_blocks(qd, kd, w.bq, w.bk, causal, tc, 0)
        r_idx, r_cnt, _ = oracle.select(d["q"], k, w.bq, w.bk, causal, tc, 0)
        gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
        assert np.array_equal(gc, r_cnt), f"cnt differs at k={tc}"
        km = r_idx.shape[-1]
        assert np.array_equal(gi[..., :km], r_idx), f"idx differs at k={tc}"
        assert np.all(gi[..., km:] == -1)


@pytest.mark.parametrize("name", list(VARIANT_CASES))
def test_parity_nvfp4_tensors_mx_p(oracle, name):
    w, tc, bp = VARIANT_CASES[name]
    note(f"[parity, NVFP4 tensors + MX P] {name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S} D{w.D} bq{w.bq} topk({tc},{bp})")
    d = W.generate(w)
    g = run_gpu(d, w, 0, tc, bp, no_fp16=(bp == 0 and tc <= 0), p_fmt=1)
    r = oracle.pipeline(d["q"], d["k"], d["v"], 0, w.bq, w.bk, w.causal, tc, bp, p_fmt=1)
    assert np.array_equal(g["cnt"], r["cnt"])
    same_fp4(g["q4"], r["q4"])
    same_fp4(g["v4"], r["v4"])
    compare_out(g["o"], r["o"], g["lse"], r["lse"], r["amb"])


def test_determinism():
    import torch

    w = workload("long", Hq=4, Hkv=2, S=1536, planted=2)
    d = W.generate(w)
    a = run_gpu(d, w, 1, -1, 500)
    b = run_gpu(d, w, 1, -1, 500)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])
    assert torch.equal(a["q4"].codes, b["q4"].codes)


@pytest.mark.parametrize("fmt", [0, 1])
def test_fp16_skipped_where_nothing_promoted(fmt):
    """Query blocks without promoted pairs never read FP16 Q; FP16 K/V rows
    outside promoted blocks are never read (NaN poison leaves O unchanged)."""
    import torch

    from fp16_attention_amd import api

    w = workload("prefill", Hq=2, Hkv=1, S=768)
    d = W.generate(w)
    g = run_gpu(d, w, fmt, -1, 1000)
    q, k, v, idx, cnt = g["tensors"]
    cnt2 = cnt.clone()
    idx2 = idx.clone()
    cnt2[0, 0, 2] = 0
    idx2[0, 0, 2] = -1
    o1 = api.thrift_attention_fwd(q, k, v, g["q4"], g["k4"], g["v4"], idx2, cnt2, w.bq, w.bk,
                                  w.causal, out_fp32=True)
    qp, kp, vp = q.clone(), k.clone(), v.clone()
    c = cnt2.cpu().numpy()
    ix = idx2.cpu().numpy()
    promoted = set(int(j) for j in ix[c[..., None] > np.arange(ix.shape[-1])].ravel())
    for j in range(-(-w.S // w.bk)):
        if j not in promoted:
            kp[:, :, j * w.bk:(j + 1) * w.bk] = float("nan")
            vp[:, :, j * w.bk:(j + 1) * w.bk] = float("nan")
    for h in range(w.Hq):
        for i in range(c.shape[2]):
            if c[0, h, i] == 0:
                qp[0, h, i * w.bq:(i + 1) * w.bq] = float("nan")
    o2 = api.thrift_attention_fwd(qp, kp, vp, g["q4"], g["k4"], g["v4"], idx2, cnt2, w.bq, w.bk,
                                  w.causal, out_fp32=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_fp16_output_matches_fp32_output():
    import torch

    from fp16_attention_amd import api

    w = workload("prefill", Hq=2, Hkv=2, S=640)
    d = W.generate(w)
    g = run_gpu(d, w, 1, -1, 500)
    q, k, v, idx, cnt = g["tensors"]
    o16 = api.thrift_attention_fwd(q, k, v, g["q4"], g["k4"], g["v4"], idx, cnt, w.bq, w.bk, w.causal)
    torch.cuda.synchronize()
    assert o16.dtype == torch.float16
    np.testing.assert_array_equal(o16.cpu().numpy(), g["o"].astype(np.float32).astype(np.float16))
