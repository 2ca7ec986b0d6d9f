"""GPU parity of the middle precision tier (a variant: MXFP8 blocks between
the FP4 and FP16 paths, MX format) through the C ABI, against the oracle.

  - thrift_quantize_fp8 bit for bit (codes and E8M0 scales, both axes, ragged
    sequences, ties at E4M3 midpoints, saturation, E4M3 subnormals, zeros and
    -0);
  - thrift_attention_fwd_tiered: both selections bit for bit, the output
    within the bounds of the other parity tests (max-abs 2e-3 beyond the
    oracle's decision uncertainty, rel-L2 1e-3, LSE), with mixed tiers, every
    block FP8, GQA, block_q 64 and 128, D 64 and 128, causal or not;
  - with no FP8 block the three-tier kernel gives the two-tier kernel's output
    bit for bit;
  - the long workload at full size with the FP16 tier at 5% and the FP8 tier
    at a further 10%, on sampled query blocks.
"""
import numpy as np
import pytest

from fp16_attention_amd import workloads as W
from tests.gpu_harness import compare_out, note, same_fp4, workload
from tests.test_oracle_fp8 import _special_tensor

pytestmark = pytest.mark.gpu


def _dev(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


@pytest.mark.parametrize("S,D", [(64, 64), (100, 128), (37, 64), (1000, 128)])
@pytest.mark.parametrize("axis", [0, 1])
def test_quantize_fp8_bit_exact(oracle, S, D, axis):
    from fp16_attention_amd import api

    note(f"[fp8 quantise] S{S} D{D} axis{axis}")
    x = _special_tensor(S, D, 20 + S + axis)
    g = api.thrift_quantize_fp8(_dev(x), axis)
    r = oracle.quantize_fp8(x, axis)
    gc, gs = g.codes.cpu().numpy(), g.scales.cpu().numpy()
    bad = np.argwhere(gc != r.codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:3].tolist()}: {gc[tuple(bad[0])]:#x} vs {r.codes[tuple(bad[0])]:#x}"
    np.testing.assert_array_equal(gs, r.scales)


def _run_tiered(d, w, bp16, bp8, no_fp16=False):
    import torch

    from fp16_attention_amd import api

    q, k, v = (_dev(d[n]) for n in ("q", "k", "v"))
    q4, qbar = api.thrift_quantize_fp4_means(q, api.THRIFT_MXFP4, w.bq)
    k4, kbar = api.thrift_quantize_fp4_means(k, api.THRIFT_MXFP4, w.bk)
    v4 = api.thrift_quantize_fp4(v, api.THRIFT_GROUP_S, api.THRIFT_MXFP4)
    q8, k8 = api.thrift_quantize_fp8(q, api.THRIFT_GROUP_D), api.thrift_quantize_fp8(k, api.THRIFT_GROUP_D)
    v8 = api.thrift_quantize_fp8(v, api.THRIFT_GROUP_S)
    idx, cnt = api.thrift_select_blocks_means(qbar, kbar, w.S, w.S, w.bq, w.bk, w.causal, -1, bp16)
    idx2, cnt2 = api.thrift_select_blocks_means(qbar, kbar, w.S, w.S, w.bq, w.bk, w.causal, -1, bp16 + bp8)
    fp16 = (None, None, None) if no_fp16 else (q, k, v)  # fp16 tensors may be absent when no block is FP16
    o, lse = api.thrift_attention_fwd_tiered(*fp16, q4, k4, v4, q8, k8, v8, idx, cnt, idx2, cnt2, w.bq, w.bk,
                                             w.causal, out_fp32=True, with_lse=True)
    torch.cuda.synchronize()
    cpu = lambda t: t.cpu().numpy()  # noqa: E731
    return dict(idx=cpu(idx), cnt=cpu(cnt), idx2=cpu(idx2), cnt2=cpu(cnt2), q4=q4, k4=k4, v4=v4, q8=q8, k8=k8,
                v8=v8, o=cpu(o).astype(np.float64), lse=cpu(lse).astype(np.float64),
                tensors=(q, k, v, q4, k4, v4, idx, cnt))


def _same_sel(g, idx, cnt, gi, gc):
    assert np.array_equal(gc, cnt), "cnt differs"
    km = idx.shape[-1]
    assert np.array_equal(gi[..., :km], idx), "idx differs"
    assert np.all(gi[..., km:] == -1)


def _same_fp8(g, r):
    assert np.array_equal(g.codes.cpu().numpy(), r.codes), "FP8 codes differ"
    assert np.array_equal(g.scales.cpu().numpy(), r.scales), "FP8 scales differ"


CASES = {
    # name: (workload, bp16, bp8)
    "prefill_mixed": (workload("prefill", Hq=2, Hkv=2, S=700), 1000, 2000),
    "gqa_ragged": (workload("sweep", B=2, Hq=4, Hkv=2, S=333), 500, 3000),
    "all_fp8": (workload("prefill", Hq=2, Hkv=1, S=300), 0, 10000),
    "bq64_d64_noncausal": (workload("dit", Hq=2, Hkv=2, S=257, bq=64), 500, 2500),
    "sink_planted": (workload("long", Hq=4, Hkv=2, S=1024, planted=4), 500, 1000),
    "one_ragged_block": (workload("prefill", Hq=2, Hkv=1, S=37), 0, 10000),
}


@pytest.mark.parametrize("name", list(CASES))
def test_tiered_parity(oracle, name):
    w, bp16, bp8 = CASES[name]
    note(f"[tiered] {name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S} D{w.D} causal{int(w.causal)} bq{w.bq} "
         f"bp16 {bp16} bp8 {bp8}")
    d = W.generate(w)
    g = _run_tiered(d, w, bp16, bp8, no_fp16=bp16 == 0)
    r = oracle.pipeline_tiers(d["q"], d["k"], d["v"], w.bq, w.bk, w.causal, bp16, bp8)
    _same_sel(g, r["idx"], r["cnt"], g["idx"], g["cnt"])
    _same_sel(g, r["idx2"], r["cnt2"], g["idx2"], g["cnt2"])
    n8 = int(r["cnt2"].sum() - r["cnt"].sum())
    note(f"    FP16 blocks {int(r['cnt'].sum())}, FP8 blocks {n8}")
    assert n8 > 0
    for gn, rn in (("q4", "q4"), ("k4", "k4"), ("v4", "v4")):
        same_fp4(g[gn], r[rn])
    for n in ("q8", "k8", "v8"):
        _same_fp8(g[n], r[n])
    compare_out(g["o"], r["o"], g["lse"], r["lse"], r["amb"])


def test_tiered_without_fp8_blocks_is_two_tier():
    from fp16_attention_amd import api

    w = workload("prefill", Hq=2, Hkv=1, S=700)
    d = W.generate(w)
    g = _run_tiered(d, w, 1000, 0)
    q, k, v, q4, k4, v4, idx, cnt = g["tensors"]
    o2 = api.thrift_attention_fwd(q, k, v, q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal, out_fp32=True)
    np.testing.assert_array_equal(g["o"], o2.cpu().numpy().astype(np.float64))


@pytest.mark.slow
def test_tiered_long_fullsize(oracle):
    w = W.WORKLOADS["long"]
    bp16, bp8 = w.topk_bp, 2 * w.topk_bp
    note(f"[tiered] long full size: B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S} D{w.D} bp16 {bp16} bp8 {bp8}")
    d = W.generate(w)
    g = _run_tiered(d, w, bp16, bp8)
    idx, cnt, _ = oracle.select(d["q"], d["k"], w.bq, w.bk, w.causal, -1, bp16)
    idx2, cnt2, _ = oracle.select(d["q"], d["k"], w.bq, w.bk, w.causal, -1, bp16 + bp8)
    _same_sel(g, idx, cnt, g["idx"], g["cnt"])
    _same_sel(g, idx2, cnt2, g["idx2"], g["cnt2"])
    q4, k4, v4 = (oracle.quantize(d[n], a, oracle.MX) for n, a in (("q", 0), ("k", 0), ("v", 1)))
    q8, k8, v8 = (oracle.quantize_fp8(d[n], a) for n, a in (("q", 0), ("k", 0), ("v", 1)))
    for n, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _same_fp8(g[n], t)
    nq = idx.shape[2]
    pb, ph, pi = d["planted"][0][:3]
    work = sorted({(0, 0, 0), (0, w.Hq - 1, nq - 1), (0, 5, nq // 2), (0, 6, nq // 2), (pb, ph, pi)})
    note(f"    sampled query blocks (b, hq, i): {work}")
    o, lse, amb = oracle.attention_tiers(d["q"], d["k"], d["v"], q4, k4, v4, q8, k8, v8, idx, cnt, idx2, cnt2,
                                       w.bq, w.bk, w.causal, work=work, with_amb=True)
    rows = [(b, h, slice(i * w.bq, min(w.S, (i + 1) * w.bq))) for b, h, i in work]
    compare_out(g["o"], o, g["lse"], lse, amb, rows=rows)
