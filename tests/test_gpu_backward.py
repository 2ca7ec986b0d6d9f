"""GPU parity of the Attn-QAT backward (Attn-QAT summary, "Methodik": P
recomputed from the forward's log-sum-exp in the forward's own precision, row
term from the high-precision output O') and of O' itself, through the C ABI,
against the oracle, in both formats.

Selection, FP4 codes and scales are checked bit for bit on the way.  Each
entry point is compared on the same inputs as the oracle: O' from the
oracle's LSE, the gradients from the oracle's LSE and O'.  O', dQ, dK and dV:
max-abs within 2e-3 times max(1, the largest magnitude of the oracle's
tensor) and rel-L2 within 1e-3.  The bound is relative to the tensor's scale
because gradients are sums over a whole row or column of products with dO:
their size grows with the sequence and the attention's concentration, while
each term carries the fp16 rounding of one MFMA operand (probability or dS,
2^-11 relative) and fp32 accumulation.

dV's allowance is the sum, over the oracle's listed decisions of the
quantised probabilities (E2M1 codes and block scales of P, fp16 rounding on
FP16 pairs, whose exact inputs lie within the device's evaluation error of a
rounding boundary), of each decision's change of that dV element: a bound on
any set of them taken the other way.  The report counts the elements beyond
the bound without it.

The whole chain (the GPU forward's own LSE and O' into the GPU backward) is
checked link by link: the GPU forward's LSE against the oracle's within the
forward's bound (1e-3 + 1e-5 |LSE|), its O' against the oracle's to the
bounds above, and the GPU gradients against the oracle's backward run on
that same LSE and O', to the same bounds.  The gradients against the
all-oracle chain are reported too: the row term D_r = dO . O' enters every
dS = p (dP - D_r), so where dP and D_r nearly cancel, the forward's
admissible fp32 deviations (its scores are summed in fp32 on the matrix
cores: the fp16 instruction's 16-channel slices for NVFP4 and FP16 pairs,
the FP4 instruction's 64-channel ones for MX) grow in the gradients' relative
error; that comparison is printed, not bounded.
"""
import numpy as np
import pytest

from fp16_attention_amd import workloads as W
from tests.gpu_harness import note, same_fp4, workload

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-3
REL_L2 = 1e-3

CASES = {
    # name: (workload, topk_count, topk_bp, format: 1 MXFP4, 0 NVFP4)
    "prefill_mixed_mx": (workload("prefill", Hq=2, Hkv=2, S=700), -1, 1000, 1),
    "prefill_mixed_nvfp4": (workload("prefill", Hq=2, Hkv=2, S=700), -1, 1000, 0),
    "gqa_ragged_b2_mx": (workload("sweep", B=2, Hq=4, Hkv=2, S=333), -1, 2500, 1),
    "gqa_ragged_b2_nvfp4": (workload("sweep", B=2, Hq=4, Hkv=2, S=333), -1, 2500, 0),
    "dit_noncausal_d64_bq64_mx": (workload("dit", Hq=2, Hkv=2, S=300, bq=64), -1, 500, 1),
    "dit_noncausal_d64_bq64_nvfp4": (workload("dit", Hq=2, Hkv=2, S=300, bq=64), -1, 500, 0),
    "all_fp16": (workload("prefill", Hq=2, Hkv=1, S=256), -1, 10000, 1),
    "all_fp16_nvfp4": (workload("prefill", Hq=2, Hkv=1, S=256), -1, 10000, 0),
    "no_fp16_mx": (workload("prefill", Hq=2, Hkv=1, S=256), -1, 0, 1),
    "no_fp16_nvfp4": (workload("prefill", Hq=2, Hkv=1, S=256), -1, 0, 0),
    "short_tail_mx": (workload("prefill", Hq=1, Hkv=1, S=37), -1, 500, 1),
    "short_tail_nvfp4": (workload("prefill", Hq=1, Hkv=1, S=37), -1, 500, 0),
    "long_sink_planted_gqa4_mx": (workload("long", Hq=4, Hkv=1, S=1024, planted=2), -1, 500, 1),
    "long_sink_planted_gqa4_nvfp4": (workload("long", Hq=4, Hkv=1, S=1024, planted=2), -1, 500, 0),
    "causal_d64_bq128_mx": (workload("prefill", Hq=2, Hkv=1, S=450, D=64), -1, 1500, 1),
    "causal_d64_bq128_nvfp4": (workload("prefill", Hq=2, Hkv=1, S=450, D=64), -1, 1500, 0),
}


def compare(name, g, r, u=None):
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    err = np.abs(g - r)
    scale = max(1.0, float(np.abs(r).max()))
    rel = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    bound = MAX_ABS * scale
    over = int((err > bound).sum())
    excess = err - (0.0 if u is None else u)
    note(f"    {name}: max-abs {err.max():.3e} (bound {bound:.3e}; elements beyond it {over} of {err.size}"
         f"{'' if u is None else f', beyond it after the decisions allowance {int((excess > bound).sum())}'})"
         f"  rel-L2 {rel:.3e}")
    assert excess.max() <= bound, f"{name}: max-abs {excess.max():.3e} > {bound:.3e}"
    assert rel <= REL_L2, f"{name}: rel-L2 {rel:.3e}"


def check_chain(oracle, d, w, do, q4, k4, v4, idx, cnt, lse, ohp, e, ref):
    """The chain e (the GPU forward's LSE and O' into the GPU backward):
    LSE and O' against the oracle's; the gradients against the oracle's
    backward on the GPU's LSE and O'; the all-oracle chain ref reported."""
    lerr = np.abs(e["lse"] - lse)
    note(f"    LSE: max-abs {lerr.max():.3e}")
    assert np.all(lerr <= 1e-3 + 1e-5 * np.abs(lse)), f"LSE max-abs {lerr.max():.3e}"
    compare("O'", e["ohp"], ohp)
    dq2, dk2, dv2, udv2 = oracle.attention_bwd(d["q"], d["k"], d["v"], q4, k4, v4, idx, cnt, w.bq, w.bk,
                                               w.causal, e["lse"], e["ohp"], do, with_u=True)
    compare("dQ", e["dq"], dq2)
    compare("dK", e["dk"], dk2)
    compare("dV", e["dv"], dv2, udv2)
    for nm, gv, rv in zip(("dQ", "dK", "dV"), (e["dq"], e["dk"], e["dv"]), ref):
        rel = np.linalg.norm(gv - rv) / max(np.linalg.norm(rv), 1e-30)
        note(f"    {nm} against the all-oracle chain: max-abs {np.abs(gv - rv).max():.3e}  rel-L2 {rel:.3e}")


def gpu_backward(d, w, do, tc, bp, fmt=1, lse_in=None, ohp_in=None):
    """The chain on the GPU; lse_in / ohp_in (host arrays) replace the GPU
    forward's LSE for O' and the backward, and O' for the backward."""
    import torch

    from fp16_attention_amd import api

    dev = torch.device("cuda:0")
    q, k, v, dot = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (d["q"], d["k"], d["v"], do))
    idx, cnt = api.thrift_select_blocks(q, k, w.bq, w.bk, w.causal, tc, bp)
    q4 = api.thrift_quantize_fp4(q, api.THRIFT_GROUP_D, fmt)
    k4 = api.thrift_quantize_fp4(k, api.THRIFT_GROUP_D, fmt)
    v4 = api.thrift_quantize_fp4(v, api.THRIFT_GROUP_S, fmt)
    _, lse = api.thrift_attention_fwd(q, k, v, q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal, out_fp32=True,
                                      with_lse=True)
    if lse_in is not None:
        lse = torch.from_numpy(np.ascontiguousarray(lse_in, np.float32)).to(dev)
    ws = api.thrift_attention_bwd_workspace(w.B, w.Hq, w.Hkv, w.S, w.D, w.bq, dev)
    ohp = api.thrift_attention_fwd_hp(q, k, v, q4, k4, v4, idx, cnt, lse, w.bq, w.bk, w.causal, workspace=ws)
    ohp_b = ohp if ohp_in is None else torch.from_numpy(np.ascontiguousarray(ohp_in, np.float32)).to(dev)
    dq, dk, dv = api.thrift_attention_bwd(q, k, v, q4, k4, v4, idx, cnt, lse, ohp_b, dot, w.bq, w.bk, w.causal,
                                          workspace=ws)
    torch.cuda.synchronize()
    cpu = lambda t: t.cpu().numpy()  # noqa: E731
    return dict(idx=cpu(idx), cnt=cpu(cnt), q4=q4, k4=k4, v4=v4, lse=cpu(lse), ohp=cpu(ohp).astype(np.float64),
                dq=cpu(dq).astype(np.float64), dk=cpu(dk).astype(np.float64), dv=cpu(dv).astype(np.float64))


def output_grad(w, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((w.B, w.Hq, w.S, w.D)).astype(np.float16)


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(oracle, name):
    w, tc, bp, fmt = CASES[name]
    note(f"[backward] {name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S} D{w.D} causal{int(w.causal)} bq{w.bq} "
         f"topk({tc},{bp}) fmt{fmt}")
    d = W.generate(w)
    do = output_grad(w, 7 + len(name))
    idx, cnt, _ = oracle.select(d["q"], d["k"], w.bq, w.bk, w.causal, tc, bp)
    q4 = oracle.quantize(d["q"], oracle.AXIS_D, fmt)
    k4 = oracle.quantize(d["k"], oracle.AXIS_D, fmt)
    v4 = oracle.quantize(d["v"], oracle.AXIS_S, fmt)
    _, lse, ohp = oracle.attention_hp(d["q"], d["k"], d["v"], q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal)
    dq, dk, dv, udv = oracle.attention_bwd(d["q"], d["k"], d["v"], q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal,
                                           lse, ohp, do, with_u=True)
    # each entry point on the oracle's inputs
    g = gpu_backward(d, w, do, tc, bp, fmt, lse_in=lse, ohp_in=ohp)
    assert np.array_equal(g["cnt"], cnt), "cnt differs"
    assert np.array_equal(g["idx"][..., :idx.shape[-1]], idx), "idx differs"
    same_fp4(g["q4"], q4)
    same_fp4(g["k4"], k4)
    same_fp4(g["v4"], v4)
    compare("O'", g["ohp"], ohp)
    compare("dQ", g["dq"], dq)
    compare("dK", g["dk"], dk)
    compare("dV", g["dv"], dv, udv)
    # the whole chain: the GPU forward's own LSE and O', link by link
    e = gpu_backward(d, w, do, tc, bp, fmt)
    note("    chain:")
    check_chain(oracle, d, w, do, q4, k4, v4, idx, cnt, lse, ohp, e, (dq, dk, dv))


@pytest.mark.parametrize("fmt", [1, 0])
def test_backward_fullsize_prefill(oracle, fmt):
    """The prefill workload at full size (B1 H32 S8192 D128 causal, 5%), in the
    benchmark's launch configuration; the oracle computes head 0: dQ of three
    query blocks, dK and dV of three key blocks."""
    w = W.WORKLOADS["prefill"].with_(fmt=fmt)
    note(f"[backward] prefill full size: B{w.B} Hq{w.Hq} S{w.S} D{w.D} fmt{fmt}")
    d = W.generate(w)
    do = output_grad(w, 99)
    g = gpu_backward(d, w, do, w.topk_count, w.topk_bp, fmt)
    idx, cnt, _ = oracle.select(d["q"], d["k"], w.bq, w.bk, w.causal, w.topk_count, w.topk_bp)
    km = idx.shape[-1]
    assert np.array_equal(g["cnt"], cnt) and np.array_equal(g["idx"][..., :km], idx)
    q4 = oracle.quantize(d["q"], oracle.AXIS_D, fmt)
    k4 = oracle.quantize(d["k"], oracle.AXIS_D, fmt)
    v4 = oracle.quantize(d["v"], oracle.AXIS_S, fmt)
    same_fp4(g["q4"], q4)
    nq, nk = -(-w.S // w.bq), -(-w.S // w.bk)
    head0 = [(0, 0, i) for i in range(nq)]
    _, lse, ohp = oracle.attention_hp(d["q"], d["k"], d["v"], q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal,
                                      work=head0)
    qb, kb = [0, nq // 2, nq - 1], [0, nk // 3, nk - 1]
    dq, dk, dv, udv = oracle.attention_bwd(d["q"], d["k"], d["v"], q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal,
                                           lse, ohp, do, qwork=[(0, 0, i) for i in qb],
                                           kwork=[(0, 0, j) for j in kb], with_u=True)
    # the chain, link by link: the GPU forward's LSE and O' of head 0 against
    # the oracle's, then the gradients against the oracle's backward on them
    lerr = np.abs(g["lse"][0, 0] - lse[0, 0])
    note(f"    LSE (head 0): max-abs {lerr.max():.3e}")
    assert np.all(lerr <= 1e-3 + 1e-5 * np.abs(lse[0, 0])), f"LSE max-abs {lerr.max():.3e}"
    compare("O' (head 0)", g["ohp"][0, 0], ohp[0, 0])
    dq2, dk2, dv2, udv2 = oracle.attention_bwd(d["q"], d["k"], d["v"], q4, k4, v4, idx, cnt, w.bq, w.bk,
                                               w.causal, g["lse"], g["ohp"], do, qwork=[(0, 0, i) for i in qb],
                                               kwork=[(0, 0, j) for j in kb], with_u=True)
    rq = np.concatenate([np.arange(i * w.bq, min(w.S, (i + 1) * w.bq)) for i in qb])
    rk = np.concatenate([np.arange(j * w.bk, min(w.S, (j + 1) * w.bk)) for j in kb])
    compare("dQ (3 query blocks)", g["dq"][0, 0, rq], dq2[0, 0, rq])
    compare("dK (3 key blocks)", g["dk"][0, 0, rk], dk2[0, 0, rk])
    compare("dV (3 key blocks)", g["dv"][0, 0, rk], dv2[0, 0, rk], udv2[0, 0, rk])
    for nm, gv, rv in (("dQ", g["dq"][0, 0, rq], dq[0, 0, rq]), ("dK", g["dk"][0, 0, rk], dk[0, 0, rk]),
                       ("dV", g["dv"][0, 0, rk], dv[0, 0, rk])):
        rel = np.linalg.norm(gv - rv) / max(np.linalg.norm(rv), 1e-30)
        note(f"    {nm} against the all-oracle chain: max-abs {np.abs(gv - rv).max():.3e}  rel-L2 {rel:.3e}")


def test_backward_fullsize_long(oracle):
    """The long workload at full size (B1 Hq32 Hkv8 S32768 D128 causal, sink,
    planted pairs, 5%, MXFP4): the whole chain on the GPU, then O' and the
    gradients again with head 0's LSE and O' taken from the oracle; the oracle
    computes query head 0's O' (every row) and the dQ of three of its query
    blocks."""
    w = W.WORKLOADS["long"].with_(fmt=1)
    note(f"[backward] long full size: B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S} D{w.D}")
    d = W.generate(w)
    do = output_grad(w, 98)
    g = gpu_backward(d, w, do, w.topk_count, w.topk_bp, 1)
    idx, cnt, _ = oracle.select(d["q"], d["k"], w.bq, w.bk, w.causal, w.topk_count, w.topk_bp)
    assert np.array_equal(g["cnt"], cnt) and np.array_equal(g["idx"][..., :idx.shape[-1]], idx)
    q4 = oracle.quantize(d["q"], oracle.AXIS_D, 1)
    k4 = oracle.quantize(d["k"], oracle.AXIS_D, 1)
    v4 = oracle.quantize(d["v"], oracle.AXIS_S, 1)
    nq = -(-w.S // w.bq)
    _, lse, ohp = oracle.attention_hp(d["q"], d["k"], d["v"], q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal,
                                      work=[(0, 0, i) for i in range(nq)])
    qb = [1, nq // 2, nq - 1]
    nk = -(-w.S // w.bk)  # (one cheap key block: the work list may not be empty; its dK/dV is not compared)
    dq, _, _ = oracle.attention_bwd(d["q"], d["k"], d["v"], q4, k4, v4, idx, cnt, w.bq, w.bk, w.causal, lse, ohp,
                                    do, qwork=[(0, 0, i) for i in qb], kwork=[(0, 0, nk - 1)])
    rq = np.concatenate([np.arange(i * w.bq, min(w.S, (i + 1) * w.bq)) for i in qb])
    note("    chain:")
    compare("O' (head 0)", g["ohp"][0, 0], ohp[0, 0])
    compare("dQ (3 query blocks)", g["dq"][0, 0, rq], dq[0, 0, rq])
    # each entry point on the oracle's inputs for head 0 (a row's O' and dQ
    # depend only on its own LSE and O'); the other heads keep the GPU's
    lse_in, ohp_in = g["lse"].copy(), g["ohp"].copy()
    lse_in[0, 0], ohp_in[0, 0] = lse[0, 0], ohp[0, 0]
    u = gpu_backward(d, w, do, w.topk_count, w.topk_bp, 1, lse_in=lse_in, ohp_in=ohp_in)
    note("    on the oracle's LSE and O':")
    compare("O' (head 0)", u["ohp"][0, 0], ohp[0, 0])
    compare("dQ (3 query blocks)", u["dq"][0, 0, rq], dq[0, 0, rq])


def test_backward_deterministic():
    """Two runs give bit-identical gradients (no atomics)."""
    w = workload("sweep", B=1, Hq=4, Hkv=2, S=700)
    d = W.generate(w)
    do = output_grad(w, 5)
    a = gpu_backward(d, w, do, -1, 2500)
    b = gpu_backward(d, w, do, -1, 2500)
    for key in ("ohp", "dq", "dk", "dv"):
        assert np.array_equal(a[key], b[key]), key
