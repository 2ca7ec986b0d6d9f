"""Pins of the oracle's backward pass (CPU only): Attn-QAT ("Methodik"), the
gradient of the mixed FP4/FP16 forward with the selection held fixed and every
quantiser passed straight through, P recomputed from the forward's
log-sum-exp in the forward's own precision, and the row term taken from the
high-precision output O'.

  B1  every block promoted: the gradients of textbook softmax attention on the
      fp16 inputs, by torch autograd in float64, with the probabilities of the
      PV product rounded to fp16 through a straight-through term (built here
      from numpy, no oracle value involved);
  B2  any selection, both formats: torch autograd of the forward written
      densely (scores from the FP4 operands decoded by the tests' own decoder
      on FP4 pairs, fp16 operands on FP16 pairs, straight-through FP4
      quantisers on Q, K, V, and the forward's quantised probabilities as a
      straight-through constant); the quantised probabilities themselves
      reproduce the oracle's forward output;
  B3  each row's score gradients sum to zero, so with one precision per row
      the key gradients of a key head sum to zero; O' is the exact-softmax
      output, so using O in its place breaks B2;
  B4  the backward on a key-block or query-block work list equals the same
      rows of the full backward.
"""
import numpy as np
import pytest
import torch

from tests import pins

SCALE_DO = 1.0


def _inputs(S, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, S, D)).astype(np.float16)
    k = rng.standard_normal((1, Hkv, S, D)).astype(np.float16)
    v = rng.standard_t(3, size=(1, Hkv, S, D)).astype(np.float16)
    do = (rng.standard_normal((1, Hq, S, D)) * SCALE_DO).astype(np.float16)
    return q, k, v, do


def _forward_backward(oracle, q, k, v, do, fmt, bq, bk, causal, topk_count, topk_bp):
    idx, cnt, _ = oracle.select(q, k, bq, bk, causal, topk_count, topk_bp)
    q4 = oracle.quantize(q, oracle.AXIS_D, fmt)
    k4 = oracle.quantize(k, oracle.AXIS_D, fmt)
    v4 = oracle.quantize(v, oracle.AXIS_S, fmt)
    o, lse, ohp = oracle.attention_hp(q, k, v, q4, k4, v4, idx, cnt, bq, bk, causal)
    dq, dk, dv = oracle.attention_bwd(q, k, v, q4, k4, v4, idx, cnt, bq, bk, causal, lse, ohp, do)
    return dict(idx=idx, cnt=cnt, q4=q4, k4=k4, v4=v4, o=o, lse=lse, ohp=ohp, dq=dq, dk=dk, dv=dv)


def _close(a, b, rtol=1e-9):
    scale = max(1.0, float(np.abs(b).max()))
    np.testing.assert_allclose(a, b, rtol=0, atol=rtol * scale)


def _autograd(q, k, v, do, kind, pt, qd, kd, vd, sm_scale, use_o=None):
    """Dense float64 autograd of the forward: per (head, row, key) the pair's
    path kind (0 masked, 1 FP4, 2 FP16) and pt the probability its PV
    product used.  qd/kd/vd are the decoded FP4 operands (straight-through)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    Q = torch.tensor(q[0].astype(np.float64), requires_grad=True)
    K = torch.tensor(k[0].astype(np.float64), requires_grad=True)
    V = torch.tensor(v[0].astype(np.float64), requires_grad=True)
    Qs = Q + (torch.tensor(qd[0]) - Q).detach()
    Ks = K + (torch.tensor(kd[0]) - K).detach()
    Vs = V + (torch.tensor(vd[0]) - V).detach()
    Ke, Kse = K.repeat_interleave(G, 0), Ks.repeat_interleave(G, 0)
    Ve, Vse = V.repeat_interleave(G, 0), Vs.repeat_interleave(G, 0)
    kind_t = torch.tensor(kind)
    s4 = Qs @ Kse.transpose(1, 2) * sm_scale
    s16 = Q @ Ke.transpose(1, 2) * sm_scale
    s = torch.where(kind_t == 1, s4, s16).masked_fill(kind_t == 0, float("-inf"))
    p = torch.softmax(s, dim=-1)
    pu = p + (torch.tensor(pt) - p).detach()
    o = (pu * (kind_t == 1)) @ Vse + (pu * (kind_t == 2)) @ Ve
    (o * torch.tensor(do[0].astype(np.float64))).sum().backward()
    return Q.grad.numpy()[None], K.grad.numpy()[None], V.grad.numpy()[None], o.detach().numpy()[None]


@pytest.mark.parametrize("causal", [True, False])
def test_b1_all_promoted_vs_textbook_autograd(oracle, causal):
    S, Hq, Hkv, D, bq, bk = 200, 4, 2, 64, 64, 64
    q, k, v, do = _inputs(S, Hq, Hkv, D, 11)
    r = _forward_backward(oracle, q, k, v, do, oracle.MX, bq, bk, causal, 10 ** 6, 0)
    assert (r["cnt"] == [[[pins.valid_blocks(i, S, bq, bk, causal) for i in range(4)]] * Hq]).all()
    sm = 1.0 / np.sqrt(D)
    G = Hq // Hkv
    qf, kf = q.astype(np.float64), k.astype(np.float64)
    s = np.einsum("bhsd,bhtd->bhst", qf, np.repeat(kf, G, 1)) * sm
    if causal:
        s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    kind = np.where(np.isfinite(s[0]), 2, 0).astype(np.int32)
    pt = p[0].astype(np.float16).astype(np.float64)  # the fp16 operand of the PV product
    gq, gk, gv, _ = _autograd(q, k, v, do, kind, pt, qf, kf, v.astype(np.float64), sm)
    _close(r["dq"], gq)
    _close(r["dk"], gk)
    _close(r["dv"], gv)


@pytest.mark.parametrize("fmt", ["nv", "mx"])
@pytest.mark.parametrize("sel", ["none", "mixed"])
def test_b2_selection_vs_dense_autograd(oracle, fmt, sel):
    S, Hq, Hkv, D, bq, bk, causal = 200, 2, 1, 64, 64, 64, True
    f = oracle.NVFP4 if fmt == "nv" else oracle.MX
    q, k, v, do = _inputs(S, Hq, Hkv, D, 12 if sel == "none" else 13)
    tc, bp = (0, 0) if sel == "none" else (-1, 3000)
    r = _forward_backward(oracle, q, k, v, do, f, bq, bk, causal, tc, bp)
    if sel == "mixed":
        assert 0 < int(r["cnt"].sum()) < sum(pins.valid_blocks(i, S, bq, bk, causal) for i in range(4)) * Hq
    kind = np.zeros((Hq, S, S), np.int32)
    pt = np.zeros((Hq, S, S))
    for hq in range(Hq):
        for row in range(S):
            kd_, _, ptr = oracle.row_probs(q, k, v, r["q4"], r["k4"], r["v4"], r["idx"], r["cnt"], bq, bk,
                                           causal, r["lse"], 0, hq, row)
            kind[hq, row], pt[hq, row] = kd_, ptr
    qd = pins.decode_fp4(r["q4"].codes, r["q4"].scales, r["q4"].tensor_scale, f, 0, q.shape)
    kd = pins.decode_fp4(r["k4"].codes, r["k4"].scales, r["k4"].tensor_scale, f, 0, k.shape)
    vd = pins.decode_fp4(r["v4"].codes, r["v4"].scales, r["v4"].tensor_scale, f, 1, v.shape)
    gq, gk, gv, o = _autograd(q, k, v, do, kind, pt, qd, kd, vd, 1.0 / np.sqrt(D))
    _close(r["dq"], gq)
    _close(r["dk"], gk)
    _close(r["dv"], gv)
    # the recomputed probabilities are the forward's: they reproduce its output
    # (FP4 pairs exactly; FP16 pairs within the fp16 rounding of each probability)
    np.testing.assert_allclose(o, r["o"], rtol=0, atol=2e-3 * np.abs(r["o"]).max())
    if sel == "none":
        _close(o, r["o"], 1e-12)


@pytest.mark.parametrize("fmt", ["nv", "mx"])
@pytest.mark.parametrize("sel", ["none", "all"])
def test_b3_score_gradients_sum_to_zero(oracle, fmt, sel):
    S, Hq, Hkv, D, bq, bk, causal = 330, 4, 1, 64, 128, 64, True
    f = oracle.NVFP4 if fmt == "nv" else oracle.MX
    q, k, v, do = _inputs(S, Hq, Hkv, D, 14)
    tc = 0 if sel == "none" else 10 ** 6
    r = _forward_backward(oracle, q, k, v, do, f, bq, bk, causal, tc, 0)
    # sum over keys of dK = sm_scale * sum_r (sum_c dS_rc) q_r = 0
    tot = r["dk"].sum(axis=2)
    mag = np.abs(r["dk"]).sum(axis=2)
    assert (np.abs(tot) <= 1e-10 * mag + 1e-12).all()
    # O' is the exact-softmax output: rows of P sum to one, so O' lies in the
    # span of the values; with every block promoted it equals fp64 softmax
    # attention on the fp16 inputs
    if sel == "all":
        G = Hq // Hkv
        s = np.einsum("bhsd,bhtd->bhst", q.astype(np.float64), np.repeat(k.astype(np.float64), G, 1))
        s = np.where(np.tril(np.ones((S, S), bool)), s / np.sqrt(D), -np.inf)
        p = np.exp(s - s.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        ref = p @ np.repeat(v.astype(np.float64), G, 1)
        _close(r["ohp"], ref, 1e-12)


def test_b4_work_lists(oracle):
    S, Hq, Hkv, D, bq, bk, causal = 300, 4, 2, 64, 128, 64, True
    q, k, v, do = _inputs(S, Hq, Hkv, D, 15)
    r = _forward_backward(oracle, q, k, v, do, oracle.MX, bq, bk, causal, -1, 2500)
    qw = [(0, 3, 2), (0, 0, 1)]
    kw = [(0, 1, 4), (0, 0, 0)]
    dq, dk, dv = oracle.attention_bwd(q, k, v, r["q4"], r["k4"], r["v4"], r["idx"], r["cnt"], bq, bk,
                                      causal, r["lse"], r["ohp"], do, qwork=qw, kwork=kw)
    for b, hq, i in qw:
        sl = slice(i * bq, min(S, (i + 1) * bq))
        np.testing.assert_array_equal(dq[b, hq, sl], r["dq"][b, hq, sl])
    for b, hk, j in kw:
        sl = slice(j * bk, min(S, (j + 1) * bk))
        np.testing.assert_array_equal(dk[b, hk, sl], r["dk"][b, hk, sl])
        np.testing.assert_array_equal(dv[b, hk, sl], r["dv"][b, hk, sl])
    assert np.isnan(dq[0, 1]).all() and np.isnan(dk[0, 1, :64]).all()
