"""Pins of the oracle's attention forward (CPU only).

  P1  every block promoted: the result is textbook softmax attention on the
      fp16 inputs, within the rounding of P to fp16 (bound written below);
  P2  no block promoted: the result is uniform FP4 attention, restated as a
      dense two-pass computation with brute-force rounding;
  P3  any mixed selection: the online merge (FlashAttention-2 style) equals a
      two-pass softmax over the same per-block choices;
  P6  FP4 products are exact on inputs that FP4 represents exactly;
  P7  one block, top-1: textbook attention;
  P11 FP16 data outside the promoted blocks is never read (NaN poison);
  and the log-sum-exp output against a direct computation.
(ThriftAttention pages, "Gemengd-Precisie Berekening & Samenvoeging".)
"""
import numpy as np
import pytest

from fp16_attention_amd import workloads as W
from tests import pins

CASES = [
    # S, Hq, Hkv, D, causal, bq, bk
    (300, 2, 1, 64, True, 128, 64),
    (257, 1, 1, 64, False, 64, 64),
    (200, 2, 2, 128, True, 64, 64),
    (160, 4, 2, 64, True, 64, 64),  # grouped-query attention, G = 2
]


def _inputs(S, Hq, Hkv, D, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, S, D)) * scale
    k = rng.standard_normal((1, Hkv, S, D)) * scale
    v = rng.standard_t(3, size=(1, Hkv, S, D))
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)


@pytest.mark.parametrize("case", CASES)
def test_p1_all_promoted_is_exact_attention(oracle, case):
    S, Hq, Hkv, D, causal, bq, bk = case
    q, k, v = _inputs(S, Hq, Hkv, D, 1, scale=1.5)
    sm = 1.0 / np.sqrt(D)
    r = oracle.pipeline(q, k, v, oracle.MX, bq, bk, causal, -1, 10000, sm)
    qd, kd, vd = (t.astype(np.float64) for t in (q, k, v))
    O, L = pins.exact_attention(qd, kd, vd, causal, sm)
    # bound: each P value is rounded to fp16 on a power-of-two footing, so
    # |P~ - P| <= 2^-11 P + 2^-24 (relative to the row maximum)
    G = Hq // Hkv
    for hq in range(Hq):
        s = (qd[0, hq] @ kd[0, hq // G].T) * sm
        if causal:
            s = np.where(np.triu(np.ones((S, S), bool), 1), -np.inf, s)
        p = np.exp(s - s.max(1, keepdims=True))
        lrow = p.sum(1, keepdims=True)
        bound = (2.0 ** -11 * (p @ np.abs(vd[0, hq // G])) + 2.0 ** -23 * np.abs(vd[0, hq // G]).sum(0)) / lrow
        err = np.abs(r["o"][0, hq] - O[0, hq])
        assert np.all(err <= bound * 1.001 + 1e-12), err.max()
    rel = np.linalg.norm(r["o"] - O) / np.linalg.norm(O)
    assert rel < 1e-3
    np.testing.assert_allclose(r["lse"], L, rtol=0, atol=1e-12 * (1 + np.abs(L).max()))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("case", CASES)
def test_p2_none_promoted_is_uniform_fp4(oracle, case, fmt):
    S, Hq, Hkv, D, causal, bq, bk = case
    q, k, v = _inputs(S, Hq, Hkv, D, 2)
    sm = 1.0 / np.sqrt(D)
    r = oracle.pipeline(q, k, v, fmt, bq, bk, causal, 0, 0, sm)
    assert np.all(r["cnt"] == 0)
    dq = pins.decode_fp4(r["q4"].codes, r["q4"].scales, r["q4"].tensor_scale, fmt, 0, q.shape)
    dk = pins.decode_fp4(r["k4"].codes, r["k4"].scales, r["k4"].tensor_scale, fmt, 0, k.shape)
    dv = pins.decode_fp4(r["v4"].codes, r["v4"].scales, r["v4"].tensor_scale, fmt, 1, v.shape)
    O, L = pins.two_pass_attention(dq, dk, dv, None, None, None, r["idx"], r["cnt"], fmt, bq, bk,
                                   causal, sm)
    np.testing.assert_allclose(r["o"], O, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r["lse"], L, rtol=1e-12, atol=1e-12)
    # the row sum is the unquantised one: LSE is the log-sum-exp of the FP4 scores
    G = Hq // Hkv
    for hq in range(Hq):
        s = (dq[0, hq] @ dk[0, hq // G].T) * sm
        if causal:
            s = np.where(np.triu(np.ones((S, S), bool), 1), -np.inf, s)
        m = s.max(1)
        np.testing.assert_allclose(r["lse"][0, hq], m + np.log(np.exp(s - m[:, None]).sum(1)),
                                   rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("bp", [1500, 5000])
def test_p3_mixed_equals_two_pass(oracle, fmt, bp):
    S, Hq, Hkv, D, causal, bq, bk = 400, 2, 1, 64, True, 128, 64
    q, k, v = _inputs(S, Hq, Hkv, D, 3)
    sm = 1.0 / np.sqrt(D)
    r = oracle.pipeline(q, k, v, fmt, bq, bk, causal, -1, bp, sm)
    assert r["cnt"].sum() > 0 and (r["cnt"] < [[[pins.valid_blocks(i, S, bq, bk, causal)
                                                 for i in range(4)]]]).any()
    dq = pins.decode_fp4(r["q4"].codes, r["q4"].scales, r["q4"].tensor_scale, fmt, 0, q.shape)
    dk = pins.decode_fp4(r["k4"].codes, r["k4"].scales, r["k4"].tensor_scale, fmt, 0, k.shape)
    dv = pins.decode_fp4(r["v4"].codes, r["v4"].scales, r["v4"].tensor_scale, fmt, 1, v.shape)
    O, L = pins.two_pass_attention(dq, dk, dv, q.astype(np.float64), k.astype(np.float64),
                                   v.astype(np.float64), r["idx"], r["cnt"], fmt, bq, bk, causal, sm)
    # fp16 rounding of P happens on a power-of-two footing in both, so the
    # two agree to fp64 rounding except for subnormal-range probabilities
    # (below 2^-24 of the row maximum)
    np.testing.assert_allclose(r["o"], O, rtol=1e-9, atol=1e-7 * np.abs(O).max())
    np.testing.assert_allclose(r["lse"], L, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bp", [0, 2500])
def test_p3v_mx_p_with_nvfp4_tensors_equals_two_pass(oracle, bp):
    """The variant: NVFP4 Q, K, V with P quantised MX-style (E8M0 per 32 keys,
    integer level 1) equals the dense two-pass form on the NVFP4-decoded
    operands with the MX P quantiser, and differs from the NVFP4 forward."""
    S, Hq, Hkv, D, causal, bq, bk = 400, 2, 1, 64, True, 128, 64
    q, k, v = _inputs(S, Hq, Hkv, D, 5)
    sm = 1.0 / np.sqrt(D)
    r = oracle.pipeline(q, k, v, oracle.NVFP4, bq, bk, causal, -1, bp, sm, p_fmt=oracle.MX)
    dq = pins.decode_fp4(r["q4"].codes, r["q4"].scales, r["q4"].tensor_scale, 0, 0, q.shape)
    dk = pins.decode_fp4(r["k4"].codes, r["k4"].scales, r["k4"].tensor_scale, 0, 0, k.shape)
    dv = pins.decode_fp4(r["v4"].codes, r["v4"].scales, r["v4"].tensor_scale, 0, 1, v.shape)
    O, L = pins.two_pass_attention(dq, dk, dv, q.astype(np.float64), k.astype(np.float64),
                                   v.astype(np.float64), r["idx"], r["cnt"], 1, bq, bk, causal, sm)
    np.testing.assert_allclose(r["o"], O, rtol=1e-9, atol=1e-7 * np.abs(O).max())
    np.testing.assert_allclose(r["lse"], L, rtol=1e-12, atol=1e-12)
    nv = oracle.pipeline(q, k, v, oracle.NVFP4, bq, bk, causal, -1, bp, sm)
    assert np.abs(nv["o"] - r["o"]).max() > 1e-4  # the P quantiser is not NVFP4's
    np.testing.assert_array_equal(nv["lse"], r["lse"])  # the row sum is the unquantised one


def test_p6_fp4_products_exact(oracle):
    rng = np.random.default_rng(4)
    S, D = 64, 128
    codes = rng.integers(0, 16, size=(2, S, D))
    codes[..., ::32] = 7
    X = rng.integers(-6, 2, size=(2, S, D // 32)).repeat(32, -1)
    x = pins.e2m1_values_from_bits()[codes] * 2.0 ** X
    q16 = x[0][None, None].astype(np.float16)
    k16 = x[1][None, None].astype(np.float16)
    q4 = oracle.quantize(q16, 0, oracle.MX)
    k4 = oracle.quantize(k16, 0, oracle.MX)
    for rrow in (0, 17, 63):
        got = oracle.fp4_scores(q4, k4, rrow, 0, S)
        np.testing.assert_array_equal(got, x[1] @ x[0][rrow])


def test_p7_single_block_top1(oracle):
    q, k, v = _inputs(64, 1, 1, 64, 5, scale=2.0)
    sm = 0.125
    r = oracle.pipeline(q, k, v, oracle.NVFP4, 64, 64, False, 1, 0, sm)
    assert r["cnt"].tolist() == [[[1]]]
    O, L = pins.exact_attention(*(t.astype(np.float64) for t in (q, k, v)), False, sm)
    assert np.linalg.norm(r["o"] - O) / np.linalg.norm(O) < 2e-4
    np.testing.assert_allclose(r["lse"], L, rtol=1e-13)


@pytest.mark.parametrize("fmt", [0, 1])
def test_p11_fp16_read_only_for_promoted(oracle, fmt):
    S, bq, bk = 512, 128, 64
    q, k, v = _inputs(S, 2, 1, 64, 6)
    sm = 0.125
    idx, cnt, _ = oracle.select(q, k, bq, bk, True, -1, 1000)
    cnt[0, 0, 1] = 0  # a query block with no promoted pair
    idx[0, 0, 1] = -1
    q4, k4, v4 = (oracle.quantize(t, a, fmt) for t, a in ((q, 0), (k, 0), (v, 1)))
    o1, l1 = oracle.attention(q, k, v, q4, k4, v4, idx, cnt, bq, bk, True, sm)
    qp, kp, vp = q.copy(), k.copy(), v.copy()
    promoted_k = set(idx[0][cnt[0] > 0].ravel().tolist()) - {-1}
    for j in range(S // bk):
        if j not in promoted_k:
            kp[:, :, j * bk:(j + 1) * bk] = np.nan
            vp[:, :, j * bk:(j + 1) * bk] = np.nan
    for hq in range(2):
        for i in range(S // bq):
            if cnt[0, hq, i] == 0:
                qp[0, hq, i * bq:(i + 1) * bq] = np.nan
    o2, l2 = oracle.attention(qp, kp, vp, q4, k4, v4, idx, cnt, bq, bk, True, sm)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # top-k = 0 needs no FP16 tensor at all
    zero_i, zero_c = np.full_like(idx, -1), np.zeros_like(cnt)
    o3, _ = oracle.attention(None, None, None, q4, k4, v4, zero_i, zero_c, bq, bk, True, sm)
    assert np.all(np.isfinite(o3))


def test_work_list_matches_full(oracle):
    w = W.WORKLOADS["long"].with_(S=1024, Hq=4, Hkv=2, planted=2)
    d = W.generate(w)
    full = oracle.pipeline(d["q"], d["k"], d["v"], w.fmt, w.bq, w.bk, w.causal, -1, w.topk_bp)
    work = [(0, 1, 3), (0, 3, 7), (0, 0, 0)]
    part = oracle.attention(d["q"], d["k"], d["v"], full["q4"], full["k4"], full["v4"], full["idx"],
                            full["cnt"], w.bq, w.bk, w.causal, None, work)
    for b, hq, i in work:
        sl = slice(i * w.bq, (i + 1) * w.bq)
        np.testing.assert_array_equal(part[0][b, hq, sl], full["o"][b, hq, sl])
    assert np.isnan(part[0][0, 2]).all()


@pytest.mark.parametrize("fmt", [0, 1])
def test_uncertainty_bounds_decision_flips(oracle, fmt):
    """u bounds what moving every decision input by up to the stated fp32
    evaluation error can change in O (both outcomes of a decision that close
    to its boundary are valid results); it is small almost everywhere."""
    S, Hq, Hkv, D, causal, bq, bk = 448, 2, 1, 64, True, 128, 64
    rng = np.random.default_rng(12)
    q = (rng.standard_normal((1, Hq, S, D)) * 2.5).astype(np.float16)
    k = (rng.standard_normal((1, Hkv, S, D)) * 2.5).astype(np.float16)
    v = rng.standard_t(3, size=(1, Hkv, S, D)).astype(np.float16)
    sm = 1.0 / np.sqrt(D)
    r = oracle.pipeline(q, k, v, fmt, bq, bk, causal, -1, 3000, sm)
    dq = pins.decode_fp4(r["q4"].codes, r["q4"].scales, r["q4"].tensor_scale, fmt, 0, q.shape)
    dk = pins.decode_fp4(r["k4"].codes, r["k4"].scales, r["k4"].tensor_scale, fmt, 0, k.shape)
    dv = pins.decode_fp4(r["v4"].codes, r["v4"].scales, r["v4"].tensor_scale, fmt, 1, v.shape)
    u = r["u"]
    args = (dq, dk, dv, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
            r["idx"], r["cnt"], fmt, bq, bk, causal, sm)
    O0, _ = pins.two_pass_attention(*args)
    assert np.all(u >= 0) and np.mean(u > 1e-4 * np.abs(O0).max()) < 0.05
    # the error the oracle allows: ln2 * 2^-20 (A + 16) relative on 2^t, i.e.
    # 2^-20 (A + 16) absolute on t, A the score's sum of product magnitudes;
    # move by up to 90% of it
    for seed in range(3):
        prng = np.random.default_rng(seed)
        pert = lambda t, a: t + 0.9 * np.ldexp(a + 16.0, -20) * prng.uniform(-1, 1, t.shape)  # noqa: E731
        O1, _ = pins.two_pass_attention(*args, perturb=pert)
        moved = np.abs(O1 - O0)
        # slack: the two-pass form rounds fp16 P against the final maximum, the
        # oracle against the running one; they differ below 2^-24 of the row
        # maximum (subnormal fp16), as in P3
        assert np.all(moved <= u + 1e-7 * np.abs(O0).max()), (moved - u).max()
        assert moved.max() > 0  # some decision did flip
