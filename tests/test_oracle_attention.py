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
  P13 softmax shift invariance: adding one constant to every score of a row
      changes nothing (every tile's probabilities are taken against its own
      maximum, the two-level reading of the pages);
  P14 a row that sees one key returns that key's value exactly;
  P15 the evaluation-error bound is the stated model, and the lists of
      decisions that may go either way cover every decision a perturbation
      within that bound changes;
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
    # bound: each P value is rounded to fp16 against its tile's maximum, so
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
    # both round every tile's probabilities against the tile's own maximum
    np.testing.assert_allclose(r["o"], O, rtol=1e-9, atol=1e-12 * np.abs(O).max())
    np.testing.assert_allclose(r["lse"], L, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bp", [0, 2500])
def test_p3v_mx_p_with_nvfp4_tensors_equals_two_pass(oracle, bp):
    """The variant: NVFP4 Q, K, V with P quantised MX-style (level 1 the tile
    maximum, E8M0 per 32 keys) equals the dense two-pass form on the
    NVFP4-decoded operands with the MX P quantiser, and differs from the NVFP4
    forward."""
    S, Hq, Hkv, D, causal, bq, bk = 400, 2, 1, 64, True, 128, 64
    q, k, v = _inputs(S, Hq, Hkv, D, 5)
    sm = 1.0 / np.sqrt(D)
    r = oracle.pipeline(q, k, v, oracle.NVFP4, bq, bk, causal, -1, bp, sm, p_fmt=oracle.MX)
    dq = pins.decode_fp4(r["q4"].codes, r["q4"].scales, r["q4"].tensor_scale, 0, 0, q.shape)
    dk = pins.decode_fp4(r["k4"].codes, r["k4"].scales, r["k4"].tensor_scale, 0, 0, k.shape)
    dv = pins.decode_fp4(r["v4"].codes, r["v4"].scales, r["v4"].tensor_scale, 0, 1, v.shape)
    O, L = pins.two_pass_attention(dq, dk, dv, q.astype(np.float64), k.astype(np.float64),
                                   v.astype(np.float64), r["idx"], r["cnt"], 1, bq, bk, causal, sm)
    np.testing.assert_allclose(r["o"], O, rtol=1e-9, atol=1e-12 * np.abs(O).max())
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


def _shift_inputs(fmt, seed, S=320, D=128):
    """Q, K, V and a second K whose every key differs only in channel 96 (the
    first channel of the last FP4 group): there every key holds one same
    value (1.0) in K and 0 in the second K, the rest of that group is zero, so
    a query row's scores against the two differ by one constant per row."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 2, S, D)) * 1.5
    k = rng.standard_normal((1, 1, S, D)) * 1.5
    v = rng.standard_t(3, size=(1, 1, S, D))
    k[..., 96:] = 0.0
    # query values in channel 96 alone in their group, of the form 2^e or
    # 1.5 * 2^e, which an MX group of one element represents exactly
    q[..., 97:] = 0.0
    q[..., 96] = rng.choice([1.0, 1.5, -1.0, -1.5], size=(1, 2, S)) * 2.0 ** rng.integers(-2, 3, (1, 2, S))
    k0 = k.copy()
    k[..., 96] = 1.0
    return q.astype(np.float16), k.astype(np.float16), k0.astype(np.float16), v.astype(np.float16)


@pytest.mark.parametrize("fmt,bp", [(0, 0), (0, 10000), (1, 0), (1, 2000), (1, 10000)])
def test_p13_shift_invariance(oracle, fmt, bp):
    """Adding a constant to every score of a row leaves the output unchanged
    and moves the log-sum-exp by that constant, on both paths.  (With NVFP4 the
    decoded channel-96 products differ between the two paths, so a mixed
    selection would not shift a row uniformly: NVFP4 runs all-FP4 and
    all-FP16.)"""
    S, bq, bk = 320, 64, 64
    q, k, k0, v = _shift_inputs(fmt, 21)
    sm = 1.0 / np.sqrt(q.shape[-1])
    idx, cnt, _ = oracle.select(q, k, bq, bk, True, -1, bp)
    q4, v4 = oracle.quantize(q, 0, fmt), oracle.quantize(v, 1, fmt)
    k4a, k4b = oracle.quantize(k, 0, fmt), oracle.quantize(k0, 0, fmt)
    ka, kb = oracle.dequantize(k4a), oracle.dequantize(k4b)
    assert np.all(ka[..., :96] == kb[..., :96]) and np.all(ka[..., 97:] == 0) and np.all(kb[..., 96:] == 0)
    assert np.ptp(ka[..., 96]) == 0 and ka[0, 0, 0, 96] > 0  # one value for every key
    oa, la = oracle.attention(q, k, v, q4, k4a, v4, idx, cnt, bq, bk, True, sm)
    ob, lb = oracle.attention(q, k0, v, q4, k4b, v4, idx, cnt, bq, bk, True, sm)
    np.testing.assert_allclose(oa, ob, rtol=1e-10, atol=1e-12 * np.abs(ob).max())
    # the shift itself: the query's channel 96 times the key's, decoded on the
    # FP4 path (MX represents both exactly), fp16 on the FP16 path
    qd = oracle.dequantize(q4) if bp < 10000 else q.astype(np.float64)
    kd = ka[0, 0, 0, 96] if bp < 10000 else 1.0
    if fmt == 1:
        np.testing.assert_array_equal(oracle.dequantize(q4)[..., 96], q.astype(np.float64)[..., 96])
    shift = qd[..., 96] * kd * sm
    np.testing.assert_allclose(la - lb, shift, rtol=1e-9, atol=1e-9)
    assert np.abs(shift).max() > 0.1


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("promoted", [False, True])
def test_p14_single_key_row_is_its_value(oracle, fmt, promoted):
    """Causal row 0 sees key 0 only: its output is key 0's value exactly (the
    FP4-decoded value on the FP4 path, the fp16 one on the FP16 path)."""
    S, D = 200, 64
    q, k, v = _inputs(S, 2, 1, D, 23, scale=3.0)
    r = oracle.pipeline(q, k, v, fmt, 64, 64, True, 1 if promoted else 0, 0, 0.3)
    vref = v.astype(np.float64)[0, 0, 0] if promoted else oracle.dequantize(r["v4"])[0, 0, 0]
    for h in range(2):
        np.testing.assert_array_equal(r["o"][0, h, 0], vref)
    assert len(r["amb"].for_row(0, 0, 0)) == 0  # the tile maximum's decisions are exact


def _model_rel(path, b, bmax, dt, mt):
    """The evaluation-error model restated (u = 2^-24): kappa u times the
    chain sums of the key's and the maximum's scores (kappa 2.5 for the MX
    block-scaled FP4 instruction, 6 for the fp16 one); the multiplier's
    roundings (3; 5 with NVFP4 tensors) and the fused multiply-add on t - mt, one on mt;
    exp2 within one ulp; NVFP4 four more roundings; times 1 + 2^-10."""
    u = 2.0 ** -24
    kappa = 2.5 if path == 0 else 6.0
    nc = 5 if path in (1, 4) else 3
    arg = kappa * u * (b + bmax) + (nc + 1) * u * abs(dt) + u * abs(mt)
    return (np.log(2.0) * arg + 2.0 ** -23 + (4 * u if path == 1 else 0.0)) * (1 + 2.0 ** -10)


def test_p15_eval_bound_is_the_model(oracle):
    rng = np.random.default_rng(31)
    for _ in range(400):
        path = int(rng.integers(0, 5))
        b, bmax = rng.uniform(0, 4000, 2)
        dt, mt = -rng.uniform(0, 200), rng.uniform(-500, 900)
        got, want = oracle.eval_rel(path, b, bmax, dt, mt), _model_rel(path, b, bmax, dt, mt)
        assert abs(got / want - 1) < 1e-12, (path, got, want)


def _perturbed_case(oracle, fmt, bp, seed):
    S, Hq, Hkv, D, causal, bq, bk = 448, 2, 1, 128, True, 128, 64
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((1, Hq, S, D)) * 3.0).astype(np.float16)
    k = (rng.standard_normal((1, Hkv, S, D)) * 3.0)
    k[..., :64, :] *= 4.0  # a sink: large scores, wide evaluation error
    k = k.astype(np.float16)
    v = rng.standard_t(3, size=(1, Hkv, S, D)).astype(np.float16)
    sm = 1.0 / np.sqrt(D)
    r = oracle.pipeline(q, k, v, fmt, bq, bk, causal, -1, bp, sm)
    dq = pins.decode_fp4(r["q4"].codes, r["q4"].scales, r["q4"].tensor_scale, fmt, 0, q.shape)
    dk = pins.decode_fp4(r["k4"].codes, r["k4"].scales, r["k4"].tensor_scale, fmt, 0, k.shape)
    dv = pins.decode_fp4(r["v4"].codes, r["v4"].scales, r["v4"].tensor_scale, fmt, 1, v.shape)
    args = (dq, dk, dv, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
            r["idx"], r["cnt"], fmt, bq, bk, causal, sm)
    return r, args


@pytest.mark.parametrize("fmt", [0, 1])
def test_p15_flip_lists_cover_perturbed_decisions(oracle, fmt):
    """Every tile value is moved by up to 0.95 of its evaluation-error bound
    before its rounding decisions (the tile maximum stays exact, as on a
    device that subtracts the maximum's own score).  Each decision that
    flips must be in the oracle's list for its row with the same change of
    the output row, and the output must move by exactly the listed changes of
    the flipped decisions."""
    path = 1 if fmt == 0 else 0
    r, args = _perturbed_case(oracle, fmt, 1200, 41)
    O0, _ = pins.two_pass_attention(*args)
    scale = np.abs(O0).max()
    np.testing.assert_allclose(O0, r["o"], rtol=1e-9, atol=1e-12 * scale)
    nrec = 0
    for seed in range(3):
        prng = np.random.default_rng(100 + seed)

        def eta_fn(t, b, m, kind):
            mt = np.max(np.where(m, -np.inf, t))
            imax = int(np.argmax(np.where(m, -np.inf, t)))
            p = {4: path, 8: 2, 16: 3}[kind]
            rel = np.array([0.0 if m[c] else _model_rel(p, b[c], b[imax], t[c] - mt, mt) for c in range(len(t))])
            eta = 1.0 + 0.95 * rel * prng.uniform(-1, 1, len(t))
            eta[imax] = 1.0
            return eta

        rec = []
        O1, _ = pins.two_pass_attention(*args, eta_fn=eta_fn, record=rec)
        moved = np.zeros_like(O1)
        for b, h, row, ch in rec:
            listed = r["amb"].for_row(b, h, row)
            d = np.abs(listed - ch[None, :]).max(1) if len(listed) else np.array([np.inf])
            assert d.min() <= 1e-10 * scale, (seed, h, row, np.abs(ch).max(), len(listed), d.min())
            moved[b, h, row] += ch
        np.testing.assert_allclose(O1 - r["o"], moved, rtol=0, atol=1e-10 * scale)
        nrec += len(rec)
    assert nrec > 0  # decisions did flip (FP4 codes, FP4 block scales and fp16 roundings, in this case)


def _tile(vs, b=3000.0, mt=37.3):
    """A 64-key tile row: key 0 the maximum (score mt, log2 units), key c
    with value vs[c] relative to it (0: masked), every chain sum b."""
    t = np.full(64, -np.inf)
    mask = np.ones(64, np.int32)
    t[0], mask[0] = mt, 0
    for c, v in vs.items():
        t[c], mask[c] = mt + np.log2(v), 0
    return t, np.full(64, b), mask


# (precision, keys placed at f relative bounds from a boundary): for each
# case the boundary value of v and the two outcomes (values relative to the
# tile maximum) of the decision there
BOUNDARIES = {
    # MX: element codes in the maximum's group (block scale 2^-2): 3.5 * 2^-2
    # between 3 and 4; 1.25 * 2^-2 between 1 and 1.5
    "mx_code_3.5": (0, 5, 0.875, (0.75, 1.0)),
    "mx_code_1.25": (0, 9, 0.3125, (0.25, 0.375)),
    # MX: a second group's maximum at a power of two (its block scale flips)
    "mx_scale": (0, 40, 0.5, None),
    # NVFP4: the maximum's group has block scale 448 (value code * 448 / 2688):
    # 6 v = 3.5 between codes 3 and 4
    "nv_code_3.5": (1, 3, 3.5 / 6.0, (3.0 / 6.0, 4.0 / 6.0)),
    # NVFP4: a second group whose maximum / 6 sits between E4M3 208 and 224
    "nv_scale": (1, 20, 216.0 * 6.0 / 2688.0, None),
    # MXFP8: E4M3 codes of 256 v, 216 between 208 and 224
    "f8_code": (2, 7, 216.0 / 256.0, (208.0 / 256.0, 224.0 / 256.0)),
    # MXFP8: a second group's maximum at a power of two
    "f8_scale": (2, 33, 0.25, None),
    # FP16: a midpoint of fp16 values near 0.75
    "f16": (3, 11, 0.75 + 2.0 ** -12, (0.75, 0.75 + 2.0 ** -11)),
}


@pytest.mark.parametrize("name", sorted(BOUNDARIES))
@pytest.mark.parametrize("f", [0.5, -0.5, 0.9, 2.0, -2.0, 4.0])
def test_p16_decisions_listed_exactly_within_the_bound(oracle, name, f):
    """A value placed f relative error bounds from a rounding boundary is
    listed as a decision iff |f| < 1, with the other outcome as its change;
    values well away from every boundary (and the tile maximum) are not."""
    prec, key, v0, outcomes = BOUNDARIES[name]
    b = 100.0 if prec == 3 else 3000.0
    t, tb, mask = _tile({key: v0}, b)
    rel = oracle.eval_rel(prec, b, b, t[key] - t[0], t[0])
    t, tb, mask = _tile({key: v0 * (1 + f * rel), (key + 1) % 64 or 2: 1e-30}, b)
    pq, dec = oracle.p_tile_decisions(t, tb, mask, prec)
    hit = [d for d in dec if d[0] <= key < d[1]]
    if abs(f) >= 1:
        assert not hit, (name, f, hit)
        assert not dec, (name, f, dec)
        return
    assert len(hit) == 1 and len(dec) == 1, (name, f, dec)
    k0, k1, dp = hit[0]
    if outcomes is not None:  # an element's code: the change is to the other outcome
        assert (k0, k1) == (key, key + 1)
        lo, hi = outcomes
        assert pq[key] == (hi if f > 0 else lo) and pq[key] + dp[key] == (lo if f > 0 else hi)
    else:  # a block scale: the change covers the group, the key moves to its value under the other scale
        assert k1 - k0 == {0: 32, 1: 16, 2: 32}[prec] and np.count_nonzero(dp) >= 1
        assert np.sign(dp[key]) == (1 if f < 0 else -1)  # the other scale rounds the other way
