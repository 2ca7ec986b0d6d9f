"""Pins of the oracle's decode-shaped forward (CPU only): S_q new queries at
the end of a key sequence of S_k positions (causal masks aligned at the
ends), the shape of new tokens attending to the dual KV cache (ThriftAttention
summaries, "Resultaten": decode speed-ups; "Betekenis en Beweringen": the FP16
and FP4 copies of the cache).

  D1  selection equals brute-force repeated argmax of qbar . kbar over the
      blocks a query block may see;
  D2  every block promoted: textbook softmax attention on the fp16 inputs,
      within the rounding of P to fp16;
  D3  no block promoted, and any mixed selection: the dense two-pass form;
  D4  S_q = one full query block at the end of the sequence gives exactly
      the rows of the full-sequence forward for that block (MX, whose codes
      do not depend on the rest of the tensor).
"""
import numpy as np
import pytest

from tests import pins

CASES = [
    # Sq, Sk, Hq, Hkv, D, causal, bq
    (1, 700, 4, 2, 64, True, 128),
    (5, 513, 2, 1, 128, True, 128),
    (16, 1000, 4, 1, 64, False, 128),
    (64, 300, 2, 2, 64, True, 64),
]


def _inputs(Sq, Sk, Hq, Hkv, D, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((1, Hq, Sq, D)) * scale).astype(np.float16)
    k = (rng.standard_normal((1, Hkv, Sk, D)) * scale).astype(np.float16)
    v = rng.standard_t(3, size=(1, Hkv, Sk, D)).astype(np.float16)
    return q, k, v


def _decoded(oracle, r, fmt, q, k, v):
    dq = pins.decode_fp4(r["q4"].codes, r["q4"].scales, r["q4"].tensor_scale, fmt, 0, q.shape)
    dk = pins.decode_fp4(r["k4"].codes, r["k4"].scales, r["k4"].tensor_scale, fmt, 0, k.shape)
    dv = pins.decode_fp4(r["v4"].codes, r["v4"].scales, r["v4"].tensor_scale, fmt, 1, v.shape)
    return dq, dk, dv


@pytest.mark.parametrize("case", CASES)
def test_d1_select_vs_bruteforce(oracle, case):
    Sq, Sk, Hq, Hkv, D, causal, bq = case
    q, k, _ = _inputs(Sq, Sk, Hq, Hkv, D, 7)
    k[:, :, :64] *= 3  # a strong first block, as a sink would make it
    bk, bp = 64, 2500
    idx, cnt, _ = oracle.select(q, k, bq, bk, causal, -1, bp)
    G = Hq // Hkv
    nq, nk = -(-Sq // bq), -(-Sk // bk)
    qm = np.stack([q[:, :, i * bq:(i + 1) * bq].astype(np.float64).mean(2) for i in range(nq)], 2)
    km = np.stack([k[:, :, j * bk:(j + 1) * bk].astype(np.float64).mean(2) for j in range(nk)], 2)
    checked = 0
    for hq in range(Hq):
        for i in range(nq):
            n = pins.valid_blocks(i, Sq, bq, bk, causal, Sk)
            s = km[0, hq // G, :n] @ qm[0, hq, i]
            kk = min(n, -(-n * bp // 10000))
            order = sorted(range(n), key=lambda j: (-s[j], j))
            want = sorted(order[:kk])
            assert cnt[0, hq, i] == kk
            got = idx[0, hq, i, :kk].tolist()
            assert np.all(idx[0, hq, i, kk:] == -1)
            gap = s[order[kk - 1]] - s[order[kk]] if 0 < kk < n else np.inf
            if gap > 1e-5 * np.abs(s).max():
                assert got == want
                checked += 1
    assert checked >= 1


@pytest.mark.parametrize("case", CASES)
def test_d2_all_promoted_is_exact_attention(oracle, case):
    Sq, Sk, Hq, Hkv, D, causal, bq = case
    q, k, v = _inputs(Sq, Sk, Hq, Hkv, D, 8, scale=1.5)
    sm = 1.0 / np.sqrt(D)
    r = oracle.pipeline(q, k, v, oracle.MX, bq, 64, causal, -1, 10000, sm)
    qd, kd, vd = (t.astype(np.float64) for t in (q, k, v))
    O, L = pins.exact_attention(qd, kd, vd, causal, sm)
    G = Hq // Hkv
    for hq in range(Hq):
        s = (qd[0, hq] @ kd[0, hq // G].T) * sm
        if causal:
            s = np.where(np.triu(np.ones((Sq, Sk), bool), 1 + Sk - Sq), -np.inf, s)
        p = np.exp(s - s.max(1, keepdims=True))
        lrow = p.sum(1, keepdims=True)
        bound = (2.0 ** -11 * (p @ np.abs(vd[0, hq // G])) + 2.0 ** -23 * np.abs(vd[0, hq // G]).sum(0)) / lrow
        err = np.abs(r["o"][0, hq] - O[0, hq])
        assert np.all(err <= bound * 1.001 + 1e-12), err.max()
    np.testing.assert_allclose(r["lse"], L, rtol=0, atol=1e-12 * (1 + np.abs(L).max()))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("bp", [0, 2500])
@pytest.mark.parametrize("case", CASES)
def test_d3_equals_two_pass(oracle, case, bp, fmt):
    Sq, Sk, Hq, Hkv, D, causal, bq = case
    q, k, v = _inputs(Sq, Sk, Hq, Hkv, D, 9)
    sm = 1.0 / np.sqrt(D)
    r = oracle.pipeline(q, k, v, fmt, bq, 64, causal, -1, bp, sm)
    dq, dk, dv = _decoded(oracle, r, fmt, q, k, v)
    O, L = pins.two_pass_attention(dq, dk, dv, q.astype(np.float64), k.astype(np.float64),
                                   v.astype(np.float64), r["idx"], r["cnt"], fmt, bq, 64, causal, sm)
    np.testing.assert_allclose(r["o"], O, rtol=1e-9, atol=1e-7 * np.abs(O).max())
    np.testing.assert_allclose(r["lse"], L, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_d4_last_block_equals_full_forward(oracle, causal):
    Sk, Hq, Hkv, D, bq = 640, 4, 2, 64, 128
    qf, k, v = _inputs(Sk, Sk, Hq, Hkv, D, 10)
    full = oracle.pipeline(qf, k, v, oracle.MX, bq, 64, causal, -1, 2000)
    qd = np.ascontiguousarray(qf[:, :, Sk - bq:])
    dec = oracle.pipeline(qd, k, v, oracle.MX, bq, 64, causal, -1, 2000)
    assert np.array_equal(dec["cnt"][:, :, 0], full["cnt"][:, :, -1])
    km = dec["idx"].shape[-1]
    assert np.array_equal(dec["idx"][:, :, 0], full["idx"][:, :, -1, :km])
    assert np.array_equal(dec["o"], full["o"][:, :, Sk - bq:])
    assert np.array_equal(dec["lse"], full["lse"][:, :, Sk - bq:])
