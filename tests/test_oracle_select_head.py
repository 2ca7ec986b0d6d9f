"""Pins of the oracle's per-head selection variant (CPU only): one budget
over all valid block pairs of a query head, the other reading of "the top-k
highest-scoring block pairs" (ThriftAttention summaries, "Heuristische
Blokkenselectie"; the budget is stated as a share of all query-key block
pairs, "Resultaten").

  H1  the kept pairs equal brute force over fp64 scores (pairs sorted by
      score, ties by lower query block then lower key block), wherever the
      K-th and (K+1)-th scores are separated beyond fp32 evaluation error;
  H2  counts: sum(cnt) per head = ceil(P * bp / 10^4) (or the absolute
      count), rows ascending and padded with -1;
  H3  all scores equal (Q = 0): the first K valid pairs in (query block,
      key block) order;
  H4  a single query block: identical to the per-query-block selection.
"""
import numpy as np
import pytest

from tests import pins

CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, bq, bp
    (1, 2, 1, 1000, 1000, 64, True, 128, 1000),
    (2, 4, 2, 700, 700, 64, False, 64, 500),
    (1, 2, 2, 300, 1300, 128, True, 128, 2500),
    (1, 1, 1, 5000, 5000, 64, True, 128, 200),
]


def _inputs(B, Hq, Hkv, Sq, Sk, D, seed):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, Hq, Sq, D)) * 0.7).astype(np.float16)
    k = (rng.standard_normal((B, Hkv, Sk, D)) * 0.7).astype(np.float16)
    k[:, :, :64] *= 3  # a sink-like first block
    return q, k


def _pairs(q, k, bq, bk, causal, b, hq, G):
    Sq, Sk = q.shape[2], k.shape[2]
    nq, nk = -(-Sq // bq), -(-Sk // bk)
    qm = np.stack([q[b, hq, i * bq:(i + 1) * bq].astype(np.float64).mean(0) for i in range(nq)])
    km = np.stack([k[b, hq // G, j * bk:(j + 1) * bk].astype(np.float64).mean(0) for j in range(nk)])
    out = []
    for i in range(nq):
        n = pins.valid_blocks(i, Sq, bq, 64, causal, Sk)
        s = km[:n] @ qm[i]
        out += [(float(s[j]), i, j) for j in range(n)]
    return out


@pytest.mark.parametrize("case", CASES)
def test_h1_h2_bruteforce(oracle, case):
    B, Hq, Hkv, Sq, Sk, D, causal, bq, bp = case
    q, k = _inputs(B, Hq, Hkv, Sq, Sk, D, 11)
    idx, cnt = oracle.select_head(q, k, bq, 64, causal, -1, bp)
    G = Hq // Hkv
    checked = 0
    for b in range(B):
        for hq in range(Hq):
            pairs = _pairs(q, k, bq, 64, causal, b, hq, G)
            P = len(pairs)
            K = min(P, -(-P * bp // 10000))
            assert cnt[b, hq].sum() == K
            got = set()
            for i in range(idx.shape[2]):
                row = idx[b, hq, i]
                c = cnt[b, hq, i]
                assert np.all(np.diff(row[:c]) > 0) and np.all(row[c:] == -1)
                got |= {(i, int(j)) for j in row[:c]}
            order = sorted(pairs, key=lambda p: (-p[0], p[1], p[2]))
            scale = max(abs(p[0]) for p in pairs)
            if K < P and order[K - 1][0] - order[K][0] > 1e-5 * scale:
                assert got == {(p[1], p[2]) for p in order[:K]}
                checked += 1
    assert checked >= 1


def test_h2_absolute_count(oracle):
    q, k = _inputs(1, 2, 1, 1000, 1000, 64, 12)
    idx, cnt = oracle.select_head(q, k, 128, 64, True, 7, 0)
    assert np.all(cnt.sum(axis=2) == 7)
    idx, cnt = oracle.select_head(q, k, 128, 64, True, 10 ** 6, 0)  # more than there are pairs
    assert np.all(cnt[0, 0] == [pins.valid_blocks(i, 1000, 128, 64, True) for i in range(8)])


@pytest.mark.parametrize("causal", [True, False])
def test_h3_all_equal_scores(oracle, causal):
    q, k = _inputs(1, 1, 1, 1000, 1000, 64, 13)
    q[:] = 0
    idx, cnt = oracle.select_head(q, k, 128, 64, causal, -1, 1500)
    valid = [(i, j) for i in range(8) for j in range(pins.valid_blocks(i, 1000, 128, 64, causal))]
    K = -(-len(valid) * 1500 // 10000)
    got = sorted((i, int(j)) for i in range(8) for j in idx[0, 0, i, : cnt[0, 0, i]])
    assert got == valid[:K]


def test_h4_single_query_block_equals_per_block(oracle):
    q, k = _inputs(1, 4, 2, 100, 3000, 128, 14)
    for bp in (0, 300, 2500, 10000):
        a_idx, a_cnt = oracle.select_head(q, k, 128, 64, True, -1, bp)
        b_idx, b_cnt, _ = oracle.select(q, k, 128, 64, True, -1, bp)
        assert np.array_equal(a_cnt, b_cnt)
        assert np.array_equal(a_idx[..., : b_idx.shape[-1]], b_idx)
