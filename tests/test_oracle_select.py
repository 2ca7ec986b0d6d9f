"""Pins of the oracle's block selection (CPU only).

  - token means against numpy's fp64 mean (exact sums, one rounding);
  - the per-query-block budget against its closed form at the workload
    shapes (5% of the valid pairs, rounded up);
  - the selected set against brute-force repeated argmax of qbar_i . kbar_j
    in fp64, ties to the lowest block index (ThriftAttention pages,
    "Heuristische Blokkenselectie");
  - invariances: token order inside a key block, block permutations, planted
    high-similarity pairs.
"""
import numpy as np
import pytest

from fp16_attention_amd import workloads as W
from tests import pins


def test_block_means_exact(oracle):
    rng = np.random.default_rng(0)
    x = (rng.standard_t(3, size=(2, 3, 333, 64)) * 50).astype(np.float16)
    for blk in (64, 128):
        got = oracle.block_means(x, blk)
        nb = -(-333 // blk)
        for j in range(nb):
            seg = x[:, :, j * blk:(j + 1) * blk].astype(np.float64)
            want = (seg.sum(axis=2) / seg.shape[2]).astype(np.float32)
            np.testing.assert_array_equal(got[:, :, j], want)


def _budget(n, bp):
    return min(n, -(-n * bp // 10000))


@pytest.mark.parametrize("name,total,kmax", [("long", 3406, 26), ("prefill", 238, 7)])
def test_budget_closed_form(oracle, name, total, kmax):
    w = W.WORKLOADS[name]
    nq = w.S // w.bq
    ks = [_budget(2 * i + 2, w.topk_bp) for i in range(nq)]  # causal, bq = 2 bk
    assert sum(ks) == total
    assert oracle.kmax(w.S, w.bq, w.bk, w.causal, -1, w.topk_bp) == kmax == max(ks)
    pairs = sum(2 * i + 2 for i in range(nq))
    assert abs(100.0 * total / pairs - 5) < 0.75  # the pages' 5% budget, rounded up per block


def _brute_select(q, k, bq, bk, causal, G, k_of):
    """Repeated argmax over fp64 scores; returns dict (b,hq,i) -> (set, min gap)."""
    B, Hq, S, D = q.shape
    nq, nk = -(-S // bq), -(-S // bk)
    qm = np.stack([q[:, :, i * bq:(i + 1) * bq].astype(np.float64).mean(2) for i in range(nq)], 2)
    km = np.stack([k[:, :, j * bk:(j + 1) * bk].astype(np.float64).mean(2) for j in range(nk)], 2)
    out = {}
    for b in range(B):
        for hq in range(Hq):
            for i in range(nq):
                n = pins.valid_blocks(i, S, bq, bk, causal)
                s = km[b, hq // G, :n] @ qm[b, hq, i]
                kk = k_of(n)
                chosen, rest = [], list(range(n))
                for _ in range(kk):
                    best = max(rest, key=lambda j: (s[j], -j))
                    chosen.append(best)
                    rest.remove(best)
                gap = np.inf
                if 0 < kk < n:
                    gap = min(s[j] for j in chosen) - max(s[j] for j in rest)
                out[(b, hq, i)] = (sorted(chosen), gap, np.abs(s).max())
    return out


@pytest.mark.parametrize("S,Hq,Hkv,causal,bq,bk,bp", [
    (700, 4, 2, True, 128, 64, 2000),
    (1000, 2, 2, False, 128, 64, 1500),
    (256, 1, 1, False, 64, 64, 5000),
    (513, 3, 1, True, 64, 64, 3000),
])
def test_select_vs_bruteforce(oracle, S, Hq, Hkv, causal, bq, bk, bp):
    rng = np.random.default_rng(S + Hq)
    q = (rng.standard_normal((1, Hq, S, 64)) + rng.standard_normal((1, Hq, 1, 64))).astype(np.float16)
    k = (rng.standard_normal((1, Hkv, S, 64)) * 2).astype(np.float16)
    idx, cnt, _ = oracle.select(q, k, bq, bk, causal, -1, bp)
    brute = _brute_select(q, k, bq, bk, causal, Hq // Hkv, lambda n: _budget(n, bp))
    checked = 0
    for (b, hq, i), (want, gap, scale) in brute.items():
        c = cnt[b, hq, i]
        assert c == len(want)
        got = idx[b, hq, i, :c].tolist()
        assert np.all(idx[b, hq, i, c:] == -1)
        assert got == sorted(got)
        if gap > 1e-5 * scale:  # far from a near-tie between fp32 and fp64 scores
            assert got == want, (b, hq, i)
            checked += 1
    assert checked >= 0.9 * len(brute)


def test_select_ties_lowest_index(oracle):
    rng = np.random.default_rng(1)
    S, D = 64 * 6, 64
    base = rng.standard_normal((1, 1, 64, D))
    k = rng.standard_normal((1, 1, S, D)) * 0.1
    k[:, :, 64:128] = base  # blocks 1, 3 and 4 identical and best
    k[:, :, 192:256] = base
    k[:, :, 256:320] = base[:, :, ::-1]  # same tokens, another order: same mean
    q = np.repeat(base.mean(2, keepdims=True), S, axis=2)
    q16, k16 = q.astype(np.float16), k.astype(np.float16)
    for kk, want in ((1, [1]), (2, [1, 3]), (3, [1, 3, 4])):
        idx, cnt, sc = oracle.select(q16, k16, 64, 64, False, kk, 0, with_scores=True)
        assert sc[0, 0, 0, 1] == sc[0, 0, 0, 3] == sc[0, 0, 0, 4]
        assert idx[0, 0, 0, :kk].tolist() == want


def test_select_block_permutation(oracle):
    rng = np.random.default_rng(2)
    S, D, bk = 64 * 8, 64, 64
    q = rng.standard_normal((1, 1, S, D)).astype(np.float16)
    k = rng.standard_normal((1, 1, S, D)).astype(np.float16)
    perm = rng.permutation(8)
    kp = k.reshape(1, 1, 8, bk, D)[:, :, perm].reshape(1, 1, S, D)
    a, _, _ = oracle.select(q, k, 128, bk, False, 3, 0)
    b, _, _ = oracle.select(q, kp, 128, bk, False, 3, 0)
    inv = np.argsort(perm)
    for i in range(a.shape[2]):
        assert sorted(inv[a[0, 0, i]].tolist()) == b[0, 0, i].tolist()
    # shuffling tokens inside each key block changes nothing
    ks = k.reshape(1, 1, 8, bk, D)[:, :, :, rng.permutation(bk)].reshape(1, 1, S, D)
    c, _, _ = oracle.select(q, ks, 128, bk, False, 3, 0)
    np.testing.assert_array_equal(a, c)


def test_planted_pairs_selected(oracle):
    w = W.WORKLOADS["long"].with_(S=4096, Hq=4, Hkv=2, planted=4)
    d = W.generate(w)
    idx, cnt, _ = oracle.select(d["q"], d["k"], w.bq, w.bk, w.causal, -1, w.topk_bp)
    assert len(d["planted"]) == 16
    for b, hq, i, j in d["planted"]:
        assert j in idx[b, hq, i, :cnt[b, hq, i]].tolist()


def test_planted_pairs_need_distinct_query_blocks():
    """The generator plants each head's pairs in distinct query blocks after
    the first, so it refuses more pairs than that (instead of searching
    forever)."""
    w = W.WORKLOADS["long"].with_(Hq=2, Hkv=1, S=1024)  # 7 query blocks after the first, 16 pairs asked
    with pytest.raises(ValueError):
        W.generate(w)
    assert len(W.generate(w.with_(planted=7))["planted"]) == 2 * 7
