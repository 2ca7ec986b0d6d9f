"""Seeded synthetic inputs for the ThriftAttention forward pass.

This module only draws numbers: it holds none of the method's arithmetic and
is shared by the tests, the benchmark and the smoke check so that the HIP
path and the CPU oracle see the same inputs.  numpy's PCG64 generator
(``default_rng(seed)``) draws every value in fp64; values are then scaled and
rounded to fp16 (round to nearest even, saturating at +-65504).

The workloads stand in for the pages' long-context evaluation (LLM prefill
at 8K-131K tokens with grouped-query attention, and a video-diffusion
attention shape): no dataset or trained weight is used.  Heavy tails and
outlier channels stand in for the heavy-tailed attention activations that
make uniform FP4 attention lose quality.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

NVFP4 = 0
MX = 1


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    causal: bool
    bq: int
    bk: int
    topk_count: int  # >= 0: absolute promoted blocks per query block
    topk_bp: int  # used when topk_count < 0: basis points of the valid pairs
    fmt: int
    seed: int
    dist: str  # "gauss_outliers" | "heavy" | "ar1"
    sink: bool = False
    planted: int = 0
    Sq: int = 0  # > 0: decode shape, the last Sq positions are the queries (S = cache length)
    extra: dict = field(default_factory=dict)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 4x4 block pairs, top-2 per query block, NVFP4-style scales
    "tiny": Workload("tiny", 1, 1, 1, 256, 64, False, 64, 64, 2, 0, NVFP4, 0, "gauss_outliers"),
    # causal prefill, 5% of each query block's valid pairs
    "prefill": Workload("prefill", 1, 32, 32, 8192, 128, True, 128, 64, -1, 500, MX, 2, "heavy"),
    # budget sweep (the bench sweeps topk_bp over 0, 100, 500, 2500, 10000)
    "sweep": Workload("sweep", 2, 16, 16, 16384, 128, True, 128, 64, -1, 500, MX, 3, "heavy"),
    # long context, GQA 32/8, attention sink and planted pairs
    "long": Workload("long", 1, 32, 8, 32768, 128, True, 128, 64, -1, 500, MX, 4, "heavy",
                     sink=True, planted=16),
    # very long, GQA 8/2, 2% budget
    "verylong": Workload("verylong", 1, 8, 2, 131072, 128, True, 128, 64, -1, 200, MX, 5, "heavy"),
    # non-causal video-DiT shape with smooth AR(1) queries and keys, ragged tail
    "dit": Workload("dit", 1, 24, 24, 17550, 64, False, 128, 64, -1, 500, MX, 6, "ar1"),
    # decode: one new token per sequence against a 32K-token cache (GQA 32/8,
    # the long-context distribution with its sink), 5% of the key blocks in FP16
    "decode": Workload("decode", 8, 32, 8, 32768, 128, True, 128, 64, -1, 500, MX, 7, "heavy",
                       sink=True, Sq=1),
}


def _to_half(x: np.ndarray) -> np.ndarray:
    return np.clip(x, -65504.0, 65504.0).astype(np.float16)


def _heavy(rng, B, H, S, D):
    """Student-t (nu = 3) scaled 0.5, times a log-normal(0, 1) magnitude drawn
    per (head, channel)."""
    mag = rng.lognormal(0.0, 1.0, size=(H, D))
    x = rng.standard_t(3.0, size=(B, H, S, D)) * 0.5
    x *= mag[None, :, None, :]
    return x


def _ar1(rng, B, H, S, D, rho=0.9):
    """Per-channel AR(1) along the sequence: x_t = rho x_{t-1} + sqrt(1-rho^2) e_t."""
    e = rng.standard_normal(size=(B, H, S, D))
    x = np.empty_like(e)
    x[:, :, 0] = e[:, :, 0]
    c = np.sqrt(1.0 - rho * rho)
    for t in range(1, S):
        x[:, :, t] = rho * x[:, :, t - 1] + c * e[:, :, t]
    return x


def generate(w: Workload):
    """Return dict(q, k, v) of fp16 arrays [B, H, S, D] plus 'planted' pairs;
    for a decode shape (w.Sq > 0) q holds w.Sq positions, the last ones."""
    rng = np.random.default_rng(w.seed)
    B, Hq, Hkv, S, D = w.B, w.Hq, w.Hkv, w.S, w.D
    Sq = w.Sq if w.Sq else S
    planted = []
    if w.dist == "gauss_outliers":
        q = rng.standard_normal((B, Hq, Sq, D))
        k = rng.standard_normal((B, Hkv, S, D))
        v = rng.standard_normal((B, Hkv, S, D))
        for t in (q, k, v):  # two outlier channels in distinct 16- and 32-groups
            t[..., 5] *= 20.0
            t[..., 40 % D] *= 20.0
    elif w.dist == "heavy":
        q = _heavy(rng, B, Hq, Sq, D)
        k = _heavy(rng, B, Hkv, S, D)
        v = _heavy(rng, B, Hkv, S, D)
    elif w.dist == "ar1":
        q = _ar1(rng, B, Hq, Sq, D)
        k = _ar1(rng, B, Hkv, S, D)
        v = rng.standard_normal((B, Hkv, S, D))
    else:
        raise ValueError(w.dist)
    if w.sink:  # the first key block carries an attention sink: norm x8
        k[:, :, : min(w.bk, S)] *= 8.0
    if w.planted and not w.Sq:
        planted = _plant(rng, w, q, k)
    return dict(q=_to_half(np.ascontiguousarray(q)), k=_to_half(k), v=_to_half(v), planted=planted)


def _block_mean(x, blk):
    B, H, S, D = x.shape
    nb = -(-S // blk)
    out = np.zeros((B, H, nb, D))
    for j in range(nb):
        out[:, :, j] = x[:, :, j * blk:(j + 1) * blk].mean(axis=2)
    return out


def _plant(rng, w: Workload, q, k):
    """Plant w.planted high-similarity (query block, key block) pairs per query
    head: a random unit vector u times c is added to the query block's rows
    and to the key block's rows on that head's KV head.  c grows until every
    planted pair is the top-scoring valid key block of its query block, with
    a 10% margin; the final check is a brute-force pass over the block means
    of the fp16-rounded inputs."""
    B, Hq, S, D = q.shape
    G = Hq // w.Hkv
    nq = -(-S // w.bq)
    if w.planted > nq - 1:
        raise ValueError(f"{w.planted} planted pairs per head need as many distinct query blocks after the "
                         f"first; S = {S} has {nq - 1}")
    pairs = []
    for b in range(B):
        for hq in range(Hq):
            rows = set()
            while len(rows) < w.planted:
                i = int(rng.integers(1, nq))
                jmax = ((min(S, (i + 1) * w.bq) - 1) // w.bk) if w.causal else (-(-S // w.bk) - 1)
                j = int(rng.integers(1, jmax + 1))
                if i in rows:
                    continue
                rows.add(i)
                u = rng.standard_normal(D)
                u /= np.linalg.norm(u)
                pairs.append((b, hq, i, j, u))
    qm0 = _block_mean(q, w.bq)
    km0 = _block_mean(k, w.bk)

    def dominated(qm, km):
        for b, hq, i, j, _ in pairs:
            jmax = ((min(S, (i + 1) * w.bq) - 1) // w.bk) if w.causal else (km.shape[2] - 1)
            sc = km[b, hq // G, : jmax + 1] @ qm[b, hq, i]
            if int(np.argmax(sc)) != j or np.sort(sc)[-2] > 0.9 * sc[j]:
                return False
        return True

    c = 4.0
    for _ in range(60):
        qm, km = qm0.copy(), km0.copy()
        for b, hq, i, j, u in pairs:
            qm[b, hq, i] += c * u
            km[b, hq // G, j] += c * u
        if dominated(qm, km):
            qq, kk = q.copy(), k.copy()
            for b, hq, i, j, u in pairs:
                qq[b, hq, i * w.bq:(i + 1) * w.bq] += c * u
                kk[b, hq // G, j * w.bk:(j + 1) * w.bk] += c * u
            if dominated(_block_mean(_to_half(qq).astype(np.float64), w.bq),
                         _block_mean(_to_half(kk).astype(np.float64), w.bk)):
                q[...] = qq
                k[...] = kk
                return [(b, hq, i, j) for b, hq, i, j, _ in pairs]
        c *= 1.25
    raise RuntimeError("planting did not separate the pairs")
