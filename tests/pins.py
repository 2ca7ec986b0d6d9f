"""Independent restatements used to pin the oracle (test helpers only).

Nothing here calls the oracle's C code: formats are rebuilt from their bit
fields, roundings by brute-force nearest-value search, and the attention
forward as a dense two-pass computation, so that a slip in the oracle's own
version (a dropped term, a wrong sign, a transposed operand) shows up as a
disagreement.
"""
from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


def e2m1_values_from_bits():
    """E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit)."""
    out = []
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = (m / 2.0) if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
        out.append(-mag if s else mag)
    return np.array(out)


def e4m3_values_from_bits():
    """Non-negative finite E4M3 values, codes 0..126 (bias 7, 3 mantissa bits)."""
    out = []
    for code in range(127):
        e, m = code >> 3, code & 7
        out.append(m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0))
    return np.array(out)


E2M1_POS = e2m1_values_from_bits()[:8]
E4M3_POS = e4m3_values_from_bits()


def nearest_code(q, table):
    """Brute-force nearest entry of an ascending non-negative table for |q|,
    ties to the even code; values past the end saturate to the last entry."""
    q = np.abs(np.asarray(q, np.float64))
    d = np.abs(q[..., None] - table)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    idx = np.arange(len(table))
    # among tied candidates prefer the even code
    even = cand & (idx % 2 == 0)
    has_even = even.any(axis=-1)
    first_even = np.argmax(even, axis=-1)
    first = np.argmax(cand, axis=-1)
    return np.where(has_even, first_even, first)


def e2m1_code(x, s):
    x = np.asarray(x, np.float64)
    c = nearest_code(x / s, E2M1_POS)
    return c | np.where(np.signbit(x), 8, 0)


def mx_exponent(amax):
    amax = np.asarray(amax, np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    x = np.clip(e - 1 - 2, -127, 127)
    return np.where(amax > 0, x, -127)


def decode_fp4(codes_u8, scales_u8, tensor_scale, fmt, axis, shape):
    """Decode FP4 tensors (two codes per byte, even element in the low nibble)
    to fp64 [B, H, S, D]."""
    B, H, S, D = shape
    lo = codes_u8 & 0xF
    hi = codes_u8 >> 4
    codes = np.stack([lo, hi], -1).reshape(*codes_u8.shape[:-1], -1)
    vals = e2m1_values_from_bits()[codes]
    g = 16 if fmt == 0 else 32
    if fmt == 0:
        sc = e4m3_values_from_bits()[scales_u8.astype(np.int64) & 0x7F] * np.asarray(
            tensor_scale, np.float64).reshape(B, H, 1, 1)
    else:
        sc = 2.0 ** (scales_u8.astype(np.float64) - 127)
    vals = vals * np.repeat(sc, g, axis=-1)
    if axis == 0:
        return vals
    return np.swapaxes(vals[..., :S], -1, -2)


def mx8_exponent(amax):
    """MXFP8 shared exponent: the largest power of two not above amax over
    E4M3's largest power of two, 2^8 (OCP MX); amax = 0 gives -127."""
    amax = np.asarray(amax, np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    x = np.clip(e - 1 - 8, -127, 127)
    return np.where(amax > 0, x, -127)


def fp8_quantize(x, axis):
    """MXFP8 restated: groups of 32 along D (axis 0) or along the sequence
    (axis 1, stored transposed and padded to 64 with zeros); the element code
    is the brute-force nearest E4M3 value of |x| / 2^X (ties to the even code,
    saturating at 448) with the sign bit of x."""
    x = np.asarray(x, np.float64)
    B, H, S, D = x.shape
    if axis == 1:
        Sp = -(-S // 64) * 64
        xt = np.zeros((B, H, D, Sp))
        xt[..., :S] = np.swapaxes(x, -1, -2)
        x = xt
    g = x.reshape(*x.shape[:-1], -1, 32)
    X = mx8_exponent(np.abs(g).max(-1))
    q = np.abs(g) / 2.0 ** X[..., None]
    codes = nearest_code(q, E4M3_POS) | np.where(np.signbit(g), 0x80, 0)
    return codes.reshape(x.shape).astype(np.uint8), (X + 127).astype(np.uint8)


def decode_fp8(codes_u8, scales_u8, axis, shape):
    """MXFP8 codes (one E4M3 byte each) and E8M0 scales to fp64 [B,H,S,D]."""
    B, H, S, D = shape
    mag = E4M3_POS[np.minimum(codes_u8 & 0x7F, 126)]
    vals = np.where(codes_u8 & 0x80, -mag, mag) * np.repeat(2.0 ** (scales_u8.astype(np.float64) - 127), 32, -1)
    if axis == 0:
        return vals
    return np.swapaxes(vals[..., :S], -1, -2)


def quantize_p_tile8(t, mask, eta=None):
    """P of a middle-tier (MXFP8) tile restated: v = 2^(t - max t) (level 1,
    the tile maximum), per 32 keys X = mx8_exponent(max v), brute-force E4M3
    codes of v / 2^X.  eta (optional) multiplies each v before its decisions.
    Returns (pq, mt): values relative to 2^mt."""
    mt = np.max(np.where(mask, -np.inf, t))
    v = np.where(mask, 0.0, np.exp2(np.where(mask, 0, t) - mt))
    if eta is not None:
        v = v * eta
    pq = np.zeros(len(t))
    for g0 in range(0, len(t), 32):
        seg = v[g0:g0 + 32]
        s2 = 2.0 ** mx8_exponent(seg.max())
        pq[g0:g0 + 32] = E4M3_POS[nearest_code(seg / s2, E4M3_POS)] * s2
    return pq, mt


def valid_blocks(i, S, bq, bk, causal, Sk=None):
    """Key blocks query block i may see; with Sk keys (default S) the S
    queries are the last S positions of the key sequence."""
    Sk = S if Sk is None else Sk
    nk = -(-Sk // bk)
    if not causal:
        return nk
    return (Sk - S + min(S, (i + 1) * bq) - 1) // bk + 1


def fp16_round(x):
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def quantize_p_tile(t, mask, fmt, eta=None):
    """Two-level P quantisation of one tile row (the oracle's reading of the
    pages: level 1 the tile maximum, v = 2^(t - max t); level 2 by format),
    restated with brute-force rounding.  eta (optional) multiplies each v
    before its decisions.  Returns (pq, mt): values relative to 2^mt."""
    mt = np.max(np.where(mask, -np.inf, t))
    n = len(t)
    pq = np.zeros(n)
    v = np.where(mask, 0.0, np.exp2(np.where(mask, 0, t) - mt))
    if eta is not None:
        v = v * eta
    if fmt == 0:
        v = 2688.0 * v
        for g0 in range(0, n, 16):
            seg = v[g0:g0 + 16]
            s2 = E4M3_POS[nearest_code(seg.max() / 6.0, E4M3_POS)]
            if s2 > 0:
                pq[g0:g0 + 16] = E2M1_POS[nearest_code(seg / s2, E2M1_POS)] * s2 / 2688.0
    else:
        for g0 in range(0, n, 32):
            seg = v[g0:g0 + 32]
            s2 = 2.0 ** mx_exponent(seg.max())
            pq[g0:g0 + 32] = E2M1_POS[nearest_code(seg / s2, E2M1_POS)] * s2
    return pq, mt


def fp16_tile(t, mask, eta=None):
    """FP16-path values of one tile row: fp16(2^(t - max t)) (level 1 the tile
    maximum, as the FP4 path).  Returns (pq, mt)."""
    mt = np.max(np.where(mask, -np.inf, t))
    v = np.where(mask, 0.0, np.exp2(np.where(mask, 0, t) - mt))
    if eta is not None:
        v = v * eta
    return np.where(mask, 0.0, fp16_round(v)), mt


def two_pass_attention(q4, k4, v4, q16, k16, v16, idx, cnt, fmt, bq, bk, causal, sm_scale,
                       eta_fn=None, mid=None, record=None):
    """Dense two-pass restatement of the forward pass: every score first,
    then one global maximum per row, then the weighted sum.  q4/k4/v4 and
    q16/k16/v16 are fp64 [B,H,S,D] (dequantised FP4 / decoded fp16).
    eta_fn(t, b, mask, kind) -> eta, if given, multiplies every tile value
    before its rounding decisions (only the decisions: level 1 and the row sum
    stay exact), as a lower-precision evaluation of the decision inputs would;
    b holds each score's chain sum (chain_sum) in the same log2 units.
    record (a list), with eta_fn: receives (b, hq, r, change) for every
    decision the perturbation flipped, change being that decision's effect
    on the output row (a block scale that flipped counts as one decision
    over its group, otherwise each element's code or fp16 rounding).
    mid = (q8, k8, v8, idx2, cnt2) adds the middle tier: blocks idx2 lists and
    idx does not use the decoded MXFP8 operands and the E4M3 P quantiser (MX
    format)."""
    B, Hq, S, D = q4.shape
    Hkv, Sk = k4.shape[1], k4.shape[2]
    G = Hq // Hkv
    nq = -(-S // bq)
    off = Sk - S  # queries are the last S positions
    O = np.zeros((B, Hq, S, D))
    L = np.zeros((B, Hq, S))
    for b in range(B):
        for hq in range(Hq):
            hk = hq // G
            t4 = (q4[b, hq] @ k4[b, hk].T) * sm_scale * LOG2E
            t16 = None if q16 is None else (q16[b, hq] @ k16[b, hk].T) * sm_scale * LOG2E
            a4 = a16 = a8 = None
            if eta_fn is not None:
                a4 = chain_sum(q4[b, hq], k4[b, hk], 64 if fmt == 1 else 16) * sm_scale * LOG2E
                a16 = None if q16 is None else chain_sum(q16[b, hq], k16[b, hk], 16) * sm_scale * LOG2E
            if mid is not None:
                t8 = (mid[0][b, hq] @ mid[1][b, hk].T) * sm_scale * LOG2E
                if eta_fn is not None:
                    a8 = chain_sum(mid[0][b, hq], mid[1][b, hk], 16) * sm_scale * LOG2E
            for i in range(nq):
                promoted = set(int(j) for j in idx[b, hq, i, : cnt[b, hq, i]])
                tier8 = set() if mid is None else set(int(j) for j in mid[3][b, hq, i, : mid[4][b, hq, i]])
                tier8 -= promoted
                nval = valid_blocks(i, S, bq, bk, causal, Sk)
                for r in range(i * bq, min(S, (i + 1) * bq)):
                    tiles = []  # (t row, mask, kind, c0, c1, a row)
                    for j in range(nval):
                        c0, c1 = j * bk, min(Sk, (j + 1) * bk)
                        keys = np.arange(c0, c1)
                        mask = (keys > r + off) if causal else np.zeros(len(keys), bool)
                        if mask.all():
                            continue
                        kind = 16 if j in promoted else (8 if j in tier8 else 4)
                        src, asrc = {16: (t16, a16), 8: (t8, a8) if mid is not None else None, 4: (t4, a4)}[kind]
                        tiles.append((src[r, c0:c1], mask, kind, c0, c1, None if asrc is None else asrc[r, c0:c1]))
                    M = max(np.max(np.where(m, -np.inf, t)) for t, m, _, _, _, _ in tiles)
                    l = 0.0
                    acc = np.zeros(D)
                    changes = []
                    for t, m, kind, c0, c1, a in tiles:
                        eta = None if eta_fn is None else eta_fn(t, a, m, kind)
                        l += np.where(m, 0.0, np.exp2(np.where(m, 0, t) - M)).sum()
                        vt = {8: mid[2] if mid is not None else None, 16: v16, 4: v4}[kind][b, hk, c0:c1]
                        quant = {8: quantize_p_tile8, 16: fp16_tile,
                                 4: lambda t_, m_, e_: quantize_p_tile(t_, m_, fmt, e_)}[kind]
                        pq, mt = quant(t, m, eta)
                        acc += (pq * np.exp2(mt - M)) @ vt
                        if record is not None and eta is not None:
                            p0, _ = quant(t, m, None)
                            gs = 1 if kind == 16 else (16 if (kind == 4 and fmt == 0) else 32)
                            for g0 in range(0, len(t), gs):
                                diff = (pq - p0)[g0:g0 + gs]
                                idxs = np.nonzero(diff)[0]
                                if len(idxs) == 0:
                                    continue
                                changes.append((diff * np.exp2(mt - M)) @ vt[g0:g0 + gs])
                    O[b, hq, r] = acc / l
                    L[b, hq, r] = M * LN2 + np.log(l)
                    for ch in changes:
                        record.append((b, hq, r, ch / l))
    return O, L


def chain_sum(q, k, width):
    """Per (query, key) score the chain sum of the evaluation-error model: over
    the contraction's slices of `width` channels in ascending order, the
    magnitude of the exact partial sum before the slice plus the slice's sum
    of |products|."""
    D = q.shape[-1]
    b = np.zeros((q.shape[0], k.shape[0]))
    part = np.zeros_like(b)
    for d0 in range(0, D, width):
        sl = slice(d0, min(D, d0 + width))
        b += np.abs(part) + np.abs(q[:, sl]) @ np.abs(k[:, sl]).T
        part += q[:, sl] @ k[:, sl].T
    return b


def exact_attention(q, k, v, causal, sm_scale):
    """Textbook softmax attention in fp64 (GQA by head groups); with more
    keys than queries, the queries are the last positions."""
    B, Hq, S, D = q.shape
    G, Sk = Hq // k.shape[1], k.shape[2]
    O = np.zeros_like(q)
    L = np.zeros((B, Hq, S))
    for b in range(B):
        for hq in range(Hq):
            s = (q[b, hq] @ k[b, hq // G].T) * sm_scale
            if causal:
                s = np.where(np.triu(np.ones((S, Sk), bool), 1 + Sk - S), -np.inf, s)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            O[b, hq] = (p @ v[b, hq // G]) / l
            L[b, hq] = (m + np.log(l))[:, 0]
    return O, L
