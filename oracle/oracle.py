"""ctypes front end of the CPU oracle (oracle/thrift_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the product
package never does.  Arrays are numpy, host memory, [batch, head, seq, dim];
fp16 tensors are passed as ``np.float16`` and read bit by bit by the C side.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

NVFP4 = 0
MX = 1
NVFP4_MXP = 2  # attention only: NVFP4 tensors, P quantised MX-style
AXIS_D = 0
AXIS_S = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# THRIFT_ORACLE_LIB lets the mutation tests load a deliberately broken copy
_LIB_PATH = os.environ.get("THRIFT_ORACLE_LIB") or os.path.join(_HERE, "libthrift_oracle.so")
_lib = None


def lib():
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build_oracle  # noqa: PLC0415

            build_oracle.build()
        _lib = C.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


_P = C.c_void_p
_I = C.c_int
_D = C.c_double
_SZ = C.c_size_t


def _declare(L):
    L.tho_half_to_double.restype = _D
    L.tho_half_to_double.argtypes = [C.c_uint16]
    L.tho_round_to_half.restype = _D
    L.tho_round_to_half.argtypes = [_D]
    L.tho_e2m1_value.restype = _D
    L.tho_e2m1_value.argtypes = [_I]
    L.tho_e2m1_encode.restype = _I
    L.tho_e2m1_encode.argtypes = [_D, _D]
    L.tho_e4m3_value.restype = _D
    L.tho_e4m3_value.argtypes = [_I]
    L.tho_e4m3_encode_ratio.restype = _I
    L.tho_e4m3_encode_ratio.argtypes = [_D, _D]
    L.tho_mx_exponent.restype = _I
    L.tho_mx_exponent.argtypes = [_D]
    L.tho_group_size.restype = _I
    L.tho_group_size.argtypes = [_I]
    L.tho_pad_s.restype = _I
    L.tho_pad_s.argtypes = [_I]
    L.tho_kmax.restype = _I
    L.tho_kmax.argtypes = [_I] * 6
    L.tho_block_means.restype = None
    L.tho_block_means.argtypes = [_P, _I, _I, _I, _I, _I, _P]
    L.tho_block_score.restype = C.c_float
    L.tho_block_score.argtypes = [_P, _P, _I]
    L.tho_select.restype = None
    L.tho_select.argtypes = [_P, _P] + [_I] * 10 + [_P, _P, _I, _P]
    L.tho_kmax_kv.restype = _I
    L.tho_kmax_kv.argtypes = [_I] * 7
    L.tho_select_kv.restype = None
    L.tho_select_kv.argtypes = [_P, _P] + [_I] * 11 + [_P, _P, _I, _P]
    L.tho_select_head_kv.restype = None
    L.tho_select_head_kv.argtypes = [_P, _P] + [_I] * 11 + [_P, _P, _I]
    L.tho_quantize.restype = None
    L.tho_quantize.argtypes = [_P, _I, _I, _I, _I, _I, _I, _P, _P, _P]
    L.tho_dequantize.restype = None
    L.tho_dequantize.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P]
    L.tho_attention.restype = None
    L.tho_attention.argtypes = [_P] * 12 + [_I, _P, _P, _I] + [_I] * 8 + [_D, _P, _I, _P, _P, _P, _P, _I, _P]
    L.tho_attention_kv.restype = None
    L.tho_attention_kv.argtypes = ([_P] * 12 + [_I, _P, _P, _I] + [_I] * 9
                                   + [_D, _P, _I, _P, _P, _P, _P, _I, _P])
    L.tho_attention_hp.restype = None
    L.tho_attention_hp.argtypes = [_P] * 12 + [_I, _P, _P, _I] + [_I] * 8 + [_D, _P, _I, _P, _P, _P]
    L.tho_attention_bwd.restype = None
    L.tho_attention_bwd.argtypes = ([_P] * 12 + [_I, _P, _P, _I] + [_I] * 8 + [_D, _P, _P, _P]
                                    + [_P, _I, _P, _I] + [_P] * 4)
    L.tho_row_probs.restype = None
    L.tho_row_probs.argtypes = [_P] * 12 + [_I, _P, _P, _I] + [_I] * 8 + [_D, _P, _I, _I, _I] + [_P] * 3
    L.tho_mx8_exponent.restype = _I
    L.tho_mx8_exponent.argtypes = [_D]
    L.tho_e4m3_encode_signed.restype = _I
    L.tho_e4m3_encode_signed.argtypes = [_D, _D]
    L.tho_quantize_fp8.restype = None
    L.tho_quantize_fp8.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P]
    L.tho_dequantize_fp8.restype = None
    L.tho_dequantize_fp8.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P]
    L.tho_attention_tiers.restype = None
    L.tho_attention_tiers.argtypes = ([_P] * 17 + [_I, _P, _P, _I] + [_I] * 8
                                      + [_D, _P, _I, _P, _P, _P, _P, _I, _P])
    L.tho_p_tile_decisions.restype = _I
    L.tho_p_tile_decisions.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _I]
    L.tho_eval_rel.restype = _D
    L.tho_eval_rel.argtypes = [_I, _D, _D, _D, _D]
    L.tho_fp4_scores.restype = None
    L.tho_fp4_scores.argtypes = [_P] * 6 + [_I] * 6 + [_P]
    L.tho_e2m1_encode_array.restype = None
    L.tho_e2m1_encode_array.argtypes = [_P, _P, _SZ, _P]
    L.tho_e4m3_encode_ratio_array.restype = None
    L.tho_e4m3_encode_ratio_array.argtypes = [_P, _P, _SZ, _P]
    L.tho_round_to_half_array.restype = None
    L.tho_round_to_half_array.argtypes = [_P, _SZ, _P]
    L.tho_half_to_double_array.restype = None
    L.tho_half_to_double_array.argtypes = [_P, _SZ, _P]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def group_size(fmt: int) -> int:
    return 16 if fmt == NVFP4 else 32


def pad_s(S: int) -> int:
    return lib().tho_pad_s(S)


def kmax(S, bq, bk, causal, topk_count, topk_bp, Sk=None) -> int:
    """Largest per-query-block budget; Sk (keys, default S) for S queries at
    the end of a longer key sequence."""
    return lib().tho_kmax_kv(S, S if Sk is None else Sk, bq, bk, int(causal), topk_count, topk_bp)


# ---- scalar / array format routines ------------------------------------

def e2m1_encode(x, s):
    x = _c(np.broadcast_to(x, np.broadcast(x, s).shape), np.float64)
    s = _c(np.broadcast_to(s, x.shape), np.float64)
    out = np.empty(x.shape, np.uint8)
    lib().tho_e2m1_encode_array(_ptr(x), _ptr(s), x.size, _ptr(out))
    return out


def e4m3_encode_ratio(num, den):
    num = _c(np.broadcast_to(num, np.broadcast(num, den).shape), np.float64)
    den = _c(np.broadcast_to(den, num.shape), np.float64)
    out = np.empty(num.shape, np.uint8)
    lib().tho_e4m3_encode_ratio_array(_ptr(num), _ptr(den), num.size, _ptr(out))
    return out


def e2m1_value(code: int) -> float:
    return lib().tho_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return lib().tho_e4m3_value(int(code))


def mx_exponent(amax: float) -> int:
    return lib().tho_mx_exponent(float(amax))


def round_to_half(x):
    x = _c(x, np.float64)
    out = np.empty_like(x)
    lib().tho_round_to_half_array(_ptr(x), x.size, _ptr(out))
    return out


def half_to_double(h):
    h = _c(h, np.float16).view(np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().tho_half_to_double_array(_ptr(h), h.size, _ptr(out))
    return out


# ---- selection ------------------------------------------------------------

def block_means(x16, blk):
    x16 = _c(x16, np.float16)
    B, H, S, D = x16.shape
    nb = -(-S // blk)
    out = np.empty((B, H, nb, D), np.float32)
    lib().tho_block_means(_ptr(x16), B, H, S, D, blk, _ptr(out))
    return out


def select(q16, k16, bq, bk, causal, topk_count=-1, topk_bp=0, kmax_=None, with_scores=False):
    """Per-query-block top-k: returns (idx [B,Hq,nQ,kmax] int32, cnt [B,Hq,nQ] int32, scores).
    k16 may hold more positions than q16 (queries = the last positions)."""
    q16 = _c(q16, np.float16)
    k16 = _c(k16, np.float16)
    B, Hq, S, D = q16.shape
    Hkv, Sk = k16.shape[1], k16.shape[2]
    nq, nk = -(-S // bq), -(-Sk // bk)
    km = kmax(S, bq, bk, causal, topk_count, topk_bp, Sk) if kmax_ is None else kmax_
    idx = np.empty((B, Hq, nq, max(km, 0)), np.int32)
    cnt = np.empty((B, Hq, nq), np.int32)
    scores = np.empty((B, Hq, nq, nk), np.float32) if with_scores else None
    lib().tho_select_kv(_ptr(q16), _ptr(k16), B, Hq, Hkv, S, Sk, D, bq, bk, int(causal), topk_count,
                        topk_bp, _ptr(idx), _ptr(cnt), km, _ptr(scores))
    return idx, cnt, scores


def kmax_head(S, bq, bk, causal, Sk=None) -> int:
    """Row length that always holds a per-head selection: the largest n_i."""
    Sk = S if Sk is None else Sk
    nq = -(-S // bq)
    return max(((Sk - S + min(S, (i + 1) * bq) - 1) // bk + 1) if causal else -(-Sk // bk) for i in range(nq))


def select_head(q16, k16, bq, bk, causal, topk_count=-1, topk_bp=0, kmax_=None):
    """One budget per query head over all its valid block pairs: returns
    (idx [B,Hq,nQ,kmax] int32, cnt [B,Hq,nQ] int32)."""
    q16 = _c(q16, np.float16)
    k16 = _c(k16, np.float16)
    B, Hq, S, D = q16.shape
    Hkv, Sk = k16.shape[1], k16.shape[2]
    nq = -(-S // bq)
    km = kmax_head(S, bq, bk, causal, Sk) if kmax_ is None else kmax_
    idx = np.empty((B, Hq, nq, km), np.int32)
    cnt = np.empty((B, Hq, nq), np.int32)
    lib().tho_select_head_kv(_ptr(q16), _ptr(k16), B, Hq, Hkv, S, Sk, D, bq, bk, int(causal), topk_count,
                             topk_bp, _ptr(idx), _ptr(cnt), km)
    return idx, cnt


# ---- quantisation -----------------------------------------------------------

class FP4Tensor:
    """Codes, block scales and (NVFP4-style only) per-slice fp32 scales."""

    def __init__(self, codes, scales, tensor_scale, fmt, axis, shape):
        self.codes, self.scales, self.tensor_scale = codes, scales, tensor_scale
        self.fmt, self.axis, self.shape = fmt, axis, shape


def quantize(x16, axis, fmt) -> FP4Tensor:
    x16 = _c(x16, np.float16)
    B, H, S, D = x16.shape
    g = group_size(fmt)
    if axis == AXIS_D:
        codes = np.empty((B, H, S, D // 2), np.uint8)
        scales = np.empty((B, H, S, D // g), np.uint8)
    else:
        Sp = pad_s(S)
        codes = np.empty((B, H, D, Sp // 2), np.uint8)
        scales = np.empty((B, H, D, Sp // g), np.uint8)
    ts = np.empty((B, H), np.float32) if fmt == NVFP4 else None
    lib().tho_quantize(_ptr(x16), B, H, S, D, axis, fmt, _ptr(codes), _ptr(scales), _ptr(ts))
    return FP4Tensor(codes, scales, ts, fmt, axis, (B, H, S, D))


def dequantize(t: FP4Tensor):
    B, H, S, D = t.shape
    out = np.empty((B, H, S, D), np.float64)
    lib().tho_dequantize(_ptr(t.codes), _ptr(t.scales), _ptr(t.tensor_scale), B, H, S, D, t.axis,
                         t.fmt, _ptr(out))
    return out


class FP8Tensor:
    """MXFP8 codes (one E4M3 byte per element) and E8M0 scales per 32."""

    def __init__(self, codes, scales, axis, shape):
        self.codes, self.scales, self.axis, self.shape = codes, scales, axis, shape


def mx8_exponent(amax: float) -> int:
    return lib().tho_mx8_exponent(float(amax))


def e4m3_encode_signed(x: float, s: float) -> int:
    return lib().tho_e4m3_encode_signed(float(x), float(s))


def quantize_fp8(x16, axis) -> FP8Tensor:
    """MXFP8 of x16 [B,H,S,D]: along D, codes [B,H,S,D] and scales
    [B,H,S,D/32]; along the sequence (V), codes [B,H,D,Sp], scales
    [B,H,D,Sp/32] with zero padding tokens."""
    x16 = _c(x16, np.float16)
    B, H, S, D = x16.shape
    if axis == AXIS_D:
        codes = np.empty((B, H, S, D), np.uint8)
        scales = np.empty((B, H, S, D // 32), np.uint8)
    else:
        Sp = pad_s(S)
        codes = np.empty((B, H, D, Sp), np.uint8)
        scales = np.empty((B, H, D, Sp // 32), np.uint8)
    lib().tho_quantize_fp8(_ptr(x16), B, H, S, D, axis, _ptr(codes), _ptr(scales))
    return FP8Tensor(codes, scales, axis, (B, H, S, D))


def dequantize_fp8(t: FP8Tensor):
    B, H, S, D = t.shape
    out = np.empty((B, H, S, D), np.float64)
    lib().tho_dequantize_fp8(_ptr(t.codes), _ptr(t.scales), B, H, S, D, t.axis, _ptr(out))
    return out


def fp4_scores(q4: FP4Tensor, k4: FP4Tensor, r, c0, c1):
    """Raw FP4-path dot products of query row r with keys [c0, c1) (B = H = 1)."""
    _, _, S, D = q4.shape
    out = np.empty(c1 - c0, np.float64)
    lib().tho_fp4_scores(_ptr(q4.codes), _ptr(q4.scales), _ptr(q4.tensor_scale), _ptr(k4.codes),
                         _ptr(k4.scales), _ptr(k4.tensor_scale), q4.fmt, S, D, r, c0, c1, _ptr(out))
    return out


# ---- attention ----------------------------------------------------------------

class Ambiguity:
    """Decisions of a forward whose exact input lies within device evaluation
    error of its rounding boundary (both outcomes are valid results): for
    decision k, rows[k] is the flat row index (b * Hq + hq) * S + r and
    delta[k] the change of that output row if the decision takes its other
    outcome."""

    def __init__(self, rows, delta, shape):
        self.rows, self.delta, self.shape = rows, delta, shape

    def for_row(self, b, hq, r):
        B, Hq, S, D = self.shape
        return self.delta[self.rows == (b * Hq + hq) * S + r]

    def count_rows(self):
        return len(np.unique(self.rows))


def _call_amb(call, B, Hq, S, D, rows_hint):
    """Run call(amb_row, amb_delta, cap, n_ptr) with enough room for the list."""
    cap = max(4096, 2 * rows_hint)
    while True:
        rows = np.zeros(cap, np.int32)
        delta = np.zeros((cap, D), np.float64)
        n = np.zeros(1, np.int32)
        call(_ptr(rows), _ptr(delta), cap, _ptr(n))
        k = int(n[0])
        if k <= cap:
            return Ambiguity(rows[:k].astype(np.int64), delta[:k], (B, Hq, S, D))
        cap = k


def attention(q16, k16, v16, q4: FP4Tensor, k4: FP4Tensor, v4: FP4Tensor, idx, cnt, bq, bk,
              causal, sm_scale=None, work=None, with_amb=False, p_fmt=None):
    """Forward pass.  Returns (o fp64 [B,Hq,S,D], lse fp64 [B,Hq,S]) and, with
    with_amb, the Ambiguity list of decisions within device evaluation error
    of their boundary; with a work list of (b, hq, i) triples only those query
    blocks are filled (the rest stay NaN).  p_fmt=MX with NVFP4 tensors
    quantises P MX-style (the variant)."""
    B, Hq, S, D = q4.shape
    Hkv, Sk = k4.shape[1], k4.shape[2]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    q16 = None if q16 is None else _c(q16, np.float16)
    k16 = None if k16 is None else _c(k16, np.float16)
    v16 = None if v16 is None else _c(v16, np.float16)
    idx = _c(idx, np.int32)
    cnt = _c(cnt, np.int32)
    km = idx.shape[-1]
    o = np.full((B, Hq, S, D), np.nan, np.float64)
    lse = np.full((B, Hq, S), np.nan, np.float64)
    w = None if work is None else _c(np.asarray(work).reshape(-1, 3), np.int32)
    nw = 0 if w is None else w.shape[0]

    def call(ar, ad, cap, n):
        lib().tho_attention_kv(_ptr(q16), _ptr(k16), _ptr(v16), _ptr(q4.codes), _ptr(q4.scales),
                               _ptr(q4.tensor_scale), _ptr(k4.codes), _ptr(k4.scales),
                               _ptr(k4.tensor_scale), _ptr(v4.codes), _ptr(v4.scales),
                               _ptr(v4.tensor_scale),
                               NVFP4_MXP if (q4.fmt == NVFP4 and p_fmt == MX) else q4.fmt, _ptr(idx),
                               _ptr(cnt), km, B, Hq, Hkv, S, Sk, D, bq, bk, int(causal),
                               float(sm_scale), _ptr(w), nw, _ptr(o), _ptr(lse), ar, ad, cap, n)

    if not with_amb:
        call(None, None, 0, None)
        return o, lse
    amb = _call_amb(call, B, Hq, S, D, (nw * bq if w is not None else B * Hq * S))
    return o, lse, amb


def attention_tiers(q16, k16, v16, q4: FP4Tensor, k4: FP4Tensor, v4: FP4Tensor, q8: FP8Tensor,
                    k8: FP8Tensor, v8: FP8Tensor, idx, cnt, idx2, cnt2, bq, bk, causal, sm_scale=None,
                    work=None, with_amb=False):
    """Forward with the middle (MXFP8) tier, MX format: blocks idx lists run
    in FP16, blocks idx2 lists and idx does not in FP8, the rest in FP4.
    Returns (o, lse) and with with_amb the Ambiguity list."""
    B, Hq, S, D = q4.shape
    Hkv = k4.shape[1]
    assert q4.fmt == MX
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    q16 = None if q16 is None else _c(q16, np.float16)
    k16 = None if k16 is None else _c(k16, np.float16)
    v16 = None if v16 is None else _c(v16, np.float16)
    idx, cnt = _c(idx, np.int32), _c(cnt, np.int32)
    idx2, cnt2 = _c(idx2, np.int32), _c(cnt2, np.int32)
    o = np.full((B, Hq, S, D), np.nan, np.float64)
    lse = np.full((B, Hq, S), np.nan, np.float64)
    w = None if work is None else _c(np.asarray(work).reshape(-1, 3), np.int32)
    nw = 0 if w is None else w.shape[0]

    def call(ar, ad, cap, n):
        lib().tho_attention_tiers(_ptr(q16), _ptr(k16), _ptr(v16), _ptr(q4.codes), _ptr(q4.scales),
                                  _ptr(k4.codes), _ptr(k4.scales), _ptr(v4.codes), _ptr(v4.scales),
                                  _ptr(q8.codes), _ptr(q8.scales), _ptr(k8.codes), _ptr(k8.scales),
                                  _ptr(v8.codes), _ptr(v8.scales), _ptr(idx), _ptr(cnt), idx.shape[-1],
                                  _ptr(idx2), _ptr(cnt2), idx2.shape[-1], B, Hq, Hkv, S, D, bq, bk,
                                  int(causal), float(sm_scale), _ptr(w), nw, _ptr(o), _ptr(lse), ar, ad,
                                  cap, n)

    if not with_amb:
        call(None, None, 0, None)
        return o, lse
    amb = _call_amb(call, B, Hq, S, D, (nw * bq if w is not None else B * Hq * S))
    return o, lse, amb


def p_tile_decisions(t, tb, mask, prec, epath=None):
    """Test hook: (pq, decisions) of one tile row: values relative to 2^max t
    and a list of (k0, k1, change of each key's value) per decision that may
    go either way."""
    n = len(t)
    t, tb = _c(t, np.float64), _c(tb, np.float64)
    mask = _c(mask, np.int32)
    pq = np.zeros(n)
    cap = 600
    k0, k1 = np.zeros(cap, np.int32), np.zeros(cap, np.int32)
    dp = np.zeros((cap, 64))
    nf = lib().tho_p_tile_decisions(_ptr(t), _ptr(tb), _ptr(mask), n, int(prec),
                                    int(prec if epath is None else epath), _ptr(pq), _ptr(k0), _ptr(k1),
                                    _ptr(dp), cap)
    assert nf <= cap
    return pq, [(int(k0[f]), int(k1[f]), dp[f, :n].copy()) for f in range(nf)]


def eval_rel(path, b, bmax, dt, mt):
    """The oracle's relative evaluation-error bound of a tile value (path 0 MX
    FP4, 1 NVFP4 FP4, 2 MXFP8 tier, 3 FP16; b, bmax the chain sums)."""
    return lib().tho_eval_rel(int(path), float(b), float(bmax), float(dt), float(mt))


def attention_hp(q16, k16, v16, q4: FP4Tensor, k4: FP4Tensor, v4: FP4Tensor, idx, cnt, bq, bk,
                 causal, sm_scale=None, work=None):
    """Forward with Attn-QAT's high-precision output: (o, lse, ohp), ohp the
    output with the exact softmax probabilities (fp64 [B,Hq,S,D]).  Sq = Sk."""
    B, Hq, S, D = q4.shape
    Hkv = k4.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    q16 = None if q16 is None else _c(q16, np.float16)
    k16 = None if k16 is None else _c(k16, np.float16)
    v16 = None if v16 is None else _c(v16, np.float16)
    idx = _c(idx, np.int32)
    cnt = _c(cnt, np.int32)
    o = np.full((B, Hq, S, D), np.nan, np.float64)
    lse = np.full((B, Hq, S), np.nan, np.float64)
    ohp = np.full((B, Hq, S, D), np.nan, np.float64)
    w = None if work is None else _c(np.asarray(work).reshape(-1, 3), np.int32)
    nw = 0 if w is None else w.shape[0]
    lib().tho_attention_hp(_ptr(q16), _ptr(k16), _ptr(v16), _ptr(q4.codes), _ptr(q4.scales),
                           _ptr(q4.tensor_scale), _ptr(k4.codes), _ptr(k4.scales),
                           _ptr(k4.tensor_scale), _ptr(v4.codes), _ptr(v4.scales),
                           _ptr(v4.tensor_scale), q4.fmt, _ptr(idx), _ptr(cnt), idx.shape[-1], B, Hq,
                           Hkv, S, D, bq, bk, int(causal), float(sm_scale), _ptr(w), nw, _ptr(o),
                           _ptr(lse), _ptr(ohp))
    return o, lse, ohp


def attention_bwd(q16, k16, v16, q4: FP4Tensor, k4: FP4Tensor, v4: FP4Tensor, idx, cnt, bq, bk,
                  causal, lse, ohp, do16, sm_scale=None, qwork=None, kwork=None, with_u=False):
    """Backward (Attn-QAT).  Returns (dq, dk, dv) fp64, and with with_u the
    decision-uncertainty bound of dv; with work lists of (b, hq, i) query
    blocks and (b, hk, j) key blocks only those rows are filled (the rest
    stay NaN)."""
    B, Hq, S, D = q4.shape
    Hkv = k4.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    q16 = None if q16 is None else _c(q16, np.float16)
    k16 = None if k16 is None else _c(k16, np.float16)
    v16 = None if v16 is None else _c(v16, np.float16)
    idx = _c(idx, np.int32)
    cnt = _c(cnt, np.int32)
    lse = _c(lse, np.float64)
    ohp = _c(ohp, np.float64)
    do16 = _c(do16, np.float16)
    dq = np.full((B, Hq, S, D), np.nan, np.float64)
    dk = np.full((B, Hkv, S, D), np.nan, np.float64)
    dv = np.full((B, Hkv, S, D), np.nan, np.float64)
    udv = np.full((B, Hkv, S, D), np.nan, np.float64) if with_u else None
    qw = None if qwork is None else _c(np.asarray(qwork).reshape(-1, 3), np.int32)
    kw = None if kwork is None else _c(np.asarray(kwork).reshape(-1, 3), np.int32)
    lib().tho_attention_bwd(_ptr(q16), _ptr(k16), _ptr(v16), _ptr(q4.codes), _ptr(q4.scales),
                            _ptr(q4.tensor_scale), _ptr(k4.codes), _ptr(k4.scales),
                            _ptr(k4.tensor_scale), _ptr(v4.codes), _ptr(v4.scales),
                            _ptr(v4.tensor_scale), q4.fmt, _ptr(idx), _ptr(cnt), idx.shape[-1], B,
                            Hq, Hkv, S, D, bq, bk, int(causal), float(sm_scale), _ptr(lse),
                            _ptr(ohp), _ptr(do16), _ptr(qw), 0 if qw is None else qw.shape[0],
                            _ptr(kw), 0 if kw is None else kw.shape[0], _ptr(dq), _ptr(dk),
                            _ptr(dv), _ptr(udv))
    return (dq, dk, dv, udv) if with_u else (dq, dk, dv)


def row_probs(q16, k16, v16, q4: FP4Tensor, k4: FP4Tensor, v4: FP4Tensor, idx, cnt, bq, bk, causal,
              lse, b, hq, r, sm_scale=None):
    """Test hook: (kind, p, pt) of query row r of head (b, hq) against every
    key, as the backward recomputes them (kind 0 masked/invalid, 1 FP4 path,
    2 FP16 path; p the exact probability; pt the one the forward's PV product
    used)."""
    B, Hq, S, D = q4.shape
    Hkv = k4.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    q16 = None if q16 is None else _c(q16, np.float16)
    k16 = None if k16 is None else _c(k16, np.float16)
    v16 = None if v16 is None else _c(v16, np.float16)
    idx = _c(idx, np.int32)
    cnt = _c(cnt, np.int32)
    lse = _c(lse, np.float64)
    kind = np.zeros(S, np.int32)
    p = np.zeros(S, np.float64)
    pt = np.zeros(S, np.float64)
    lib().tho_row_probs(_ptr(q16), _ptr(k16), _ptr(v16), _ptr(q4.codes), _ptr(q4.scales),
                        _ptr(q4.tensor_scale), _ptr(k4.codes), _ptr(k4.scales),
                        _ptr(k4.tensor_scale), _ptr(v4.codes), _ptr(v4.scales),
                        _ptr(v4.tensor_scale), q4.fmt, _ptr(idx), _ptr(cnt), idx.shape[-1], B, Hq,
                        Hkv, S, D, bq, bk, int(causal), float(sm_scale), _ptr(lse), b, hq, r,
                        _ptr(kind), _ptr(p), _ptr(pt))
    return kind, p, pt


def pipeline(q16, k16, v16, fmt, bq, bk, causal, topk_count=-1, topk_bp=0, sm_scale=None,
             work=None, p_fmt=None, with_amb=True):
    """Selection, quantisation of Q/K/V and attention, all on the oracle
    (with_amb: also the list of decisions that may go either way)."""
    idx, cnt, _ = select(q16, k16, bq, bk, causal, topk_count, topk_bp)
    q4 = quantize(q16, AXIS_D, fmt)
    k4 = quantize(k16, AXIS_D, fmt)
    v4 = quantize(v16, AXIS_S, fmt)
    res = attention(q16, k16, v16, q4, k4, v4, idx, cnt, bq, bk, causal, sm_scale, work, with_amb=with_amb,
                    p_fmt=p_fmt)
    return dict(idx=idx, cnt=cnt, q4=q4, k4=k4, v4=v4, o=res[0], lse=res[1], amb=res[2] if with_amb else None)


def pipeline_tiers(q16, k16, v16, bq, bk, causal, bp16, bp8, sm_scale=None, work=None, with_amb=True):
    """The three-tier forward on the oracle (MX format): the FP16 tier is the
    selection under budget bp16, the FP16 and FP8 tiers together the
    selection under bp16 + bp8 (basis points each)."""
    idx, cnt, _ = select(q16, k16, bq, bk, causal, -1, bp16)
    idx2, cnt2, _ = select(q16, k16, bq, bk, causal, -1, bp16 + bp8)
    q4, k4, v4 = quantize(q16, AXIS_D, MX), quantize(k16, AXIS_D, MX), quantize(v16, AXIS_S, MX)
    q8, k8, v8 = quantize_fp8(q16, AXIS_D), quantize_fp8(k16, AXIS_D), quantize_fp8(v16, AXIS_S)
    res = attention_tiers(q16, k16, v16, q4, k4, v4, q8, k8, v8, idx, cnt, idx2, cnt2, bq, bk,
                          causal, sm_scale, work, with_amb=with_amb)
    return dict(idx=idx, cnt=cnt, idx2=idx2, cnt2=cnt2, q4=q4, k4=k4, v4=v4, q8=q8, k8=k8, v8=v8,
                o=res[0], lse=res[1], amb=res[2] if with_amb else None)
