"""The device arithmetic behind the parity bound (GPU).

The oracle lists a decision as one that may go either way when its exact
input lies within the bound of tho_eval_rel, whose constants model the
device's arithmetic: a block-scaled FP4 matrix instruction returns within
2.5 u (|C| + sum of |products|) of exact, an fp16 matrix instruction within
6 u (...), and exp2 within one ulp (u = 2^-24; the products of both
instructions are exact).  These are not documented properties; this test
measures them on random operands (E2M1 codes with block scales spread over
2^+-20, fp16 values spread over 2^+-8, accumulators zero and not) and
requires every error within the model's constant and the largest at least a
quarter of it (so the bound is not loose by 4x or more).  The kernels are
the test-only probes in tests/arith_probe.hip, built beside the library.
"""
import ctypes as C
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
U = 2.0 ** -24
KAPPA_FP4, KAPPA_F16 = 2.5, 6.0  # the oracle's model (thrift_oracle.c, tho_eval_rel)
NT = 64
E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, 0, -.5, -1, -1.5, -2, -3, -4, -6], np.longdouble)


def _lib():
    path = os.path.join(HERE, "libarith_probe.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build()")
    L = C.CDLL(path)
    P, I = C.c_void_p, C.c_int
    L.arith_probe_fp4.argtypes = [P] * 5 + [I, P]
    L.arith_probe_f16.argtypes = [P] * 3 + [I, P]
    L.arith_probe_exp2.argtypes = [P, P, I, P]
    L.arith_probe_nv_factor.argtypes = [P, P, I, P]
    return L


def _rows(out):
    """[NT, 64 lanes, 16 registers] -> [NT, 32, 32]: lane (n, h), register i
    holds row (i // 4) * 8 + 4 h + i % 4 of column n."""
    M = np.zeros((out.shape[0], 32, 32), out.dtype)
    for lane in range(64):
        n, h = lane % 32, lane // 32
        for i in range(16):
            M[:, (i // 4) * 8 + 4 * h + i % 4, n] = out[:, lane, i]
    return M


def _lanes(M):
    out = np.zeros((M.shape[0], 64, 16), M.dtype)
    for lane in range(64):
        n, h = lane % 32, lane // 32
        for i in range(16):
            out[:, lane, i] = M[:, (i // 4) * 8 + 4 * h + i % 4, n]
    return out


def _dev(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def _stream():
    import torch

    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr())


def test_block_scaled_fp4_instruction():
    import torch

    rng = np.random.default_rng(5)
    ca = rng.integers(0, 16, (NT, 32, 64))
    cb = rng.integers(0, 16, (NT, 64, 32))
    ea = rng.integers(-20, 21, (NT, 32, 2))
    eb = rng.integers(-20, 21, (NT, 32, 2))
    c0 = np.zeros((NT, 32, 32), np.float32)
    c0[NT // 2:] = (rng.standard_normal((NT // 2, 32, 32)) * 2.0 ** rng.integers(-10, 20, (NT // 2, 32, 32)))
    A = np.zeros((NT, 64, 16), np.uint8)
    Bm = np.zeros((NT, 64, 16), np.uint8)
    sa = np.zeros((NT, 64), np.uint32)
    sb = np.zeros((NT, 64), np.uint32)
    for lane in range(64):
        m, h = lane % 32, lane // 32
        x, y = ca[:, m, 32 * h:32 * h + 32], cb[:, 32 * h:32 * h + 32, m]
        A[:, lane] = (x[:, 0::2] | (x[:, 1::2] << 4)).astype(np.uint8)
        Bm[:, lane] = (y[:, 0::2] | (y[:, 1::2] << 4)).astype(np.uint8)
        sa[:, lane] = 127 + ea[:, m, h]
        sb[:, lane] = 127 + eb[:, m, h]
    out = _dev(_lanes(c0))
    a, b, ta, tb = _dev(A), _dev(Bm), _dev(sa), _dev(sb)
    assert _lib().arith_probe_fp4(_ptr(a), _ptr(b), _ptr(ta), _ptr(tb), _ptr(out), NT, _stream()) == 0
    torch.cuda.synchronize()
    G = _rows(out.cpu().numpy()).astype(np.longdouble)
    # exact products, summed in 80-bit long double (error far below u)
    va = E2M1[ca] * np.exp2(np.repeat(ea, 32, axis=2).astype(np.longdouble))
    vb = E2M1[cb] * np.exp2(np.repeat(eb, 32, axis=2).transpose(0, 2, 1).astype(np.longdouble))
    exact = c0.astype(np.longdouble) + np.einsum("tmk,tkn->tmn", va, vb)
    mag = np.abs(c0).astype(np.longdouble) + np.einsum("tmk,tkn->tmn", np.abs(va), np.abs(vb))
    ok = mag > 0
    ratio = float((np.abs(G - exact)[ok] / mag[ok]).max()) / U
    print(f"block-scaled FP4 instruction: max error {ratio:.3f} u of |C| + sum |products|", flush=True)
    assert ratio <= KAPPA_FP4
    assert ratio >= KAPPA_FP4 / 4


def test_fp16_instruction():
    import torch

    rng = np.random.default_rng(6)
    a16 = (rng.standard_normal((NT, 32, 16)) * 2.0 ** rng.integers(-8, 9, (NT, 32, 16))).astype(np.float16)
    b16 = (rng.standard_normal((NT, 16, 32)) * 2.0 ** rng.integers(-8, 9, (NT, 16, 32))).astype(np.float16)
    c0 = np.zeros((NT, 32, 32), np.float32)
    c0[NT // 2:] = rng.standard_normal((NT // 2, 32, 32)) * 2.0 ** rng.integers(-6, 12, (NT // 2, 32, 32))
    A = np.zeros((NT, 64, 8), np.float16)
    Bm = np.zeros((NT, 64, 8), np.float16)
    for lane in range(64):
        m, h = lane % 32, lane // 32
        A[:, lane] = a16[:, m, 8 * h:8 * h + 8]
        Bm[:, lane] = b16[:, 8 * h:8 * h + 8, m]
    out = _dev(_lanes(c0))
    a, b = _dev(A), _dev(Bm)
    assert _lib().arith_probe_f16(_ptr(a), _ptr(b), _ptr(out), NT, _stream()) == 0
    torch.cuda.synchronize()
    G = _rows(out.cpu().numpy()).astype(np.longdouble)
    va, vb = a16.astype(np.longdouble), b16.astype(np.longdouble)
    exact = c0.astype(np.longdouble) + np.einsum("tmk,tkn->tmn", va, vb)
    mag = np.abs(c0).astype(np.longdouble) + np.einsum("tmk,tkn->tmn", np.abs(va), np.abs(vb))
    ratio = float((np.abs(G - exact) / mag).max()) / U
    print(f"fp16 instruction: max error {ratio:.3f} u of |C| + sum |products|", flush=True)
    assert ratio <= KAPPA_F16
    assert ratio >= KAPPA_F16 / 4


def test_exp2():
    import torch

    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-126, 127, 1 << 20), rng.uniform(-1, 1, 1 << 20),
                        (np.arange(-126, 127)[:, None] + rng.uniform(-1e-5, 1e-5, (253, 256))).ravel()])
    x = x.astype(np.float32)
    xd = _dev(x)
    yd = torch.empty_like(xd)
    assert _lib().arith_probe_exp2(_ptr(xd), _ptr(yd), len(x), _stream()) == 0
    torch.cuda.synchronize()
    y = yd.cpu().numpy().astype(np.float64)
    ex = np.exp2(x.astype(np.float64))
    normal = ex >= 2.0 ** -126
    ulp = np.ldexp(1.0, np.floor(np.log2(ex[normal])).astype(int) - 23)
    err = float((np.abs(y[normal] - ex[normal]) / ulp).max())
    print(f"exp2: max error {err:.3f} ulp", flush=True)
    assert err <= 1.0 and err >= 0.25
    assert np.all(y[~normal] <= 2.0 ** -126)  # results below the normal range flush toward zero


def test_nvfp4_level2_factor():
    """The NVFP4 P quantisation scales a probability by 2688 / s2 (s2 the
    group's E4M3 block scale), formed as 2688 times the hardware reciprocal.
    The model allows that value four roundings in all (u each: the factor
    2688, the reciprocal, the products); the factor must stay within two of
    them, checked over every positive finite E4M3 value."""
    import torch

    vals = []
    for b in range(1, 127):  # positive finite E4M3 (0x7F is NaN)
        e, m = (b >> 3) & 0xF, b & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    x = np.array(vals, np.float32)
    xd = _dev(x)
    yd = torch.empty_like(xd)
    assert _lib().arith_probe_nv_factor(_ptr(xd), _ptr(yd), len(x), _stream()) == 0
    torch.cuda.synchronize()
    y = yd.cpu().numpy().astype(np.float64)
    ex = 2688.0 / x.astype(np.float64)
    err = float((np.abs(y - ex) / ex).max() / U)
    print(f"2688 * rcp(s2): max error {err:.3f} u over all {len(x)} positive E4M3 values", flush=True)
    assert err <= 2.0
