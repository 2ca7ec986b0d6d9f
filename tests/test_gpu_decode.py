"""GPU parity of the decode-shaped forward (thrift_select_blocks_kv,
thrift_attention_decode) against the CPU oracle, through the C ABI, in both
FP4 formats.

Bit-exact: selected blocks, counts and FP4 codes/scales.  Output: fp32 O and
LSE to the bounds of the prefill parity tests (max-abs 2e-3 beyond the
oracle's evaluation uncertainty u, rel-L2 1e-3).  Sizes span one to several
workgroup key splits, ragged cache lengths, GQA packing of several heads and
rows into one query tile, both masks, and the budget extremes; the last case
is the decode workload at full size, every row compared.
"""
import numpy as np
import pytest

from fp16_attention_amd import workloads as W
from tests.gpu_harness import compare_out, note, same_fp4

pytestmark = pytest.mark.gpu

CASES = {
    # name: (B, Hq, Hkv, Sq, Sk, D, causal, topk_bp, fmt)
    "one_token_gqa4": (2, 8, 2, 1, 2048, 128, True, 500, 1),
    "rows5_ragged": (1, 4, 1, 5, 1000, 128, True, 1000, 1),
    "rows8_gqa4": (1, 8, 2, 8, 4096, 128, True, 500, 1),
    "d64_noncausal": (1, 4, 2, 3, 777, 64, False, 2500, 1),
    "no_fp16": (1, 8, 2, 2, 1500, 128, True, 0, 1),
    "all_fp16": (1, 4, 4, 4, 640, 128, True, 10000, 1),
    "short_cache": (1, 2, 1, 16, 40, 128, True, 5000, 1),
    "g32_one_token": (1, 32, 1, 1, 3000, 128, True, 500, 1),
    "nv_one_token_gqa4": (2, 8, 2, 1, 2048, 128, True, 500, 0),
    "nv_rows5_ragged": (1, 4, 1, 5, 1000, 128, True, 1000, 0),
    "nv_d64_noncausal": (1, 4, 2, 3, 777, 64, False, 2500, 0),
    "nv_no_fp16": (1, 8, 2, 2, 1500, 128, True, 0, 0),
    "nv_g32_one_token": (1, 32, 1, 1, 3000, 128, True, 500, 0),
    "nv_long_cache": (1, 8, 2, 1, 8192, 128, True, 500, 0),
    # more than 32 query columns per key head: one workgroup per 32-column group
    "rows8_gqa8": (1, 16, 2, 8, 2048, 128, True, 500, 1),  # 64 columns
    "g16_rows8": (1, 16, 1, 8, 1500, 128, True, 1000, 1),  # 128 columns
    "d64_g6_rows9": (1, 12, 2, 9, 777, 64, False, 2500, 1),  # 54: a ragged last group
    "nv_rows8_gqa8": (1, 16, 2, 8, 2048, 128, True, 500, 0),
    "nv_g4_rows32": (1, 8, 2, 32, 1200, 128, True, 1000, 0),  # 128 columns of 32 rows per head
}


def _run(oracle, w, bp, fmt=1):
    import torch

    from fp16_attention_amd import api

    d = W.generate(w)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(np.ascontiguousarray(d[n])).to(dev) for n in ("q", "k", "v"))
    idx, cnt = api.thrift_select_blocks(q, k, 128, 64, w.causal, -1, bp)
    q4 = api.thrift_quantize_fp4(q, api.THRIFT_GROUP_D, fmt)
    k4 = api.thrift_quantize_fp4(k, api.THRIFT_GROUP_D, fmt)
    v4 = api.thrift_quantize_fp4(v, api.THRIFT_GROUP_S, fmt)
    o, lse = api.thrift_attention_decode(q, k, v, q4, k4, v4, idx, cnt, 64, w.causal, out_fp32=True,
                                         with_lse=True)
    torch.cuda.synchronize()
    r = oracle.pipeline(d["q"], d["k"], d["v"], fmt, 128, 64, w.causal, -1, bp)
    g_cnt, g_idx = cnt.cpu().numpy(), idx.cpu().numpy()
    assert np.array_equal(g_cnt, r["cnt"]), "cnt differs"
    km = r["idx"].shape[-1]
    assert np.array_equal(g_idx[..., :km], r["idx"]), "idx differs"
    assert np.all(g_idx[..., km:] == -1)
    same_fp4(q4, r["q4"])
    same_fp4(k4, r["k4"])
    same_fp4(v4, r["v4"])
    compare_out(o.cpu().numpy().astype(np.float64), r["o"], lse.cpu().numpy().astype(np.float64),
                r["lse"], r["amb"])
    return o, r


@pytest.mark.parametrize("name", list(CASES))
def test_decode_parity(oracle, name):
    B, Hq, Hkv, Sq, Sk, D, causal, bp, fmt = CASES[name]
    w = W.WORKLOADS["decode"].with_(B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, S=Sk, D=D, causal=causal, topk_bp=bp,
                                    seed=len(name))
    note(f"[decode] {name}: B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} D{D} causal{int(causal)} bp{bp} fmt{fmt}")
    _run(oracle, w, bp, fmt)


def test_decode_fp16_output_matches_fp32(oracle):
    import torch

    from fp16_attention_amd import api

    w = W.WORKLOADS["decode"].with_(B=1, Hq=8, Hkv=2, Sq=2, S=1100, seed=11)
    d = W.generate(w)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(np.ascontiguousarray(d[n])).to(dev) for n in ("q", "k", "v"))
    k4 = api.thrift_quantize_fp4(k, api.THRIFT_GROUP_D, api.THRIFT_MXFP4)
    v4 = api.thrift_quantize_fp4(v, api.THRIFT_GROUP_S, api.THRIFT_MXFP4)
    o32 = api.thrift_decode(q, k, v, k4, v4, out_fp32=True)
    o16 = api.thrift_decode(q, k, v, k4, v4)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o16.cpu().numpy(), o32.cpu().numpy().astype(np.float16))


@pytest.mark.slow
def test_decode_full_size(oracle):
    w = W.WORKLOADS["decode"]
    note(f"[decode] full size: B{w.B} Hq{w.Hq} Hkv{w.Hkv} Sq{w.Sq} Sk{w.S} D{w.D} bp{w.topk_bp}")
    _run(oracle, w, w.topk_bp)


@pytest.mark.parametrize("fmt", [1, 0])
def test_cache_maintenance_matches_oracle(oracle, fmt):
    """Key-block means kept beside the cache and range re-encoding of its
    FP4 copy: bit-identical to the oracle's means and codes of the cache as
    it is after new tokens are written, with blocks and groups outside the
    updated range untouched; selection from the kept means equals selection
    from the fp16 keys.  NVFP4 keeps its slice scales: the new tokens are
    drawn from the slice's own rows, so its maximum does not change."""
    import torch

    from fp16_attention_amd import api

    w = W.WORKLOADS["decode"].with_(B=2, Hq=8, Hkv=2, Sq=3, S=1000, seed=21)
    d = W.generate(w)
    note(f"[decode] cache maintenance: B{w.B} Hq{w.Hq} Hkv{w.Hkv} Sq{w.Sq} Sk{w.S} fmt{fmt}")
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(np.ascontiguousarray(d[n])).to(dev) for n in ("q", "k", "v"))
    kbar = api.thrift_block_means(k, 64)
    k4 = api.thrift_quantize_fp4(k, api.THRIFT_GROUP_D, fmt)
    v4 = api.thrift_quantize_fp4(v, api.THRIFT_GROUP_S, fmt)
    torch.cuda.synchronize()
    assert np.array_equal(kbar.cpu().numpy(), oracle.block_means(d["k"], 64))
    # new tokens at positions 990..999 (the last key block, two V tiles' worth of groups)
    s0, s1 = 990, 1000
    rng = np.random.default_rng(5)
    knew, vnew = d["k"].copy(), d["v"].copy()
    src = rng.integers(0, s0, size=s1 - s0)
    knew[:, :, s0:s1] = d["k"][:, :, src][:, :, ::-1] * np.float16(0.5)
    vnew[:, :, s0:s1] = d["v"][:, :, src] * np.float16(-0.5)
    if fmt == 0:  # the premise of keeping the slice scales
        for old, new, ax in ((d["k"], knew, oracle.AXIS_D), (d["v"], vnew, oracle.AXIS_S)):
            assert np.array_equal(oracle.quantize(old, ax, 0).tensor_scale, oracle.quantize(new, ax, 0).tensor_scale)
    k.copy_(torch.from_numpy(knew))
    v.copy_(torch.from_numpy(vnew))
    before = kbar.clone(), k4.codes.clone(), k4.scales.clone(), v4.codes.clone(), v4.scales.clone()
    # the one-launch update on copies, against the three separate calls below
    copies = (kbar.clone(), api.FP4Tensor(k4.codes.clone(), k4.scales.clone(), k4.tensor_scale, k4.fmt, k4.axis),
              api.FP4Tensor(v4.codes.clone(), v4.scales.clone(), v4.tensor_scale, v4.fmt, v4.axis))
    api.thrift_cache_update(k, v, *copies, s0, s1)
    api.thrift_block_means(k, 64, s0 // 64, -(-s1 // 64), out=kbar)
    api.thrift_quantize_fp4_range(k, k4, s0, s1)
    api.thrift_quantize_fp4_range(v, v4, s0, s1)
    torch.cuda.synchronize()
    assert torch.equal(copies[0], kbar)
    assert torch.equal(copies[1].codes, k4.codes) and torch.equal(copies[1].scales, k4.scales)
    assert torch.equal(copies[2].codes, v4.codes) and torch.equal(copies[2].scales, v4.scales)
    assert np.array_equal(kbar.cpu().numpy(), oracle.block_means(knew, 64))
    assert torch.equal(kbar[:, :, : s0 // 64], before[0][:, :, : s0 // 64])
    same_fp4(k4, oracle.quantize(knew, oracle.AXIS_D, fmt))
    same_fp4(v4, oracle.quantize(vnew, oracle.AXIS_S, fmt))
    assert torch.equal(k4.codes[:, :, :s0], before[1][:, :, :s0])
    assert torch.equal(k4.scales[:, :, :s0], before[2][:, :, :s0])
    t0 = s0 // 128 * 2  # V: key blocks of 64 before the first re-encoded 128-position tile
    assert torch.equal(v4.codes[:, :, :t0], before[3][:, :, :t0])
    assert torch.equal(v4.scales[:, :, :t0], before[4][:, :, :t0])
    idx_a, cnt_a = api.thrift_select_blocks_kbar(q, kbar, w.S, 128, 64, True, -1, 1000)
    idx_b, cnt_b = api.thrift_select_blocks(q, k, 128, 64, True, -1, 1000)
    torch.cuda.synchronize()
    assert torch.equal(cnt_a, cnt_b) and torch.equal(idx_a, idx_b)
    ridx, rcnt, _ = oracle.select(d["q"], knew, 128, 64, True, -1, 1000)
    assert np.array_equal(cnt_a.cpu().numpy(), rcnt)
    assert np.array_equal(idx_a.cpu().numpy()[..., : ridx.shape[-1]], ridx)


def test_decode_nvfp4_rejects_a_promoted_table_beyond_its_lds():
    """64 query heads on one key head against a 262144-key cache: the NVFP4
    split kernel's promoted-block table (64 heads x 128 words) does not fit
    beside its four fp16 stages, so the call returns THRIFT_EUNSUPPORTED and
    launches nothing; MXFP4 (smaller stages) takes the same shape.  Every
    buffer is real and sized for the shape."""
    import torch

    from fp16_attention_amd import _lib, api

    dev = torch.device("cuda:0")
    Hq, Hkv, Sq, Sk, D = 64, 1, 1, 262144, 128
    note(f"[decode] lds budget: Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} D{D}")
    g = torch.Generator(device="cpu").manual_seed(5)
    q = torch.randn((1, Hq, Sq, D), generator=g).to(torch.float16).to(dev)
    k = torch.randn((1, Hkv, Sk, D), generator=g).to(torch.float16).to(dev)
    v = torch.randn((1, Hkv, Sk, D), generator=g).to(torch.float16).to(dev)
    idx, cnt = api.thrift_select_blocks(q, k, 128, 64, True, -1, 500)
    for fmt in (api.THRIFT_NVFP4, api.THRIFT_MXFP4):
        q4 = api.thrift_quantize_fp4(q, api.THRIFT_GROUP_D, fmt)
        k4 = api.thrift_quantize_fp4(k, api.THRIFT_GROUP_D, fmt)
        v4 = api.thrift_quantize_fp4(v, api.THRIFT_GROUP_S, fmt)
        if fmt == api.THRIFT_NVFP4:
            with pytest.raises(_lib.ThriftError) as e:
                api.thrift_attention_decode(q, k, v, q4, k4, v4, idx, cnt, 64, True, out_fp32=True)
            assert e.value.status == _lib.THRIFT_EUNSUPPORTED
        else:
            o = api.thrift_attention_decode(q, k, v, q4, k4, v4, idx, cnt, 64, True, out_fp32=True)
            torch.cuda.synchronize()
            assert torch.isfinite(o).all()
