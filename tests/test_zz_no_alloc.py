"""The allocation-free decode entry point (thrift_attention_decode_noalloc,
for callers that cannot allocate: its split partials live in the library's
static per-GPU array) against thrift_attention_decode with a caller
workspace, through the C ABI: two calls in a row, the second on a smaller
input, in both FP4 formats.  The two run the same kernels on the same split,
so their outputs and LSE must be identical bit for bit; a shape whose
partials exceed the array is rejected."""
import numpy as np
import pytest

from fp16_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Sq, Sk, D, causal, topk_bp): calls in a row on the shared array, each
# later one smaller than the one before (the first with 64 query columns per key
# head, two 32-column groups)
CALLS = [(2, 16, 2, 8, 3000, 128, True, 500), (2, 16, 4, 4, 2500, 128, True, 500),
         (1, 4, 2, 1, 700, 64, True, 1000)]


def _inputs(dev, fmt, B, Hq, Hkv, Sq, Sk, D, causal, bp, seed):
    import torch

    from fp16_attention_amd import api

    w = W.WORKLOADS["decode"].with_(B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, S=Sk, D=D, causal=causal, topk_bp=bp, seed=seed)
    d = W.generate(w)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(d[n])).to(dev) for n in ("q", "k", "v"))
    idx, cnt = api.thrift_select_blocks(q, k, 128, 64, causal, -1, bp)
    q4 = api.thrift_quantize_fp4(q, api.THRIFT_GROUP_D, fmt)
    k4 = api.thrift_quantize_fp4(k, api.THRIFT_GROUP_D, fmt)
    v4 = api.thrift_quantize_fp4(v, api.THRIFT_GROUP_S, fmt)
    return q, k, v, q4, k4, v4, idx, cnt


@pytest.mark.parametrize("fmt", [1, 0])
def test_noalloc_decode_matches_workspace_decode(fmt):
    import torch

    from fp16_attention_amd import _lib, api

    dev = torch.device("cuda:0")
    for n, (B, Hq, Hkv, Sq, Sk, D, causal, bp) in enumerate(CALLS):
        print(f"noalloc call {n}: B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} D{D} fmt {fmt}", flush=True)
        q, k, v, q4, k4, v4, idx, cnt = _inputs(dev, fmt, B, Hq, Hkv, Sq, Sk, D, causal, bp, 11 + n)
        o_ref, lse_ref = api.thrift_attention_decode(q, k, v, q4, k4, v4, idx, cnt, 64, causal, out_fp32=True,
                                                     with_lse=True)
        out = torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.float32, device=dev)
        lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
        api.thrift_attention_decode_noalloc(q, k, v, q4, k4, v4, idx, cnt, 64, causal, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), (n, (out - o_ref).abs().max().item())
        assert torch.equal(lse, lse_ref), (n, (lse - lse_ref).abs().max().item())
        assert _lib.load().thrift_attention_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, idx.shape[-1]) <= 16 << 20


def test_noalloc_decode_rejects_shapes_beyond_its_array():
    import torch

    from fp16_attention_amd import _lib, api

    dev = torch.device("cuda:0")
    # 16 sequences x 64 heads, every one of the 32 key blocks promotable: the
    # split partials need more than 16 MiB
    B, Hq, Hkv, Sq, Sk, D, kmax = 16, 64, 64, 1, 2048, 128, 32
    assert _lib.load().thrift_attention_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, kmax) > 16 << 20
    q = torch.zeros((B, Hq, Sq, D), dtype=torch.float16, device=dev)
    k = torch.zeros((B, Hkv, Sk, D), dtype=torch.float16, device=dev)
    q4 = api.thrift_quantize_fp4(q, api.THRIFT_GROUP_D, api.THRIFT_MXFP4)
    k4 = api.thrift_quantize_fp4(k, api.THRIFT_GROUP_D, api.THRIFT_MXFP4)
    v4 = api.thrift_quantize_fp4(k, api.THRIFT_GROUP_S, api.THRIFT_MXFP4)
    idx = torch.full((B, Hq, 1, kmax), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros((B, Hq, 1), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, Sq, D), dtype=torch.float32, device=dev)
    with pytest.raises(api.ThriftError) as e:
        api.thrift_attention_decode_noalloc(q, k, k, q4, k4, v4, idx, cnt, 64, True, out=out)
    assert e.value.status == _lib.THRIFT_EWORKSPACE
