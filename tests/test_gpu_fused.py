"""GPU parity of the one-pass block means + FP4 quantisation
(thrift_quantize_fp4_means) and of selection from precomputed means
(thrift_select_blocks_means), through the C ABI.

Bit-exact throughout: the means against the oracle's block means, codes,
block scales and slice scales against the oracle's quantisation, and both
against the library's separate entry points; selection from the means
against selection from the fp16 tensors and against the oracle.  Sizes span
ragged tails, a sequence shorter than one block, both head dimensions, both
block sizes and both formats.
"""
import numpy as np
import pytest

from tests.gpu_harness import note, same_fp4

pytestmark = pytest.mark.gpu

CASES = {
    # name: (B, H, S, D, blk, fmt)
    "mx_d128_b128_ragged": (1, 3, 1000, 128, 128, 1),
    "mx_d64_b64_ragged": (2, 2, 777, 64, 64, 1),
    "mx_short": (1, 1, 37, 128, 128, 1),
    "nv_d128_b64": (1, 4, 1000, 128, 64, 0),
    "nv_d64_b128": (1, 2, 513, 64, 128, 0),
}


def _tensor(shape, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=shape) * 0.5 * rng.lognormal(0, 1, size=(1, shape[1], 1, shape[3]))
    x[:, :, :, 5] *= 20  # an outlier channel
    return x.astype(np.float16)


@pytest.mark.parametrize("name", list(CASES))
def test_means_and_codes_in_one_pass(oracle, name):
    import torch

    from fp16_attention_amd import api

    B, H, S, D, blk, fmt = CASES[name]
    note(f"[fused] {name}: B{B} H{H} S{S} D{D} blk{blk} fmt{fmt}")
    x = _tensor((B, H, S, D), len(name))
    xd = torch.from_numpy(x).to("cuda:0")
    t4, means = api.thrift_quantize_fp4_means(xd, fmt, blk)
    sep4 = api.thrift_quantize_fp4(xd, api.THRIFT_GROUP_D, fmt)
    sepm = api.thrift_block_means(xd, blk)
    torch.cuda.synchronize()
    assert np.array_equal(means.cpu().numpy(), oracle.block_means(x, blk))
    assert torch.equal(means, sepm)
    same_fp4(t4, oracle.quantize(x, oracle.AXIS_D, fmt))
    assert torch.equal(t4.codes, sep4.codes) and torch.equal(t4.scales, sep4.scales)
    if fmt == 0:
        assert torch.equal(t4.tensor_scale, sep4.tensor_scale)


@pytest.mark.parametrize("Sq,Sk,causal", [(1000, 1000, True), (1000, 1000, False), (5, 1300, True)])
def test_select_from_means(oracle, Sq, Sk, causal):
    import torch

    from fp16_attention_amd import api

    note(f"[fused] select from means: Sq{Sq} Sk{Sk} causal{int(causal)}")
    q = _tensor((1, 8, Sq, 128), 1)
    k = _tensor((1, 2, Sk, 128), 2)
    qd, kd = torch.from_numpy(q).to("cuda:0"), torch.from_numpy(k).to("cuda:0")
    _, qbar = api.thrift_quantize_fp4_means(qd, 1, 128)
    _, kbar = api.thrift_quantize_fp4_means(kd, 1, 64)
    idx_a, cnt_a = api.thrift_select_blocks_means(qbar, kbar, Sq, Sk, 128, 64, causal, -1, 1500)
    idx_b, cnt_b = api.thrift_select_blocks(qd, kd, 128, 64, causal, -1, 1500)
    torch.cuda.synchronize()
    assert torch.equal(cnt_a, cnt_b) and torch.equal(idx_a, idx_b)
    ridx, rcnt, _ = oracle.select(q, k, 128, 64, causal, -1, 1500)
    assert np.array_equal(cnt_a.cpu().numpy(), rcnt)
    assert np.array_equal(idx_a.cpu().numpy()[..., : ridx.shape[-1]], ridx)


@pytest.mark.parametrize("S,causal", [(8300, True), (40000, True), (40000, False)])
def test_select_query_block_runs(oracle, S, causal):
    """Selection when several query blocks share a workgroup: a ragged last
    run (65 query blocks in runs of four) and runs of two (625 key blocks)."""
    import torch

    from fp16_attention_amd import api

    note(f"[fused] select, query-block runs: S{S} causal{int(causal)}")
    q = _tensor((1, 4, S, 64), 3)
    k = _tensor((1, 1, S, 64), 4)
    qd, kd = torch.from_numpy(q).to("cuda:0"), torch.from_numpy(k).to("cuda:0")
    idx, cnt = api.thrift_select_blocks(qd, kd, 128, 64, causal, -1, 300)
    torch.cuda.synchronize()
    ridx, rcnt, _ = oracle.select(q, k, 128, 64, causal, -1, 300)
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(idx.cpu().numpy()[..., : ridx.shape[-1]], ridx)
