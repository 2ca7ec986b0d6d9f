"""Python binding of the C ABI: torch tensors in, the same three calls out.

Marshalling only: each function checks dtypes, devices and contiguity,
allocates outputs and workspace with torch, passes raw device pointers and
torch's current HIP stream to libthrift.so, and raises ThriftError on a
non-zero status.  All arithmetic runs in the library's kernels.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import THRIFT_GROUP_D, THRIFT_GROUP_S, THRIFT_MXFP4, THRIFT_NVFP4, THRIFT_NVFP4_MXP, ThriftError

__all__ = ["thrift_select_kmax", "thrift_select_blocks", "thrift_block_means",
           "thrift_select_blocks_kbar", "thrift_select_blocks_means", "thrift_select_blocks_head",
           "thrift_quantize_fp4",
           "thrift_quantize_fp4_means", "thrift_quantize_fp4_range", "thrift_cache_update",
           "thrift_attention_fwd", "thrift_attention_decode", "thrift_attention_decode_noalloc",
           "thrift_decode", "FP4Tensor",
           "fp4_transposed", "thrift_forward", "thrift_attention_bwd_workspace", "thrift_attention_fwd_hp",
           "thrift_attention_bwd", "THRIFT_NVFP4", "THRIFT_MXFP4", "THRIFT_NVFP4_MXP", "THRIFT_GROUP_D",
           "THRIFT_GROUP_S", "ThriftError", "FP8Tensor", "thrift_quantize_fp8", "thrift_attention_fwd_tiered",
           "thrift_forward_tiered"]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(t, dtype, name):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous {dtype} CUDA tensor")


def _call(fn, *args):
    st = getattr(_lib.load(), fn)(*args)
    if st != _lib.THRIFT_OK:
        raise ThriftError(fn, st)


def thrift_select_kmax(S, block_q, block_k, causal, topk_count, topk_bp, Sk=None) -> int:
    """Largest per-query-block budget; Sk (default S) keys for S queries at their end."""
    return _lib.load().thrift_select_kmax_kv(S, S if Sk is None else Sk, block_q, block_k, int(causal),
                                             topk_count, topk_bp)


def thrift_select_blocks(q16, k16, block_q=128, block_k=64, causal=True, topk_count=-1,
                         topk_bp=500, kmax=None):
    """Block means, pair scores and per-query-block top-k.  Returns (idx, cnt).
    k16 may hold more positions than q16: the queries are then its last ones."""
    _check(q16, torch.float16, "q16")
    _check(k16, torch.float16, "k16")
    B, Hq, S, D = q16.shape
    Hkv, Sk = k16.shape[1], k16.shape[2]
    if kmax is None:
        kmax = max(1, thrift_select_kmax(S, block_q, block_k, causal, topk_count, topk_bp, Sk))
    nq = -(-S // block_q)
    dev = q16.device
    idx = torch.empty((B, Hq, nq, kmax), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hq, nq), dtype=torch.int32, device=dev)
    wsb = _lib.load().thrift_select_workspace_bytes_kv(B, Hq, Hkv, S, Sk, D, block_q, block_k)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    _call("thrift_select_blocks_kv", _ptr(q16), _ptr(k16), B, Hq, Hkv, S, Sk, D, block_q, block_k,
          int(causal), topk_count, topk_bp, _ptr(idx), _ptr(cnt), kmax, _ptr(ws), wsb, _stream())
    return idx, cnt


def thrift_block_means(x16, blk=64, j0=0, j1=None, out=None):
    """fp32 means [B,H,ceil(S/blk),D] of the blocks of x16; with out given,
    only blocks j0 <= j < j1 of it are rewritten (a cache's last block after
    new keys)."""
    _check(x16, torch.float16, "x16")
    B, H, S, D = x16.shape
    nb = -(-S // blk)
    if out is None:
        out = torch.empty((B, H, nb, D), dtype=torch.float32, device=x16.device)
    _check(out, torch.float32, "out")
    if tuple(out.shape) != (B, H, nb, D):
        raise ValueError(f"out must have shape {(B, H, nb, D)}")
    _call("thrift_block_means", _ptr(x16), B, H, S, D, blk, j0, nb if j1 is None else j1, _ptr(out),
          _stream())
    return out


def thrift_select_blocks_kbar(q16, kbar, Sk, block_q=128, block_k=64, causal=True, topk_count=-1,
                              topk_bp=500, kmax=None):
    """thrift_select_blocks against Sk keys given by their block means kbar
    [B,Hkv,ceil(Sk/block_k),D] (thrift_block_means).  Returns (idx, cnt)."""
    _check(q16, torch.float16, "q16")
    _check(kbar, torch.float32, "kbar")
    B, Hq, S, D = q16.shape
    Hkv = kbar.shape[1]
    if tuple(kbar.shape) != (B, Hkv, -(-Sk // block_k), D):
        raise ValueError("kbar must be [B, Hkv, ceil(Sk/block_k), D]")
    if kmax is None:
        kmax = max(1, thrift_select_kmax(S, block_q, block_k, causal, topk_count, topk_bp, Sk))
    nq = -(-S // block_q)
    dev = q16.device
    idx = torch.empty((B, Hq, nq, kmax), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hq, nq), dtype=torch.int32, device=dev)
    wsb = B * Hq * nq * D * 4
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _call("thrift_select_blocks_kbar", _ptr(q16), _ptr(kbar), B, Hq, Hkv, S, Sk, D, block_q, block_k,
          int(causal), topk_count, topk_bp, _ptr(idx), _ptr(cnt), kmax, _ptr(ws), wsb, _stream())
    return idx, cnt


def thrift_select_blocks_means(qbar, kbar, Sq, Sk, block_q=128, block_k=64, causal=True, topk_count=-1,
                               topk_bp=500, kmax=None):
    """Selection from block means computed beforehand: qbar [B,Hq,ceil(Sq/block_q),D],
    kbar [B,Hkv,ceil(Sk/block_k),D] (thrift_quantize_fp4_means, thrift_block_means)."""
    _check(qbar, torch.float32, "qbar")
    _check(kbar, torch.float32, "kbar")
    B, Hq, nq, D = qbar.shape
    Hkv = kbar.shape[1]
    if nq != -(-Sq // block_q) or tuple(kbar.shape) != (B, Hkv, -(-Sk // block_k), D):
        raise ValueError("qbar / kbar do not match Sq, Sk and the block sizes")
    if kmax is None:
        kmax = max(1, thrift_select_kmax(Sq, block_q, block_k, causal, topk_count, topk_bp, Sk))
    dev = qbar.device
    idx = torch.empty((B, Hq, nq, kmax), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hq, nq), dtype=torch.int32, device=dev)
    _call("thrift_select_blocks_means", _ptr(qbar), _ptr(kbar), B, Hq, Hkv, Sq, Sk, D, block_q, block_k,
          int(causal), topk_count, topk_bp, _ptr(idx), _ptr(cnt), kmax, _stream())
    return idx, cnt


def thrift_select_blocks_head(qbar, kbar, Sq, Sk, block_q=128, block_k=64, causal=True, topk_count=-1,
                              topk_bp=500, kmax=None):
    """Per-head budget: one top-k over all valid block pairs of each query
    head, from block means as thrift_select_blocks_means takes them."""
    _check(qbar, torch.float32, "qbar")
    _check(kbar, torch.float32, "kbar")
    B, Hq, nq, D = qbar.shape
    Hkv = kbar.shape[1]
    if nq != -(-Sq // block_q) or tuple(kbar.shape) != (B, Hkv, -(-Sk // block_k), D):
        raise ValueError("qbar / kbar do not match Sq, Sk and the block sizes")
    L = _lib.load()
    if kmax is None:
        kmax = L.thrift_select_head_kmax(Sq, Sk, block_q, block_k, int(causal))
    dev = qbar.device
    idx = torch.empty((B, Hq, nq, kmax), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hq, nq), dtype=torch.int32, device=dev)
    wsb = L.thrift_select_head_workspace_bytes(B, Hq, Sq, Sk, block_q, block_k)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _call("thrift_select_blocks_head", _ptr(qbar), _ptr(kbar), B, Hq, Hkv, Sq, Sk, D, block_q, block_k,
          int(causal), topk_count, topk_bp, _ptr(idx), _ptr(cnt), kmax, _ptr(ws), wsb, _stream())
    return idx, cnt


@dataclass
class FP4Tensor:
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor | None
    fmt: int
    axis: int


def thrift_quantize_fp4(x16, axis=THRIFT_GROUP_D, fmt=THRIFT_MXFP4) -> FP4Tensor:
    """FP16 -> E2M1 codes + block scales (+ per-slice fp32 scale for NVFP4)."""
    _check(x16, torch.float16, "x16")
    B, H, S, D = x16.shape
    g = 16 if fmt == THRIFT_NVFP4 else 32
    dev = x16.device
    if axis == THRIFT_GROUP_D:
        codes = torch.empty((B, H, S, D // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, H, S, D // g), dtype=torch.uint8, device=dev)
    else:
        Sp = -(-S // 64) * 64  # key-block-major V^T: [B, H, Sp/64, D, ...]
        codes = torch.empty((B, H, Sp // 64, D, 32), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, H, Sp // 64, D, 64 // g), dtype=torch.uint8, device=dev)
    ts = torch.empty((B, H), dtype=torch.float32, device=dev) if fmt == THRIFT_NVFP4 else None
    wsb = _lib.load().thrift_quantize_workspace_bytes(B, H, S, D, fmt)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    _call("thrift_quantize_fp4", _ptr(x16), B, H, S, D, axis, fmt, _ptr(codes), _ptr(scales),
          _ptr(ts), _ptr(ws), wsb, _stream())
    return FP4Tensor(codes, scales, ts, fmt, axis)


def thrift_quantize_fp4_means(x16, fmt=THRIFT_MXFP4, blk=128):
    """FP4 codes along D (as thrift_quantize_fp4 with THRIFT_GROUP_D) and the
    fp32 block means [B,H,ceil(S/blk),D] from one pass.  Returns (FP4Tensor, means)."""
    _check(x16, torch.float16, "x16")
    B, H, S, D = x16.shape
    g = 16 if fmt == THRIFT_NVFP4 else 32
    dev = x16.device
    codes = torch.empty((B, H, S, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((B, H, S, D // g), dtype=torch.uint8, device=dev)
    ts = torch.empty((B, H), dtype=torch.float32, device=dev) if fmt == THRIFT_NVFP4 else None
    means = torch.empty((B, H, -(-S // blk), D), dtype=torch.float32, device=dev)
    wsb = _lib.load().thrift_quantize_means_workspace_bytes(B, H, S, D, fmt, blk)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    _call("thrift_quantize_fp4_means", _ptr(x16), B, H, S, D, fmt, blk, _ptr(codes), _ptr(scales), _ptr(ts),
          _ptr(means), _ptr(ws), wsb, _stream())
    return FP4Tensor(codes, scales, ts, fmt, THRIFT_GROUP_D), means


def thrift_quantize_fp4_range(x16, t: FP4Tensor, s0, s1):
    """Re-encode, in place in t (an FP4 copy of x16), the groups that hold
    positions s0 <= s < s1 of x16 (NVFP4: under t's slice scales, kept)."""
    _check(x16, torch.float16, "x16")
    B, H, S, D = x16.shape
    _call("thrift_quantize_fp4_range", _ptr(x16), B, H, S, D, t.axis, t.fmt, s0, s1, _ptr(t.codes),
          _ptr(t.scales), _ptr(t.tensor_scale), _stream())
    return t


def thrift_cache_update(k16, v16, kbar, k4: FP4Tensor, v4: FP4Tensor, s0, s1, block_k=64):
    """After new tokens were written to positions s0..s1-1 of the fp16 cache
    (k16, v16): their key blocks' means into kbar, their K rows' and V tiles'
    FP4 codes into k4, v4 (in place), in one launch."""
    _check(k16, torch.float16, "k16")
    _check(v16, torch.float16, "v16")
    _check(kbar, torch.float32, "kbar")
    B, H, S, D = k16.shape
    _call("thrift_cache_update", _ptr(k16), _ptr(v16), B, H, S, D, block_k, s0, s1, k4.fmt, _ptr(kbar),
          _ptr(k4.codes), _ptr(k4.scales), _ptr(k4.tensor_scale), _ptr(v4.codes), _ptr(v4.scales),
          _ptr(v4.tensor_scale), _stream())
    return kbar, k4, v4


def fp4_transposed(t: FP4Tensor):
    """(codes, scales) of a THRIFT_GROUP_S tensor as plain transposed arrays
    [B,H,D,Sp/2] and [B,H,D,Sp/g] (copies; the stored order is key-block-major).
    THRIFT_GROUP_D tensors are returned as stored."""
    if t.axis != THRIFT_GROUP_S:
        return t.codes, t.scales
    B, H, nb, D, cb = t.codes.shape
    sb = t.scales.shape[-1]
    codes = t.codes.permute(0, 1, 3, 2, 4).reshape(B, H, D, nb * cb)
    scales = t.scales.permute(0, 1, 3, 2, 4).reshape(B, H, D, nb * sb)
    return codes, scales


def thrift_attention_fwd(q16, k16, v16, q4: FP4Tensor, k4: FP4Tensor, v4: FP4Tensor, idx, cnt,
                         block_q=128, block_k=64, causal=True, sm_scale=None, out_fp32=False,
                         with_lse=False, out=None, p_fmt=None):
    """Mixed FP4/FP16 forward.  Returns o (and lse if with_lse).  p_fmt=THRIFT_MXFP4
    with NVFP4 tensors quantises P MX-style (the THRIFT_NVFP4_MXP variant)."""
    B, Hq, S = q4.codes.shape[:3]
    D = q4.codes.shape[3] * 2
    Hkv = k4.codes.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    for name, t in (("q16", q16), ("k16", k16), ("v16", v16)):
        if t is not None:
            _check(t, torch.float16, name)
    _check(idx, torch.int32, "idx")
    _check(cnt, torch.int32, "cnt")
    dev = q4.codes.device
    if out is None:
        out = torch.empty((B, Hq, S, D), dtype=torch.float32 if out_fp32 else torch.float16, device=dev)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev) if with_lse else None
    _call("thrift_attention_fwd", _ptr(q16), _ptr(k16), _ptr(v16), _ptr(q4.codes),
          _ptr(q4.scales), _ptr(q4.tensor_scale), _ptr(k4.codes), _ptr(k4.scales),
          _ptr(k4.tensor_scale), _ptr(v4.codes), _ptr(v4.scales), _ptr(v4.tensor_scale),
          THRIFT_NVFP4_MXP if (q4.fmt == THRIFT_NVFP4 and p_fmt == THRIFT_MXFP4) else q4.fmt,
          _ptr(idx), _ptr(cnt), idx.shape[-1], B, Hq, Hkv, S, D, block_q, block_k, int(causal),
          float(sm_scale), _ptr(out), int(out.dtype == torch.float32), _ptr(lse), _stream())
    return (out, lse) if with_lse else out


@dataclass
class FP8Tensor:
    codes: torch.Tensor
    scales: torch.Tensor
    axis: int


def thrift_quantize_fp8(x16, axis=THRIFT_GROUP_D) -> FP8Tensor:
    """FP16 -> MXFP8 (E4M3 codes, E8M0 scale per 32) for the middle tier:
    along D codes [B,H,S,D] and scales [B,H,S,D/32]; along S (V) codes
    [B,H,D,Sp] and scales [B,H,D,Sp/32]."""
    _check(x16, torch.float16, "x16")
    B, H, S, D = x16.shape
    dev = x16.device
    if axis == THRIFT_GROUP_D:
        codes = torch.empty((B, H, S, D), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, H, S, D // 32), dtype=torch.uint8, device=dev)
    else:
        Sp = -(-S // 64) * 64
        codes = torch.empty((B, H, D, Sp), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, H, D, Sp // 32), dtype=torch.uint8, device=dev)
    _call("thrift_quantize_fp8", _ptr(x16), B, H, S, D, axis, _ptr(codes), _ptr(scales), _stream())
    return FP8Tensor(codes, scales, axis)


def thrift_attention_fwd_tiered(q16, k16, v16, q4: FP4Tensor, k4: FP4Tensor, v4: FP4Tensor, q8: FP8Tensor,
                                k8: FP8Tensor, v8: FP8Tensor, idx, cnt, idx2, cnt2, block_q=128, block_k=64,
                                causal=True, sm_scale=None, out_fp32=False, with_lse=False, out=None):
    """Three-tier forward (MX format): blocks idx lists in FP16, blocks idx2
    lists and idx does not in MXFP8, the rest in MXFP4."""
    B, Hq, S, D = q8.codes.shape
    Hkv = k8.codes.shape[1]
    if q4.fmt != THRIFT_MXFP4:
        raise ValueError("the middle tier is built for the MX format")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    for name, t in (("q16", q16), ("k16", k16), ("v16", v16)):
        if t is not None:
            _check(t, torch.float16, name)
    for name, t in (("idx", idx), ("cnt", cnt), ("idx2", idx2), ("cnt2", cnt2)):
        _check(t, torch.int32, name)
    dev = q8.codes.device
    if out is None:
        out = torch.empty((B, Hq, S, D), dtype=torch.float32 if out_fp32 else torch.float16, device=dev)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev) if with_lse else None
    _call("thrift_attention_fwd_tiered", _ptr(q16), _ptr(k16), _ptr(v16), _ptr(q4.codes), _ptr(q4.scales),
          _ptr(k4.codes), _ptr(k4.scales), _ptr(v4.codes), _ptr(v4.scales), _ptr(q8.codes), _ptr(q8.scales),
          _ptr(k8.codes), _ptr(k8.scales), _ptr(v8.codes), _ptr(v8.scales), _ptr(idx), _ptr(cnt),
          idx.shape[-1], _ptr(idx2), _ptr(cnt2), idx2.shape[-1], B, Hq, Hkv, S, D, block_q, block_k,
          int(causal), float(sm_scale), _ptr(out), int(out.dtype == torch.float32), _ptr(lse), _stream())
    return (out, lse) if with_lse else out


def thrift_attention_bwd_workspace(B, Hq, Hkv, S, D, block_q=128, device="cuda"):
    """Workspace tensor for thrift_attention_fwd_hp / thrift_attention_bwd."""
    n = _lib.load().thrift_attention_bwd_workspace_bytes(B, Hq, Hkv, S, D, block_q)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def thrift_attention_fwd_hp(q16, k16, v16, q4: FP4Tensor, k4: FP4Tensor, v4: FP4Tensor, idx, cnt, lse,
                            block_q=128, block_k=64, causal=True, sm_scale=None, workspace=None, out=None):
    """Attn-QAT's high-precision output O' (fp32 [B,Hq,S,D]): the forward with
    the exact softmax probabilities, from the forward's lse."""
    B, Hq, S, D = q16.shape
    Hkv = k16.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    for name, t in (("q16", q16), ("k16", k16), ("v16", v16)):
        _check(t, torch.float16, name)
    _check(idx, torch.int32, "idx")
    _check(cnt, torch.int32, "cnt")
    _check(lse, torch.float32, "lse")
    if workspace is None:
        workspace = thrift_attention_bwd_workspace(B, Hq, Hkv, S, D, block_q, q16.device)
    if out is None:
        out = torch.empty((B, Hq, S, D), dtype=torch.float32, device=q16.device)
    _call("thrift_attention_fwd_hp", _ptr(q16), _ptr(k16), _ptr(v16), _ptr(q4.codes), _ptr(q4.scales),
          _ptr(q4.tensor_scale), _ptr(k4.codes), _ptr(k4.scales), _ptr(k4.tensor_scale), _ptr(v4.codes),
          _ptr(v4.scales), _ptr(v4.tensor_scale), q4.fmt, _ptr(idx), _ptr(cnt),
          idx.shape[-1], B, Hq, Hkv, S, D, block_q, block_k, int(causal), float(sm_scale), _ptr(lse),
          _ptr(out), _ptr(workspace), workspace.numel(), _stream())
    return out


def thrift_attention_bwd(q16, k16, v16, q4: FP4Tensor, k4: FP4Tensor, v4: FP4Tensor, idx, cnt, lse, ohp,
                         do16, block_q=128, block_k=64, causal=True, sm_scale=None, workspace=None):
    """Attn-QAT backward: (dq fp32 [B,Hq,S,D], dk, dv fp32 [B,Hkv,S,D]) from the
    output gradient do16, the forward's lse and O'."""
    B, Hq, S, D = q16.shape
    Hkv = k16.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    for name, t in (("q16", q16), ("k16", k16), ("v16", v16), ("do16", do16)):
        _check(t, torch.float16, name)
    _check(idx, torch.int32, "idx")
    _check(cnt, torch.int32, "cnt")
    _check(lse, torch.float32, "lse")
    _check(ohp, torch.float32, "ohp")
    if workspace is None:
        workspace = thrift_attention_bwd_workspace(B, Hq, Hkv, S, D, block_q, q16.device)
    dev = q16.device
    dq = torch.empty((B, Hq, S, D), dtype=torch.float32, device=dev)
    dk = torch.empty((B, Hkv, S, D), dtype=torch.float32, device=dev)
    dv = torch.empty((B, Hkv, S, D), dtype=torch.float32, device=dev)
    _call("thrift_attention_bwd", _ptr(q16), _ptr(k16), _ptr(v16), _ptr(q4.codes), _ptr(q4.scales),
          _ptr(q4.tensor_scale), _ptr(k4.codes), _ptr(k4.scales), _ptr(k4.tensor_scale), _ptr(v4.codes),
          _ptr(v4.scales), _ptr(v4.tensor_scale), q4.fmt, _ptr(idx), _ptr(cnt),
          idx.shape[-1], B, Hq, Hkv, S, D, block_q, block_k, int(causal), float(sm_scale), _ptr(lse),
          _ptr(ohp), _ptr(do16), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _stream())
    return dq, dk, dv


def thrift_attention_decode(q16, k16, v16, q4: FP4Tensor, k4: FP4Tensor, v4: FP4Tensor, idx, cnt,
                            block_k=64, causal=True, sm_scale=None, out_fp32=False, with_lse=False,
                            out=None):
    """Decode-shaped forward: the Sq rows of q16 are the last positions of the
    Sk-key cache (k16, v16 and their FP4 copies).  Returns o (and lse)."""
    B, Hq, Sq, D = q16.shape
    Hkv, Sk = k16.shape[1], k16.shape[2]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    for name, t in (("q16", q16), ("k16", k16), ("v16", v16)):
        _check(t, torch.float16, name)
    _check(idx, torch.int32, "idx")
    _check(cnt, torch.int32, "cnt")
    dev = q16.device
    kmax = idx.shape[-1]
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=torch.float32 if out_fp32 else torch.float16, device=dev)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev) if with_lse else None
    wsb = _lib.load().thrift_attention_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, kmax)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    _call("thrift_attention_decode", _ptr(q16), _ptr(k16), _ptr(v16), _ptr(q4.codes),
          _ptr(q4.scales), _ptr(q4.tensor_scale), _ptr(k4.codes), _ptr(k4.scales),
          _ptr(k4.tensor_scale), _ptr(v4.codes), _ptr(v4.scales), _ptr(v4.tensor_scale), q4.fmt,
          _ptr(idx), _ptr(cnt), kmax, B, Hq, Hkv, Sq, Sk, D, block_k, int(causal), float(sm_scale),
          _ptr(out), int(out.dtype == torch.float32), _ptr(lse), _ptr(ws), wsb, _stream())
    return (out, lse) if with_lse else out


def thrift_attention_decode_noalloc(q16, k16, v16, q4: FP4Tensor, k4: FP4Tensor, v4: FP4Tensor, idx, cnt,
                                    block_k=64, causal=True, sm_scale=None, out=None, lse=None):
    """thrift_attention_decode without any device allocation inside the call:
    the split partials live in the library's static per-GPU array; the
    caller passes the output (and optional lse) tensors."""
    B, Hq, Sq, D = q16.shape
    Hkv, Sk = k16.shape[1], k16.shape[2]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    for name, t in (("q16", q16), ("k16", k16), ("v16", v16)):
        _check(t, torch.float16, name)
    _check(idx, torch.int32, "idx")
    _check(cnt, torch.int32, "cnt")
    if out is None or tuple(out.shape) != (B, Hq, Sq, D) or out.dtype not in (torch.float16, torch.float32):
        raise ValueError("out must be a [B, Hq, Sq, D] fp16 or fp32 tensor")
    if lse is not None:
        _check(lse, torch.float32, "lse")
    _call("thrift_attention_decode_noalloc", _ptr(q16), _ptr(k16), _ptr(v16), _ptr(q4.codes),
          _ptr(q4.scales), _ptr(q4.tensor_scale), _ptr(k4.codes), _ptr(k4.scales),
          _ptr(k4.tensor_scale), _ptr(v4.codes), _ptr(v4.scales), _ptr(v4.tensor_scale), q4.fmt,
          _ptr(idx), _ptr(cnt), idx.shape[-1], B, Hq, Hkv, Sq, Sk, D, block_k, int(causal), float(sm_scale),
          _ptr(out), int(out.dtype == torch.float32), _ptr(lse), _stream())
    return out


def thrift_decode(q16, k16, v16, k4: FP4Tensor, v4: FP4Tensor, fmt=THRIFT_MXFP4, block_q=128,
                  block_k=64, causal=True, topk_count=-1, topk_bp=500, sm_scale=None,
                  out_fp32=False, with_lse=False):
    """One decode step against a dual cache (fp16 k16/v16 and their FP4 k4/v4):
    selection, FP4 quantisation of the new queries, decode forward."""
    idx, cnt = thrift_select_blocks(q16, k16, block_q, block_k, causal, topk_count, topk_bp)
    q4 = thrift_quantize_fp4(q16, THRIFT_GROUP_D, fmt)
    return thrift_attention_decode(q16, k16, v16, q4, k4, v4, idx, cnt, block_k, causal, sm_scale,
                                   out_fp32, with_lse)


def thrift_forward(q16, k16, v16, fmt=THRIFT_MXFP4, block_q=128, block_k=64, causal=True,
                   topk_count=-1, topk_bp=500, sm_scale=None, out_fp32=False, with_lse=False,
                   budget="block"):
    """The whole path: Q and K each read once for their block means and FP4
    codes, V quantised, selection from the means (budget "block": per query
    block; "head": one budget over each query head's pairs), mixed attention."""
    q4, qbar = thrift_quantize_fp4_means(q16, fmt, block_q)
    k4, kbar = thrift_quantize_fp4_means(k16, fmt, block_k)
    v4 = thrift_quantize_fp4(v16, THRIFT_GROUP_S, fmt)
    sel = {"block": thrift_select_blocks_means, "head": thrift_select_blocks_head}[budget]
    idx, cnt = sel(qbar, kbar, q16.shape[2], k16.shape[2], block_q, block_k, causal, topk_count, topk_bp)
    return thrift_attention_fwd(q16, k16, v16, q4, k4, v4, idx, cnt, block_q, block_k, causal,
                                sm_scale, out_fp32, with_lse)


def thrift_forward_tiered(q16, k16, v16, block_q=128, block_k=64, causal=True, bp16=500, bp8=1000,
                          sm_scale=None, out_fp32=False, with_lse=False):
    """The three-tier path (MX format): block means and FP4 codes of Q and K
    in one pass, MXFP8 copies of Q, K and V, the selection from the means
    under bp16 (the FP16 tier) and under bp16 + bp8 (FP16 and FP8 tiers
    together), then the three-tier attention."""
    q4, qbar = thrift_quantize_fp4_means(q16, THRIFT_MXFP4, block_q)
    k4, kbar = thrift_quantize_fp4_means(k16, THRIFT_MXFP4, block_k)
    v4 = thrift_quantize_fp4(v16, THRIFT_GROUP_S, THRIFT_MXFP4)
    q8, k8 = thrift_quantize_fp8(q16, THRIFT_GROUP_D), thrift_quantize_fp8(k16, THRIFT_GROUP_D)
    v8 = thrift_quantize_fp8(v16, THRIFT_GROUP_S)
    Sq, Sk = q16.shape[2], k16.shape[2]
    idx, cnt = thrift_select_blocks_means(qbar, kbar, Sq, Sk, block_q, block_k, causal, -1, bp16)
    idx2, cnt2 = thrift_select_blocks_means(qbar, kbar, Sq, Sk, block_q, block_k, causal, -1, bp16 + bp8)
    return thrift_attention_fwd_tiered(q16, k16, v16, q4, k4, v4, q8, k8, v8, idx, cnt, idx2, cnt2, block_q,
                                       block_k, causal, sm_scale, out_fp32, with_lse)
