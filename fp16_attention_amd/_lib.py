"""ctypes declarations of libthrift.so (the C ABI in include/thrift.h)."""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libthrift.so")

THRIFT_OK, THRIFT_EINVAL, THRIFT_EUNSUPPORTED, THRIFT_EALIGN, THRIFT_EWORKSPACE, THRIFT_EHIP = range(6)
THRIFT_NVFP4, THRIFT_MXFP4, THRIFT_NVFP4_MXP = 0, 1, 2
THRIFT_GROUP_D, THRIFT_GROUP_S = 0, 1

EXPORTS = ("thrift_select_kmax", "thrift_select_workspace_bytes", "thrift_select_blocks",
           "thrift_select_kmax_kv", "thrift_select_workspace_bytes_kv", "thrift_select_blocks_kv",
           "thrift_block_means", "thrift_select_blocks_kbar", "thrift_select_blocks_means",
           "thrift_select_head_kmax", "thrift_select_head_workspace_bytes", "thrift_select_blocks_head",
           "thrift_quantize_means_workspace_bytes", "thrift_quantize_fp4_means",
           "thrift_quantize_workspace_bytes", "thrift_quantize_fp4", "thrift_quantize_fp4_range", "thrift_cache_update",
           "thrift_attention_fwd", "thrift_quantize_fp8", "thrift_attention_fwd_tiered",
           "thrift_attention_decode_workspace_bytes", "thrift_attention_decode",
           "thrift_attention_decode_noalloc",
           "thrift_attention_bwd_workspace_bytes", "thrift_attention_fwd_hp", "thrift_attention_bwd",
           "thrift_status_string")

_lib = None


class ThriftError(RuntimeError):
    def __init__(self, fn, status):
        msg = load().thrift_status_string(status).decode()
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


def load():
    """Load the built HIP library; fails loudly when it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                              "python -m fp16_attention_amd.build")
        L = C.CDLL(LIB_PATH)
        P, I, F, SZ = C.c_void_p, C.c_int, C.c_float, C.c_size_t
        L.thrift_select_kmax.restype = I
        L.thrift_select_kmax.argtypes = [I] * 6
        L.thrift_select_workspace_bytes.restype = SZ
        L.thrift_select_workspace_bytes.argtypes = [I] * 7
        L.thrift_select_blocks.restype = I
        L.thrift_select_blocks.argtypes = [P, P] + [I] * 10 + [P, P, I, P, SZ, P]
        L.thrift_select_kmax_kv.restype = I
        L.thrift_select_kmax_kv.argtypes = [I] * 7
        L.thrift_select_workspace_bytes_kv.restype = SZ
        L.thrift_select_workspace_bytes_kv.argtypes = [I] * 8
        L.thrift_select_blocks_kv.restype = I
        L.thrift_select_blocks_kv.argtypes = [P, P] + [I] * 11 + [P, P, I, P, SZ, P]
        L.thrift_block_means.restype = I
        L.thrift_block_means.argtypes = [P] + [I] * 7 + [P, P]
        L.thrift_select_blocks_kbar.restype = I
        L.thrift_select_blocks_kbar.argtypes = [P, P] + [I] * 11 + [P, P, I, P, SZ, P]
        L.thrift_select_blocks_means.restype = I
        L.thrift_select_blocks_means.argtypes = [P, P] + [I] * 11 + [P, P, I, P]
        L.thrift_quantize_means_workspace_bytes.restype = SZ
        L.thrift_quantize_means_workspace_bytes.argtypes = [I] * 6
        L.thrift_quantize_fp4_means.restype = I
        L.thrift_quantize_fp4_means.argtypes = [P] + [I] * 6 + [P, P, P, P, P, SZ, P]
        L.thrift_select_head_kmax.restype = I
        L.thrift_select_head_kmax.argtypes = [I] * 5
        L.thrift_select_head_workspace_bytes.restype = SZ
        L.thrift_select_head_workspace_bytes.argtypes = [I] * 6
        L.thrift_select_blocks_head.restype = I
        L.thrift_select_blocks_head.argtypes = [P, P] + [I] * 11 + [P, P, I, P, SZ, P]
        L.thrift_cache_update.restype = I
        L.thrift_cache_update.argtypes = [P, P] + [I] * 8 + [P] * 7 + [P]
        L.thrift_quantize_fp4_range.restype = I
        L.thrift_quantize_fp4_range.argtypes = [P] + [I] * 8 + [P, P, P, P]
        L.thrift_attention_decode_workspace_bytes.restype = SZ
        L.thrift_attention_decode_workspace_bytes.argtypes = [I] * 7
        L.thrift_attention_decode.restype = I
        L.thrift_attention_decode.argtypes = [P] * 12 + [I, P, P] + [I] * 9 + [F, P, I, P, P, SZ, P]
        L.thrift_attention_decode_noalloc.restype = I
        L.thrift_attention_decode_noalloc.argtypes = [P] * 12 + [I, P, P] + [I] * 9 + [F, P, I, P, P]
        L.thrift_quantize_workspace_bytes.restype = SZ
        L.thrift_quantize_workspace_bytes.argtypes = [I] * 5
        L.thrift_quantize_fp4.restype = I
        L.thrift_quantize_fp4.argtypes = [P, I, I, I, I, I, I, P, P, P, P, SZ, P]
        L.thrift_attention_fwd.restype = I
        L.thrift_attention_fwd.argtypes = [P] * 12 + [I, P, P] + [I] * 9 + [F, P, I, P, P]
        L.thrift_quantize_fp8.restype = I
        L.thrift_quantize_fp8.argtypes = [P, I, I, I, I, I, P, P, P]
        L.thrift_attention_fwd_tiered.restype = I
        L.thrift_attention_fwd_tiered.argtypes = [P] * 15 + [P, P, I, P, P, I] + [I] * 8 + [F, P, I, P, P]
        L.thrift_attention_bwd_workspace_bytes.restype = SZ
        L.thrift_attention_bwd_workspace_bytes.argtypes = [I] * 6
        L.thrift_attention_fwd_hp.restype = I
        L.thrift_attention_fwd_hp.argtypes = [P] * 12 + [I, P, P, I] + [I] * 8 + [F, P, P, P, SZ, P]
        L.thrift_attention_bwd.restype = I
        L.thrift_attention_bwd.argtypes = [P] * 12 + [I, P, P, I] + [I] * 8 + [F] + [P] * 7 + [SZ, P]
        L.thrift_status_string.restype = C.c_char_p
        L.thrift_status_string.argtypes = [I]
        _lib = L
    return _lib
