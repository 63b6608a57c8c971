"""Python binding of libselattn.so (selected-key / split-K flash attention, gfx950).

Argument marshalling only: every step of the attention runs in the HIP kernels
behind the C ABI declared in include/sel_attn.h.  PyTorch supplies device
memory and the stream.  There is no fallback: if the library is not built, or
a call is refused, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libselattn.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
F32, F16, BF16, I8, FP8 = 0, 1, 2, 3, 4
OP_DECODE, OP_PREFILL, OP_COMBINE = 1, 2, 3
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024     # SEL_ATTN_NOALLOC_SCRATCH_BYTES

_i32, _i64, _f32, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("n_stream", _i32), ("n_row", _i32), ("n_head_q", _i32), ("n_head_kv", _i32),
        ("head_dim", _i32), ("cap", _i32),
        ("q", _p), ("k", _p), ("v", _p), ("kv_dtype", _i32),
        ("kv_stride_stream", _i64), ("kv_stride_cell", _i64), ("kv_stride_head", _i64),
        ("k_scale", _p), ("v_scale", _p),
        ("sc_stride_stream", _i64), ("sc_stride_cell", _i64), ("sc_stride_head", _i64),
        ("kv_len", _p), ("causal", _i32), ("scale", _f32), ("softcap", _f32),
        ("alibi_slopes", _p), ("slice_len", _i32), ("n_slices_max", _i32),
        ("part_o", _p), ("part_ml", _p), ("dbg_visit", _p), ("tree_parent", _p),
    ]


class CombineArgs(ctypes.Structure):
    _fields_ = [
        ("n_stream", _i32), ("n_row", _i32), ("n_head_q", _i32), ("head_dim", _i32),
        ("n_slices_max", _i32), ("kv_len", _p), ("slice_len", _i32), ("cap", _i32),
        ("part_o", _p), ("part_ml", _p), ("out", _p), ("sinks", _p),
    ]


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("n_row", _i32), ("n_head_q", _i32), ("n_head_kv", _i32), ("head_dim", _i32),
        ("n_kv", _i32), ("q", _p), ("k", _p), ("v", _p), ("kv_dtype", _i32),
        ("kv_stride_cell", _i64), ("kv_stride_head", _i64),
        ("k_scale", _p), ("v_scale", _p), ("sc_stride_cell", _i64), ("sc_stride_head", _i64),
        ("q_pos", _p), ("scale", _f32), ("softcap", _f32), ("alibi_slopes", _p),
        ("sel", _p), ("n_sel", _i32), ("block_size", _i32),
        ("mask", _p), ("mask_stride_row", _i64), ("mask_stride_head", _i64), ("causal", _i32),
        ("n_splits", _i32), ("out", _p), ("part_o", _p), ("part_ml", _p),
        ("dbg_visit", _p), ("dbg_sel", _p), ("sinks", _p),
    ]


class SelAttnError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: status {status} ({strerror(status)})")


_lib = None


def load(path):
    """Load a build of the library from `path` with the entry points typed as
    below (lib() uses it for the in-tree build)."""
    L = ctypes.CDLL(path)
    for name, argt in (("sel_attn_decode", [ctypes.POINTER(DecodeArgs), _p]),
                       ("sel_attn_split_combine", [ctypes.POINTER(CombineArgs), _p]),
                       ("sel_attn_prefill", [ctypes.POINTER(PrefillArgs), _p]),
                       ("sel_attn_supports", [ctypes.c_int, _p]),
                       ("sel_attn_decode_workspace",
                        [ctypes.POINTER(DecodeArgs), ctypes.POINTER(ctypes.c_size_t),
                         ctypes.POINTER(ctypes.c_size_t)]),
                       ("sel_attn_decode_path", [ctypes.POINTER(DecodeArgs)]),
                       ("sel_attn_decode_noalloc", [ctypes.POINTER(DecodeArgs), _p, _p, _p]),
                       ("sel_attn_prefill_path", [ctypes.POINTER(PrefillArgs)]),
                       ("sel_attn_abi_version", []),
                       ("sel_attn_args_size", [ctypes.c_int]),
                       ("sel_attn_strerror", [ctypes.c_int])):
        fn = getattr(L, name)
        fn.argtypes = argt
        fn.restype = ctypes.c_int
    L.sel_attn_strerror.restype = ctypes.c_char_p
    L.sel_attn_args_size.restype = ctypes.c_size_t
    for op, cls in ((OP_DECODE, DecodeArgs), (OP_PREFILL, PrefillArgs), (OP_COMBINE, CombineArgs)):
        if L.sel_attn_args_size(op) != ctypes.sizeof(cls):
            raise ImportError(f"argument struct mismatch for op {op}")
    return L


def lib():
    """Load libselattn.so (built in-tree by build.build()); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m split_flash_attention_amd.build`")
        _lib = load(LIB_PATH)
    return _lib


def strerror(status: int) -> str:
    return lib().sel_attn_strerror(int(status)).decode()


def _check(status, what):
    if status != OK:
        raise SelAttnError(status, what)


# ----------------------------------------------------------------------------
# torch tensor marshalling
# ----------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def kv_dtype_code(t) -> int:
    import torch
    m = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.int8: I8,
         torch.uint8: FP8, torch.float8_e4m3fn: FP8}        # uint8 holds e4m3 codes
    if t.dtype not in m:
        raise TypeError(f"unsupported K/V dtype {t.dtype}")
    return m[t.dtype]


def decode_args(*, q, k, v, kv_len, part_o, part_ml, causal=True, scale, softcap=0.0,
                alibi=None, slice_len, k_scale=None, v_scale=None, dbg_visit=None,
                tree_parent=None) -> DecodeArgs:
    """Fill the decode struct from tensors: q [S][R][Hq][D] fp32 contiguous,
    k/v [S][cap][Hkv][D] (dim contiguous), scales [S][cap][Hkv], kv_len int32 [S],
    part_o [S][R][Hq][ns][D], part_ml [S][R][Hq][ns][2] (both None for
    sel_attn_decode_noalloc), tree_parent int32 [S][R]."""
    S, R, Hq, D = q.shape
    a = DecodeArgs()
    a.n_stream, a.n_row, a.n_head_q, a.head_dim = S, R, Hq, D
    a.n_head_kv = k.shape[2]
    a.cap = k.shape[1]
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.kv_dtype = kv_dtype_code(k)
    a.kv_stride_stream, a.kv_stride_cell, a.kv_stride_head = k.stride(0), k.stride(1), k.stride(2)
    if k_scale is not None:
        a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
        a.sc_stride_stream, a.sc_stride_cell, a.sc_stride_head = k_scale.stride()
    a.kv_len = _ptr(kv_len)
    a.causal = int(bool(causal))
    a.scale, a.softcap = float(scale), float(softcap)
    a.alibi_slopes = _ptr(alibi)
    a.slice_len = int(slice_len)
    a.n_slices_max = 0 if part_o is None else part_o.shape[3]
    a.part_o, a.part_ml, a.dbg_visit = _ptr(part_o), _ptr(part_ml), _ptr(dbg_visit)
    a.tree_parent = _ptr(tree_parent)
    return a


def sel_attn_decode(args: DecodeArgs, stream=None):
    _check(lib().sel_attn_decode(ctypes.byref(args), _stream(stream)), "sel_attn_decode")


def sel_attn_decode_noalloc(args: DecodeArgs, out, sinks=None, stream=None):
    """Decode + combine with the partials in the library's own scratch (no
    allocation): `args` without partial buffers, out fp32 [S][R][Hq][D]."""
    _check(lib().sel_attn_decode_noalloc(ctypes.byref(args), _ptr(out), _ptr(sinks), _stream(stream)),
           "sel_attn_decode_noalloc")


def combine_args(*, part_o, part_ml, out, kv_len=None, slice_len=0, cap=0,
                 sinks=None) -> CombineArgs:
    """part_o [S][R][Hq][ns][D], part_ml [S][R][Hq][ns][2], out [S][R][Hq][D], sinks fp32 [Hq]."""
    S, R, Hq, ns, D = part_o.shape
    a = CombineArgs()
    a.n_stream, a.n_row, a.n_head_q, a.head_dim, a.n_slices_max = S, R, Hq, D, ns
    a.kv_len = _ptr(kv_len)
    a.slice_len, a.cap = int(slice_len), int(cap)
    a.part_o, a.part_ml, a.out = _ptr(part_o), _ptr(part_ml), _ptr(out)
    a.sinks = _ptr(sinks)
    return a


def sel_attn_split_combine(args: CombineArgs, stream=None):
    _check(lib().sel_attn_split_combine(ctypes.byref(args), _stream(stream)), "sel_attn_split_combine")


def prefill_args(*, q, k, v, out=None, scale, softcap=0.0, alibi=None, q_pos=None, sel=None,
                 block_size=1, mask=None, mask_stride_head=0, causal=False, k_scale=None,
                 v_scale=None, n_splits=1, part_o=None, part_ml=None, dbg_visit=None,
                 dbg_sel=None, sinks=None) -> PrefillArgs:
    """q [R][Hq][D] fp32; k/v [N][Hkv][D]; sel int32 [R][n_sel] or mask fp32 [R][N]
    (row stride taken from the tensor, head stride as given, 0 = broadcast);
    sinks fp32 [Hq] (read when n_splits == 1)."""
    R, Hq, D = q.shape
    a = PrefillArgs()
    a.n_row, a.n_head_q, a.head_dim = R, Hq, D
    a.n_head_kv = k.shape[1]
    a.n_kv = k.shape[0]
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.kv_dtype = kv_dtype_code(k)
    a.kv_stride_cell, a.kv_stride_head = k.stride(0), k.stride(1)
    if k_scale is not None:
        a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
        a.sc_stride_cell, a.sc_stride_head = k_scale.stride()
    a.q_pos = _ptr(q_pos)
    a.scale, a.softcap = float(scale), float(softcap)
    a.alibi_slopes = _ptr(alibi)
    if sel is not None:
        a.sel, a.n_sel, a.block_size = _ptr(sel), sel.shape[1], int(block_size)
    if mask is not None:
        a.mask, a.mask_stride_row, a.mask_stride_head = _ptr(mask), mask.stride(0), int(mask_stride_head)
    a.causal = int(bool(causal))
    a.n_splits = int(n_splits)
    a.out, a.part_o, a.part_ml = _ptr(out), _ptr(part_o), _ptr(part_ml)
    a.dbg_visit, a.dbg_sel = _ptr(dbg_visit), _ptr(dbg_sel)
    a.sinks = _ptr(sinks)
    return a


def sel_attn_prefill(args: PrefillArgs, stream=None):
    _check(lib().sel_attn_prefill(ctypes.byref(args), _stream(stream)), "sel_attn_prefill")


def supports(op: int, args) -> bool:
    return bool(lib().sel_attn_supports(int(op), ctypes.cast(ctypes.byref(args), _p)))


def decode_path(args: DecodeArgs) -> int:
    return lib().sel_attn_decode_path(ctypes.byref(args))


def prefill_path(args: PrefillArgs) -> int:
    return lib().sel_attn_prefill_path(ctypes.byref(args))


def decode_workspace(args: DecodeArgs):
    o, ml = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().sel_attn_decode_workspace(ctypes.byref(args), ctypes.byref(o), ctypes.byref(ml)),
           "sel_attn_decode_workspace")
    return o.value, ml.value
