"""C-ABI checks that need no GPU: symbols, struct layout, host-side validation.

Nothing here launches a kernel: every call either is host-only (supports,
workspace, path, strerror) or returns an error before any HIP call.
"""

import ctypes
import os
import re

import pytest

import split_flash_attention_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sel_attn.h")

FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced here


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sa.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return sa.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(sel_attn_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"sel_attn_decode", "sel_attn_prefill", "sel_attn_split_combine"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_struct_sizes_match(L):
    assert L.sel_attn_args_size(sa.OP_DECODE) == ctypes.sizeof(sa.DecodeArgs)
    assert L.sel_attn_args_size(sa.OP_PREFILL) == ctypes.sizeof(sa.PrefillArgs)
    assert L.sel_attn_args_size(sa.OP_COMBINE) == ctypes.sizeof(sa.CombineArgs)
    assert L.sel_attn_abi_version() == 2
    assert sa.strerror(sa.EWORKSPACE).startswith("partial buffer")


def good_decode(**over):
    a = sa.DecodeArgs()
    a.n_stream, a.n_row, a.n_head_q, a.n_head_kv, a.head_dim, a.cap = 16, 1, 32, 4, 256, 32768
    a.q = a.k = a.v = a.kv_len = a.part_o = a.part_ml = FAKE
    a.kv_dtype = sa.BF16
    a.kv_stride_stream, a.kv_stride_cell, a.kv_stride_head = 32768 * 1024, 1024, 256
    a.causal, a.scale, a.softcap = 1, 0.0625, 0.0
    a.slice_len, a.n_slices_max = 1024, 32
    for k, v in over.items():
        setattr(a, k, v)
    return a


def good_prefill(**over):
    a = sa.PrefillArgs()
    a.n_row, a.n_head_q, a.n_head_kv, a.head_dim, a.n_kv = 2048, 16, 2, 256, 32048
    a.q = a.k = a.v = a.out = FAKE
    a.kv_dtype = sa.BF16
    a.kv_stride_cell, a.kv_stride_head = 512, 256
    a.scale = 0.0625
    a.sel, a.n_sel, a.block_size = FAKE, 512, 4
    a.n_splits = 1
    for k, v in over.items():
        setattr(a, k, v)
    return a


def good_combine(**over):
    a = sa.CombineArgs()
    a.n_stream, a.n_row, a.n_head_q, a.head_dim, a.n_slices_max = 16, 1, 32, 256, 32
    a.part_o = a.part_ml = a.out = FAKE
    for k, v in over.items():
        setattr(a, k, v)
    return a


def _status(fn, args):
    return fn(ctypes.byref(args), None)


def test_good_arguments_are_supported(L):
    assert sa.supports(sa.OP_DECODE, good_decode())
    assert sa.supports(sa.OP_PREFILL, good_prefill())
    assert sa.supports(sa.OP_COMBINE, good_combine())
    assert not sa.supports(99, good_decode())
    # one-byte rows with fp32 row scales: int8 and e4m3 (fp8)
    for dt in (sa.I8, sa.FP8):
        a = good_decode(kv_dtype=dt, k_scale=FAKE, v_scale=FAKE, kv_stride_stream=32768 * 1024,
                        kv_stride_cell=1024, kv_stride_head=256)
        assert sa.supports(sa.OP_DECODE, a)
        assert sa.decode_path(a) == 1                        # the matrix-core kernels take it
    # tree windows up to 64 rows; sink logits on the combine and the unsplit prefill
    assert sa.supports(sa.OP_DECODE, good_decode(tree_parent=FAKE, n_row=64))
    assert sa.supports(sa.OP_COMBINE, good_combine(sinks=FAKE))
    assert sa.supports(sa.OP_PREFILL, good_prefill(sinks=FAKE))


@pytest.mark.parametrize("over,code", [
    (dict(q=None), sa.EINVAL),
    (dict(kv_len=None), sa.EINVAL),
    (dict(part_o=None), sa.EINVAL),
    (dict(n_stream=0), sa.EINVAL),
    (dict(n_head_q=30), sa.EINVAL),            # 30 % 4 != 0
    (dict(slice_len=0), sa.EINVAL),
    (dict(kv_dtype=sa.I8), sa.EINVAL),         # int8 without scales
    (dict(kv_dtype=sa.FP8), sa.EINVAL),        # e4m3 without scales
    (dict(kv_dtype=5), sa.EUNSUPPORTED),       # no storage type 5
    (dict(head_dim=96, kv_stride_head=96), sa.EUNSUPPORTED),
    (dict(kv_dtype=7), sa.EUNSUPPORTED),
    (dict(softcap=-1.0), sa.EUNSUPPORTED),
    (dict(softcap=float("inf")), sa.EUNSUPPORTED),
    (dict(scale=float("nan")), sa.EUNSUPPORTED),
    (dict(k=FAKE + 2), sa.EUNSUPPORTED),       # misaligned
    (dict(kv_stride_cell=1001), sa.EUNSUPPORTED),
    (dict(n_slices_max=31), sa.EWORKSPACE),    # 31 * 1024 < 32768
    (dict(tree_parent=FAKE, n_row=65), sa.EUNSUPPORTED),   # one 64-bit path mask per row
])
def test_decode_validation(L, over, code):
    a = good_decode(**over)
    assert _status(L.sel_attn_decode, a) == code
    assert not sa.supports(sa.OP_DECODE, a)
    assert L.sel_attn_decode_path(ctypes.byref(a)) == code


@pytest.mark.parametrize("over,code", [
    (dict(mask=FAKE, mask_stride_row=32048), sa.EINVAL),      # both modes
    (dict(sel=None), sa.EINVAL),                              # neither mode
    (dict(n_sel=0), sa.EINVAL),
    (dict(n_sel=4097), sa.EINVAL),
    (dict(block_size=0), sa.EINVAL),
    (dict(out=None), sa.EINVAL),
    (dict(n_splits=2), sa.EINVAL),                            # partials missing
    (dict(alibi_slopes=FAKE), sa.EINVAL),                     # ALiBi needs q_pos
    (dict(n_head_kv=3), sa.EINVAL),
    (dict(head_dim=100), sa.EUNSUPPORTED),
    (dict(n_head_q=66, n_head_kv=1), sa.EUNSUPPORTED),        # group of 66 heads
    (dict(softcap=-30.0), sa.EUNSUPPORTED),
    (dict(kv_dtype=sa.F32, kv_stride_cell=1024, kv_stride_head=512), sa.EUNSUPPORTED),
    (dict(head_dim=64, kv_stride_cell=128, kv_stride_head=64), sa.EUNSUPPORTED),
    (dict(out=FAKE + 4), sa.EUNSUPPORTED),
])
def test_prefill_validation(L, over, code):
    a = good_prefill(**over)
    assert _status(L.sel_attn_prefill, a) == code
    assert not sa.supports(sa.OP_PREFILL, a)


def test_prefill_mask_mode_validation(L):
    a = good_prefill(sel=None, n_sel=0, mask=FAKE, mask_stride_row=32048, causal=1)
    assert _status(L.sel_attn_prefill, a) == sa.EINVAL      # causal needs q_pos
    a.q_pos = FAKE
    assert sa.supports(sa.OP_PREFILL, a)
    a.mask_stride_row = 0
    assert not sa.supports(sa.OP_PREFILL, a)


@pytest.mark.parametrize("over,code", [
    (dict(out=None), sa.EINVAL),
    (dict(n_slices_max=0), sa.EINVAL),
    (dict(kv_len=FAKE, slice_len=0, cap=10), sa.EINVAL),
    (dict(head_dim=32), sa.EUNSUPPORTED),
    (dict(out=FAKE + 8), sa.EUNSUPPORTED),          # out not 16-byte aligned
    (dict(part_o=FAKE + 4), sa.EUNSUPPORTED),       # part_o not 16-byte aligned
    (dict(part_ml=FAKE + 4), sa.EUNSUPPORTED),      # part_ml not 8-byte aligned
])
def test_combine_validation(L, over, code):
    assert _status(L.sel_attn_split_combine, good_combine(**over)) == code


def test_workspace_query(L):
    o, ml = sa.decode_workspace(good_decode())
    assert o == 16 * 1 * 32 * 32 * 256 * 4
    assert ml == 16 * 1 * 32 * 32 * 2 * 4
    assert L.sel_attn_decode_workspace(None, None, None) == sa.EINVAL


def test_null_struct_pointers(L):
    assert L.sel_attn_decode(None, None) == sa.EINVAL
    assert L.sel_attn_prefill(None, None) == sa.EINVAL
    assert L.sel_attn_split_combine(None, None) == sa.EINVAL


def test_noalloc_validates_before_any_device_call(L):
    """sel_attn_decode_noalloc refuses bad calls on the host, before it looks up its
    scratch: partial buffers given, a NULL output, partials beyond the scratch."""
    out = ctypes.c_void_p(FAKE)
    a = good_decode()
    assert L.sel_attn_decode_noalloc(ctypes.byref(a), out, None, None) == sa.EINVAL   # partials given
    a = good_decode(part_o=None, part_ml=None)
    assert L.sel_attn_decode_noalloc(ctypes.byref(a), None, None, None) == sa.EINVAL  # no output
    # 16 x 16 x 48 x 64 slices x 258 x 4 B = 203 MB > the 64 MiB scratch
    a = good_decode(part_o=None, part_ml=None, n_row=16, n_head_q=48, cap=65536)
    assert L.sel_attn_decode_noalloc(ctypes.byref(a), out, None, None) == sa.EWORKSPACE
    # huge sizes do not overflow the size check
    a = good_decode(part_o=None, part_ml=None, n_stream=2 ** 31 - 1, n_row=2 ** 31 - 1,
                    n_head_q=2 ** 31 - 1 - (2 ** 31 - 1) % 4, n_head_kv=4, slice_len=1)
    assert L.sel_attn_decode_noalloc(ctypes.byref(a), out, None, None) == sa.EWORKSPACE
    # a call that fits but that decode itself refuses (head_dim 96): decode's status
    a = good_decode(part_o=None, part_ml=None, head_dim=96)
    assert L.sel_attn_decode_noalloc(ctypes.byref(a), out, None, None) == sa.EUNSUPPORTED
    a = good_decode(part_o=None, part_ml=None, n_head_q=30)                 # 30 % 4 != 0
    assert L.sel_attn_decode_noalloc(ctypes.byref(a), out, None, None) == sa.EINVAL
    assert sa.NOALLOC_SCRATCH_BYTES == 64 * 1024 * 1024


def test_planted_variants_are_declared_and_guarded():
    """Each planted-mistake build names a define that the sources guard with #ifdef
    (so a product build, which sets none, never contains it) and a GPU control."""
    import glob
    from split_flash_attention_amd import build
    from tests.test_gpu_planted import CONTROLS
    assert set(build.PLANTS) == set(CONTROLS)
    csrc = glob.glob(os.path.join(os.path.dirname(build.__file__), "csrc", "*"))
    text = "".join(open(f).read() for f in csrc if f.endswith((".h", ".hip")))
    for name, (src, define) in build.PLANTS.items():
        assert src in build.SOURCES
        assert f"#ifdef {define}" in text, define
    assert "#define SELATTN_PLANT" not in text
