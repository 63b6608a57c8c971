"""GPU parity: NaN and +-Inf in V (or in an int8 row scale) on keys that some
query vectors of a tile see and others do not.

A key outside a query vector's visible set must contribute nothing to it, even
when its V row is NaN or Inf: the masked cells are skipped, not weighted with
zero (strix-llama.cpp PR #115, "Measurements", the poison=1 cases), while a
visible NaN still reaches the output dim it sits in and a visible +-Inf makes
that dim +-Inf (both signs: NaN) (HartsyInference PR #910, review of
attention_softmax.cu).  The cases put such values where visibility differs
inside one work-group: a draft row's own cell in a causal verify window (seen
by the later rows only), one branch of a tree window (not seen by its
siblings), and a cell whose mask entry is -inf for one row and finite for
another.  Every output is compared with the FP64 oracle element by element:
values within the tolerance, NaN and Inf positions identical.
"""

import numpy as np
import pytest
import torch

import oracle
from tests import hip_run
from tests.test_gpu_parity import TOL, nmse_check, oracle_decode, oracle_prefill
from workloads import gen

pytestmark = pytest.mark.gpu

NAN16 = {"bf16": np.uint16(0x7FC0), "f16": np.float16(np.nan)}
PINF16 = {"bf16": np.uint16(0x7F80), "f16": np.float16(np.inf)}
NINF16 = {"bf16": np.uint16(0xFF80), "f16": np.float16(-np.inf)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def plant(wl, where, kind, dims=None):
    """Puts a non-finite value into V at `where` = (stream, cell, kv head) for decode
    or (cell, kv head) for prefill: kind 'nan' / '+inf' / '-inf' in the listed dims
    (all dims when None) for 16-bit data, the e4m3 NaN code for fp8, and a NaN or
    Inf row scale for int8 ('nan' / '+inf'), which makes the whole row non-finite."""
    v = wl.v.copy()
    dsel = slice(None) if dims is None else list(dims)
    if wl.kv_dtype == "i8":
        vs = wl.v_scale.copy()
        vs[where] = np.nan if kind == "nan" else np.inf
        wl.v_scale = vs
        return
    if wl.kv_dtype == "fp8":
        assert kind == "nan", "e4m3 has no infinities"
        v[where + (dsel,)] = np.uint8(0xFF)
    else:
        val = {"nan": NAN16, "+inf": PINF16, "-inf": NINF16}[kind][wl.kv_dtype]
        v[where + (dsel,)] = val
    wl.v = v


def check(wl, out, ref, what):
    nmse_check(out, ref, TOL[wl.kv_dtype], what)
    assert np.isnan(ref).any() or np.isinf(ref).any(), f"{what}: the plant reached no output"
    assert np.isfinite(ref).any(), f"{what}: nothing stayed finite"


# ----------------------------------------------------------------------------
# causal verify windows: a row's own cell is seen by that row and the later ones
# ----------------------------------------------------------------------------

WINDOW_SHAPES = {
    # one wave per unit: 2 rows x 8 heads = 16 query vectors
    "one_wave": dict(n_stream=2, n_row=2, n_head_q=16, n_head_kv=2, head_dim=256, cap=700, depths=[700, 333],
                     slice_len=256),
    # work-group kernels: 5 x 8 = 40 query vectors (4 waves), 16 x 8 (8 waves), 16 x 12 (12 waves)
    "w4": dict(n_stream=2, n_row=5, n_head_q=16, n_head_kv=2, head_dim=128, cap=600, depths=[600, 290],
               slice_len=256),
    "w8": dict(n_stream=2, n_row=16, n_head_q=16, n_head_kv=2, head_dim=256, cap=520, depths=[520, 300],
               slice_len=512),
    "w12": dict(n_stream=2, n_row=16, n_head_q=48, n_head_kv=4, head_dim=256, cap=2116, depths=[700, 2116],
                slice_len=512),
}


@pytest.mark.parametrize("dtype", ["bf16", "f16", "fp8", "i8"])
@pytest.mark.parametrize("shape", sorted(WINDOW_SHAPES))
def test_window_row_cell_nonfinite(shape, dtype):
    kw = WINDOW_SHAPES[shape]
    wl = gen.make_decode(seed=[31, len(shape), len(dtype)], kv_dtype=dtype, **kw)
    R = wl.n_row
    for b in range(wl.n_stream):
        n = int(wl.kv_len[b])
        own = lambda r: n - R + r                  # row r's own cell
        if dtype in ("fp8", "i8"):
            plant(wl, (b, own(R // 2), 0), "nan")
            plant(wl, (b, own(R - 1), wl.n_head_kv - 1), "nan" if dtype == "fp8" else "+inf")
        else:
            plant(wl, (b, own(R // 2), 0), "nan")                       # every dim
            plant(wl, (b, own(R // 3), 1), "+inf", dims=[3, 70])
            plant(wl, (b, own(R - 1), 1), "-inf", dims=[3])             # with the +inf: NaN
            plant(wl, (b, own(0), wl.n_head_kv - 1), "-inf", dims=[9])
    out = hip_run.run_decode(wl)
    ref = oracle_decode(wl)
    check(wl, out, ref, f"window {shape} {dtype}")
    if R > 1:
        # the rows before the planted row stay finite in the planted kv head's heads
        G = wl.n_head_q // wl.n_head_kv
        assert np.isfinite(out[:, :R // 2, :G]).all()


def test_window_nonfinite_split_partials():
    """The partials of the slice holding the window carry the same rule."""
    wl = gen.make_decode(seed=32, n_stream=1, n_row=16, n_head_q=48, n_head_kv=4, head_dim=256,
                         cap=1040, kv_dtype="bf16", depths=[1040], slice_len=1024)
    plant(wl, (0, 1040 - 16 + 7, 2), "nan", dims=[0, 255])
    out = hip_run.run_decode(wl, slice_len=1024)
    check(wl, out, oracle_decode(wl), "window split 1024")
    out = hip_run.run_decode(wl, slice_len=32)
    check(wl, out, oracle_decode(wl), "window split 32")


# ----------------------------------------------------------------------------
# tree windows: a branch is not seen by its siblings
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp8", "i8"])
@pytest.mark.parametrize("shape", ["one_wave", "w12"])
def test_tree_branch_nonfinite(shape, dtype):
    if shape == "one_wave":
        kw = dict(n_stream=2, n_row=4, n_head_q=8, n_head_kv=2, head_dim=256, cap=400, depths=[400, 150],
                  slice_len=128)
    else:
        kw = dict(n_stream=2, n_row=16, n_head_q=48, n_head_kv=4, head_dim=256, cap=1100, depths=[1100, 600],
                  slice_len=512)
    wl = gen.make_decode(seed=[33, len(shape), len(dtype)], kv_dtype=dtype, tree="heap", **kw)
    R = wl.n_row
    for b in range(wl.n_stream):
        start = int(wl.kv_len[b]) - R
        # node 1 (children 3, 4) is not on the paths of node 2 and its subtree
        plant(wl, (b, start + 1, 0), "nan")
        if dtype == "bf16":
            plant(wl, (b, start + 2, 1), "+inf", dims=[5])
    out = hip_run.run_decode(wl)
    ref = oracle.decode(q=wl.q, k=wl.k, v=wl.v, kv_dtype=wl.kv_dtype, kv_len=wl.kv_len, causal=True,
                        scale=wl.scale, k_scale=wl.k_scale, v_scale=wl.v_scale,
                        tree_parent=wl.tree_parent)
    check(wl, out, ref, f"tree {shape} {dtype}")
    G = wl.n_head_q // wl.n_head_kv
    assert np.isfinite(out[:, 2, :G]).all() and np.isnan(out[:, 1, :G]).all()


# ----------------------------------------------------------------------------
# mask mode: a cell masked for one row and seen by another of the same work-group
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,head_dim", [("f16", 128), ("bf16", 256), ("fp8", 256), ("i8", 128)])
def test_mask_row_excluded_nonfinite(dtype, head_dim):
    wl = gen.make_prefill_mask(seed=[34, head_dim, len(dtype)], n_row=40, n_head_q=16, n_head_kv=4,
                               head_dim=head_dim, n_kv=500, kv_dtype=dtype, causal=True,
                               excluded_rows=2, softcap=30.0, alibi=True)
    mask = wl.mask.copy()
    c0, c1 = 100, 205
    # rows 0..15 share the first work-group (4 heads each): c0 is -inf for even rows,
    # c1 for rows 3 and 7 only
    mask[0:16:2, c0] = -np.inf
    mask[[3, 7], c1] = -np.inf
    wl.mask = mask
    plant(wl, (c0, 0), "nan")
    if dtype in ("f16", "bf16"):
        plant(wl, (c1, 1), "+inf", dims=[2, 3])
        plant(wl, (c1 + 1, 1), "-inf", dims=[3])       # seen with c1 by most rows: NaN at dim 3
    else:
        plant(wl, (c1, 1), "nan")
    out = hip_run.run_prefill(wl)
    ref = oracle_prefill(wl)
    check(wl, out, ref, f"mask {dtype}")
    ex = wl.meta["excluded_rows"]
    assert np.all(out[ex] == 0) and not np.signbit(out[ex]).any()
    # even rows of the first work-group do not see c0: their kv-head-0 heads stay finite
    even = [r for r in range(0, 16, 2) if r not in set(ex.tolist())]
    assert np.isfinite(out[even, 0:4]).all()
    # splits: the same rule per key range
    check(wl, hip_run.run_prefill(wl, n_splits=3), ref, f"mask {dtype} split")


def test_full_tiles_still_propagate():
    """Keys every query vector sees: a NaN V dim reaches every row, an Inf likewise."""
    wl = gen.make_decode(seed=35, n_stream=1, n_row=2, n_head_q=16, n_head_kv=2, head_dim=256,
                         cap=300, kv_dtype="bf16", depths=[300], slice_len=256)
    plant(wl, (0, 10, 0), "nan", dims=[4])
    plant(wl, (0, 11, 1), "-inf", dims=[6])
    out = hip_run.run_decode(wl)
    check(wl, out, oracle_decode(wl), "full tiles")
    assert np.isnan(out[0, :, :8, 4]).all() and np.isneginf(out[0, :, 8:, 6]).all()
