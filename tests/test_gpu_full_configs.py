"""The five named workloads at full size, in the launch configuration bench.py
times, checked against the FP64 oracle on sampled streams / rows (the oracle
computes those exactly) and by properties that hold everywhere (finite output,
visited sets)."""

import numpy as np
import pytest
import torch

import bench
import oracle
from tests import hip_run
from tests.test_gpu_parity import TOL, nmse_check
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def _decode_streams(wl, idx):
    idx = np.asarray(idx)
    return oracle.decode(q=wl.q[idx], k=wl.k[idx], v=wl.v[idx], kv_dtype=wl.kv_dtype,
                         kv_len=wl.kv_len[idx], causal=wl.causal, scale=wl.scale,
                         softcap=wl.softcap, alibi=wl.alibi,
                         k_scale=None if wl.k_scale is None else wl.k_scale[idx],
                         v_scale=None if wl.v_scale is None else wl.v_scale[idx],
                         tree_parent=None if wl.tree_parent is None else wl.tree_parent[idx],
                         sinks=wl.sinks)


def test_config2_split_k_decode_full():
    wl = gen.config2()
    out, dev = hip_run.run_decode(wl, dbg=False, return_dev=True)
    assert np.isfinite(out).all()
    order = np.argsort(wl.kv_len)
    idx = sorted({int(order[0]), int(order[-1]), 0})       # shallowest, deepest, first
    nmse_check(out[idx], _decode_streams(wl, idx), TOL["bf16"], "config2 sampled streams")
    again = hip_run.run_decode(wl)
    assert again.tobytes() == out.tobytes(), "not deterministic across runs"


@pytest.mark.parametrize("depth", [12000, 32000])
def test_config5_int8_verify_full(depth):
    wl = gen.config5(depth)
    out = hip_run.run_decode(wl)
    assert np.isfinite(out).all()
    idx = [0, 15]
    nmse_check(out[idx], _decode_streams(wl, idx), TOL["i8"], f"config5 depth {depth}")


def test_config5_tree_verify_full():
    """The int8 verify workload at depth 32000 with every window a 16-node binary tree in
    heap order (the launch bench.py times), on two sampled streams, with the visited
    cells of every row and slice of those streams."""
    wl = gen.config5(32000, tree="heap")
    out, dev = hip_run.run_decode(wl, dbg=True, return_dev=True)
    assert np.isfinite(out).all()
    idx = [0, 15]
    nmse_check(out[idx], _decode_streams(wl, idx), TOL["i8"], "tree verify depth 32000")
    st = oracle.visited_decode(kv_len=wl.kv_len[idx], n_row=wl.n_row, causal=True,
                               slice_len=wl.slice_len, n_head_kv=wl.n_head_kv,
                               tree_parent=wl.tree_parent[idx])
    assert np.array_equal(dev.dbg.cpu().numpy()[idx], st)


def test_config2_fp8_decode_full():
    """The split-K workload with e4m3 rows and fp32 row scales (the launch bench.py
    times), on the shallowest and deepest streams."""
    wl = gen.config2(kv_dtype="fp8")
    out = hip_run.run_decode(wl)
    assert np.isfinite(out).all()
    order = np.argsort(wl.kv_len)
    idx = sorted({int(order[0]), int(order[-1])})
    nmse_check(out[idx], _decode_streams(wl, idx), TOL["fp8"], "fp8 split-K sampled streams")


def test_config3_selected_key_prefill_full():
    wl = gen.config3()
    out, dev = hip_run.run_prefill(wl, dbg=True, return_dev=True)
    assert np.isfinite(out).all()
    rng = np.random.default_rng(0)
    rows = sorted(set([0, wl.n_row - 1] + list(rng.choice(wl.n_row, 30, replace=False))))
    ref = oracle.prefill(q=wl.q, k=wl.k, v=wl.v, kv_dtype="bf16", scale=wl.scale, q_pos=wl.q_pos,
                         sel=wl.sel, block_size=wl.block_size, rows=rows)
    nmse_check(out[rows], ref[rows], TOL["bf16"], "config3 sampled rows")
    cells, ids = oracle.visited_prefill(n_kv=wl.n_kv, n_head_kv=wl.n_head_kv, sel=wl.sel,
                                        block_size=wl.block_size, rows=rows)
    dsel = dev.dbg_sel.cpu().numpy()
    dv = dev.dbg.cpu().numpy()
    for i, r in enumerate(rows):
        for g in range(wl.n_head_kv):
            n = int(dsel[r, g, 0])
            assert n == ids[i].size == 476
            assert np.array_equal(dsel[r, g, 1:1 + n], ids[i])
            c = cells[i]
            assert dv[r, g, 0].tolist() == [c.size, int(c.sum()), int((c * c).sum())]


@pytest.mark.parametrize("nan", [True, False])
@pytest.mark.parametrize("n_splits", [1, bench.EDGE_SPLITS])
def test_config4_semantic_edge_prefill_full(nan, n_splits):
    """Both the unsplit call and the launch bench.py times (key-range splits, then
    the combine) against the oracle."""
    wl = gen.config4(nan=nan)
    out = hip_run.run_prefill(wl, n_splits=n_splits)
    ref = oracle.prefill(q=wl.q, k=wl.k, v=wl.v, kv_dtype="f16", scale=wl.scale, softcap=wl.softcap,
                         alibi=wl.alibi, q_pos=wl.q_pos, mask=wl.mask, causal=True)
    nmse_check(out, ref, TOL["f16"], f"config4 nan={nan} splits={n_splits}")
    ex = wl.meta["excluded_rows"]
    assert ex.size == 8
    assert np.all(out[ex] == 0) and not np.signbit(out[ex]).any()
    if nan:
        # every row that sees anything sees a NaN key in each kv head group
        assert np.isnan(np.delete(out, ex, axis=0)).all()
    else:
        assert np.isfinite(out).all()


def test_selected_key_decode_full():
    """The selected-key decode workload in the launch configuration bench.py times
    (32 key-range splits + combine), against the oracle on every row."""
    wl = gen.sel_decode()
    out = hip_run.run_prefill(wl, n_splits=bench.SEL_DECODE_SPLITS)
    assert np.isfinite(out).all()
    ref = oracle.prefill(q=wl.q, k=wl.k, v=wl.v, kv_dtype="bf16", scale=wl.scale, q_pos=wl.q_pos,
                         sel=wl.sel, block_size=wl.block_size)
    nmse_check(out, ref, TOL["bf16"], "selected-key decode")
