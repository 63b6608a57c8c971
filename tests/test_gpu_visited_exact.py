"""GPU: the exact set of cells every query vector combines, per slice, read back
through the split partials of the public decode call.

Construction: Q = 0, so every score a query vector can see is 0, its weight
exp(0 - 0) is exactly 1 and the slice's running sum l is the number of cells
combined; V row `cell` is one-hot on dim `cell mod D` (value 1, row scale 1 for
the byte formats).  With slices of at most D cells the residues of a slice's
cells are distinct, so dim d of a slice's unnormalised partial o is 1 exactly
when the cell with residue d was combined and 0 otherwise.  Every (stream, row,
query head, slice) is compared with the oracle's visible set (TensorFold PR
#2595, attn_decode contract: causal verify windows see the cells up to their
own; tree windows the prefix plus their path), covering each decode kernel the
library routes to: one wave per unit (up to 16 query vectors), the int8 wide
kernel (more than 32), the work-group kernel (the other shapes) and the
vector-ALU kernel (fp32 rows).
"""

import numpy as np
import pytest
import torch

import oracle
from tests import hip_run
from workloads import gen

pytestmark = pytest.mark.gpu

ONE = {"bf16": np.uint16(0x3F80), "f16": np.float16(1.0), "f32": np.float32(1.0),
       "i8": np.int8(1), "fp8": np.uint8(0x38)}      # 1.0 in each storage format (e4m3 0x38)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def one_hot_workload(**kw):
    wl = gen.make_decode(seed=41, **kw)
    S, cap, hkv, D = wl.v.shape
    v = np.zeros_like(wl.v)
    cells = np.arange(cap)
    v[:, cells, :, cells % D] = ONE[wl.kv_dtype]
    wl.v = v
    if wl.v_scale is not None:
        wl.v_scale = np.ones_like(wl.v_scale)
    wl.q = np.zeros_like(wl.q)
    return wl


def check_sets(wl, what):
    d = hip_run.DecodeDev(wl, "cuda")
    d.run()
    torch.cuda.synchronize()
    po = d.part_o.cpu().numpy()
    pml = d.part_ml.cpu().numpy()
    S, R, Hq, D = wl.q.shape
    L = d.slice_len
    assert L <= D
    checked = 0
    for b in range(S):
        n = int(wl.kv_len[b])
        ns_b = -(-n // L)
        for r in range(R):
            par = None if wl.tree_parent is None else wl.tree_parent[b]
            cells = oracle.visible_decode_row(n, R, r, wl.causal, par)
            for t in range(ns_b):
                want = np.zeros(D)
                c = cells[(cells >= t * L) & (cells < (t + 1) * L)]
                want[c % D] = 1.0
                for h in range(Hq):
                    got = po[b, r, h, t]
                    assert np.array_equal(got, want), (
                        f"{what}: stream {b} row {r} head {h} slice {t}: cells "
                        f"{sorted(t * L + (np.flatnonzero(got != want) - t * L) % D)} differ "
                        f"({int(got.sum())} combined, {c.size} visible)")
                    assert pml[b, r, h, t, 1] == c.size, f"{what}: l is not the visible count"
                    checked += 1
    assert checked > 0


CASES = {
    # one wave per unit: 2 rows x 8 heads, causal and tree
    "lean_bf16": dict(n_stream=2, n_row=2, n_head_q=16, n_head_kv=2, head_dim=256, cap=700,
                      kv_dtype="bf16", depths=[700, 333], slice_len=256),
    "lean_fp8_tree": dict(n_stream=2, n_row=2, n_head_q=16, n_head_kv=2, head_dim=128, cap=400,
                          kv_dtype="fp8", depths=[400, 131], slice_len=128, tree="chain"),
    # the int8 wide kernel: 16 rows x 12 heads = 192 query vectors; 5 x 8 = 40 at D = 128
    "wide_i8": dict(n_stream=2, n_row=16, n_head_q=48, n_head_kv=4, head_dim=256, cap=1100,
                    kv_dtype="i8", depths=[1100, 517], slice_len=256),
    "wide_i8_tree": dict(n_stream=2, n_row=16, n_head_q=48, n_head_kv=4, head_dim=256, cap=900,
                         kv_dtype="i8", depths=[900, 300], slice_len=256, tree="heap"),
    "wide_i8_d128_half_slices": dict(n_stream=2, n_row=5, n_head_q=16, n_head_kv=2, head_dim=128,
                                     cap=600, kv_dtype="i8", depths=[600, 290], slice_len=64),
    # the work-group kernel: 16 x 8 = 128 and 5 x 8 = 40 query vectors
    "group_bf16": dict(n_stream=2, n_row=16, n_head_q=16, n_head_kv=2, head_dim=256, cap=520,
                       kv_dtype="bf16", depths=[520, 300], slice_len=256),
    "group_f16_tree": dict(n_stream=2, n_row=16, n_head_q=16, n_head_kv=2, head_dim=128, cap=500,
                           kv_dtype="f16", depths=[500, 77], slice_len=128, tree="random"),
    "group_fp8": dict(n_stream=2, n_row=5, n_head_q=16, n_head_kv=2, head_dim=128, cap=600,
                      kv_dtype="fp8", depths=[600, 290], slice_len=128),
    # fp32 rows: the vector-ALU kernel
    "valu_f32": dict(n_stream=2, n_row=4, n_head_q=8, n_head_kv=2, head_dim=128, cap=400,
                     kv_dtype="f32", depths=[400, 129], slice_len=128),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_visited_cells_exact(name):
    check_sets(one_hot_workload(**CASES[name]), name)


def test_visited_cells_exact_non_causal():
    check_sets(one_hot_workload(**dict(CASES["group_bf16"], causal=False)), "non-causal")
