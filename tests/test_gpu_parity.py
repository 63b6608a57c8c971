"""GPU parity: the HIP library through its C ABI against the FP64 oracle.

Bars (from the workload statement): NMSE <= 1e-6 for fp32 K/V and <= 5e-5 for
bf16 / fp16 / int8 K/V over every element whose reference is finite, and the
same bar for each (row, head) output vector on its own; NaN
positions identical; excluded (row, head) outputs exactly zero; visited cells
identical to the oracle's (count, sum, sum of squares per row and slice, and
the sorted id list in selection mode); bit-identical results across runs.
"""

import numpy as np
import pytest
import torch

import oracle
from tests import hip_run
from workloads import gen

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-6, "f16": 5e-5, "bf16": 5e-5, "i8": 5e-5, "fp8": 5e-5}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import split_flash_attention_amd as sa
    sa.lib()


def nmse_check(out, ref, tol, what=""):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    assert out.shape == ref.shape
    nan_ref, nan_out = np.isnan(ref), np.isnan(out)
    assert np.array_equal(nan_ref, nan_out), f"{what}: NaN pattern differs " \
        f"({nan_ref.sum()} ref vs {nan_out.sum()} gpu)"
    inf_ref = np.isinf(ref)
    assert np.array_equal(out[inf_ref], ref[inf_ref]), f"{what}: inf pattern differs"
    zero = ref == 0.0
    assert np.all(out[zero] == 0.0), f"{what}: {np.sum(out[zero] != 0.0)} nonzero where ref is 0"
    fin = np.isfinite(ref)
    if not fin.any():
        return 0.0
    assert np.isfinite(out[fin]).all(), f"{what}: non-finite gpu where ref is finite"
    err = float(((out[fin] - ref[fin]) ** 2).sum() / max((ref[fin] ** 2).sum(), 1e-300))
    assert err <= tol, f"{what}: NMSE {err:.3e} > {tol:.1e}"
    # the same bar per (row, head): the global figure would hide one dropped cell
    row_err = row_nmse_max(out, ref)
    assert row_err <= tol, f"{what}: per-(row, head) NMSE {row_err:.3e} > {tol:.1e}"
    return err


def row_nmse_max(out, ref):
    """Largest NMSE over the output vectors (last axis) whose finite reference
    elements are not all zero."""
    fin = np.isfinite(ref)
    d = np.where(fin, out - ref, 0.0)
    r = np.where(fin, ref, 0.0)
    num = (d ** 2).sum(axis=-1)
    den = (r ** 2).sum(axis=-1)
    live = den > 0
    return float((num[live] / den[live]).max()) if live.any() else 0.0


def oracle_decode(wl, streams=None):
    sl = slice(None) if streams is None else streams
    return oracle.decode(q=wl.q[sl], k=wl.k[sl], v=wl.v[sl], kv_dtype=wl.kv_dtype,
                         kv_len=wl.kv_len[sl], causal=wl.causal, scale=wl.scale,
                         softcap=wl.softcap, alibi=wl.alibi,
                         k_scale=None if wl.k_scale is None else wl.k_scale[sl],
                         v_scale=None if wl.v_scale is None else wl.v_scale[sl])


def oracle_prefill(wl, rows=None):
    return oracle.prefill(q=wl.q, k=wl.k, v=wl.v, kv_dtype=wl.kv_dtype, scale=wl.scale,
                          softcap=wl.softcap, alibi=wl.alibi, q_pos=wl.q_pos, sel=wl.sel,
                          block_size=wl.block_size, mask=wl.mask, causal=wl.causal,
                          k_scale=wl.k_scale, v_scale=wl.v_scale, rows=rows)


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

def test_config1_dense_decode_tiny():
    wl = gen.config1()
    out = hip_run.run_decode(wl)
    nmse_check(out, oracle_decode(wl), TOL["f32"], "config1")


DECODE_CASES = {
    # name: make_decode kwargs (several tiles, ragged tails, all dtypes and features)
    "bf16_gqa8_d256": dict(n_stream=3, n_row=1, n_head_q=32, n_head_kv=4, head_dim=256,
                           cap=2600, kv_dtype="bf16", depths=[1, 1500, 2600], slice_len=1024),
    "i8_verify_gqa12": dict(n_stream=2, n_row=16, n_head_q=48, n_head_kv=4, head_dim=256,
                            cap=2116, kv_dtype="i8", depths=[716, 2116], slice_len=512),
    "f16_softcap_alibi_d128": dict(n_stream=2, n_row=4, n_head_q=16, n_head_kv=4, head_dim=128,
                                   cap=777, kv_dtype="f16", depths=[777, 130], slice_len=256,
                                   softcap=30.0, alibi=True),
    "f32_short_rows_d64": dict(n_stream=2, n_row=4, n_head_q=8, n_head_kv=2, head_dim=64,
                               cap=40, kv_dtype="f32", depths=[3, 40], slice_len=16),
    "bf16_noncausal_d128": dict(n_stream=2, n_row=3, n_head_q=4, n_head_kv=1, head_dim=128,
                                cap=300, kv_dtype="bf16", depths=[300, 65], slice_len=64,
                                causal=False),
    # more than 16 query vectors per unit: the work-group kernel with 4, 8 and 12
    # waves, a partly filled last block, and two query chunks per unit
    "bf16_verify_w4_d128": dict(n_stream=2, n_row=5, n_head_q=16, n_head_kv=2, head_dim=128,
                                cap=1500, kv_dtype="bf16", depths=[1500, 37], slice_len=512),
    "f16_verify_w8_softcap_alibi": dict(n_stream=2, n_row=16, n_head_q=8, n_head_kv=1, head_dim=256,
                                        cap=700, kv_dtype="f16", depths=[700, 300], slice_len=256,
                                        softcap=20.0, alibi=True),
    "bf16_verify_two_chunks": dict(n_stream=2, n_row=16, n_head_q=16, n_head_kv=1, head_dim=256,
                                   cap=600, kv_dtype="bf16", depths=[600, 100], slice_len=256),
    # 12 waves (two K buffers in LDS): bf16 with softcap and ALiBi, f16 at D = 128
    # with a ragged last block of query vectors, e4m3 at D = 256
    "bf16_verify_w12_softcap_alibi": dict(n_stream=2, n_row=16, n_head_q=24, n_head_kv=2,
                                          head_dim=256, cap=1100, kv_dtype="bf16",
                                          depths=[1100, 47], slice_len=512, softcap=15.0,
                                          alibi=True),
    "f16_verify_w12_d128": dict(n_stream=2, n_row=11, n_head_q=16, n_head_kv=1, head_dim=128,
                                cap=800, kv_dtype="f16", depths=[800, 95], slice_len=256),
    "fp8_verify_w12_d256": dict(n_stream=1, n_row=12, n_head_q=16, n_head_kv=1, head_dim=256,
                                cap=700, kv_dtype="fp8", depths=[700], slice_len=256),
    "i8_verify_w12_d128": dict(n_stream=2, n_row=12, n_head_q=32, n_head_kv=2, head_dim=128,
                               cap=650, kv_dtype="i8", depths=[650, 64], slice_len=256),
    "fp8_verify_w12_d128_noncausal": dict(n_stream=1, n_row=16, n_head_q=12, n_head_kv=1,
                                          head_dim=128, cap=520, kv_dtype="fp8", depths=[520],
                                          slice_len=512, causal=False),
    # byte rows on one wave per unit (raw tiles streamed into LDS two tiles ahead,
    # K widened as read): ragged depths, two-row windows with softcap and ALiBi, trees
    "i8_gqa8_d256": dict(n_stream=3, n_row=1, n_head_q=32, n_head_kv=4, head_dim=256,
                         cap=2600, kv_dtype="i8", depths=[1, 1500, 2599], slice_len=1024),
    "i8_rows2_d128_softcap_alibi": dict(n_stream=2, n_row=2, n_head_q=16, n_head_kv=2, head_dim=128,
                                        cap=900, kv_dtype="i8", depths=[900, 33], slice_len=256,
                                        softcap=25.0, alibi=True),
    "fp8_rows2_d256_tree": dict(n_stream=2, n_row=2, n_head_q=16, n_head_kv=2, head_dim=256,
                                cap=700, kv_dtype="fp8", depths=[700, 18], slice_len=512, tree="heap"),
    # e4m3 K/V rows with fp32 row scales: one block per unit, and a work-group unit
    "fp8_gqa8_d256": dict(n_stream=2, n_row=1, n_head_q=32, n_head_kv=4, head_dim=256,
                          cap=1800, kv_dtype="fp8", depths=[1800, 700], slice_len=512),
    "fp8_verify_gqa12_d128": dict(n_stream=2, n_row=8, n_head_q=24, n_head_kv=2, head_dim=128,
                                  cap=900, kv_dtype="fp8", depths=[900, 333], slice_len=256),
    "i8_verify_noncausal_d128": dict(n_stream=2, n_row=7, n_head_q=24, n_head_kv=2, head_dim=128,
                                     cap=900, kv_dtype="i8", depths=[900, 250], slice_len=384,
                                     causal=False),
}


@pytest.mark.parametrize("name", sorted(DECODE_CASES))
def test_decode_parity(name):
    kw = DECODE_CASES[name]
    wl = gen.make_decode(seed=[77, len(name)], **kw)
    out, dev = hip_run.run_decode(wl, dbg=True, return_dev=True)
    nmse_check(out, oracle_decode(wl), TOL[wl.kv_dtype], name)
    # visited cells: exactly the oracle's, per row and slice
    st = oracle.visited_decode(kv_len=wl.kv_len, n_row=wl.n_row, causal=wl.causal,
                               slice_len=wl.slice_len, n_head_kv=wl.n_head_kv)
    got = dev.dbg.cpu().numpy()
    for b in range(wl.n_stream):
        ns_b = -(-int(wl.kv_len[b]) // wl.slice_len)
        assert np.array_equal(got[b, :, :, :ns_b], st[b, :, :, :ns_b]), (name, b)


def test_decode_split_partials_match_oracle():
    wl = gen.make_decode(seed=5, n_stream=2, n_row=2, n_head_q=8, n_head_kv=2, head_dim=128,
                         cap=700, kv_dtype="bf16", depths=[700, 300], slice_len=256, softcap=5.0)
    out, dev = hip_run.run_decode(wl, return_dev=True)
    _, po, pm, pl = oracle.decode_split(q=wl.q, k=wl.k, v=wl.v, kv_dtype="bf16", kv_len=wl.kv_len,
                                        causal=True, scale=wl.scale, slice_len=256, softcap=5.0)
    gml = dev.part_ml.double().cpu().numpy()
    gpo = dev.part_o.double().cpu().numpy()
    for b in range(2):
        ns_b = -(-int(wl.kv_len[b]) // 256)
        m2 = gml[b, :, :, :ns_b, 0]
        ref_m2 = pm[b, :, :, :ns_b]
        assert np.array_equal(np.isneginf(m2), np.isneginf(ref_m2))
        fin = np.isfinite(ref_m2)
        # the running max carries the bf16 rounding of Q (relative 2^-9 of |s|)
        assert np.abs(m2[fin] - ref_m2[fin]).max() < 5e-2
        # o / l is the slice's own normalised output
        gl = gml[b, :, :, :ns_b, 1]
        rl = pl[b, :, :, :ns_b]
        nz = rl > 0
        nmse_check(gpo[b, :, :, :ns_b][nz] / gl[nz][:, None], po[b][:, :, :ns_b][nz] / rl[nz][:, None],
                   5e-5, "partials")


def test_decode_deterministic_and_poison_immune():
    wl = gen.make_decode(seed=6, n_stream=2, n_row=4, n_head_q=32, n_head_kv=4, head_dim=256,
                         cap=2100, kv_dtype="bf16", depths=[2100, 1025], slice_len=1024)
    ref = hip_run.run_decode(wl)
    for _ in range(2):
        again = hip_run.run_decode(wl)
        assert ref.tobytes() == again.tobytes()
    # NaN in every cell no row can see (past kv_len) changes nothing
    k, v = wl.k.copy(), wl.v.copy()
    k[1, 1025:] = 0x7FC0
    v[1, 1025:] = 0x7FC0
    wl.k, wl.v = k, v
    poisoned = hip_run.run_decode(wl)
    assert ref.tobytes() == poisoned.tobytes()


def test_decode_slice_size_invariance():
    wl = gen.make_decode(seed=8, n_stream=2, n_row=1, n_head_q=32, n_head_kv=4, head_dim=256,
                         cap=4100, kv_dtype="bf16", depths=[4100, 2049], slice_len=1024)
    ref = oracle_decode(wl)
    for L in (256, 1024, 2048, 4100):
        nmse_check(hip_run.run_decode(wl, slice_len=L), ref, TOL["bf16"], f"slice {L}")


@pytest.mark.parametrize("depth", [33, 34, 1023, 1024, 1025, 8193])
def test_decode_boundary_depths(depth):
    wl = gen.make_decode(seed=[9, depth], n_stream=1, n_row=16, n_head_q=48, n_head_kv=4,
                         head_dim=256, cap=depth, kv_dtype="i8", depths=[depth], slice_len=1024)
    nmse_check(hip_run.run_decode(wl), oracle_decode(wl), TOL["i8"], f"depth {depth}")


def test_decode_empty_rows_are_zero():
    # kv_len 0 and kv_len < n_row: rows with nothing visible give exact +0.0
    wl = gen.make_decode(seed=10, n_stream=3, n_row=4, n_head_q=8, n_head_kv=2, head_dim=128,
                         cap=64, kv_dtype="bf16", depths=[0, 2, 64], slice_len=32)
    out = hip_run.run_decode(wl)
    ref = oracle_decode(wl)
    nmse_check(out, ref, TOL["bf16"], "empty rows")
    assert np.all(out[0] == 0) and not np.signbit(out[0]).any()
    assert np.all(out[1, :2] == 0)


@pytest.mark.parametrize("kind", ["one_block_bf16", "work_group_bf16", "work_group_i8", "work_group_fp8"])
def test_decode_nan_propagation(kind):
    """A NaN key element (or int8 key scale) makes exactly the query vectors that
    see that key NaN; causal rows that cannot see it stay finite."""
    shapes = {"one_block_bf16": dict(n_row=1, n_head_q=8, kv_dtype="bf16"),
              "work_group_bf16": dict(n_row=6, n_head_q=16, kv_dtype="bf16"),
              "work_group_i8": dict(n_row=6, n_head_q=24, kv_dtype="i8"),
              "work_group_fp8": dict(n_row=6, n_head_q=24, kv_dtype="fp8")}[kind]
    wl = gen.make_decode(seed=[12, len(kind)], n_stream=2, n_head_kv=2, head_dim=128, cap=700,
                         depths=[700, 500], slice_len=256, **shapes)
    R, G = wl.n_row, wl.n_head_q // wl.n_head_kv
    k = wl.k.copy()
    ks = None if wl.k_scale is None else wl.k_scale.copy()
    for b, cell, g in [(0, 300, 1), (1, 497, 0)]:
        if wl.kv_dtype == "i8":
            ks[b, cell, g] = np.nan                # int8 has no NaN: a NaN row scale
        elif wl.kv_dtype == "fp8":
            k[b, cell, g, 5] = 0x7F                # the e4m3 NaN code
        else:
            k[b, cell, g, 5] = 0x7FC0
    wl.k, wl.k_scale = k, ks
    out = hip_run.run_decode(wl)
    nmse_check(out, oracle_decode(wl), TOL[wl.kv_dtype], kind)
    assert np.isnan(out[0, :, G:2 * G]).all() and np.isfinite(out[0, :, :G]).all()
    # stream 1: row r sits at 500 - R + r and sees cell 497 iff 497 <= 500 - R + r
    for r in range(R):
        sees = 497 <= 500 - R + r
        assert np.isnan(out[1, r, :G]).all() == sees and np.isfinite(out[1, r, :G]).all() != sees
        assert np.isfinite(out[1, r, G:]).all()


# ----------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------

def sel_small(seed=11, dtype="bf16", **over):
    kw = dict(n_row=40, n_head_q=16, n_head_kv=2, head_dim=256, n_kv=3001, kv_dtype=dtype,
              n_sel=128, n_dup=6, n_invalid=3, block_size=4, first_pos=2000)
    kw.update(over)
    return gen.make_prefill_sel(seed=seed, **kw)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "i8", "fp8"])
def test_prefill_selection_parity(dtype):
    wl = sel_small(dtype=dtype)
    out, dev = hip_run.run_prefill(wl, dbg=True, return_dev=True)
    nmse_check(out, oracle_prefill(wl), TOL[dtype], f"sel {dtype}")
    cells, ids = oracle.visited_prefill(n_kv=wl.n_kv, n_head_kv=wl.n_head_kv, sel=wl.sel,
                                        block_size=wl.block_size)
    dsel = dev.dbg_sel.cpu().numpy()
    dv = dev.dbg.cpu().numpy()
    for r in range(wl.n_row):
        for g in range(wl.n_head_kv):
            n = int(dsel[r, g, 0])
            assert n == ids[r].size
            assert np.array_equal(dsel[r, g, 1:1 + n], ids[r])
            c = cells[r]
            assert dv[r, g, 0].tolist() == [c.size, int(c.sum()), int((c * c).sum())]


@pytest.mark.parametrize("head_dim,n_kv,bs", [
    (128, 32768, 1),     # 32768 blocks: the largest list the LDS block bitmap takes at D = 128
    (128, 32769, 1),     # one block more: the sorting-network path
    (256, 70001, 1),     # past the bitmap at D = 256 too
    (256, 40000, 3),     # a partial last block
])
def test_prefill_selection_block_counts(head_dim, n_kv, bs):
    """Both ways of ordering a row's ids (an LDS bitmap over the blocks when it fits,
    else a sorting network) give the oracle's sorted unique ids and outputs."""
    wl = sel_small(seed=[18, n_kv], dtype="bf16", n_row=8, head_dim=head_dim, n_kv=n_kv,
                   n_sel=300, n_dup=15, n_invalid=6, block_size=bs, first_pos=n_kv - 8)
    sel = wl.sel.copy()
    last = (n_kv + bs - 1) // bs - 1
    sel[0, :4] = [last, last, last + 1, 0]          # the last valid block, its repeat, the first invalid
    wl.sel = sel
    out, dev = hip_run.run_prefill(wl, dbg=True, return_dev=True)
    nmse_check(out, oracle_prefill(wl), TOL["bf16"], f"sel blocks {n_kv}/{bs}")
    _, ids = oracle.visited_prefill(n_kv=wl.n_kv, n_head_kv=wl.n_head_kv, sel=wl.sel,
                                    block_size=wl.block_size)
    dsel = dev.dbg_sel.cpu().numpy()
    for r in range(wl.n_row):
        for g in range(wl.n_head_kv):
            n = int(dsel[r, g, 0])
            assert n == ids[r].size and np.array_equal(dsel[r, g, 1:1 + n], ids[r]), (r, g)


def test_prefill_selection_fp32_is_refused():
    # selection mode runs on the matrix-core kernel only; fp32 K/V is refused
    import split_flash_attention_amd as sa
    wl = sel_small(dtype="f32", n_row=2)
    with pytest.raises(sa.SelAttnError) as e:
        hip_run.run_prefill(wl)
    assert e.value.status == sa.EUNSUPPORTED


def test_prefill_selection_features_and_poison():
    wl = sel_small(seed=12, n_row=24, n_head_q=8, n_head_kv=1, head_dim=128, n_kv=1999,
                   block_size=3, softcap=20.0, alibi=True)
    ref = oracle_prefill(wl)
    out = hip_run.run_prefill(wl)
    nmse_check(out, ref, TOL["bf16"], "sel softcap+alibi")
    # poison every cell no row selects
    cells, _ = oracle.visited_prefill(n_kv=wl.n_kv, n_head_kv=1, sel=wl.sel, block_size=3)
    used = np.zeros(wl.n_kv, bool)
    for c in cells:
        used[c] = True
    k, v = wl.k.copy(), wl.v.copy()
    k[~used] = 0x7FC0
    v[~used] = 0x7FC0
    wl.k, wl.v = k, v
    assert hip_run.run_prefill(wl).tobytes() == out.tobytes()
    # permuting each list gives bit-identical output
    rng = np.random.default_rng(1)
    wl.sel = np.stack([r[rng.permutation(r.size)] for r in wl.sel])
    assert hip_run.run_prefill(wl).tobytes() == out.tobytes()


def test_prefill_selection_edge_lists():
    wl = sel_small(seed=13, n_row=6, n_sel=20, n_dup=0, n_invalid=0)
    sel = wl.sel.copy()
    sel[0] = -1                      # all invalid -> +0.0
    sel[1] = 750                     # one id repeated -> 4 cells
    sel[2, :] = 750
    sel[2, 5] = 751                  # last block of N=3001: cell 3000 only ... and 3004 is past N
    sel[3] = np.arange(20) * 37
    wl.sel = sel.astype(np.int32)
    out = hip_run.run_prefill(wl)
    ref = oracle_prefill(wl)
    nmse_check(out, ref, TOL["bf16"], "edge lists")
    assert np.all(out[0] == 0)


@pytest.mark.parametrize("case", ["max_list", "one_id", "big_blocks", "all_repeats", "unsorted_edges"])
def test_prefill_selection_list_extremes(case):
    """List shapes at the edges of the API: 4096 ids (the maximum), a single id,
    64-cell blocks with a partial last block, one id repeated 4096 times, and a
    list that names the first and last blocks among invalid ids of both kinds."""
    if case == "max_list":
        wl = sel_small(seed=22, n_row=6, n_kv=30000, n_sel=4096, n_dup=200, n_invalid=96,
                       block_size=4, first_pos=29990)
    elif case == "one_id":
        wl = sel_small(seed=23, n_row=6, n_sel=1, n_dup=0, n_invalid=0)
    elif case == "big_blocks":
        wl = sel_small(seed=24, n_row=6, n_kv=3001, n_sel=30, n_dup=3, n_invalid=2, block_size=64,
                       first_pos=2990)
    elif case == "all_repeats":
        wl = sel_small(seed=25, n_row=4, n_sel=8, n_dup=0, n_invalid=0)
        wl.sel = np.repeat(np.array([[7], [0], [500], [250]], np.int32), 4096, axis=1)
    else:
        wl = sel_small(seed=26, n_row=4, n_sel=16, n_dup=0, n_invalid=0)
        n_blocks = -(-wl.n_kv // wl.block_size)
        sel = np.full((4, 16), -1, np.int32)
        sel[:, 3] = n_blocks - 1
        sel[:, 7] = 0
        sel[:, 9] = n_blocks                       # one past the last valid block
        sel[:, 11] = np.iinfo(np.int32).max        # far past the cache
        sel[:, 12] = np.iinfo(np.int32).min
        wl.sel = sel
    out, dev = hip_run.run_prefill(wl, dbg=True, return_dev=True)
    nmse_check(out, oracle_prefill(wl), TOL["bf16"], case)
    _, ids = oracle.visited_prefill(n_kv=wl.n_kv, n_head_kv=wl.n_head_kv, sel=wl.sel,
                                    block_size=wl.block_size)
    dsel = dev.dbg_sel.cpu().numpy()
    for r in range(wl.n_row):
        n = int(dsel[r, 0, 0])
        assert n == ids[r].size and np.array_equal(dsel[r, 0, 1:1 + n], ids[r]), (case, r)


def test_prefill_selection_splits():
    wl = sel_small(seed=14, n_row=16)
    ref = oracle_prefill(wl)
    for n in (2, 5):
        nmse_check(hip_run.run_prefill(wl, n_splits=n), ref, TOL["bf16"], f"splits {n}")


@pytest.mark.parametrize("gqa", [(16, 4), (16, 2), (48, 4)])
@pytest.mark.parametrize("n_splits", [1, 7, 16])
def test_selected_key_decode(gqa, n_splits):
    """Decode-shaped selection calls (16 rows, head dim 256, GQA 4 / 8 / 12): the key
    range split over n_splits work-groups per row, partials merged by the combine;
    each split visits exactly its share of the row's selected cells."""
    hq, hkv = gqa
    wl = gen.make_prefill_sel(seed=[21, hq // hkv, n_splits], n_row=16, n_head_q=hq, n_head_kv=hkv,
                              head_dim=256, n_kv=3001, kv_dtype="bf16", n_sel=96, n_dup=9,
                              n_invalid=5, block_size=4, first_pos=2985)
    sel = wl.sel.copy()
    sel[3] = -1                                   # a row with nothing valid
    sel[5, :] = sel[5, 0]                         # a row with one block, repeated
    wl.sel = sel
    out, dev = hip_run.run_prefill(wl, n_splits=n_splits, dbg=True, return_dev=True)
    ref = oracle_prefill(wl)
    nmse_check(out, ref, TOL["bf16"], f"sel decode {gqa} splits {n_splits}")
    assert np.all(out[3] == 0) and not np.signbit(out[3]).any()
    # per split: the cells combined are the row's cells inside the split's range
    cells, _ = oracle.visited_prefill(n_kv=wl.n_kv, n_head_kv=hkv, sel=wl.sel,
                                      block_size=wl.block_size, rows=list(range(16)))
    step = -(-wl.n_kv // n_splits)
    dv = dev.dbg.cpu().numpy()
    for r in range(16):
        for t in range(n_splits):
            c = cells[r][(cells[r] >= t * step) & (cells[r] < (t + 1) * step)]
            for g in range(hkv):
                assert dv[r, g, t].tolist() == [c.size, int(c.sum()), int((c * c).sum())], (r, g, t)


def mask_small(nan=True, seed=15, **over):
    kw = dict(n_row=48, n_head_q=16, n_head_kv=4, head_dim=128, n_kv=700, kv_dtype="f16",
              causal=True, excluded_rows=3, nan_k=40 if nan else 0, softcap=30.0, alibi=True)
    kw.update(over)
    return gen.make_prefill_mask(seed=seed, **kw)


def test_prefill_mask_semantics():
    wl = mask_small(nan=True)
    out, dev = hip_run.run_prefill(wl, dbg=True, return_dev=True)
    ref = oracle_prefill(wl)
    nmse_check(out, ref, TOL["f16"], "mask with NaN")
    ex = wl.meta["excluded_rows"]
    assert np.all(out[ex] == 0) and not np.signbit(out[ex]).any()
    cells, _ = oracle.visited_prefill(n_kv=wl.n_kv, n_head_kv=4, q_pos=wl.q_pos, mask=wl.mask,
                                      causal=True)
    dv = dev.dbg.cpu().numpy()
    for r in range(wl.n_row):
        c = cells[r]
        for g in range(4):
            assert dv[r, g, 0].tolist() == [c.size, int(c.sum()), int((c * c).sum())]


def test_prefill_mask_softcap_then_alibi():
    """A soft cap of 2 with ALiBi slopes down to 2^-8: scores of order 1 and biases
    of order 1 to 10, so capping before the bias (the pages' order) and after it
    give different weights on keys that carry real weight."""
    wl = mask_small(nan=False, softcap=2.0, excluded_rows=0)
    nmse_check(hip_run.run_prefill(wl), oracle_prefill(wl), TOL["f16"], "softcap then ALiBi")


def test_prefill_mask_control_without_nan():
    wl = mask_small(nan=False)
    nmse_check(hip_run.run_prefill(wl), oracle_prefill(wl), TOL["f16"], "mask control")


@pytest.mark.parametrize("dtype", ["bf16", "f32", "i8", "fp8"])
def test_prefill_mask_dtypes_and_splits(dtype):
    wl = mask_small(nan=False, seed=16, kv_dtype=dtype, head_dim=256, n_row=20, n_kv=333,
                    softcap=0.0, alibi=False, excluded_rows=1)
    ref = oracle_prefill(wl)
    nmse_check(hip_run.run_prefill(wl), ref, TOL[dtype], f"mask {dtype}")
    nmse_check(hip_run.run_prefill(wl, n_splits=3), ref, TOL[dtype], f"mask {dtype} split")


def test_valu_nan_propagation():
    """fp32 K/V run on the vector-ALU kernel: NaN keys make exactly the query vectors
    that see them NaN, in mask-mode prefill and in decode."""
    wl = mask_small(nan=True, seed=19, kv_dtype="f32", n_row=24, n_kv=300, head_dim=64)
    nmse_check(hip_run.run_prefill(wl), oracle_prefill(wl), TOL["f32"], "vector-ALU mask with NaN")
    wl = gen.make_decode(seed=20, n_stream=2, n_row=3, n_head_q=8, n_head_kv=2, head_dim=64, cap=100,
                         kv_dtype="f32", depths=[100, 60], slice_len=32)
    k = wl.k.copy()
    k[0, 40, 1, 3] = np.nan
    k[1, 58, 0, 0] = np.nan                       # seen by rows 1 and 2 of stream 1 only
    wl.k = k
    out = hip_run.run_decode(wl)
    nmse_check(out, oracle_decode(wl), TOL["f32"], "vector-ALU decode with NaN")
    assert np.isfinite(out[1, 0]).all() and np.isnan(out[1, 1:, :4]).all()


def test_finite_sentinel_and_bias_range_on_gpu():
    # the PR #910 controls at kernel level: a -1e30 row gives the uniform mean of V,
    # biases 100000/100001 give e/(1+e) weights (no F16 clamp)
    wl = mask_small(nan=False, seed=17, n_row=4, n_kv=64, softcap=0.0, alibi=False,
                    excluded_rows=0, causal=False)
    wl.mask[0, :] = -1e30
    wl.mask[1, :] = -np.finfo(np.float32).max
    wl.mask[2, :] = -np.inf
    wl.mask[2, 0], wl.mask[2, 1] = 100000.0, 100001.0
    nmse_check(hip_run.run_prefill(wl), oracle_prefill(wl), TOL["f16"], "sentinels")
