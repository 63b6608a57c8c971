"""GPU parity of tree-shaped verify windows and of the attention-sink logit.

Tree windows (TensorFold PR #2595, "Kernel contract": tree widths 1, 2, 4, 8,
12, 16 with heap-order parents at 33, 34, 8193 and 32768..32770 visible keys):
every decode kernel family (single wave, work-group, vector ALU, and the
general kernel that takes caches past 32-bit byte offsets) against the oracle,
with the visited cells of every (row, slice) compared exactly.

Sink logit (HartsyInference PR #910, review of the CPU fix): through the split
combine after decode, and in the unsplit epilogue of every prefill kernel,
with -inf, +inf, NaN and dominant sinks and with empty rows.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import split_flash_attention_amd as sa
from tests import hip_run
from tests.test_gpu_parity import TOL, nmse_check
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    sa.lib()


def oracle_decode(wl):
    return oracle.decode(q=wl.q, k=wl.k, v=wl.v, kv_dtype=wl.kv_dtype, kv_len=wl.kv_len,
                         causal=wl.causal, scale=wl.scale, softcap=wl.softcap, alibi=wl.alibi,
                         k_scale=wl.k_scale, v_scale=wl.v_scale, tree_parent=wl.tree_parent,
                         sinks=wl.sinks)


def oracle_prefill(wl, n_splits=1):
    kw = dict(q=wl.q, k=wl.k, v=wl.v, kv_dtype=wl.kv_dtype, scale=wl.scale, softcap=wl.softcap,
              alibi=wl.alibi, q_pos=wl.q_pos, sel=wl.sel, block_size=wl.block_size, mask=wl.mask,
              causal=wl.causal, k_scale=wl.k_scale, v_scale=wl.v_scale, sinks=wl.sinks)
    return oracle.prefill(**kw) if n_splits == 1 else oracle.prefill_split(n_splits=n_splits, **kw)


def check_visited(wl, dev, what):
    st = oracle.visited_decode(kv_len=wl.kv_len, n_row=wl.n_row, causal=wl.causal,
                               slice_len=dev.slice_len, n_head_kv=wl.n_head_kv,
                               tree_parent=wl.tree_parent)
    got = dev.dbg.cpu().numpy()
    for b in range(wl.n_stream):
        ns_b = -(-int(wl.kv_len[b]) // dev.slice_len)
        assert np.array_equal(got[b, :, :, :ns_b], st[b, :, :, :ns_b]), (what, b)


# ----------------------------------------------------------------------------
# tree windows
# ----------------------------------------------------------------------------

TREE_CASES = {
    # up to 16 query vectors per unit: the single-wave kernel
    "bf16_heap_w2_gqa8": dict(n_stream=2, n_row=2, n_head_q=16, n_head_kv=2, head_dim=256,
                              cap=1500, kv_dtype="bf16", depths=[1500, 40], slice_len=512,
                              tree="heap"),
    "f16_random_w4_softcap_alibi_d128": dict(n_stream=2, n_row=4, n_head_q=8, n_head_kv=2,
                                             head_dim=128, cap=900, kv_dtype="f16",
                                             depths=[900, 5], slice_len=256, tree="random",
                                             softcap=25.0, alibi=True),
    "fp8_heap_w1_gqa8": dict(n_stream=2, n_row=1, n_head_q=16, n_head_kv=2, head_dim=256,
                             cap=700, kv_dtype="fp8", depths=[700, 1], slice_len=256, tree="heap"),
    # more: the work-group kernel with 8 and 12 waves and two query chunks
    "bf16_heap_w16_gqa8_softcap_alibi": dict(n_stream=3, n_row=16, n_head_q=16, n_head_kv=2,
                                             head_dim=256, cap=2100, kv_dtype="bf16",
                                             depths=[2100, 700, 17], slice_len=1024, tree="heap",
                                             softcap=10.0, alibi=True),
    "i8_random_w12_gqa12": dict(n_stream=2, n_row=12, n_head_q=48, n_head_kv=4, head_dim=256,
                                cap=1300, kv_dtype="i8", depths=[1300, 12], slice_len=512,
                                tree="random"),
    "fp8_heap_w8_gqa12_d128": dict(n_stream=2, n_row=8, n_head_q=24, n_head_kv=2, head_dim=128,
                                   cap=900, kv_dtype="fp8", depths=[900, 333], slice_len=256,
                                   tree="heap"),
    "bf16_random_w64": dict(n_stream=2, n_row=64, n_head_q=4, n_head_kv=1, head_dim=128,
                            cap=800, kv_dtype="bf16", depths=[800, 64], slice_len=256,
                            tree="random"),
    # 64 rows x 8 heads = 512 query vectors: the work-group kernel in several query chunks
    "bf16_random_w64_gqa8_chunks": dict(n_stream=2, n_row=64, n_head_q=16, n_head_kv=2, head_dim=128,
                                        cap=700, kv_dtype="bf16", depths=[700, 70], slice_len=256,
                                        tree="random"),
    # caches shorter than the window: nodes before cell 0 do not exist
    "i8_heap_w16_short_caches": dict(n_stream=3, n_row=16, n_head_q=48, n_head_kv=4, head_dim=256,
                                     cap=40, kv_dtype="i8", depths=[40, 9, 1], slice_len=32,
                                     tree="heap"),
    # fp32 K/V: the vector-ALU kernel
    "f32_random_w8_d64": dict(n_stream=2, n_row=8, n_head_q=8, n_head_kv=2, head_dim=64,
                              cap=100, kv_dtype="f32", depths=[100, 8], slice_len=32,
                              tree="random"),
    # the tree replaces the causal flag: the same windows with causal off
    "bf16_random_w8_noncausal_flag": dict(n_stream=2, n_row=8, n_head_q=16, n_head_kv=2,
                                          head_dim=128, cap=600, kv_dtype="bf16", depths=[600, 50],
                                          slice_len=256, tree="random", causal=False),
}


@pytest.mark.parametrize("name", sorted(TREE_CASES))
def test_tree_decode_parity(name):
    wl = gen.make_decode(seed=[81, len(name)], **TREE_CASES[name])
    print(f"tree case {name}", flush=True)
    out, dev = hip_run.run_decode(wl, dbg=True, return_dev=True)
    nmse_check(out, oracle_decode(wl), TOL[wl.kv_dtype], name)
    check_visited(wl, dev, name)


@pytest.fixture(scope="module")
def gate_base():
    """bf16 caches at the gate's visible-key counts, one stream each, 16 rows of Q."""
    return gen.make_decode(seed=82, n_stream=6, n_row=16, n_head_q=16, n_head_kv=2, head_dim=256,
                           cap=32770, kv_dtype="bf16", depths=[33, 34, 8193, 32768, 32769, 32770],
                           slice_len=1024)


@pytest.mark.parametrize("width", [1, 2, 4, 8, 12, 16])
def test_tree_gate_widths(gate_base, width):
    wl = dataclasses.replace(gate_base, q=np.ascontiguousarray(gate_base.q[:, :width]), n_row=width,
                             tree_parent=np.tile(gen.heap_parents(width), (6, 1)))
    print(f"tree gate width {width}", flush=True)
    out, dev = hip_run.run_decode(wl, dbg=True, return_dev=True)
    nmse_check(out, oracle_decode(wl), TOL["bf16"], f"width {width}")
    check_visited(wl, dev, f"width {width}")
    # the chain table gives the causal window bit for bit
    if width > 1:
        chain = dataclasses.replace(wl, tree_parent=np.tile(gen.chain_parents(width), (6, 1)))
        causal = dataclasses.replace(wl, tree_parent=None, causal=True)
        assert hip_run.run_decode(chain).tobytes() == hip_run.run_decode(causal).tobytes()


def test_tree_decode_past_32bit_offsets():
    """A cache declared with cap * cell bytes past 2^31 runs on the general kernel; only
    the cells below kv_len exist in memory (the library never reads past them)."""
    wl = gen.make_decode(seed=83, n_stream=2, n_row=6, n_head_q=8, n_head_kv=2, head_dim=128,
                         cap=1200, kv_dtype="bf16", depths=[1200, 300], slice_len=512,
                         tree="random", sinks="draw")
    dev = hip_run.DecodeDev(wl)
    cell_bytes = wl.n_head_kv * wl.head_dim * 2
    big_cap = (1 << 31) // cell_bytes + 1000
    ns = -(-big_cap // dev.slice_len)
    S, R, Hq, D = wl.q.shape
    dev.part_o = torch.full((S, R, Hq, ns, D), float("nan"), dtype=torch.float32, device=dev.device)
    dev.part_ml = torch.full((S, R, Hq, ns, 2), float("nan"), dtype=torch.float32, device=dev.device)
    dev.ns = ns
    a = dev.args(dbg=True)
    a.cap = big_cap
    c = dev.combine_args()
    c.cap = big_cap
    assert sa.decode_path(a) == 1
    print("general decode kernel, cap", big_cap, flush=True)
    sa.sel_attn_decode(a)
    sa.sel_attn_split_combine(c)
    torch.cuda.synchronize()
    out = dev.out.double().cpu().numpy()
    nmse_check(out, oracle_decode(wl), TOL["bf16"], "past 32-bit offsets")
    check_visited(wl, dev, "past 32-bit offsets")


def test_tree_rejects_more_than_64_rows():
    wl = gen.make_decode(seed=84, n_stream=1, n_row=65, n_head_q=2, n_head_kv=1, head_dim=128,
                         cap=100, kv_dtype="bf16", depths=[100], slice_len=64, tree="heap")
    dev = hip_run.DecodeDev(wl)
    a = dev.args()
    assert not sa.supports(sa.OP_DECODE, a)
    with pytest.raises(sa.SelAttnError):
        sa.sel_attn_decode(a)


# ----------------------------------------------------------------------------
# sink logit
# ----------------------------------------------------------------------------

def special_sinks(n_head, seed):
    s = gen.draw_sinks(np.random.default_rng(seed), n_head)
    s[0], s[1], s[2] = -np.inf, np.inf, np.nan
    s[3] = 40.0                      # far above every score: the output nearly vanishes
    return s


SINK_DECODE_CASES = {
    "one_block_bf16": dict(n_row=1, n_head_q=16, n_head_kv=2, head_dim=256, kv_dtype="bf16"),
    "work_group_i8": dict(n_row=8, n_head_q=16, n_head_kv=2, head_dim=256, kv_dtype="i8"),
    "work_group_fp8_tree": dict(n_row=8, n_head_q=24, n_head_kv=2, head_dim=128, kv_dtype="fp8",
                                tree="heap"),
    "valu_f32": dict(n_row=3, n_head_q=8, n_head_kv=2, head_dim=64, kv_dtype="f32"),
}


@pytest.mark.parametrize("name", sorted(SINK_DECODE_CASES))
def test_sink_decode(name):
    kw = SINK_DECODE_CASES[name]
    wl = gen.make_decode(seed=[85, len(name)], n_stream=3, cap=1100, depths=[1100, 2, 0],
                         slice_len=256, sinks=special_sinks(kw["n_head_q"], 86), **kw)
    print(f"sink decode {name}", flush=True)
    out = hip_run.run_decode(wl)
    ref = oracle_decode(wl)
    nmse_check(out, ref, TOL[wl.kv_dtype], name)
    # heads with a +inf or NaN sink are NaN everywhere; empty rows are +0.0 otherwise
    assert np.isnan(out[:, :, 1:3]).all()
    assert np.all(out[2][:, [0, 3]] == 0) and not np.signbit(out[2][:, [0, 3]]).any()
    # the -inf sink changes nothing
    plain = dataclasses.replace(wl, sinks=None)
    assert hip_run.run_decode(plain)[:, :, 0].tobytes() == out[:, :, 0].tobytes()


def sel_sink(dtype="bf16"):
    wl = gen.make_prefill_sel(seed=87, n_row=24, n_head_q=16, n_head_kv=2, head_dim=256,
                              n_kv=2100, kv_dtype=dtype, n_sel=96, n_dup=4, n_invalid=3,
                              block_size=4, first_pos=1500)
    wl.sinks = special_sinks(16, 88)
    return wl


def mask_sink(dtype="f16"):
    wl = gen.make_prefill_mask(seed=89, n_row=32, n_head_q=16, n_head_kv=4, head_dim=128,
                               n_kv=600, kv_dtype=dtype, causal=True, excluded_rows=3,
                               softcap=30.0, alibi=True)
    wl.sinks = special_sinks(16, 90)
    return wl


@pytest.mark.parametrize("kind", ["sel_bf16", "sel_i8", "mask_f16", "mask_bf16", "mask_f32"])
@pytest.mark.parametrize("n_splits", [1, 4])
def test_sink_prefill(kind, n_splits):
    mode, dtype = kind.split("_")
    wl = sel_sink(dtype) if mode == "sel" else mask_sink(dtype)
    print(f"sink prefill {kind} splits {n_splits}", flush=True)
    out = hip_run.run_prefill(wl, n_splits=n_splits)
    nmse_check(out, oracle_prefill(wl), TOL[dtype], f"{kind} / {n_splits}")
    assert np.isnan(out[:, 1:3]).all()
    if mode == "mask":
        ex = wl.meta["excluded_rows"]
        assert np.all(out[ex][:, [0, 3]] == 0) and not np.signbit(out[ex][:, [0, 3]]).any()
