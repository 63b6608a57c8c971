"""Pins for the FP64 oracle: values fixed by the pages and by mathematics.

Each pin is a function of the oracle module so that the planted-mistake tests
at the end can re-run it against a deliberately broken oracle (monkeypatched on
the CPU) and show it goes red.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.attention as OA
from oracle import brute
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _mask_prefill(q, k, v, mask, *, scale, softcap=0.0, alibi=None, q_pos=None, causal=False,
                  dtype="f32"):
    return oracle.prefill(q=q, k=k, v=v, kv_dtype=dtype, scale=scale, softcap=softcap,
                          alibi=alibi, q_pos=q_pos, mask=mask, causal=causal)


def _sel_prefill(q, k, v, sel, *, scale, block_size=1, softcap=0.0, alibi=None, q_pos=None,
                 dtype="f32"):
    return oracle.prefill(q=q, k=k, v=v, kv_dtype=dtype, scale=scale, softcap=softcap,
                          alibi=alibi, q_pos=q_pos, sel=sel, block_size=block_size)


# ----------------------------------------------------------------------------
# pins written from the pages' examples
# ----------------------------------------------------------------------------

def pin_m03_excluded_row():
    g = _load("m03_excluded_row.json")
    q = np.array(g["q"], np.float32)[0].transpose(1, 0, 2)       # [rows][heads][D]
    k = np.array(g["k"], np.float32)[0].transpose(1, 0, 2)       # [keys][kvheads][D]
    v = np.full_like(k, g["v_fill"])
    mask = np.array([[float(x) for x in row] for row in g["bias"]], np.float32)
    out = _mask_prefill(q, k, v, mask, scale=g["scale"])
    exp = np.array(g["expected"], np.float64)[0].transpose(1, 0, 2)
    assert np.array_equal(out, exp), out
    assert not np.signbit(out).any(), "excluded row must be +0.0"


def pin_softcap_before_alibi():
    g = _load("softcap_alibi_order.json")
    q = np.array([[[1.0]]], np.float32)
    k = np.zeros((29, 1, 1), np.float32)
    v = np.zeros((29, 1, 1), np.float32)
    k[0, 0, 0] = 60.0
    v[0, 0, 0] = 1.0
    sel = np.array([[0, 28]], np.int32)
    out = _sel_prefill(q, k, v, sel, scale=1.0, softcap=30.0,
                       alibi=np.array([1.0], np.float32), q_pos=np.array([28], np.int32))
    assert abs(out[0, 0, 0] - g["expected_output"]) < 1e-14, out
    # independent closed form, worked by hand
    s_a = 30.0 * math.tanh(2.0) - 28.0
    assert abs(out[0, 0, 0] - 1.0 / (1.0 + math.exp(-s_a))) < 1e-14


def pin_bias_range():
    g = _load("bias_range.json")
    D = 3
    q = np.ones((1, 1, D), np.float32)
    k = np.zeros((2, 1, D), np.float32)
    v = np.stack([np.zeros((1, D)), np.ones((1, D))]).astype(np.float32)
    mask = np.array([[100000.0, 100001.0]], np.float32)
    out = _mask_prefill(q, k, v, mask, scale=1.0)
    assert np.allclose(out, g["expected_output"], rtol=0, atol=1e-15), out
    assert abs(out[0, 0, 0] - math.e / (1.0 + math.e)) < 1e-15


def pin_finite_sentinel():
    # nonzero dots (the review's point that tests only produced zero scores)
    rng = np.random.default_rng(7)
    for sentinel in (-1e30, -np.finfo(np.float32).max):
        q = rng.standard_normal((1, 2, 8)).astype(np.float32)
        k = rng.standard_normal((5, 1, 8)).astype(np.float32)
        v = rng.standard_normal((5, 1, 8)).astype(np.float32)
        mask = np.full((1, 5), sentinel, np.float32)
        out = _mask_prefill(q, k, v, mask, scale=0.5)
        mean = v[:, 0].astype(np.float64).mean(axis=0)
        assert np.allclose(out[0, 0], mean, rtol=1e-14, atol=1e-15)
        assert np.allclose(out[0, 1], mean, rtol=1e-14, atol=1e-15)


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def pin_one_key_returns_v():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 4, 16)).astype(np.float32)
    k = rng.standard_normal((9, 2, 16)).astype(np.float32)
    v = rng.standard_normal((9, 2, 16)).astype(np.float32)
    out = _sel_prefill(q, k, v, np.array([[5]], np.int32), scale=0.25)
    for h in range(4):
        assert np.array_equal(out[0, h], v[5, h // 2].astype(np.float64))


def pin_zero_query_mean():
    rng = np.random.default_rng(12)
    S, R, Hq, Hkv, D, cap = 2, 3, 4, 2, 8, 10
    q = np.zeros((S, R, Hq, D), np.float32)
    k = rng.standard_normal((S, cap, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((S, cap, Hkv, D)).astype(np.float32)
    kv_len = np.array([7, 10], np.int32)
    out = oracle.decode(q=q, k=k, v=v, kv_dtype="f32", kv_len=kv_len, causal=True, scale=1.0)
    for b in range(S):
        for r in range(R):
            lim = kv_len[b] - R + r + 1
            for h in range(Hq):
                mean = v[b, :lim, h // 2].astype(np.float64).mean(axis=0)
                assert np.allclose(out[b, r, h], mean, rtol=1e-13, atol=1e-15)


def pin_two_key_logistic():
    # scores a and b: weight of key 1 = 1 / (1 + exp(a - b))
    q = np.array([[[1.0, 2.0]]], np.float32)
    k = np.array([[[0.5, 0.25]], [[-1.0, 0.75]]], np.float32)
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]], np.float32)
    out = _mask_prefill(q, k, v, np.zeros((1, 2), np.float32), scale=0.5)
    a = 0.5 * (0.5 + 0.5)
    b = 0.5 * (-1.0 + 1.5)
    w1 = 1.0 / (1.0 + math.exp(a - b))
    assert abs(out[0, 0, 1] - w1) < 1e-15 and abs(out[0, 0, 0] - (1 - w1)) < 1e-15


def pin_weights_sum_to_one():
    # V = 1 everywhere -> output 1 whatever the scores (sum of weights is 1)
    wl = gen.make_prefill_mask(seed=3, n_row=5, n_head_q=4, n_head_kv=2, head_dim=8, n_kv=37,
                               kv_dtype="f32", softcap=30.0, alibi=True)
    v = np.ones_like(wl.v)
    out = _mask_prefill(wl.q, wl.k, v, wl.mask, scale=wl.scale, softcap=30.0, alibi=wl.alibi,
                        q_pos=wl.q_pos, causal=True)
    assert np.allclose(out, 1.0, rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------
# reductions to library routines
# ----------------------------------------------------------------------------

def pin_scipy_softmax_dense():
    from scipy.special import softmax
    wl = gen.make_decode(seed=21, n_stream=2, n_row=1, n_head_q=6, n_head_kv=3, head_dim=16,
                         cap=40, kv_dtype="bf16", depths=[40, 23], causal=False)
    out = oracle.decode(q=wl.q, k=wl.k, v=wl.v, kv_dtype="bf16", kv_len=wl.kv_len, causal=False,
                        scale=wl.scale)
    for b in range(2):
        n = wl.kv_len[b]
        k64 = (wl.k[b, :n].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        v64 = (wl.v[b, :n].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        for h in range(6):
            s = wl.scale * (k64[:, h // 2] @ wl.q[b, 0, h].astype(np.float64))
            ref = softmax(s) @ v64[:, h // 2]
            assert np.allclose(out[b, 0, h], ref, rtol=1e-12, atol=1e-14)


def pin_torch_sdpa_mask_alibi_gqa():
    import torch
    wl = gen.make_prefill_mask(seed=22, n_row=6, n_head_q=8, n_head_kv=2, head_dim=16, n_kv=50,
                               kv_dtype="f16", causal=True, alibi=True)
    out = _mask_prefill(wl.q, wl.k, wl.v, wl.mask, scale=wl.scale, alibi=wl.alibi,
                        q_pos=wl.q_pos, causal=True, dtype="f16")
    q = torch.from_numpy(wl.q.astype(np.float64)).permute(1, 0, 2)[None]          # [1,H,R,D]
    k = torch.from_numpy(wl.k.astype(np.float64)).permute(1, 0, 2)
    v = torch.from_numpy(wl.v.astype(np.float64)).permute(1, 0, 2)
    k = k.repeat_interleave(4, dim=0)[None].contiguous()
    v = v.repeat_interleave(4, dim=0)[None].contiguous()
    j = np.arange(50)[None, :]
    bias = np.empty((8, 6, 50))
    for h in range(8):
        bias[h] = wl.mask.astype(np.float64) + wl.alibi[h] * (j - wl.q_pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=torch.from_numpy(bias)[None], scale=wl.scale)[0].permute(1, 0, 2).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# invariances
# ----------------------------------------------------------------------------

def pin_split_equals_unsplit():
    wl = gen.make_decode(seed=31, n_stream=3, n_row=4, n_head_q=4, n_head_kv=2, head_dim=8,
                         cap=21, kv_dtype="i8", depths=[21, 9, 4], causal=True, softcap=5.0,
                         alibi=True)
    kw = dict(q=wl.q, k=wl.k, v=wl.v, kv_dtype="i8", kv_len=wl.kv_len, causal=True,
              scale=wl.scale, softcap=5.0, alibi=wl.alibi, k_scale=wl.k_scale, v_scale=wl.v_scale)
    ref = oracle.decode(**kw)
    for L in range(1, 23):
        out, po, pm, pl = oracle.decode_split(slice_len=L, **kw)
        err = np.abs(out - ref).max() / np.abs(ref).max()
        assert err < 1e-13, (L, err)


def pin_split_prefill_equals_unsplit():
    wl = gen.make_prefill_sel(seed=32, n_row=3, n_head_q=4, n_head_kv=1, head_dim=8, n_kv=40,
                              kv_dtype="bf16", n_sel=9, n_dup=2, n_invalid=1, block_size=4)
    kw = dict(q=wl.q, k=wl.k, v=wl.v, kv_dtype="bf16", scale=wl.scale, q_pos=wl.q_pos,
              sel=wl.sel, block_size=4)
    ref = oracle.prefill(**kw)
    for n in (1, 2, 3, 7, 40):
        out = oracle.prefill_split(n_splits=n, **kw)
        assert np.allclose(out, ref, rtol=1e-13, atol=1e-15), n


def pin_selection_invariances():
    wl = gen.make_prefill_sel(seed=41, n_row=4, n_head_q=4, n_head_kv=2, head_dim=8, n_kv=30,
                              kv_dtype="bf16", n_sel=8, n_dup=2, n_invalid=2, block_size=3)
    kw = dict(q=wl.q, k=wl.k, v=wl.v, kv_dtype="bf16", scale=wl.scale, q_pos=wl.q_pos,
              block_size=3)
    ref = oracle.prefill(sel=wl.sel, **kw)
    rng = np.random.default_rng(0)
    perm = np.stack([row[rng.permutation(row.size)] for row in wl.sel])
    assert np.array_equal(oracle.prefill(sel=perm, **kw), ref)
    more = np.concatenate([wl.sel, wl.sel[:, :3], np.full((4, 2), -7, np.int32),
                           np.full((4, 1), 10, np.int32)], axis=1)   # id 10: cells 30..32 >= N
    assert np.array_equal(oracle.prefill(sel=more, **kw), ref)
    # selection == dense mask mode with -inf outside the visible set
    mask = np.full((4, 30), -np.inf, np.float32)
    for r in range(4):
        mask[r, oracle.visible_selection(wl.sel[r], 3, 30)] = 0.0
    dense = oracle.prefill(mask=mask, **kw)
    assert np.allclose(dense, ref, rtol=1e-14, atol=1e-16)
    # an all-cells list equals plain attention
    allc = np.tile(np.arange(10, dtype=np.int32), (4, 1))
    plain = oracle.prefill(mask=np.zeros((4, 30), np.float32), **kw)
    assert np.allclose(oracle.prefill(sel=allc, **kw), plain, rtol=1e-14, atol=1e-16)


def pin_gqa_equals_mha():
    wl = gen.make_decode(seed=51, n_stream=2, n_row=2, n_head_q=6, n_head_kv=2, head_dim=8,
                         cap=12, kv_dtype="f16", depths=[12, 7], causal=True, alibi=False)
    kw = dict(kv_dtype="f16", kv_len=wl.kv_len, causal=True, scale=wl.scale)
    ref = oracle.decode(q=wl.q, k=wl.k, v=wl.v, **kw)
    k_rep = np.repeat(wl.k, 3, axis=2)
    v_rep = np.repeat(wl.v, 3, axis=2)
    mha = oracle.decode(q=wl.q, k=k_rep, v=v_rep, **kw)
    assert np.array_equal(ref, mha)


# ----------------------------------------------------------------------------
# NaN / infinity rules
# ----------------------------------------------------------------------------

def pin_nan_rules():
    rng = np.random.default_rng(61)
    D = 4
    q = rng.standard_normal((1, 2, D)).astype(np.float32)
    k = rng.standard_normal((6, 1, D)).astype(np.float32)
    v = rng.standard_normal((6, 1, D)).astype(np.float32)
    base_mask = np.zeros((1, 6), np.float32)
    base_mask[0, 4:] = -np.inf
    ref = _mask_prefill(q, k, v, base_mask, scale=0.5)
    assert np.isfinite(ref).all()
    # NaN in an excluded key / value: no effect
    k2, v2 = k.copy(), v.copy()
    k2[4:] = np.nan
    v2[4:] = np.nan
    assert np.array_equal(_mask_prefill(q, k2, v2, base_mask, scale=0.5), ref)
    # NaN in a visible K element -> every head of that kv group is NaN
    k3 = k.copy()
    k3[1, 0, 2] = np.nan
    assert np.isnan(_mask_prefill(q, k3, v, base_mask, scale=0.5)).all()
    # NaN in one dim of a visible V -> only that dim is NaN
    v3 = v.copy()
    v3[2, 0, 1] = np.nan
    o3 = _mask_prefill(q, k, v3, base_mask, scale=0.5)
    assert np.isnan(o3[..., 1]).all() and np.isfinite(o3[..., [0, 2, 3]]).all()
    # NaN in V where the weight underflows to 0 still poisons that dim
    mask4 = base_mask.copy()
    mask4[0, 3] = -1e4
    v4 = v.copy()
    v4[3, 0, 0] = np.nan
    o4 = _mask_prefill(q, k, v4, mask4, scale=0.5)
    assert np.isnan(o4[..., 0]).all() and np.isfinite(o4[..., 1:]).all()
    # +inf score -> NaN row
    mask5 = base_mask.copy()
    mask5[0, 0] = np.inf
    assert np.isnan(_mask_prefill(q, k, v, mask5, scale=0.5)).all()
    # every visible score -inf -> +0.0
    s = np.array([[-np.inf, -np.inf]])
    o7 = OA.attend_scores(s, np.ones((2, 3)))
    assert np.array_equal(o7, np.zeros((1, 3))) and not np.signbit(o7).any()


def pin_combine_rules():
    D = 3
    o = np.array([[[1.0, 2.0, 3.0]], [[0.0, 0.0, 0.0]]])
    m = np.array([[0.5], [-np.inf]])
    l = np.array([[2.0], [0.0]])
    assert np.allclose(OA.combine_partials(o, m, l), [[0.5, 1.0, 1.5]])
    m_nan = np.array([[0.5], [np.nan]])
    assert np.isnan(OA.combine_partials(o, m_nan, l)).all()
    m_inf = np.array([[0.5], [np.inf]])
    assert np.isnan(OA.combine_partials(o, m_inf, l)).all()
    m_empty = np.array([[-np.inf], [-np.inf]])
    z = OA.combine_partials(np.zeros_like(o), m_empty, np.zeros_like(l))
    assert np.array_equal(z, np.zeros((1, D))) and not np.signbit(z).any()
    # NaN carried in a partial's value vector survives the merge
    o_nan = o.copy()
    o_nan[0, 0, 1] = np.nan
    c = OA.combine_partials(o_nan, m, l)
    assert np.isnan(c[0, 1]) and np.isfinite(c[0, [0, 2]]).all()


def pin_storage_decoding():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x3EAB], np.uint16)
    got = OA.kv_to_f64(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == np.inf
    assert got[3] == 2.0 ** -133 and got[4] == 0.333984375
    assert OA.kv_to_f64(np.array([0x3C00], np.uint16).view(np.float16), "f16")[0] == 1.0
    i8 = np.array([[-127, 0, 5]], np.int8)
    sc = np.array([0.5], np.float32)
    assert np.array_equal(OA.kv_to_f64(i8, "i8", sc), [[-63.5, 0.0, 2.5]])
    # the generator's bf16 rounding: nearest, ties to even
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9], np.float32)
    assert list(gen.f32_to_bf16_bits(x)) == [0x3F80, 0x3F82, 0x3F80]


def pin_e4m3_decoding():
    """e4m3 bytes (TensorFold PR #911: e4m3 rows, scale amax / 448): values that
    follow from the format's definition, then all 256 codes against torch's
    float8_e4m3fn decoding (a library routine)."""
    import torch
    t = OA.E4M3_TABLE
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x38] == 1.0 and t[0xB8] == -1.0 and t[0x30] == 0.5 and t[0x3C] == 1.5
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.isfinite(np.delete(t, [0x7F, 0xFF])).all()
    assert np.all(np.diff(t[:0x7F]) > 0)                     # monotone over the positive codes
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ref), np.isnan(t))
    fin = ~np.isnan(t)
    assert np.array_equal(ref[fin], t[fin])
    rows = np.array([[0x38, 0xC0, 0x7E]], np.uint8)
    assert np.array_equal(OA.kv_to_f64(rows, "fp8", np.array([0.25], np.float32)), [[0.25, -0.5, 112.0]])


def pin_e4m3_encoding():
    """The generator's e4m3 rounding: nearest, ties to the even code, saturating at
    448; against torch's float -> float8_e4m3fn conversion on random values."""
    import torch
    # ties: 1.0625 between 0x38 and 0x39 -> 0x38; 1.1875 between 0x39 and 0x3A -> 0x3A;
    # 2^-10 halfway between 0 and the smallest subnormal 2^-9 -> 0; 3 * 2^-11 -> 2^-9
    x = np.array([1.0625, 1.1875, 500.0, -500.0, 2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -11, -0.0, 0.0],
                 np.float32)
    assert list(gen.f32_to_e4m3_bits(x)) == [0x38, 0x3A, 0x7E, 0xFE, 0x00, 0x00, 0x01, 0x00, 0x00]
    fin = np.flatnonzero(np.isfinite(OA.E4M3_TABLE))
    vals = OA.E4M3_TABLE[fin].astype(np.float32)
    back = gen.f32_to_e4m3_bits(vals)
    assert np.array_equal(OA.E4M3_TABLE[back], OA.E4M3_TABLE[fin])   # every value maps to itself
    rng = np.random.default_rng(7)
    r = (rng.standard_normal(20000) * rng.choice([1e-3, 1.0, 60.0], 20000)).astype(np.float32)
    r = np.clip(r, -448, 448)
    ref = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(OA.E4M3_TABLE[gen.f32_to_e4m3_bits(r)], OA.E4M3_TABLE[ref])
    q, sc = gen.quantize_rows_e4m3(np.array([[1.0, -3.5, 0.25], [0.0, 0.0, 0.0]], np.float32))
    assert sc[0] == np.float32(3.5) / np.float32(448.0) and sc[1] == 0.0
    assert q[0, 1] == 0xFE and np.all(q[1] == 0)
    # the row quantiser (fast path) against the reference rounding, row by row
    x = (rng.standard_normal((200, 64)) * rng.choice([1e-3, 1.0, 50.0], (200, 1))).astype(np.float32)
    q, sc = gen.quantize_rows_e4m3(x)
    y = (x / sc[:, None]).astype(np.float32)
    assert np.array_equal(q, gen.f32_to_e4m3_bits(y))


# ----------------------------------------------------------------------------
# the scalar twin
# ----------------------------------------------------------------------------

def _close_with_pattern(a, b, tol):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    fin = np.isfinite(b)
    assert np.array_equal(a[~fin & ~np.isnan(b)], b[~fin & ~np.isnan(b)])
    z = b == 0
    assert np.array_equal(a[z], b[z])
    if fin.any():
        assert np.abs(a[fin] - b[fin]).max() <= tol * max(1.0, np.abs(b[fin]).max())


def pin_brute_decode():
    for i, dt in enumerate(("f32", "f16", "bf16", "i8", "fp8")):
        wl = gen.make_decode(seed=100 + i, n_stream=2, n_row=3, n_head_q=4, n_head_kv=2,
                             head_dim=4, cap=9, kv_dtype=dt, depths=[9, 2], causal=(i % 2 == 0),
                             softcap=(3.0 if i >= 2 else 0.0), alibi=(i % 2 == 1))
        kw = dict(q=wl.q, k=wl.k, v=wl.v, kv_dtype=dt, kv_len=wl.kv_len, causal=wl.causal,
                  scale=wl.scale, softcap=wl.softcap, alibi=wl.alibi, k_scale=wl.k_scale,
                  v_scale=wl.v_scale)
        _close_with_pattern(oracle.decode(**kw), brute.decode(**kw), 1e-13)


def pin_brute_prefill():
    wl = gen.make_prefill_mask(seed=120, n_row=4, n_head_q=4, n_head_kv=2, head_dim=4, n_kv=9,
                               kv_dtype="bf16", excluded_rows=1, nan_k=2, softcap=30.0, alibi=True)
    kw = dict(q=wl.q, k=wl.k, v=wl.v, kv_dtype="bf16", scale=wl.scale, softcap=30.0,
              alibi=wl.alibi, q_pos=wl.q_pos, mask=wl.mask, causal=True)
    _close_with_pattern(oracle.prefill(**kw), brute.prefill(**kw), 1e-13)
    wl = gen.make_prefill_sel(seed=121, n_row=3, n_head_q=2, n_head_kv=1, head_dim=4, n_kv=11,
                              kv_dtype="f16", n_sel=5, n_dup=1, n_invalid=1, block_size=2,
                              alibi=True)
    kw = dict(q=wl.q, k=wl.k, v=wl.v, kv_dtype="f16", scale=wl.scale, alibi=wl.alibi,
              q_pos=wl.q_pos, sel=wl.sel, block_size=2)
    _close_with_pattern(oracle.prefill(**kw), brute.prefill(**kw), 1e-13)


def pin_visited_sets():
    st = oracle.visited_decode(kv_len=np.array([5, 3]), n_row=2, causal=True, slice_len=2,
                               n_head_kv=1)
    # stream 0: row 0 sees 0..3, row 1 sees 0..4; slices [0,2) [2,4) [4,6)
    assert st[0, 0, 0].tolist() == [[2, 1, 1], [2, 5, 13], [0, 0, 0]]
    assert st[0, 1, 0].tolist() == [[2, 1, 1], [2, 5, 13], [1, 4, 16]]
    assert st[1, 1, 0].tolist() == [[2, 1, 1], [1, 2, 4], [0, 0, 0]]
    cells, ids = oracle.visited_prefill(n_kv=10, n_head_kv=1,
                                        sel=np.array([[4, -1, 1, 4, 2, 9]]), block_size=3)
    assert ids[0].tolist() == [1, 2] and cells[0].tolist() == [3, 4, 5, 6, 7, 8]


# ----------------------------------------------------------------------------
# tree-shaped verify windows (TensorFold PR #2595, "Kernel contract": widths
# 1..16 with heap-order parents, visible keys 33, 34, 8193, 32768..32770)
# ----------------------------------------------------------------------------

def _closure_mask(parent):
    """Row r sees window node c iff c is reachable from r by parent steps (zero or
    more), computed as a boolean transitive closure of the parent relation."""
    W = len(parent)
    A = np.zeros((W, W), dtype=bool)
    for a, up in enumerate(parent):
        if -1 < up < a:
            A[a, up] = True
    reach = np.eye(W, dtype=bool)
    for _ in range(W):
        reach = reach | ((reach.astype(np.int64) @ A.astype(np.int64)) > 0)
    return reach


def pin_tree_heap_visible_counts():
    # binary heap: node r (1-based r + 1) has ancestors (r + 1) >> k, k = 1..floor(log2(r + 1))
    for W in (1, 2, 4, 8, 12, 16):
        par = gen.heap_parents(W)
        for n in (33, 34, 8193, 32768, 32769, 32770):
            start = n - W
            for r in range(W):
                depth = (r + 1).bit_length() - 1
                cells = OA.visible_decode_row(n, W, r, True, par)
                assert cells.size == start + depth + 1, (W, n, r)
                win = [start + ((r + 1) >> kk) - 1 for kk in range(depth, -1, -1)]
                assert cells[start:].tolist() == win
                assert np.array_equal(cells[:start], np.arange(start))


def pin_tree_chain_is_causal():
    wl = gen.make_decode(seed=71, n_stream=3, n_row=6, n_head_q=4, n_head_kv=2, head_dim=8,
                         cap=20, kv_dtype="bf16", depths=[20, 9, 4], causal=True, alibi=True,
                         softcap=4.0, tree="chain")
    kw = dict(q=wl.q, k=wl.k, v=wl.v, kv_dtype="bf16", kv_len=wl.kv_len, scale=wl.scale,
              softcap=4.0, alibi=wl.alibi)
    causal = oracle.decode(causal=True, **kw)
    assert np.array_equal(oracle.decode(causal=False, tree_parent=wl.tree_parent, **kw), causal)
    # a width-1 tree is the plain single-row decode over every cell
    one = gen.make_decode(seed=72, n_stream=2, n_row=1, n_head_q=2, n_head_kv=1, head_dim=8,
                          cap=11, kv_dtype="f16", depths=[11, 5], causal=False, tree="heap")
    kw1 = dict(q=one.q, k=one.k, v=one.v, kv_dtype="f16", kv_len=one.kv_len, scale=one.scale)
    assert np.array_equal(oracle.decode(causal=True, tree_parent=one.tree_parent, **kw1),
                          oracle.decode(causal=False, **kw1))


def pin_tree_torch_sdpa():
    import torch
    rng = np.random.default_rng(73)
    W, n, Hq, Hkv, D = 12, 40, 4, 2, 16
    par = gen.random_parents(rng, W)
    par[5] = 9          # not in [-1, 5): node 5 becomes a root
    par[7] = -3         # likewise
    wl = gen.make_decode(seed=74, n_stream=1, n_row=W, n_head_q=Hq, n_head_kv=Hkv, head_dim=D,
                         cap=n, kv_dtype="f32", depths=[n], causal=True, tree=par)
    out = oracle.decode(q=wl.q, k=wl.k, v=wl.v, kv_dtype="f32", kv_len=wl.kv_len, causal=True,
                        scale=wl.scale, tree_parent=wl.tree_parent)
    reach = _closure_mask(par)
    bias = np.zeros((W, n))
    bias[:, n - W:] = np.where(reach, 0.0, -np.inf)
    q = torch.from_numpy(wl.q[0].astype(np.float64)).permute(1, 0, 2)[None]       # [1,H,W,D]
    k = torch.from_numpy(wl.k[0].astype(np.float64)).permute(1, 0, 2)
    v = torch.from_numpy(wl.v[0].astype(np.float64)).permute(1, 0, 2)
    k = k.repeat_interleave(Hq // Hkv, dim=0)[None].contiguous()
    v = v.repeat_interleave(Hq // Hkv, dim=0)[None].contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=torch.from_numpy(bias)[None, None], scale=wl.scale)[0]
    assert np.allclose(out[0], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-14)


def pin_tree_split_and_visited():
    wl = gen.make_decode(seed=75, n_stream=3, n_row=8, n_head_q=4, n_head_kv=2, head_dim=8,
                         cap=30, kv_dtype="i8", depths=[30, 13, 5], causal=True, tree="random",
                         alibi=True)
    kw = dict(q=wl.q, k=wl.k, v=wl.v, kv_dtype="i8", kv_len=wl.kv_len, causal=True,
              scale=wl.scale, alibi=wl.alibi, k_scale=wl.k_scale, v_scale=wl.v_scale,
              tree_parent=wl.tree_parent)
    ref = oracle.decode(**kw)
    for L in (1, 3, 4, 7, 30):
        out = oracle.decode_split(slice_len=L, **kw)[0]
        assert np.allclose(out, ref, rtol=1e-13, atol=1e-15), L
        st = oracle.visited_decode(kv_len=wl.kv_len, n_row=8, causal=True, slice_len=L,
                                   n_head_kv=2, tree_parent=wl.tree_parent)
        for b in range(3):
            reach = _closure_mask(wl.tree_parent[b])
            start = int(wl.kv_len[b]) - 8
            for r in range(8):
                cells = [j for j in range(int(wl.kv_len[b]))
                         if j < start or (j >= start and reach[r, j - start])]
                c = np.array(cells, np.int64)
                assert st[b, r, 0, :, 0].sum() == c.size
                assert st[b, r, 1, :, 1].sum() == c.sum()


# ----------------------------------------------------------------------------
# attention-sink logit (HartsyInference PR #910: PR body, review of the CPU fix)
# ----------------------------------------------------------------------------

def pin_sink_one_key_closed_form():
    # one key with score a, value x, sink z: out = x / (1 + exp(z - a))
    q = np.array([[[1.5, -0.5]]], np.float32)
    k = np.array([[[0.75, 0.25]]], np.float32)
    v = np.array([[[2.0, -3.0]]], np.float32)
    a = 0.5 * (1.5 * 0.75 - 0.5 * 0.25)
    for z in (-3.0, 0.0, 0.5, 4.0, 60.0):
        out = oracle.prefill(q=q, k=k, v=v, kv_dtype="f32", scale=0.5,
                             mask=np.zeros((1, 1), np.float32), sinks=np.array([z], np.float32))
        w = 1.0 / (1.0 + math.exp(z - a))
        assert np.allclose(out[0, 0], [2.0 * w, -3.0 * w], rtol=1e-15, atol=1e-300), z


def pin_sink_scipy_softmax():
    # the sink is one more logit in the softmax whose value row is zero
    from scipy.special import softmax
    wl = gen.make_decode(seed=76, n_stream=2, n_row=3, n_head_q=4, n_head_kv=2, head_dim=8,
                         cap=17, kv_dtype="f16", depths=[17, 6], causal=True, sinks="draw")
    out = oracle.decode(q=wl.q, k=wl.k, v=wl.v, kv_dtype="f16", kv_len=wl.kv_len, causal=True,
                        scale=wl.scale, sinks=wl.sinks)
    for b in range(2):
        n = int(wl.kv_len[b])
        for r in range(3):
            lim = n - 3 + r + 1
            for h in range(4):
                k64 = wl.k[b, :lim, h // 2].astype(np.float64)
                v64 = wl.v[b, :lim, h // 2].astype(np.float64)
                s = wl.scale * (k64 @ wl.q[b, r, h].astype(np.float64))
                w = softmax(np.append(s, float(wl.sinks[h])))[:-1]
                assert np.allclose(out[b, r, h], w @ v64, rtol=1e-12, atol=1e-14)


def pin_sink_review_cases():
    D = 3
    empty = np.zeros((1, 0))
    none = np.zeros((0, D))
    # an empty row: -inf sink -> +0.0; +inf or NaN sink -> NaN; a finite sink -> +0.0
    z = OA.attend_scores(empty, none, sink=np.array([-np.inf]))
    assert np.array_equal(z, np.zeros((1, D))) and not np.signbit(z).any()
    assert np.isnan(OA.attend_scores(empty, none, sink=np.array([np.inf]))).all()
    assert np.isnan(OA.attend_scores(empty, none, sink=np.array([np.nan]))).all()
    f = OA.attend_scores(empty, none, sink=np.array([2.5]))
    assert np.array_equal(f, np.zeros((1, D))) and not np.signbit(f).any()
    # a -inf sink is no sink; a +inf or NaN sink poisons a non-empty row
    s = np.array([[0.3, -1.2, 2.0]])
    vc = np.arange(9.0).reshape(3, 3)
    assert np.array_equal(OA.attend_scores(s, vc, sink=np.array([-np.inf])), OA.attend_scores(s, vc))
    assert np.isnan(OA.attend_scores(s, vc, sink=np.array([np.inf]))).all()
    assert np.isnan(OA.attend_scores(s, vc, sink=np.array([np.nan]))).all()
    # the same through the combine of split partials
    o = np.array([[[1.0, 2.0, 3.0]], [[0.0, 0.0, 0.0]]])
    m = np.array([[0.5], [-np.inf]])
    l = np.array([[2.0], [0.0]])
    w = 2.0 / (2.0 + math.exp(1.0 - 0.5))
    assert np.allclose(OA.combine_partials(o, m, l, sink=np.array([1.0])),
                       [[0.5 * w, 1.0 * w, 1.5 * w]], rtol=1e-15)
    assert np.array_equal(OA.combine_partials(o, m, l, sink=np.array([-np.inf])),
                          OA.combine_partials(o, m, l))
    m_empty = np.array([[-np.inf], [-np.inf]])
    for zz, nan in ((-np.inf, False), (np.inf, True), (np.nan, True), (0.0, False)):
        c = OA.combine_partials(np.zeros_like(o), m_empty, np.zeros_like(l), sink=np.array([zz]))
        if nan:
            assert np.isnan(c).all(), zz
        else:
            assert np.array_equal(c, np.zeros((1, D))) and not np.signbit(c).any(), zz


def pin_sink_split_equals_unsplit():
    wl = gen.make_decode(seed=77, n_stream=2, n_row=4, n_head_q=4, n_head_kv=2, head_dim=8,
                         cap=19, kv_dtype="bf16", depths=[19, 7], causal=True, sinks="draw",
                         tree="heap")
    kw = dict(q=wl.q, k=wl.k, v=wl.v, kv_dtype="bf16", kv_len=wl.kv_len, causal=True,
              scale=wl.scale, sinks=wl.sinks, tree_parent=wl.tree_parent)
    ref = oracle.decode(**kw)
    for L in (1, 2, 5, 19):
        assert np.allclose(oracle.decode_split(slice_len=L, **kw)[0], ref, rtol=1e-13, atol=1e-15)
    pw = gen.make_prefill_sel(seed=78, n_row=3, n_head_q=4, n_head_kv=2, head_dim=8, n_kv=30,
                              kv_dtype="bf16", n_sel=7, n_dup=1, n_invalid=1, block_size=3)
    sinks = gen.draw_sinks(np.random.default_rng(79), 4)
    kwp = dict(q=pw.q, k=pw.k, v=pw.v, kv_dtype="bf16", scale=pw.scale, q_pos=pw.q_pos,
               sel=pw.sel, block_size=3, sinks=sinks)
    ref = oracle.prefill(**kwp)
    for n in (1, 2, 4, 30):
        assert np.allclose(oracle.prefill_split(n_splits=n, **kwp), ref, rtol=1e-13, atol=1e-15)


def pin_brute_tree_sink():
    for i, dt in enumerate(("f32", "bf16", "i8", "fp8")):
        wl = gen.make_decode(seed=130 + i, n_stream=2, n_row=5, n_head_q=4, n_head_kv=2,
                             head_dim=4, cap=9, kv_dtype=dt, depths=[9, 3], causal=True,
                             alibi=(i % 2 == 1), tree="random", sinks="draw")
        sinks = wl.sinks.copy()
        if i == 3:
            sinks[1], sinks[2] = -np.inf, np.nan
        kw = dict(q=wl.q, k=wl.k, v=wl.v, kv_dtype=dt, kv_len=wl.kv_len, causal=True,
                  scale=wl.scale, alibi=wl.alibi, k_scale=wl.k_scale, v_scale=wl.v_scale,
                  tree_parent=wl.tree_parent, sinks=sinks)
        _close_with_pattern(oracle.decode(**kw), brute.decode(**kw), 1e-13)
    wl = gen.make_prefill_mask(seed=134, n_row=4, n_head_q=4, n_head_kv=2, head_dim=4, n_kv=9,
                               kv_dtype="f16", excluded_rows=1, softcap=20.0, alibi=True)
    sinks = np.array([0.5, -np.inf, np.inf, 3.0], np.float32)
    kw = dict(q=wl.q, k=wl.k, v=wl.v, kv_dtype="f16", scale=wl.scale, softcap=20.0,
              alibi=wl.alibi, q_pos=wl.q_pos, mask=wl.mask, causal=True, sinks=sinks)
    _close_with_pattern(oracle.prefill(**kw), brute.prefill(**kw), 1e-13)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# planted mistakes in the oracle (CPU only): each must turn a pin red
# ----------------------------------------------------------------------------

def _expect_red(pin):
    with pytest.raises(AssertionError):
        pin()


def test_planted_alibi_before_softcap(monkeypatch):
    real = OA.scores

    def swapped(q, kc, cells, *, scale, softcap=0.0, slopes=None, pos=0, mask_vals=None):
        s = float(scale) * (np.asarray(q, np.float64) @ np.asarray(kc, np.float64).T)
        if slopes is not None:
            s = s + np.asarray(slopes, np.float64)[:, None] * (np.asarray(cells, np.float64) - pos)[None, :]
        if softcap and softcap > 0:
            s = softcap * np.tanh(s / softcap)
        if mask_vals is not None:
            s = s + np.asarray(mask_vals, np.float64)[None, :]
        return s

    monkeypatch.setattr(OA, "scores", swapped)
    _expect_red(pin_softcap_before_alibi)
    monkeypatch.setattr(OA, "scores", real)
    pin_softcap_before_alibi()


def test_planted_combine_nan_to_zero(monkeypatch):
    real = OA.combine_partials

    def lossy(o, m, l, **kw):
        m = np.nan_to_num(np.asarray(m, np.float64), nan=-np.inf)
        return np.nan_to_num(real(o, m, l, **kw), nan=0.0)

    monkeypatch.setattr(OA, "combine_partials", lossy)
    _expect_red(pin_combine_rules)


def test_planted_no_dedup(monkeypatch):
    def no_dedup(ids, block_size, n_kv):
        ids = np.asarray(ids, dtype=np.int64)
        ok = (ids >= 0) & (ids * block_size < n_kv)
        blocks = np.sort(ids[ok])
        cells = (blocks[:, None] * block_size + np.arange(block_size)[None, :]).reshape(-1)
        return cells[cells < n_kv]

    monkeypatch.setattr(OA, "visible_selection", no_dedup)
    _expect_red(pin_selection_invariances)


def test_planted_excluded_row_nan(monkeypatch):
    real = OA.attend_scores

    def nan_rows(s, vc, **kw):
        out = real(s, vc, **kw)
        s = np.asarray(s)
        for h in range(s.shape[0]):
            if s.shape[1] == 0 or np.all(s[h] == -np.inf):
                out[h] = np.nan
        return out

    monkeypatch.setattr(OA, "attend_scores", nan_rows)
    _expect_red(pin_m03_excluded_row)


def test_planted_wrong_gqa_mapping(monkeypatch):
    real = OA.decode

    def modulo_heads(**kw):
        q = kw["q"]
        Hkv = kw["k"].shape[2]
        G = q.shape[2] // Hkv
        # planted: query head h reads kv head h % Hkv instead of h // G
        order = np.array([(h % Hkv) * G + h // Hkv for h in range(q.shape[2])])
        kw = dict(kw, q=q[:, :, order])
        out = real(**kw)
        inv = np.argsort(order)
        return out[:, :, inv]

    monkeypatch.setattr(oracle, "decode", modulo_heads)
    _expect_red(pin_scipy_softmax_dense)


def test_planted_dropped_scale(monkeypatch):
    real = OA.scores

    def unscaled(q, kc, cells, *, scale, **kw):
        return real(q, kc, cells, scale=1.0, **kw)

    monkeypatch.setattr(OA, "scores", unscaled)
    _expect_red(pin_torch_sdpa_mask_alibi_gqa)


def test_planted_tree_sibling_visible(monkeypatch):
    # planted: a row also sees the node just before it (a chain step mixed into the tree)
    real = OA.tree_path

    def leaky(parent, r):
        nodes = set(real(parent, r))
        if r > 0:
            nodes.add(r - 1)
        return sorted(nodes)

    monkeypatch.setattr(OA, "tree_path", leaky)
    _expect_red(pin_tree_heap_visible_counts)
    _expect_red(pin_tree_torch_sdpa)


def test_planted_sink_counted_twice(monkeypatch):
    # planted: the sink enters each slice's partial as well as the final combine
    real = OA.combine_partials

    def twice(o, m, l, sink=None):
        if sink is None:
            return real(o, m, l)
        m = np.asarray(m, np.float64)
        l2 = np.array(l, np.float64)
        for t in range(m.shape[0]):
            for h in range(m.shape[1]):
                if np.isfinite(m[t, h]):
                    l2[t, h] += math.exp(float(sink[h]) - m[t, h])
        return real(o, m, l2, sink=sink)

    monkeypatch.setattr(OA, "combine_partials", twice)
    _expect_red(pin_sink_split_equals_unsplit)


def test_planted_sink_guard_missing(monkeypatch):
    # planted: no guard for M = -inf, so a -inf sink on an empty row computes exp(-inf - -inf)
    real = OA.attend_scores

    def unguarded(s, vc, sink=None):
        s = np.asarray(s, np.float64)
        if sink is not None and s.shape[1] == 0:
            z = np.asarray(sink, np.float64)
            with np.errstate(invalid="ignore"):
                den = np.exp(z - np.maximum(z, -np.inf))
            return np.zeros((s.shape[0], np.asarray(vc).shape[1])) / den[:, None]
        return real(s, vc, sink=sink)

    monkeypatch.setattr(OA, "attend_scores", unguarded)
    _expect_red(pin_sink_review_cases)
