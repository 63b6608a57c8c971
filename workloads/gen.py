"""Seeded input generator for the five attention workloads and for test shapes.

Every array is produced from ``np.random.default_rng(seed)`` in a fixed order:
Q, then K, then V, then the structure (depths, masks, selection lists, NaN
positions).  Storage conversions are plain round-to-nearest-even (fp16, bf16)
and symmetric per-row int8 quantisation (scale = amax / 127); they only decide
the bits both sides read, never an attention result.

Shapes follow the workload descriptions of the selected-key prefill PR
(strix-llama.cpp #115, commit message of the Vulkan selected-key kernel: one
list of block ids per query, GQA groups at head dim 256), the XPU split decode
PR (TensorFold #2595, "Kernel contract": bf16 K/V caches split into slices),
the 27B CUDA PR (TensorFold #911, the fp8 commit: one scale per (position, key
head) row, verify windows of up to 16 streams x 16 rows) and the semantics PR
(HartsyInference #910: softcap, ALiBi, F32 additive mask, NaN data).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

KV_DTYPES = ("f32", "f16", "bf16", "i8", "fp8")
SCALED_DTYPES = ("i8", "fp8")        # 1-byte rows with an fp32 scale per (cell, kv head) row


# ----------------------------------------------------------------------------
# storage conversions (input preparation only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = ((u + (((u >> 16) & 1) + np.uint32(0x7FFF))) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def quantize_rows_i8(x: np.ndarray):
    """Symmetric int8 quantisation of each last-axis row.

    scale = amax / 127 in fp32; q = clamp(rint(x / scale), -127, 127) with ties
    to even; an all-zero row gets scale 0 and q = 0.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint(x / safe[..., None])
    q = np.clip(q, -127, 127).astype(np.int8)
    q[scale == 0] = 0
    return q, scale


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round to the nearest e4m3 value (format with maximum 448: 4 exponent bits,
    bias 7, 3 mantissa bits, subnormals m * 2^-9), ties to the even code,
    saturating at 448; return uint8 codes.  Inputs here are finite."""
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x), np.float32(448.0))
    bits = a.view(np.uint32).astype(np.int64)
    # normal range (>= 2^-6): keep 3 of the 23 fraction bits, round half to even on
    # the whole bit pattern (a carry moves into the exponent), rebias 127 -> 7
    r = (bits + 0x7FFFF + ((bits >> 20) & 1)) >> 20
    normal = ((r >> 3) - (127 - 7)) * 8 + (r & 7)
    # subnormal range: multiples of 2^-9, rint rounds half to even; 8 * 2^-9 is code 8
    sub = np.rint(a.astype(np.float64) * 512.0).astype(np.int64)
    code = np.where(a < np.float32(2.0 ** -6), sub, normal)
    code = np.minimum(code, 0x7E).astype(np.uint8)
    code |= np.where(np.signbit(x) & (code != 0), 0x80, 0).astype(np.uint8)
    return code


def quantize_rows_e4m3(x: np.ndarray):
    """e4m3 rows with one fp32 scale per row: scale = amax / 448 in fp32, codes =
    nearest e4m3 of x / scale (computed in fp32); an all-zero row gets scale 0.
    The rounding runs through torch's float8_e4m3fn conversion (nearest, ties to
    even; the values are within +-448 here), which the oracle pins check against
    f32_to_e4m3_bits; it is the fast path for large caches."""
    import torch
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = np.clip(x / safe[..., None], -448.0, 448.0).astype(np.float32)
    q = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    q[q == 0x80] = 0                                    # -0 is stored as +0
    q[scale == 0] = 0
    return q, scale


def _to_storage(x32: np.ndarray, dtype: str):
    """fp32 draw -> (storage array, scale or None)."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32), None
    if dtype == "f16":
        return x32.astype(np.float16), None
    if dtype == "bf16":
        return f32_to_bf16_bits(x32), None
    if dtype == "i8":
        return quantize_rows_i8(x32)
    if dtype == "fp8":
        return quantize_rows_e4m3(x32)
    raise ValueError(f"unknown kv dtype {dtype!r}")


def _draw_kv(rng, lead_shape, head_dim, dtype):
    """Draw N(0,1) K or V rows stream by stream (same sequence as one big draw)."""
    lead_shape = tuple(lead_shape)
    n0 = lead_shape[0]
    store = None
    scales = None
    for i in range(n0):
        x = rng.standard_normal(lead_shape[1:] + (head_dim,), dtype=np.float32)
        s, sc = _to_storage(x, dtype)
        if store is None:
            store = np.empty(lead_shape + (head_dim,), dtype=s.dtype)
            if sc is not None:
                scales = np.empty(lead_shape, dtype=np.float32)
        store[i] = s
        if sc is not None:
            scales[i] = sc
    return store, scales


def alibi_slopes(n_head: int) -> np.ndarray:
    """Standard ALiBi slopes 2^(-8(h+1)/H) for a power-of-two head count."""
    h = np.arange(n_head, dtype=np.float64)
    return np.power(2.0, -8.0 * (h + 1.0) / n_head).astype(np.float32)


# ----------------------------------------------------------------------------
# workload containers
# ----------------------------------------------------------------------------

@dataclass
class DecodeWorkload:
    """Split-K decode / verify-window input.

    q      fp32 [S][R][Hq][D]
    k, v   storage [S][cap][Hkv][D] (fp32, fp16, bf16 bits as uint16, int8)
    k_scale, v_scale  fp32 [S][cap][Hkv] (int8 only)
    kv_len int32 [S]: cells in each stream's cache, the window's rows included
    Row r of stream b sits at position kv_len[b] - R + r; with causal it sees
    cells [0, that position], else [0, kv_len[b]).
    tree_parent int32 [S][R] or None: each stream's window as a tree in heap order
    sinks fp32 [Hq] or None: one sink logit per query head
    """

    name: str
    n_stream: int
    n_row: int
    n_head_q: int
    n_head_kv: int
    head_dim: int
    cap: int
    kv_dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    k_scale: Optional[np.ndarray]
    v_scale: Optional[np.ndarray]
    kv_len: np.ndarray
    causal: bool
    scale: float
    softcap: float
    alibi: Optional[np.ndarray]
    slice_len: int
    tree_parent: Optional[np.ndarray] = None
    sinks: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def n_slices_max(self) -> int:
        return max(1, -(-int(self.kv_len.max()) // self.slice_len))


@dataclass
class PrefillWorkload:
    """Prefill input in one of two modes.

    q      fp32 [R][Hq][D]
    k, v   storage [N][Hkv][D]; k_scale, v_scale fp32 [N][Hkv] (int8 only)
    q_pos  int32 [R] query positions (ALiBi and causal)
    Selection mode: sel int32 [R][n_sel] block ids, block_size cells per id.
    Mask mode: mask fp32 [R][N] additive (broadcast over heads), causal flag.
    sinks  fp32 [Hq] or None: one sink logit per query head
    """

    name: str
    n_row: int
    n_head_q: int
    n_head_kv: int
    head_dim: int
    n_kv: int
    kv_dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    k_scale: Optional[np.ndarray]
    v_scale: Optional[np.ndarray]
    q_pos: Optional[np.ndarray]
    scale: float
    softcap: float
    alibi: Optional[np.ndarray]
    sel: Optional[np.ndarray] = None
    block_size: int = 1
    mask: Optional[np.ndarray] = None
    causal: bool = False
    sinks: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def mode(self) -> str:
        return "sel" if self.sel is not None else "mask"


# ----------------------------------------------------------------------------
# generic builders (tests use them at small sizes)
# ----------------------------------------------------------------------------

def heap_parents(width: int) -> np.ndarray:
    """Binary tree in heap order: node i > 0 hangs off node (i - 1) // 2, node 0 is the root."""
    return np.array([-1] + [(i - 1) // 2 for i in range(1, width)], dtype=np.int32)


def chain_parents(width: int) -> np.ndarray:
    """A chain: node i hangs off node i - 1 (the causal window as a tree)."""
    return np.arange(-1, width - 1, dtype=np.int32)


def random_parents(rng, width: int) -> np.ndarray:
    """Random tree in heap order: node i's parent uniform over {-1, 0, ..., i - 1}."""
    return np.array([int(rng.integers(-1, i)) for i in range(width)], dtype=np.int32)


def aux_rng(seed):
    """A generator independent of the main draw of `seed` (trees, sinks), so that
    adding them leaves Q, K, V and the lengths unchanged."""
    return np.random.default_rng(np.random.SeedSequence(seed).spawn(1)[0])


def draw_sinks(rng, n_head: int) -> np.ndarray:
    """Sink logits U[-2, 6): from below the typical score maximum to well above it."""
    return rng.uniform(-2.0, 6.0, size=n_head).astype(np.float32)


def _draw_kv_prefix(rng, n_stream, cap, n_head_kv, head_dim, dtype, kv_len):
    """K or V for cells [0, kv_len[b]) of each stream; unused capacity is NaN
    (int8: 0 with a NaN row scale; e4m3: the NaN code and a NaN scale), so a read
    past kv_len cannot go unnoticed."""
    shape = (n_stream, cap, n_head_kv, head_dim)
    if dtype == "f32":
        store = np.full(shape, np.nan, np.float32)
    elif dtype == "f16":
        store = np.full(shape, np.nan, np.float16)
    elif dtype == "bf16":
        store = np.full(shape, 0x7FC0, np.uint16)
    elif dtype == "fp8":
        store = np.full(shape, 0x7F, np.uint8)                    # the e4m3 NaN code
    else:
        store = np.zeros(shape, np.int8)
    scales = np.full((n_stream, cap, n_head_kv), np.nan, np.float32) if dtype in SCALED_DTYPES else None
    for b in range(n_stream):
        n = int(kv_len[b])
        x = rng.standard_normal((n, n_head_kv, head_dim), dtype=np.float32)
        st, sc = _to_storage(x, dtype)
        store[b, :n] = st
        if sc is not None:
            scales[b, :n] = sc
    return store, scales


def make_decode(*, seed, n_stream, n_row, n_head_q, n_head_kv, head_dim, cap,
                kv_dtype, depths=None, depth_range=None, causal=True,
                slice_len=1024, scale=None, softcap=0.0, alibi=False, tree=None,
                sinks=None, name="decode") -> DecodeWorkload:
    """Decode workload.

    With fixed `depths`: Q, K, V ~ N(0,1) over the whole capacity, in that order.
    With `depth_range`: Q, then the depths U[lo, hi] (inclusive), then K and V
    for the cells below each depth only (unused capacity holds NaN).
    tree: None, "heap", "chain", "random" (one random tree per stream) or an
    int array [R] used by every stream.  sinks: None, "draw" or an array [Hq].
    Trees and sinks come from aux_rng(seed).
    """
    assert kv_dtype in KV_DTYPES
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_stream, n_row, n_head_q, head_dim), dtype=np.float32)
    if depths is not None:
        k, ks = _draw_kv(rng, (n_stream, cap, n_head_kv), head_dim, kv_dtype)
        v, vs = _draw_kv(rng, (n_stream, cap, n_head_kv), head_dim, kv_dtype)
        kv_len = np.asarray(depths, dtype=np.int32).reshape(n_stream)
    else:
        lo, hi = depth_range
        kv_len = rng.integers(lo, hi, size=n_stream, endpoint=True).astype(np.int32)
        k, ks = _draw_kv_prefix(rng, n_stream, cap, n_head_kv, head_dim, kv_dtype, kv_len)
        v, vs = _draw_kv_prefix(rng, n_stream, cap, n_head_kv, head_dim, kv_dtype, kv_len)
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    slopes = alibi_slopes(n_head_q) if alibi else None
    aux = aux_rng(seed)
    parents = None
    if isinstance(tree, str) and tree == "random":
        parents = np.stack([random_parents(aux, n_row) for _ in range(n_stream)])
    elif tree is not None:
        one = {"heap": heap_parents, "chain": chain_parents}[tree](n_row) if isinstance(tree, str) \
            else np.asarray(tree, np.int32)
        parents = np.tile(one, (n_stream, 1)).astype(np.int32)
    sk = None
    if isinstance(sinks, str):
        sk = draw_sinks(aux, n_head_q)
    elif sinks is not None:
        sk = np.asarray(sinks, np.float32)
    return DecodeWorkload(name, n_stream, n_row, n_head_q, n_head_kv, head_dim, cap,
                          kv_dtype, q, k, v, ks, vs, kv_len, bool(causal), float(scale),
                          float(softcap), slopes, int(slice_len), tree_parent=parents,
                          sinks=sk)


def make_prefill_mask(*, seed, n_row, n_head_q, n_head_kv, head_dim, n_kv, kv_dtype,
                      first_pos=None, causal=True, excluded_rows=0, nan_k=0,
                      softcap=0.0, alibi=False, scale=None, mask_kind="normal",
                      name="prefill_mask") -> PrefillWorkload:
    """Mask-mode prefill: Q, K, V, then mask values, excluded rows, NaN spots.

    Query r sits at position first_pos + r (default: the newest n_row cells).
    The mask is N(0,1) where visible, -inf past the causal limit, and -inf on
    every key of `excluded_rows` rows drawn without replacement.  `nan_k` K
    elements (drawn without replacement over the whole K array) are NaN.
    mask_kind "zero" gives a zero bias instead of N(0,1).
    """
    assert kv_dtype in KV_DTYPES
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_row, n_head_q, head_dim), dtype=np.float32)
    k, ks = _draw_kv(rng, (n_kv, n_head_kv), head_dim, kv_dtype)
    v, vs = _draw_kv(rng, (n_kv, n_head_kv), head_dim, kv_dtype)
    if first_pos is None:
        first_pos = n_kv - n_row
    q_pos = (first_pos + np.arange(n_row)).astype(np.int32)
    if mask_kind == "normal":
        mask = rng.standard_normal((n_row, n_kv), dtype=np.float32)
    elif mask_kind == "zero":
        mask = np.zeros((n_row, n_kv), dtype=np.float32)
    else:
        raise ValueError(mask_kind)
    if causal:
        j = np.arange(n_kv)[None, :]
        mask[j > q_pos[:, None]] = -np.inf
    if excluded_rows:
        rows = rng.choice(n_row, size=excluded_rows, replace=False)
        mask[rows, :] = -np.inf
    else:
        rows = np.zeros(0, dtype=np.int64)
    nan_idx = np.zeros(0, dtype=np.int64)
    if nan_k:
        nan_idx = rng.choice(k.size, size=nan_k, replace=False)
        if kv_dtype == "i8":
            raise ValueError("NaN injection needs a floating-point K")
        flat = k.reshape(-1)
        if kv_dtype == "bf16":
            flat[nan_idx] = np.uint16(0x7FC0)
        elif kv_dtype == "fp8":
            flat[nan_idx] = np.uint8(0x7F)
        else:
            flat[nan_idx] = np.nan
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    slopes = alibi_slopes(n_head_q) if alibi else None
    return PrefillWorkload(name, n_row, n_head_q, n_head_kv, head_dim, n_kv, kv_dtype,
                           q, k, v, ks, vs, q_pos, float(scale), float(softcap), slopes,
                           mask=mask, causal=bool(causal),
                           meta={"excluded_rows": np.sort(rows), "nan_k_index": np.sort(nan_idx)})


def make_prefill_sel(*, seed, n_row, n_head_q, n_head_kv, head_dim, n_kv, kv_dtype,
                     n_sel, n_dup, n_invalid, block_size, first_pos=None,
                     softcap=0.0, alibi=False, scale=None,
                     name="prefill_sel") -> PrefillWorkload:
    """Selection-mode prefill.

    Row r sits at position first_pos + r.  Its list holds n_sel - n_dup -
    n_invalid distinct block ids drawn uniformly from the causal blocks
    {b : b * block_size <= pos}, n_dup copies of its own valid ids, and
    n_invalid invalid ids (-1, or a block starting at or beyond n_kv), shuffled.
    """
    assert kv_dtype in KV_DTYPES
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_row, n_head_q, head_dim), dtype=np.float32)
    k, ks = _draw_kv(rng, (n_kv, n_head_kv), head_dim, kv_dtype)
    v, vs = _draw_kv(rng, (n_kv, n_head_kv), head_dim, kv_dtype)
    if first_pos is None:
        first_pos = n_kv - n_row
    q_pos = (first_pos + np.arange(n_row)).astype(np.int32)
    n_blocks = -(-n_kv // block_size)
    n_valid = n_sel - n_dup - n_invalid
    assert n_valid >= 1 or (n_dup == 0)
    sel = np.empty((n_row, n_sel), dtype=np.int32)
    for r in range(n_row):
        causal_blocks = int(q_pos[r]) // block_size + 1
        causal_blocks = min(causal_blocks, n_blocks)
        nv = min(n_valid, causal_blocks)
        valid = rng.choice(causal_blocks, size=nv, replace=False)
        dup = rng.choice(valid, size=n_dup, replace=True) if n_dup and nv else np.zeros(0, np.int64)
        pad = n_valid - nv  # only when a row has fewer causal blocks than asked
        kinds = rng.integers(0, 2, size=n_invalid + pad)
        far = rng.integers(n_blocks, 2 * n_blocks + 1, size=n_invalid + pad)
        inval = np.where(kinds == 0, -1, far)
        row = np.concatenate([valid, dup, inval]).astype(np.int32)
        sel[r] = row[rng.permutation(n_sel)]
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    slopes = alibi_slopes(n_head_q) if alibi else None
    return PrefillWorkload(name, n_row, n_head_q, n_head_kv, head_dim, n_kv, kv_dtype,
                           q, k, v, ks, vs, q_pos, float(scale), float(softcap), slopes,
                           sel=sel, block_size=int(block_size))


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------

def config1() -> DecodeWorkload:
    """Dense decode, tiny: S=1, R=1, GQA 4 (4/1 heads), D=256, 64 keys, fp32, scale 1/16."""
    return make_decode(seed=[1, 0], n_stream=1, n_row=1, n_head_q=4, n_head_kv=1,
                       head_dim=256, cap=64, kv_dtype="f32", depths=[64], causal=True,
                       slice_len=64, scale=1.0 / 16.0, name="dense_decode_tiny")


def config2(cap: int = 32768, kv_dtype: str = "bf16") -> DecodeWorkload:
    """Split-K decode: 16 streams x 1 row, 32/4 heads, D=256, bf16, depths U[1024, 32768], slices of 1024.
    kv_dtype="fp8" stores the same draws as e4m3 rows with fp32 row scales."""
    return make_decode(seed=[2, 0], n_stream=16, n_row=1, n_head_q=32, n_head_kv=4,
                       head_dim=256, cap=cap, kv_dtype=kv_dtype, depth_range=(1024, 32768),
                       causal=True, slice_len=1024, name=f"split_k_decode_{kv_dtype}")


def config3() -> PrefillWorkload:
    """Selected-key prefill: 2048 rows at 30000..32047, 16/2 heads, D=256, bf16, N=32048,
    512 ids per row over 4-cell blocks (476 distinct valid + 26 duplicates + 10 invalid)."""
    return make_prefill_sel(seed=[3, 0], n_row=2048, n_head_q=16, n_head_kv=2, head_dim=256,
                            n_kv=32048, kv_dtype="bf16", n_sel=512, n_dup=26, n_invalid=10,
                            block_size=4, first_pos=30000, name="selected_key_prefill_bf16")


def config4(nan: bool = True) -> PrefillWorkload:
    """Semantic edge prefill: 256 rows x 4096 keys, 16/4 heads, D=128, fp16, softcap 30,
    ALiBi, F32 mask (causal -inf, 8 rows all -inf, else N(0,1)), 2097 NaN K elements.
    nan=False is the control without NaN injection (same draw otherwise)."""
    return make_prefill_mask(seed=[4, 0], n_row=256, n_head_q=16, n_head_kv=4, head_dim=128,
                             n_kv=4096, kv_dtype="f16", first_pos=3840, causal=True,
                             excluded_rows=8, nan_k=2097 if nan else 0, softcap=30.0,
                             alibi=True, name="semantic_edge_prefill_f16" + ("" if nan else "_control"))


def config5(depth: int = 32000, tree=None) -> DecodeWorkload:
    """INT8-cache verify decode: 16 streams x 16-row causal windows, 48/4 heads, D=256,
    int8 rows + fp32 per-row scales, `depth` cached cells before the window, slices of 2048.
    tree="heap": each window is a binary tree in heap order instead of a chain."""
    variant = {12000: 0, 32000: 1}.get(depth, 2)
    w = 16
    return make_decode(seed=[5, variant], n_stream=16, n_row=w, n_head_q=48, n_head_kv=4,
                       head_dim=256, cap=depth + w, kv_dtype="i8", depths=[depth + w] * 16,
                       causal=True, slice_len=2048, tree=tree,
                       name=f"int8_{'tree_' if tree else ''}verify_decode_d{depth}")


def sel_decode(n_head_q: int = 16, n_head_kv: int = 2, n_kv: int = 32048) -> PrefillWorkload:
    """Selected-key decode: 16 query rows (one new token of each of 16 sequences in one
    unified cache) at the 16 newest positions, D=256, bf16, 512 ids per row over 4-cell
    blocks (476 distinct valid + 26 duplicates + 10 invalid); run as the selection-mode
    call with the key range split so that the rows fill the GPU."""
    return make_prefill_sel(seed=[6, n_head_q // n_head_kv], n_row=16, n_head_q=n_head_q,
                            n_head_kv=n_head_kv, head_dim=256, n_kv=n_kv, kv_dtype="bf16",
                            n_sel=512, n_dup=26, n_invalid=10, block_size=4,
                            first_pos=n_kv - 16, name="selected_key_decode_bf16")


CONFIGS = {
    "1": config1,
    "2": config2,
    "3": config3,
    "4": config4,
    "4c": lambda: config4(nan=False),
    "5a": lambda: config5(12000),
    "5b": lambda: config5(32000),
    "5t": lambda: config5(32000, tree="heap"),
    "sd": sel_decode,
}
