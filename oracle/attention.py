"""Plain FP64 attention: the definition the HIP kernels are checked against.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.

Every input is widened exactly to float64 (fp32, fp16 and bf16 values exactly;
an int8 value q with row scale s as q*s, exact in float64).  No tiling, no
fusion: for each query row and query head the visible key set is formed, every
visible key is scored, and a softmax-weighted sum of the visible values is
taken.  Only visible keys are ever read, so data in other cells (NaN included)
cannot reach a result.

Passages followed (page title; part of the page):
* Online softmax / LSE: TensorFold PR #985 "drama: backbone attention runs the
  reference's 64-key softmax tiles", section "What this changes" (running max
  m, correction exp(m_old - m), l and o rescaled, o / l at the end).  The
  oracle computes the closed form these recurrences reach: exp(s - max) / sum.
* Split over key slices merged afterwards: TensorFold PR #2595 (attn_decode
  grid of rows, heads, slices; "Kernel contract": attn_decode then attn_merge
  over fp32 partials) and strix-llama.cpp PR #115, commit message of the Vulkan
  selected-key kernel (rows split, parts combined by a split-K reduce).
* Softcap before ALiBi, unclamped F32 additive mask, exact zero for a fully
  excluded row, NaN carried through the max, the sum, the split combine and the
  epilogue: HartsyInference PR #910, PR body bullet list and the review of
  flash_attn_f32.cu / attention_softmax.cu, and the follow-up comment with
  case M03.
* Maskless selected-key visibility (only the per-query list decides; the list
  is sorted, invalid and duplicate entries skipped; K/V gathered by block):
  strix-llama.cpp PR #115, "Overview" and the commit message of the Vulkan
  selected-key kernel.
* Tree-shaped verify windows (a parent table in heap order instead of a
  causal chain; widths 1 to 16): TensorFold PR #2595, "Kernel contract" gate
  on tree widths and visible-key counts.
* Attention-sink logit (a per-head logit that joins the softmax denominator;
  -inf sink on an empty row gives 0, +inf or NaN gives NaN): HartsyInference
  PR #910, PR body first paragraph and the review of the CPU fix.

Readings where the pages are silent (each also listed in the design notes):
* a -inf mask entry excludes the key before any arithmetic (NaN data in that
  key cannot reach the row); the mask is added after ALiBi;
* an excluded row (empty visible set, or every visible score -inf) is +0.0;
* a NaN score anywhere in the visible set, or a +inf maximum, makes the whole
  row NaN; a NaN in V at dim d makes that output dim NaN;
* query head h reads kv head h // (Hq / Hkv);
* selection ids are block ids over `block_size` cells; id < 0 or
  id * block_size >= N is invalid; cells of a last partial block at or past N
  are dropped; the union over the list is a set (duplicates collapse);
* decode row r of stream b sits at position kv_len[b] - R + r;
* tree window: the last R cells of a stream are the window's nodes in order;
  node r's parent is parent[b][r] (heap order: parent < child; -1, or any
  entry outside [-1, r), makes r a root hanging off the cached prefix); row r
  sees every cell before the window plus the cells of r and its ancestors;
  ALiBi keeps the cache slot kv_len[b] - R + r as the row's position;
* the sink is a logit without a value: out = sum_j e^(s_j - M) v_j /
  (sum_j e^(s_j - M) + e^(sink - M)) with M = max(max_j s_j, sink); it is
  taken once per (row, head), after the combine of a split call, not per slice;
  it is used as given (no scale, softcap, ALiBi or mask); the NaN / +inf /
  -inf rules of the scores apply to it as to one more score.

Parity pins (tests/test_oracle_pins.py): the printed M03 example, closed forms
(softcap-then-ALiBi, F32 bias range, finite sentinel, one key, Q = 0, two-key
logistic, one key against a sink, binary-heap ancestor counts), library
reductions (scipy softmax, torch CPU SDPA in float64), invariances (split ==
unsplit, list permutation / duplicates / invalid ids, GQA == MHA with repeated
heads, chain tree == causal window, sink == one more key with a zero value),
the sink cases the review lists, and a scalar pure-Python twin (brute.py).
"""

from __future__ import annotations

import numpy as np

NAN = float("nan")
INF = float("inf")


# ----------------------------------------------------------------------------
# storage -> float64
# ----------------------------------------------------------------------------

def e4m3_value(code):
    """The real number an e4m3 byte stands for (format with maximum 448): sign
    bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 gives
    subnormals (m / 8) * 2^-6; codes 0x7f and 0xff are NaN; no infinities
    (TensorFold PR #911: e4m3 rows, scale amax / 448)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def kv_to_f64(arr, dtype, scale=None):
    """Exact widening of K or V rows to float64.

    fp32 / fp16: the value itself.  bf16 (uint16 bits): the fp32 whose high
    half is those bits.  int8: q * scale, with the per-row fp32 scale
    broadcast over the last axis (exact in float64: 8 x 24 significant bits).
    e4m3 (fp8): the byte's value times the row scale, likewise exact.
    """
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(arr, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "i8":
        q = np.asarray(arr, dtype=np.int8).astype(np.float64)
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        return q * s[..., None]
    if dtype == "fp8":
        q = E4M3_TABLE[np.asarray(arr, dtype=np.uint8)]
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        return q * s[..., None]
    raise ValueError(f"unknown kv dtype {dtype!r}")


# ----------------------------------------------------------------------------
# visible key sets
# ----------------------------------------------------------------------------

def tree_path(parent, r):
    """Window nodes row r of a tree window sees: r, its parent, and so on up to a root.

    parent[a] in [-1, a) is a's parent; any other entry ends the walk (a root)."""
    nodes = []
    a = int(r)
    while a >= 0:
        nodes.append(a)
        up = int(parent[a])
        a = up if -1 <= up < a else -1
    return sorted(nodes)


def visible_decode_row(kv_len, n_row, r, causal, parent=None):
    """Cells row r of a decode window sees: [0, kv_len - n_row + r] or [0, kv_len);
    with a tree parent table, the cells before the window plus r's path in it."""
    kv_len = int(kv_len)
    if parent is not None:
        start = kv_len - n_row
        win = start + np.asarray(tree_path(parent, r), dtype=np.int64)
        cells = np.concatenate([np.arange(max(0, start), dtype=np.int64), win])
        return cells[(cells >= 0) & (cells < kv_len)]
    lim = kv_len - n_row + r + 1 if causal else kv_len
    lim = max(0, min(lim, kv_len))
    return np.arange(lim, dtype=np.int64)


def visible_mask_row(mask_row, n_kv, causal, pos):
    """Mask mode: keys j < n_kv whose mask entry is not -inf (and j <= pos if causal)."""
    j = np.arange(n_kv, dtype=np.int64)
    keep = np.asarray(mask_row[:n_kv], dtype=np.float32) != -np.inf
    if causal:
        keep &= j <= int(pos)
    return j[keep]


def visible_selection(ids, block_size, n_kv):
    """Selection mode: the set union of the cells of every valid listed block.

    Invalid ids (id < 0 or id * block_size >= n_kv) are skipped, duplicates
    collapse, and cells at or past n_kv are dropped.  Returned sorted.
    """
    ids = np.asarray(ids, dtype=np.int64)
    ok = (ids >= 0) & (ids * block_size < n_kv)
    blocks = np.unique(ids[ok])
    cells = (blocks[:, None] * block_size + np.arange(block_size)[None, :]).reshape(-1)
    return cells[cells < n_kv]


# ----------------------------------------------------------------------------
# scores and the softmax-weighted sum
# ----------------------------------------------------------------------------

def scores(q, kc, cells, *, scale, softcap=0.0, slopes=None, pos=0, mask_vals=None):
    """Score pipeline for one query row: s = scale * q.k, then softcap, ALiBi, mask.

    q [nh][D] and kc [n][D] float64; cells [n] absolute key positions.
    softcap c > 0: s = c * tanh(s / c) (before ALiBi).  ALiBi: s += slope_h * (j - pos).
    Mask: s += mask value of that key (F32, used as is).
    """
    s = float(scale) * (np.asarray(q, np.float64) @ np.asarray(kc, np.float64).T)
    if softcap and softcap > 0:
        c = float(softcap)
        s = c * np.tanh(s / c)
    if slopes is not None:
        rel = (np.asarray(cells, np.float64) - float(pos))[None, :]
        s = s + np.asarray(slopes, np.float64)[:, None] * rel
    if mask_vals is not None:
        s = s + np.asarray(mask_vals, np.float32).astype(np.float64)[None, :]
    return s


def _row_max(sh):
    """Max of one row of scores with NaN taking precedence; -inf when empty."""
    if sh.size == 0:
        return -INF
    if np.isnan(sh).any():
        return NAN
    return float(sh.max())


def _with_sink(m, z):
    """Row maximum once the sink logit z (None = no sink) joins the scores."""
    if z is None:
        return m
    if np.isnan(m) or np.isnan(z):
        return NAN
    return max(m, z)


def attend_scores(s, vc, sink=None):
    """Normalised attention output for each score row.

    s [nh][n], vc [n][D], sink [nh] or None.  M = max of the row's scores and
    its sink.  NaN anywhere in a row or in its sink, or M = +inf, gives a NaN
    row; an empty row with no sink, or M = -inf, gives +0.0; otherwise
    sum_j exp(s_j - M) v_j / (sum_j exp(s_j - M) + exp(sink - M)).
    """
    s = np.asarray(s, np.float64)
    vc = np.asarray(vc, np.float64)
    nh = s.shape[0]
    d = vc.shape[1]
    out = np.zeros((nh, d), dtype=np.float64)
    for h in range(nh):
        z = None if sink is None else float(np.float32(sink[h]))
        m = _with_sink(_row_max(s[h]), z)
        if np.isnan(m) or m == INF:
            out[h] = NAN
        elif m == -INF:
            out[h] = 0.0
        else:
            p = np.exp(s[h] - m)
            den = p.sum() + (0.0 if z is None else np.exp(z - m))
            out[h] = (p @ vc) / den
    return out


def partial_scores(s, vc):
    """Unnormalised split partial (o, m, l) for each score row.

    Empty or all -inf: m = -inf, l = 0, o = 0.  NaN score: m = NaN (o, l NaN).
    +inf maximum: m = +inf (o, l NaN).  Else m = max, p = exp(s - m),
    l = sum p, o = sum p v.
    """
    s = np.asarray(s, np.float64)
    vc = np.asarray(vc, np.float64)
    nh = s.shape[0]
    d = vc.shape[1]
    o = np.zeros((nh, d))
    m = np.full(nh, -INF)
    l = np.zeros(nh)
    for h in range(nh):
        mh = _row_max(s[h])
        m[h] = mh
        if np.isnan(mh) or mh == INF:
            o[h] = NAN
            l[h] = NAN
        elif mh == -INF:
            pass
        else:
            p = np.exp(s[h] - mh)
            l[h] = p.sum()
            o[h] = p @ vc
    return o, m, l


def combine_partials(o, m, l, sink=None):
    """Log-sum-exp merge of split partials.

    o [ns][nh][D], m [ns][nh], l [ns][nh], sink [nh] or None.  M = max over
    slices (and the sink) with NaN propagating; M NaN or +inf -> NaN; M = -inf
    -> +0.0; otherwise slices with m_s = -inf are skipped and
    out = sum_s w_s o_s / (sum_s w_s l_s + exp(sink - M)) with w_s = exp(m_s - M).
    """
    o = np.asarray(o, np.float64)
    m = np.asarray(m, np.float64)
    l = np.asarray(l, np.float64)
    ns, nh, d = o.shape
    out = np.zeros((nh, d))
    for h in range(nh):
        mh = m[:, h]
        z = None if sink is None else float(np.float32(sink[h]))
        if np.isnan(mh).any() or (z is not None and np.isnan(z)):
            out[h] = NAN
            continue
        big = _with_sink(mh.max() if ns else -INF, z)
        if big == INF:
            out[h] = NAN
            continue
        if big == -INF:
            out[h] = 0.0
            continue
        num = np.zeros(d)
        den = 0.0
        for t in range(ns):
            if mh[t] == -INF:
                continue
            w = np.exp(mh[t] - big)
            num = num + w * o[t, h]
            den = den + w * l[t, h]
        if z is not None:
            den = den + np.exp(z - big)
        out[h] = num / den
    return out


# ----------------------------------------------------------------------------
# decode (split-K over slices, verify windows)
# ----------------------------------------------------------------------------

def _decode_row_scores(q64, k64, b, r, g, G, n_row, kv_len, causal, scale, softcap, slopes,
                       tree_parent=None):
    cells = visible_decode_row(kv_len[b], n_row, r, causal,
                               None if tree_parent is None else tree_parent[b])
    pos = int(kv_len[b]) - n_row + r
    heads = slice(g * G, (g + 1) * G)
    s = scores(q64[b, r, heads], k64[cells], cells, scale=scale, softcap=softcap,
               slopes=None if slopes is None else slopes[heads], pos=pos)
    return cells, s


def _sink_args(sinks, heads):
    return {} if sinks is None else {"sink": np.asarray(sinks)[heads]}


def decode(*, q, k, v, kv_dtype, kv_len, causal, scale, softcap=0.0, alibi=None,
           k_scale=None, v_scale=None, tree_parent=None, sinks=None):
    """Unsplit decode output [S][R][Hq][D] in float64 (the method's plain definition).

    tree_parent [S][R] (or None): each stream's window as a tree, overriding
    `causal`; sinks [Hq] (or None): one sink logit per query head."""
    S, R, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    q64 = np.asarray(q, np.float32).astype(np.float64)
    out = np.zeros((S, R, Hq, D))
    for b in range(S):
        n = int(kv_len[b])
        for g in range(Hkv):
            k64 = kv_to_f64(k[b, :n, g], kv_dtype, None if k_scale is None else k_scale[b, :n, g])
            v64 = kv_to_f64(v[b, :n, g], kv_dtype, None if v_scale is None else v_scale[b, :n, g])
            for r in range(R):
                cells, s = _decode_row_scores(q64, k64, b, r, g, G, R, kv_len, causal,
                                              scale, softcap, alibi, tree_parent)
                hs = slice(g * G, (g + 1) * G)
                out[b, r, hs] = attend_scores(s, v64[cells], **_sink_args(sinks, hs))
    return out


def decode_split(*, q, k, v, kv_dtype, kv_len, causal, scale, slice_len, softcap=0.0,
                 alibi=None, k_scale=None, v_scale=None, tree_parent=None, sinks=None):
    """Split form: per-slice partials, then the LSE combine.

    Slice t covers cells [t*L, (t+1)*L); stream b has ceil(kv_len[b] / L)
    slices.  Returns (out [S][R][Hq][D], part_o [S][R][Hq][ns][D],
    part_m [S][R][Hq][ns], part_l [S][R][Hq][ns]) with ns = max slice count.
    Slices past a stream's count stay (m=-inf, l=0, o=0).
    """
    S, R, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    L = int(slice_len)
    ns = max(1, max(-(-int(n) // L) for n in kv_len))
    q64 = np.asarray(q, np.float32).astype(np.float64)
    po = np.zeros((S, R, Hq, ns, D))
    pm = np.full((S, R, Hq, ns), -INF)
    pl = np.zeros((S, R, Hq, ns))
    out = np.zeros((S, R, Hq, D))
    for b in range(S):
        n = int(kv_len[b])
        nsb = -(-n // L)
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            k64 = kv_to_f64(k[b, :n, g], kv_dtype, None if k_scale is None else k_scale[b, :n, g])
            v64 = kv_to_f64(v[b, :n, g], kv_dtype, None if v_scale is None else v_scale[b, :n, g])
            for r in range(R):
                cells, s = _decode_row_scores(q64, k64, b, r, g, G, R, kv_len, causal,
                                              scale, softcap, alibi, tree_parent)
                for t in range(nsb):
                    sel = (cells >= t * L) & (cells < (t + 1) * L)
                    o_t, m_t, l_t = partial_scores(s[:, sel], v64[cells[sel]])
                    po[b, r, hs, t] = o_t
                    pm[b, r, hs, t] = m_t
                    pl[b, r, hs, t] = l_t
                out[b, r, hs] = combine_partials(po[b, r, hs, :nsb].transpose(1, 0, 2),
                                                 pm[b, r, hs, :nsb].T, pl[b, r, hs, :nsb].T,
                                                 **_sink_args(sinks, hs))
    return out, po, pm, pl


def visited_decode(*, kv_len, n_row, causal, slice_len, n_head_kv, tree_parent=None):
    """Per (stream, row, kv head, slice): (count, sum of cells, sum of cells^2) visited."""
    S = len(kv_len)
    L = int(slice_len)
    ns = max(1, max(-(-int(n) // L) for n in kv_len))
    st = np.zeros((S, n_row, n_head_kv, ns, 3), dtype=np.int64)
    for b in range(S):
        for r in range(n_row):
            cells = visible_decode_row(kv_len[b], n_row, r, causal,
                                       None if tree_parent is None else tree_parent[b])
            for t in range(ns):
                c = cells[(cells >= t * L) & (cells < (t + 1) * L)]
                st[b, r, :, t] = (c.size, int(c.sum()), int((c * c).sum()))
    return st


# ----------------------------------------------------------------------------
# prefill (selection mode and mask mode)
# ----------------------------------------------------------------------------

def _prefill_row_cells(r, *, n_kv, q_pos, sel, block_size, mask, causal):
    if sel is not None:
        return visible_selection(sel[r], block_size, n_kv)
    return visible_mask_row(mask[r], n_kv, causal, 0 if q_pos is None else q_pos[r])


def prefill(*, q, k, v, kv_dtype, scale, softcap=0.0, alibi=None, q_pos=None,
            sel=None, block_size=1, mask=None, causal=False, k_scale=None, v_scale=None,
            rows=None, sinks=None):
    """Prefill output [R][Hq][D] in float64; `rows` limits the work to a subset
    (the other rows are left NaN so that a sampled comparison cannot pass by accident);
    sinks [Hq] or None."""
    R, Hq, D = q.shape
    n_kv, Hkv = k.shape[0], k.shape[1]
    G = Hq // Hkv
    q64 = np.asarray(q, np.float32).astype(np.float64)
    out = np.full((R, Hq, D), NAN)
    row_ids = range(R) if rows is None else rows
    for r in row_ids:
        cells = _prefill_row_cells(r, n_kv=n_kv, q_pos=q_pos, sel=sel, block_size=block_size,
                                   mask=mask, causal=causal)
        pos = 0 if q_pos is None else int(q_pos[r])
        mvals = None if mask is None else mask[r, cells]
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            kc = kv_to_f64(k[cells, g], kv_dtype, None if k_scale is None else k_scale[cells, g])
            vc = kv_to_f64(v[cells, g], kv_dtype, None if v_scale is None else v_scale[cells, g])
            s = scores(q64[r, hs], kc, cells, scale=scale, softcap=softcap,
                       slopes=None if alibi is None else alibi[hs], pos=pos, mask_vals=mvals)
            out[r, hs] = attend_scores(s, vc, **_sink_args(sinks, hs))
    return out


def prefill_split(*, n_splits, q, k, v, kv_dtype, scale, softcap=0.0, alibi=None,
                  q_pos=None, sel=None, block_size=1, mask=None, causal=False,
                  k_scale=None, v_scale=None, rows=None, sinks=None):
    """Split prefill: key range [0, N) cut into n_splits contiguous ranges of
    ceil(N / n_splits) cells, partials per range, LSE combine."""
    R, Hq, D = q.shape
    n_kv, Hkv = k.shape[0], k.shape[1]
    G = Hq // Hkv
    step = -(-n_kv // n_splits)
    q64 = np.asarray(q, np.float32).astype(np.float64)
    out = np.full((R, Hq, D), NAN)
    row_ids = range(R) if rows is None else rows
    for r in row_ids:
        cells = _prefill_row_cells(r, n_kv=n_kv, q_pos=q_pos, sel=sel, block_size=block_size,
                                   mask=mask, causal=causal)
        pos = 0 if q_pos is None else int(q_pos[r])
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            parts = []
            for t in range(n_splits):
                c = cells[(cells >= t * step) & (cells < (t + 1) * step)]
                kc = kv_to_f64(k[c, g], kv_dtype, None if k_scale is None else k_scale[c, g])
                vc = kv_to_f64(v[c, g], kv_dtype, None if v_scale is None else v_scale[c, g])
                s = scores(q64[r, hs], kc, c, scale=scale, softcap=softcap,
                           slopes=None if alibi is None else alibi[hs], pos=pos,
                           mask_vals=None if mask is None else mask[r, c])
                parts.append(partial_scores(s, vc))
            o = np.stack([p[0] for p in parts])
            m = np.stack([p[1] for p in parts])
            l = np.stack([p[2] for p in parts])
            out[r, hs] = combine_partials(o, m, l, **_sink_args(sinks, hs))
    return out


def visited_prefill(*, n_kv, n_head_kv, q_pos=None, sel=None, block_size=1, mask=None,
                    causal=False, rows=None):
    """Per row: sorted visited cells, and for selection mode the sorted unique
    valid block ids.  Returns (list of cell arrays, list of id arrays or None)."""
    R = (sel if sel is not None else mask).shape[0]
    row_ids = range(R) if rows is None else rows
    cells_out, ids_out = [], []
    for r in row_ids:
        cells_out.append(_prefill_row_cells(r, n_kv=n_kv, q_pos=q_pos, sel=sel,
                                            block_size=block_size, mask=mask, causal=causal))
        if sel is not None:
            ids = np.asarray(sel[r], np.int64)
            ok = (ids >= 0) & (ids * block_size < n_kv)
            ids_out.append(np.unique(ids[ok]))
    return cells_out, (ids_out if sel is not None else None)
