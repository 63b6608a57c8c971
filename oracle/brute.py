"""Scalar pure-Python twin of the oracle, for tiny shapes only.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

It is written independently of attention.py: keys are walked one at a time in
position order with the online-softmax recurrence of TensorFold PR #985
("What this changes": running max m, correction c = exp(m_old - m),
l = l*c + p, o = o*c + p*v, o / l at the end) instead of the closed form, every
storage value is decoded with `struct`, and visibility is decided per key from
the rules rather than from precomputed sets.  Tree windows are decided from
node paths built forward in index order (a node's path is its parent's path
plus itself), not by walking up; the sink logit (HartsyInference PR #910) is
fed to the recurrence as one more key whose value is zero.  Agreement with
attention.py to ~1e-13 pins the vectorised indexing (GQA head mapping,
strides, causal limits, tree paths, selection dedup) and the
recurrence/closed-form equivalence.
"""

from __future__ import annotations

import math
import struct

NAN = float("nan")
INF = float("inf")


def _value(arr, idx, dtype, scale_arr=None, scale_idx=None):
    x = arr[idx]
    if dtype == "f32":
        return struct.unpack("<f", struct.pack("<f", float(x)))[0]
    if dtype == "f16":
        return struct.unpack("<e", struct.pack("<e", float(x)))[0]
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", int(x) << 16))[0]
    if dtype == "i8":
        s = struct.unpack("<f", struct.pack("<f", float(scale_arr[scale_idx])))[0]
        return int(x) * s
    if dtype == "fp8":
        # e4m3: sign, exponent (bias 7, field 0 subnormal), 3-bit mantissa; 0x7f/0xff NaN
        s = struct.unpack("<f", struct.pack("<f", float(scale_arr[scale_idx])))[0]
        c = int(x) & 0xFF
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            return float("nan")
        mag = math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10)
        return (-mag if c & 0x80 else mag) * s
    raise ValueError(dtype)


class _Online:
    """One query's running state over the keys it sees."""

    def __init__(self, d):
        self.m = -INF
        self.l = 0.0
        self.o = [0.0] * d
        self.nan = False
        self.seen = 0

    def push(self, s, vrow):
        self.seen += 1
        if math.isnan(s):
            self.nan = True
            return
        m_new = max(self.m, s)
        c = 0.0 if self.m == -INF else (math.exp(self.m - m_new) if m_new != INF else NAN)
        if s == -INF:
            p = 0.0
        elif m_new == INF:
            p = NAN
        else:
            p = math.exp(s - m_new)
        self.l = self.l * c + p if self.m != -INF else p
        self.o = [(oi * c if self.m != -INF else 0.0) + p * vi for oi, vi in zip(self.o, vrow)]
        self.m = m_new

    def result(self):
        d = len(self.o)
        if self.nan or self.m == INF or (self.m != self.m):
            return [NAN] * d
        if self.seen == 0 or self.m == -INF:
            return [0.0] * d
        return [oi / self.l for oi in self.o]


def _score(qv, kv, scale, softcap, slope, j, pos, maskv):
    s = 0.0
    for a, b in zip(qv, kv):
        s += a * b
    s *= scale
    if softcap > 0:
        s = softcap * math.tanh(s / softcap)
    if slope is not None:
        s += slope * (j - pos)
    if maskv is not None:
        s += maskv
    return s


def _tree_paths(parent):
    """paths[a] = the window nodes a sees, built in index order."""
    paths = []
    for a in range(len(parent)):
        up = int(parent[a])
        paths.append((paths[up] if 0 <= up < a else frozenset()) | {a})
    return paths


def _push_sink(st, sinks, h, d):
    if sinks is not None:
        z = struct.unpack("<f", struct.pack("<f", float(sinks[h])))[0]
        st.push(z, [0.0] * d)


def decode(*, q, k, v, kv_dtype, kv_len, causal, scale, softcap=0.0, alibi=None,
           k_scale=None, v_scale=None, tree_parent=None, sinks=None):
    S, R, Hq, D = q.shape
    cap, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = [[[None] * Hq for _ in range(R)] for _ in range(S)]
    for b in range(S):
        n = int(kv_len[b])
        paths = None if tree_parent is None else _tree_paths(tree_parent[b])
        for r in range(R):
            pos = n - R + r
            for h in range(Hq):
                g = h // G
                qv = [float(q[b, r, h, d]) for d in range(D)]
                st = _Online(D)
                for j in range(cap):
                    if j >= n:
                        continue
                    if paths is not None:
                        if j >= n - R and (j - (n - R)) not in paths[r]:
                            continue
                    elif causal and j > pos:
                        continue
                    kv = [_value(k, (b, j, g, d), kv_dtype, k_scale, (b, j, g)) for d in range(D)]
                    vv = [_value(v, (b, j, g, d), kv_dtype, v_scale, (b, j, g)) for d in range(D)]
                    s = _score(qv, kv, scale, softcap, None if alibi is None else float(alibi[h]),
                               j, pos, None)
                    st.push(s, vv)
                _push_sink(st, sinks, h, D)
                out[b][r][h] = st.result()
    return out


def prefill(*, q, k, v, kv_dtype, scale, softcap=0.0, alibi=None, q_pos=None, sel=None,
            block_size=1, mask=None, causal=False, k_scale=None, v_scale=None, sinks=None):
    R, Hq, D = q.shape
    n_kv, Hkv = k.shape[0], k.shape[1]
    G = Hq // Hkv
    out = [[None] * Hq for _ in range(R)]
    for r in range(R):
        pos = 0 if q_pos is None else int(q_pos[r])
        if sel is not None:
            ids = sorted(set(int(e) for e in sel[r] if int(e) >= 0 and int(e) * block_size < n_kv))
            keys = [e * block_size + t for e in ids for t in range(block_size)
                    if e * block_size + t < n_kv]
        else:
            keys = []
            for j in range(n_kv):
                if float(mask[r, j]) == -INF:
                    continue
                if causal and j > pos:
                    continue
                keys.append(j)
        for h in range(Hq):
            g = h // G
            qv = [float(q[r, h, d]) for d in range(D)]
            st = _Online(D)
            for j in keys:
                kv = [_value(k, (j, g, d), kv_dtype, k_scale, (j, g)) for d in range(D)]
                vv = [_value(v, (j, g, d), kv_dtype, v_scale, (j, g)) for d in range(D)]
                mv = None if mask is None else float(mask[r, j])
                s = _score(qv, kv, scale, softcap, None if alibi is None else float(alibi[h]),
                           j, pos, mv)
                st.push(s, vv)
            _push_sink(st, sinks, h, D)
            out[r][h] = st.result()
    return out
