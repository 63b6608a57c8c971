"""Run the HIP library on generator workloads (device tensors via torch).

Marshalling only: numpy arrays from `workloads` become device tensors, the
C-ABI entry points run through the binding, results come back as numpy.
"""

from __future__ import annotations

import numpy as np
import torch

import split_flash_attention_amd as sa


def kv_tensor(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
    if dtype == "i8":
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint8)).to(device)
    raise ValueError(dtype)


def _t(a, device, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


class DecodeDev:
    """Device copies of a decode workload plus output / partial buffers."""

    def __init__(self, wl, device="cuda", slice_len=None, poison_outputs=True):
        self.wl = wl
        self.device = device
        self.slice_len = int(slice_len or wl.slice_len)
        self.q = _t(wl.q, device)
        self.k = kv_tensor(wl.k, wl.kv_dtype, device)
        self.v = kv_tensor(wl.v, wl.kv_dtype, device)
        self.ks = _t(wl.k_scale, device)
        self.vs = _t(wl.v_scale, device)
        self.kv_len = _t(wl.kv_len.astype(np.int32), device)
        self.alibi = _t(wl.alibi, device)
        self.tree = _t(wl.tree_parent, device)
        self.sinks = _t(wl.sinks, device)
        S, R, Hq, D = wl.q.shape
        self.ns = -(-wl.cap // self.slice_len)
        fill = float("nan") if poison_outputs else 0.0
        self.part_o = torch.full((S, R, Hq, self.ns, D), fill, dtype=torch.float32, device=device)
        self.part_ml = torch.full((S, R, Hq, self.ns, 2), fill, dtype=torch.float32, device=device)
        self.out = torch.full((S, R, Hq, D), fill, dtype=torch.float32, device=device)
        self.dbg = None

    def args(self, dbg=False):
        wl = self.wl
        if dbg and self.dbg is None:
            S, R = wl.q.shape[:2]
            self.dbg = torch.full((S, R, wl.n_head_kv, self.ns, 3), -1, dtype=torch.int64,
                                  device=self.device)
        return sa.decode_args(q=self.q, k=self.k, v=self.v, kv_len=self.kv_len,
                              part_o=self.part_o, part_ml=self.part_ml, causal=wl.causal,
                              scale=wl.scale, softcap=wl.softcap, alibi=self.alibi,
                              slice_len=self.slice_len, k_scale=self.ks, v_scale=self.vs,
                              dbg_visit=self.dbg if dbg else None, tree_parent=self.tree)

    def combine_args(self):
        return sa.combine_args(part_o=self.part_o, part_ml=self.part_ml, out=self.out,
                               kv_len=self.kv_len, slice_len=self.slice_len, cap=self.wl.cap,
                               sinks=self.sinks)

    def run(self, dbg=False, stream=None):
        self._keep = (self.args(dbg), self.combine_args())
        sa.sel_attn_decode(self._keep[0], stream)
        sa.sel_attn_split_combine(self._keep[1], stream)


def run_decode(wl, device="cuda", slice_len=None, dbg=False, return_dev=False):
    d = DecodeDev(wl, device, slice_len)
    d.run(dbg=dbg)
    torch.cuda.synchronize()
    out = d.out.double().cpu().numpy()
    return (out, d) if return_dev else out


class PrefillDev:
    def __init__(self, wl, device="cuda", n_splits=1, poison_outputs=True):
        self.wl = wl
        self.device = device
        self.n_splits = int(n_splits)
        self.q = _t(wl.q, device)
        self.k = kv_tensor(wl.k, wl.kv_dtype, device)
        self.v = kv_tensor(wl.v, wl.kv_dtype, device)
        self.ks = _t(wl.k_scale, device)
        self.vs = _t(wl.v_scale, device)
        self.q_pos = _t(wl.q_pos, device)
        self.alibi = _t(wl.alibi, device)
        self.sel = _t(wl.sel, device)
        self.mask = _t(wl.mask, device)
        self.sinks = _t(wl.sinks, device)
        R, Hq, D = wl.q.shape
        fill = float("nan") if poison_outputs else 0.0
        self.out = torch.full((R, Hq, D), fill, dtype=torch.float32, device=device)
        self.part_o = self.part_ml = None
        if self.n_splits > 1:
            self.part_o = torch.full((1, R, Hq, self.n_splits, D), fill, dtype=torch.float32, device=device)
            self.part_ml = torch.full((1, R, Hq, self.n_splits, 2), fill, dtype=torch.float32, device=device)
        self.dbg = self.dbg_sel = None

    def args(self, dbg=False):
        wl = self.wl
        if dbg and self.dbg is None:
            R = wl.q.shape[0]
            self.dbg = torch.full((R, wl.n_head_kv, self.n_splits, 3), -1, dtype=torch.int64,
                                  device=self.device)
            if wl.sel is not None:
                self.dbg_sel = torch.full((R, wl.n_head_kv, 1 + wl.sel.shape[1]), -2,
                                          dtype=torch.int32, device=self.device)
        return sa.prefill_args(q=self.q, k=self.k, v=self.v,
                               out=self.out if self.n_splits == 1 else None,
                               scale=wl.scale, softcap=wl.softcap, alibi=self.alibi,
                               q_pos=self.q_pos, sel=self.sel, block_size=wl.block_size,
                               mask=self.mask, mask_stride_head=0, causal=wl.causal,
                               k_scale=self.ks, v_scale=self.vs, n_splits=self.n_splits,
                               part_o=self.part_o, part_ml=self.part_ml,
                               dbg_visit=self.dbg if dbg else None,
                               dbg_sel=self.dbg_sel if dbg else None, sinks=self.sinks)

    def run(self, dbg=False, stream=None):
        a = self.args(dbg)
        self._keep = [a]
        sa.sel_attn_prefill(a, stream)
        if self.n_splits > 1:
            c = sa.combine_args(part_o=self.part_o, part_ml=self.part_ml,
                                out=self.out.view(1, *self.out.shape), sinks=self.sinks)
            self._keep.append(c)
            sa.sel_attn_split_combine(c, stream)


def run_prefill(wl, device="cuda", n_splits=1, dbg=False, return_dev=False):
    d = PrefillDev(wl, device, n_splits)
    d.run(dbg=dbg)
    torch.cuda.synchronize()
    out = d.out.double().cpu().numpy()
    return (out, d) if return_dev else out
