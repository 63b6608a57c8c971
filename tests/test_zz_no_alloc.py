"""The allocation-free decode entry point (sel_attn_decode_noalloc) against the
decode + combine entry points it stands for, and against the FP64 oracle.

Two calls in a row on one device, the second smaller than the first: the
library's scratch keeps the first call's partials, and the second call must
not depend on them.  The outputs must equal those of sel_attn_decode followed
by sel_attn_split_combine bit for bit (same kernels, same partials), and the
oracle within the workload's tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
import split_flash_attention_amd as sa
from tests import hip_run
from tests.test_gpu_parity import TOL, nmse_check
from workloads import gen

pytestmark = pytest.mark.gpu


def run_noalloc(wl):
    d = hip_run.DecodeDev(wl, "cuda")
    a = sa.decode_args(q=d.q, k=d.k, v=d.v, kv_len=d.kv_len, part_o=None, part_ml=None,
                       causal=wl.causal, scale=wl.scale, softcap=wl.softcap, alibi=d.alibi,
                       slice_len=wl.slice_len, k_scale=d.ks, v_scale=d.vs, tree_parent=d.tree)
    out = torch.full(tuple(wl.q.shape), float("nan"), dtype=torch.float32, device="cuda")
    sa.sel_attn_decode_noalloc(a, out, d.sinks)
    return out


def test_noalloc_two_calls_match_decode_and_combine():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    big = gen.make_decode(seed=[41, 1], n_stream=8, n_row=4, n_head_q=32, n_head_kv=4, head_dim=256,
                          cap=9000, kv_dtype="bf16", depth_range=(1024, 9000), slice_len=1024,
                          sinks="draw")
    small = gen.make_decode(seed=[41, 2], n_stream=2, n_row=1, n_head_q=8, n_head_kv=2, head_dim=128,
                            cap=700, kv_dtype="i8", depths=[700, 95], slice_len=256)
    need = [wl.n_stream * wl.n_row * wl.n_head_q * -(-wl.cap // wl.slice_len) * (wl.head_dim + 2) * 4
            for wl in (big, small)]
    assert need[0] > need[1] and need[0] <= sa.NOALLOC_SCRATCH_BYTES
    for wl in (big, small):
        got = run_noalloc(wl)
        ref_dev = hip_run.DecodeDev(wl, "cuda")
        ref_dev.run()
        torch.cuda.synchronize()
        got_np = got.cpu().numpy()
        ref_np = ref_dev.out.cpu().numpy()
        assert got_np.tobytes() == ref_np.tobytes(), f"{wl.kv_dtype}: differs from decode + combine"
        ref = oracle.decode(q=wl.q, k=wl.k, v=wl.v, kv_dtype=wl.kv_dtype, kv_len=wl.kv_len,
                            causal=wl.causal, scale=wl.scale, softcap=wl.softcap, alibi=wl.alibi,
                            k_scale=wl.k_scale, v_scale=wl.v_scale, sinks=wl.sinks)
        nmse_check(got_np, ref, TOL[wl.kv_dtype], f"noalloc {wl.kv_dtype}")


def test_noalloc_refuses_oversize_and_partials():
    wl = gen.make_decode(seed=[41, 3], n_stream=1, n_row=1, n_head_q=4, n_head_kv=1, head_dim=128,
                         cap=64, kv_dtype="bf16", depths=[64], slice_len=64)
    d = hip_run.DecodeDev(wl, "cuda")
    out = torch.empty(tuple(wl.q.shape), dtype=torch.float32, device="cuda")
    a = sa.decode_args(q=d.q, k=d.k, v=d.v, kv_len=d.kv_len, part_o=d.part_o, part_ml=d.part_ml,
                       scale=wl.scale, slice_len=64)
    with pytest.raises(sa.SelAttnError) as e:
        sa.sel_attn_decode_noalloc(a, out)
    assert e.value.status == sa.EINVAL
