"""The 16x16x32 and 32x32x16 MFMA lane layouts and the e4m3 widening that the
matrix-core kernels rely on, checked on the GPU with exact inputs (one wave,
fixed 64-lane buffers)."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "probe", "libmfma_probe.so")


def expected(a_vals, b_vals):
    # A[m][k] held by lane (k // 8) * 16 + m, element k % 8; B[k][n] by lane (k // 8) * 16 + n
    A = np.zeros((16, 32))
    B = np.zeros((32, 16))
    for l in range(64):
        for j in range(8):
            A[l % 16, 8 * (l // 16) + j] = a_vals[l, j]
            B[8 * (l // 16) + j, l % 16] = b_vals[l, j]
    C = A @ B
    d = np.zeros((64, 4))
    for l in range(64):
        for i in range(4):
            d[l, i] = C[4 * (l // 16) + i, l % 16]
    return d


@pytest.mark.parametrize("f16", [0, 1])
def test_mfma_16x16x32_layout(f16):
    if not torch.cuda.is_available():
        pytest.fail("needs a GPU")
    lib = ctypes.CDLL(LIB)
    rng = np.random.default_rng(3)
    a_vals = rng.integers(-4, 5, size=(64, 8)).astype(np.float32)
    b_vals = rng.integers(-4, 5, size=(64, 8)).astype(np.float32)
    if f16:
        a_bits = a_vals.astype(np.float16).view(np.uint16)
        b_bits = b_vals.astype(np.float16).view(np.uint16)
    else:
        a_bits = (a_vals.view(np.uint32) >> 16).astype(np.uint16)
        b_bits = (b_vals.view(np.uint32) >> 16).astype(np.uint16)
    a = torch.from_numpy(a_bits.view(np.int16).copy()).cuda()
    b = torch.from_numpy(b_bits.view(np.int16).copy()).cuda()
    d = torch.zeros((64, 4), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert lib.mfma_probe(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                          ctypes.c_void_p(d.data_ptr()), f16, ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), expected(a_vals, b_vals))


def expected32(a_vals, b_vals):
    # A[m][k] held by lane (k // 8) * 32 + m, element k % 8; B[k][n] by lane (k // 8) * 32 + n;
    # D[m][n] by lane (m // 4 % 2) * 32 + n, element (m // 8) * 4 + m % 4
    A = np.zeros((32, 16))
    B = np.zeros((16, 32))
    for l in range(64):
        for j in range(8):
            A[l % 32, 8 * (l // 32) + j] = a_vals[l, j]
            B[8 * (l // 32) + j, l % 32] = b_vals[l, j]
    C = A @ B
    d = np.zeros((64, 16))
    for l in range(64):
        for i in range(16):
            d[l, i] = C[8 * (i // 4) + 4 * (l // 32) + i % 4, l % 32]
    return d


def test_mfma_32x32x16_bf16_layout():
    if not torch.cuda.is_available():
        pytest.fail("needs a GPU")
    lib = ctypes.CDLL(LIB)
    rng = np.random.default_rng(4)
    a_vals = rng.integers(-4, 5, size=(64, 8)).astype(np.float32)
    b_vals = rng.integers(-4, 5, size=(64, 8)).astype(np.float32)
    a_bits = (a_vals.view(np.uint32) >> 16).astype(np.uint16)
    b_bits = (b_vals.view(np.uint32) >> 16).astype(np.uint16)
    a = torch.from_numpy(a_bits.view(np.int16).copy()).cuda()
    b = torch.from_numpy(b_bits.view(np.int16).copy()).cuda()
    d = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert lib.mfma32_probe(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                            ctypes.c_void_p(d.data_ptr()), ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), expected32(a_vals, b_vals))


def test_fp8_convert_matches_e4m3_definition():
    """v_cvt_f32_fp8 (the e4m3 widening the kernels use for fp8 K/V) on all 256
    codes equals the oracle's e4m3 values (TensorFold PR #911: e4m3, scale
    amax / 448): exact for every finite code, NaN for 0x7f and 0xff."""
    if not torch.cuda.is_available():
        pytest.fail("needs a GPU")
    import oracle.attention as OA
    lib = ctypes.CDLL(LIB)
    codes = np.arange(256, dtype=np.uint8)
    w = torch.from_numpy(codes.view(np.int32).copy()).cuda()          # 64 words of 4 codes
    out = torch.zeros((64, 4), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert lib.fp8_probe(ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                         ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(256).astype(np.float64)
    ref = OA.E4M3_TABLE
    assert np.array_equal(np.isnan(got), np.isnan(ref)), np.flatnonzero(np.isnan(got) != np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin]), np.flatnonzero(got[fin] != ref[fin])


def test_fp8_pair_convert_matches_e4m3_definition():
    """v_cvt_scalef32_pk_bf16_fp8 with scale 1 (the pair widening the kernels use for
    fp8 K/V): every code at every byte position gives the bf16 of its e4m3 value
    exactly (e4m3 values are all representable in bf16), NaN for 0x7f and 0xff; the
    low half of the result is the lower byte."""
    if not torch.cuda.is_available():
        pytest.fail("needs a GPU")
    import oracle.attention as OA
    lib = ctypes.CDLL(LIB)
    lanes = np.arange(256)
    codes = np.stack([(lanes + j) % 256 for j in range(4)], axis=1).astype(np.uint8)   # word l: l .. l + 3
    w = torch.from_numpy(codes.reshape(-1).view(np.int32).copy()).cuda()
    out = torch.zeros((256, 2), dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert lib.fp8_pk_probe(ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                            ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    halves = np.stack([got[:, 0] & 0xFFFF, got[:, 0] >> 16, got[:, 1] & 0xFFFF, got[:, 1] >> 16], axis=1)
    val = (halves.astype(np.uint32) << 16).view(np.float32).astype(np.float64)           # bf16 -> value
    ref = OA.E4M3_TABLE[codes]
    assert np.array_equal(np.isnan(val), np.isnan(ref)), np.argwhere(np.isnan(val) != np.isnan(ref))[:8]
    fin = ~np.isnan(ref)
    assert np.array_equal(val[fin], ref[fin]), np.argwhere((val != ref) & fin)[:8]


@pytest.mark.parametrize("num_records", [0, 64, 100, 256])
def test_buffer_range_check_covers_scalar_offset(num_records):
    """The kernels carry a tile's row offset in the scalar operand of their buffer
    loads and rely on rows past the descriptor's end reading as zeros: reads past
    num_records must return 0 whether the offset sits in the VGPR or the SGPR
    operand (every address read lies inside the allocation)."""
    if not torch.cuda.is_available():
        pytest.fail("needs a GPU")
    lib = ctypes.CDLL(LIB)
    src = torch.arange(1, 1025, dtype=torch.int32, device="cuda")
    out = torch.full((128,), -1, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert lib.buffer_range_probe(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                  num_records, ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    want = np.where(np.arange(64) * 4 < num_records, np.arange(1, 65), 0)
    assert np.array_equal(o[:64], want)
    assert np.array_equal(o[64:], want)


def test_buffer_load_to_lds_places_lane_l_at_16l():
    """buffer_load_dwordx4 ... lds (the wide int8 kernel stages raw tiles this way):
    lane l's 16 bytes land at the wave's LDS base + 16 l, whatever address it read."""
    if not torch.cuda.is_available():
        pytest.fail("needs a GPU")
    lib = ctypes.CDLL(LIB)
    src = torch.arange(1024, dtype=torch.int32, device="cuda")
    out = torch.full((256, 4), -1, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert lib.lds_dma_probe(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                             ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    s = np.arange(1024).reshape(4, 64, 4)           # [wave][16-byte chunk][word]
    want = s[:, ::-1, :].reshape(256, 4)            # lane l of wave w read chunk 63 - l
    assert np.array_equal(o, want)


def test_permlane_swaps_pair_each_lane_with_its_partner():
    """v_permlane32_swap / v_permlane16_swap with both operands x: each lane's two
    results are x[l] and x[l ^ 32] (x[l ^ 16]) in some order, so their maximum is the
    two-lane maximum the softmax kernels take with it."""
    if not torch.cuda.is_available():
        pytest.fail("needs a GPU")
    lib = ctypes.CDLL(LIB)
    x = torch.arange(1000, 1064, dtype=torch.int32, device="cuda")
    out = torch.full((64, 4), -1, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert lib.permlane_probe(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                              ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    xs = np.arange(1000, 1064)
    for l in range(64):
        assert sorted(o[l, :2]) == sorted([xs[l], xs[l ^ 32]]), (l, o[l])
        assert sorted(o[l, 2:]) == sorted([xs[l], xs[l ^ 16]]), (l, o[l])
