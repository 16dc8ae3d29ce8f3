"""Instruction-level probes on the GPU: the FP8, bf16 and fp32 MFMA operand and
accumulator lane layouts the kernels rely on (with them the OCP E4M3
reading of FP8 bytes), the lane map of the LDS transpose read, and where a
global -> LDS load with an immediate offset writes."""

import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "sparse_attention_long_fp8_amd", "libdsa_probe.so")


@pytest.fixture(scope="module")
def probe(gpu):
    lib = ctypes.CDLL(PROBE)
    for name in ("dsa_probe_fp8_32x32x64", "dsa_probe_bf16_16x16x32", "dsa_probe_bf16_32x32x16",
                 "dsa_probe_f32_16x16x4"):
        getattr(lib, name).argtypes = [ctypes.c_void_p] * 4
    lib.dsa_probe_tr16.argtypes = [ctypes.c_void_p] * 5
    lib.dsa_probe_dma_offset.argtypes = [ctypes.c_void_p] * 3
    return lib


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _fp8_frags(A, Bm):
    """A [32 x 64], B [64 x 32] uint8 -> per-lane 32-byte operand registers:
    lane l holds row (A) / column (B) l % 32 and K bytes 32*(l//32) .. +32."""
    a = np.zeros((64, 32), np.uint8)
    b = np.zeros((64, 32), np.uint8)
    for l in range(64):
        a[l] = A[l % 32, 32 * (l // 32):32 * (l // 32) + 32]
        b[l] = Bm[32 * (l // 32):32 * (l // 32) + 32, l % 32]
    return a, b


def _run_fp8(probe, gpu, A, Bm):
    a, b = _fp8_frags(A, Bm)
    da, db = torch.from_numpy(a).to(gpu), torch.from_numpy(b).to(gpu)
    dd = torch.zeros((64, 16), dtype=torch.float32, device=gpu)
    assert probe.dsa_probe_fp8_32x32x64(da.data_ptr(), db.data_ptr(), dd.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    d = dd.cpu().numpy()
    # accumulator: lane l, register i -> row 8*(i//4) + 4*(l//32) + i%4, column l%32
    D = np.full((32, 32), np.nan)
    for l in range(64):
        for i in range(16):
            D[8 * (i // 4) + 4 * (l // 32) + i % 4, l % 32] = d[l, i]
    return D


def test_fp8_mfma_layout_and_products(probe, gpu):
    rng = np.random.default_rng(0)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    A = rng.choice(finite, (32, 64))
    Bm = rng.choice(finite, (64, 32))
    D = _run_fp8(probe, gpu, A, Bm)
    ref = O.decode_e4m3(A) @ O.decode_e4m3(Bm)
    scale = np.abs(O.decode_e4m3(A)) @ np.abs(O.decode_e4m3(Bm))
    # The FP8 MFMA does not round like 64 sequential fp32 additions: its
    # error reaches ~1.5e-4 of sum |a b| (measured), far above 64 fp32
    # roundings (4e-6).  Bound it at 2^-11; the indexer parity tests bound
    # its effect on scores.
    rel = np.abs(D - ref) / scale
    print("fp8 MFMA max |error| / sum|ab| = %.3g" % rel.max())
    assert rel.max() <= 2.0 ** -11


def test_fp8_mfma_reads_every_code_as_ocp_e4m3(probe, gpu):
    """All 254 finite codes times 1.0 come out as the OCP E4M3 table says;
    a NaN code poisons its whole output row."""
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    one = 0x38
    Bm = np.zeros((64, 32), np.uint8)
    for n in range(32):
        Bm[n, n] = one                       # D[m, n] = A[m, n]
    A = np.zeros((32, 64), np.uint8)
    A[:, :32] = np.array((finite * 5)[:1024], np.uint8).reshape(32, 32)   # every finite code
    D = _run_fp8(probe, gpu, A, Bm)
    assert np.array_equal(D, O.decode_e4m3(A[:, :32]))
    for nan_code in (0x7F, 0xFF):
        A = np.zeros((32, 64), np.uint8)
        A[3, 5] = nan_code
        D = _run_fp8(probe, gpu, A, Bm)
        assert np.isnan(D[3]).all() and not np.isnan(np.delete(D, 3, 0)).any()


def test_bf16_mfma_layout(probe, gpu):
    """16x16x32 bf16: lane l holds A row / B column l % 16 and K elements
    8*(l//16) .. +8; the accumulator of lane l holds rows 4*(l//16) + i."""
    rng = np.random.default_rng(1)
    A = rng.standard_normal((16, 32)).astype(np.float32)
    Bm = rng.standard_normal((32, 16)).astype(np.float32)
    At = torch.from_numpy(A).to(torch.bfloat16)
    Bt = torch.from_numpy(Bm).to(torch.bfloat16)
    a = torch.empty((64, 8), dtype=torch.bfloat16)
    b = torch.empty((64, 8), dtype=torch.bfloat16)
    for l in range(64):
        a[l] = At[l % 16, 8 * (l // 16):8 * (l // 16) + 8]
        b[l] = Bt[8 * (l // 16):8 * (l // 16) + 8, l % 16]
    da, db = a.to(gpu), b.to(gpu)
    dd = torch.zeros((64, 4), dtype=torch.float32, device=gpu)
    assert probe.dsa_probe_bf16_16x16x32(da.data_ptr(), db.data_ptr(), dd.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    d = dd.cpu().numpy()
    D = np.zeros((16, 16))
    for l in range(64):
        for i in range(4):
            D[4 * (l // 16) + i, l % 16] = d[l, i]
    ref = At.double().numpy() @ Bt.double().numpy()
    assert np.abs(D - ref).max() <= 1e-5 * np.abs(ref).max()


def test_bf16_mfma_32x32x16_layout(probe, gpu):
    """32x32x16 bf16: lane l holds A row / B column l % 32 and K elements
    8*(l//32) .. +8; accumulator register i of lane l holds row
    8*(i//4) + 4*(l//32) + i%4, column l % 32."""
    rng = np.random.default_rng(2)
    A = rng.standard_normal((32, 16)).astype(np.float32)
    Bm = rng.standard_normal((16, 32)).astype(np.float32)
    At = torch.from_numpy(A).to(torch.bfloat16)
    Bt = torch.from_numpy(Bm).to(torch.bfloat16)
    a = torch.empty((64, 8), dtype=torch.bfloat16)
    b = torch.empty((64, 8), dtype=torch.bfloat16)
    for l in range(64):
        a[l] = At[l % 32, 8 * (l // 32):8 * (l // 32) + 8]
        b[l] = Bt[8 * (l // 32):8 * (l // 32) + 8, l % 32]
    da, db = a.to(gpu), b.to(gpu)
    dd = torch.zeros((64, 16), dtype=torch.float32, device=gpu)
    assert probe.dsa_probe_bf16_32x32x16(da.data_ptr(), db.data_ptr(), dd.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    d = dd.cpu().numpy()
    D = np.full((32, 32), np.nan)
    for l in range(64):
        for i in range(16):
            D[8 * (i // 4) + 4 * (l // 32) + i % 4, l % 32] = d[l, i]
    ref = At.double().numpy() @ Bt.double().numpy()
    assert not np.isnan(D).any()
    assert np.abs(D - ref).max() <= 1e-5 * np.abs(ref).max()


def test_f32_mfma_16x16x4_layout(probe, gpu):
    """16x16x4 fp32: lane l holds A[l % 16, l // 16] and B[l // 16, l % 16];
    accumulator register i of lane l holds row 4*(l//16) + i, column l % 16.
    The products are fp32: against float64, four terms round like fp32."""
    rng = np.random.default_rng(3)
    A = rng.standard_normal((16, 4)).astype(np.float32)
    Bm = rng.standard_normal((4, 16)).astype(np.float32)
    a = np.array([A[l % 16, l // 16] for l in range(64)], np.float32)
    b = np.array([Bm[l // 16, l % 16] for l in range(64)], np.float32)
    da, db = torch.from_numpy(a).to(gpu), torch.from_numpy(b).to(gpu)
    dd = torch.zeros((64, 4), dtype=torch.float32, device=gpu)
    assert probe.dsa_probe_f32_16x16x4(da.data_ptr(), db.data_ptr(), dd.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    d = dd.cpu().numpy()
    D = np.full((16, 16), np.nan)
    for l in range(64):
        for i in range(4):
            D[4 * (l // 16) + i, l % 16] = d[l, i]
    ref = A.astype(np.float64) @ Bm.astype(np.float64)
    scale = np.abs(A.astype(np.float64)) @ np.abs(Bm.astype(np.float64))
    assert not np.isnan(D).any()
    assert (np.abs(D - ref) <= 4 * 2.0 ** -24 * scale).all()


def test_lds_transpose_read_lane_map(probe, gpu):
    """ds_read_b64_tr_b16 with lane l pointing at words 4l..4l+3: inside each
    16-lane group G, the 64 words form four rows of 16 (row r = the words of
    lanes 4r..4r+3) and lane i receives column i, i.e. words 64G + 16r + i."""
    src = torch.arange(4096, dtype=torch.int16)
    off = np.arange(64, dtype=np.int32) * 8
    doff = torch.from_numpy(off).to(gpu)
    dst = torch.zeros((64, 4), dtype=torch.int16, device=gpu)
    dsrc = src.to(gpu)
    st = probe.dsa_probe_tr16(dsrc.data_ptr(), off.ctypes.data_as(ctypes.c_void_p), doff.data_ptr(),
                              dst.data_ptr(), _stream())
    assert st == 0
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    want = np.array([[64 * (l // 16) + 16 * r + l % 16 for r in range(4)] for l in range(64)])
    assert np.array_equal(got, want)


def test_lds_dma_immediate_offset(probe, gpu):
    """global_load_lds_dwordx4 with M0 = the LDS buffer and an immediate offset
    of 256: lane l's 16 bytes come from src + 256 + 16 l and land at LDS byte
    256 + 16 l -- the immediate moves the LDS address as well as the global
    one, which the attention gather compensates for in M0."""
    src = torch.arange(512, dtype=torch.int32).view(torch.uint8).to(gpu)
    dst = torch.zeros(4096, dtype=torch.uint8, device=gpu)
    assert probe.dsa_probe_dma_offset(src.data_ptr(), dst.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    want = src.cpu().numpy()[256:1280]
    at0 = np.array_equal(got[:1024], want) and not got[1024:].any()
    at256 = np.array_equal(got[256:1280], want) and not got[:256].any() and not got[1280:].any()
    assert at256 and not at0
