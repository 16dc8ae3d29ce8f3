"""Machine ceilings measured by the rate probes of libdsa_probe.so: dense MFMA
rates with independent accumulators (bf16 16x16x32 and 32x32x16, FP8
32x32x64), the wave64 VALU issue rate, VALU work beside running FP8 MFMAs, and
conflict-free LDS read bandwidth.  Each test prints its figures; the asserts
only catch a broken probe (a rate far below the datasheet's order of
magnitude, or the two bf16 shapes far apart), not a slow machine."""

import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "sparse_attention_long_fp8_amd", "libdsa_probe.so")
CUS = 256
SIMDS = 4 * CUS
BLOCKS = 2 * CUS  # 256-thread blocks: two waves per SIMD


@pytest.fixture(scope="module")
def lib(gpu):
    h = ctypes.CDLL(PROBE)
    h.dsa_probe_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
    h.dsa_probe_rate.restype = ctypes.c_int
    return h


@pytest.fixture(scope="module")
def out(gpu):
    return torch.empty(4096 * 1024, dtype=torch.float32, device=gpu)


def _ms(lib, out, kind, valu=0, blocks=BLOCKS, threads=256, iters=20000):
    """Milliseconds of one launch (after a short warm-up launch)."""
    stream = torch.cuda.current_stream()
    assert lib.dsa_probe_rate(kind, valu, blocks, threads, 10, out.data_ptr(), stream.cuda_stream) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    assert lib.dsa_probe_rate(kind, valu, blocks, threads, iters, out.data_ptr(), stream.cuda_stream) == 0
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def test_mfma_rates(lib, out):
    iters = 20000
    waves = BLOCKS * 4
    rates = {}
    for kind, name, flop_iter in ((0, "bf16 16x16x32", 4 * 16 * 16 * 32 * 2),
                                  (1, "bf16 32x32x16", 2 * 32 * 32 * 16 * 2),
                                  (2, "fp8 32x32x64", 2 * 32 * 32 * 64 * 2)):
        ms = _ms(lib, out, kind, iters=iters)
        rates[name] = waves * iters * flop_iter / (ms * 1e-3) / 1e15
        print("[rate] %s MFMA: %.2f PFLOP/s (%.3f ms)" % (name, rates[name], ms), flush=True)
    assert rates["bf16 16x16x32"] > 0.8 and rates["bf16 32x32x16"] > 0.8 and rates["fp8 32x32x64"] > 2.0
    assert 0.6 < rates["bf16 16x16x32"] / rates["bf16 32x32x16"] < 1.6


def test_valu_issue_and_coissue(lib, out):
    iters = 20000
    waves = BLOCKS * 4
    ms_valu = _ms(lib, out, 3, iters=iters)
    ns_per_instr = ms_valu * 1e6 / (waves * iters * 64 / SIMDS)
    print("[rate] VALU fp32 FMA, two waves per SIMD: %.3f ns per wave64 instruction per SIMD" % ns_per_instr,
          flush=True)
    base = _ms(lib, out, 2, 0, iters=iters)
    for valu in (16, 32):
        ms = _ms(lib, out, 2, valu, iters=iters)
        print("[rate] FP8 MFMA + %d VALU per MFMA: %.2fx the MFMA-only time" % (valu, ms / base), flush=True)
        assert ms >= 0.9 * base


def test_lds_read_bandwidth(lib, out):
    iters = 4000
    for threads in (256, 512, 1024):
        ms = _ms(lib, out, 4, blocks=CUS, threads=threads, iters=iters)
        per_cu = CUS * threads * iters * 8 * 16 / (ms * 1e-3) / CUS / 1e9
        print("[rate] ds_read_b128, %d threads per CU: %.0f B/ns per CU" % (threads, per_cu), flush=True)
        assert per_cu > 50
