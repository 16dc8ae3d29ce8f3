"""Machine ceilings measured by the rate probes of libdsa_probe.so: dense MFMA
rates with independent accumulators (bf16 16x16x32 and 32x32x16, FP8
32x32x64), the wave64 VALU issue rate, VALU work beside running FP8 MFMAs, and
conflict-free LDS read bandwidth, and the read rates of the attention
kernel's LDS access patterns against plain reads of the same width.  Each
test prints its figures; the asserts
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


def test_lds_attention_patterns(lib, out):
    """16-byte QK operand reads (1040-byte rows, permuted tokens) and 8-byte
    transpose reads of the P.V product against plain reads of the same width.
    A pattern whose rows meet in LDS banks reads at a fraction of the plain
    rate; the attention kernel's patterns are laid out to avoid that."""
    iters = 4000
    threads = 512
    rate = {}
    for kind, name, width in ((5, "16-byte plain", 16), (6, "16-byte QK operand", 16), (7, "16-byte QK, tokens in order", 16),
                              (8, "8-byte plain", 8), (9, "8-byte P.V transpose", 8)):
        ms = _ms(lib, out, kind, blocks=CUS, threads=threads, iters=iters)
        rate[kind] = CUS * threads * iters * 8 * width / (ms * 1e-3) / CUS / 1e9
        print("[rate] LDS %s reads, %d threads per CU: %.0f B/ns per CU" % (name, threads, rate[kind]), flush=True)
    assert rate[6] > 0.5 * rate[5] and rate[9] > 0.3 * rate[8]


def _tok(m):
    # token of A-operand row m of a 16-token half in the attention kernel
    return 4 * (m & 3) + (((m >> 1) & 2) | ((m >> 3) & 1))


def _qk_table(layout):
    """Byte offsets of eight 16-byte QK operand reads per lane (read r: half
    r % 2, K-step r // 2; lane (g, m) reads token 16 half + tok(m), 16-byte
    chunk 4 K-step + g of the row)."""
    tab = []
    for r in range(8):
        h, ks = r & 1, r >> 1
        for lane in range(64):
            g, m = lane >> 4, lane & 15
            t, c = 16 * h + _tok(m), 4 * ks + g
            tab.append({"plain": 1024 * r + 16 * lane,
                        "pitch1040": 1040 * t + 16 * c,
                        "chunk_major": 512 * c + 16 * t,
                        "chunk_major_swz": 512 * c + 16 * (t ^ (c & 1))}[layout])
    return tab


def _pv_table(layout):
    """Byte offsets of eight 8-byte transpose reads per lane (read r: half
    r % 2, 16-dim tile r // 2; lane (g, n) reads token 16 half +
    tok(4 g + n // 4), dims 4 (n % 4) .. +3 of the tile)."""
    tab = []
    for r in range(8):
        h, nt = r & 1, r >> 1
        for lane in range(64):
            g, n = lane >> 4, lane & 15
            t, q = 16 * h + _tok(4 * g + (n >> 2)), n & 3
            c = 2 * nt + (q >> 1)
            tab.append({"plain": 512 * r + 8 * lane,
                        "pitch1040": 1040 * t + 32 * nt + 8 * q,
                        "chunk_major": 512 * c + 16 * t + 8 * (q & 1),
                        "chunk_major_swz": 512 * c + 16 * (t ^ (c & 1)) + 8 * (q & 1)}[layout])
    return tab


def test_lds_tile_layouts(gpu, out):
    """Read rates of the attention tile's QK and P.V operand patterns under
    candidate LDS layouts of the 32 x 1152-byte tile: the 1040-byte row pitch,
    and chunk-major (each 16-byte column of the 32 rows contiguous, rows of
    odd columns swapped in pairs)."""
    h = ctypes.CDLL(PROBE)
    h.dsa_probe_lds_table.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    h.dsa_probe_lds_table.restype = ctypes.c_int
    iters, threads = 4000, 512
    stream = torch.cuda.current_stream()
    rates = {}
    for width, make in ((16, _qk_table), (8, _pv_table)):
        for layout in ("plain", "pitch1040", "chunk_major", "chunk_major_swz"):
            tab = make(layout)
            assert min(tab) >= 0 and max(tab) + width <= 32768 and all(o % width == 0 for o in tab)
            dtab = torch.tensor(tab, dtype=torch.int32, device=gpu)
            assert h.dsa_probe_lds_table(width, dtab.data_ptr(), 0, CUS, threads, 10, out.data_ptr(),
                                         stream.cuda_stream) == 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            assert h.dsa_probe_lds_table(width, dtab.data_ptr(), 0, CUS, threads, iters, out.data_ptr(),
                                         stream.cuda_stream) == 0
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            rates[(width, layout)] = threads * iters * 8 * width / (ms * 1e-3) / 1e9
            print("[rate] LDS %d-byte %s reads, layout %s: %.0f B/ns per CU" % (
                width, "QK operand" if width == 16 else "P.V transpose", layout, rates[(width, layout)]), flush=True)
    assert all(r > 50 for r in rates.values())
