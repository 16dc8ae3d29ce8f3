"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and argument validation returns the documented status
codes before anything is launched."""

import ctypes

import pytest

from sparse_attention_long_fp8_amd import binding as B


def _batch(T=4, B_=1, maxq=4, maxk=8):
    # fake, never-dereferenced device addresses: validation only reads host fields
    return B.dsa_batch_t(B_, T, 0x1000, 0x2000, maxq, maxk)


def _layout(rows=8):
    return B.dsa_kv_layout_t(0, 0x3000, None, 0, 64, rows)


def test_exports_match_header():
    lib = B.lib()
    names = B.header_functions()
    assert len(names) == 17
    for name in names:
        assert hasattr(lib, name), name


def test_projection_library_exports_and_keeps_blaslt_out_of_libdsa():
    proj = B.proj_lib()
    names = B.header_functions(B.PROJ_HEADER)
    assert names == ["dsa_blaslt_create", "dsa_blaslt_destroy", "dsa_output_projection",
                     "dsa_output_projection_workspace_size"]
    for name in names:
        assert hasattr(proj, name), name
    # the hot-path library does not link the GEMM library
    import subprocess
    deps = subprocess.run(["readelf", "-d", B.LIB_PATH], capture_output=True, text=True).stdout
    assert "hipblaslt" not in deps.lower()
    assert "hipblaslt" in subprocess.run(["readelf", "-d", B.PROJ_LIB_PATH], capture_output=True,
                                         text=True).stdout.lower()


def test_version_and_strings():
    assert B.dsa_abi_version() == 1
    assert B.dsa_status_string(0) == "DSA_OK"
    assert B.dsa_status_string(4) == "DSA_ERR_HIP"
    assert "unknown" in B.dsa_status_string(99)


def test_null_and_bad_arguments():
    lib = B.lib()
    st = lib.dsa_indexer_scores(None, None, B.DSA_F32, 4, 32, None, None, None, None, None, 1.0, None, 8, None)
    assert st == B.DSA_ERR_INVALID_ARGUMENT
    assert "batch" in B.dsa_last_error()
    bt, ly = _batch(), _layout()
    # f32 indexer must not be given scales
    st = B.dsa_indexer_scores(bt, ly, B.DSA_F32, 4, 32, 0x10, 0x20, 0x30, 0x40, 0x50, 1.0, 0x60, 8, check=False)
    assert st == B.DSA_ERR_INVALID_ARGUMENT
    # FP8 indexer only implements d_i = 128
    st = B.dsa_indexer_scores(bt, ly, B.DSA_FP8_E4M3, 64, 64, 0x100, 0x20, 0x30, 0x200, 0x50, 1.0, 0x60, 8,
                              check=False)
    assert st == B.DSA_ERR_UNSUPPORTED
    # ld_scores shorter than the longest history
    st = B.dsa_indexer_scores(bt, ly, B.DSA_F32, 4, 32, 0x10, None, 0x30, 0x40, None, 1.0, 0x60, 7, check=False)
    assert st == B.DSA_ERR_INVALID_ARGUMENT
    # queries must be the last tokens of their history
    bad = _batch(T=4, maxq=9, maxk=8)
    st = B.dsa_topk(bad, 0x1000, 8, 4, 0x2000, check=False)
    assert st == B.DSA_ERR_INVALID_ARGUMENT
    # k range, alignment of the score rows
    assert B.dsa_topk(bt, 0x1000, 8, 0, 0x2000, check=False) == B.DSA_ERR_INVALID_ARGUMENT
    assert B.dsa_topk(bt, 0x1004, 8, 4, 0x2000, check=False) == B.DSA_ERR_INVALID_ARGUMENT
    assert B.dsa_topk(bt, 0x1000, 10, 4, 0x2000, check=False) == B.DSA_ERR_INVALID_ARGUMENT
    # bf16 MLA only implements 576 / 512
    st = B.dsa_sparse_mla_fwd(bt, ly, B.DSA_BF16, 128, 128, 128, 0x100, 0x200, 0x300, 4, 0.1, 0x400, None,
                              check=False)
    assert st == B.DSA_ERR_UNSUPPORTED
    st = B.dsa_sparse_mla_fwd(bt, ly, B.DSA_BF16, 96, 576, 512, 0x100, 0x200, 0x300, 4, 0.1, 0x400, None,
                              check=False)
    assert st == B.DSA_ERR_UNSUPPORTED
    # non-finite softmax scale
    st = B.dsa_sparse_mla_fwd(bt, ly, B.DSA_F32, 4, 80, 64, 0x100, 0x200, 0x300, 4, float("inf"), 0x400, None,
                              check=False)
    assert st == B.DSA_ERR_INVALID_ARGUMENT
    # paged layout: only 64-token pages, table must cover max_k_len
    paged = B.dsa_kv_layout_t(1, None, 0x5000, 1, 32, 10)
    st = B.dsa_sparse_mla_fwd(bt, paged, B.DSA_F32, 4, 80, 64, 0x100, 0x200, 0x300, 4, 0.1, 0x400, None,
                              check=False)
    assert st == B.DSA_ERR_UNSUPPORTED
    paged = B.dsa_kv_layout_t(1, None, 0x5000, 0, 64, 10)
    st = B.dsa_sparse_mla_fwd(bt, paged, B.DSA_F32, 4, 80, 64, 0x100, 0x200, 0x300, 4, 0.1, 0x400, None,
                              check=False)
    assert st == B.DSA_ERR_INVALID_ARGUMENT


def test_workspace_sizes_and_too_small():
    # decode-sized batch: the split MLA needs partials; prefill-sized: none
    dec = B.dsa_batch_t(32, 32, 0x1000, 0x2000, 1, 32768)
    ws = B.dsa_sparse_mla_workspace_size(dec, B.DSA_BF16, 128, 576, 512, 2048)
    assert ws > 0 and ws % 4 == 0
    pre = B.dsa_batch_t(1, 16384, 0x1000, 0x2000, 16384, 16384)
    assert B.dsa_sparse_mla_workspace_size(pre, B.DSA_BF16, 128, 576, 512, 2048) == 0
    assert B.dsa_topk_workspace_size(pre, 2048) == 0
    # top-k in two passes (32768-long parts): candidate positions and scores,
    # [T, round4(min(parts * k, max_k_len))] each, 256-byte aligned
    def tk(T, max_k_len, k):
        return B.dsa_topk_workspace_size(B.dsa_batch_t(T, T, 0x1000, 0x2000, 1, max_k_len), k)
    assert tk(32, 32768, 2048) == 0                          # rows fit the LDS cache: one pass
    assert tk(32, 32769, 2048) == 2 * 32 * 4096 * 4          # a one-score second part
    assert tk(255, 70000, 2048) == 2 * 255 * 6144 * 4        # three parts
    assert tk(255, 70000, 30000) == 2 * (-(-255 * 70000 * 4 // 256) * 256)  # the list never exceeds the row
    assert tk(256, 70000, 2048) == 0                         # enough rows to fill the chip
    st = B.dsa_sparse_mla_fwd(dec, _layout(1 << 20), B.DSA_BF16, 128, 576, 512, 0x100, 0x200, 0x300, 2048, 0.04,
                              0x400, None, None, ws - 1, check=False)
    assert st == B.DSA_ERR_WORKSPACE_TOO_SMALL
    args = B.forward_args(dec, _layout(1 << 20), index_dtype=B.DSA_FP8_E4M3, h_i=64, d_i=128, q_idx=0x1000,
                          q_scale=0x2000, w=0x3000, k_idx=0x4000, k_scale=0x5000, index_scale=1.0, top_k=2048,
                          mla_dtype=B.DSA_BF16, heads=128, d_qk=576, d_v=512, q=0x6000, kv=0x7000,
                          sm_scale=0.04, out=0x8000)
    need = B.dsa_forward_workspace_size(args)
    # scores [32, 32768] fp32 + indices [32, 2048] int32 + MLA partials, each 256-byte aligned
    assert need >= 32 * 32768 * 4 + 32 * 2048 * 4 + ws
    assert B.dsa_forward(args, 0x100000, need - 1, check=False) == B.DSA_ERR_WORKSPACE_TOO_SMALL
    assert B.dsa_forward(args, 0x100010, need, check=False) == B.DSA_ERR_INVALID_ARGUMENT  # misaligned


def test_fused_indexer_topk_workspace_choice():
    """dsa_indexer_topk takes the fused kernel (candidate lists, 8 bytes per
    entry, 3k + 128 entries rounded to 64 per row, whatever the history) for
    prefill batches with contiguous keys or paged histories up to 131072 keys;
    past that, and for decode batches, the two stages (fp32 score rows, then
    top-k's own)."""
    k = 2048

    def cap(maxk):
        return (3 * k + 128 + 63) // 64 * 64

    def r256(x):
        return -(-x // 256) * 256

    def ws(T, maxq, maxk, paged):
        bt = B.dsa_batch_t(T // maxq, T, 0x1000, 0x2000, maxq, maxk)
        ly = (B.dsa_kv_layout_t(1, None, 0x5000, -(-maxk // 64), 64, 1 << 22) if paged
              else B.dsa_kv_layout_t(0, 0x3000, None, 0, 64, 1 << 22))
        return B.dsa_indexer_topk_workspace_size(bt, ly, B.DSA_FP8_E4M3, 64, 128, k)

    def unfused(T, maxq, maxk):
        return r256(T * (-(-maxk // 4) * 4) * 4) + B.dsa_topk_workspace_size(
            B.dsa_batch_t(T // maxq, T, 0x1000, 0x2000, maxq, maxk), k)

    def fused(maxk):
        return 2 * r256(4096 * cap(maxk) * 4)

    for maxk in (4096, 4097, 16384, 65536, 131072):
        assert ws(4096, 4096, maxk, False) == fused(maxk), maxk
    assert ws(4096, 4096, 131072, True) == fused(131072)
    assert ws(4096, 4096, 131073, True) == unfused(4096, 4096, 131073)
    assert ws(4096, 4096, 140000, False) == fused(140000)     # contiguous keys: no length limit
    assert ws(4096, 4096, 10 ** 6, False) == fused(10 ** 6)
    assert ws(32, 1, 32768, False) == unfused(32, 1, 32768)   # decode rows: the two stages


def test_empty_batch_launches_nothing():
    empty = B.dsa_batch_t(1, 0, None, None, 0, 0)
    ly = _layout(1)
    assert B.dsa_topk(empty, None, 0, 8, None, check=False) == B.DSA_OK
    assert B.dsa_indexer_scores(empty, ly, B.DSA_F32, 4, 32, None, None, None, None, None, 1.0, None, 0,
                                check=False) == B.DSA_OK
    assert B.dsa_sparse_mla_fwd(empty, ly, B.DSA_F32, 4, 80, 64, None, None, None, 8, 0.1, None, None,
                                check=False) == B.DSA_OK


def test_struct_layouts_match_c():
    # the ctypes mirrors must have the C sizes (x86-64 SysV)
    assert ctypes.sizeof(B.dsa_batch_t) == 32
    assert ctypes.sizeof(B.dsa_kv_layout_t) == 40
    assert B.dsa_forward_args_t.ld_scores.offset % 8 == 0


def test_struct_offsets_match_a_c_compiler(tmp_path):
    """Offsets of the ctypes mirrors equal what gcc computes from the header."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    fields = [f for f, _ in B.dsa_forward_args_t._fields_]
    src = tmp_path / "offs.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "libdsa.h"\nint main(void){\n'
        '  printf("%zu %zu %zu\\n", sizeof(dsa_batch_t), sizeof(dsa_kv_layout_t), sizeof(dsa_forward_args_t));\n'
        + "".join('  printf("%%zu\\n", offsetof(dsa_forward_args_t, %s));\n' % f for f in fields)
        + "  return 0;\n}\n")
    exe = tmp_path / "offs"
    inc = B.HEADER.rsplit("/", 1)[0]
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + inc, str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    sizes = [int(x) for x in out[:3]]
    assert sizes == [ctypes.sizeof(B.dsa_batch_t), ctypes.sizeof(B.dsa_kv_layout_t),
                     ctypes.sizeof(B.dsa_forward_args_t)]
    assert [int(x) for x in out[3:]] == [getattr(B.dsa_forward_args_t, f).offset for f in fields]


def test_cache_append_validation():
    lib = B.lib()
    ly = _layout()
    assert lib.dsa_cache_append(None, 1, 0x10, 0x20, 128, 0x100, 0x200, 0x300, 576, 0x400, 0x500, None) \
        == B.DSA_ERR_INVALID_ARGUMENT
    # d_i must be a multiple of 4, d_c a multiple of 8
    assert B.dsa_cache_append(ly, 1, 0x10, 0x20, 126, 0x100, 0x200, 0x300, check=False) == B.DSA_ERR_UNSUPPORTED
    assert B.dsa_cache_append(ly, 1, 0x10, 0x20, 128, 0x100, 0x200, 0x300, 20, 0x400, 0x500,
                              check=False) == B.DSA_ERR_UNSUPPORTED
    # alignment of the fp32 keys and of the latent rows
    assert B.dsa_cache_append(ly, 1, 0x10, 0x20, 128, 0x104, 0x200, 0x300, check=False) \
        == B.DSA_ERR_INVALID_ARGUMENT
    assert B.dsa_cache_append(ly, 1, 0x10, 0x20, 128, 0x100, 0x200, 0x300, 576, 0x408, 0x500,
                              check=False) == B.DSA_ERR_INVALID_ARGUMENT
    # a missing latent pool with d_c > 0
    assert B.dsa_cache_append(ly, 1, 0x10, 0x20, 128, 0x100, 0x200, 0x300, 576, 0x400, None,
                              check=False) == B.DSA_ERR_INVALID_ARGUMENT
    # paged pools: only 64-token pages
    paged = B.dsa_kv_layout_t(1, None, 0x3000, 4, 32, 8)
    assert B.dsa_cache_append(paged, 1, 0x10, 0x20, 128, 0x100, 0x200, 0x300, check=False) == B.DSA_ERR_UNSUPPORTED
    # no tokens: nothing to check beyond the shapes, nothing launched
    assert B.dsa_cache_append(ly, 0, None, None, 128, None, None, None, check=False) == B.DSA_OK


def test_module_forward_validation():
    """Argument checks of dsa_module_forward run before anything is launched."""
    nb = B.dsa_module_forward_workspace_size(2, 100, 64, 4, 16, 64, 8)
    ptrs = [0x100 * (i + 1) for i in range(11)]

    def call(sizes=(2, 100, 64, 4, 16, 64, 8, 32), ptr=ptrs, ws=0x10000, nbytes=nb):
        return B.dsa_module_forward(*sizes, *ptr, ws, nbytes, check=False)

    assert call(sizes=(2, 0, 64, 4, 16, 64, 8, 32)) == B.DSA_ERR_INVALID_ARGUMENT
    assert call(sizes=(2, 100, 64, 65, 16, 64, 8, 32)) == B.DSA_ERR_UNSUPPORTED    # > 64 heads
    assert call(sizes=(2, 100, 64, 4, 16, 257, 8, 32)) == B.DSA_ERR_UNSUPPORTED    # latent > 256
    assert call(sizes=(2, 100, 16385, 4, 16, 64, 8, 32)) == B.DSA_ERR_UNSUPPORTED  # hidden > 16384
    assert call(sizes=(65536, 4, 64, 4, 16, 64, 8, 32)) == B.DSA_ERR_UNSUPPORTED   # batch > 65535
    assert call(sizes=(2, 100, 64, 4, 16, 64, 8, 0)) == B.DSA_ERR_INVALID_ARGUMENT
    assert call(sizes=(32768, 65536, 64, 4, 16, 64, 8, 32)) == B.DSA_ERR_UNSUPPORTED
    assert call(ptr=ptrs[:5] + [0] + ptrs[6:]) == B.DSA_ERR_INVALID_ARGUMENT
    assert call(nbytes=nb - 1) == B.DSA_ERR_WORKSPACE_TOO_SMALL
    assert call(ws=0x10010) == B.DSA_ERR_INVALID_ARGUMENT                          # not 256-byte aligned
    assert B.lib().dsa_module_forward_workspace_size(2, 100, 64, 4, 16, 64, 8, None) == B.DSA_ERR_INVALID_ARGUMENT


def test_validate_argument_errors():
    """dsa_validate's host-side checks; nothing is launched on these."""
    bt, ly = _batch(), _layout()
    assert B.dsa_validate(bt, ly, None, 0, None, 0, None, check=False) == B.DSA_ERR_INVALID_ARGUMENT  # no report
    assert B.dsa_validate(bt, ly, None, 0, None, 0, 0x102, check=False) == B.DSA_ERR_INVALID_ARGUMENT  # unaligned
    assert B.dsa_validate(bt, ly, 0x400, 0, None, 0, 0x100, check=False) == B.DSA_ERR_INVALID_ARGUMENT  # k < 1
    assert B.dsa_validate(bt, ly, None, 0, 0x500, 7, 0x100, check=False) == B.DSA_ERR_INVALID_ARGUMENT  # ld < max_k
    paged = B.dsa_kv_layout_t(1, None, 0x3000, 4, 32, 8)
    assert B.dsa_validate(bt, paged, None, 0, None, 0, 0x100, check=False) == B.DSA_ERR_UNSUPPORTED   # page size
    bad = B.dsa_batch_t(0, 4, 0x1000, 0x2000, 4, 8)
    assert B.dsa_validate(bad, ly, None, 0, None, 0, 0x100, check=False) == B.DSA_ERR_INVALID_ARGUMENT


def test_descriptors_keep_their_arrays_alive():
    # the descriptors carry raw pointers: a temporary array passed in must live
    # as long as the descriptor, or its memory could be handed to another tensor
    import gc
    import weakref
    import torch
    arrs = [torch.arange(5, dtype=torch.int32), torch.ones(4, dtype=torch.int32), torch.zeros(2, dtype=torch.int64),
            torch.zeros((4, 3), dtype=torch.int32)]
    refs = [weakref.ref(a) for a in arrs]
    held = [B.make_batch(arrs[0], arrs[1], 4, 4, 1, 10), B.make_contiguous_layout(arrs[2], 10),
            B.make_paged_layout(arrs[3], 3, 12)]
    del arrs
    gc.collect()
    assert all(r() is not None for r in refs)
    del held
    gc.collect()
    assert all(r() is None for r in refs)
