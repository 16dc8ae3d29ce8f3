#!/usr/bin/env python3
"""Throughput of the DSA hot path (lightning indexer -> top-k -> sparse MLA)
on one MI355X, through the libdsa C ABI.

A step is one dsa_forward call over the workload's batch (indexer, top-k and
sparse MLA, with the split merge where the selections are split).  Inputs are
resident in HBM before timing starts; for the decode workloads several copies
of every input are rotated so that no step finds its inputs in the 256 MB
Infinity Cache left there by the previous one.  A second loop runs the same
passes stage by stage with HIP events recorded around each stage on the
launch stream, which gives every stage's average duration for the rooflines.

Prints one JSON line.  The headline workload (default) is the causal prefill
of 65536 tokens: FP8 indexer 64 x 128, k = 2048, 128-head 576/512 bf16 MLA,
keys with a per-256-token block drift.  The same line carries a `workloads`
object with the other four workloads, each built, timed and freed in turn.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "query-tokens/sec through indexer+top-k+sparse MLA; decode µs/step; % roofline"
HBM_PEAK = 8.0e12      # bytes/s, MI355X HBM3E
FP8_PEAK = 5.0e15      # dense FP8 MFMA flop/s
BF16_PEAK = 2.5e15     # dense BF16 MFMA flop/s
PROFILES = os.path.join(ROOT, "profiles")
# the headline: the largest workload that fits one GPU, the long causal prefill
HEADLINE = "prefill_64k"
ALL_WORKLOADS = ("prefill_64k", "prefill_16k", "decode_32k", "paged_decode", "tiny_prefill")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps of the headline workload (default: 10 prefill, 200 decode)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default: 3 prefill, 20 decode)")
    ap.add_argument("--workload", default=HEADLINE,
                    help="decode_32k | prefill_16k | prefill_64k | paged_decode | tiny_prefill")
    ap.add_argument("--others", default="all",
                    help="the other workloads measured into the line's `workloads` object: "
                         "all (default), none, or a comma-separated list")
    ap.add_argument("--copies", type=int, default=None, help="input copies rotated across steps")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of CPU oracle work for the baseline (decode and small prefill workloads)")
    ap.add_argument("--cpu-sample", type=int, default=256,
                    help="query rows of the oracle sample on prefill workloads past 16384 rows")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run the plain copy kernel on MIB mebibytes (counter calibration) and exit")
    ap.add_argument("--op", default="forward",
                    choices=["forward", "cache_append", "output_projection", "module_forward"],
                    help="forward: the hot path (default); cache_append: the decode-step cache append "
                         "(--workload append_prefill_16k | append_decode_64); output_projection: W_UV then W_O "
                         "(--workload proj_decode_32 | proj_prefill_16k); module_forward: the complete fp32 "
                         "module at its verification shape (--workload module_2x16k)")
    return ap.parse_args()


# --------------------------------------------------------------------------
# algorithmic work of each stage (what the method must move / compute)
# --------------------------------------------------------------------------
def stage_work(wl, lay):
    rows_n = []
    for b in range(wl.batch):
        nq = int(lay.q_seq_start[b + 1] - lay.q_seq_start[b])
        kl = int(lay.k_len[b])
        rows_n.extend(range(kl - nq + 1, kl + 1))
    n = np.array(rows_n, dtype=np.float64)
    T = len(rows_n)
    m = np.minimum(n, wl.top_k)
    pairs, sel = n.sum(), m.sum()
    if wl.fp8:
        idx_bytes = pairs * (wl.d_i + 4 + 4) + T * (wl.h_i * wl.d_i + 4 + 4 * wl.h_i)
        el = 2
    else:
        idx_bytes = pairs * (4 * wl.d_i + 4) + T * (4 * wl.h_i * wl.d_i + 4 * wl.h_i)
        el = 4
    return {
        "indexer": {"bytes": idx_bytes, "flops": pairs * wl.h_i * wl.d_i * 2,
                    "peak_flops": FP8_PEAK if wl.fp8 else 157.3e12},
        "topk": {"bytes": pairs * 4 + T * wl.top_k * 4, "flops": 0.0, "peak_flops": None},
        "mla": {"bytes": sel * wl.d_qk * el + T * wl.heads * (wl.d_qk + wl.d_v) * el + T * wl.heads * 4
                + T * wl.top_k * 4,
                "flops": sel * wl.heads * (wl.d_qk + wl.d_v) * 2,
                "peak_flops": BF16_PEAK if wl.fp8 else 157.3e12},
        "pairs": pairs, "selected": sel, "queries": T,
    }


KERNEL_SOURCES = {"indexer": "indexer.hip", "topk": "topk.hip", "mla": "sparse_mla.hip", "indexer_topk": "indexer.hip"}
def kernel_name(stage, wl, lay):
    """The kernel a stage's time is attributed to (the launcher's choice)."""
    if stage == "indexer_topk":
        return "indexer_topk_fused_kernel"
    if stage == "indexer":
        if not wl.fp8:
            return "indexer_f32_kernel"
        return "indexer_fp8_tiled_kernel" if lay.max_q_per_seq >= 8 else "indexer_fp8_staged_kernel"
    if stage == "topk":
        # rows loaded before their length is known: decode batches (one query
        # row per sequence) selected in one pass (not past 32768 keys in a
        # batch of fewer than 256 rows)
        two_pass = lay.num_queries < 256 and lay.max_k_len > 32768
        one_per_seq = lay.num_queries == wl.batch and lay.max_q_per_seq == 1
        return "topk_kernel<true>" if one_per_seq and not two_pass else "topk_kernel<false>"
    if not wl.fp8:
        return "mla_f32_kernel"
    # the bf16 launcher's split count: about one workgroup per CU, at least four
    # 32-slot tiles and at most 2048 slots per range, at most 32 ranges
    T, k = lay.num_queries, wl.top_k
    s = min(-(-256 // max(T, 1)), -(-k // 128))
    s = min(max(s, -(-k // 2048)), 32)
    return "mla_bf16_kernel + mla_combine_kernel" if s > 1 else "mla_bf16_kernel"


def fused_applies(wl, lay):
    """Whether dsa_forward without kept scores takes the fused indexer ->
    top-k kernel (the launcher's choice): FP8, 32, 64 or 128 x 128 indexer
    heads, contiguous keys or paged histories of at most 131072 keys, at
    least 8 query rows per sequence."""
    return (wl.fp8 and wl.h_i in (32, 64, 128) and wl.d_i == 128 and lay.max_q_per_seq >= 8
            and (not wl.paged or lay.max_k_len <= 131072))


def source_hash(stage):
    """Hash of the stage's kernel source and of the device helpers every
    kernel includes: a change to either invalidates the stage's counters."""
    csrc = os.path.join(ROOT, "sparse_attention_long_fp8_amd", "csrc")
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[stage], "dsa_device.h"):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def traffic_of(stage, workload):
    """HBM bytes per launch from committed counter summaries, if they were
    taken on the current kernel source; None otherwise."""
    path = os.path.join(PROFILES, "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(stage)
    if not rec or rec.get("source_sha256_16") != source_hash(stage):
        return None
    return rec["hbm_bytes_per_launch"]


# --------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the same workload)
# --------------------------------------------------------------------------
def host_info():
    """BLAS threads the oracle runs on, the CPU model and the BLAS library."""
    cores, blas = 1, "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            cores = max(i["num_threads"] for i in libs)
            blas = "%s %s" % (libs[0].get("internal_api"), libs[0].get("version"))
    except Exception:  # pragma: no cover
        pass
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return int(cores), model, blas


def prefill_sample_rows(L, k, count, seed=0):
    """Deterministic oracle sample of a long causal prefill: the rows at the
    ends and around the k boundary (0, 1, k-2, k-1, k, k+1, L-1), plus one
    seeded row in each of count-7 equal strata of [0, L)."""
    fixed = sorted({r for r in (0, 1, k - 2, k - 1, k, k + 1, L - 1) if 0 <= r < L})
    n_strata = max(count - len(fixed), 0)
    rng = np.random.default_rng(seed)
    edges = np.linspace(0, L, n_strata + 1).astype(np.int64)
    strat = [int(rng.integers(edges[i], max(edges[i + 1], edges[i] + 1))) for i in range(n_strata)]
    return fixed, strat


def cpu_baseline(wl, synth_obj, budget_s, sample_rows=256):
    """The oracle as it stands, timed on this host over a bounded sample.

    Long prefills (more than 16384 rows): the fixed + stratified rows of
    prefill_sample_rows, each stage timed apart; the indexer and top-k times
    scale to every row by sum(t + 1) (the candidates), the attention time by
    sum(min(k, t + 1)) (the selected rows).  Other workloads: rows in order
    (decode) or a seeded permutation (prefill), each row repeated until its
    share of budget_s is spent.  Regenerating a row's inputs is never timed."""
    from oracle import dsa_oracle as O
    lay = synth_obj.layout
    rows = O.query_rows(lay.q_seq_start, lay.k_len)
    cores, model, blas = host_info()
    host = {"cores": cores, "cpu_model": model, "blas": blas}
    dec = (lambda c, s: O.dequant_e4m3(c, s)) if wl.fp8 else (lambda c, s: c.astype(np.float64))
    dec_bf = O.decode_bf16 if wl.fp8 else (lambda x: x.astype(np.float64))

    if wl.kind == "prefill" and len(rows) > 16384:
        L, k = len(rows), wl.top_k
        fixed, strat = prefill_sample_rows(L, k, sample_rows)
        sample = sorted(set(fixed) | set(strat))
        kc, ks = synth_obj.ki(0, L)
        keys = dec(kc, ks)
        kv = dec_bf(synth_obj.kv(0, L))
        # every sampled row's inputs first (each regenerates its 256-row chunk,
        # so the rows are drawn in parallel), then the timed oracle calls
        from concurrent.futures import ThreadPoolExecutor

        def inputs(t):
            qc, qs = synth_obj.qi(t, t + 1)
            return dec(qc, qs)[0], synth_obj.w(t, t + 1)[0], dec_bf(synth_obj.q(t, t + 1))[0]

        with ThreadPoolExecutor(min(16, max(cores, 1))) as ex:
            row_in = dict(zip(sample, ex.map(inputs, sample)))
        t_sel = t_att = 0.0
        for t in sample:
            n = rows[t][2]
            qi_h, w, q_h = row_in.pop(t)
            t0 = time.perf_counter()
            sc = O.indexer_scores(qi_h, w, keys[:n], wl.index_scale)
            idx = O.topk_indices(sc, k)
            t1 = time.perf_counter()
            O.sparse_mla(q_h, kv[:n], idx, wl.d_v, wl.sm_scale)
            t2 = time.perf_counter()
            t_sel += t1 - t0
            t_att += t2 - t1
        n_all = np.arange(1, L + 1, dtype=np.float64)
        n_smp = np.array([rows[t][2] for t in sample], dtype=np.float64)
        f_sel = n_all.sum() / n_smp.sum()
        f_att = np.minimum(n_all, k).sum() / np.minimum(n_smp, k).sum()
        total = t_sel * f_sel + t_att * f_att
        return dict(host, value=L / total, unit="query-tokens/s", kind="oracle", extrapolated=True,
                    sample="%d of %d query rows of %s (rows %s, plus one seeded row in each of %d equal strata); "
                           "indexer + top-k time %.2f s scaled by sum(t+1) (x%.1f), attention time %.2f s "
                           "scaled by sum(min(k, t+1)) (x%.1f): extrapolated %.0f s for all rows; float64 numpy"
                           % (len(sample), L, wl.name, fixed, len(strat), t_sel, f_sel, t_att, f_att, total))

    order = list(range(len(rows)))
    if wl.kind == "prefill":  # spread the sample over the causal range
        order = list(np.random.default_rng(0).permutation(len(rows)))
    done = rows_seen = 0
    elapsed = 0.0
    # Each row's inputs are generated once and its oracle call repeats until
    # the row's share of the budget is spent, so a workload of few rows (32
    # decodes) still gets a sample of about budget_s seconds.
    per_row = budget_s / len(order)
    for t in order:
        b, p, n = rows[t]
        base = int(lay.k_seq_start[b])
        qc, qs = synth_obj.qi(t, t + 1)
        kc, ks = synth_obj.ki(base, base + n)
        qi_h, ki_h = dec(qc, qs)[0], dec(kc, ks)
        q_h, kv_h = dec_bf(synth_obj.q(t, t + 1))[0], dec_bf(synth_obj.kv(base, base + n))
        w = synth_obj.w(t, t + 1)[0]
        row_time = 0.0
        while True:
            t0 = time.perf_counter()
            O.forward_row(qi_h, w, ki_h, q_h, kv_h, n, wl.top_k, wl.index_scale, wl.d_v, wl.sm_scale)
            dt = time.perf_counter() - t0
            elapsed += dt
            row_time += dt
            done += 1
            if row_time >= per_row or elapsed > budget_s:
                break
        rows_seen += 1
        if elapsed > budget_s:
            break
    return dict(host, value=done / elapsed, unit="query-tokens/s", kind="oracle", extrapolated=False,
                sample="%d oracle calls over %d of %d query rows of %s (%s), each the full path: indexer over "
                       "all n_t keys, top-k, sparse MLA; float64 numpy; %.1f s of oracle time" % (
                           done, rows_seen, len(rows), wl.name,
                           "first rows" if wl.kind != "prefill" else "random rows", elapsed))


# --------------------------------------------------------------------------
def calibrate_copy(mib):
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_long_fp8_amd", "libdsa_probe.so"))
    lib.dsa_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p]
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        assert lib.dsa_probe_copy(src.data_ptr(), dst.data_ptr(), n, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


# --------------------------------------------------------------------------
APPEND_WORKLOADS = {
    # one new token for each of 64 paged sequences of 4096 cached tokens
    "append_decode_64": {"tokens": 64, "paged": True, "seqs": 64, "k_len": 4096},
    # a 16384-token prefill chunk written into one contiguous history
    "append_prefill_16k": {"tokens": 16384, "paged": False, "seqs": 1, "k_len": 16384},
}


def bench_cache_append(args):
    """Times dsa_cache_append and prints one JSON line (its own metric)."""
    import torch
    from oracle import cache_oracle  # CPU baseline leg only
    from sparse_attention_long_fp8_amd import binding as B

    name = args.workload if args.workload in APPEND_WORKLOADS else "append_prefill_16k"
    cfg = APPEND_WORKLOADS[name]
    d_i, d_c, ps = 128, 576, 64
    N, S, L = cfg["tokens"], cfg["seqs"], cfg["k_len"]
    steps = args.steps if args.steps is not None else 200
    warmup = args.warmup if args.warmup is not None else 20
    copies = args.copies if args.copies is not None else 4
    dev = torch.device("cuda:0")
    B.lib()
    rng = np.random.default_rng(21)
    if cfg["paged"]:
        pages = S * (L // ps)
        table = rng.permutation(pages).astype(np.int32).reshape(S, L // ps)
        tab_d = torch.from_numpy(table).to(dev)
        layout = B.make_paged_layout(tab_d, L // ps, pages, ps)
        layout_np = {"paged": True, "page_table": table, "page_size": ps}
        rows_shape = (pages, ps)
        seq = np.arange(S, dtype=np.int32)
        pos = np.full(S, L - 1, np.int32)
    else:
        ks = np.array([0, L], np.int64)
        ks_d = torch.from_numpy(ks).to(dev)
        layout = B.make_contiguous_layout(ks_d, L)
        layout_np = {"k_seq_start": ks}
        rows_shape = (L,)
        seq = np.zeros(N, np.int32)
        pos = np.arange(N, dtype=np.int32)
    k_pool = torch.zeros(rows_shape + (d_i,), dtype=torch.uint8, device=dev)
    s_pool = torch.zeros(rows_shape, dtype=torch.float32, device=dev)
    l_pool = torch.zeros(rows_shape + (d_c,), dtype=torch.int16, device=dev)
    seq_d, pos_d = torch.from_numpy(seq).to(dev), torch.from_numpy(pos).to(dev)
    k_new = [torch.randn(N, d_i, device=dev) for _ in range(copies)]
    lat = [torch.randint(-16384, 16384, (N, d_c), dtype=torch.int16, device=dev) for _ in range(copies)]
    stream = torch.cuda.current_stream()

    def step(i):
        B.dsa_cache_append(layout, N, seq_d, pos_d, d_i, k_new[i % copies], k_pool, s_pool, d_c,
                           lat[i % copies], l_pool, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    per_token = d_i * 4 + d_c * 2 + 8 + d_i + 4 + d_c * 2  # reads (key, latent, seq, pos) + writes
    achieved = N * per_token / (ms / 1e3)
    result = {
        "metric": "tokens/sec appended to the caches (E4M3 indexer key + scale, bf16 latent row)",
        "value": N / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32->e4m3+bf16", "data": "synthetic",
        "config": {"workload": name, "tokens": N, "d_i": d_i, "d_c": d_c, "paged": cfg["paged"],
                   "input_copies": copies},
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK, "traffic": None, "kernel": "cache_append_kernel",
                     "bytes_per_token": per_token},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        m = min(N, 2048)
        kn = k_new[0][:m].cpu().numpy()
        ln = lat[0][:m].cpu().numpy().view(np.uint16)
        kp = np.zeros(rows_shape + (d_i,), np.uint8)
        sp = np.zeros(rows_shape, np.float32)
        lp = np.zeros(rows_shape + (d_c,), np.uint16)
        t0 = time.perf_counter()
        cache_oracle.cache_append(layout_np, seq[:m], pos[:m], kn, ln, kp, sp, lp)
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": m / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                  "sample": "first %d of %d tokens of %s; float32/float64 numpy, one thread of "
                                            "Python per token; %.2f s" % (m, N, name, el)}
    print(json.dumps(result))


PROJ_WORKLOADS = {"proj_decode_32": 32, "proj_prefill_16k": 16384}


def bench_output_projection(args):
    """Times dsa_output_projection (DeepSeek-V3 widths: 128 heads, d_c 512,
    d_h 128, hidden 7168) and prints one JSON line (its own metric)."""
    import torch
    from sparse_attention_long_fp8_amd import binding as B

    name = args.workload if args.workload in PROJ_WORKLOADS else "proj_prefill_16k"
    T = PROJ_WORKLOADS[name]
    H, d_c, d_h, hidden = 128, 512, 128, 7168
    decode = T <= 64
    steps = args.steps if args.steps is not None else (200 if decode else 20)
    warmup = args.warmup if args.warmup is not None else (20 if decode else 3)
    dev = torch.device("cuda:0")
    B.lib()
    g = torch.Generator(device=dev).manual_seed(5)
    o = torch.randn(T, H, d_c, device=dev, generator=g).to(torch.bfloat16)
    w_uv = (torch.randn(H * d_h, d_c, device=dev, generator=g) / d_c ** 0.5).to(torch.bfloat16)
    # weights rotate over copies so that decode steps stream them from HBM
    copies = 2 if decode else 1
    w_o = [(torch.randn(hidden, H * d_h, device=dev, generator=g) / (H * d_h) ** 0.5).to(torch.bfloat16)
           for _ in range(copies)]
    out = torch.empty(T, hidden, dtype=torch.bfloat16, device=dev)
    nb = B.dsa_output_projection_workspace_size(T, H, d_h)
    ws = torch.empty(nb + 256, dtype=torch.uint8, device=dev)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    h = B.dsa_blaslt_create()
    stream = torch.cuda.current_stream()

    def step(i):
        B.dsa_output_projection(h, T, H, d_c, d_h, hidden, o, w_uv, w_o[i % copies], out, base, nb, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    B.dsa_blaslt_destroy(h)
    flops = 2.0 * T * (H * d_h * d_c + hidden * H * d_h)
    nbytes = 2.0 * (H * d_h * d_c + hidden * H * d_h + T * H * d_c + T * hidden + 2 * T * H * d_h)
    if decode:
        roof = {"bound": "hbm", "achieved": nbytes / (ms / 1e3) / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": nbytes / (ms / 1e3) / HBM_PEAK}
    else:
        roof = {"bound": "mfma", "achieved": flops / (ms / 1e3) / 1e12, "peak": BF16_PEAK / 1e12,
                "unit": "TFLOP/s", "frac": flops / (ms / 1e3) / BF16_PEAK}
    roof.update({"traffic": None, "kernel": "hipBLASLt GEMMs (W_UV batched over heads, then W_O)",
                 "flops": flops, "bytes": nbytes})
    print(json.dumps({
        "metric": "query-tokens/sec through the output projections (W_UV per head, then W_O)",
        "value": T / (ms / 1e3), "unit": "query-tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "queries": T, "heads": H, "d_c": d_c, "d_h": d_h, "hidden": hidden,
                   "weight_copies": copies},
        "roofline": roof, "cpu_baseline": None}))


MODULE_WORKLOADS = {"module_2x16k": dict(B=2, S=16384, hidden=1024, H=16, d_h=64, d_c=256, d_i=32, top_k=512)}


def module_cpu_baseline(c, budget_s):
    """The oracle's module (float64 numpy) on whole batch elements of the
    same shape until budget_s seconds of oracle time have passed."""
    from oracle import module_oracle as M
    rng = np.random.default_rng(11)
    lin = lambda o, i: rng.uniform(-i ** -0.5, i ** -0.5, (o, i)).astype(np.float32)
    hidden, H, d_h, d_c, d_i = c["hidden"], c["H"], c["d_h"], c["d_c"], c["d_i"]
    W = [lin(d_i, hidden), lin(d_i, hidden), lin(H * d_h, hidden), lin(H * d_h, d_c), lin(H * d_h, d_c),
         lin(hidden, H * d_h)]
    qh = rng.standard_normal((1, hidden)).astype(np.float32)
    hist = rng.standard_normal((1, c["S"], hidden)).astype(np.float32)
    lat = rng.standard_normal((1, c["S"], d_c)).astype(np.float32)
    done, elapsed = 0, 0.0
    while elapsed < budget_s:  # one input set, reused: generating it is not timed and costs more than a call
        t0 = time.perf_counter()
        M.module_forward(qh, hist, lat, *W, c["top_k"], H, d_h)
        elapsed += time.perf_counter() - t0
        done += 1
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max(i["num_threads"] for i in blas) if blas else 1
    except Exception:  # pragma: no cover
        cores = 1
    return {"value": done / elapsed, "unit": "query-tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": "%d calls on one batch element (one query over a %d-token history), the whole module; "
                      "float64 numpy; %.1f s of oracle time" % (done, c["S"], elapsed)}


def bench_module_forward(args):
    """Times dsa_module_forward (fp32: indexer projections, indexer scores,
    top-k, query projection and W_UK absorption, sparse softmax over latent
    rows, W_UV and W_out) at the verification shape of the module's page and
    prints one JSON line (its own metric)."""
    import torch
    from sparse_attention_long_fp8_amd import binding as B

    name = args.workload if args.workload in MODULE_WORKLOADS else "module_2x16k"
    c = MODULE_WORKLOADS[name]
    Bn, S, hidden, H, d_h, d_c, d_i, k = (c[x] for x in ("B", "S", "hidden", "H", "d_h", "d_c", "d_i", "top_k"))
    steps = args.steps if args.steps is not None else 100
    warmup = args.warmup if args.warmup is not None else 10
    dev = torch.device("cuda:0")
    B.lib()
    g = torch.Generator(device=dev).manual_seed(9)
    lin = lambda o, i: (torch.rand(o, i, device=dev, generator=g) * 2 - 1) * i ** -0.5
    W = [lin(d_i, hidden), lin(d_i, hidden), lin(H * d_h, hidden), lin(H * d_h, d_c), lin(H * d_h, d_c),
         lin(hidden, H * d_h)]
    # three copies of the history (3 x 134 MB) rotate so that every step reads it from HBM, not the
    # 256 MB last-level cache
    copies = 3
    qh = [torch.randn(Bn, hidden, device=dev, generator=g) for _ in range(copies)]
    hist = [torch.randn(Bn, S, hidden, device=dev, generator=g) for _ in range(copies)]
    lat = [torch.randn(Bn, S, d_c, device=dev, generator=g) for _ in range(copies)]
    out = torch.empty(Bn, hidden, device=dev)
    idx = torch.empty(Bn, k, dtype=torch.int32, device=dev)
    nb = B.dsa_module_forward_workspace_size(Bn, S, hidden, H, d_h, d_c, d_i)
    ws = torch.empty(nb + 256, dtype=torch.uint8, device=dev)
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    stream = torch.cuda.current_stream()

    def step(i):
        j = i % copies
        B.dsa_module_forward(Bn, S, hidden, H, d_h, d_c, d_i, k, qh[j], hist[j], lat[j], *W, out, idx, base, nb,
                             stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    m = min(k, S)
    weights = d_i * hidden * 2 + H * d_h * hidden + 2 * H * d_h * d_c + hidden * H * d_h
    # history once, score rows written and read once, selected latent rows, weights, h_q and out
    nbytes = 4.0 * (Bn * S * hidden + Bn * S * 2 + Bn * m * d_c + weights + 2 * Bn * hidden)
    cpu = None if args.no_cpu_baseline else module_cpu_baseline(c, args.cpu_budget)
    print(json.dumps({
        "metric": "query-tokens/sec through the complete DSA module (fp32)",
        "value": Bn / (ms / 1e3), "unit": "query-tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, **c, "input_copies": copies},
        "roofline": {"bound": "hbm", "achieved": nbytes / (ms / 1e3) / 1e9, "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": nbytes / (ms / 1e3) / HBM_PEAK, "traffic": None,
                     "kernel": "whole step (most of its bytes are the history read by the indexer scoring)",
                     "bytes": nbytes},
        "cpu_baseline": cpu}))


def measure(wl, steps, warmup, copies, dev, log):
    """Times one workload on the GPU: the dsa_forward loop (the step), the
    stage-by-stage loop (each stage's duration), and where dsa_forward takes
    the fused indexer -> top-k kernel, that call alone.  Returns the figures
    of the line (everything but the CPU baseline) and the device workload."""
    import torch
    from sparse_attention_long_fp8_amd import binding as B
    from sparse_attention_long_fp8_amd.workload import DeviceWorkload

    decode = wl.kind != "prefill"
    dw = DeviceWorkload(wl, dev, copies=copies, log=log)
    lay, T = dw.lay, dw.T
    stream = torch.cuda.current_stream()

    log("%s: warmup %d, timed %d steps, %d input copies" % (wl.name, warmup, steps, copies))
    dw.prepare_forward()
    for i in range(warmup):
        dw.forward_prepared(i, stream)
        dw.step(i, stream)
    torch.cuda.synchronize()
    # Throughput: back-to-back passes through the fused entry point, nothing
    # else on the stream inside the timed region.
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(steps):
        dw.forward_prepared(warmup + i, stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_begin.elapsed_time(t_end) / steps
    # Per-kernel durations: the same passes stage by stage with HIP events
    # recorded around each stage on the launch stream (the event records add
    # a few microseconds between stages, so this loop does not give the step).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        dw.step(warmup + i, stream, evs[i])
    torch.cuda.synchronize()
    stage_ms = {
        "indexer": float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
        "topk": float(np.mean([e[1].elapsed_time(e[2]) for e in evs])),
        "mla": float(np.mean([e[2].elapsed_time(e[3]) for e in evs])),
    }
    # Where dsa_forward takes the fused indexer -> top-k kernel (prefill), time
    # that call too: it replaces the first two stages inside the step.
    fused = fused_applies(wl, lay)
    if fused:
        qi0, qs0, w0, _, ki0, ks0, _ = dw.sets[0]
        nb = B.dsa_indexer_topk_workspace_size(dw.batch, dw.layout, dw.index_dtype, wl.h_i, wl.d_i, wl.top_k)
        fws = torch.empty(nb + 256, dtype=torch.uint8, device=dev)
        fbase = fws.data_ptr() + (-fws.data_ptr()) % 256

        def fused_call():
            B.dsa_indexer_topk(dw.batch, dw.layout, dw.index_dtype, wl.h_i, wl.d_i, qi0, qs0, w0, ki0, ks0,
                               wl.index_scale, wl.top_k, dw.idx, fbase, nb, stream=stream)

        fused_call()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        f0.record(stream)
        for _ in range(steps):
            fused_call()
        f1.record(stream)
        torch.cuda.synchronize()
        stage_ms["indexer_topk"] = f0.elapsed_time(f1) / steps
        del fws
    work = stage_work(wl, lay)
    work["indexer_topk"] = dict(work["indexer"])
    rooflines = {}
    for st_name in stage_ms:
        t_s = stage_ms[st_name] / 1e3
        wk = work[st_name]
        if decode or wk["peak_flops"] is None:
            ach = wk["bytes"] / t_s
            rooflines[st_name] = {"bound": "hbm", "achieved": ach / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                                  "frac": ach / HBM_PEAK}
        else:
            ach = wk["flops"] / t_s
            rooflines[st_name] = {"bound": "mfma", "achieved": ach / 1e12, "peak": wk["peak_flops"] / 1e12,
                                  "unit": "TFLOP/s", "frac": ach / wk["peak_flops"]}
        rooflines[st_name]["traffic"] = traffic_of(st_name, wl.name)
        rooflines[st_name]["kernel"] = kernel_name(st_name, wl, lay)
        rooflines[st_name]["us"] = stage_ms[st_name] * 1e3
    # The kernels the step runs: with the fused kernel, indexer_topk replaces
    # the indexer and top-k stages.
    in_step = ["indexer_topk", "mla"] if fused else ["indexer", "topk", "mla"]
    dominant = max(in_step, key=stage_ms.get)
    # The path's own fraction over indexer + attention (decode: algorithmic
    # bytes of both against HBM, top-k apart; prefill: both stages' flops each
    # at its own dtype's peak).  With the fused kernel the indexer time is the
    # fused call's, which includes the selection.
    t_ix = stage_ms["indexer_topk"] if fused else stage_ms["indexer"]
    t_path = (t_ix + stage_ms["mla"]) / 1e3
    if decode:
        path = {"bound": "hbm", "frac": (work["indexer"]["bytes"] + work["mla"]["bytes"]) / HBM_PEAK / t_path,
                "definition": "(indexer bytes + attention bytes) / (8 TB/s x (t_indexer + t_attention))"}
    else:
        f_ideal = work["indexer"]["flops"] / work["indexer"]["peak_flops"] + work["mla"]["flops"] / work["mla"]["peak_flops"]
        path = {"bound": "mfma", "frac": f_ideal / t_path,
                "definition": ("(indexer flops / FP8 peak + attention flops / bf16 peak) / (t_indexer_topk "
                               "+ t_attention): the fused indexer -> top-k call as the step runs it")
                if fused else "(indexer flops / its peak + attention flops / its peak) / (t_indexer + t_attention)"}
        if fused:
            path["unfused_frac"] = f_ideal / ((stage_ms["indexer"] + stage_ms["mla"]) / 1e3)
    path["us"] = t_path * 1e6
    fig = {
        "value": T / (ms_step / 1e3),
        "ms_per_step": ms_step,
        "steps": steps,
        "warmup": warmup,
        "decode_us_per_step": ms_step * 1e3 if decode else None,
        "dtype": "fp8_e4m3+bf16" if wl.fp8 else "f32",
        "config": {"workload": wl.name, "queries": T, "batch": wl.batch, "kind": wl.kind,
                   "max_ctx": lay.max_k_len, "top_k": wl.top_k, "h_i": wl.h_i, "d_i": wl.d_i,
                   "heads": wl.heads, "d_qk": wl.d_qk, "d_v": wl.d_v, "paged": wl.paged,
                   "needles": wl.needles, "drift_block": wl.drift_block, "seed": wl.seed,
                   "input_copies": copies},
        "roofline": dict(rooflines[dominant]),
        "stages": rooflines,
        "path_roofline": path,
    }
    return fig, dw


def default_counts(wl, steps, warmup, copies):
    decode = wl.kind != "prefill"
    return (steps if steps is not None else (200 if decode else 10),
            warmup if warmup is not None else (20 if decode else 3),
            copies if copies is not None else (4 if decode else 1))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the path has no multi-GPU form in this library "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.op == "cache_append":
        bench_cache_append(args)
        return
    if args.op == "output_projection":
        bench_output_projection(args)
        return
    if args.op == "module_forward":
        bench_module_forward(args)
        return
    from sparse_attention_long_fp8_amd import binding as B
    from sparse_attention_long_fp8_amd import synth

    dev = torch.device("cuda:0")
    B.lib()  # fail loudly now if the library is missing

    def log(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    wl = synth.WORKLOADS[args.workload]
    steps, warmup, copies = default_counts(wl, args.steps, args.warmup, args.copies)
    fig, dw = measure(wl, steps, warmup, copies, dev, log)
    synth_obj = dw.synth
    del dw
    torch.cuda.empty_cache()
    result = {
        "metric": METRIC,
        "value": fig["value"],
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": fig["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": fig["dtype"],
        "data": "synthetic",
        "config": fig["config"],
        "decode_us_per_step": fig["decode_us_per_step"],
        "roofline": fig["roofline"],
        "stages": fig["stages"],
        "path_roofline": fig["path_roofline"],
    }
    # The other workloads, each built, timed and freed in turn.  They run the
    # headline's step count (decode: at least 100 steps, since a step is
    # about 0.1 ms) and their own warm-up and input-copy defaults.
    others = [] if args.others == "none" else (
        [w for w in ALL_WORKLOADS if w != wl.name] if args.others == "all" else
        [w for w in args.others.split(",") if w and w != wl.name])
    table = {}
    for name in others:
        owl = synth.WORKLOADS[name]
        o_steps = steps if owl.kind == "prefill" else max(steps, 100)
        o_steps, o_warm, o_copies = default_counts(owl, o_steps, None, None)
        ofig, odw = measure(owl, o_steps, o_warm, o_copies, dev, log)
        del odw
        torch.cuda.empty_cache()
        table[name] = {
            "ms_per_step": ofig["ms_per_step"], "query_tokens_per_s": ofig["value"],
            "decode_us_per_step": ofig["decode_us_per_step"], "steps": o_steps, "warmup": o_warm,
            "dtype": ofig["dtype"], "config": ofig["config"],
            "stages": {k: {"us": v["us"], "frac": v["frac"], "bound": v["bound"], "kernel": v["kernel"],
                           "traffic": v["traffic"]} for k, v in ofig["stages"].items()},
            "path_roofline": ofig["path_roofline"],
        }
    result["workloads"] = table
    if not args.no_cpu_baseline:
        log("CPU oracle baseline on %s" % wl.name)
        result["cpu_baseline"] = cpu_baseline(wl, synth_obj, args.cpu_budget, args.cpu_sample)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
