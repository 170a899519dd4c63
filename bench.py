#!/usr/bin/env python3
"""Benchmark of the CSA decode path on one MI355X.

Workload (default): million-token decode, batch 4, 1,048,576 raw tokens per
sequence -> 262,144 compressed entries (ratio 4); indexer 64 heads x 128;
top-512; 128-token window; 64 query heads x 512 with one shared KV head; sink.
Inputs are seeded synthetic tensors, resident in HBM before timing.

One step = one pass of the CSA layer's hot path through the fused entry
point csa_attention: indexer scores -> top-k -> sparse MQA with sink, over
the whole batch.  Steps are captured in a HIP graph and replayed; the index-key and KV
caches rotate between enough device copies (at least twice the 256 MiB
last-level cache in all, for every workload) that no step finds the previous
steps' rows in that cache.  The paired HCA layer, the other
decode workloads and the per-kernel times are reported under "breakdown".

Prints one JSON line.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA decode queries/s at 64K–1M ctx; achieved HBM GB/s vs peak (1 GPU)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16 MFMA, MI355X datasheet
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_index_scores_decode_b4_1m.json")
SCORER_SRC = [os.path.join(ROOT, "compressed_sparse_attention_indexer_amd", "csrc", f)
              for f in ("scorer.hip", "scorer_common.hpp")]


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode_b4_1m")
    p.add_argument("--copies", type=int, default=2, help="device copies of the caches, rotated per step")
    p.add_argument("--graph-steps", type=int, default=10, help="steps captured per graph")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--quick", action="store_true", help="skip the other decode workloads")
    p.add_argument("--prefill", action="store_true", help="also time the 2048-token prefill chunk")
    p.add_argument("--profile-kernels", action="store_true",
                   help="run only eager scorer launches (for rocprofv3 counter runs)")
    return p.parse_args()


def sha_of(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ algorithmic bytes (per call)

def csa_step_bytes(n_ent, n_queries):
    """Per query: index keys 256 B/entry, q_idx 16 KiB, weights 256 B, q 64 KiB,
    512 selected + 128 window rows of 1 KiB, sink 256 B, fp32 output 128 KiB."""
    return int(sum(256 * int(n) for n in n_ent)) + 868864 * n_queries


def visible_counts(case):
    """Compressed entries each query sees (complete 4-token spans ending at or before its position)."""
    import numpy as np
    wl = case.wl
    b = np.arange(wl.batch * wl.q_len) // wl.q_len
    return np.minimum(case.seq_len[b] // wl.ratio, (case.q_pos.astype(np.int64) + 1) // wl.ratio)


def scorer_bytes(n_ent, n_queries):
    """Index keys (256 B per entry) plus index query and weights (16,640 B per query)."""
    return int(sum(256 * int(n) for n in n_ent)) + 16640 * n_queries


def hca_bytes(n_h, n_queries):
    return int(sum(1024 * (int(n) + 128) for n in n_h)) + 196864 * n_queries


# ------------------------------------------------------------------ timing helpers

class Timer:
    """Times a callable that enqueues work on torch's current stream: HIP
    events around `reps` back-to-back calls, average per call in ms."""

    def __init__(self, torch):
        self.torch = torch

    def per_call_ms(self, fn, reps):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / reps


def capture(torch, fn, n):
    """HIP graph of n calls of fn (each enqueues kernels on the capture stream)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)  # warm the code path outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


class CsaRunner:
    """Pre-allocated buffers and rotated cache copies for one CSA workload."""

    def __init__(self, torch, csa, dc, copies):
        self.t, self.csa, self.dc = torch, csa, dc
        self.dims = dc.csa_dims()
        d = self.dims
        dev = "cuda"
        self.scores = torch.empty((d.batch, d.q_len, d.max_entries), dtype=torch.float32, device=dev)
        self.idx = torch.empty((d.batch, d.q_len, d.topk), dtype=torch.int32, device=dev)
        self.out = torch.empty((d.batch, d.q_len, d.n_heads, d.head_dim), dtype=torch.float32, device=dev)
        self.lse = torch.empty((d.batch, d.q_len, d.n_heads), dtype=torch.float32, device=dev)
        self.ws_topk = self._ws(csa.workspace_size(d, csa._lib.CSA_OP_TOPK))
        self.ws_mqa = self._ws(csa.workspace_size(d, csa._lib.CSA_OP_SPARSE_MQA))
        self.ws_all = self._ws(csa.workspace_size(d, csa._lib.CSA_OP_ATTENTION))
        self.kidx_p, self.kv_p = [dc.k_idx_p], [dc.kv_p]
        self.keep = []
        for _ in range(copies - 1):
            k2 = [x.clone() for x in dc.k_idx]
            v2 = [x.clone() for x in dc.kv]
            self.keep += [k2, v2]
            self.kidx_p.append(csa.ptr_array(k2, dev))
            self.kv_p.append(csa.ptr_array(v2, dev))

    def _ws(self, n):
        return self.t.zeros(max(n, 256), dtype=self.t.uint8, device="cuda")

    def scores_call(self, i):
        dc = self.dc
        self.csa.csa_index_scores(self.dims, dc.q_idx, dc.w, self.kidx_p[i % len(self.kidx_p)], dc.seq_len,
                                  dc.q_pos, scores=self.scores)

    def topk_call(self, i):
        dc = self.dc
        self.csa.csa_topk_select(self.dims, self.scores, dc.seq_len, dc.q_pos, topk_idx=self.idx,
                                 workspace=self.ws_topk)

    def attn_call(self, i):
        dc = self.dc
        self.csa.csa_sparse_mqa_decode(self.dims, dc.q, self.kv_p[i % len(self.kv_p)], None, self.idx, dc.win_p,
                                       None, dc.win_pos0, dc.win_rows, dc.seq_len, dc.q_pos, dc.sink,
                                       out=self.out, lse=self.lse, workspace=self.ws_mqa)

    def step(self, i):
        self.scores_call(i)
        self.topk_call(i)
        self.attn_call(i)

    def fused(self, i):
        dc = self.dc
        self.csa.csa_attention(self.dims, dc.q, dc.q_idx, dc.w, self.kidx_p[i % len(self.kidx_p)],
                               self.kv_p[i % len(self.kv_p)], None, dc.win_p, None, dc.win_pos0, dc.win_rows,
                               dc.seq_len, dc.q_pos, dc.sink, out=self.out, lse=self.lse, workspace=self.ws_all)


LLC_BYTES = 256 << 20  # MI355X last-level (Infinity) cache


def rotation(bytes_per_copy, minimum):
    """Cache copies to rotate so the whole set is at least twice the last-level
    cache: a cyclic pass over more than the cache then finds nothing of the
    previous pass in it."""
    need = -(-2 * LLC_BYTES // max(1, int(bytes_per_copy)))
    return max(minimum, min(need, 256))


def time_graph(torch, g, graph_steps, steps, warmup):
    for _ in range(max(1, warmup // graph_steps)):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // graph_steps)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return a.elapsed_time(b) / (reps * graph_steps), wall, reps * graph_steps


def bench_csa(torch, csa, case, args, detail):
    from compressed_sparse_attention_indexer_amd.staging import DeviceCase
    dc = DeviceCase(case)
    copies = rotation(sum(x.numel() * x.element_size() for x in dc.k_idx), args.copies)
    r = CsaRunner(torch, csa, dc, copies)
    Q = r.dims.batch * r.dims.q_len
    n_ent = case.n_entries
    gs = max(args.graph_steps, copies)  # every copy is used within one replay
    g_step = capture(torch, r.fused, gs)
    ms, wall, n = time_graph(torch, g_step, gs, args.steps, args.warmup)
    # graph replay result == eager result (deterministic kernels)
    out_graph = r.out.clone()
    r.fused((n - 1) % copies)
    torch.cuda.synchronize()
    same = bool(torch.equal(out_graph, r.out))
    res = {"ms_per_step": ms, "queries_per_s": Q / (ms * 1e-3), "steps": n, "wall_s": wall, "cache_copies": copies,
           "graph_matches_eager": same,
           "alg_bytes_per_step": csa_step_bytes(n_ent, Q),
           "step_GBps": csa_step_bytes(n_ent, Q) / (ms * 1e-3) / 1e9}
    res["step_frac_hbm_peak"] = res["step_GBps"] / HBM_PEAK_GBS
    if detail:
        per = {}
        for name, fn in (("index_scores", r.scores_call), ("topk_select", r.topk_call),
                         ("sparse_mqa", r.attn_call)):
            g = capture(torch, fn, gs)
            per[name], _, _ = time_graph(torch, g, gs, args.steps, args.warmup)
        g_s = capture(torch, r.step, gs)
        res["separate_entry_points_ms"], _, _ = time_graph(torch, g_s, gs, args.steps, args.warmup)
        res["kernel_ms"] = per
        res["scorer_alg_bytes"] = scorer_bytes(n_ent, Q)
        # indexer flops: 2 * 64 heads * 128 dims per (query, visible entry)
        nvis = visible_counts(case)
        res["scorer_flops"] = 2 * r.dims.index_heads * r.dims.index_dim * int(nvis.sum())
        res["scorer_TFLOPs"] = res["scorer_flops"] / (per["index_scores"] * 1e-3) / 1e12
        res["scorer_frac_mfma_peak"] = res["scorer_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS
    return res, r


def bench_hca(torch, csa, case, args):
    from compressed_sparse_attention_indexer_amd.staging import DeviceCase
    dc = DeviceCase(case)
    d = dc.hca_dims()
    Q = d.batch * d.q_len
    out = torch.empty((d.batch, d.q_len, d.n_heads, d.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((d.batch, d.q_len, d.n_heads), dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(256, csa.workspace_size(d, csa._lib.CSA_OP_HCA_MQA)), dtype=torch.uint8, device="cuda")
    copies = [dc.hca_kv_p]
    keep = []
    n_copies = rotation(sum(x.numel() * x.element_size() for x in dc.hca_kv), args.copies)
    for _ in range(n_copies - 1):
        k2 = [x.clone() for x in dc.hca_kv]
        keep.append(k2)
        copies.append(csa.ptr_array(k2, "cuda"))
    gs = max(args.graph_steps, n_copies)

    def call(i):
        csa.hca_mqa_decode(d, dc.hca_q, copies[i % len(copies)], None, dc.hca_win_p, None, dc.win_pos0,
                           dc.win_rows, dc.seq_len, dc.q_pos, dc.hca_sink, out=out, lse=lse, workspace=ws)

    g = capture(torch, call, gs)
    ms, _, n = time_graph(torch, g, gs, args.steps, args.warmup)
    n_h = case.seq_len // case.wl.hca_ratio
    b = hca_bytes(n_h, Q)
    return {"ms_per_call": ms, "queries_per_s": Q / (ms * 1e-3), "alg_bytes": b, "cache_copies": n_copies,
            "GBps": b / (ms * 1e-3) / 1e9, "frac_hbm_peak": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def fp8_scorer_bytes(n_ent, n_queries):
    """fp8 index keys: 128 B codes + 4 B scale per entry; per query 8 KiB of codes, 256 B of
    query scales and 256 B of weights."""
    return int(sum(132 * int(n) for n in n_ent)) + 8704 * n_queries


def bench_fp8_scores(torch, csa, case, args):
    """The indexer scorer on fp8 (E4M3) index tensors with per-row scales, same shapes."""
    from compressed_sparse_attention_indexer_amd import inputs
    wl = case.wl
    q8, qs, k8, ks = inputs.make_fp8_index(case)
    dev = "cuda"
    q8_t, qs_t = torch.from_numpy(q8).to(dev), torch.from_numpy(qs).to(dev)
    w_t = torch.from_numpy(case.w).to(dev)
    copies = []
    n_copies = rotation(sum(k.nbytes for k in k8) + sum(x.nbytes for x in ks), args.copies)
    k_0 = [torch.from_numpy(k).to(dev) for k in k8]
    s_0 = [torch.from_numpy(x).to(dev) for x in ks]
    for c in range(n_copies):
        k_t = k_0 if c == 0 else [x.clone() for x in k_0]
        s_t = s_0 if c == 0 else [x.clone() for x in s_0]
        copies.append((k_t, s_t, csa.ptr_array(k_t, dev), csa.ptr_array(s_t, dev)))
    gs = max(args.graph_steps, n_copies)
    seq_t, pos_t = torch.from_numpy(case.seq_len).to(dev), torch.from_numpy(case.q_pos).to(dev)
    dims = csa.make_dims(batch=wl.batch, q_len=wl.q_len, max_entries=case.max_entries)
    scores = torch.empty((wl.batch, wl.q_len, case.max_entries), dtype=torch.float32, device=dev)

    def call(i):
        c = copies[i % len(copies)]
        csa.csa_index_scores_fp8(dims, q8_t, qs_t, w_t, c[2], c[3], seq_t, pos_t, scores=scores)

    g = capture(torch, call, gs)
    ms, _, _ = time_graph(torch, g, gs, args.steps, args.warmup)
    Q = wl.batch * wl.q_len
    b = fp8_scorer_bytes(case.n_entries, Q)
    return {"ms_per_call": ms, "alg_bytes": b, "GBps": b / (ms * 1e-3) / 1e9, "cache_copies": n_copies,
            "frac_hbm_peak": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "vs_bf16_scorer": None}


COMPRESS_CASES = (
    # name, tokens, out_dim, ratio, window, first entry, entries, hadamard: one new entry at a decode
    # step (its window), and the entries of a 2,048-token prefill chunk (plus the 4 tokens of
    # overlap), for the 512-d KV cache, the 128-d index keys (Hadamard) and the 128:1 HCA cache
    ("kv_decode_entry", 8, 512, 4, 8, 262143, 1, False),
    ("index_key_decode_entry", 8, 128, 4, 8, 262143, 1, True),
    ("hca_decode_entry", 128, 512, 128, 128, 8191, 1, False),
    ("kv_prefill_chunk_2048", 2052, 512, 4, 8, 261632, 512, False),
    ("index_key_prefill_chunk_2048", 2052, 128, 4, 8, 261632, 512, True),
    ("hca_prefill_chunk_2048", 2048, 512, 128, 128, 8176, 16, False),
)
COMPRESS_HIDDEN = 4096


def bench_compress(torch, csa, args):
    """csa_compress on decode and prefill-chunk shapes (hidden 4096, RoPE on 64 dims).  Bytes: the
    two weight matrices, the x rows and the bf16 output; flops: the two projections."""
    import numpy as np
    from compressed_sparse_attention_indexer_amd import inputs
    dev, res = "cuda", {}
    for name, T, D, r, w, fe, ne, had in COMPRESS_CASES:
        x, wkv, wg, ape, gamma = inputs.make_compressor_inputs(11, T, COMPRESS_HIDDEN, D, w)
        bf = lambda a: torch.from_numpy(a.view(np.int16)).to(dev)
        X, WK, WG = bf(x), bf(wkv), bf(wg)
        AP, GM = torch.from_numpy(ape).to(dev), torch.from_numpy(gamma).to(dev)
        pos0 = r * fe + r - w
        dims = csa.make_compress_dims(tokens=T, hidden=COMPRESS_HIDDEN, out_dim=D, ratio=r, window=w,
                                      first_entry=fe, n_entries=ne, pos0=pos0, rope_dims=64, hadamard=had)
        out = torch.empty((ne, D), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(256, csa.compress_workspace_size(dims)), dtype=torch.uint8, device=dev)
        g = capture(torch, lambda i: csa.csa_compress(dims, X, WK, WG, AP, GM, out=out, workspace=ws),
                    args.graph_steps)
        ms, _, _ = time_graph(torch, g, args.graph_steps, max(args.steps, 20), args.warmup)
        byt = 2 * D * COMPRESS_HIDDEN * 2 + T * COMPRESS_HIDDEN * 2 + ne * D * 2
        fl = 2.0 * T * COMPRESS_HIDDEN * 2 * D
        gbs, tfs = byt / (ms * 1e-3) / 1e9, fl / (ms * 1e-3) / 1e12
        res[name] = {"us_per_call": ms * 1e3, "entries": ne, "tokens": T, "alg_bytes": byt, "GBps": gbs,
                     "frac_hbm_peak": gbs / HBM_PEAK_GBS, "flops": fl, "TFLOPs": tfs,
                     "frac_mfma_peak": tfs / MFMA_BF16_PEAK_TFLOPS}
        del X, WK, WG, AP, GM, out, ws, g
    return res


def traffic_from_profile():
    """HBM bytes per scorer launch from the committed rocprofv3 counter runs,
    only while the scorer source is the one the counters were taken on."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None, "no counter profile committed"
    rec = json.load(open(PROFILE_TRAFFIC))
    if rec.get("scorer_sha") != sha_of(SCORER_SRC):
        return None, "scorer changed since the counters were taken"
    return int(rec["hbm_bytes_per_launch"]), rec.get("note", "")


def cpu_baseline(case):
    import oracle
    wl = case.wl
    # repeat the whole step until about 10 s of CPU work is done
    runs, t_total = 0, 0.0
    while runs < 3 or t_total < 10.0:
        t0 = time.perf_counter()
        oracle.csa_attention(case)
        t_total += time.perf_counter() - t0
        runs += 1
    Q = wl.batch * wl.q_len
    return {"value": Q * runs / t_total, "unit": "queries/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"whole CSA step of {wl.name} ({Q} queries x {case.max_entries} entries: scores, "
                      f"top-k, attention), repeated {runs} times, {t_total:.1f} s in all"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this path has no multi-GPU "
              f"mode: run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import compressed_sparse_attention_indexer_amd as csa
    from compressed_sparse_attention_indexer_amd import inputs

    torch.cuda.set_device(0)
    csa.load_library()
    wl = inputs.WORKLOADS[args.workload]
    t0 = time.perf_counter()
    case = inputs.make_case(wl)
    print(f"[bench] generated {wl.name} in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    if args.profile_kernels:  # eager scorer launches only, for counter collection
        from compressed_sparse_attention_indexer_amd.staging import DeviceCase
        r = CsaRunner(torch, csa, DeviceCase(case), args.copies)
        for i in range(args.steps):
            r.scores_call(i)
        torch.cuda.synchronize()
        # calibration for the byte counters: a plain device copy of 256 MiB
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile_kernels": args.steps, "copy_bytes": src.numel() * 4}))
        return

    main_res, runner = bench_csa(torch, csa, case, args, detail=True)
    print(f"[bench] {wl.name}: {main_res['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    breakdown = {wl.name: main_res}
    if case.hca_q is not None:
        breakdown[wl.name + "_hca"] = bench_hca(torch, csa, case, args)
    if wl.dtype == "bf16":
        f8 = bench_fp8_scores(torch, csa, case, args)
        f8["vs_bf16_scorer"] = main_res["kernel_ms"]["index_scores"] / f8["ms_per_call"]
        breakdown[wl.name + "_fp8_index_scores"] = f8
    breakdown["compressor"] = bench_compress(torch, csa, args)
    Q = wl.batch * wl.q_len
    scorer_ms = main_res["kernel_ms"]["index_scores"]
    alg = main_res["scorer_alg_bytes"]
    traffic, traffic_note = traffic_from_profile()
    roofline = {"kernel": "index_scores_bf16_kernel", "bound": "hbm",
                "achieved": alg / (scorer_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": alg / (scorer_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
                "alg_bytes_per_launch": alg, "avg_launch_ms": scorer_ms, "traffic_note": traffic_note}
    del runner
    torch.cuda.empty_cache()

    if not args.quick:
        for name in ("decode_b1_64k", "decode_b32_ragged_64k_128k", "pro_decode_b4_1m"):
            if name == wl.name:
                continue
            c2 = inputs.make_case(inputs.WORKLOADS[name])
            r2, rr = bench_csa(torch, csa, c2, args, detail=True)
            breakdown[name] = r2
            del rr, c2
            torch.cuda.empty_cache()
    if args.prefill:
        c4 = inputs.make_case(inputs.WORKLOADS["prefill_t2048_1m"])
        a2 = argparse.Namespace(**vars(args))
        a2.steps, a2.warmup, a2.graph_steps, a2.copies = 3, 1, 1, 1  # the rotation still covers 2x the LLC
        r4, rr = bench_csa(torch, csa, c4, a2, detail=True)
        breakdown["prefill_t2048_1m"] = r4
        del rr, c4

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case)

    line = {
        "metric": METRIC, "value": main_res["queries_per_s"], "unit": "queries/s", "n_gpus": 1,
        "steps": main_res["steps"], "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; N(0,1)/sqrt(d) activations and caches, U(0,1) weights, N(0,1) sink)",
        "config": {"workload": wl.name, "batch": wl.batch, "q_len": wl.q_len, "context": wl.seq_len,
                   "compressed_entries": int(case.max_entries), "ratio": wl.ratio, "topk": wl.topk,
                   "window": wl.window, "heads": wl.n_heads, "head_dim": wl.head_dim,
                   "index_heads": wl.index_heads, "index_dim": wl.index_dim,
                   "step": "csa_attention (index_scores -> topk_select -> sparse_mqa + sink), graph-replayed",
                   "cache_copies_rotated": main_res["cache_copies"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "breakdown": breakdown,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
