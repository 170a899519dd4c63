#!/usr/bin/env python3
"""Benchmark of the CSA decode path on one MI355X.

Workload (default): million-token decode, batch 4, 1,048,576 raw tokens per
sequence -> 262,144 compressed entries (ratio 4); indexer 64 heads x 128;
top-512; 128-token window; 64 query heads x 512 with one shared KV head; sink.
Inputs are seeded synthetic tensors, resident in HBM before timing.

One step = one pass of the CSA layer's hot path through the fused entry
point csa_attention: indexer scores -> top-k -> sparse MQA with sink, over
the whole batch.  Steps are captured in HIP graphs and replayed (two steps
per replay, a HIP event after every replay: the line gives the mean over the
timed steps and the p10/median/p90 of the per-replay figures); the index-key
and KV caches rotate between enough device copies (at least twice the 256 MiB
last-level cache in all, for every workload) that no step finds the previous
steps' rows in that cache.  The roofline block is for the indexer scorer (the
dominant kernel; each entry point is also timed alone, 20 launches per graph)
and for the whole step, against the 8 TB/s datasheet figure and against a
plain streaming-read kernel measured in the same run over the same byte count.
The breakdown holds the paired HCA layer, the fp8-index scorer and step, the
compressor, the other decode workloads, the 2,048-query prefill chunk, the
oracle's rates on the host, and amd-smi clock samples (before, under load and
after).

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
PROFILE_STEP = os.path.join(ROOT, "profiles", "trace_decode_b4_1m.json")
_CSRC = os.path.join(ROOT, "compressed_sparse_attention_indexer_amd", "csrc")
SCORER_SRC = [os.path.join(_CSRC, f) for f in ("scorer.hip", "scorer_common.hpp")]
STEP_SRC = [os.path.join(_CSRC, f) for f in ("scorer.hip", "scorer_common.hpp", "topk.hip", "topk_hist.hpp",
                                              "attention.hip", "common.hpp", "launch.hpp", "api.cpp")]


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode_b4_1m")
    p.add_argument("--copies", type=int, default=2, help="device copies of the caches, rotated per step")
    p.add_argument("--graph-steps", type=int, default=2,
                   help="steps captured per graph (at least the cache copies); each replay is one timing sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--quick", action="store_true", help="skip the other decode workloads")
    p.add_argument("--no-prefill", action="store_true", help="skip the 2048-token prefill chunk")
    p.add_argument("--prefill", action="store_true", help=argparse.SUPPRESS)  # timed by default
    p.add_argument("--profile-kernels", nargs="?", const="scorer", default=None,
                   choices=("scorer", "step", "hca", "fp8", "prefill"),
                   help="run only eager launches of one part (for rocprofv3 counter runs): the bf16 scorer, "
                        "the fused decode step, the HCA layer, the fp8 scorer or the prefill chunk")
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
    """W untimed warmup steps, then about `steps` steps as replays of g (graph_steps
    steps each) between two synchronizations.  Returns the mean over the timed
    steps (first to last HIP event), the distribution of per-replay step times
    (a HIP event after every replay), the wall time and the number of steps."""
    for _ in range(max(1, warmup // graph_steps)):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // graph_steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(reps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(ev[i].elapsed_time(ev[i + 1]) / graph_steps for i in range(reps))
    pick = lambda f: per[min(len(per) - 1, int(round(f * (len(per) - 1))))]
    n = reps * graph_steps
    return {"ms": ev[0].elapsed_time(ev[-1]) / n, "median_ms": pick(0.5), "p10_ms": pick(0.1), "p90_ms": pick(0.9),
            "samples": reps, "wall_s": wall, "steps": n}


def bench_csa(torch, csa, case, args, detail, min_samples=None):
    from compressed_sparse_attention_indexer_amd.staging import DeviceCase
    dc = DeviceCase(case)
    copies = rotation(sum(x.numel() * x.element_size() for x in dc.k_idx), args.copies)
    r = CsaRunner(torch, csa, dc, copies)
    Q = r.dims.batch * r.dims.q_len
    n_ent = case.n_entries
    gs = max(args.graph_steps, copies)  # every copy is used within one replay
    g_step = capture(torch, r.fused, gs)
    r.graph = g_step
    # the headline workload times exactly args.steps steps; the others at least
    # 50 replays, so that the distribution has 50 samples
    steps = args.steps if min_samples is None else max(args.steps, min_samples * gs)
    tg = time_graph(torch, g_step, gs, steps, args.warmup)
    ms, wall, n = tg["ms"], tg["wall_s"], tg["steps"]
    # graph replay result == eager result (deterministic kernels)
    out_graph = r.out.clone()
    r.fused((n - 1) % copies)
    torch.cuda.synchronize()
    same = bool(torch.equal(out_graph, r.out))
    res = {"ms_per_step": ms, "queries_per_s": Q / (ms * 1e-3), "steps": n, "wall_s": wall, "cache_copies": copies,
           "median_ms": tg["median_ms"], "p10_ms": tg["p10_ms"], "p90_ms": tg["p90_ms"], "samples": tg["samples"],
           "graph_matches_eager": same,
           "alg_bytes_per_step": csa_step_bytes(n_ent, Q),
           "step_GBps": csa_step_bytes(n_ent, Q) / (ms * 1e-3) / 1e9}
    res["step_frac_hbm_peak"] = res["step_GBps"] / HBM_PEAK_GBS
    if detail:
        # Each entry point alone, 20 launches per graph (copies rotated), so that
        # the per-launch figure is the kernel time plus the gap between dependent
        # kernels, and the replay's own launch cost is spread thin; three replays
        # of warm-up (the first replays of a new graph read high), ten timed.
        per = {}
        gk = max(gs, 20)
        for name, fn in (("index_scores", r.scores_call), ("topk_select", r.topk_call),
                         ("sparse_mqa", r.attn_call)):
            g = capture(torch, fn, gk)
            per[name] = time_graph(torch, g, gk, max(args.steps, 10 * gk), max(args.warmup, 3 * gk))["ms"]
        g_s = capture(torch, r.step, gs)
        res["separate_entry_points_ms"] = time_graph(torch, g_s, gs, args.steps, args.warmup)["ms"]
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
    tg = time_graph(torch, g, gs, max(args.steps, 50 * gs), args.warmup)
    ms = tg["ms"]
    n_h = case.seq_len // case.wl.hca_ratio
    b = hca_bytes(n_h, Q)
    return {"ms_per_call": ms, "median_ms": tg["median_ms"], "p10_ms": tg["p10_ms"], "p90_ms": tg["p90_ms"],
            "samples": tg["samples"], "queries_per_s": Q / (ms * 1e-3), "alg_bytes": b, "cache_copies": n_copies,
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
    gs = max(args.graph_steps, n_copies, 20)  # 20 launches per graph, as for the other per-kernel figures
    seq_t, pos_t = torch.from_numpy(case.seq_len).to(dev), torch.from_numpy(case.q_pos).to(dev)
    dims = csa.make_dims(batch=wl.batch, q_len=wl.q_len, max_entries=case.max_entries)
    scores = torch.empty((wl.batch, wl.q_len, case.max_entries), dtype=torch.float32, device=dev)

    def call(i):
        c = copies[i % len(copies)]
        csa.csa_index_scores_fp8(dims, q8_t, qs_t, w_t, c[2], c[3], seq_t, pos_t, scores=scores)

    g = capture(torch, call, gs)
    ms = time_graph(torch, g, gs, max(args.steps, 5 * gs), args.warmup)["ms"]
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


def fp8_step_bytes(n_ent, n_queries):
    """The decode step with fp8 index tensors: the fp8 scorer's bytes plus, per query, q 64 KiB,
    512 selected + 128 window rows of 1 KiB, sink 256 B and the fp32 output 128 KiB."""
    return fp8_scorer_bytes(n_ent, n_queries) + (868864 - 16640) * n_queries


def bench_fp8_step(torch, csa, case, args):
    """The whole decode step with fp8 (E4M3) index tensors: csa_attention_fp8
    (fp8 scorer with the selection's histograms and emitted entries, selection,
    bf16 attention, combine), graph-replayed like the bf16 step, with the fp8
    key caches, their scales and the KV cache rotated over copies."""
    from compressed_sparse_attention_indexer_amd import inputs
    from compressed_sparse_attention_indexer_amd.staging import DeviceCase
    dev = "cuda"
    dc = DeviceCase(case)
    dims = dc.csa_dims()
    q8, qs, k8, ks = inputs.make_fp8_index(case)
    q8_t, qs_t = torch.from_numpy(q8).to(dev), torch.from_numpy(qs).to(dev)
    k_0 = [torch.from_numpy(k).to(dev) for k in k8]
    s_0 = [torch.from_numpy(x).to(dev) for x in ks]
    n_copies = rotation(sum(k.nbytes for k in k8) + sum(x.nbytes for x in ks), args.copies)
    copies = []
    for c in range(n_copies):
        k_t = k_0 if c == 0 else [x.clone() for x in k_0]
        s_t = s_0 if c == 0 else [x.clone() for x in s_0]
        v_t = dc.kv if c == 0 else [x.clone() for x in dc.kv]
        copies.append((k_t, s_t, v_t, csa.ptr_array(k_t, dev), csa.ptr_array(s_t, dev),
                       dc.kv_p if c == 0 else csa.ptr_array(v_t, dev)))
    out = torch.empty((dims.batch, dims.q_len, dims.n_heads, dims.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((dims.batch, dims.q_len, dims.n_heads), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(256, csa.workspace_size(dims, csa._lib.CSA_OP_ATTENTION_FP8)), dtype=torch.uint8,
                     device=dev)

    def call(i):
        c = copies[i % len(copies)]
        csa.csa_attention_fp8(dims, dc.q, q8_t, qs_t, dc.w, c[3], c[4], c[5], None, dc.win_p, None, dc.win_pos0,
                              dc.win_rows, dc.seq_len, dc.q_pos, dc.sink, out=out, lse=lse, workspace=ws)

    gs = max(args.graph_steps, n_copies)
    g = capture(torch, call, gs)
    tg = time_graph(torch, g, gs, max(args.steps, 50 * gs), args.warmup)
    ms = tg["ms"]
    out_graph = out.clone()
    call((tg["steps"] - 1) % n_copies)
    torch.cuda.synchronize()
    Q = dims.batch * dims.q_len
    b = fp8_step_bytes(case.n_entries, Q)
    return {"ms_per_step": ms, "queries_per_s": Q / (ms * 1e-3), "median_ms": tg["median_ms"], "p10_ms": tg["p10_ms"],
            "p90_ms": tg["p90_ms"], "samples": tg["samples"], "steps": tg["steps"], "cache_copies": n_copies,
            "graph_matches_eager": bool(torch.equal(out_graph, out)), "alg_bytes_per_step": b,
            "step_GBps": b / (ms * 1e-3) / 1e9, "step_frac_hbm_peak": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


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
        ms = time_graph(torch, g, args.graph_steps, max(args.steps, 20), args.warmup)["ms"]
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


def _oracle_step_rate(case, min_s, min_runs, max_runs):
    """Queries/s of the oracle's whole step on a case: repeated until min_s of CPU
    work and min_runs runs (at most max_runs), best run."""
    import oracle
    runs, t_total, best = 0, 0.0, float("inf")
    while runs < max_runs and (runs < min_runs or t_total < min_s):
        t0 = time.perf_counter()
        oracle.csa_attention(case)
        dt = time.perf_counter() - t0
        t_total += dt
        best = min(best, dt)
        runs += 1
    Q = case.wl.batch * case.wl.q_len
    return Q / best, runs, t_total


def cpu_baseline(case):
    """The headline workload's whole step on the oracle (host cores)."""
    import oracle
    wl = case.wl
    rate, runs, t_total = _oracle_step_rate(case, 10.0, 3, 50)
    Q = wl.batch * wl.q_len
    return {"value": rate, "unit": "queries/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu": _cpu_model(),
            "sample": f"whole CSA step of {wl.name} ({Q} queries x {case.max_entries} entries: scores, "
                      f"top-k, attention), best of {runs} runs ({t_total:.1f} s in all)"}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baselines_other(inputs):
    """The oracle on the other workloads: the 64K single query (best of 3), the
    ragged 32-sequence batch (one run) and a sample of the prefill chunk (4
    evenly spaced queries, extrapolated to its 2,048 queries and labelled so)."""
    import numpy as np
    import oracle
    res = {}
    c1 = inputs.make_case(inputs.WORKLOADS["decode_b1_64k"])
    rate, runs, t = _oracle_step_rate(c1, 0.0, 3, 3)
    res["decode_b1_64k"] = {"value": rate, "unit": "queries/s", "sample": f"whole step, best of {runs} ({t:.1f} s)"}
    del c1
    c2 = inputs.make_case(inputs.WORKLOADS["decode_b32_ragged_64k_128k"])
    rate, runs, t = _oracle_step_rate(c2, 0.0, 1, 1)
    res["decode_b32_ragged_64k_128k"] = {"value": rate, "unit": "queries/s",
                                         "sample": f"whole step of 32 queries, one run ({t:.1f} s)"}
    del c2
    import dataclasses
    c4 = inputs.make_case(inputs.WORKLOADS["prefill_t2048_1m"], with_hca=False)
    ts = np.linspace(0, c4.wl.q_len - 1, 4).astype(int)
    sub = dataclasses.replace(c4, wl=dataclasses.replace(c4.wl, q_len=len(ts)), q_pos=c4.q_pos[ts].copy(),
                              q=c4.q[:, ts].copy(), q_idx=c4.q_idx[:, ts].copy(), w=c4.w[:, ts].copy())
    t0 = time.perf_counter()
    oracle.csa_attention(sub)
    t = time.perf_counter() - t0
    res["prefill_t2048_1m"] = {"value": len(ts) / t, "unit": "queries/s", "extrapolated": True,
                               "sample": f"queries {ts.tolist()} of the 2,048 ({t:.1f} s); a whole chunk would take "
                                         f"about {t * c4.wl.q_len / len(ts):.0f} s (extrapolated x{c4.wl.q_len // len(ts)})"}
    res["cores"] = oracle.num_threads()
    return res


def stream_read_peak(torch, sizes=()):
    """HBM read rate of a plain streaming-read kernel (libcsa_bench.so): over a
    4 GiB buffer, and over buffers of each given size (rotated over enough
    copies to exceed twice the last-level cache, as the path's own caches are),
    at several grid sizes, launches captured in HIP graphs.  Returns the best
    rate per size and the rates by grid size."""
    import ctypes
    from compressed_sparse_attention_indexer_amd import build as pkg_build
    if not os.path.exists(pkg_build.BENCH_LIB):
        return None
    lib = ctypes.CDLL(pkg_build.BENCH_LIB)
    lib.csa_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.csa_bench_stream_read.restype = ctypes.c_int
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")
    res = {}
    for nbytes in (4 << 30, *sizes):
        nbytes = int(nbytes) // 16 * 16
        n_buf = rotation(nbytes, 1)
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n_buf)]
        by_grid = {}
        for blocks in (256, 512, 1024, 4096, 8192):
            reps = max(2, -(-8 // n_buf)) * n_buf  # whole passes over the copies

            def call(i):
                rc = lib.csa_bench_stream_read(bufs[i % n_buf].data_ptr(), nbytes, sink.data_ptr(), blocks,
                                               torch.cuda.current_stream().cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"stream read launch failed ({rc})")
            g = capture(torch, call, reps)
            t = time_graph(torch, g, reps, 3 * reps, reps)
            by_grid[str(blocks)] = nbytes / (t["ms"] * 1e-3) / 1e9
        del bufs
        torch.cuda.empty_cache()
        res[str(nbytes)] = {"best_GBps": max(by_grid.values()), "copies": n_buf, "GBps_by_workgroups": by_grid}
    return {"best_GBps": res[str(4 << 30)]["best_GBps"], "by_bytes": res}


_CLOCK_CMDS = (["amd-smi", "metric", "--clock", "--json"], ["amd-smi", "metric", "-c", "--json"])


def _clock_summary(text):
    """GPU (per XCD) and memory clocks from amd-smi's JSON."""
    data = json.loads(text)
    gpus = data.get("gpu_data", data) if isinstance(data, dict) else data
    clk = gpus[0]["clock"]
    val = lambda e: e["clk"]["value"] if isinstance(e.get("clk"), dict) else None
    gfx = [val(v) for k, v in sorted(clk.items()) if k.startswith("gfx_")]
    one = next(v for k, v in clk.items() if k.startswith("gfx_"))
    return {"gfx_MHz": gfx, "gfx_max_MHz": one["max_clk"]["value"] if isinstance(one.get("max_clk"), dict) else None,
            "gfx_locked": one.get("clk_locked"), "mem_MHz": val(clk["mem_0"]) if "mem_0" in clk else None}


def gpu_clocks(busy=None):
    """One amd-smi sample of the GPU clocks.  With `busy` (a callable that
    enqueues GPU work and waits for it), the sample is taken while that work
    runs back to back, so it shows the clocks under load."""
    import subprocess
    t0 = time.perf_counter()
    while busy is not None and time.perf_counter() - t0 < 2.0:  # the clocks settle under the load first
        busy()
    for cmd in _CLOCK_CMDS:
        try:
            proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
        except OSError:
            continue
        t0 = time.perf_counter()
        while busy is not None and proc.poll() is None and time.perf_counter() - t0 < 20:
            busy()
        try:
            out, _ = proc.communicate(timeout=30)
        except subprocess.TimeoutExpired:
            proc.kill()
            proc.communicate()
            continue
        if proc.returncode == 0 and out.strip():
            try:
                return {"cmd": " ".join(cmd), "under_load": busy is not None, **_clock_summary(out)}
            except (ValueError, KeyError, IndexError, StopIteration, TypeError):
                return {"cmd": " ".join(cmd), "under_load": busy is not None, "raw": out.strip()[:400]}
    return None


def step_profile():
    """Kernel averages of the committed kernel-trace summary of the fused decode
    step, if its sources are the ones the trace was taken on."""
    if not os.path.exists(PROFILE_STEP):
        return None
    rec = json.load(open(PROFILE_STEP))
    if rec.get("src_sha") != sha_of(STEP_SRC):
        return {"note": "the path's sources changed since the trace was taken", "command": rec.get("command")}
    return rec


def profile_kernels(torch, csa, inputs, case, args):
    """Eager launches of one part of the path, then a plain 256 MiB device copy
    (the calibration for the byte counters), for rocprofv3 counter runs."""
    from compressed_sparse_attention_indexer_amd.staging import DeviceCase
    what = args.profile_kernels
    if what == "prefill":
        case = inputs.make_case(inputs.WORKLOADS["prefill_t2048_1m"], with_hca=False)
    dc = DeviceCase(case)
    if what in ("scorer", "step", "prefill"):
        r = CsaRunner(torch, csa, dc, args.copies if what != "prefill" else 1)
        fn = r.scores_call if what == "scorer" else r.fused
    elif what == "hca":
        d = dc.hca_dims()
        out = torch.empty((d.batch, d.q_len, d.n_heads, d.head_dim), dtype=torch.float32, device="cuda")
        lse = torch.empty((d.batch, d.q_len, d.n_heads), dtype=torch.float32, device="cuda")
        ws = torch.zeros(max(256, csa.workspace_size(d, csa._lib.CSA_OP_HCA_MQA)), dtype=torch.uint8, device="cuda")

        def fn(i):
            csa.hca_mqa_decode(d, dc.hca_q, dc.hca_kv_p, None, dc.hca_win_p, None, dc.win_pos0, dc.win_rows,
                               dc.seq_len, dc.q_pos, dc.hca_sink, out=out, lse=lse, workspace=ws)
    else:  # fp8 scorer
        wl = case.wl
        q8, qs, k8, ks = inputs.make_fp8_index(case)
        t = lambda a: torch.from_numpy(a).to("cuda")
        q8_t, qs_t, w_t = t(q8), t(qs), t(case.w)
        k_t, s_t = [t(k) for k in k8], [t(x) for x in ks]
        kp, sp = csa.ptr_array(k_t, "cuda"), csa.ptr_array(s_t, "cuda")
        dims = csa.make_dims(batch=wl.batch, q_len=wl.q_len, max_entries=case.max_entries)
        scores = torch.empty((wl.batch, wl.q_len, case.max_entries), dtype=torch.float32, device="cuda")

        def fn(i):
            csa.csa_index_scores_fp8(dims, q8_t, qs_t, w_t, kp, sp, dc.seq_len, dc.q_pos, scores=scores)
    for i in range(args.steps):
        fn(i)
    torch.cuda.synchronize()
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile_kernels": what, "launches": args.steps, "copy_bytes": src.numel() * 4}))


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

    if args.profile_kernels:  # eager launches of one part only, for counter collection
        profile_kernels(torch, csa, inputs, case, args)
        return

    clocks = [gpu_clocks()]
    main_res, runner = bench_csa(torch, csa, case, args, detail=True)

    def busy():
        for _ in range(20):
            runner.graph.replay()
        torch.cuda.synchronize()
    clocks.append(gpu_clocks(busy))
    print(f"[bench] {wl.name}: {main_res['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    breakdown = {wl.name: main_res}
    if case.hca_q is not None:
        breakdown[wl.name + "_hca"] = bench_hca(torch, csa, case, args)
    if wl.dtype == "bf16":
        f8 = bench_fp8_scores(torch, csa, case, args)
        f8["vs_bf16_scorer"] = main_res["kernel_ms"]["index_scores"] / f8["ms_per_call"]
        breakdown[wl.name + "_fp8_index_scores"] = f8
        breakdown[wl.name + "_fp8_step"] = bench_fp8_step(torch, csa, case, args)
    breakdown["compressor"] = bench_compress(torch, csa, args)
    Q = wl.batch * wl.q_len
    scorer_ms = main_res["kernel_ms"]["index_scores"]
    alg = main_res["scorer_alg_bytes"]
    traffic, traffic_note = traffic_from_profile()
    del runner
    torch.cuda.empty_cache()
    peak = stream_read_peak(torch, sizes=(alg,))
    print(f"[bench] streaming read: {peak and peak.get('best_GBps')}", file=sys.stderr, flush=True)
    # the streaming rate a plain read kernel reaches over the scorer's own byte count
    same_size = peak["by_bytes"][str(int(alg) // 16 * 16)]["best_GBps"] if peak else None
    achieved = alg / (scorer_ms * 1e-3) / 1e9
    step_gbs = main_res["step_GBps"]
    roofline = {"kernel": "index_scores_bf16_kernel (the indexer scorer, launched alone)", "bound": "hbm",
                "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": traffic, "traffic_note": traffic_note,
                "alg_bytes_per_launch": alg, "avg_launch_ms": scorer_ms,
                "measured_stream_read_GBps": peak and peak.get("best_GBps"),
                "measured_stream_read_same_bytes_GBps": same_size,
                "frac_of_measured_stream_read": (achieved / same_size) if same_size else None,
                "step": {"what": "the whole fused decode step (csa_attention: scorer with the selection's "
                                 "histograms and emitted entries, selection, attention, combine)",
                         "alg_bytes": main_res["alg_bytes_per_step"], "ms": main_res["ms_per_step"],
                         "GBps": step_gbs, "frac": step_gbs / HBM_PEAK_GBS,
                         "frac_of_measured_stream_read": (step_gbs / same_size) if same_size else None}}
    prof = step_profile()
    if prof and "kernels" in prof:
        k = prof["kernels"].get(prof.get("scorer_in_step", ""))
        if k:
            roofline["in_step_scorer"] = {"kernel": prof["scorer_in_step"], "avg_us_in_trace": k["avg_us"],
                                          "frac": alg / (k["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                          "source": os.path.relpath(PROFILE_STEP, ROOT)}
    elif prof:
        roofline["in_step_scorer"] = prof

    if not args.quick:
        for name in ("decode_b1_64k", "decode_b32_ragged_64k_128k", "pro_decode_b4_1m"):
            if name == wl.name:
                continue
            c2 = inputs.make_case(inputs.WORKLOADS[name])
            r2, rr = bench_csa(torch, csa, c2, args, detail=True, min_samples=50)
            breakdown[name] = r2
            del rr, c2
            torch.cuda.empty_cache()
    if not args.no_prefill:
        c4 = inputs.make_case(inputs.WORKLOADS["prefill_t2048_1m"], with_hca=False)
        a2 = argparse.Namespace(**vars(args))
        a2.steps, a2.warmup, a2.graph_steps, a2.copies = 4, 1, 1, 1  # the rotation still covers 2x the LLC
        r4, rr = bench_csa(torch, csa, c4, a2, detail=True, min_samples=20)
        breakdown["prefill_t2048_1m"] = r4
        del rr, c4
        torch.cuda.empty_cache()
    clocks.append(gpu_clocks())

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case)
        if not args.quick:
            breakdown["cpu_baselines_other_workloads"] = cpu_baselines_other(inputs)

    line = {
        "metric": METRIC, "value": main_res["queries_per_s"], "unit": "queries/s", "n_gpus": 1,
        "steps": main_res["steps"], "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "median_ms_per_step": main_res["median_ms"], "p10_ms_per_step": main_res["p10_ms"],
        "p90_ms_per_step": main_res["p90_ms"], "timing_samples": main_res["samples"],
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
        "stream_read_peak": peak,
        "gpu_clocks": {"before": clocks[0], "under_load": clocks[1], "after": clocks[2]},
        "breakdown": breakdown,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
