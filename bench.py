#!/usr/bin/env python3
"""Throughput of the dynamic-sparse-attention hot path on one MI355X.

A step is one pass of the whole decode hot path -- block-table walk, FP8
indexer scoring, Top-K selection, gather + split-K attention and merge --
through the fused entry point, over one batch of 32 decode queries with a
32768-token paged context each (64-token blocks, 64 query / 8 KV heads of
128, indexer 8 x 128 E4M3, Top-K 32).  Inputs are resident in HBM before the
timed region.  Distinct query batches rotate over the same cache so that
consecutive steps select different blocks (the 256 MiB last-level cache
cannot serve a step from the previous one).

Printed: one JSON line with queries/s (K back-to-back steps between two
synchronizations, launched from the host: a HIP graph replay per step adds a
fixed ~5 us on this ROCm, and its rate is printed beside), per-step HIP-event
times (median, p10, p90; back to back and after a 1 GiB cache flush), the
roofline of the step's dominant kernel (the attention kernel that selects its
blocks from the scores, launched alone through dsa_sparse_attn_decode_topk:
algorithmic bytes over its time from back-to-back launches in one HIP graph,
so that the time is the kernel's and not a lone call's; per-call times
beside it), the same for the whole step and for the given-list attention
kernel, each against the 8 TB/s spec and the streaming-read ceiling
measured in the same run, and the oracle timed on the host's cores on a
bounded sample.  Extra fields report the other workloads (tiny, ragged,
million-token decode; the chunked-prefill indexer) with their own rooflines,
and the chip's measured ceilings.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode queries/sec + achieved HBM GB/s (% roofline); prefill indexer MFMA %"
HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
INT8_PEAK_TOPS = 5000.0
# what one fused step of the batched decode launches (the roofline's scope)
STEP_KERNELS = "index_score_i8_rows + sparse_attn_split (selects its blocks)"
# the step's dominant kernel (the roofline's), as the kernel trace names it
SELECT_KERNEL = "sparse_attn_split<4, 2, 1, 0, 0, true>"
# the sources of the batched-decode step's kernels (the traffic counters are keyed to them)
ATTN_SRCS = [os.path.join(ROOT, "dynamic_sparse_attention_paged_amd", "csrc", f)
             for f in ("attn.hip", "attn_tile.h", "cand_common.h", "select_common.h",
                       "score_common.h", "score_i8_lds.h", "digit_mfma.h", "dsa_internal.h",
                       "index_score.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sparse_attn_split_batched_decode.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def attn_bytes(w, cnt):
    """Algorithmic HBM bytes of the attention kernel for one launch over the batch:
    whole selected K+V blocks of each KV head, the selected ids and their table
    entries, Q (bf16), out (fp32) and lse (fp32)."""
    blk = w.block_size * w.num_kv_heads * w.head_dim * 2 * 2
    per_q_fixed = w.num_q_heads * w.head_dim * (2 + 4) + w.num_q_heads * 4 + 4
    return int(sum(int(c) * (blk + 8) for c in cnt)) + w.num_queries * per_q_fixed


def select_attn_bytes(w, cnt):
    """Algorithmic bytes of the attention kernel that selects its blocks itself:
    those of the given-list kernel plus each query's row of scores (4 B per
    candidate block)."""
    return attn_bytes(w, cnt) + sum(4 * (int(p) // w.block_size) for p in w.q_pos)


def index_bytes(w):
    """Algorithmic bytes of the block-table walk + scoring: per visible block a
    table entry, a coarse key row and a scale; per query q_idx (bf16) and w."""
    tot = 0
    for qi in range(w.num_queries):
        nvis = int(w.q_pos[qi]) // w.block_size + 1
        tot += nvis * (4 + w.idx_dim + 4) + w.idx_heads * (w.idx_dim * 2 + 4) + 4
    return tot


def index_flops(w):
    return sum(2 * w.idx_heads * w.idx_dim * (int(p) // w.block_size + 1) for p in w.q_pos)


class Device:
    """One workload on the device, with `nsets` rotating query batches."""

    def __init__(self, w, nsets, qseed0=5000, kv_layout=None):
        import torch
        import dynamic_sparse_attention_paged_amd as dsa
        from dsa_synth import device as synth_dev, workload

        self.w = w
        self.kv_layout = KV_LAYOUT if kv_layout is None else kv_layout
        t = synth_dev.upload(w)
        if self.kv_layout == dsa.KV_HEAD_MAJOR:  # same values, [P, Hkv, bs, 128]
            for name in ("k_cache", "v_cache"):
                t[name] = t[name].permute(0, 2, 1, 3).contiguous()
            torch.cuda.empty_cache()
        self.kv = dsa.PagedKV(t["k_cache"], t["v_cache"], t["idx_keys"], t["idx_scale"],
                              t["block_table"], t["seq_lens"], kv_layout=self.kv_layout)
        self.sets = [dsa.Queries(t["q"], t["q_idx"], t["w_idx"], t["q_seq"], t["q_pos"])]
        self.hosts = [w]
        for i in range(1, nsets):
            v = workload.with_query_seed(w, qseed0 + i)
            self.hosts.append(v)

            def dev(a, dtype=None):
                import numpy as np
                x = torch.from_numpy(np.ascontiguousarray(a))
                return (x.view(dtype) if dtype is not None else x).cuda()
            import numpy as np
            self.sets.append(dsa.Queries(dev(v.q_bits.view(np.int16), torch.bfloat16),
                                         dev(v.q_idx_bits.view(np.int16), torch.bfloat16),
                                         dev(v.w), t["q_seq"], t["q_pos"]))
        nq, hq = w.num_queries, w.num_q_heads
        self.out = torch.empty(nq, hq, w.head_dim, dtype=torch.float32, device="cuda")
        self.lse = torch.empty(nq, hq, dtype=torch.float32, device="cuda")
        self.idx = [torch.empty(nq, w.top_k, dtype=torch.int32, device="cuda") for _ in self.sets]
        self.cnt = [torch.empty(nq, dtype=torch.int32, device="cuda") for _ in self.sets]
        from dynamic_sparse_attention_paged_amd import _lib
        op = _lib.OP_DECODE_FUSED if w.decode else _lib.OP_INDEX_TOPK
        self.ws = dsa.make_workspace(op, self.kv, self.sets[0], w.top_k)
        self.ws_attn = dsa.make_workspace(_lib.OP_ATTN_DECODE, self.kv, self.sets[0], w.top_k)
        self.scores = torch.empty(nq, w.block_table.shape[1], dtype=torch.float32, device="cuda")
        self.dsa = dsa
        self.sc_sets = None  # per query set: its scores (for the selecting attention alone)
        self.graphs_of = {}

    def fused(self, i, with_idx=False):
        s = i % len(self.sets)
        self.dsa.decode_fused(self.kv, self.sets[s], self.w.top_k, self.w.softmax_scale,
                              out=self.out, lse=self.lse,
                              block_idx=self.idx[s] if with_idx else None,
                              block_cnt=self.cnt[s] if with_idx else None, workspace=self.ws)

    def capture(self):
        """One HIP graph per query set holding a whole fused step (the library
        allocates and synchronizes nothing, so a step is capturable)."""
        import torch
        self.graphs = []
        torch.cuda.synchronize()
        for s in range(len(self.sets)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.fused(s)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def replay(self, i):
        self.graphs[i % len(self.graphs)].replay()

    def capture_attn(self, reps=16):
        """One HIP graph of `reps` back-to-back given-list attention launches over
        the query sets: the kernel's own duration, without a lone call's gap."""
        import torch
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                self.attn(i)
        torch.cuda.synchronize()
        self.attn_graph, self.attn_reps = g, reps

    def attn_launch_ms(self, n):
        """Average HIP-event time (ms) of one attention launch over n replays of
        the back-to-back graph."""
        if getattr(self, "attn_graph", None) is None:
            self.capture_attn()
        return event_time_ms(lambda i: self.attn_graph.replay(), n, 2) / self.attn_reps

    def score_sets(self):
        """Every query set's scores (dsa_index_score), kept for attn_sel."""
        import torch
        self.sc_sets = [torch.empty_like(self.scores) for _ in self.sets]
        for s in range(len(self.sets)):
            self.dsa.index_score(self.kv, self.sets[s], scores=self.sc_sets[s])
        torch.cuda.synchronize()

    def attn_sel(self, i):
        """The fused step's attention kernel alone: it selects each query's blocks
        from the scores, then attends them (dsa_sparse_attn_decode_topk)."""
        s = i % len(self.sets)
        self.dsa.sparse_attn_decode_topk(self.kv, self.sets[s], self.sc_sets[s], self.w.top_k,
                                         self.w.softmax_scale, out=self.out, lse=self.lse,
                                         workspace=self.ws_attn)

    def launch_ms(self, name, fn, n, reps=16):
        """Average HIP-event time (ms) of one launch of fn, from n replays of one
        HIP graph holding `reps` back-to-back calls fn(0), fn(1), ..."""
        import torch
        if name not in self.graphs_of:
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(reps):
                    fn(i)
            torch.cuda.synchronize()
            self.graphs_of[name] = g
        g = self.graphs_of[name]
        return event_time_ms(lambda i: g.replay(), n, 2) / reps

    def select(self):
        for s in range(len(self.sets)):
            self.dsa.index_topk(self.kv, self.sets[s], self.w.top_k, block_idx=self.idx[s],
                                block_cnt=self.cnt[s], workspace=self.ws)

    def attn(self, i):
        s = i % len(self.sets)
        if self.w.decode:
            self.dsa.sparse_attn_decode(self.kv, self.sets[s], self.idx[s], self.cnt[s],
                                        self.w.top_k, self.w.softmax_scale, out=self.out,
                                        lse=self.lse, workspace=self.ws_attn)
        else:
            self.dsa.sparse_attn_prefill(self.kv, self.sets[s], self.idx[s], self.cnt[s],
                                         self.w.top_k, self.w.softmax_scale, out=self.out,
                                         lse=self.lse)

    def itopk(self, i):
        """Scoring and selection in one call (dsa_index_topk)."""
        s = i % len(self.sets)
        self.dsa.index_topk(self.kv, self.sets[s], self.w.top_k, block_idx=self.idx[s],
                            block_cnt=self.cnt[s], workspace=self.ws)

    def score(self, i):
        s = i % len(self.sets)
        self.dsa.index_score(self.kv, self.sets[s], scores=self.scores)

    def topk(self, i):
        s = i % len(self.sets)
        self.dsa.topk_blocks(self.scores, self.kv, self.sets[s], self.w.top_k,
                             block_idx=self.idx[s], block_cnt=self.cnt[s])


def event_time_ms(fn, n, warmup):
    """Average HIP-event time (ms) of fn(i) over n back-to-back calls on the current stream."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


class Flusher:
    """Writes a 1 GiB scratch buffer (dsa_cache_flush), more than the L2s and the
    256 MiB last-level cache hold, so that the next step finds none of its
    inputs cached."""

    def __init__(self, nbytes=1 << 30):
        import torch
        from dynamic_sparse_attention_paged_amd import _lib
        self.lib = _lib.load()
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.n = 0

    def __call__(self):
        import torch
        self.n += 1
        rc = self.lib.dsa_cache_flush(self.buf.data_ptr(), self.buf.numel(), self.n,
                                      torch.cuda.current_stream().cuda_stream)
        assert rc == 0, "dsa_cache_flush failed"


def step_times_ms(fn, n, warmup, flush=None):
    """Per-call HIP-event times (ms) of fn(i): every call bracketed by its own
    pair of events on the current stream; with `flush`, an untimed cache flush
    runs on the same stream before each call."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i in range(n):
        if flush is not None:
            flush()
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def dist(ts):
    """median / p10 / p90 / mean of a list of times (ms)."""
    import numpy as np
    a = np.asarray(ts, dtype=np.float64)
    return dict(median=round(float(np.median(a)), 5), p10=round(float(np.percentile(a, 10)), 5),
                p90=round(float(np.percentile(a, 90)), 5), mean=round(float(a.mean()), 5),
                n=int(a.size))


# Order inside a cache block, by its dsa_kv_layout value.
LAYOUT_NAMES = ["token_major", "head_major"]
KV_LAYOUT = 1


def traffic_from_profile():
    """Measured HBM bytes (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated on a
    device copy) of the batched-decode step, of its selecting attention kernel
    and of the given-list attention kernel, if the counters in profiles/ were
    taken on the current sources: (step, selecting, given_list), else Nones."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        src = hashlib.sha256(b"".join(open(f, "rb").read() for f in ATTN_SRCS)).hexdigest()
        if t.get("src_sha256") != src or t.get("kv_layout") != LAYOUT_NAMES[KV_LAYOUT]:
            return None, None, None
        sel = t.get("kernels", {}).get(SELECT_KERNEL, {}).get("bytes_per_dispatch")
        return t.get("step_bytes"), sel, t.get("given_list_bytes")
    except (OSError, ValueError):
        return None, None, None


def _oracle_decode_loop(w, budget_s, qseed0):
    """The oracle on decode queries of w for ~budget_s of compute: scoring,
    selection and attention timed, K/V regeneration (input generation) not.
    Each pass over the batch takes fresh query seeds.  Returns (queries, s)."""
    import numpy as np
    from oracle import bf16_bits_to_f64, select_blocks, sparse_attention
    from oracle.pipeline import score_query
    from dsa_synth import workload
    spent, done = 0.0, 0
    src = w
    for i in range(1 << 30):
        qi = i % w.num_queries
        if i and qi == 0:  # a fresh batch of queries over the same cache
            src = workload.with_query_seed(w, qseed0 + i // w.num_queries)
        s, pos = int(w.q_seq[qi]), int(w.q_pos[qi])
        L = int(w.seq_lens[s])
        qidx = bf16_bits_to_f64(src.q_idx_bits[qi])
        t0 = time.perf_counter()
        cand, sc, loc = score_query(qidx, src.w[qi], w.block_table[s], pos, L, w.block_size,
                                    w.idx_keys, w.idx_scale)
        idx, cnt = select_blocks(cand, sc.astype(np.float32), loc, w.top_k)
        t1 = time.perf_counter()
        blocks = {int(w.block_table[s][j]): (bf16_bits_to_f64(w.k_block_bits(int(w.block_table[s][j]))),
                                             bf16_bits_to_f64(w.v_block_bits(int(w.block_table[s][j]))))
                  for j in idx[:cnt]}
        t2 = time.perf_counter()
        sparse_attention(bf16_bits_to_f64(src.q_bits[qi]), idx[:cnt], w.block_table[s], pos, L,
                         w.block_size, lambda p: blocks[p][0], lambda p: blocks[p][1],
                         w.softmax_scale, w.num_kv_heads)
        t3 = time.perf_counter()
        spent += (t1 - t0) + (t3 - t2)
        done += 1
        if spent >= budget_s:
            break
    return done, spent


def _oracle_worker(args):
    w, budget_s, qseed0 = args
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return _oracle_decode_loop(w, budget_s, qseed0)


def host_cores():
    """CPUs this process may run on (the GPU machine grants 16 per GPU)."""
    return len(os.sched_getaffinity(0))


def cpu_baseline(w, budget_s, prefill_w=None):
    """The oracle (float64 NumPy, as it stands) timed on the host's cores over a
    bounded sample of the workload: one process per core, each running decode
    queries of the batch for ~budget_s of compute (BLAS held to one thread per
    process), queries/s summed; the same on one thread; and a sample of
    chunked-prefill queries on one thread."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    cores = host_cores()
    procs = min(cores, 16)
    with threadpool_limits(limits=1):
        d1, s1 = _oracle_decode_loop(w, budget_s / 3, 7000)
    ctx = mp.get_context("fork")
    with ctx.Pool(procs) as pool:
        parts = pool.map(_oracle_worker, [(w, budget_s / 3, 9000 + 1000 * i) for i in range(procs)])
    done = sum(p[0] for p in parts)
    rate = sum(p[0] / p[1] for p in parts)
    res = dict(value=round(rate, 2), unit="queries/s", cores=procs, kind="oracle",
               sample=f"{done} decode queries of {w.name} in {procs} processes (one per core, "
                      f"BLAS 1 thread each; batches of {w.num_queries} with fresh query seeds; "
                      f"~{budget_s / 3:.0f} s of compute per process; K/V regeneration not "
                      f"timed); float64 NumPy",
               host_cpus=cores,
               single_thread=dict(value=round(d1 / s1, 2), unit="queries/s", queries=d1,
                                  seconds=round(s1, 2)))
    if prefill_w is not None:
        import numpy as np
        from oracle import bf16_bits_to_f64, select_blocks, sparse_attention
        from oracle.pipeline import score_query
        pw = prefill_w
        spent, done = 0.0, 0
        qis = np.linspace(0, pw.num_queries - 1, 64).astype(int)
        with threadpool_limits(limits=1):
            for qi in qis:
                s, pos = int(pw.q_seq[qi]), int(pw.q_pos[qi])
                L = int(pw.seq_lens[s])
                t0 = time.perf_counter()
                cand, sc, loc = score_query(bf16_bits_to_f64(pw.q_idx_bits[qi]), pw.w[qi],
                                            pw.block_table[s], pos, L, pw.block_size,
                                            pw.idx_keys, pw.idx_scale)
                idx, cnt = select_blocks(cand, sc.astype(np.float32), loc, pw.top_k)
                t1 = time.perf_counter()
                blk = {int(pw.block_table[s][j]): (bf16_bits_to_f64(pw.k_block_bits(int(pw.block_table[s][j]))),
                                                   bf16_bits_to_f64(pw.v_block_bits(int(pw.block_table[s][j]))))
                       for j in idx[:cnt]}
                t2 = time.perf_counter()
                sparse_attention(bf16_bits_to_f64(pw.q_bits[qi]), idx[:cnt], pw.block_table[s],
                                 pos, L, pw.block_size, lambda p: blk[p][0], lambda p: blk[p][1],
                                 pw.softmax_scale, pw.num_kv_heads)
                t3 = time.perf_counter()
                spent += (t1 - t0) + (t3 - t2)
                done += 1
                if spent >= budget_s / 3:
                    break
        res["prefill_single_thread"] = dict(
            value=round(done / spent, 2), unit="queries/s", queries=done, seconds=round(spent, 2),
            sample=f"{done} queries spread over the {pw.num_queries}-query chunk of {pw.name}")
    return res


def hbm_roofline(nbytes, ms, kernel, scope, ceil_gbps=None, traffic=None):
    """Roofline object for an HBM-bound launch sequence: algorithmic bytes per
    step over the step's HIP-event time."""
    gbps = nbytes / (ms * 1e-3) / 1e9
    r = {"kernel": kernel, "scope": scope, "bound": "hbm", "achieved": round(gbps, 1),
         "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
         "traffic": traffic, "bytes_per_launch": int(nbytes), "avg_launch_ms": round(ms, 5)}
    if ceil_gbps:
        r["measured_ceiling"] = round(ceil_gbps, 1)
        r["frac_of_measured_ceiling"] = round(gbps / ceil_gbps, 4)
    return r


def decode_extra(w, steps, nsets, kv_layout=None, ceil_gbps=None):
    """q/s and HBM GB/s of a decode workload through the fused entry point.
    The rate (ms_per_step, queries_per_s, the step roofline) comes from `steps`
    back-to-back host launches between two HIP events, as the headline figure
    does (graph_replay_ms_per_step: the same with one HIP graph replay a step);
    step_ms and step_ms_flushed are per-call HIP-event times (each step
    bracketed by its own events, so they include the launch gap a lone call
    pays; the second after a cache flush).  The attention kernel is timed
    alone on the same selection."""
    import torch
    D = Device(w, nsets, kv_layout=kv_layout)
    D.capture()
    ms = event_time_ms(D.fused, steps, 3)
    g_ms = event_time_ms(D.replay, steps, 3)
    b2b = step_times_ms(D.fused, steps, 3)
    fl = step_times_ms(D.fused, max(5, steps // 2), 1, flush=Flusher())
    D.select()
    torch.cuda.synchronize()
    attn = step_times_ms(D.attn, steps, 3)
    attn_ms = D.attn_launch_ms(max(3, steps // 8))
    cnt = D.cnt[0].cpu().numpy()
    a_bytes = attn_bytes(w, cnt)
    byts = a_bytes + index_bytes(w)
    res = dict(workload=w.name, kv_layout=LAYOUT_NAMES[D.kv_layout], queries=w.num_queries,
               ms_per_step=round(ms, 5), graph_replay_ms_per_step=round(g_ms, 5),
               step_ms=dist(b2b), step_ms_flushed=dist(fl),
               queries_per_s=round(w.num_queries / (ms * 1e-3), 1),
               roofline=hbm_roofline(byts, ms, "dsa_sparse_decode_fused (every launch of the step)",
                                     "step", ceil_gbps),
               attention_kernel=hbm_roofline(a_bytes, attn_ms,
                                             "sparse_attn_split (given lists)", "kernel",
                                             ceil_gbps))
    res["attention_kernel"]["per_call_ms"] = dist(attn)
    del D
    torch.cuda.empty_cache()
    return res


def ceilings_extra(quick=False):
    """What the chip sustains, from the library's support probes: a streaming
    read of 4 GiB (plain and non-temporal loads, several grid sizes) and
    back-to-back MFMAs (FP8 scaled 16x16x128, int8 16x16x64, bf16 16x16x32)."""
    import torch
    from dynamic_sparse_attention_paged_amd import _lib
    lib = _lib.load()
    st = torch.cuda.current_stream().cuda_stream
    nbytes = 4 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(16384 * 256, dtype=torch.int32, device="cuda")
    rows = []
    grids = (512, 1024) if quick else (256, 512, 768, 1024, 2048, 8192)
    for var in (0, 1):
        for grid in grids:
            def f(i, var=var, grid=grid):
                assert lib.dsa_probe_stream_read(buf.data_ptr(), nbytes, var, sink.data_ptr(), grid,
                                                 st) == 0
            ts = step_times_ms(f, 6, 2)
            med = dist(ts)["median"]
            rows.append(dict(loads="nt" if var else "plain", grid=grid, ms=med,
                             gbps=round(nbytes / (med * 1e-3) / 1e9, 1)))
    del buf
    torch.cuda.empty_cache()
    best = max(rows, key=lambda r: r["gbps"])
    res = dict(stream_read=rows, stream_read_best_gbps=best["gbps"],
               stream_read_best_frac_of_spec=round(best["gbps"] / HBM_PEAK_GBPS, 4))
    if not quick:
        sinkf = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
        mf = {}
        for kind, name, fl, peak in ((0, "fp8_16x16x128", 65536, FP8_PEAK_TFLOPS),
                                     (1, "i8_16x16x64", 32768, INT8_PEAK_TOPS),
                                     (2, "bf16_16x16x32", 16384, 2500.0)):
            grid, iters = 1024, 2000

            def f(i, kind=kind):
                assert lib.dsa_probe_mfma_rate(kind, iters, grid, sinkf.data_ptr(), st) == 0
            med = dist(step_times_ms(f, 4, 1))["median"]
            tf = grid * 4 * iters * 8 * fl / (med * 1e-3) / 1e12
            mf[name] = dict(tflops=round(tf, 1), frac_of_spec=round(tf / peak, 4))
        res["mfma"] = mf
    return res


def block_size_extra(steps):
    """The batched decode shape at 64, 128, 256 and 512 tokens per block, with
    top_k = 2048 / block_size (the same attended tokens): the pages' block-size
    tuning sweep through the fused entry point."""
    from dsa_synth import workload
    res = {}
    for bs in (64, 128, 256, 512):
        log(f"extra: block size {bs}")
        res[f"bs{bs}"] = decode_extra(workload.batched_decode_blocks(bs), steps, 4)
    return res


def moe_extra(steps):
    """MXFP4 expert layer (synthetic weights and routing): 64 experts with
    W_e [4096 x 7168] in MXFP4, each token routed to 8 distinct experts.  A
    decode batch (256 tokens: 2048 pairs, ~32 per expert) is bound by reading
    the weights; a prefill batch (4096 tokens) by the matrix cores.  Both modes
    of the grouped matmul: FP4 weights straight to the scaled matrix cores, and
    the pages' online unpack to an FP8 workspace followed by the FP8 matmul."""
    import torch
    import dynamic_sparse_attention_paged_amd as dsa
    from dynamic_sparse_attention_paged_amd import _lib
    e_n, n, k, top = 64, 4096, 7168, 8
    g = torch.Generator(device="cuda")
    g.manual_seed(7001)
    w_fp4 = torch.randint(0, 256, (e_n, n, k // 2), dtype=torch.uint8, device="cuda", generator=g)
    w_scale = torch.randint(118, 131, (e_n, n, k // 32), dtype=torch.uint8, device="cuda",
                            generator=g)
    w = dsa.MxExperts(w_fp4, w_scale)
    res = {}
    for label, t in (("decode_256_tokens", 256), ("prefill_4096_tokens", 4096)):
        x = torch.randn(t, k, device="cuda", generator=g).to(torch.bfloat16)
        route = torch.rand(t, e_n, device="cuda", generator=g).argsort(dim=1)[:, :top]
        route = route.to(torch.int32).contiguous()
        xc, xs = dsa.mx_quantize(x)
        out = torch.empty(t, top, n, dtype=torch.float32, device="cuda")
        active = int(torch.unique(route).numel())
        pairs = t * top
        flops = 2.0 * pairs * n * k
        w_bytes = active * (n * k // 2 + n * k // 32)
        io_bytes = pairs * n * 4 + t * (k + k // 32)
        row = dict(tokens=t, pairs=pairs, active_experts=active)
        for mode, name in ((_lib.MOE_FP4_DIRECT, "fp4_direct"), (_lib.MOE_FP8_WORKSPACE,
                                                                 "fp8_workspace")):
            ws = dsa._workspace(dsa.moe_workspace_size(w, t, top, mode), x.device)

            def step(i):
                dsa.moe_grouped_gemm(w, xc, xs, route, mode=mode, out=out, workspace=ws)
            ms = event_time_ms(step, steps, 2)
            row[name] = dict(ms=round(ms, 4), tflops=round(flops / (ms * 1e-3) / 1e12, 1),
                             weight_gbps=round(w_bytes / (ms * 1e-3) / 1e9, 1),
                             frac_of_hbm_mxfp4_bytes=round((w_bytes + io_bytes) / (ms * 1e-3)
                                                           / 1e9 / HBM_PEAK_GBPS, 4),
                             workspace_gb=round(ws.numel() / 1e9, 3))
            del ws
        q_ms = event_time_ms(lambda i: dsa.mx_quantize(x, codes=xc, scales=xs), steps, 2)
        row["mx_quantize_ms"] = round(q_ms, 4)
        res[label] = row
        del x, out, xc, xs
    res["note"] = ("weight bytes = MXFP4 codes + scales of the routed experts; tflops counts "
                   "2 * pairs * N * K; fp8 frac_of_fp8_mfma_peak for the prefill batch: "
                   "tflops / 5000")
    del w, w_fp4, w_scale
    torch.cuda.empty_cache()
    return res


def write_path_extra(steps):
    """The paged write path at the chunked-prefill shape: one chunk of 8192
    tokens written into a 2048-block pool (HBM-bound copy through the block
    table), the 128 coarse keys of the chunk's blocks, and a 32-token decode
    append (latency)."""
    import numpy as np
    import torch
    import dynamic_sparse_attention_paged_amd as dsa
    from dsa_synth import gen
    P, hkv, d, di, n = 2048, 8, 128, 128, 8192
    k = torch.zeros((P, 64, hkv, d), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    keys = torch.zeros((P, di), dtype=torch.uint8, device="cuda")
    scale = torch.zeros(P, dtype=torch.float32, device="cuda")
    perm = torch.from_numpy(gen.permutation(4242, gen.TAG_TABLE, P).astype(np.int32)).cuda()
    table = perm.view(1, P)
    seq_lens = torch.tensor([P * 64], dtype=torch.int32, device="cuda")
    kv = dsa.PagedKV(k, v, keys, scale, table, seq_lens)
    k_new = torch.randn((n, hkv, d), device="cuda").to(torch.bfloat16)
    v_new = torch.randn((n, hkv, d), device="cuda").to(torch.bfloat16)
    tok_seq = torch.zeros(n, dtype=torch.int32, device="cuda")
    tok_pos = torch.arange(P * 64 - n, P * 64, dtype=torch.int32, device="cuda")
    ms = event_time_ms(lambda i: dsa.kv_write(kv, k_new, v_new, tok_seq, tok_pos), steps, 3)
    moved = 2 * 2 * k_new.numel() * 2  # K and V, read and written
    blocks = perm[P - n // 64:].contiguous()
    coarse = torch.randn((n // 64, di), device="cuda")
    key_ms = event_time_ms(lambda i: dsa.index_key_write(kv, blocks, coarse), steps, 3)
    # decode append: 32 sequences, the newest token of each
    tables = perm[:32 * 64].view(32, 64).contiguous()
    kv32 = dsa.PagedKV(k, v, keys, scale, tables,
                       torch.full((32,), 64 * 64, dtype=torch.int32, device="cuda"))
    app_ms = event_time_ms(lambda i: dsa.kv_write(kv32, k_new[:32], v_new[:32]), steps, 3)
    res = dict(workload="kv_write_8192_tokens_hkv8", kv_write_ms=round(ms, 4),
               bytes_moved=moved, gbps=round(moved / (ms * 1e-3) / 1e9, 1),
               frac_of_hbm=round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
               index_key_write_128_blocks_us=round(key_ms * 1e3, 2),
               decode_append_32_tokens_us=round(app_ms * 1e3, 2))
    del kv, kv32, k, v
    torch.cuda.empty_cache()
    return res


def prefill_indexer_extra(steps):
    """Chunked-prefill indexer: TFLOP/s and fraction of the FP8 MFMA peak."""
    import torch
    from dsa_synth import workload
    w = workload.chunked_prefill()
    D = Device(w, 1)
    sc_t = step_times_ms(D.score, steps, 2)
    ms = dist(sc_t)["mean"]
    fl = index_flops(w)
    tk_ms = event_time_ms(D.topk, steps, 2)
    at_ms = event_time_ms(D.attn, max(2, steps // 4), 1)
    res = dict(workload=w.name, score_kernel_ms=round(ms, 4),
               algorithmic_gflop=round(fl / 1e9, 3),
               tflops=round(fl / (ms * 1e-3) / 1e12, 2),
               frac_of_fp8_mfma_peak=round(fl / (ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
               int8_digit_tops=round(9 * fl / (ms * 1e-3) / 1e12, 2),
               frac_of_int8_mfma_peak=round(9 * fl / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
               note="exact scoring on the int8 matrix cores: each E4M3 product is nine "
                    "base-128 digit products (the FP8 MFMA accumulation is inexact on gfx950); "
                    "frac_of_fp8_mfma_peak counts the algorithmic FP8 flops, "
                    "frac_of_int8_mfma_peak the digit products issued for them",
               topk_ms=round(tk_ms, 4), attention_ms=round(at_ms, 3),
               score_kernel_step_ms=dist(sc_t))
    # scoring + selection in one launch (approximate FP8 scores, exact ones
    # where the bound leaves the boundary undecided): the graded indexer.  Its
    # roofline takes the kernel's own duration, from back-to-back launches
    # between two HIP events (a lone call's launch gap is not the kernel's);
    # per-call times beside it
    it_t = step_times_ms(D.itopk, steps, 2)
    it_ms = event_time_ms(D.itopk, max(steps, 20), 3)
    res.update(index_topk_ms=round(it_ms, 5), index_topk_step_ms=dist(it_t),
               roofline={"kernel": "index_topk_fp8 (dsa_index_topk: scoring + selection)",
                         "scope": "kernel", "bound": "mfma",
                         "achieved": round(fl / (it_ms * 1e-3) / 1e12, 2),
                         "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(fl / (it_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                         "traffic": None, "flops_per_launch": int(fl),
                         "avg_launch_ms": round(it_ms, 5)})
    # the one-call prefill: scoring, selection and the block-inverted attention
    from dynamic_sparse_attention_paged_amd import _lib
    ws = D.dsa.make_workspace(_lib.OP_PREFILL_FUSED, D.kv, D.sets[0], w.top_k)

    def fused(i):
        D.dsa.prefill_fused(D.kv, D.sets[0], w.top_k, w.softmax_scale, out=D.out, lse=D.lse,
                            workspace=ws)
    f_ms = event_time_ms(fused, max(2, steps // 2), 1)
    res.update(prefill_fused_ms=round(f_ms, 3),
               prefill_fused_queries_per_s=round(w.num_queries / (f_ms * 1e-3), 1),
               prefill_fused_workspace_gb=round(ws.numel() / 1e9, 2),
               prefill_stagewise_ms=round(ms + tk_ms + at_ms, 3))
    del ws
    del D
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--query-sets", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=30.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time per-step HIP graph replays instead of host launches (a replay "
                         "adds a fixed ~5 us a step on this ROCm; the other mode is reported "
                         "beside the figure either way)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--kv-layout", choices=["head_major", "token_major"], default="head_major",
                    help="order inside a cache block: [head][token][dim] or the pages' "
                         "[token][head][dim] (the other one is timed as an extra)")
    ap.add_argument("--extra", choices=["tiny_decode", "million_decode", "ragged_decode",
                                        "chunked_prefill", "write_path", "block_sizes", "moe",
                                        "ceilings"],
                    help="run only this secondary workload (for profiling) and print its line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from dsa_synth import workload

    global KV_LAYOUT
    KV_LAYOUT = LAYOUT_NAMES.index(args.kv_layout)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.extra:
        if args.extra == "chunked_prefill":
            res = prefill_indexer_extra(args.steps)
        elif args.extra == "write_path":
            res = write_path_extra(args.steps)
        elif args.extra == "block_sizes":
            res = block_size_extra(args.steps)
        elif args.extra == "moe":
            res = moe_extra(args.steps)
        elif args.extra == "ceilings":
            res = ceilings_extra()
        else:
            fn = getattr(workload, args.extra)
            res = decode_extra(fn(), args.steps, 4 if args.extra != "tiny_decode" else 8)
        print(json.dumps(res), flush=True)
        return
    log("ceilings: streaming read")
    ceil = ceilings_extra(quick=True)
    ceil_gbps = ceil["stream_read_best_gbps"]
    w = workload.batched_decode()
    log(f"workload {w.name}: pool {w.num_blocks} blocks, {args.query_sets} query sets")
    D = Device(w, args.query_sets)

    # timed region: K fused steps launched back to back from the host (or, with
    # --graph, replayed from one HIP graph a step), inputs resident
    D.capture()
    step = D.replay if args.graph else D.fused
    other = D.fused if args.graph else D.replay
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    log(f"fused step {ms_step * 1e3:.1f} us")
    # the same K steps between two HIP events on the launch stream (the step
    # roofline's time), the other launch mode likewise, and each step bracketed
    # by its own events, back to back and after a 1 GiB cache flush
    ms_ev = event_time_ms(step, args.steps, 2)
    ms_other = event_time_ms(other, args.steps, 2)
    b2b = step_times_ms(step, args.steps, 2)
    flushed = step_times_ms(step, args.steps, 2, flush=Flusher())

    # the attention kernel alone on the step's selection, and the stages
    D.select()
    torch.cuda.synchronize()
    attn_t = step_times_ms(D.attn, args.steps, 3)
    attn_ms = D.attn_launch_ms(max(3, args.steps // 8))
    score_ms = event_time_ms(D.score, args.steps, 3)
    topk_ms = event_time_ms(D.topk, args.steps, 3)
    # the step's own attention kernel (it selects from the scores) alone
    D.score_sets()
    sel_t = step_times_ms(D.attn_sel, args.steps, 3)
    sel_ms = D.launch_ms("attn_sel", D.attn_sel, max(3, args.steps // 8))
    cnt = D.cnt[0].cpu().numpy()
    a_bytes = attn_bytes(w, cnt)
    s_bytes = select_attn_bytes(w, cnt)
    path_bytes = a_bytes + index_bytes(w)
    traffic, traffic_sel, traffic_given = traffic_from_profile()

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    result = {
        "metric": METRIC,
        "value": round(w.num_queries / (ms_step * 1e-3), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.num_queries, "context_tokens": 32768,
                   "block_size": 64, "q_heads": 64, "kv_heads": 8, "head_dim": 128,
                   "idx_heads": 8, "idx_dim": 128, "top_k": w.top_k,
                   "query_sets": args.query_sets, "kv_layout": args.kv_layout,
                   "entry": "dsa_sparse_decode_fused",
                   "launch": "hip_graph_replay" if args.graph else "host_launch"},
        "hbm_gbps": round(path_bytes / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(path_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "step_ms_events": round(ms_ev, 5),
        "other_launch": {"launch": "host_launch" if args.graph else "hip_graph_replay",
                         "ms_per_step": round(ms_other, 5)},
        "step_ms": dist(b2b),
        "step_ms_flushed": dist(flushed),
        "roofline": hbm_roofline(s_bytes, sel_ms,
                                 f"{SELECT_KERNEL}: the step's attention kernel, selecting its "
                                 "blocks from the scores (dsa_sparse_attn_decode_topk)",
                                 "kernel", ceil_gbps, traffic_sel),
        "step_roofline": hbm_roofline(path_bytes, ms_ev, STEP_KERNELS, "step", ceil_gbps, traffic),
        "attention_kernel": hbm_roofline(a_bytes, attn_ms,
                                         "sparse_attn_split (given lists)", "kernel", ceil_gbps,
                                         traffic_given),
        "stages_ms": {"index_score": round(score_ms, 5), "topk": round(topk_ms, 5),
                      "sparse_attn": round(attn_ms, 5), "sparse_attn_topk": round(sel_ms, 5)},
        "ceilings": ceil,
    }
    result["attention_kernel"]["per_call_ms"] = dist(attn_t)
    result["roofline"]["per_call_ms"] = dist(sel_t)
    del D
    torch.cuda.empty_cache()

    if not args.no_extras:
        extras = {}
        for name, fn, steps in (("tiny_decode", workload.tiny_decode, 200),
                                ("million_decode", workload.million_decode, 50),
                                ("ragged_decode", workload.ragged_decode, 20)):
            log(f"extra: {name}")
            extras[name] = decode_extra(fn(), steps, 4 if name != "tiny_decode" else 8,
                                        ceil_gbps=ceil_gbps)
        other = 1 - KV_LAYOUT
        log(f"extra: batched decode, {LAYOUT_NAMES[other]} cache")
        extras["batched_decode_" + LAYOUT_NAMES[other]] = decode_extra(w, 50, 8, kv_layout=other,
                                                                       ceil_gbps=ceil_gbps)
        log("extra: chunked_prefill indexer")
        extras["chunked_prefill"] = prefill_indexer_extra(5)
        log("extra: write path")
        extras["write_path"] = write_path_extra(20)
        extras["block_sizes"] = block_size_extra(20)
        log("extra: MXFP4 expert layer")
        extras["moe_mxfp4"] = moe_extra(10)
        log("extra: ceilings (stream read, matrix cores)")
        extras["ceilings"] = ceilings_extra()
        result["extras"] = extras

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds,
                                              prefill_w=workload.chunked_prefill())
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
