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

Printed: one JSON line with queries/s, the roofline of the dominant kernel
(sparse attention: HBM bytes per launch / its HIP-event duration), and the
oracle timed on the host on a bounded sample.  Extra fields report the other
workloads (tiny, ragged, million-token decode; the chunked-prefill indexer).

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
# the decode attention kernel's sources (the traffic counters are keyed to them)
ATTN_SRCS = [os.path.join(ROOT, "dynamic_sparse_attention_paged_amd", "csrc", f)
             for f in ("attn.hip", "attn_tile.h")]
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

    def score(self, i):
        s = i % len(self.sets)
        self.dsa.index_score(self.kv, self.sets[s], scores=self.scores)

    def topk(self, i):
        s = i % len(self.sets)
        self.dsa.topk_blocks(self.scores, self.kv, self.sets[s], self.w.top_k,
                             block_idx=self.idx[s], block_cnt=self.cnt[s])


def event_time_ms(fn, n, warmup):
    """Average HIP-event time (ms) of fn(i) over n calls on the current stream."""
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


# Order inside a cache block, by its dsa_kv_layout value.
LAYOUT_NAMES = ["token_major", "head_major"]
KV_LAYOUT = 1


def traffic_from_profile():
    """Measured HBM bytes per launch of the attention kernel, if the counters in
    profiles/ were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        src = hashlib.sha256(b"".join(open(f, "rb").read() for f in ATTN_SRCS)).hexdigest()
        if t.get("attn_src_sha256") != src or t.get("kv_layout") != LAYOUT_NAMES[KV_LAYOUT]:
            return None
        return t.get("bytes_per_launch")
    except (OSError, ValueError):
        return None


def cpu_baseline(w, budget_s):
    """The oracle on the host: scoring + selection + attention for as many queries
    of the batch as fit in ~budget_s (K/V generation excluded from the timing)."""
    import numpy as np
    from oracle import bf16_bits_to_f64, select_blocks, sparse_attention
    from oracle.pipeline import score_query
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    from dsa_synth import workload
    spent, done = 0.0, 0
    src = w
    for i in range(1 << 30):
        qi = i % w.num_queries
        if i and qi == 0:  # a fresh batch of queries over the same cache
            src = workload.with_query_seed(w, 7000 + i // w.num_queries)
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
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return dict(value=done / spent, unit="queries/s", cores=1, kind="oracle",
                sample=f"{done} decode queries of {w.name} (batches of {w.num_queries} with "
                       f"fresh query seeds; float64 NumPy, 1 thread; K/V regeneration not "
                       f"timed)", seconds=round(spent, 2))


def decode_extra(w, steps, nsets, kv_layout=None):
    """q/s and HBM GB/s of a decode workload through the fused entry point."""
    import torch
    D = Device(w, nsets, kv_layout=kv_layout)
    D.capture()
    ms = event_time_ms(D.replay, steps, 3)
    D.select()
    torch.cuda.synchronize()
    attn_ms = event_time_ms(D.attn, steps, 3)
    cnt = D.cnt[0].cpu().numpy()
    byts = attn_bytes(w, cnt) + index_bytes(w)
    res = dict(workload=w.name, kv_layout=LAYOUT_NAMES[D.kv_layout], queries=w.num_queries,
               ms_per_step=round(ms, 5),
               queries_per_s=round(w.num_queries / (ms * 1e-3), 1),
               path_gbps=round(byts / (ms * 1e-3) / 1e9, 1),
               path_frac_of_hbm=round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
               attn_kernel_ms=round(attn_ms, 5),
               attn_kernel_gbps=round(attn_bytes(w, cnt) / (attn_ms * 1e-3) / 1e9, 1),
               attn_kernel_frac_of_hbm=round(attn_bytes(w, cnt) / (attn_ms * 1e-3) / 1e9 /
                                             HBM_PEAK_GBPS, 4))
    del D
    torch.cuda.empty_cache()
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
    ms = event_time_ms(D.score, steps, 2)
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
               topk_ms=round(tk_ms, 4), attention_ms=round(at_ms, 3))
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
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every step from Python instead of replaying HIP graphs")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--kv-layout", choices=["head_major", "token_major"], default="head_major",
                    help="order inside a cache block: [head][token][dim] or the pages' "
                         "[token][head][dim] (the other one is timed as an extra)")
    ap.add_argument("--extra", choices=["tiny_decode", "million_decode", "ragged_decode",
                                        "chunked_prefill", "write_path", "block_sizes", "moe"],
                    help="run only this secondary workload (for profiling) and print its line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
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
        else:
            fn = getattr(workload, args.extra)
            res = decode_extra(fn(), args.steps, 4 if args.extra != "tiny_decode" else 8)
        print(json.dumps(res), flush=True)
        return
    w = workload.batched_decode()
    log(f"workload {w.name}: pool {w.num_blocks} blocks, {args.query_sets} query sets")
    D = Device(w, args.query_sets)

    # timed region: K fused steps replayed from HIP graphs, inputs resident
    step = D.fused
    if not args.no_graph:
        D.capture()
        step = D.replay
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

    # dominant kernel (attention) on the same stream, HIP events over the loop
    D.select()
    torch.cuda.synchronize()
    attn_ms = event_time_ms(D.attn, args.steps, 3)
    score_ms = event_time_ms(D.score, args.steps, 3)
    topk_ms = event_time_ms(D.topk, args.steps, 3)
    cnt = D.cnt[0].cpu().numpy()
    a_bytes = attn_bytes(w, cnt)
    path_bytes = a_bytes + index_bytes(w)
    achieved = a_bytes / (attn_ms * 1e-3) / 1e9
    traffic = traffic_from_profile()

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
                   "launch": "eager" if args.no_graph else "hip_graph_replay"},
        "hbm_gbps": round(path_bytes / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(path_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"kernel": "sparse_attn_split", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "bytes_per_launch": a_bytes,
                     "avg_launch_ms": round(attn_ms, 5)},
        "stages_ms": {"index_score": round(score_ms, 5), "topk": round(topk_ms, 5),
                      "sparse_attn": round(attn_ms, 5)},
    }
    del D
    torch.cuda.empty_cache()

    if not args.no_extras:
        extras = {}
        for name, fn, steps in (("tiny_decode", workload.tiny_decode, 200),
                                ("million_decode", workload.million_decode, 50),
                                ("ragged_decode", workload.ragged_decode, 20)):
            log(f"extra: {name}")
            extras[name] = decode_extra(fn(), steps, 4 if name != "tiny_decode" else 8)
        other = 1 - KV_LAYOUT
        log(f"extra: batched decode, {LAYOUT_NAMES[other]} cache")
        extras["batched_decode_" + LAYOUT_NAMES[other]] = decode_extra(w, 50, 8, kv_layout=other)
        log("extra: chunked_prefill indexer")
        extras["chunked_prefill"] = prefill_indexer_extra(5)
        log("extra: write path")
        extras["write_path"] = write_path_extra(20)
        extras["block_sizes"] = block_size_extra(20)
        log("extra: MXFP4 expert layer")
        extras["moe_mxfp4"] = moe_extra(10)
        result["extras"] = extras

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
