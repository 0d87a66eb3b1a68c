"""Per-wave timeline of one batched-decode attention launch (diagnostic).

Loads libdsa_clocks.so, the library built with per-wave clock stamps in the
attention kernel (the default libdsa.so has none), runs the batched decode
(32 x 32768 tokens, 64-token blocks, Top-K 32; head-major cache unless
--layout token_major) through
dsa_sparse_attn_decode_topk -- the fused step's attention kernel, which
selects its blocks from the scores -- and prints one JSON line: the launch's
span, each wave's start-to-end time summarized per XCD (XCC_ID) and per KV
head, and the spread of start and end times.  Clocks are the constant-rate
wall clock, converted at the rate the device reports (100 MHz on MI355X).

    python -m dynamic_sparse_attention_paged_amd.wave_clocks [--layout head_major|token_major]
"""

import argparse
import ctypes
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _stats(a):
    a = np.asarray(a, dtype=np.float64)
    return dict(median=round(float(np.median(a)), 2), p10=round(float(np.percentile(a, 10)), 2),
                p90=round(float(np.percentile(a, 90)), 2), min=round(float(a.min()), 2),
                max=round(float(a.max()), 2), n=int(a.size))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--layout", choices=["head_major", "token_major"], default="head_major")
    ap.add_argument("--warmup", type=int, default=5)
    args = ap.parse_args()

    from dynamic_sparse_attention_paged_amd import _lib
    _lib.LIB_PATH = os.path.join(HERE, "libdsa_clocks.so")
    import torch
    import dynamic_sparse_attention_paged_amd as dsa
    from dsa_synth import device as synth_dev, workload

    assert torch.cuda.is_available(), "wave_clocks needs a GPU"
    lib = _lib.load()
    read = lib.dsa_wave_clocks_read
    read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    read.restype = ctypes.c_int
    khz = ctypes.c_int(0)
    assert lib.dsa_wave_clock_khz(ctypes.byref(khz)) == 0 and khz.value > 0, "wall-clock rate"
    tick_us = 1e3 / khz.value

    w = workload.batched_decode()
    t = synth_dev.upload(w)
    layout = dsa.KV_HEAD_MAJOR if args.layout == "head_major" else dsa.KV_TOKEN_MAJOR
    if layout == dsa.KV_HEAD_MAJOR:
        for name in ("k_cache", "v_cache"):
            t[name] = t[name].permute(0, 2, 1, 3).contiguous()
    kv = dsa.PagedKV(t["k_cache"], t["v_cache"], t["idx_keys"], t["idx_scale"], t["block_table"],
                     t["seq_lens"], kv_layout=layout)
    qs = dsa.Queries(t["q"], t["q_idx"], t["w_idx"], t["q_seq"], t["q_pos"])
    scores = dsa.index_score(kv, qs)
    ws = dsa.make_workspace(_lib.OP_ATTN_DECODE, kv, qs, w.top_k)
    out = torch.empty(w.num_queries, w.num_q_heads, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.num_queries, w.num_q_heads, dtype=torch.float32, device="cuda")

    def launch():
        dsa.sparse_attn_decode_topk(kv, qs, scores, w.top_k, w.softmax_scale, out=out, lse=lse,
                                    workspace=ws)
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    launch()  # the recorded launch: the stamps hold its waves
    torch.cuda.synchronize()

    # every record this process wrote belongs to a launch of this one shape, so
    # the nonzero ones are the recorded launch's waves, in the kernel's order
    # ((KV head * Nq + query) * splits + split) * waves + wave
    cap = 1 << 16
    clocks = np.zeros((cap, 2), dtype=np.uint64)
    where = np.zeros((cap, 2), dtype=np.uint32)
    rc = read(clocks.ctypes.data, where.ctypes.data, cap)
    assert rc == 0, f"dsa_wave_clocks_read: {rc}"
    n = int(np.count_nonzero(clocks[:, 0]))
    hkv, nq, waves = w.num_kv_heads, w.num_queries, 4
    assert n > 0 and n % (hkv * nq * waves) == 0 and np.all(clocks[:n, 0] != 0), n
    splits = n // (hkv * nq * waves)
    clocks, where = clocks[:n], where[:n]
    start = clocks[:, 0].astype(np.int64)
    end = clocks[:, 1].astype(np.int64)
    t0 = start.min()
    s_us = (start - t0) * tick_us
    e_us = (end - t0) * tick_us
    body = e_us - s_us
    xcc = (where[:, 1] & 0xF).astype(int)
    hw = where[:, 0].astype(np.int64)
    cu_key = xcc * 4096 + ((hw >> 13) & 7) * 512 + ((hw >> 12) & 1) * 256 + ((hw >> 8) & 15)
    g = np.arange(n) // (nq * splits * waves)
    res = dict(workload=w.name, kv_layout=args.layout, wall_clock_khz=khz.value,
               kernel="sparse_attn_split<4, 2, 1, 0, 0, true> (dsa_sparse_attn_decode_topk)",
               waves=n, splits=splits, span_us=round(float(e_us.max()), 2),
               wave_start_us=_stats(s_us), wave_end_us=_stats(e_us), wave_body_us=_stats(body),
               per_xcc_body_us={int(x): _stats(body[xcc == x]) for x in sorted(set(xcc))},
               per_xcc_end_us={int(x): _stats(e_us[xcc == x]) for x in sorted(set(xcc))},
               per_kv_head_body_us={int(h): _stats(body[g == h]) for h in range(hkv)},
               distinct_cus=int(np.unique(cu_key).size))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
