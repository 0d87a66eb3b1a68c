"""Helpers shared by the GPU parity tests, smoke() and bench.py.

Upload a synthetic workload to the device, run the oracle on chosen queries
(regenerating the needed K/V blocks from the counter-based generator) and
compare with the library's outputs.
"""

import numpy as np

from dsa_synth import gen

ATT_ABS_TOL = 2e-3     # max-abs over all output elements
ATT_REL_TOL = 1e-2     # max-rel over elements with |oracle| >= REL_FLOOR
REL_FLOOR = 0.2
NEAR_TIE_REL = 1e-6    # allowed index swaps: oracle scores within this relative gap


def to_device(w, device="cuda", kv_layout=0):
    """PagedKV / Queries on the device (pools filled by the device filler).
    kv_layout 1 stores the same pool values head-major, [P, Hkv, bs, 128]."""
    import dynamic_sparse_attention_paged_amd as dsa
    from dsa_synth import device as synth_dev

    t = synth_dev.upload(w, device)
    if kv_layout == dsa.KV_HEAD_MAJOR:
        for name in ("k_cache", "v_cache"):
            t[name] = t[name].permute(0, 2, 1, 3).contiguous()
    kv = dsa.PagedKV(t["k_cache"], t["v_cache"], t["idx_keys"], t["idx_scale"],
                     t["block_table"], t["seq_lens"], kv_layout=kv_layout)
    qs = dsa.Queries(t["q"], t["q_idx"], t["w_idx"], t["q_seq"], t["q_pos"])
    return kv, qs


def oracle_query(w, qi, top_k=None, sel_override=None):
    """Oracle result for query qi of workload w (float64)."""
    from oracle import bf16_bits_to_f64
    from oracle.pipeline import score_query
    from oracle import select_blocks, sparse_attention

    s = int(w.q_seq[qi])
    pos = int(w.q_pos[qi])
    L = int(w.seq_lens[s])
    k = w.top_k if top_k is None else top_k
    qidx = bf16_bits_to_f64(w.q_idx_bits[qi])
    cand, sc, loc = score_query(qidx, w.w[qi], w.block_table[s], pos, L, w.block_size,
                                w.idx_keys, w.idx_scale)
    idx, cnt = select_blocks(cand, sc.astype(np.float32), loc, k)
    sel = idx[:cnt] if sel_override is None else sel_override
    out, lse = sparse_attention(bf16_bits_to_f64(w.q_bits[qi]), sel, w.block_table[s], pos, L,
                                w.block_size, lambda p: bf16_bits_to_f64(w.k_block_bits(p)),
                                lambda p: bf16_bits_to_f64(w.v_block_bits(p)),
                                w.softmax_scale, w.num_kv_heads)
    return dict(cand=cand, scores=sc, idx=idx, cnt=cnt, out=out, lse=lse, local=loc)


def oracle_select(w, qi, top_k=None):
    """Oracle scores and selection (no attention) for query qi of workload w."""
    from oracle import bf16_bits_to_f64, select_blocks
    from oracle.pipeline import score_query

    s = int(w.q_seq[qi])
    pos = int(w.q_pos[qi])
    k = w.top_k if top_k is None else top_k
    cand, sc, loc = score_query(bf16_bits_to_f64(w.q_idx_bits[qi]), w.w[qi], w.block_table[s],
                                pos, int(w.seq_lens[s]), w.block_size, w.idx_keys, w.idx_scale)
    idx, cnt = select_blocks(cand, sc.astype(np.float32), loc, k)
    return dict(cand=cand, scores=sc, idx=idx, cnt=cnt, local=loc)


def check_scores_exact(gpu_row, ref, maxb):
    """GPU fp32 scores equal the oracle's float64 score rounded to fp32; -inf elsewhere."""
    row = np.asarray(gpu_row)
    want = np.full(maxb, -np.inf, dtype=np.float32)
    want[ref["cand"]] = ref["scores"].astype(np.float32)
    bad = np.flatnonzero(row.view(np.uint32) != want.view(np.uint32))
    return bad


def check_indices(gpu_idx, gpu_cnt, ref, top_k):
    """Indices equal the oracle's, or differ only by swaps among blocks whose
    oracle scores are within NEAR_TIE_REL of the oracle's boundary score.
    Returns (ok, n_swapped)."""
    gi = np.asarray(gpu_idx)
    if int(gpu_cnt) != ref["cnt"]:
        return False, -1
    if np.array_equal(gi, ref["idx"]):
        return True, 0
    cnt = ref["cnt"]
    if np.any(gi[cnt:] != -1) or np.any(np.diff(gi[:cnt]) <= 0) or ref["local"] not in gi[:cnt]:
        return False, -1
    a, b = set(gi[:cnt].tolist()), set(ref["idx"][:cnt].tolist())
    diff = a ^ b
    sc = dict(zip(ref["cand"].tolist(), ref["scores"].tolist()))
    if any(j not in sc for j in diff):
        return False, -1
    others = [sc[j] for j in b if j != ref["local"]]
    bound = min(others) if others else 0.0
    for j in diff:
        if abs(sc[j] - bound) > NEAR_TIE_REL * max(abs(bound), 1e-300):
            return False, -1
    return True, len(diff) // 2


def attn_errors(gpu, ref):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    err = np.abs(g - r)
    big = np.abs(r) >= REL_FLOOR
    max_abs = float(err.max()) if err.size else 0.0
    max_rel = float((err[big] / np.abs(r[big])).max()) if big.any() else 0.0
    return max_abs, max_rel


def attn_ok(gpu, ref):
    a, r = attn_errors(gpu, ref)
    return a <= ATT_ABS_TOL and r <= ATT_REL_TOL, a, r
