"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of an oracle function (on the CPU,
patched into every module that holds a reference to it) and checks that at
least one of the pins in tests/test_oracle_*.py then fails.  The pins
themselves pass on the real oracle (the rest of the suite).
"""

import numpy as np
import pytest

import oracle
import oracle.dsa as D
import oracle.fp8 as F
import oracle.moe as M
import oracle.pipeline as P
import oracle.write as W
from tests import test_oracle_attention as TA
from tests import test_oracle_fp8 as TF
from tests import test_oracle_moe as TM
from tests import test_oracle_score as TS
from tests import test_oracle_select as TSEL
from tests import test_oracle_write as TW

_MODULES = (oracle, D, F, M, P, W, TA, TF, TM, TS, TSEL, TW)
_real = {name: getattr(D, name, None) or getattr(F, name, None) or getattr(P, name, None)
         or getattr(W, name)
         for name in ("e4m3_decode", "e4m3_encode", "quantize_q_idx", "index_scores",
                      "select_blocks", "visible_blocks", "_gather_tokens",
                      "attention_partial", "merge_partials", "sparse_attention",
                      "dense_attention", "score_query", "quantize_coarse_key", "kv_write")}
_real.update({name: getattr(M, name) for name in ("e2m1_decode", "unpack_fp4", "mxfp4_dequant",
                                                    "mx_quantize_e4m3", "mx_dequant_e4m3",
                                                    "grouped_gemm_abs")})


def _patch(monkeypatch, name, fn):
    for m in _MODULES:
        if hasattr(m, name):
            monkeypatch.setattr(m, name, fn)


# ---------------------------------------------------------------------------
# mutants: each is the real function with one plausible mistake
# ---------------------------------------------------------------------------
def decode_wrong_bias(codes):
    return _real["e4m3_decode"](codes) * 0.5  # exponent bias 8 instead of 7


def encode_ties_away(x):
    # nearest representable magnitude, ties to the larger one (not to even)
    x = np.asarray(x, dtype=np.float64)
    vals = _real["e4m3_decode"](np.arange(0x7F, dtype=np.uint8))  # +0 .. 448
    a = np.minimum(np.abs(x), 448.0)
    dist = np.abs(a[..., None] - vals)
    best = dist.min(axis=-1, keepdims=True)
    code = (np.where(dist == best, np.arange(0x7F), -1)).max(axis=-1)  # larger on ties
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def q_scale_not_power_of_two(q_idx):
    q = np.asarray(q_idx, dtype=np.float64)
    amax = np.max(np.abs(q), axis=-1)
    scale = np.where(amax == 0.0, 1.0, amax / 448.0)
    return _real["e4m3_encode"](q / scale[..., None]), scale


def scores_without_relu(qc, sq, w, kc, ks, activation="relu"):
    return _real["index_scores"](qc, sq, w, kc, ks, activation="identity")


def scores_relu_after_head_sum(qc, sq, w, kc, ks, activation="relu"):
    s = _real["index_scores"](qc, sq, w, kc, ks, activation="identity")
    return np.where(s > 0.0, s, 0.0)


def scores_ignore_key_scale(qc, sq, w, kc, ks, activation="relu"):
    return _real["index_scores"](qc, sq, w, kc, np.ones_like(np.asarray(ks, np.float64)),
                                 activation=activation)


def select_ties_to_higher_id(cand, scores, local, top_k):
    cand = np.asarray(cand, dtype=np.int64)
    if cand.size <= top_k:
        sel = np.sort(cand)
    else:
        others = [(j, s) for j, s in zip(cand.tolist(), np.asarray(scores).tolist()) if j != local]
        others.sort(key=lambda js: (-js[1], -js[0]))
        sel = np.sort(np.asarray([j for j, _ in others[:top_k - 1]] + [int(local)]))
    out = np.full(top_k, -1, dtype=np.int32)
    out[:sel.size] = sel
    return out, int(sel.size)


def select_local_not_forced(cand, scores, local, top_k):
    cand = np.asarray(cand, dtype=np.int64)
    order = sorted(zip(cand.tolist(), np.asarray(scores).tolist()), key=lambda js: (-js[1], js[0]))
    sel = np.sort(np.asarray([j for j, _ in order[:top_k]], dtype=np.int64))
    out = np.full(top_k, -1, dtype=np.int32)
    out[:sel.size] = sel
    return out, int(sel.size)


def select_in_score_order(cand, scores, local, top_k):
    idx, cnt = _real["select_blocks"](cand, scores, local, top_k)
    pos = {int(j): i for i, j in enumerate(np.asarray(cand).tolist())}
    s = np.asarray(scores)
    head = sorted(idx[:cnt].tolist(), key=lambda j: (-s[pos[j]], j))
    out = idx.copy()
    out[:cnt] = head
    return out, cnt


def visible_off_by_one(pos, seq_len, block_size):
    nb = -(-int(seq_len) // int(block_size))
    j = np.arange(nb, dtype=np.int64)
    return j[j * int(block_size) < int(pos)]  # drops a local block starting at pos


def gather_ignores_causality(block_ids, table_row, pos, seq_len, block_size, k_block, v_block):
    # tokens after the query inside its own block are not masked
    return _real["_gather_tokens"](block_ids, table_row, seq_len - 1, seq_len, block_size, k_block,
                                   v_block)


def partial_wrong_gqa_grouping(q, K, V, softmax_scale, num_kv_heads):
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[0]
    m, l, o = np.empty(hq), np.empty(hq), np.empty_like(q)
    for h in range(hq):
        g = h % num_kv_heads  # interleaved instead of contiguous groups
        x = float(softmax_scale) * (K[:, g, :] @ q[h])
        m[h] = x.max()
        p = np.exp(x - m[h])
        l[h] = p.sum()
        o[h] = (p @ V[:, g, :]) / l[h]
    return m, l, o


def partial_without_scale(q, K, V, softmax_scale, num_kv_heads):
    return _real["attention_partial"](q, K, V, 1.0, num_kv_heads)


def merge_unweighted(parts):
    o = sum(p[2] for p in parts) / len(parts)
    m = np.max(np.stack([p[0] for p in parts]), axis=0)
    return o, m + np.log(sum(p[1] * np.exp(p[0] - m) for p in parts))


def sparse_lse_in_log2(q, block_ids, table_row, pos, seq_len, block_size, k_block, v_block,
                       softmax_scale, num_kv_heads):
    K, V, _ = D._gather_tokens(block_ids, table_row, pos, seq_len, block_size, k_block, v_block)
    m, l, o = D.attention_partial(q, K, V, softmax_scale, num_kv_heads)
    return o, m + np.log2(l)


def dense_not_causal(q, table_row, pos, seq_len, block_size, k_block, v_block, softmax_scale,
                     num_kv_heads):
    return _real["dense_attention"](q, table_row, seq_len - 1, seq_len, block_size, k_block,
                                    v_block, softmax_scale, num_kv_heads)


def score_query_skips_table(q_idx, w, table_row, pos, seq_len, block_size, key_codes, key_scale,
                            activation="relu"):
    ident = np.arange(len(table_row))  # logical id used as the physical one
    return _real["score_query"](q_idx, w, ident, pos, seq_len, block_size, key_codes, key_scale,
                                activation=activation)


def coarse_key_scale_240(x):
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) or np.float32(1.0)
    ks = np.float32(amax / np.float32(240.0))  # the E4M3 range taken as 240
    y = np.clip((x / ks).astype(np.float32), -448.0, 448.0)
    return F.e4m3_encode(y.astype(np.float64)), ks


def coarse_key_power_of_two_scale(x):
    x = np.asarray(x, dtype=np.float32)
    amax = float(np.max(np.abs(x))) or 1.0
    ks = np.float32(2.0 ** np.ceil(np.log2(amax / 448.0)))  # the query's rule instead
    y = np.clip((x / ks).astype(np.float32), -448.0, 448.0)
    return F.e4m3_encode(y.astype(np.float64)), ks


def coarse_key_truncated(x):
    codes, ks = _real["quantize_coarse_key"](x)
    y = np.clip((np.asarray(x, np.float32) / ks).astype(np.float32), -448.0, 448.0)
    v = F.e4m3_decode(codes)
    over = np.abs(v) > np.abs(y)  # round toward zero instead of to nearest
    down = np.where(codes & 0x7F, codes - 1, codes).astype(np.uint8)
    return np.where(over, down, codes).astype(np.uint8), ks


def kv_write_position_off_by_one(k_pool, v_pool, table, seq_lens, tok_seq, tok_pos, k_new,
                                 v_new, block_size):
    pos = None if tok_pos is None else np.maximum(np.asarray(tok_pos) - 1, 0)
    lens = np.asarray(seq_lens) - (1 if tok_pos is None else 0)
    return _real["kv_write"](k_pool, v_pool, table, np.maximum(lens, 1), tok_seq, pos, k_new,
                             v_new, block_size)


def e2m1_exponent_bias_zero(codes):
    c = np.asarray(codes).astype(np.int64)
    v = _real["e2m1_decode"](c)
    return np.where(((c >> 1) & 3) > 0, 2 * v, v)  # normals doubled


def unpack_high_nibble_first(packed, k):
    p = np.asarray(packed).astype(np.uint8)
    return _real["unpack_fp4"](((p & 0x0F) << 4) | (p >> 4), k)


def mxfp4_scale_bias_128(packed, scales):
    return _real["mxfp4_dequant"](packed, scales) * 0.5


def mx_quantize_emax_7(x):
    # shared exponent floor(log2 amax) - 7: block maxima land in [128, 256)
    x = np.asarray(x, dtype=np.float64)
    _, s = _real["mx_quantize_e4m3"](x)
    s2 = np.where(s > 0, s.astype(np.int64) + 1, 0)
    y = x / np.repeat(np.exp2(s2 - 127.0), 32, -1)
    return F.e4m3_encode(np.clip(y, -448.0, 448.0)), s2.astype(np.uint8)


def mx_quantize_ceil_log2(x):
    x = np.asarray(x, dtype=np.float64)
    codes, s = _real["mx_quantize_e4m3"](x)
    blocks = np.abs(x).reshape(x.shape[:-1] + (-1, 32)).max(-1)
    pow2 = (blocks > 0) & (np.frexp(np.where(blocks > 0, blocks, 1.0))[0] == 0.5)
    bump = (blocks > 0) & ~pow2
    c2, _ = _real["mx_quantize_e4m3"](x / np.repeat(np.where(bump, 2.0, 1.0), 32, -1))
    return c2, np.where(bump, s + 1, s).astype(np.uint8)


def mx_dequant_ignores_scale(codes, scales):
    return F.e4m3_decode(codes)


def gemm_abs_ignores_activation_scales(x_codes, x_scales, w_packed, w_scales, route):
    xq = np.abs(F.e4m3_decode(x_codes))
    route = np.asarray(route)
    out = np.zeros(route.shape + (np.asarray(w_scales).shape[1],))
    for e in np.unique(route[route >= 0]):
        w = np.abs(M.mxfp4_dequant(w_packed[e], w_scales[e]))
        tt, jj = np.nonzero(route == e)
        out[tt, jj] = xq[tt] @ w.T
    return out


CASES = [
    ("e4m3_decode", decode_wrong_bias, ["TF.test_spot_codes"]),
    ("e4m3_encode", encode_ties_away, ["TF.test_encode_ties_to_even",
                                       "TF.test_encode_matches_brute_force_all_bf16"]),
    ("quantize_q_idx", q_scale_not_power_of_two, ["TS.test_q_scale_closed_form_and_invariant"]),
    ("index_scores", scores_without_relu, ["TS.test_scores_exact_integer_recomputation"]),
    ("index_scores", scores_relu_after_head_sum, ["TS.test_scores_exact_integer_recomputation"]),
    ("index_scores", scores_ignore_key_scale, ["TS.test_scores_exact_integer_recomputation"]),
    ("select_blocks", select_ties_to_higher_id, ["TSEL.test_select_brute_force_random"]),
    ("select_blocks", select_local_not_forced, ["TSEL.test_select_brute_force_random",
                                                "TSEL.test_hand_examples_select"]),
    ("select_blocks", select_in_score_order, ["TSEL.test_select_brute_force_random"]),
    ("visible_blocks", visible_off_by_one, ["TSEL.test_visible_blocks_are_the_causal_prefix"]),
    ("_gather_tokens", gather_ignores_causality,
     ["TA.test_all_blocks_equals_dense_and_torch", "TA.test_hand_examples_attention"]),
    ("attention_partial", partial_wrong_gqa_grouping, ["TA.test_all_blocks_equals_dense_and_torch"]),
    ("attention_partial", partial_without_scale, ["TA.test_all_blocks_equals_dense_and_torch"]),
    ("merge_partials", merge_unweighted, ["TA.test_merge_identity"]),
    ("sparse_attention", sparse_lse_in_log2, ["TA.test_hand_examples_attention",
                                              "TA.test_all_blocks_equals_dense_and_torch"]),
    ("dense_attention", dense_not_causal, ["TA.test_all_blocks_equals_dense_and_torch"]),
    ("score_query", score_query_skips_table, ["TS.test_scores_use_the_block_table"]),
    ("quantize_coarse_key", coarse_key_scale_240, ["TW.test_hand_examples_coarse_key",
                                                   "TW.test_largest_entry_and_error_bound"]),
    ("quantize_coarse_key", coarse_key_power_of_two_scale, ["TW.test_hand_examples_coarse_key"]),
    ("quantize_coarse_key", coarse_key_truncated, ["TW.test_codes_match_torch_float8_conversion",
                                                   "TW.test_largest_entry_and_error_bound"]),
    ("kv_write", kv_write_position_off_by_one, ["TW.test_kv_write_round_trip"]),
    ("e2m1_decode", e2m1_exponent_bias_zero, ["TM.test_e2m1_matches_the_spec_table"]),
    ("unpack_fp4", unpack_high_nibble_first, ["TM.test_fp4_packing_low_nibble_first",
                                              "TM.test_grouped_gemm_brute_force"]),
    ("mxfp4_dequant", mxfp4_scale_bias_128, ["TM.test_fp8_workspace_is_exact_and_matches_torch_encoder",
                                             "TM.test_grouped_gemm_brute_force"]),
    ("mx_quantize_e4m3", mx_quantize_emax_7, ["TM.test_mxfp8_hand_example",
                                              "TM.test_mxfp8_matches_torch_encoder_and_range"]),
    ("mx_quantize_e4m3", mx_quantize_ceil_log2, ["TM.test_mxfp8_hand_example",
                                                 "TM.test_mxfp8_matches_torch_encoder_and_range"]),
    ("mx_dequant_e4m3", mx_dequant_ignores_scale, ["TM.test_grouped_gemm_brute_force"]),
    ("grouped_gemm_abs", gemm_abs_ignores_activation_scales,
     ["TM.test_grouped_gemm_abs_brute_force"]),
]


@pytest.mark.parametrize("name,mutant,pins", CASES, ids=[c[1].__name__ for c in CASES])
def test_pins_catch_mutant(monkeypatch, golden, name, mutant, pins):
    _patch(monkeypatch, name, mutant)
    mods = {"TA": TA, "TF": TF, "TM": TM, "TS": TS, "TSEL": TSEL, "TW": TW}
    failures = 0
    for pin in pins:
        mod, fn = pin.split(".")
        f = getattr(mods[mod], fn)
        try:
            f(golden) if "golden" in f.__code__.co_varnames[:f.__code__.co_argcount] else f()
        except AssertionError:  # a pin's check failed (not a crash of the mutant)
            failures += 1
    assert failures > 0, f"no pin caught the mutant {mutant.__name__} of {name}"
