"""The C ABI on the host: the library loads, exports every symbol that
include/dsa.h declares, and rejects invalid arguments before touching the
GPU (these calls never reach a kernel launch, so they run without a GPU)."""

import ctypes
import os
import re

import pytest

from dynamic_sparse_attention_paged_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libdsa.so not built: run __graft_entry__.build()")
    return _lib.load()


def _declared(header="dsa.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(_lib.EXPORTS) == set(names)
    assert lib.dsa_abi_version() == 2


def test_every_header_is_exported(lib):
    """Every function declared in any include/*.h is exported by libdsa.so."""
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert "dsa_support.h" in headers
    for h in headers:
        for n in _declared(h):
            assert hasattr(lib, n), f"{h}: {n}"
    assert set(_lib.SUPPORT_EXPORTS) == set(_declared("dsa_support.h"))


def test_support_calls_reject_bad_arguments(lib):
    """The measurement-support calls validate before launching anything."""
    assert lib.dsa_probe_stream_read(None, 1 << 20, 0, FAKE, 8, None) == -1
    assert lib.dsa_probe_stream_read(FAKE + 4, 1 << 20, 0, FAKE, 8, None) == -4
    assert lib.dsa_probe_stream_read(FAKE, (1 << 20) + 8, 0, FAKE, 8, None) == -4
    assert lib.dsa_probe_stream_read(FAKE, 1 << 20, 0, FAKE, 0, None) == -1
    assert lib.dsa_cache_flush(None, 1 << 20, 1, None) == -1
    assert lib.dsa_cache_flush(FAKE, 100, 1, None) == -4
    assert lib.dsa_probe_mfma_rate(7, 10, 8, FAKE, None) == -3
    assert lib.dsa_probe_mfma_rate(0, 0, 8, FAKE, None) == -1
    assert lib.dsa_probe_fp8_mfma(FAKE, FAKE, FAKE, 0, FAKE, None) == -1
    assert lib.dsa_probe_fp8_mfma(FAKE + 8, FAKE, FAKE, 1, FAKE, None) == -4


FAKE = 0x10000  # a 64 KiB-aligned non-NULL address: never dereferenced on the host


def _kv(**over):
    f = dict(k_cache=FAKE, v_cache=FAKE, idx_keys=FAKE, idx_scale=FAKE, block_table=FAKE,
             seq_lens=FAKE, num_blocks=10, block_size=64, num_kv_heads=2, head_dim=128,
             idx_dim=128, num_seqs=2, max_blocks_per_seq=5)
    f.update(over)
    return _lib.PagedKVStruct(**f)


def _qs(**over):
    f = dict(num_queries=2, num_q_heads=8, idx_heads=4, q_seq=None, q_pos=None, q=FAKE,
             q_idx=FAKE, w_idx=FAKE)
    f.update(over)
    return _lib.QueriesStruct(**f)


def _score(lib, kv, qs, scores=FAKE):
    return lib.dsa_index_score(ctypes.byref(kv), ctypes.byref(qs), scores, None)


def _attn(lib, kv, qs, top_k=4, ws=FAKE, ws_bytes=1 << 30, out=FAKE):
    return lib.dsa_sparse_attn_decode(ctypes.byref(kv), ctypes.byref(qs), FAKE, FAKE, top_k,
                                      0.1, out, None, ws, ws_bytes, None)


def test_validation_errors(lib):
    E = {v: k for k, v in _lib.STATUS.items()}
    assert lib.dsa_index_score(None, None, FAKE, None) == E["DSA_ERR_NULL"]
    assert "NULL" in lib.dsa_last_error().decode()
    for bs in (32, 96, 1024):
        assert _score(lib, _kv(block_size=bs), _qs()) == E["DSA_ERR_UNSUPPORTED"]
    # positions past 2^31 - 1
    assert _score(lib, _kv(block_size=512, max_blocks_per_seq=1 << 22), _qs()) == \
        E["DSA_ERR_UNSUPPORTED"]
    assert _score(lib, _kv(head_dim=64), _qs()) == E["DSA_ERR_UNSUPPORTED"]
    assert _score(lib, _kv(idx_dim=96), _qs()) == E["DSA_ERR_UNSUPPORTED"]
    assert _score(lib, _kv(), _qs(idx_heads=17)) == E["DSA_ERR_UNSUPPORTED"]
    assert _score(lib, _kv(idx_keys=None), _qs()) == E["DSA_ERR_NULL"]
    assert _score(lib, _kv(idx_keys=FAKE + 8), _qs()) == E["DSA_ERR_ALIGN"]
    assert _score(lib, _kv(), _qs(), scores=None) == E["DSA_ERR_NULL"]
    assert _score(lib, _kv(), _qs(num_queries=3)) == E["DSA_ERR_SHAPE"]  # decode: Nq > seqs
    assert _score(lib, _kv(num_blocks=0), _qs()) == E["DSA_ERR_SHAPE"]
    assert _score(lib, _kv(), _qs(num_queries=65536)) == E["DSA_ERR_UNSUPPORTED"]  # grid rows
    assert _attn(lib, _kv(), _qs(num_q_heads=7)) == E["DSA_ERR_SHAPE"]  # Hq % Hkv
    assert _attn(lib, _kv(num_kv_heads=1), _qs(num_q_heads=32)) == E["DSA_ERR_UNSUPPORTED"]
    assert _attn(lib, _kv(), _qs(), top_k=0) == E["DSA_ERR_SHAPE"]
    assert _attn(lib, _kv(), _qs(), top_k=5000) == E["DSA_ERR_SHAPE"]
    assert _attn(lib, _kv(k_cache=FAKE + 2), _qs()) == E["DSA_ERR_ALIGN"]
    for layout in (-1, 2):  # only token-major (0) and head-major (1) blocks
        assert _attn(lib, _kv(kv_layout=layout), _qs()) == E["DSA_ERR_UNSUPPORTED"]
        assert _score(lib, _kv(kv_layout=layout), _qs()) == E["DSA_ERR_UNSUPPORTED"]
    assert _attn(lib, _kv(), _qs(), out=None) == E["DSA_ERR_NULL"]
    assert lib.dsa_sparse_attn_prefill(ctypes.byref(_kv()), ctypes.byref(_qs()), FAKE, FAKE, 4,
                                       0.1, FAKE, None, None) == E["DSA_ERR_NULL"]  # q_seq/q_pos


def test_check_inputs_validation(lib):
    E = {v: k for k, v in _lib.STATUS.items()}

    def chk(kv, qs, bi=None, bc=None, top_k=0, flags=FAKE):
        return lib.dsa_check_inputs(ctypes.byref(kv) if kv is not None else None,
                                    ctypes.byref(qs), bi, bc, top_k, flags, None)
    assert chk(None, _qs()) == E["DSA_ERR_NULL"]
    assert chk(_kv(), _qs(), flags=None) == E["DSA_ERR_NULL"]
    assert chk(_kv(), _qs(), flags=FAKE + 2) == E["DSA_ERR_ALIGN"]
    assert chk(_kv(block_table=None), _qs()) == E["DSA_ERR_NULL"]
    assert chk(_kv(num_seqs=0), _qs()) == E["DSA_ERR_SHAPE"]
    assert chk(_kv(block_size=32), _qs()) == E["DSA_ERR_UNSUPPORTED"]
    assert chk(_kv(), _qs(num_queries=3)) == E["DSA_ERR_SHAPE"]  # decode: Nq > seqs
    assert chk(_kv(), _qs(), bi=FAKE) == E["DSA_ERR_NULL"]       # block_idx without block_cnt
    assert chk(_kv(), _qs(), bi=FAKE, bc=FAKE, top_k=0) == E["DSA_ERR_SHAPE"]
    assert chk(_kv(), _qs(), bi=FAKE + 1, bc=FAKE, top_k=4) == E["DSA_ERR_ALIGN"]


def test_write_path_validation(lib):
    E = {v: k for k, v in _lib.STATUS.items()}

    def kvw(kv, n=2, ts=None, tp=None, kn=FAKE, vn=FAKE):
        return lib.dsa_kv_write(ctypes.byref(kv) if kv is not None else None, n, ts, tp, kn, vn,
                                None)
    assert kvw(None) == E["DSA_ERR_NULL"]
    assert kvw(_kv(), n=-1) == E["DSA_ERR_SHAPE"]
    assert kvw(_kv(k_cache=None)) == E["DSA_ERR_NULL"]
    assert kvw(_kv(), kn=None) == E["DSA_ERR_NULL"]
    assert kvw(_kv(), kn=FAKE + 4) == E["DSA_ERR_ALIGN"]
    assert kvw(_kv(head_dim=64)) == E["DSA_ERR_UNSUPPORTED"]
    assert kvw(_kv(), n=3) == E["DSA_ERR_SHAPE"]  # tok_seq NULL: n <= num_seqs
    assert kvw(_kv(), n=0) == 0                    # nothing to do, nothing launched

    def ikw(kv, n=2, ids=FAKE, x=FAKE):
        return lib.dsa_index_key_write(ctypes.byref(kv) if kv is not None else None, n, ids, x,
                                       None)
    assert ikw(None) == E["DSA_ERR_NULL"]
    assert ikw(_kv(), n=-1) == E["DSA_ERR_SHAPE"]
    assert ikw(_kv(idx_dim=96)) == E["DSA_ERR_UNSUPPORTED"]
    assert ikw(_kv(idx_keys=None)) == E["DSA_ERR_NULL"]
    assert ikw(_kv(), ids=None) == E["DSA_ERR_NULL"]
    assert ikw(_kv(), x=FAKE + 2) == E["DSA_ERR_ALIGN"]
    assert ikw(_kv(), n=0) == 0


def test_decode_topk_contract(lib):
    """Decode attention that selects from given scores: its own checks."""
    E = {v: k for k, v in _lib.STATUS.items()}
    kv, qs = _kv(), _qs()

    def call(kv=kv, sc=FAKE, top_k=4, out=FAKE, lse=None, bi=None, bc=None, ws=FAKE, n=1 << 20):
        return lib.dsa_sparse_attn_decode_topk(ctypes.byref(kv), ctypes.byref(qs), sc, top_k, 0.1,
                                               out, lse, bi, bc, ws, n, None)
    assert call(sc=None) == E["DSA_ERR_NULL"]
    assert call(out=None) == E["DSA_ERR_NULL"]
    assert call(sc=FAKE + 2) == E["DSA_ERR_ALIGN"]
    assert call(bc=FAKE + 2) == E["DSA_ERR_ALIGN"]
    assert call(top_k=0) == E["DSA_ERR_SHAPE"]
    # the selection inside attention covers at most 2048 blocks and top_k <= 2048
    assert call(top_k=2049) == E["DSA_ERR_UNSUPPORTED"]
    assert call(kv=_kv(max_blocks_per_seq=2049, num_blocks=4100)) == E["DSA_ERR_UNSUPPORTED"]
    # the split partials' workspace is checked like dsa_sparse_attn_decode's
    n = ctypes.c_size_t(0)
    assert lib.dsa_workspace_size(_lib.OP_ATTN_DECODE, ctypes.byref(kv), ctypes.byref(qs), 4,
                                  ctypes.byref(n)) == 0
    if n.value > 0:
        assert call(ws=None) == E["DSA_ERR_WORKSPACE"]
        assert call(n=n.value - 1) == E["DSA_ERR_WORKSPACE"]


def test_workspace_contract(lib):
    E = {v: k for k, v in _lib.STATUS.items()}
    kv, qs = _kv(), _qs()
    n = ctypes.c_size_t(0)
    assert lib.dsa_workspace_size(_lib.OP_DECODE_FUSED, ctypes.byref(kv), ctypes.byref(qs), 4,
                                  ctypes.byref(n)) == 0
    assert n.value > 0
    st = lib.dsa_sparse_decode_fused(ctypes.byref(kv), ctypes.byref(qs), 4, 0.1, FAKE, None, None,
                                     None, FAKE, n.value - 1, None)
    assert st == E["DSA_ERR_WORKSPACE"]
    st = lib.dsa_sparse_decode_fused(ctypes.byref(kv), ctypes.byref(qs), 4, 0.1, FAKE, None, None,
                                     None, FAKE + 64, n.value, None)
    assert st == E["DSA_ERR_ALIGN"]
    m = ctypes.c_size_t(0)
    assert lib.dsa_workspace_size(_lib.OP_INDEX_TOPK, ctypes.byref(kv), ctypes.byref(qs), 4,
                                  ctypes.byref(m)) == 0
    assert m.value >= 2 * 5 * 4
    assert lib.dsa_workspace_size(99, ctypes.byref(kv), ctypes.byref(qs), 4,
                                  ctypes.byref(m)) == E["DSA_ERR_SHAPE"]


def test_prefill_fused_contract(lib):
    E = {v: k for k, v in _lib.STATUS.items()}
    kv, qs = _kv(), _qs(q_seq=FAKE, q_pos=FAKE)
    n = ctypes.c_size_t(0)
    assert lib.dsa_workspace_size(_lib.OP_PREFILL_FUSED, ctypes.byref(kv), ctypes.byref(qs), 4,
                                  ctypes.byref(n)) == 0
    # at least one partial state {o[128], m, l} per (query, pick, head)
    assert n.value >= qs.num_queries * 4 * qs.num_q_heads * 130 * 4

    def call(kv=kv, qs=qs, top_k=4, out=FAKE, ws=FAKE, nbytes=n.value, bi=None, bc=None):
        return lib.dsa_sparse_prefill_fused(ctypes.byref(kv), ctypes.byref(qs), top_k, 0.1, out,
                                            None, bi, bc, ws, nbytes, None)
    assert call(nbytes=n.value - 1) == E["DSA_ERR_WORKSPACE"]
    assert call(ws=FAKE + 64) == E["DSA_ERR_ALIGN"]
    assert call(out=FAKE + 4) == E["DSA_ERR_ALIGN"]
    assert call(out=None) == E["DSA_ERR_NULL"]
    assert call(bi=FAKE) == E["DSA_ERR_NULL"]          # block_idx_out without block_cnt_out
    assert call(qs=_qs(q_seq=None, q_pos=FAKE)) == E["DSA_ERR_NULL"]
    assert call(top_k=0) == E["DSA_ERR_SHAPE"]
    assert call(kv=_kv(block_size=96)) == E["DSA_ERR_UNSUPPORTED"]
    assert call(qs=_qs(q_seq=FAKE, q_pos=FAKE, num_queries=0)) == 0



def test_empty_batch_is_a_noop(lib):
    # Nq == 0 returns DSA_OK without launching anything (no GPU needed)
    assert _score(lib, _kv(), _qs(num_queries=0)) == 0
    assert _attn(lib, _kv(), _qs(num_queries=0)) == 0
    assert lib.dsa_last_error().decode() == ""


def test_status_strings(lib):
    for s in _lib.STATUS:
        assert lib.dsa_status_str(s)


def _mx(**over):
    f = dict(w_fp4=FAKE, w_scale=FAKE, num_experts=4, n=64, k=256)
    f.update(over)
    return _lib.MxExpertsStruct(**f)


def test_moe_validation(lib):
    E = {v: k for k, v in _lib.STATUS.items()}
    n = ctypes.c_size_t(0)
    w = _mx()
    for mode in (_lib.MOE_FP8_WORKSPACE, _lib.MOE_FP4_DIRECT):
        assert lib.dsa_moe_workspace_size(ctypes.byref(w), 8, 2, mode, ctypes.byref(n)) == 0
    # the FP8 workspace holds min(experts, pairs) unpacked experts
    fp8 = ctypes.c_size_t(0)
    lib.dsa_moe_workspace_size(ctypes.byref(w), 8, 2, _lib.MOE_FP8_WORKSPACE, ctypes.byref(fp8))
    assert fp8.value >= 4 * 64 * 256 + 4 * 64 * 8
    assert lib.dsa_moe_workspace_size(ctypes.byref(_mx(k=200)), 8, 2, 1, ctypes.byref(n)) == \
        E["DSA_ERR_UNSUPPORTED"]
    assert lib.dsa_moe_workspace_size(ctypes.byref(_mx(n=0)), 8, 2, 1, ctypes.byref(n)) == \
        E["DSA_ERR_SHAPE"]
    assert lib.dsa_moe_workspace_size(ctypes.byref(_mx(w_fp4=None)), 8, 2, 1, ctypes.byref(n)) == \
        E["DSA_ERR_NULL"]
    assert lib.dsa_moe_workspace_size(ctypes.byref(_mx(w_fp4=FAKE + 8)), 8, 2, 1,
                                      ctypes.byref(n)) == E["DSA_ERR_ALIGN"]
    assert lib.dsa_moe_workspace_size(ctypes.byref(w), 8, 2, 7, ctypes.byref(n)) == E["DSA_ERR_SHAPE"]
    # size limits: more than 2^30 pairs; a launch of 2^24 or more (row tile,
    # column block) work items (2^24 pairs in 128-pair tiles x 512 column blocks)
    assert lib.dsa_moe_workspace_size(ctypes.byref(w), (1 << 29) + 1, 2, 1, ctypes.byref(n)) == \
        E["DSA_ERR_UNSUPPORTED"]
    wide = _mx(n=65536, k=128)
    assert lib.dsa_moe_workspace_size(ctypes.byref(wide), 1 << 20, 16, 1, ctypes.byref(n)) == \
        E["DSA_ERR_UNSUPPORTED"]
    assert lib.dsa_moe_workspace_size(ctypes.byref(wide), 1 << 10, 16, 1, ctypes.byref(n)) == 0
    lib.dsa_moe_workspace_size(ctypes.byref(w), 8, 2, 1, ctypes.byref(n))

    def gemm(ws=FAKE, nbytes=n.value, out=FAKE, route=FAKE, tokens=8, mode=1):
        return lib.dsa_moe_grouped_gemm(ctypes.byref(w), FAKE, FAKE, tokens, route, 2, mode, out,
                                        ws, nbytes, None)
    assert gemm(nbytes=n.value - 1) == E["DSA_ERR_WORKSPACE"]
    assert lib.dsa_moe_grouped_gemm(ctypes.byref(w), FAKE, FAKE + 1, 8, FAKE, 2, 1, FAKE, FAKE,
                                    n.value, None) == E["DSA_ERR_ALIGN"]   # x_scales 4 B
    assert gemm(ws=FAKE + 64) == E["DSA_ERR_ALIGN"]
    assert gemm(out=None) == E["DSA_ERR_NULL"]
    assert gemm(tokens=0) == 0
    assert lib.dsa_mx_quantize(FAKE, 4, 48, FAKE, FAKE, None) == E["DSA_ERR_UNSUPPORTED"]
    assert lib.dsa_mx_quantize(FAKE + 8, 4, 64, FAKE, FAKE, None) == E["DSA_ERR_ALIGN"]
    assert lib.dsa_mx_quantize(None, 0, 64, None, None, None) == 0
    assert lib.dsa_mxfp4_to_fp8(ctypes.byref(w), None, 2, FAKE, FAKE, None) == E["DSA_ERR_NULL"]
    assert lib.dsa_mxfp4_to_fp8(ctypes.byref(w), FAKE, 0, None, None, None) == 0



def test_noalloc_rejects_oversized_scratch(lib):
    """The fused decode without a workspace refuses, before touching the GPU, a
    call whose scratch would exceed the library's per-GPU array."""
    kv = _kv(num_seqs=4096, max_blocks_per_seq=8192)
    qs = _qs(num_queries=4096, num_q_heads=16, idx_heads=8)
    rc = lib.dsa_sparse_decode_fused_noalloc(ctypes.byref(kv), ctypes.byref(qs), 8, 0.1, FAKE,
                                             FAKE, None, None, None)
    assert rc == -3
    assert b"scratch" in lib.dsa_last_error()
    assert _lib.NOALLOC_SCRATCH_BYTES == 16 * 1024 * 1024


def test_wave_clock_build_is_separate(lib):
    """The per-wave clock reader exists only in the diagnostic library
    (libdsa_clocks.so), which exports the same entry points besides it; the
    reader rejects a null buffer or a count outside 1..65536 on the host."""
    assert not hasattr(lib, "dsa_wave_clocks_read")
    path = os.path.join(_lib.HERE, "libdsa_clocks.so")
    if not os.path.exists(path):
        pytest.fail("libdsa_clocks.so not built: run __graft_entry__.build()")
    clk = ctypes.CDLL(path)
    for n in _declared():
        assert hasattr(clk, n), n
    read = clk.dsa_wave_clocks_read
    read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    read.restype = ctypes.c_int
    buf = (ctypes.c_ulonglong * 2)()
    where = (ctypes.c_uint * 2)()
    assert read(None, ctypes.addressof(where), 1) == -1
    assert read(ctypes.addressof(buf), None, 1) == -1
    assert read(ctypes.addressof(buf), ctypes.addressof(where), 0) == -1
    assert read(ctypes.addressof(buf), ctypes.addressof(where), (1 << 16) + 1) == -1
    assert clk.dsa_wave_clock_khz(None) == -1
    assert not hasattr(lib, "dsa_wave_clock_khz")
