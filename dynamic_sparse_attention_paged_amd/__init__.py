"""MI355X (gfx950) dynamic sparse attention over a paged KV cache.

A thin Python binding over libdsa.so (C ABI in include/dsa.h): argument
marshalling only.  Every step of the method runs in the library's HIP
kernels; PyTorch provides device memory and the current stream.  There is no
CPU or PyTorch fallback: if libdsa.so is missing the calls raise.

    kv = PagedKV(k_cache, v_cache, idx_keys, idx_scale, block_table, seq_lens)
    qs = Queries(q, q_idx, w_idx, q_seq=None, q_pos=None)
    out, lse = decode_fused(kv, qs, top_k, softmax_scale)
"""

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib

__all__ = ["PagedKV", "Queries", "DSAError", "index_score", "topk_blocks",
           "sparse_attn_decode", "sparse_attn_decode_topk", "sparse_attn_prefill", "decode_fused",
           "decode_fused_noalloc",
           "index_topk",
           "workspace_size", "make_workspace", "KV_TOKEN_MAJOR", "KV_HEAD_MAJOR", "abi_version", "check_inputs",
           "kv_write", "index_key_write"]


class DSAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_lib.STATUS.get(status, status)}: {message}")
        self.status = status


KV_TOKEN_MAJOR = 0  # [P, bs, Hkv, 128]: the pages' [block][token][head][dim]
KV_HEAD_MAJOR = 1   # [P, Hkv, bs, 128]: one contiguous run per (block, head)


@dataclass
class PagedKV:
    k_cache: torch.Tensor      # bf16 [P, bs, Hkv, 128] (token-major) or [P, Hkv, bs, 128] (head-major)
    v_cache: torch.Tensor      # bf16, same shape and layout as k_cache
    idx_keys: torch.Tensor     # uint8 (E4M3 codes) [P, dI]
    idx_scale: torch.Tensor    # f32 [P]
    block_table: torch.Tensor  # int32 [B, max_blocks]
    seq_lens: torch.Tensor     # int32 [B]
    block_size: Optional[int] = None  # tokens per block when k_cache is None (default 64)
    kv_layout: int = KV_TOKEN_MAJOR   # KV_TOKEN_MAJOR or KV_HEAD_MAJOR (order inside a block)

    @property
    def tokens_per_block(self):
        if self.k_cache is None:
            return 64 if self.block_size is None else int(self.block_size)
        bs = int(self.k_cache.shape[2 if self.kv_layout == KV_HEAD_MAJOR else 1])
        if self.block_size is not None and int(self.block_size) != bs:
            raise ValueError(f"block_size {self.block_size} != the cache's {bs} tokens per block")
        return bs

    @property
    def kv_heads(self):
        if self.k_cache is None:
            return 1
        return int(self.k_cache.shape[1 if self.kv_layout == KV_HEAD_MAJOR else 2])

    def struct(self):
        def ptr(t):
            return t.data_ptr() if t is not None else None
        k = self.k_cache
        P, d = (k.shape[0], k.shape[3]) if k is not None else (self.idx_keys.shape[0], 128)
        return _lib.PagedKVStruct(
            ptr(self.k_cache), ptr(self.v_cache), ptr(self.idx_keys), ptr(self.idx_scale),
            ptr(self.block_table), ptr(self.seq_lens), P, self.tokens_per_block, self.kv_heads, d,
            self.idx_keys.shape[1] if self.idx_keys is not None else 0,
            self.block_table.shape[0], self.block_table.shape[1], int(self.kv_layout))


@dataclass
class Queries:
    q: Optional[torch.Tensor]        # bf16 [Nq, Hq, 128]
    q_idx: Optional[torch.Tensor]    # bf16 [Nq, HI, dI]
    w_idx: Optional[torch.Tensor]    # f32 [Nq, HI]
    q_seq: Optional[torch.Tensor] = None  # int32 [Nq]
    q_pos: Optional[torch.Tensor] = None  # int32 [Nq]

    @property
    def num_queries(self):
        for t in (self.q, self.q_idx, self.q_pos, self.q_seq):
            if t is not None:
                return t.shape[0]
        raise ValueError("Queries needs q, q_idx, q_pos or q_seq to know its size")

    def struct(self):
        def ptr(t):
            return t.data_ptr() if t is not None else None
        hq = self.q.shape[1] if self.q is not None else 0
        hi = self.q_idx.shape[1] if self.q_idx is not None else 0
        return _lib.QueriesStruct(self.num_queries, hq, hi, ptr(self.q_seq), ptr(self.q_pos),
                                  ptr(self.q), ptr(self.q_idx), ptr(self.w_idx))


def _check_tensors(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous CUDA (HIP) tensors")


def _check(status):
    if status != 0:
        lib = _lib.load()
        raise DSAError(status, lib.dsa_last_error().decode())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _kv_tensors(kv):
    return (kv.k_cache, kv.v_cache, kv.idx_keys, kv.idx_scale, kv.block_table, kv.seq_lens)


def _q_tensors(qs):
    return (qs.q, qs.q_idx, qs.w_idx, qs.q_seq, qs.q_pos)


def abi_version():
    return _lib.load().dsa_abi_version()


def workspace_size(op, kv, qs, top_k):
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    kvs, qss = kv.struct(), qs.struct()
    _check(lib.dsa_workspace_size(op, ctypes.byref(kvs), ctypes.byref(qss), top_k,
                                  ctypes.byref(n)))
    return n.value


def _workspace(nbytes, device):
    # (the library needs no particular contents; zero-filled for reproducibility)
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def make_workspace(op, kv, qs, top_k):
    """A workspace for ``op``, reusable by later calls (of any sizes it covers)."""
    return _workspace(workspace_size(op, kv, qs, top_k), kv.block_table.device)


def index_score(kv, qs, scores=None):
    """fp32 [Nq, max_blocks] block scores (-inf where not visible)."""
    lib = _lib.load()
    _check_tensors(*_kv_tensors(kv), *_q_tensors(qs))
    dev = kv.idx_keys.device
    if scores is None:
        scores = torch.empty(qs.num_queries, kv.block_table.shape[1], dtype=torch.float32,
                             device=dev)
    kvs, qss = kv.struct(), qs.struct()
    _check(lib.dsa_index_score(ctypes.byref(kvs), ctypes.byref(qss), scores.data_ptr(),
                               _stream(dev)))
    return scores


def topk_blocks(scores, kv, qs, top_k, block_idx=None, block_cnt=None):
    """(int32 [Nq, top_k] ascending logical ids, -1 padded; int32 [Nq] counts)."""
    lib = _lib.load()
    _check_tensors(scores, *_kv_tensors(kv), *_q_tensors(qs))
    dev = scores.device
    nq = qs.num_queries
    if block_idx is None:
        block_idx = torch.empty(nq, top_k, dtype=torch.int32, device=dev)
    if block_cnt is None:
        block_cnt = torch.empty(nq, dtype=torch.int32, device=dev)
    kvs, qss = kv.struct(), qs.struct()
    _check(lib.dsa_topk_blocks(scores.data_ptr(), ctypes.byref(kvs), ctypes.byref(qss), top_k,
                               block_idx.data_ptr(), block_cnt.data_ptr(), _stream(dev)))
    return block_idx, block_cnt


def sparse_attn_decode(kv, qs, block_idx, block_cnt, top_k, softmax_scale, out=None,
                       lse=None, workspace=None):
    lib = _lib.load()
    _check_tensors(block_idx, block_cnt, *_kv_tensors(kv), *_q_tensors(qs))
    dev = kv.k_cache.device
    nq, hq = qs.q.shape[0], qs.q.shape[1]
    if out is None:
        out = torch.empty(nq, hq, 128, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(nq, hq, dtype=torch.float32, device=dev)
    need = workspace_size(_lib.OP_ATTN_DECODE, kv, qs, top_k)
    if workspace is None:
        workspace = _workspace(need, dev)
    kvs, qss = kv.struct(), qs.struct()
    _check(lib.dsa_sparse_attn_decode(ctypes.byref(kvs), ctypes.byref(qss), block_idx.data_ptr(),
                                      block_cnt.data_ptr(), top_k, float(softmax_scale),
                                      out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                                      workspace.numel(), _stream(dev)))
    return out, lse


def sparse_attn_decode_topk(kv, qs, scores, top_k, softmax_scale, out=None, lse=None,
                            block_idx=None, block_cnt=None, workspace=None):
    """Decode attention that selects each query's blocks from its indexer scores
    (as index_score writes them) itself.  Returns (out, lse, block_idx, block_cnt);
    block_idx / block_cnt are None unless tensors are passed in to receive them."""
    lib = _lib.load()
    _check_tensors(scores, block_idx, block_cnt, *_kv_tensors(kv), *_q_tensors(qs))
    dev = kv.k_cache.device
    nq, hq = qs.q.shape[0], qs.q.shape[1]
    if out is None:
        out = torch.empty(nq, hq, 128, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(nq, hq, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _workspace(workspace_size(_lib.OP_ATTN_DECODE, kv, qs, top_k), dev)
    kvs, qss = kv.struct(), qs.struct()
    _check(lib.dsa_sparse_attn_decode_topk(
        ctypes.byref(kvs), ctypes.byref(qss), scores.data_ptr(), top_k, float(softmax_scale),
        out.data_ptr(), lse.data_ptr(), block_idx.data_ptr() if block_idx is not None else None,
        block_cnt.data_ptr() if block_cnt is not None else None, workspace.data_ptr(),
        workspace.numel(), _stream(dev)))
    return out, lse, block_idx, block_cnt


def sparse_attn_prefill(kv, qs, block_idx, block_cnt, top_k, softmax_scale, out=None, lse=None):
    lib = _lib.load()
    _check_tensors(block_idx, block_cnt, *_kv_tensors(kv), *_q_tensors(qs))
    dev = kv.k_cache.device
    nq, hq = qs.q.shape[0], qs.q.shape[1]
    if out is None:
        out = torch.empty(nq, hq, 128, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(nq, hq, dtype=torch.float32, device=dev)
    kvs, qss = kv.struct(), qs.struct()
    _check(lib.dsa_sparse_attn_prefill(ctypes.byref(kvs), ctypes.byref(qss),
                                       block_idx.data_ptr(), block_cnt.data_ptr(), top_k,
                                       float(softmax_scale), out.data_ptr(), lse.data_ptr(),
                                       _stream(dev)))
    return out, lse


def decode_fused(kv, qs, top_k, softmax_scale, out=None, lse=None, block_idx=None,
                 block_cnt=None, workspace=None):
    """Scoring, selection and attention in one call.  Returns (out, lse, block_idx, block_cnt);
    block_idx / block_cnt are None unless tensors are passed in to receive them."""
    lib = _lib.load()
    _check_tensors(block_idx, block_cnt, *_kv_tensors(kv), *_q_tensors(qs))
    dev = kv.k_cache.device
    nq, hq = qs.q.shape[0], qs.q.shape[1]
    if out is None:
        out = torch.empty(nq, hq, 128, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(nq, hq, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _workspace(workspace_size(_lib.OP_DECODE_FUSED, kv, qs, top_k), dev)
    kvs, qss = kv.struct(), qs.struct()
    _check(lib.dsa_sparse_decode_fused(
        ctypes.byref(kvs), ctypes.byref(qss), top_k, float(softmax_scale), out.data_ptr(),
        lse.data_ptr(), block_idx.data_ptr() if block_idx is not None else None,
        block_cnt.data_ptr() if block_cnt is not None else None, workspace.data_ptr(),
        workspace.numel(), _stream(dev)))
    return out, lse, block_idx, block_cnt


def decode_fused_noalloc(kv, qs, top_k, softmax_scale, out=None, lse=None, block_idx=None,
                         block_cnt=None):
    """decode_fused without a workspace: the library's own per-GPU scratch
    (dsa_sparse_decode_fused_noalloc; calls on one GPU must not overlap).
    Returns (out, lse, block_idx, block_cnt) as decode_fused does."""
    lib = _lib.load()
    _check_tensors(block_idx, block_cnt, *_kv_tensors(kv), *_q_tensors(qs))
    dev = kv.k_cache.device
    nq, hq = qs.q.shape[0], qs.q.shape[1]
    if out is None:
        out = torch.empty(nq, hq, 128, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(nq, hq, dtype=torch.float32, device=dev)
    kvs, qss = kv.struct(), qs.struct()
    _check(lib.dsa_sparse_decode_fused_noalloc(
        ctypes.byref(kvs), ctypes.byref(qss), top_k, float(softmax_scale), out.data_ptr(),
        lse.data_ptr(), block_idx.data_ptr() if block_idx is not None else None,
        block_cnt.data_ptr() if block_cnt is not None else None, _stream(dev)))
    return out, lse, block_idx, block_cnt


def prefill_fused(kv, qs, top_k, softmax_scale, out=None, lse=None, block_idx=None,
                  block_cnt=None, workspace=None):
    """Chunked prefill in one call: scoring, selection and the block-inverted
    attention (each K/V tile read once for all the queries that picked it).
    q_seq and q_pos are required.  Returns (out, lse, block_idx, block_cnt);
    block_idx / block_cnt are None unless tensors are passed in to receive them.
    The workspace holds one partial state per (query, pick, head): see
    workspace_size(OP_PREFILL_FUSED, ...)."""
    lib = _lib.load()
    _check_tensors(block_idx, block_cnt, *_kv_tensors(kv), *_q_tensors(qs))
    dev = kv.k_cache.device
    nq, hq = qs.q.shape[0], qs.q.shape[1]
    if out is None:
        out = torch.empty(nq, hq, 128, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(nq, hq, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _workspace(workspace_size(_lib.OP_PREFILL_FUSED, kv, qs, top_k), dev)
    kvs, qss = kv.struct(), qs.struct()
    _check(lib.dsa_sparse_prefill_fused(
        ctypes.byref(kvs), ctypes.byref(qss), top_k, float(softmax_scale), out.data_ptr(),
        lse.data_ptr(), block_idx.data_ptr() if block_idx is not None else None,
        block_cnt.data_ptr() if block_cnt is not None else None, workspace.data_ptr(),
        workspace.numel(), _stream(dev)))
    return out, lse, block_idx, block_cnt


def index_topk(kv, qs, top_k, block_idx=None, block_cnt=None, workspace=None):
    lib = _lib.load()
    _check_tensors(block_idx, block_cnt, *_kv_tensors(kv), *_q_tensors(qs))
    dev = kv.idx_keys.device
    nq = qs.num_queries
    if block_idx is None:
        block_idx = torch.empty(nq, top_k, dtype=torch.int32, device=dev)
    if block_cnt is None:
        block_cnt = torch.empty(nq, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = _workspace(workspace_size(_lib.OP_INDEX_TOPK, kv, qs, top_k), dev)
    kvs, qss = kv.struct(), qs.struct()
    _check(lib.dsa_index_topk(ctypes.byref(kvs), ctypes.byref(qss), top_k, block_idx.data_ptr(),
                              block_cnt.data_ptr(), workspace.data_ptr(), workspace.numel(),
                              _stream(dev)))
    return block_idx, block_cnt


def check_inputs(kv, qs, block_idx=None, block_cnt=None, top_k=0):
    """Check the device-side contract (tables, lengths, positions and, when
    given, a selection).  Returns the sorted names of the violated rules
    (empty if none); waits for the check to finish."""
    lib = _lib.load()
    _check_tensors(kv.block_table, kv.seq_lens, qs.q_seq, qs.q_pos, block_idx, block_cnt)
    dev = kv.block_table.device
    flags = torch.empty(1, dtype=torch.int32, device=dev)
    kvs, qss = _check_struct(kv), qs.struct()
    _check(lib.dsa_check_inputs(ctypes.byref(kvs), ctypes.byref(qss),
                                block_idx.data_ptr() if block_idx is not None else None,
                                block_cnt.data_ptr() if block_cnt is not None else None,
                                int(top_k), flags.data_ptr(), _stream(dev)))
    f = int(flags.item()) & 0xFFFFFFFF
    return sorted(name for bit, name in _lib.CHECK_FLAGS.items() if f & bit)


def _check_struct(kv):
    """PagedKV struct for the check: only the table, lengths and pool size matter."""
    num_blocks = (kv.k_cache.shape[0] if kv.k_cache is not None else
                  kv.idx_keys.shape[0] if kv.idx_keys is not None else 1)
    return _lib.PagedKVStruct(None, None, None, None, kv.block_table.data_ptr(),
                              kv.seq_lens.data_ptr(), num_blocks, kv.tokens_per_block, 1, 128, 64,
                              kv.block_table.shape[0], kv.block_table.shape[1], 0)


def kv_write(kv, k_new, v_new, tok_seq=None, tok_pos=None):
    """Write tokens' K/V rows (bf16 [n, Hkv, 128]) into kv.k_cache / kv.v_cache
    through the block table: token i goes to sequence tok_seq[i] (default i)
    at position tok_pos[i] (default seq_lens[s] - 1)."""
    lib = _lib.load()
    _check_tensors(kv.k_cache, kv.v_cache, kv.block_table, kv.seq_lens, k_new, v_new, tok_seq,
                   tok_pos)
    kvs = kv.struct()
    ptr = (lambda t: t.data_ptr() if t is not None else None)
    _check(lib.dsa_kv_write(ctypes.byref(kvs), int(k_new.shape[0]), ptr(tok_seq), ptr(tok_pos),
                            k_new.data_ptr(), v_new.data_ptr(), _stream(kv.k_cache.device)))


def index_key_write(kv, block_ids, coarse):
    """Store coarse keys (fp32 [n, idx_dim]) of physical blocks block_ids
    (int32 [n]) as E4M3 codes with scale max|x| / 448 into kv.idx_keys /
    kv.idx_scale."""
    lib = _lib.load()
    _check_tensors(kv.idx_keys, kv.idx_scale, block_ids, coarse)
    kvs = kv.struct()
    _check(lib.dsa_index_key_write(ctypes.byref(kvs), int(block_ids.shape[0]),
                                   block_ids.data_ptr(), coarse.data_ptr(),
                                   _stream(kv.idx_keys.device)))


# ---------------------------------------------------------------------------
# MXFP4 expert weights
# ---------------------------------------------------------------------------
@dataclass
class MxExperts:
    w_fp4: torch.Tensor    # uint8 [E, N, K/2]: E2M1 codes, element 2i in the low nibble
    w_scale: torch.Tensor  # uint8 [E, N, K/32]: E8M0 scales

    def struct(self):
        e, n, kh = self.w_fp4.shape
        return _lib.MxExpertsStruct(self.w_fp4.data_ptr(), self.w_scale.data_ptr(), e, n, 2 * kh)


def mx_quantize(x, codes=None, scales=None):
    """bf16 [rows, K] -> MXFP8 (E4M3 codes uint8 [rows, K], E8M0 scales uint8 [rows, K/32])."""
    lib = _lib.load()
    _check_tensors(x, codes, scales)
    rows, k = x.shape
    if codes is None:
        codes = torch.empty(rows, k, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(rows, k // 32, dtype=torch.uint8, device=x.device)
    _check(lib.dsa_mx_quantize(x.data_ptr(), rows, k, codes.data_ptr(), scales.data_ptr(),
                               _stream(x.device)))
    return codes, scales


def mxfp4_to_fp8(w, experts, ws_codes=None, ws_scales=None):
    """The online conversion of experts (int32 [n]) into FP8 workspace slots:
    (E4M3 codes uint8 [n, N, K], E8M0 scales uint8 [n, N, K/32])."""
    lib = _lib.load()
    _check_tensors(w.w_fp4, w.w_scale, experts, ws_codes, ws_scales)
    e, n, kh = w.w_fp4.shape
    m = experts.shape[0]
    if ws_codes is None:
        ws_codes = torch.empty(m, n, 2 * kh, dtype=torch.uint8, device=experts.device)
    if ws_scales is None:
        ws_scales = torch.empty(m, n, 2 * kh // 32, dtype=torch.uint8, device=experts.device)
    ws = w.struct()
    _check(lib.dsa_mxfp4_to_fp8(ctypes.byref(ws), experts.data_ptr(), m, ws_codes.data_ptr(),
                                ws_scales.data_ptr(), _stream(experts.device)))
    return ws_codes, ws_scales


def moe_workspace_size(w, tokens, slots, mode):
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    ws = w.struct()
    _check(lib.dsa_moe_workspace_size(ctypes.byref(ws), tokens, slots, mode, ctypes.byref(n)))
    return n.value


def moe_grouped_gemm(w, x_codes, x_scales, route, mode=None, out=None, workspace=None):
    """out[t, j, :] = xq[t] . W[route[t, j]]^T (fp32 [T, slots, N]); rows of
    slots routed to no expert (-1) are zero.  mode: MOE_FP4_DIRECT (default:
    FP4 weights straight to the matrix cores) or MOE_FP8_WORKSPACE (the routed
    experts unpacked to FP8 in the workspace first)."""
    lib = _lib.load()
    _check_tensors(w.w_fp4, w.w_scale, x_codes, x_scales, route, out)
    mode = _lib.MOE_FP4_DIRECT if mode is None else mode
    t, slots = route.shape
    n = w.w_fp4.shape[1]
    if out is None:
        out = torch.empty(t, slots, n, dtype=torch.float32, device=route.device)
    if workspace is None:
        workspace = _workspace(moe_workspace_size(w, t, slots, mode), route.device)
    ws = w.struct()
    _check(lib.dsa_moe_grouped_gemm(ctypes.byref(ws), x_codes.data_ptr(), x_scales.data_ptr(), t,
                                    route.data_ptr(), slots, mode, out.data_ptr(),
                                    workspace.data_ptr(), workspace.numel(),
                                    _stream(route.device)))
    return out
