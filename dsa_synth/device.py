"""ctypes loader for the device filler (input data only)."""

import ctypes
import os

import numpy as np

from . import gen

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_synth.so")
_lib = None
_tables = {}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        _lib = ctypes.CDLL(LIB_PATH)
        f = _lib.dsa_synth_fill_bf16_normal
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                      ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    return _lib


def _table(device):
    import torch
    key = str(device)
    if key not in _tables:
        t = torch.from_numpy(gen.normal_table_bf16().view(np.int16).copy())
        _tables[key] = t.to(device)
    return _tables[key]


def fill_bf16_normal(t, seed, tag, offset=0):
    """Fill the contiguous bf16 CUDA tensor ``t`` with stream (seed, tag) from ``offset``."""
    import torch
    assert t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous()
    stream = torch.cuda.current_stream(t.device).cuda_stream
    rc = lib().dsa_synth_fill_bf16_normal(t.data_ptr(), t.numel(), offset, seed, tag,
                                          _table(t.device).data_ptr(), stream)
    if rc != 0:
        raise RuntimeError(f"dsa_synth_fill_bf16_normal failed: {rc}")
    return t


def upload(w, device="cuda"):
    """Device tensors of workload ``w``: K/V pools filled on the device, the
    small tensors copied from the host.  Returns a dict of torch tensors."""
    import torch

    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    k = torch.empty(shape, dtype=torch.bfloat16, device=device)
    v = torch.empty(shape, dtype=torch.bfloat16, device=device)
    fill_bf16_normal(k, w.seed, gen.TAG_K)
    fill_bf16_normal(v, w.seed, gen.TAG_V)

    def t(a, dtype=None):
        x = torch.from_numpy(np.ascontiguousarray(a))
        if dtype is not None:
            x = x.view(dtype)
        return x.to(device)

    return dict(
        k_cache=k, v_cache=v, idx_keys=t(w.idx_keys), idx_scale=t(w.idx_scale),
        block_table=t(w.block_table.astype(np.int32)), seq_lens=t(w.seq_lens.astype(np.int32)),
        q=t(w.q_bits.view(np.int16), torch.bfloat16),
        q_idx=t(w.q_idx_bits.view(np.int16), torch.bfloat16), w_idx=t(w.w),
        q_seq=None if w.decode else t(w.q_seq), q_pos=None if w.decode else t(w.q_pos))
