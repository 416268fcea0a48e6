"""Python binding of libsa.so, the C ABI of the indexer-routed sparse-attention path.

Argument marshalling only: each ``sa_*`` function checks that every torch tensor
lives on the same HIP device as the first input, is contiguous and has the dtype and
full shape the C function expects, passes the data pointers, sizes and that device's
current stream to the C function of the same name, and raises ``SAError`` on a
non-zero status. Every step of the computation runs in the HIP
kernels of libsa.so; there is no other code path. Importing this package fails
loudly if libsa.so is missing (build it with ``python -m
indexer_routed_sparse_amd.build``).

The convenience wrappers at the end (``indexer_topk``, ``sparse_mla`` ...) only
allocate output tensors and call the ``sa_*`` functions.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "SAError", "SA_F32", "SA_BF16", "lib", "abi_version", "status_string",
    "sa_indexer_workspace_bytes", "indexer_workspace", "sa_indexer_scores", "sa_sparse_mla_bwd",
    "sparse_mla_bwd", "sa_block_sparse_gqa_bwd", "block_sparse_gqa_bwd", "sa_attn_teacher",
    "attn_teacher", "sa_indexer_kl_bwd", "indexer_kl_bwd", "sa_kpool_expand", "kpool_expand",
    "sa_append_window", "append_window", "sa_topk_select", "sa_sparse_mla_fwd", "sa_block_sparse_gqa_fwd",
    "indexer_scores", "indexer_topk", "topk_select", "sparse_mla", "block_sparse_gqa",
]

SA_F32 = 0
SA_BF16 = 1
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsa.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build the HIP library first "
        "(python -m indexer_routed_sparse_amd.build)")
lib = ctypes.CDLL(_LIB_PATH)

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float

lib.sa_status_string.restype = ctypes.c_char_p
lib.sa_status_string.argtypes = [ctypes.c_int]
lib.sa_abi_version.restype = ctypes.c_int
lib.sa_abi_version.argtypes = []
lib.sa_indexer_scores.restype = ctypes.c_int
lib.sa_indexer_scores.argtypes = [_p, _p, _p, ctypes.c_int, _i32, _p, _i32, _i32, _i32, _i32, _i32,
                                  _p, _i64, _i32, _i32, _p, _p, _p, ctypes.c_size_t, _p]
lib.sa_indexer_workspace_bytes.restype = ctypes.c_size_t
lib.sa_indexer_workspace_bytes.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _i32]
lib.sa_topk_select.restype = ctypes.c_int
lib.sa_topk_select.argtypes = [_p, _p, _i64, _i32, _p, _i32, _i32, _i32, _i32, _i32, _p, _p, _p]
lib.sa_sparse_mla_fwd.restype = ctypes.c_int
lib.sa_sparse_mla_fwd.argtypes = [_p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _i32,
                                  _f32, _p, _p, _p, _p]
lib.sa_sparse_mla_bwd.restype = ctypes.c_int
lib.sa_sparse_mla_bwd.argtypes = [_p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32,
                                  _i32, _f32, _p, _p, _p, _p, _p]
lib.sa_kpool_expand.restype = ctypes.c_int
lib.sa_kpool_expand.argtypes = [_p, _i32, _p, _i32, _i32, _i32, _i32, _p, _p]
lib.sa_append_window.restype = ctypes.c_int
lib.sa_append_window.argtypes = [_p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _p, _p]
lib.sa_block_sparse_gqa_bwd.restype = ctypes.c_int
lib.sa_block_sparse_gqa_bwd.argtypes = [_p, _p, _p, _p, _p, _p, ctypes.c_int, _i32, _p, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p, _p]
lib.sa_attn_teacher.restype = ctypes.c_int
lib.sa_attn_teacher.argtypes = [_p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _f32, _p, _p]
lib.sa_indexer_kl_bwd.restype = ctypes.c_int
lib.sa_indexer_kl_bwd.argtypes = [_p, _p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32,
                                  _p, _p, _p, _p, _p]
lib.sa_block_sparse_gqa_fwd.restype = ctypes.c_int
lib.sa_block_sparse_gqa_fwd.argtypes = [_p, _p, _p, _p, ctypes.c_int, _i32, _p, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p]


class SAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def abi_version() -> int:
    return lib.sa_abi_version()


def status_string(status: int) -> str:
    return lib.sa_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise SAError(status, where)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t) -> int:
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.float32:
        return SA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, device, dtype=None, shape=None, optional=False):
    """Check that ``t`` is a contiguous device tensor on ``device`` with the given dtype
    and shape (None entries of ``shape`` match any size). The kernels trust these
    facts: a host tensor or an undersized output would be read or written out of
    bounds on the device."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda" or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and int(a) != int(s)
                                        for a, s in zip(t.shape, shape)):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _device_of(t, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    return t.device


def _layout(T, cu_seqlens, max_seqlen, device):
    if cu_seqlens is None:
        return None, 0, 0
    _need(cu_seqlens, "cu_seqlens", device, torch.int32, (None,))
    if cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens needs at least two entries")
    if max_seqlen is None:
        raise ValueError("max_seqlen is required with cu_seqlens")
    return cu_seqlens, cu_seqlens.numel() - 1, int(max_seqlen)


# ------------------------------------------------------------------- C functions

def sa_indexer_workspace_bytes(dtype, T, max_seqlen, H_I, D_I, block_size, topk) -> int:
    """sa_indexer_workspace_bytes: workspace bytes of a fused selection (0: one pass)."""
    code = SA_BF16 if dtype in (torch.bfloat16, SA_BF16) else SA_F32
    return int(lib.sa_indexer_workspace_bytes(code, int(T), int(max_seqlen), int(H_I), int(D_I),
                                              int(block_size), int(topk)))


def sa_indexer_scores(q_I, k_I, w, *, cu_seqlens=None, max_seqlen=None, block_size=1,
                      scores=None, topk=0, force_own_block=False, out_idx=None, out_val=None,
                      ws=None):
    """sa_indexer_scores: dense scores (topk == 0) or fused exact top-k (topk > 0).

    ``ws`` (optional) is a uint8 device tensor used as the workspace of the two-pass
    selection; its size is checked by the library."""
    dev = _device_of(q_I, "q_I")
    if q_I.dim() != 3:
        raise ValueError("q_I must be [T, H_I, D_I]")
    T, H_I, D_I = q_I.shape
    _need(q_I, "q_I", dev)
    _need(k_I, "k_I", dev, q_I.dtype, (T, D_I))
    _need(w, "w", dev, torch.float32, (T, H_I))
    cu, nseq, maxlen = _layout(T, cu_seqlens, max_seqlen, dev)
    if topk == 0:
        _need(scores, "scores", dev, torch.float32, (T, None))
        ld = scores.shape[1]
    else:
        if scores is not None:
            raise ValueError("scores must be None with topk > 0")
        ld = 0
        _need(out_idx, "out_idx", dev, torch.int32, (T, topk))
        _need(out_val, "out_val", dev, torch.float32, (T, topk), optional=True)
    _need(ws, "ws", dev, torch.uint8, (None,), optional=True)
    ws_bytes = ws.numel() if ws is not None else 0
    _check(lib.sa_indexer_scores(_ptr(q_I), _ptr(k_I), _ptr(w), _dtype_code(q_I), T, _ptr(cu), nseq,
                                 maxlen, H_I, D_I, int(block_size), _ptr(scores), ld, int(topk),
                                 int(bool(force_own_block)), _ptr(out_idx), _ptr(out_val),
                                 _ptr(ws), ws_bytes, _stream(dev)), "sa_indexer_scores")


def sa_topk_select(vals, out_idx, *, out_val=None, cand_idx=None, cu_seqlens=None, max_seqlen=None,
                   block_size=1, force_own_block=0):
    """sa_topk_select: exact top-k of each row of ``vals`` [T, ld] into ``out_idx`` [T, topk].
    force_own_block (block mode): 0 own block competes, 1 own block kept, 2 complete
    blocks only."""
    dev = _device_of(vals, "vals")
    _need(vals, "vals", dev, torch.float32, (None, None))
    T, ld = vals.shape
    _need(out_idx, "out_idx", dev, torch.int32, (T, None))
    topk = out_idx.shape[1]
    _need(out_val, "out_val", dev, torch.float32, (T, topk), optional=True)
    _need(cand_idx, "cand_idx", dev, torch.int32, (T, ld), optional=True)
    cu, nseq, maxlen = _layout(T, cu_seqlens, max_seqlen, dev)
    _check(lib.sa_topk_select(_ptr(vals), _ptr(cand_idx), ld, T, _ptr(cu), nseq, maxlen,
                              int(block_size), topk, int(force_own_block), _ptr(out_idx),
                              _ptr(out_val), _stream(dev)), "sa_topk_select")


def sa_sparse_mla_fwd(q, kv, idx, scale, out, lse=None, sink=None):
    """sa_sparse_mla_fwd: q [T,H,d_qk], kv [S,d_qk], idx [T,topk] -> out [T,H,d_v], lse [T,H];
    sink [H] fp32 optional (a per-head logit in the softmax denominator)."""
    dev = _device_of(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d_qk]")
    T, H, d_qk = q.shape
    _need(q, "q", dev)
    _need(kv, "kv", dev, q.dtype, (None, d_qk))
    S = kv.shape[0]
    _need(idx, "idx", dev, torch.int32, (T, None))
    _need(out, "out", dev, q.dtype, (T, H, None))
    _need(lse, "lse", dev, torch.float32, (T, H), optional=True)
    _need(sink, "sink", dev, torch.float32, (H,), optional=True)
    _check(lib.sa_sparse_mla_fwd(_ptr(q), _ptr(kv), _ptr(idx), _dtype_code(q), T, S, H, d_qk,
                                 out.shape[2], idx.shape[1], float(scale), _ptr(sink), _ptr(out),
                                 _ptr(lse), _stream(dev)), "sa_sparse_mla_fwd")


def sa_sparse_mla_bwd(q, kv, idx, dout, lse, scale, dq, dkv, sink=None, dsink=None):
    """sa_sparse_mla_bwd: gradients dq [T,H,d_qk] (q's dtype) and dkv [S,d_qk] (fp32,
    overwritten) of sparse MLA from dout, given the forward's lse; with the forward's
    sink, dsink [H] (fp32, overwritten) too."""
    dev = _device_of(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d_qk]")
    T, H, d_qk = q.shape
    _need(q, "q", dev)
    _need(kv, "kv", dev, q.dtype, (None, d_qk))
    S = kv.shape[0]
    _need(idx, "idx", dev, torch.int32, (T, None))
    _need(dout, "dout", dev, q.dtype, (T, H, None))
    d_v = dout.shape[2]
    _need(lse, "lse", dev, torch.float32, (T, H))
    _need(dq, "dq", dev, q.dtype, (T, H, d_qk))
    _need(dkv, "dkv", dev, torch.float32, (S, d_qk))
    _need(sink, "sink", dev, torch.float32, (H,), optional=True)
    _need(dsink, "dsink", dev, torch.float32, (H,), optional=True)
    _check(lib.sa_sparse_mla_bwd(_ptr(q), _ptr(kv), _ptr(idx), _ptr(dout), _ptr(lse),
                                 _dtype_code(q), T, S, H, d_qk, d_v, idx.shape[1], float(scale),
                                 _ptr(sink), _ptr(dq), _ptr(dkv), _ptr(dsink), _stream(dev)),
           "sa_sparse_mla_bwd")


def sa_kpool_expand(pools, pool, out, *, cu_seqlens=None, max_seqlen=None):
    """sa_kpool_expand: pool routes [T,kp] -> token slots [T, kp*pool + pool - 1]."""
    dev = _device_of(pools, "pools")
    _need(pools, "pools", dev, torch.int32, (None, None))
    T, kp = pools.shape
    _need(out, "out", dev, torch.int32, (T, kp * pool + pool - 1))
    cu, nseq, maxlen = _layout(T, cu_seqlens, max_seqlen, dev)
    _check(lib.sa_kpool_expand(_ptr(pools), T, _ptr(cu), nseq, maxlen, kp, int(pool), _ptr(out),
                               _stream(dev)), "sa_kpool_expand")


def sa_append_window(idx, window, offset, out, *, cu_seqlens=None, max_seqlen=None):
    """sa_append_window: selected slots [T,k] + a causal window -> [T, k + window]."""
    dev = _device_of(idx, "idx")
    _need(idx, "idx", dev, torch.int32, (None, None))
    T, k = idx.shape
    _need(out, "out", dev, torch.int32, (T, k + window))
    cu, nseq, maxlen = _layout(T, cu_seqlens, max_seqlen, dev)
    _check(lib.sa_append_window(_ptr(idx), T, _ptr(cu), nseq, maxlen, k, int(window), int(offset),
                                _ptr(out), _stream(dev)), "sa_append_window")


def sa_block_sparse_gqa_fwd(q, k, v, blk, scale, out, lse=None, *, block_size, cu_seqlens=None,
                            max_seqlen=None):
    """sa_block_sparse_gqa_fwd: q [T,Hq,D], k/v [T,Hkv,D], blk [T,nblk] -> out [T,Hq,Dv]."""
    dev = _device_of(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [T, Hq, D]")
    T, Hq, D = q.shape
    _need(q, "q", dev)
    _need(k, "k", dev, q.dtype, (T, None, D))
    Hkv = k.shape[1]
    _need(v, "v", dev, q.dtype, (T, Hkv, None))
    Dv = v.shape[2]
    _need(blk, "blk", dev, torch.int32, (T, None))
    _need(out, "out", dev, q.dtype, (T, Hq, Dv))
    _need(lse, "lse", dev, torch.float32, (T, Hq), optional=True)
    cu, nseq, maxlen = _layout(T, cu_seqlens, max_seqlen, dev)
    _check(lib.sa_block_sparse_gqa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(blk), _dtype_code(q), T,
                                       _ptr(cu), nseq, maxlen, Hq, Hkv, D, Dv, int(block_size),
                                       blk.shape[1], float(scale), _ptr(out), _ptr(lse),
                                       _stream(dev)), "sa_block_sparse_gqa_fwd")


def sa_block_sparse_gqa_bwd(q, k, v, blk, dout, lse, scale, dq, dk, dv, *, block_size,
                            cu_seqlens=None, max_seqlen=None):
    """sa_block_sparse_gqa_bwd: dq [T,Hq,D] (q's dtype), dk/dv [T,Hkv,D] fp32 (overwritten)."""
    dev = _device_of(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [T, Hq, D]")
    T, Hq, D = q.shape
    _need(q, "q", dev)
    _need(k, "k", dev, q.dtype, (T, None, D))
    Hkv = k.shape[1]
    _need(v, "v", dev, q.dtype, (T, Hkv, None))
    Dv = v.shape[2]
    _need(blk, "blk", dev, torch.int32, (T, None))
    _need(dout, "dout", dev, q.dtype, (T, Hq, Dv))
    _need(lse, "lse", dev, torch.float32, (T, Hq))
    _need(dq, "dq", dev, q.dtype, (T, Hq, D))
    _need(dk, "dk", dev, torch.float32, (T, Hkv, D))
    _need(dv, "dv", dev, torch.float32, (T, Hkv, Dv))
    cu, nseq, maxlen = _layout(T, cu_seqlens, max_seqlen, dev)
    _check(lib.sa_block_sparse_gqa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(blk), _ptr(dout), _ptr(lse),
                                       _dtype_code(q), T, _ptr(cu), nseq, maxlen, Hq, Hkv, D, Dv,
                                       int(block_size), blk.shape[1], float(scale), _ptr(dq), _ptr(dk),
                                       _ptr(dv), _stream(dev)), "sa_block_sparse_gqa_bwd")


def sa_attn_teacher(q, kv, idx, lse, scale, teacher):
    """sa_attn_teacher: head-mean attention probability of every slot -> teacher [T,k] fp32."""
    dev = _device_of(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d_qk]")
    T, H, d_qk = q.shape
    _need(q, "q", dev)
    _need(kv, "kv", dev, q.dtype, (None, d_qk))
    _need(idx, "idx", dev, torch.int32, (T, None))
    _need(lse, "lse", dev, torch.float32, (T, H))
    _need(teacher, "teacher", dev, torch.float32, (T, idx.shape[1]))
    _check(lib.sa_attn_teacher(_ptr(q), _ptr(kv), _ptr(idx), _ptr(lse), _dtype_code(q), T, kv.shape[0], H,
                               d_qk, idx.shape[1], float(scale), _ptr(teacher), _stream(dev)),
           "sa_attn_teacher")


def sa_indexer_kl_bwd(q_I, k_I, w, idx, teacher, loss, dq_I, dw, dk_I, grad=None):
    """sa_indexer_kl_bwd: sparse KL loss [T] and its gradients dq_I, dw, dk_I (fp32, overwritten)."""
    dev = _device_of(q_I, "q_I")
    if q_I.dim() != 3:
        raise ValueError("q_I must be [T, H_I, D_I]")
    T, H_I, D_I = q_I.shape
    _need(q_I, "q_I", dev)
    _need(k_I, "k_I", dev, q_I.dtype, (None, D_I))
    _need(w, "w", dev, torch.float32, (T, H_I))
    _need(idx, "idx", dev, torch.int32, (T, None))
    k = idx.shape[1]
    _need(teacher, "teacher", dev, torch.float32, (T, k))
    _need(grad, "grad", dev, torch.float32, (T,), optional=True)
    _need(loss, "loss", dev, torch.float32, (T,))
    _need(dq_I, "dq_I", dev, q_I.dtype, (T, H_I, D_I))
    _need(dw, "dw", dev, torch.float32, (T, H_I))
    _need(dk_I, "dk_I", dev, torch.float32, tuple(k_I.shape))
    _check(lib.sa_indexer_kl_bwd(_ptr(q_I), _ptr(k_I), _ptr(w), _ptr(idx), _ptr(teacher), _ptr(grad),
                                 _dtype_code(q_I), T, k_I.shape[0], H_I, D_I, k, _ptr(loss), _ptr(dq_I),
                                 _ptr(dw), _ptr(dk_I), _stream(dev)), "sa_indexer_kl_bwd")


# ------------------------------------------------------- allocating conveniences

def indexer_scores(q_I, k_I, w, *, cu_seqlens=None, max_seqlen=None, block_size=1, ld=None):
    T = q_I.shape[0]
    width = max_seqlen if cu_seqlens is not None else T
    ncol = width if block_size == 1 else -(-width // block_size)
    ld = ld or ((ncol + 3) // 4 * 4)
    scores = torch.full((T, ld), float("-inf"), dtype=torch.float32, device=q_I.device)
    sa_indexer_scores(q_I, k_I, w, cu_seqlens=cu_seqlens, max_seqlen=max_seqlen,
                      block_size=block_size, scores=scores)
    return scores


def indexer_workspace(q_I, topk, *, max_seqlen=None, block_size=1):
    """A workspace tensor for a fused selection over q_I (None when it runs in one pass)."""
    T, H_I, D_I = q_I.shape
    n = sa_indexer_workspace_bytes(q_I.dtype, T, max_seqlen or T, H_I, D_I, block_size, topk)
    return torch.empty(n, dtype=torch.uint8, device=q_I.device) if n else None


def indexer_topk(q_I, k_I, w, topk, *, cu_seqlens=None, max_seqlen=None, block_size=1,
                 force_own_block=False, with_values=False, workspace=True):
    """Fused exact top-k; ``workspace`` True allocates the two-pass workspace when the
    call can use one, False runs the one-pass kernel, a tensor is used as given."""
    T = q_I.shape[0]
    idx = torch.empty((T, topk), dtype=torch.int32, device=q_I.device)
    val = torch.empty((T, topk), dtype=torch.float32, device=q_I.device) if with_values else None
    ws = workspace
    if workspace is True:
        ws = indexer_workspace(q_I, topk, max_seqlen=max_seqlen if cu_seqlens is not None else None,
                               block_size=block_size)
    elif workspace is False:
        ws = None
    sa_indexer_scores(q_I, k_I, w, cu_seqlens=cu_seqlens, max_seqlen=max_seqlen,
                      block_size=block_size, topk=topk, force_own_block=force_own_block,
                      out_idx=idx, out_val=val, ws=ws)
    return (idx, val) if with_values else idx


def topk_select(vals, topk, *, cand_idx=None, cu_seqlens=None, max_seqlen=None, block_size=1,
                force_own_block=False, with_values=False):
    T = vals.shape[0]
    idx = torch.empty((T, topk), dtype=torch.int32, device=vals.device)
    val = torch.empty((T, topk), dtype=torch.float32, device=vals.device) if with_values else None
    sa_topk_select(vals, idx, out_val=val, cand_idx=cand_idx, cu_seqlens=cu_seqlens,
                   max_seqlen=max_seqlen, block_size=block_size, force_own_block=force_own_block)
    return (idx, val) if with_values else idx


def sparse_mla(q, kv, idx, scale, d_v=512, with_lse=True, sink=None):
    T, H, _ = q.shape
    out = torch.empty((T, H, d_v), dtype=q.dtype, device=q.device)
    lse = torch.empty((T, H), dtype=torch.float32, device=q.device) if with_lse else None
    sa_sparse_mla_fwd(q, kv, idx, scale, out, lse, sink=sink)
    return (out, lse) if with_lse else out


def sparse_mla_bwd(q, kv, idx, dout, lse, scale, sink=None):
    dq = torch.empty_like(q)
    dkv = torch.empty(kv.shape, dtype=torch.float32, device=q.device)
    dsink = torch.empty(q.shape[1], dtype=torch.float32, device=q.device) if sink is not None else None
    sa_sparse_mla_bwd(q, kv, idx, dout, lse, scale, dq, dkv, sink=sink, dsink=dsink)
    return (dq, dkv) if sink is None else (dq, dkv, dsink)


def kpool_expand(pools, pool, *, cu_seqlens=None, max_seqlen=None):
    T, kp = pools.shape
    out = torch.empty((T, kp * pool + pool - 1), dtype=torch.int32, device=pools.device)
    sa_kpool_expand(pools, pool, out, cu_seqlens=cu_seqlens, max_seqlen=max_seqlen)
    return out


def append_window(idx, window, offset=0, *, cu_seqlens=None, max_seqlen=None):
    T, k = idx.shape
    out = torch.empty((T, k + window), dtype=torch.int32, device=idx.device)
    sa_append_window(idx, window, offset, out, cu_seqlens=cu_seqlens, max_seqlen=max_seqlen)
    return out


def attn_teacher(q, kv, idx, lse, scale):
    teacher = torch.empty(idx.shape, dtype=torch.float32, device=q.device)
    sa_attn_teacher(q, kv, idx, lse, scale, teacher)
    return teacher


def indexer_kl_bwd(q_I, k_I, w, idx, teacher, grad=None):
    T = q_I.shape[0]
    loss = torch.empty(T, dtype=torch.float32, device=q_I.device)
    dq_I = torch.empty_like(q_I)
    dw = torch.empty_like(w)
    dk_I = torch.empty(k_I.shape, dtype=torch.float32, device=q_I.device)
    sa_indexer_kl_bwd(q_I, k_I, w, idx, teacher, loss, dq_I, dw, dk_I, grad=grad)
    return loss, dq_I, dw, dk_I


def block_sparse_gqa_bwd(q, k, v, blk, dout, lse, scale, *, block_size, cu_seqlens=None,
                         max_seqlen=None):
    dq = torch.empty_like(q)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    sa_block_sparse_gqa_bwd(q, k, v, blk, dout, lse, scale, dq, dk, dv, block_size=block_size,
                            cu_seqlens=cu_seqlens, max_seqlen=max_seqlen)
    return dq, dk, dv


def block_sparse_gqa(q, k, v, blk, scale, *, block_size, cu_seqlens=None, max_seqlen=None,
                     with_lse=True):
    T, Hq, _ = q.shape
    out = torch.empty((T, Hq, v.shape[2]), dtype=q.dtype, device=q.device)
    lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device) if with_lse else None
    sa_block_sparse_gqa_fwd(q, k, v, blk, scale, out, lse, block_size=block_size,
                            cu_seqlens=cu_seqlens, max_seqlen=max_seqlen)
    return (out, lse) if with_lse else out
