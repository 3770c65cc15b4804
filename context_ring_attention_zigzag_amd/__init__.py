"""Python binding of libcpring: per-rank zigzag ring attention on MI355X.

Argument marshalling only. Every step of the computation runs in the HIP
kernels of ``libcpring.so``; this module turns torch tensors (used as device
memory) and torch streams into the pointers, strides and sizes the C ABI
declared in ``include/cpring.h`` expects, and turns non-zero status codes
into ``CprError``. There is no fallback: if the library is missing, every
call raises.

Tensors are [B, H, L, D] with the last dimension contiguous; position arrays
are int32 device tensors.
"""

from __future__ import annotations

import ctypes
import os

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libcpring.so")

F32, BF16 = 0, 1
ZIGZAG, CONTIGUOUS, STRIPED = 0, 1, 2
RUN_FUSED, RUN_STEPWISE = 0, 1
ROPE_INTERLEAVED, ROPE_HALF = 0, 1
OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3

# Every symbol include/cpring.h declares.
EXPORTS = (
    "cp_padded_len", "cp_zigzag_partition", "cp_shard_gather", "cp_ring_attn_init", "cp_ring_attn_step",
    "cp_ring_attn_merge", "cp_ring_attn_finalize", "cp_ring_attn_workspace_size", "cp_ring_attn_run",
    "cp_ring_attn_step_ex", "cp_ring_attn_run_ex", "cp_ring_attn_run_noalloc", "cp_ring_attn_bwd_workspace_size",
    "cp_ring_attn_bwd_workspace_size_ex", "cp_ring_attn_bwd_prep",
    "cp_ring_attn_bwd_step", "cp_ring_attn_bwd_run", "cp_rope_apply", "cp_ring_attn_tile_census", "cp_status_string", "cp_last_error",
)


class CprError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func} failed with status {status}: {detail}")
        self.status = status


class CprView(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_l", ctypes.c_int64)]


class CprAttnExt(ctypes.Structure):
    """cpr_attn_ext: K/V head count, optional per-query key-position window, and the first/last-hop flags and
    outputs read by cp_ring_attn_step_ex."""
    _fields_ = [("H_kv", ctypes.c_int32), ("kw_lo", ctypes.c_void_p), ("kw_hi", ctypes.c_void_p),
                ("step_flags", ctypes.c_int32), ("o_out", ctypes.c_void_p), ("lse_out", ctypes.c_void_p)]


STEP_FIRST, STEP_LAST = 1, 2   # CPR_STEP_FIRST, CPR_STEP_LAST


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libcpring.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m context_ring_attention_zigzag_amd.build`")
    lib = ctypes.CDLL(path)
    i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    pv = ctypes.POINTER(CprView)
    pe = ctypes.POINTER(CprAttnExt)
    sig = {
        "cp_padded_len": (i64, [i64, i32, i32]),
        "cp_zigzag_partition": (i32, [i64, i32, i32, vp, vp, vp]),
        "cp_shard_gather": (i32, [i32, i32, i32, i64, i32, pv, vp, i64, vp, vp]),
        "cp_ring_attn_init": (i32, [i32, i32, i32, i32, vp, vp, vp, vp]),
        "cp_ring_attn_step": (i32, [i32, i32, i32, i32, pv, i32, vp, pv, pv, i32, vp, i32, f32, vp, vp, vp, vp]),
        "cp_ring_attn_merge": (i32, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]),
        "cp_ring_attn_finalize": (i32, [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]),
        "cp_ring_attn_workspace_size": (ctypes.c_size_t, [i32, i32, i32, i32]),
        "cp_ring_attn_run": (i32, [i32, i32, i32, i32, i32, i32, pv, i32, vp, pv, pv, vp, i32, f32, vp, vp, vp,
                                   ctypes.c_size_t, i32, vp]),
        "cp_ring_attn_step_ex": (i32, [i32, i32, i32, i32, pv, i32, vp, pv, pv, i32, vp, i32, f32, pe, vp, vp, vp,
                                       vp]),
        "cp_ring_attn_run_ex": (i32, [i32, i32, i32, i32, i32, i32, pv, i32, vp, pv, pv, vp, i32, f32, pe, vp, vp,
                                      vp, ctypes.c_size_t, i32, vp]),
        "cp_ring_attn_run_noalloc": (i32, [i32, i32, i32, i32, i32, i32, pv, i32, vp, pv, pv, vp, i32, f32, pe, vp,
                                           vp, vp]),
        "cp_ring_attn_bwd_workspace_size": (ctypes.c_size_t, [i32, i32, i32]),
        "cp_ring_attn_bwd_workspace_size_ex": (ctypes.c_size_t, [i32, i32, i32, i32, i32, i64]),
        "cp_ring_attn_bwd_prep": (i32, [i32, i32, i32, i32, i32, pv, pv, vp, vp, i32, pe, vp, ctypes.c_size_t, vp]),
        "cp_ring_attn_bwd_step": (i32, [i32, i32, i32, i32, i32, pv, pv, i32, pv, pv, i32, vp, f32, vp,
                                        ctypes.c_size_t, vp, vp, vp, vp]),
        "cp_ring_attn_bwd_run": (i32, [i32, i32, i32, i32, i32, i32, pv, i32, vp, pv, pv, vp, pv, pv, vp, i32, f32,
                                       pe, vp, vp, vp, vp, ctypes.c_size_t, vp]),
        "cp_rope_apply": (i32, [i32, i32, i32, i32, i32, pv, vp, f32, i32, vp, vp]),
        "cp_ring_attn_tile_census": (i32, [i32, i32, vp, vp, i32, pe, vp, vp, vp]),
        "cp_status_string": (ctypes.c_char_p, [i32]),
        "cp_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, func: str):
    if status != OK:
        raise CprError(status, func, load().cp_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def view(t) -> CprView:
    """cpr_view of a [B, H, L, D] tensor (D must be contiguous)."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, H, L, D] tensor with contiguous last dim")
    return CprView(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def dtype_code(t) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {t.dtype}")


# ----------------------------------------------------------------- the ABI

def cp_padded_len(seq_len: int, cp_size: int, layout: int) -> int:
    return load().cp_padded_len(seq_len, cp_size, layout)


def cp_zigzag_partition(seq_len: int, cp_size: int, layout: int, token_idx=None, pos_ids=None, stream=None):
    _check(load().cp_zigzag_partition(seq_len, cp_size, layout, _ptr(token_idx), _ptr(pos_ids), _stream(stream)),
           "cp_zigzag_partition")


def cp_shard_gather(src, seq_len: int, token_idx, dst, stream=None):
    B, H, _, D = src.shape
    v = view(src)
    _check(load().cp_shard_gather(dtype_code(src), B, H, seq_len, D, ctypes.byref(v), _ptr(token_idx),
                                  dst.shape[2], _ptr(dst), _stream(stream)), "cp_shard_gather")


def cp_ring_attn_init(o_acc, m, l, stream=None):
    B, H, Lq, D = o_acc.shape
    _check(load().cp_ring_attn_init(B, H, Lq, D, _ptr(o_acc), _ptr(m), _ptr(l), _stream(stream)),
           "cp_ring_attn_init")


def _ext(q, k, kw_lo, kw_hi):
    """cpr_attn_ext for K/V with k.shape[1] heads and the optional windows, or None for the plain pass."""
    h, h_kv = q.shape[1], k.shape[1]
    if h_kv == h and kw_lo is None and kw_hi is None:
        return None
    return CprAttnExt(h_kv, None if kw_lo is None else kw_lo.data_ptr(), None if kw_hi is None else kw_hi.data_ptr())


def cp_ring_attn_step(q, q_pos, k, v, kv_pos, causal: bool, softmax_scale: float, o_acc, m, l, stream=None,
                      kw_lo=None, kw_hi=None, first: bool = False, last: bool = False, o_out=None, lse_out=None):
    """One ring step; k and v may have fewer heads than q (grouped-query attention). first: start from the
    empty state (o_acc, m, l not read); last: write o_out (and lse_out) instead of the state."""
    B, H, Lq, D = q.shape
    qv, kv, vv = view(q), view(k), view(v)
    ext = _ext(q, k, kw_lo, kw_hi)
    flags = (STEP_FIRST if first else 0) | (STEP_LAST if last else 0)
    if flags:
        if ext is None:
            ext = CprAttnExt(k.shape[1], None, None)
        ext.step_flags = flags
        ext.o_out = None if o_out is None else o_out.data_ptr()
        ext.lse_out = None if lse_out is None else lse_out.data_ptr()
    _check(load().cp_ring_attn_step_ex(dtype_code(q), B, H, D, ctypes.byref(qv), Lq, _ptr(q_pos), ctypes.byref(kv),
                                       ctypes.byref(vv), k.shape[2], _ptr(kv_pos), int(bool(causal)),
                                       float(softmax_scale), None if ext is None else ctypes.byref(ext), _ptr(o_acc),
                                       _ptr(m), _ptr(l), _stream(stream)),
           "cp_ring_attn_step_ex")


def cp_ring_attn_merge(o_acc, m, l, o2, m2, l2, stream=None):
    B, H, Lq, D = o_acc.shape
    _check(load().cp_ring_attn_merge(B, H, Lq, D, _ptr(o_acc), _ptr(m), _ptr(l), _ptr(o2), _ptr(m2), _ptr(l2),
                                     _stream(stream)), "cp_ring_attn_merge")


def cp_ring_attn_finalize(o_acc, m, l, o_out, lse_out=None, stream=None):
    B, H, Lq, D = o_acc.shape
    _check(load().cp_ring_attn_finalize(dtype_code(o_out), B, H, Lq, D, _ptr(o_acc), _ptr(m), _ptr(l), _ptr(o_out),
                                        _ptr(lse_out), _stream(stream)), "cp_ring_attn_finalize")


def cp_ring_attn_workspace_size(B: int, H: int, Lq: int, D: int) -> int:
    return load().cp_ring_attn_workspace_size(B, H, Lq, D)


def cp_ring_attn_run(q_local, q_pos, k_ring, v_ring, ring_pos, cp_size: int, rank: int, causal: bool,
                     softmax_scale: float, o_out, lse_out=None, workspace=None, flags: int = RUN_FUSED,
                     stream=None, kw_lo=None, kw_hi=None):
    """One rank's ring pass; k_ring and v_ring may have fewer heads than q_local (grouped-query
    attention), and kw_lo / kw_hi (int32 [Lq] or None) bound the key positions each query may attend."""
    B, H, Lq, D = q_local.shape
    qv, kv, vv = view(q_local), view(k_ring), view(v_ring)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ext = _ext(q_local, k_ring, kw_lo, kw_hi)
    if ext is None:
        _check(load().cp_ring_attn_run(dtype_code(q_local), B, H, D, cp_size, rank, ctypes.byref(qv), Lq,
                                       _ptr(q_pos), ctypes.byref(kv), ctypes.byref(vv), _ptr(ring_pos),
                                       int(bool(causal)), float(softmax_scale), _ptr(o_out), _ptr(lse_out),
                                       _ptr(workspace), ws_bytes, flags, _stream(stream)), "cp_ring_attn_run")
        return
    _check(load().cp_ring_attn_run_ex(dtype_code(q_local), B, H, D, cp_size, rank, ctypes.byref(qv), Lq,
                                      _ptr(q_pos), ctypes.byref(kv), ctypes.byref(vv), _ptr(ring_pos),
                                      int(bool(causal)), float(softmax_scale), ctypes.byref(ext), _ptr(o_out),
                                      _ptr(lse_out), _ptr(workspace), ws_bytes, flags, _stream(stream)),
           "cp_ring_attn_run_ex")


# Bytes of the scratch array cp_ring_attn_run_noalloc keeps on each GPU (CPR_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 34078720


def cp_ring_attn_run_noalloc(q_local, q_pos, k_ring, v_ring, ring_pos, cp_size: int, rank: int, causal: bool,
                             softmax_scale: float, o_out, lse_out=None, stream=None, kw_lo=None, kw_hi=None):
    """cp_ring_attn_run in fused mode without a workspace: a key split keeps its partial states in the
    library's scratch array. Allocates nothing (o_out and lse_out are the caller's)."""
    B, H, Lq, D = q_local.shape
    qv, kv, vv = view(q_local), view(k_ring), view(v_ring)
    ext = _ext(q_local, k_ring, kw_lo, kw_hi)
    _check(load().cp_ring_attn_run_noalloc(dtype_code(q_local), B, H, D, cp_size, rank, ctypes.byref(qv), Lq,
                                           _ptr(q_pos), ctypes.byref(kv), ctypes.byref(vv), _ptr(ring_pos),
                                           int(bool(causal)), float(softmax_scale),
                                           None if ext is None else ctypes.byref(ext), _ptr(o_out), _ptr(lse_out),
                                           _stream(stream)),
           "cp_ring_attn_run_noalloc")


# ------------------------------------------------------------ backward pass

def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _win_ext(h_kv: int, kw_lo, kw_hi):
    if h_kv == 0 and kw_lo is None and kw_hi is None:
        return None
    return CprAttnExt(h_kv, None if kw_lo is None else kw_lo.data_ptr(), None if kw_hi is None else kw_hi.data_ptr())


def cp_ring_attn_bwd_workspace_size(B: int, H: int, Lq: int) -> int:
    return load().cp_ring_attn_bwd_workspace_size(B, H, Lq)


def cp_ring_attn_bwd_workspace_size_ex(B: int, H: int, H_kv: int, D: int, Lq: int, Lk: int) -> int:
    """Workspace bytes with room for the split of a small backward grid (Lk: K/V rows of the call)."""
    return load().cp_ring_attn_bwd_workspace_size_ex(B, H, H_kv, D, Lq, Lk)


def cp_ring_attn_bwd_prep(o, do, lse, q_pos, causal: bool, workspace, kw_lo=None, kw_hi=None, stream=None):
    """Per-row {LSE * log2(e), rowsum(dO * O)} and per-query key windows into `workspace`."""
    B, H, Lq, D = o.shape
    ov, gv = view(o), view(do)
    ext = _win_ext(0, kw_lo, kw_hi)
    _check(load().cp_ring_attn_bwd_prep(dtype_code(o), B, H, D, Lq, ctypes.byref(ov), ctypes.byref(gv), _ptr(lse),
                                        _ptr(q_pos), int(bool(causal)), None if ext is None else ctypes.byref(ext),
                                        _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "cp_ring_attn_bwd_prep")


def cp_ring_attn_bwd_step(q, do, k, v, kv_pos, softmax_scale: float, workspace, dq_acc, dk_acc, dv_acc,
                          stream=None):
    """Add one KV block's contributions: dq_acc [B,H,Lq,D], dk_acc and dv_acc [B,H_kv,Lk,D] (float32)."""
    B, H, Lq, D = q.shape
    qv, gv, kv, vv = view(q), view(do), view(k), view(v)
    _check(load().cp_ring_attn_bwd_step(dtype_code(q), B, H, D, k.shape[1], ctypes.byref(qv), ctypes.byref(gv), Lq,
                                        ctypes.byref(kv), ctypes.byref(vv), k.shape[2], _ptr(kv_pos),
                                        float(softmax_scale), _ptr(workspace), _nbytes(workspace), _ptr(dq_acc),
                                        _ptr(dk_acc), _ptr(dv_acc), _stream(stream)),
           "cp_ring_attn_bwd_step")


def cp_ring_attn_bwd_run(q_local, q_pos, k_ring, v_ring, ring_pos, cp_size: int, rank: int, o_local, do_local,
                         lse_local, causal: bool, softmax_scale: float, dq, dk, dv, workspace, stream=None,
                         kw_lo=None, kw_hi=None):
    """One rank's backward ring pass: writes dq [B,H,Lq,D] and the rank's share of every block's
    dk, dv [B,H_kv,cp*Lq,D] (float32), in ring order."""
    B, H, Lq, D = q_local.shape
    qv, kv, vv, ov, gv = view(q_local), view(k_ring), view(v_ring), view(o_local), view(do_local)
    h_kv = k_ring.shape[1]
    ext = _win_ext(0 if h_kv == H else h_kv, kw_lo, kw_hi)
    _check(load().cp_ring_attn_bwd_run(dtype_code(q_local), B, H, D, cp_size, rank, ctypes.byref(qv), Lq,
                                       _ptr(q_pos), ctypes.byref(kv), ctypes.byref(vv), _ptr(ring_pos),
                                       ctypes.byref(ov), ctypes.byref(gv), _ptr(lse_local), int(bool(causal)),
                                       float(softmax_scale), None if ext is None else ctypes.byref(ext), _ptr(dq),
                                       _ptr(dk), _ptr(dv), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "cp_ring_attn_bwd_run")


# ----------------------------------------------------- rotary embeddings

def cp_rope_apply(x, pos, out=None, base: float = 10000.0, style: int = ROPE_INTERLEAVED, stream=None):
    """Rotate x [B, H, L, D] by the global positions pos [L] (int32, -1 = pad); returns out (contiguous,
    allocated when None; may be x itself when x is contiguous)."""
    B, H, L, D = x.shape
    if out is None:
        out = torch.empty((B, H, L, D), dtype=x.dtype, device=x.device)
    xv = view(x)
    _check(load().cp_rope_apply(dtype_code(x), B, H, L, D, ctypes.byref(xv), _ptr(pos), float(base), int(style),
                                _ptr(out), _stream(stream)), "cp_rope_apply")
    return out


# ------------------------------------------------------------- tile census

def cp_ring_attn_tile_census(q_pos, ring_pos, cp_size: int, causal: bool, kw_lo=None, kw_hi=None, stream=None):
    """(kept, masked): int32 device tensors with, per 256-query tile, the 64-key tiles the bf16 forward pass
    computes over all blocks and how many of those need the element mask."""
    lq = q_pos.numel()
    nqt = (lq + 255) // 256
    kept = torch.empty(nqt, dtype=torch.int32, device=q_pos.device)
    masked = torch.empty(nqt, dtype=torch.int32, device=q_pos.device)
    ext = None if kw_lo is None and kw_hi is None else _win_ext(0, kw_lo, kw_hi)
    _check(load().cp_ring_attn_tile_census(cp_size, lq, _ptr(q_pos), _ptr(ring_pos), int(bool(causal)),
                                           None if ext is None else ctypes.byref(ext), _ptr(kept), _ptr(masked),
                                           _stream(stream)), "cp_ring_attn_tile_census")
    return kept, masked
