"""Kimi Delta Attention (KDA) mixer hot path for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libkda.so`` (C ABI declared in ``include/kda.h``).  The
functions here only marshal torch tensors into pointers and sizes; every step of the
mixer runs in the library's HIP kernels.  PyTorch provides device memory and streams.
There is no CPU fallback: if the library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

__all__ = ["KdaConfig", "kda_decode_step", "kda_decode_step_slots", "kda_decode_multi", "kda_decode_multi_slots",
           "kda_prefill", "kda_prefill_gate_proj", "kda_prefill_noalloc", "kda_prefill_workspace_bytes",
           "kda_state_copy", "kda_test_split_carry", "kda_test_pipeline", "KdaError",
           "lib", "LIB_PATH", "EXPORTED_SYMBOLS", "PREFILL_AUTO", "PREFILL_FUSED", "PREFILL_CHUNKED",
           "PRECISION_STANDARD", "PRECISION_HIGH", "MULTI_BLOCK", "MULTI_SEQUENTIAL"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")
EXPORTED_SYMBOLS = ("kda_config_default", "kda_decode_step", "kda_decode_step_slots", "kda_decode_multi",
                    "kda_decode_multi_slots", "kda_prefill", "kda_prefill_gate_proj", "kda_prefill_noalloc",
                    "kda_prefill_workspace_bytes",
                    "kda_state_copy", "kda_test_split_carry", "kda_test_pipeline", "kda_status_str",
                    "kda_abi_version")
ABI_VERSION = 11
HEAD_DIM = 128
CONV = 4
RANK = 128  # rank of the low-rank decay projection (kda_prefill_gate_proj)


class _CConfig(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("conv_size", ctypes.c_int32),
        ("gate_lower_bound", ctypes.c_float),
        ("l2_eps", ctypes.c_float),
        ("rms_eps", ctypes.c_float),
        ("q_scale", ctypes.c_float),
        ("prefill_path", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("precision", ctypes.c_int32),
        ("decode_multi_form", ctypes.c_int32),
    ]

# kda_config.prefill_path values
PREFILL_AUTO = 0     # the layout an estimate of both times predicts faster
PREFILL_FUSED = 1    # one workgroup per (sequence, head) over all chunks; no workspace
PREFILL_CHUNKED = 2  # chunk records in parallel, then the carry; needs a workspace
# kda_config.precision values (kda_prefill)
PRECISION_STANDARD = 0  # bf16 MFMA operands, the decisive ones split hi + lo
PRECISION_HIGH = 1      # every MFMA operand of the chunk algebra split hi + lo
# kda_config.decode_multi_form values (kda_decode_multi)
MULTI_BLOCK = 0       # blocks of eight tokens in the chunk form; fp32 rounding of single steps
MULTI_SEQUENTIAL = 1  # token by token: the bits of the same number of single steps


@dataclass
class KdaConfig:
    num_heads: int = 96
    head_dim: int = HEAD_DIM
    conv_size: int = CONV
    gate_lower_bound: float = -5.0
    l2_eps: float = 1e-6
    rms_eps: float = 1e-5
    q_scale: float = 0.0  # <= 0 selects head_dim ** -0.5
    prefill_path: int = PREFILL_AUTO
    out_dtype: torch.dtype = torch.float32  # or torch.bfloat16: element type of the outputs
    precision: int = PRECISION_STANDARD     # kda_prefill operand precision
    decode_multi_form: int = MULTI_BLOCK    # kda_decode_multi evaluation form

    def _c(self) -> _CConfig:
        if self.out_dtype not in (torch.float32, torch.bfloat16):
            raise ValueError(f"out_dtype must be torch.float32 or torch.bfloat16, not {self.out_dtype}")
        return _CConfig(self.num_heads, self.head_dim, self.conv_size, self.gate_lower_bound, self.l2_eps,
                        self.rms_eps, self.q_scale, self.prefill_path, 1 if self.out_dtype == torch.bfloat16 else 0,
                        self.precision, self.decode_multi_form)


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {_lib.kda_status_str(status).decode()} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python gated_delta_rule_31_amd/build.py` "
                          "or `python __graft_entry__.py build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, fp = ctypes.c_void_p, ctypes.c_void_p
    L.kda_config_default.restype = _CConfig
    L.kda_config_default.argtypes = []
    L.kda_decode_step.restype = ctypes.c_int
    i64 = ctypes.c_int64
    L.kda_decode_step.argtypes = [ctypes.POINTER(_CConfig), ctypes.c_int32] + [fp] * 3 + [i64] + [fp] * 10 + [vp]
    L.kda_decode_step_slots.restype = ctypes.c_int
    L.kda_decode_step_slots.argtypes = ([ctypes.POINTER(_CConfig), ctypes.c_int32, vp, ctypes.c_int32] + [fp] * 3 +
                                        [i64] + [fp] * 10 + [vp])
    L.kda_decode_multi.restype = ctypes.c_int
    L.kda_decode_multi.argtypes = ([ctypes.POINTER(_CConfig), ctypes.c_int32, ctypes.c_int32, vp] + [fp] * 3 +
                                   [i64] + [fp] * 12 + [vp])
    L.kda_decode_multi_slots.restype = ctypes.c_int
    L.kda_decode_multi_slots.argtypes = ([ctypes.POINTER(_CConfig), ctypes.c_int32, ctypes.c_int32, vp, vp,
                                          ctypes.c_int32] + [fp] * 3 + [i64] + [fp] * 12 + [vp])
    L.kda_prefill.restype = ctypes.c_int
    L.kda_prefill.argtypes = ([ctypes.POINTER(_CConfig), ctypes.c_int32, ctypes.c_int32, vp] + [vp] * 3 + [i64] +
                              [vp] * 3 + [fp] * 4 + [fp] * 2 + [fp] * 3 + [vp, ctypes.c_size_t, vp])
    L.kda_prefill_gate_proj.restype = ctypes.c_int
    L.kda_prefill_gate_proj.argtypes = ([ctypes.POINTER(_CConfig), ctypes.c_int32, ctypes.c_int32, vp] + [vp] * 3 +
                                        [i64] + [vp] * 4 + [fp] * 4 + [fp] * 2 + [fp] * 3 +
                                        [vp, ctypes.c_size_t, vp])
    L.kda_prefill_noalloc.restype = ctypes.c_int
    L.kda_prefill_noalloc.argtypes = ([ctypes.POINTER(_CConfig), ctypes.c_int32, ctypes.c_int32, vp] + [vp] * 3 +
                                      [i64] + [vp] * 3 + [fp] * 4 + [fp] * 2 + [fp] * 3 + [vp])
    L.kda_prefill_workspace_bytes.restype = ctypes.c_size_t
    L.kda_prefill_workspace_bytes.argtypes = [ctypes.POINTER(_CConfig), ctypes.c_int32, ctypes.c_int32]
    L.kda_state_copy.restype = ctypes.c_int
    L.kda_state_copy.argtypes = ([ctypes.POINTER(_CConfig), ctypes.c_int32, vp, vp, ctypes.c_int32, vp, vp, vp,
                                  ctypes.c_int32, vp, vp])
    L.kda_test_split_carry.restype = None
    L.kda_test_split_carry.argtypes = [ctypes.c_int32, ctypes.c_int32]
    L.kda_test_pipeline.restype = None
    L.kda_test_pipeline.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    L.kda_status_str.restype = ctypes.c_char_p
    L.kda_status_str.argtypes = [ctypes.c_int]
    L.kda_abi_version.restype = ctypes.c_int32
    L.kda_abi_version.argtypes = []
    if L.kda_abi_version() != ABI_VERSION:
        raise ImportError(f"libkda.so ABI {L.kda_abi_version()} != binding ABI {ABI_VERSION}")
    return L


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _ptr(t: torch.Tensor | None, dtype: torch.dtype, shape: tuple, name: str):
    """Pointer of a dense device tensor of the given dtype and shape (None -> NULL)."""
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _rows_ptr(t: torch.Tensor, dtype: torch.dtype, shape: tuple, name: str):
    """Pointer and row stride (elements) of a q/k/v tensor: the given shape, channels
    contiguous, and its token rows (every index but the last, flattened) equally spaced,
    e.g. a slice of the last dimension of a fused [..., 3*H*D] projection output."""
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    if t.numel() == 0:
        return None, 0
    if t.stride()[-1] != 1 and t.shape[-1] > 1:
        raise ValueError(f"{name}: channels must be contiguous")
    # the row dimensions (all but the last) that hold more than one index, innermost first
    dims = [(t.shape[d], t.stride(d)) for d in range(t.dim() - 2, -1, -1) if t.shape[d] > 1]
    ld = dims[0][1] if dims else shape[-1]
    span = ld
    for n, st in dims:
        if st != span:
            raise ValueError(f"{name}: token rows must be equally spaced")
        span = st * n
    return ctypes.c_void_p(t.data_ptr()), int(ld)


def _qkv(q, k, v, dtype, shape):
    """Pointers of q, k, v and their common row stride (0 when all are dense)."""
    (pq, lq), (pk, lk), (pv, lv) = (_rows_ptr(x, dtype, shape, n) for x, n in ((q, "q"), (k, "k"), (v, "v")))
    lds = {l for l, p in ((lq, pq), (lk, pk), (lv, pv)) if p is not None}
    if len(lds) > 1:
        raise ValueError(f"q, k, v must share one row stride, got {sorted(lds)}")
    ld = lds.pop() if lds else 0
    return pq, pk, pv, (0 if ld == shape[-1] else ld)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def kda_decode_step(cfg: KdaConfig, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state, conv_state,
                    out=None, stream=None) -> torch.Tensor:
    """One token per sequence.  q,k,v,z,g: [B, H*D] fp32 (q, k, v may be row-strided views,
    e.g. of one [B, 3*H*D] projection output); b: [B, H]; state [B,H,D,D] and
    conv_state [B,3*H*D,3] are updated in place.  Returns out [B, H*D] (cfg.out_dtype)."""
    H, D = cfg.num_heads, cfg.head_dim
    B = q.shape[0]
    HD = H * D
    f32 = torch.float32
    if out is None:
        out = torch.empty((B, HD), dtype=cfg.out_dtype, device=q.device)
    args = [
        *_qkv(q, k, v, f32, (B, HD)),
        _ptr(z, f32, (B, HD), "z"), _ptr(b, f32, (B, H), "b"), _ptr(g, f32, (B, HD), "g"),
        _ptr(conv_w, f32, (3 * HD, CONV), "conv_w"), _ptr(A_log, f32, (H,), "A_log"),
        _ptr(dt_bias, f32, (HD,), "dt_bias"), _ptr(norm_w, f32, (D,), "norm_w"),
        _ptr(state, f32, (B, H, D, D), "state"), _ptr(conv_state, f32, (B, 3 * HD, CONV - 1), "conv_state"),
        _ptr(out, cfg.out_dtype, (B, HD), "out"),
    ]
    c = cfg._c()
    st = _lib.kda_decode_step(ctypes.byref(c), B, *args, _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_decode_step")
    return out


def kda_decode_step_slots(cfg: KdaConfig, slots, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state_pool,
                          conv_pool, out=None, stream=None) -> torch.Tensor:
    """One token per batch row against states held in a pool: row r advances pool entry
    ``slots[r]`` (int32 [B] on the GPU) of state_pool [P,H,D,D] and conv_pool
    [P,3*H*D,3], in place; rows whose slot lies outside [0, P) are skipped and their
    output rows left as they were.  q,k,v,z,g: [B, H*D] fp32; b: [B, H].  Returns out
    [B, H*D] (cfg.out_dtype)."""
    H, D = cfg.num_heads, cfg.head_dim
    B = q.shape[0]
    P = state_pool.shape[0]
    HD = H * D
    f32 = torch.float32
    if out is None:
        out = torch.empty((B, HD), dtype=cfg.out_dtype, device=q.device)
    args = [
        *_qkv(q, k, v, f32, (B, HD)),
        _ptr(z, f32, (B, HD), "z"), _ptr(b, f32, (B, H), "b"), _ptr(g, f32, (B, HD), "g"),
        _ptr(conv_w, f32, (3 * HD, CONV), "conv_w"), _ptr(A_log, f32, (H,), "A_log"),
        _ptr(dt_bias, f32, (HD,), "dt_bias"), _ptr(norm_w, f32, (D,), "norm_w"),
        _ptr(state_pool, f32, (P, H, D, D), "state_pool"),
        _ptr(conv_pool, f32, (P, 3 * HD, CONV - 1), "conv_pool"),
        _ptr(out, cfg.out_dtype, (B, HD), "out"),
    ]
    c = cfg._c()
    st = _lib.kda_decode_step_slots(ctypes.byref(c), B, _ptr(slots, torch.int32, (B,), "slots"), P, *args,
                                    _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_decode_step_slots")
    return out


def _decode_multi(cfg, slots, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state_in, conv_state_in, state_out,
                  conv_state_out, n_tokens, out, stream, where):
    H, D = cfg.num_heads, cfg.head_dim
    B, T = q.shape[0], q.shape[1]
    P = B if slots is None else state_in.shape[0]
    HD = H * D
    f32 = torch.float32
    if state_out is None:
        state_out = state_in
    if conv_state_out is None:
        conv_state_out = conv_state_in
    if out is None:
        out = torch.empty((B, T, HD), dtype=cfg.out_dtype, device=q.device)
    args = [
        *_qkv(q, k, v, f32, (B, T, HD)),
        _ptr(z, f32, (B, T, HD), "z"), _ptr(b, f32, (B, T, H), "b"), _ptr(g, f32, (B, T, HD), "g"),
        _ptr(conv_w, f32, (3 * HD, CONV), "conv_w"), _ptr(A_log, f32, (H,), "A_log"),
        _ptr(dt_bias, f32, (HD,), "dt_bias"), _ptr(norm_w, f32, (D,), "norm_w"),
        _ptr(state_in, f32, (P, H, D, D), "state_in"), _ptr(state_out, f32, (P, H, D, D), "state_out"),
        _ptr(conv_state_in, f32, (P, 3 * HD, CONV - 1), "conv_state_in"),
        _ptr(conv_state_out, f32, (P, 3 * HD, CONV - 1), "conv_state_out"),
        _ptr(out, cfg.out_dtype, (B, T, HD), "out"),
    ]
    c = cfg._c()
    nt = _ptr(n_tokens, torch.int32, (B,), "n_tokens")
    if slots is None:
        st = _lib.kda_decode_multi(ctypes.byref(c), B, T, nt, *args, _stream(stream))
    else:
        st = _lib.kda_decode_multi_slots(ctypes.byref(c), B, T, nt, _ptr(slots, torch.int32, (B,), "slots"), P,
                                         *args, _stream(stream))
    if st != 0:
        raise KdaError(st, where)
    return out


def kda_decode_multi(cfg: KdaConfig, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state_in, conv_state_in,
                     state_out=None, conv_state_out=None, n_tokens=None, out=None, stream=None) -> torch.Tensor:
    """Up to T tokens per sequence in one call.  q,k,v,z,g: [B, T, H*D] fp32; b: [B, T, H];
    n_tokens: int32 [B] on the GPU or None (T each).  The states are written to
    ``state_out`` / ``conv_state_out`` (default: in place).  Returns out [B, T, H*D] (cfg.out_dtype)
    (rows of tokens past n_tokens[b] are left as they were)."""
    return _decode_multi(cfg, None, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state_in, conv_state_in,
                         state_out, conv_state_out, n_tokens, out, stream, "kda_decode_multi")


def kda_decode_multi_slots(cfg: KdaConfig, slots, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state_in,
                           conv_state_in, state_out=None, conv_state_out=None, n_tokens=None, out=None,
                           stream=None) -> torch.Tensor:
    """kda_decode_multi over state pools: batch row r works on pool entry ``slots[r]``
    (int32 [B] on the GPU) of state_in [P,H,D,D] / conv_state_in [P,3*H*D,3] and writes it
    to the same entry of state_out / conv_state_out (default: in place); rows whose slot
    lies outside [0, P) are skipped."""
    return _decode_multi(cfg, slots, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state_in, conv_state_in,
                         state_out, conv_state_out, n_tokens, out, stream, "kda_decode_multi_slots")


def kda_prefill_workspace_bytes(cfg: KdaConfig, num_seqs: int, total_tokens: int) -> int:
    c = cfg._c()
    return int(_lib.kda_prefill_workspace_bytes(ctypes.byref(c), num_seqs, total_tokens))


def _prefill_args(cfg, cu_seqlens, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, initial_state,
                  initial_conv_state, out, final_state, final_conv_state):
    H, D = cfg.num_heads, cfg.head_dim
    B = cu_seqlens.shape[0] - 1
    N = q.shape[0]
    HD = H * D
    f32, bf = torch.float32, torch.bfloat16
    dev = q.device
    if out is None:
        out = torch.empty((N, HD), dtype=cfg.out_dtype, device=dev)
    if final_state is None:
        final_state = torch.empty((B, H, D, D), dtype=f32, device=dev)
    if final_conv_state is None:
        final_conv_state = torch.empty((B, 3 * HD, CONV - 1), dtype=f32, device=dev)
    args = [
        _ptr(cu_seqlens, torch.int32, (B + 1,), "cu_seqlens"),
        *_qkv(q, k, v, bf, (N, HD)),
        _ptr(z, bf, (N, HD), "z"), _ptr(b, bf, (N, H), "b"), _ptr(g, bf, (N, HD), "g"),
        _ptr(conv_w, f32, (3 * HD, CONV), "conv_w"), _ptr(A_log, f32, (H,), "A_log"),
        _ptr(dt_bias, f32, (HD,), "dt_bias"), _ptr(norm_w, f32, (D,), "norm_w"),
        _ptr(initial_state, f32, (B, H, D, D), "initial_state"),
        _ptr(initial_conv_state, f32, (B, 3 * HD, CONV - 1), "initial_conv_state"),
        _ptr(out, cfg.out_dtype, (N, HD), "out"), _ptr(final_state, f32, (B, H, D, D), "final_state"),
        _ptr(final_conv_state, f32, (B, 3 * HD, CONV - 1), "final_conv_state"),
    ]
    return B, N, args, out, final_state, final_conv_state


def kda_prefill(cfg: KdaConfig, cu_seqlens, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w,
                initial_state=None, initial_conv_state=None, out=None, final_state=None,
                final_conv_state=None, workspace=None, stream=None):
    """Varlen prefill.  cu_seqlens: int32 [B+1] on the GPU; q,k,v,z,g: [N, H*D] bf16 (q, k,
    v may be row-strided views, e.g. of one [N, 3*H*D] projection output); b: [N, H] bf16.
    Returns (out [N, H*D] (cfg.out_dtype), final_state, final_conv_state).
    ``final_state`` may be ``initial_state`` (in-place carry)."""
    B, N, args, out, final_state, final_conv_state = _prefill_args(
        cfg, cu_seqlens, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, initial_state, initial_conv_state, out,
        final_state, final_conv_state)
    ws_bytes = kda_prefill_workspace_bytes(cfg, B, N)
    own_ws = bool(ws_bytes) and workspace is None
    if own_ws:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    ws = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    c = cfg._c()
    st = _lib.kda_prefill(ctypes.byref(c), B, N, *args, ws, ctypes.c_size_t(ws_bytes), _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_prefill")
    if own_ws and stream is not None:
        # the workspace is released when this returns: keep the allocator from handing it
        # out again before the kernels queued on ``stream`` are done with it
        workspace.record_stream(stream)
    return out, final_state, final_conv_state


def kda_prefill_gate_proj(cfg: KdaConfig, cu_seqlens, q, k, v, f, w_fb, b, g, conv_w, A_log, dt_bias, norm_w,
                          initial_state=None, initial_conv_state=None, out=None, final_state=None,
                          final_conv_state=None, workspace=None, stream=None):
    """kda_prefill with the decay logits formed inside the library: f = W_fa x [N, 128]
    bf16 (shared by the heads) and W_fb [H*D, 128] bf16 instead of z.  Returns (out,
    final_state, final_conv_state)."""
    H, D = cfg.num_heads, cfg.head_dim
    bf = torch.bfloat16
    B, N, args, out, final_state, final_conv_state = _prefill_args(
        cfg, cu_seqlens, q, k, v, None, b, g, conv_w, A_log, dt_bias, norm_w, initial_state, initial_conv_state,
        out, final_state, final_conv_state)
    # args: cu, q, k, v, stride, z (NULL), b, ... -> cu, q, k, v, stride, f, w_fb, b, ...
    fa = [_ptr(f, bf, (N, RANK), "f"), _ptr(w_fb, bf, (H * D, RANK), "w_fb")]
    args = args[:5] + fa + args[6:]
    ws_bytes = kda_prefill_workspace_bytes(cfg, B, N)
    own_ws = bool(ws_bytes) and workspace is None
    if own_ws:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    ws = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    c = cfg._c()
    st = _lib.kda_prefill_gate_proj(ctypes.byref(c), B, N, *args, ws, ctypes.c_size_t(ws_bytes), _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_prefill_gate_proj")
    if own_ws and stream is not None:
        workspace.record_stream(stream)
    return out, final_state, final_conv_state


def kda_prefill_noalloc(cfg: KdaConfig, cu_seqlens, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w,
                        initial_state=None, initial_conv_state=None, out=None, final_state=None,
                        final_conv_state=None, stream=None):
    """kda_prefill with the chunked layout's workspace in the library's per-device
    scratch array (no workspace argument; the library allocates nothing).  Pass ``out``,
    ``final_state`` and ``final_conv_state`` to keep this wrapper from allocating them."""
    B, N, args, out, final_state, final_conv_state = _prefill_args(
        cfg, cu_seqlens, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, initial_state, initial_conv_state, out,
        final_state, final_conv_state)
    c = cfg._c()
    st = _lib.kda_prefill_noalloc(ctypes.byref(c), B, N, *args, _stream(stream))
    if st != 0:
        raise KdaError(st, "kda_prefill_noalloc")
    return out, final_state, final_conv_state


def kda_state_copy(cfg: KdaConfig, src_state, src_conv, src_slots, dst_state, dst_conv, dst_slots,
                   stream=None) -> None:
    """Copy entry src_slots[i] of (src_state [Ps,H,D,D], src_conv [Ps,3*H*D,3]) to entry
    dst_slots[i] of (dst_state, dst_conv), in order.  The buffers are GPU tensors or host
    tensors (pinned ones make the copies asynchronous on the stream); the slot lists are
    host sequences of ints."""
    H, D = cfg.num_heads, cfg.head_dim
    f32 = torch.float32

    def buf(t, shape, name):
        if t.dtype != f32:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {f32}")
        if tuple(t.shape[1:]) != shape:
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected [entries, {', '.join(map(str, shape))}]")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
        return ctypes.c_void_p(t.data_ptr()) if t.numel() else None

    ss = np.ascontiguousarray(np.asarray(src_slots, dtype=np.int32).reshape(-1))
    ds = np.ascontiguousarray(np.asarray(dst_slots, dtype=np.int32).reshape(-1))
    if ss.shape != ds.shape:
        raise ValueError(f"src_slots and dst_slots differ in length: {ss.shape[0]} vs {ds.shape[0]}")
    if src_state.shape[0] != src_conv.shape[0] or dst_state.shape[0] != dst_conv.shape[0]:
        raise ValueError("state and conv buffers of one side must hold the same number of entries")
    if stream is None and (src_state.is_cuda or dst_state.is_cuda):
        stream = torch.cuda.current_stream()
    c = cfg._c()
    st = _lib.kda_state_copy(ctypes.byref(c), int(ss.shape[0]),
                             buf(src_state, (H, D, D), "src_state"), buf(src_conv, (3 * H * D, CONV - 1), "src_conv"),
                             int(src_state.shape[0]), ss.ctypes.data_as(ctypes.c_void_p),
                             buf(dst_state, (H, D, D), "dst_state"), buf(dst_conv, (3 * H * D, CONV - 1), "dst_conv"),
                             int(dst_state.shape[0]), ds.ctypes.data_as(ctypes.c_void_p),
                             ctypes.c_void_p(stream.cuda_stream) if stream is not None else None)
    if st != 0:
        raise KdaError(st, "kda_state_copy")


def kda_test_split_carry(publish: bool, max_polls: int = 0) -> None:
    """Test hook of the chunked prefill's two-workgroup carry (kda.h): publish=False makes
    its workgroups skip publishing their row sums, so that every wait times out after
    max_polls polls (0: the library's bound) and the outputs become NaN; the states stay
    exact.  Process-wide; kda_test_split_carry(True) restores normal operation."""
    _lib.kda_test_split_carry(1 if publish else 0, int(max_polls))


def kda_test_pipeline(mode: int = 0, publish: bool = True, max_polls: int = 0) -> None:
    """Test hook of the chunked prefill whose carries run in the chunk workgroups' launch
    (kda.h, kda_test_pipeline): mode 0 the library's choice, 1 never that form, 2 wherever
    it can run; publish=False makes every carry's wait for a record time out (NaN outputs
    and NaN final states).  Process-wide; kda_test_pipeline() restores normal operation."""
    _lib.kda_test_pipeline(int(mode), 1 if publish else 0, int(max_polls))
