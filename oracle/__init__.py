"""fp64 CPU oracle of the Kimi Delta Attention (KDA) mixer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product path (``gated_delta_rule_31_amd``) never does,
and this package imports nothing from it.

The arithmetic lives in ``kda_oracle.c`` (plain fp64 C, token by token, one
(sequence, head) at a time; page "colibri/c/kimi_k3.c", header comment "KDA per-head
recurrence").  This module only compiles it, marshals numpy arrays into its job
structs and slices the library's tensor layouts into per-(sequence, head) views:

* pre-conv q/k/v, z, g: ``[N, H*D]``; channel ``h*D + i`` of head ``h``.
* beta logits b: ``[N, H]``.
* conv weights: ``[3*H*D, K]``, the q block, then k, then v; taps oldest first.
* state: ``[B, H, D, D]``, ``S[key][value]``.
* conv state: ``[B, 3*H*D, K-1]``, the K-1 previous pre-conv inputs, oldest first.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)


class _Params(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int),
        ("conv_size", ctypes.c_int),
        ("gate_lower_bound", ctypes.c_double),
        ("l2_eps", ctypes.c_double),
        ("rms_eps", ctypes.c_double),
        ("q_scale", ctypes.c_double),
        ("norm_w", _dp),
    ]


class _Job(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int),
        ("xq", _dp), ("xk", _dp), ("xv", _dp),
        ("z", _dp), ("g", _dp), ("b", _dp),
        ("ld_x", ctypes.c_ssize_t), ("ld_z", ctypes.c_ssize_t), ("ld_g", ctypes.c_ssize_t),
        ("ld_b", ctypes.c_ssize_t), ("ld_out", ctypes.c_ssize_t),
        ("wq", _dp), ("wk", _dp), ("wv", _dp),
        ("dt_bias", _dp),
        ("A_log", ctypes.c_double),
        ("S", _dp),
        ("cq", _dp), ("ck", _dp), ("cv", _dp),
        ("out", _dp),
    ]


def build(force: bool = False) -> str:
    """Compile kda_oracle.c with gcc into libkda_oracle.so (next to the source)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.kda_oracle_sigmoid.restype = ctypes.c_double
        L.kda_oracle_sigmoid.argtypes = [ctypes.c_double]
        L.kda_oracle_silu.restype = ctypes.c_double
        L.kda_oracle_silu.argtypes = [ctypes.c_double]
        L.kda_oracle_conv_step.restype = ctypes.c_double
        L.kda_oracle_conv_step.argtypes = [ctypes.c_int, _dp, _dp, ctypes.c_double]
        L.kda_oracle_rmsnorm_gate.restype = None
        L.kda_oracle_rmsnorm_gate.argtypes = [ctypes.c_int, _dp, _dp, _dp, ctypes.c_double, _dp]
        L.kda_oracle_core_step.restype = None
        L.kda_oracle_core_step.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp, _dp,
                                           ctypes.c_double, _dp]
        L.kda_oracle_run_jobs.restype = ctypes.c_int
        L.kda_oracle_run_jobs.argtypes = [ctypes.POINTER(_Params), ctypes.POINTER(_Job), ctypes.c_int,
                                          ctypes.c_int]
        assert L.kda_oracle_job_size() == ctypes.sizeof(_Job), "job struct layout mismatch"
        assert L.kda_oracle_params_size() == ctypes.sizeof(_Params), "params struct layout mismatch"
        _lib = L
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_dp)


# ---------------------------------------------------------------------------------
# Single steps, exported so that the tests can pin each one on its own.
# ---------------------------------------------------------------------------------

def sigmoid(x: float) -> float:
    return lib().kda_oracle_sigmoid(float(x))


def silu(x: float) -> float:
    return lib().kda_oracle_silu(float(x))


def conv_sequence(w, window, x):
    """ShortConv of one channel over a token sequence.  ``w``: K taps (oldest first);
    ``window``: the K-1 previous inputs (oldest first); ``x``: [T].  Returns (y, window')."""
    w = _f64(w)
    win = _f64(window).copy()
    y = np.empty(len(x))
    for t, xt in enumerate(np.asarray(x, dtype=np.float64)):
        y[t] = lib().kda_oracle_conv_step(len(w), _ptr(w), _ptr(win), float(xt))
    return y, win


def rmsnorm_gate(o, g, w, eps: float):
    o, g, w = _f64(o), _f64(g), _f64(w)
    out = np.empty_like(o)
    lib().kda_oracle_rmsnorm_gate(len(o), _ptr(o), _ptr(g), _ptr(w), float(eps), _ptr(out))
    return out


def core_step(S, q, k, v, alpha, beta: float):
    """One token of the recurrence with explicit gates.  Returns (S', o)."""
    S = _f64(S).copy()
    dk, dv = S.shape
    q, k, v, alpha = _f64(q), _f64(k), _f64(v), _f64(alpha)
    assert q.shape == (dk,) and k.shape == (dk,) and alpha.shape == (dk,) and v.shape == (dv,)
    o = np.empty(dv)
    lib().kda_oracle_core_step(dk, dv, _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), float(beta), _ptr(o))
    return S, o


# ---------------------------------------------------------------------------------
# The whole mixer over (sequence, head) pairs, in the library's tensor layouts.
# ---------------------------------------------------------------------------------

@dataclass
class MixerConfig:
    head_dim: int = 128
    conv_size: int = 4
    gate_lower_bound: float = -5.0
    l2_eps: float = 1e-6
    rms_eps: float = 1e-5
    q_scale: float = 0.0  # 0 => head_dim ** -0.5


@dataclass
class PairResult:
    out: np.ndarray         # [T, D]
    state: np.ndarray       # [D, D] final S
    conv_state: np.ndarray  # [3, D, K-1] final windows of the q, k, v channels


def forward(cfg: MixerConfig, cu_seqlens, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w,
            state=None, conv_state=None, pairs=None, threads: int | None = None, decode=None, gate_proj=None):
    """Run the oracle for every (sequence, head) in ``pairs`` (default: all).

    Activations may be any float dtype, or an encoding that ``decode`` turns into exact
    float values slice by slice (e.g. bf16 bit patterns); only the slices the pairs touch
    are converted to fp64.  ``state`` is ``[B, H, D, D]`` or None (zeros); ``conv_state``
    ``[B, 3*H*D, K-1]`` or None (zeros).  Returns ``{(s, h): PairResult}``.

    ``gate_proj = (f, w_fb)`` replaces ``z`` (pass None): the decay logits are the second
    factor of the low-rank decay projection applied to the first one's output, z = W_fb f
    per token (page "colibri/c/kimi_k3.c", header comment "KDA per-head recurrence": the
    gate's argument W_fb(W_fa x) + dt_bias; the ``Kda`` struct's ``fa, fb``), with
    ``f = W_fa x`` of shape ``[N, R]`` (shared by the heads) and ``w_fb`` of shape
    ``[H*D, R]``; channel i of head h takes row h*D + i.  Computed in fp64 from the
    (decoded) values, as one matrix product per (sequence, head).
    """
    dec = decode if decode is not None else (lambda x: x)
    D, K = cfg.head_dim, cfg.conv_size
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = len(cu) - 1
    HD = q.shape[1]
    H = HD // D
    assert HD == H * D and b.shape[1] == H and conv_w.shape == (3 * HD, K)
    if gate_proj is not None:
        assert z is None, "pass either z or gate_proj"
        f_lr, w_fb = gate_proj
        assert w_fb.shape[0] == HD and f_lr.shape[0] == q.shape[0] and f_lr.shape[1] == w_fb.shape[1]
    if pairs is None:
        pairs = [(s, h) for s in range(B) for h in range(H)]
    norm_w64 = _f64(norm_w)
    params = _Params(D, K, cfg.gate_lower_bound, cfg.l2_eps, cfg.rms_eps, cfg.q_scale, _ptr(norm_w64))

    keep = []  # holds every fp64 buffer the jobs point into
    jobs = (_Job * len(pairs))()
    pending = []
    for j, (s, h) in enumerate(pairs):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        cs = slice(h * D, (h + 1) * D)
        xq, xk, xv = _f64(dec(q[t0:t1, cs])), _f64(dec(k[t0:t1, cs])), _f64(dec(v[t0:t1, cs]))
        if gate_proj is None:
            zz = _f64(dec(z[t0:t1, cs]))
        else:  # z_t = W_fb f_t for the head's D rows of W_fb
            zz = np.ascontiguousarray(_f64(dec(f_lr[t0:t1])) @ _f64(dec(w_fb[h * D:(h + 1) * D])).T)
        gg = _f64(dec(g[t0:t1, cs]))
        bb = _f64(dec(b[t0:t1, h]))
        wq = _f64(conv_w[0 * HD + h * D:0 * HD + (h + 1) * D])
        wk = _f64(conv_w[1 * HD + h * D:1 * HD + (h + 1) * D])
        wv = _f64(conv_w[2 * HD + h * D:2 * HD + (h + 1) * D])
        dtb = _f64(dt_bias[cs])
        S = np.zeros((D, D)) if state is None else _f64(state[s, h]).copy()
        if conv_state is None:
            cq, ck, cv = (np.zeros((D, K - 1)) for _ in range(3))
        else:
            cq = _f64(conv_state[s, 0 * HD + h * D:0 * HD + (h + 1) * D]).copy()
            ck = _f64(conv_state[s, 1 * HD + h * D:1 * HD + (h + 1) * D]).copy()
            cv = _f64(conv_state[s, 2 * HD + h * D:2 * HD + (h + 1) * D]).copy()
        out = np.zeros((t1 - t0, D))
        # zero-length sequences still need valid pointers
        if t1 == t0:
            xq = xk = xv = zz = gg = np.zeros((1, D))
            bb = np.zeros(1)
        keep += [xq, xk, xv, zz, gg, bb, wq, wk, wv, dtb, S, cq, ck, cv, out]
        jb = jobs[j]
        jb.T = t1 - t0
        jb.xq, jb.xk, jb.xv = _ptr(xq), _ptr(xk), _ptr(xv)
        jb.z, jb.g, jb.b = _ptr(zz), _ptr(gg), _ptr(bb)
        jb.ld_x = jb.ld_z = jb.ld_g = jb.ld_out = D
        jb.ld_b = 1
        jb.wq, jb.wk, jb.wv = _ptr(wq), _ptr(wk), _ptr(wv)
        jb.dt_bias = _ptr(dtb)
        jb.A_log = float(A_log[h])
        jb.S = _ptr(S)
        jb.cq, jb.ck, jb.cv = _ptr(cq), _ptr(ck), _ptr(cv)
        jb.out = _ptr(out)
        pending.append(((s, h), out, S, cq, ck, cv))
    n_threads = threads or len(os.sched_getaffinity(0))
    rc = lib().kda_oracle_run_jobs(ctypes.byref(params), jobs, len(pairs), n_threads)
    if rc != 0:
        raise RuntimeError("oracle rejected its arguments")
    del keep
    return {key: PairResult(out=out, state=S, conv_state=np.stack([cq, ck, cv]))
            for key, out, S, cq, ck, cv in pending}
