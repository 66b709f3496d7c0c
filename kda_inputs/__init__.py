"""Seeded synthetic inputs for the KDA mixer's decode and prefill workloads.

Shared by the oracle side and the GPU side of the tests and by the bench.  It draws
random numbers and converts dtypes (fp32 -> bf16 with round-to-nearest-even), and holds
none of the mixer's arithmetic.

Recipe (every case):

* Each named tensor has its own numpy ``default_rng`` streams, seeded with
  ``[case_seed, stream_id, block]`` where ``stream_id`` is a fixed number per tensor
  (and per decode step) and ``block`` numbers blocks of about 2^18 elements (whole rows
  of the last dimension), so any tensor can be regenerated on its own, in parallel.
* ``N(0, s)`` means mean 0 and *standard deviation* s; draws are float32.
* ``U(a, b)``: float32 uniform on [a, b).
* Pre-conv q/k/v, decay logits z, beta logits b and output-gate logits g are N(0, 1);
  ShortConv4 weights N(0, 0.5); dt_bias U(-1, 1); A_log U(-2, 1); RMSNorm weight 1.0;
  states N(0, 0.05); conv states N(0, 1).
* bf16 cases round the activations (q, k, v, z, b, g) to bf16; parameters and states
  stay fp32.

Layouts are those of the C-ABI library: activations ``[N, H*D]`` (head-major channels),
beta logits ``[N, H]``, conv weights ``[3*H*D, 4]`` (q block, k block, v block),
states ``[B, H, D, D]``, conv states ``[B, 3*H*D, 3]``.
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

D = 128   # head dim
K = 4     # ShortConv taps

# stream ids
_S_STATE, _S_CONV_STATE, _S_CONV_W, _S_DT_BIAS, _S_A_LOG, _S_LENS = 1, 2, 3, 4, 5, 6
_S_F, _S_W_FB = 7, 8
_S_Q, _S_K, _S_V, _S_Z, _S_B, _S_G = 10, 11, 12, 13, 14, 15
_STEP_STRIDE = 100  # decode step i uses stream id  base + STEP_STRIDE * (i + 1)

_BLOCK_ELEMS = 1 << 18  # large tensors are drawn in blocks of about this many elements


def _rng(seed: int, stream: int, block: int | None = None) -> np.random.Generator:
    key = [int(seed), int(stream)] if block is None else [int(seed), int(stream), int(block)]
    return np.random.default_rng(key)


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def normal(seed: int, stream: int, shape, std: float, bf16: bool = False) -> np.ndarray:
    """N(0, std) float32 draws (or their bf16 bit patterns).  The array is cut into rows
    of its last dimension and blocks of ``max(1, 2^18 // last_dim)`` rows; block b comes
    from its own stream [seed, stream, b].  So the result does not depend on how many
    threads draw it, and a prefix of leading rows does not depend on the row count."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16 if bf16 else np.float32)
    flat = out.reshape(-1, shape[-1])
    rows = max(1, _BLOCK_ELEMS // shape[-1])
    nblk = (flat.shape[0] + rows - 1) // rows

    def draw(b):
        blk = flat[b * rows:(b + 1) * rows]
        x = _rng(seed, stream, b).standard_normal(blk.shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        blk[...] = to_bf16_bits(x) if bf16 else x

    if nblk <= 2:
        for b in range(nblk):
            draw(b)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(draw, range(nblk)))
    return out


def uniform(seed: int, stream: int, shape, lo: float, hi: float) -> np.ndarray:
    r = _rng(seed, stream)
    u = r.random(tuple(int(s) for s in shape), dtype=np.float32)
    return (np.float32(lo) + np.float32(hi - lo) * u).astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> their exact fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------------

@dataclass
class Params:
    """Per-layer parameters (fp32)."""
    H: int
    conv_w: np.ndarray   # [3*H*D, 4]
    dt_bias: np.ndarray  # [H*D]
    A_log: np.ndarray    # [H]
    norm_w: np.ndarray   # [D]


def params(seed: int, H: int) -> Params:
    return Params(
        H=H,
        conv_w=normal(seed, _S_CONV_W, (3 * H * D, K), 0.5),
        dt_bias=uniform(seed, _S_DT_BIAS, (H * D,), -1.0, 1.0),
        A_log=uniform(seed, _S_A_LOG, (H,), -2.0, 1.0),
        norm_w=np.ones(D, dtype=np.float32),
    )


@dataclass
class TokenInputs:
    """Per-token activations for N tokens (fp32 values, or bf16 bit patterns)."""
    q: np.ndarray  # [N, H*D]
    k: np.ndarray
    v: np.ndarray
    z: np.ndarray  # [N, H*D] decay logits (before dt_bias)
    b: np.ndarray  # [N, H]   beta logits
    g: np.ndarray  # [N, H*D] output-gate logits

    def as_bf16(self) -> "TokenInputs":
        return TokenInputs(*(to_bf16_bits(a) for a in (self.q, self.k, self.v, self.z, self.b, self.g)))

    def as_f32(self) -> "TokenInputs":
        """bf16 bit patterns -> exact fp32 values (identity for fp32 inputs)."""
        def cv(a):
            return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a
        return TokenInputs(*(cv(a) for a in (self.q, self.k, self.v, self.z, self.b, self.g)))


def token_inputs(seed: int, N: int, H: int, step: int | None = None, bf16: bool = False) -> TokenInputs:
    """Per-token activations; with bf16=True, their bf16 roundings (bit patterns), which
    equal ``token_inputs(...).as_bf16()``."""
    off = 0 if step is None else _STEP_STRIDE * (step + 1)
    return TokenInputs(
        q=normal(seed, _S_Q + off, (N, H * D), 1.0, bf16),
        k=normal(seed, _S_K + off, (N, H * D), 1.0, bf16),
        v=normal(seed, _S_V + off, (N, H * D), 1.0, bf16),
        z=normal(seed, _S_Z + off, (N, H * D), 1.0, bf16),
        b=normal(seed, _S_B + off, (N, H), 1.0, bf16),
        g=normal(seed, _S_G + off, (N, H * D), 1.0, bf16),
    )


# ---------------------------------------------------------------------------------
# Cases
# ---------------------------------------------------------------------------------

@dataclass
class DecodeCase:
    """``n_steps`` consecutive one-token decode steps over B sequences (fp32)."""
    name: str
    seed: int
    B: int
    H: int
    n_steps: int
    params: Params
    state: np.ndarray       # [B, H, D, D] initial
    conv_state: np.ndarray  # [B, 3*H*D, 3] initial
    _steps: list = field(default_factory=list, repr=False)

    def step(self, i: int) -> TokenInputs:
        """Inputs of decode step i: each array has B rows (one token per sequence)."""
        if self._steps and self._steps[i] is not None:
            return self._steps[i]
        return token_inputs(self.seed, self.B, self.H, step=i)


@dataclass
class PrefillCase:
    """A packed varlen batch (bf16 activations, fp32 parameters and states)."""
    name: str
    seed: int
    H: int
    cu_seqlens: np.ndarray                 # int32 [B+1]
    params: Params
    x: TokenInputs                         # bf16 bit patterns
    initial_state: np.ndarray | None       # [B, H, D, D] or None (zeros)
    initial_conv_state: np.ndarray | None  # [B, 3*H*D, 3] or None (zeros)

    @property
    def B(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def N(self) -> int:
        return int(self.cu_seqlens[-1])


def case0_decode() -> DecodeCase:
    """1 sequence, 4 heads, 64 tokens as 64 decode steps from zero state (fp32)."""
    seed, H, T = 0, 4, 64
    x = token_inputs(seed, T, H)
    steps = [TokenInputs(*(a[t:t + 1] for a in (x.q, x.k, x.v, x.z, x.b, x.g))) for t in range(T)]
    return DecodeCase("cfg0-decode", seed, 1, H, T, params(seed, H),
                      np.zeros((1, H, D, D), np.float32), np.zeros((1, 3 * H * D, K - 1), np.float32),
                      _steps=steps)


def case0_prefill() -> PrefillCase:
    """The same 64 tokens as one bf16 prefill sequence."""
    seed, H, T = 0, 4, 64
    return PrefillCase("cfg0-prefill", seed, H, np.array([0, T], np.int32), params(seed, H),
                       token_inputs(seed, T, H).as_bf16(), None, None)


def decode_case(seed: int, B: int, H: int, n_steps: int, name: str) -> DecodeCase:
    return DecodeCase(name, seed, B, H, n_steps, params(seed, H),
                      normal(seed, _S_STATE, (B, H, D, D), 0.05),
                      normal(seed, _S_CONV_STATE, (B, 3 * H * D, K - 1), 1.0))


def case1_decode(B: int = 64, H: int = 96) -> DecodeCase:
    """64 sequences x 96 heads, one decode step against resident fp32 states."""
    return decode_case(1, B, H, 1, "cfg1-decode")


def case4_decode(B: int = 512, H: int = 96, n_steps: int = 32) -> DecodeCase:
    """512 sequences x 96 heads, 32 chained decode steps."""
    return decode_case(4, B, H, n_steps, "cfg4-decode")


def prefill_case(seed: int, H: int, lengths, with_initial: bool, name: str) -> PrefillCase:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    B, N = len(lengths), int(cu[-1])
    st = normal(seed, _S_STATE, (B, H, D, D), 0.05) if with_initial else None
    cst = normal(seed, _S_CONV_STATE, (B, 3 * H * D, K - 1), 1.0) if with_initial else None
    return PrefillCase(name, seed, H, cu, params(seed, H), token_inputs(seed, N, H, bf16=True), st, cst)


def case2_prefill(T: int = 8192, H: int = 96) -> PrefillCase:
    """One long sequence, zero initial state and conv state."""
    return prefill_case(2, H, [T], False, "cfg2-prefill")


def case3_lengths(n: int = 16) -> np.ndarray:
    return _rng(3, _S_LENS).integers(512, 4097, n)


def case3_prefill(H: int = 96) -> PrefillCase:
    """16 sequences of lengths U[512, 4096], nonzero initial states and conv states."""
    return prefill_case(3, H, case3_lengths(), True, "cfg3-prefill")


def lowrank_gate(seed: int, N: int, H: int, rank: int = 128):
    """Inputs of the low-rank decay projection, as bf16 bit patterns: f = W_fa x [N, rank]
    N(0, 1) (shared by the heads) and the second factor W_fb [H*D, rank] N(0, rank^-0.5),
    so that z = W_fb f has the unit variance of the logits of the other workloads."""
    return (normal(seed, _S_F, (N, rank), 1.0, bf16=True),
            normal(seed, _S_W_FB, (H * D, rank), float(rank) ** -0.5, bf16=True))


# ---------------------------------------------------------------------------------
# Digests
# ---------------------------------------------------------------------------------

def digest(case) -> str:
    """SHA-256 of a case's generated bytes: for each array, in a fixed order, its name,
    dtype and shape, then its bytes (C order).  A decode case covers its parameters,
    states and every step's token inputs; a prefill case its cu_seqlens, parameters,
    token inputs and initial states (absent ones named with no bytes)."""
    h = hashlib.sha256()

    def put(name, a):
        if a is None:
            h.update(f"{name}:none;".encode())
            return
        a = np.ascontiguousarray(a)
        h.update(f"{name}:{a.dtype.str}:{a.shape};".encode())
        h.update(a.tobytes())

    p = case.params
    for n in ("conv_w", "dt_bias", "A_log", "norm_w"):
        put(n, getattr(p, n))
    if isinstance(case, DecodeCase):
        put("state", case.state)
        put("conv_state", case.conv_state)
        for i in range(case.n_steps):
            x = case.step(i)
            for n in "qkvzbg":
                put(f"step{i}.{n}", getattr(x, n))
    else:
        put("cu_seqlens", case.cu_seqlens)
        for n in "qkvzbg":
            put(n, getattr(case.x, n))
        put("initial_state", case.initial_state)
        put("initial_conv_state", case.initial_conv_state)
    return h.hexdigest()
