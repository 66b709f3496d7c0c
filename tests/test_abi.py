"""The C ABI of libkda.so on the host: it loads, exports every function include/kda.h
declares, and rejects bad arguments with the documented status codes before touching
the GPU (these calls queue nothing, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_31_amd as kda

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kda.h")

OK, NULL_ARG, BAD_CONFIG, BAD_SHAPE, MISALIGNED, WORKSPACE, LAUNCH = range(7)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(kda.EXPORTED_SYMBOLS)
    L = ctypes.CDLL(kda.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_defaults():
    L = kda.lib()
    assert L.kda_abi_version() == kda.ABI_VERSION
    c = L.kda_config_default()
    assert (c.num_heads, c.head_dim, c.conv_size) == (96, 128, 4)
    assert c.gate_lower_bound == -5.0 and c.l2_eps == pytest.approx(1e-6) and c.rms_eps == pytest.approx(1e-5)
    for s in range(7):
        assert isinstance(L.kda_status_str(s), bytes) and L.kda_status_str(s)


FAKE = 0x10000  # a 16-byte aligned non-NULL address; never dereferenced by rejected calls


def _decode(cfg, batch, ptrs=None):
    p = [ctypes.c_void_p(FAKE)] * 13 if ptrs is None else ptrs
    return kda.lib().kda_decode_step(ctypes.byref(cfg), batch, *p, None)


def _cfg(**over):
    c = kda.lib().kda_config_default()
    for k, v in over.items():
        setattr(c, k, v)
    return c


def test_decode_rejects_bad_config():
    assert kda.lib().kda_decode_step(None, 1, *([ctypes.c_void_p(FAKE)] * 13), None) == NULL_ARG
    assert _decode(_cfg(head_dim=64), 1) == BAD_CONFIG
    assert _decode(_cfg(conv_size=3), 1) == BAD_CONFIG
    assert _decode(_cfg(num_heads=0), 1) == BAD_CONFIG
    assert _decode(_cfg(l2_eps=-1.0), 1) == BAD_CONFIG
    assert _decode(_cfg(rms_eps=float("nan")), 1) == BAD_CONFIG


def test_decode_rejects_bad_shapes_and_pointers():
    assert _decode(_cfg(), -1) == BAD_SHAPE
    assert _decode(_cfg(num_heads=96), 2 ** 30) == BAD_SHAPE
    assert _decode(_cfg(), 0) == OK  # empty batch: nothing queued
    for i in range(13):
        p = [ctypes.c_void_p(FAKE)] * 13
        p[i] = None
        assert _decode(_cfg(), 4, p) == NULL_ARG
        p[i] = ctypes.c_void_p(FAKE + 4)
        assert _decode(_cfg(), 4, p) == MISALIGNED


def _prefill(cfg, B, N, ptrs=None, ws_bytes=0):
    p = [ctypes.c_void_p(FAKE)] * 16 if ptrs is None else ptrs
    return kda.lib().kda_prefill(ctypes.byref(cfg), B, N, *p, None, ws_bytes, None)


def test_prefill_rejects_bad_arguments():
    assert _prefill(_cfg(head_dim=256), 1, 8) == BAD_CONFIG
    assert _prefill(_cfg(), -1, 8) == BAD_SHAPE
    assert _prefill(_cfg(), 1, -8) == BAD_SHAPE
    assert _prefill(_cfg(), 0, 0) == OK
    assert _prefill(_cfg(), 0, 5) == BAD_SHAPE
    # argument order: cu, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, init_state,
    # init_conv, out, final_state, final_conv
    required = [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 13, 14, 15]
    for i in required:
        p = [ctypes.c_void_p(FAKE)] * 16
        p[i] = None
        assert _prefill(_cfg(), 2, 100, p) == NULL_ARG, i
    for i in range(16):
        p = [ctypes.c_void_p(FAKE)] * 16
        p[i] = ctypes.c_void_p(FAKE + (2 if i == 0 else 8))
        assert _prefill(_cfg(), 2, 100, p) == MISALIGNED, i
    # token arrays may be NULL when there are no tokens
    p = [ctypes.c_void_p(FAKE)] * 16
    for i in (1, 2, 3, 4, 5, 6, 13):
        p[i] = None
    p[0] = ctypes.c_void_p(FAKE + 2)  # but cu_seqlens alignment is still checked
    assert _prefill(_cfg(), 2, 0, p) == MISALIGNED


def test_workspace_query_is_host_only():
    assert kda.kda_prefill_workspace_bytes(kda.KdaConfig(), 16, 40000) >= 0
