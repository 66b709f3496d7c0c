"""The C ABI of libkda.so on the host: it loads, exports every function include/kda.h
declares, and rejects bad arguments with the documented status codes before touching
the GPU (these calls queue nothing, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_31_amd as kda

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kda.h")

OK, NULL_ARG, BAD_CONFIG, BAD_SHAPE, MISALIGNED, WORKSPACE, LAUNCH, OVERLAP = range(8)


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
    for s in range(8):
        assert isinstance(L.kda_status_str(s), bytes) and L.kda_status_str(s)
    assert L.kda_status_str(OVERLAP) != L.kda_status_str(99)


FAKE = 0x10000  # a 16-byte aligned non-NULL address; never dereferenced by rejected calls


def _decode(cfg, batch, ptrs=None, stride=0):
    p = [ctypes.c_void_p(FAKE)] * 13 if ptrs is None else ptrs
    return kda.lib().kda_decode_step(ctypes.byref(cfg), batch, *p[:3], stride, *p[3:], None)


def _cfg(**over):
    c = kda.lib().kda_config_default()
    for k, v in over.items():
        setattr(c, k, v)
    return c


def test_decode_rejects_bad_config():
    assert kda.lib().kda_decode_step(None, 1, *([ctypes.c_void_p(FAKE)] * 3), 0, *([ctypes.c_void_p(FAKE)] * 10),
                                     None) == NULL_ARG
    assert _decode(_cfg(num_heads=65537), 1) == BAD_CONFIG
    assert _decode(_cfg(head_dim=64), 1) == BAD_CONFIG
    assert _decode(_cfg(conv_size=3), 1) == BAD_CONFIG
    assert _decode(_cfg(num_heads=0), 1) == BAD_CONFIG
    assert _decode(_cfg(l2_eps=-1.0), 1) == BAD_CONFIG
    assert _decode(_cfg(rms_eps=float("nan")), 1) == BAD_CONFIG
    assert _decode(_cfg(out_dtype=2), 1) == BAD_CONFIG
    assert _decode(_cfg(out_dtype=-1), 1) == BAD_CONFIG
    assert kda.lib().kda_config_default().out_dtype == 0


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


def _prefill(cfg, B, N, ptrs=None, ws_bytes=0, stride=0, ws=None):
    p = [ctypes.c_void_p(FAKE)] * 16 if ptrs is None else ptrs
    return kda.lib().kda_prefill(ctypes.byref(cfg), B, N, *p[:4], stride, *p[4:], ws, ws_bytes, None)


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


REC_BYTES = 111616  # one chunk record


def _ws(cfg, B, N):
    return kda.lib().kda_prefill_workspace_bytes(ctypes.byref(cfg), B, N)


def test_prefill_path_selection_and_workspace_size():
    # fused: no workspace
    assert _ws(_cfg(prefill_path=1), 1, 8192) == 0
    # chunked: 2(B+1) int32 padded to 256 bytes; for one sequence where the carries run in
    # the chunk workgroups' launch, a ready word per (chunk, head) padded to 256 bytes;
    # otherwise, for B*H <= 128 in standard precision, the split carry's exchange words
    # (4096 bytes per sequence-head); then floor(N/64) + B records per head
    ready = lambda n: (n * 4 + 255) // 256 * 256
    assert _ws(_cfg(prefill_path=2, num_heads=96), 1, 8192) == 256 + ready(129 * 96) + (128 + 1) * 96 * REC_BYTES
    try:
        kda.kda_test_pipeline(1)  # never pipelined: the split carry's layout
        assert _ws(_cfg(prefill_path=2, num_heads=96), 1, 8192) == 256 + 96 * 4096 + (128 + 1) * 96 * REC_BYTES
        kda.kda_test_pipeline(2)  # pipelined wherever it can run: one sequence, H <= 128
        assert _ws(_cfg(prefill_path=2, num_heads=4), 1, 100) == 256 + ready(2 * 4) + (1 + 1) * 4 * REC_BYTES
        assert _ws(_cfg(prefill_path=2, num_heads=128), 1, 64) == 256 + ready(2 * 128) + 2 * 128 * REC_BYTES
        assert _ws(_cfg(prefill_path=2, num_heads=129), 1, 64) == 256 + 2 * 129 * REC_BYTES
        assert _ws(_cfg(prefill_path=2, num_heads=4), 2, 100) == 256 + 256 + 256 + (1 + 2) * 4 * REC_BYTES
        # three sequences of 300 tokens: 7 record rows; 32 heads: ready words, the order of the
        # 4 segments (4-chunk segments); 64 heads: B*H = 192 takes neither that form nor the split
        assert _ws(_cfg(prefill_path=2, num_heads=32), 3, 300) == 256 + 1024 + 256 + 7 * 32 * REC_BYTES
        assert _ws(_cfg(prefill_path=2, num_heads=64), 3, 300) == 256 + 7 * 64 * REC_BYTES
        # high precision: the pipelined form too (its records are 144,384 bytes)
        assert _ws(_cfg(prefill_path=2, num_heads=4, precision=1), 1, 100) == 256 + 256 + (1 + 1) * 4 * 144384
        kda.kda_test_pipeline(1)  # and its serial carry, which has no split form
        assert _ws(_cfg(prefill_path=2, num_heads=4, precision=1), 1, 100) == 256 + (1 + 1) * 4 * 144384
    finally:
        kda.kda_test_pipeline(0)
    assert _ws(_cfg(prefill_path=2, num_heads=4), 100, 1000) == 1024 + (15 + 100) * 4 * REC_BYTES
    # (two sequences of 64 heads: the pipelined plan, with the segments' row-major order)
    assert _ws(_cfg(prefill_path=2, num_heads=64), 2, 128) == 256 + 1024 + 256 + (2 + 2) * 64 * REC_BYTES
    assert _ws(_cfg(prefill_path=2, num_heads=43), 3, 128) == 256 + (2 + 3) * 43 * REC_BYTES
    assert _ws(_cfg(prefill_path=2, num_heads=96, precision=1), 1, 8192) == 256 + ready(129 * 96) + (128 + 1) * 96 * 144384
    # auto: the layout the time estimate prefers; these are the measured winners on MI355X
    # for equal sequences of 4096 tokens (fused fills whole rounds of 256 workgroups)
    chunked = lambda B, N: _ws(_cfg(num_heads=96), B, N) == _ws(_cfg(prefill_path=2, num_heads=96), B, N) > 0
    fused = lambda B, N: _ws(_cfg(num_heads=96), B, N) == 0
    assert chunked(1, 8192) and chunked(1, 4096) and chunked(3, 3 * 4096) and chunked(3, 3 * 1024)
    assert fused(2, 2 * 4096) and fused(4, 4 * 4096) and fused(5, 5 * 4096) and fused(8, 8 * 1024)
    assert fused(16, 40230) and fused(0, 0)
    # sizes the call would reject
    assert _ws(_cfg(prefill_path=2), -1, 10) == 0
    assert _ws(_cfg(prefill_path=7), 1, 10) == 0


def test_prefill_rejects_bad_path_and_small_or_misaligned_workspace():
    assert _prefill(_cfg(prefill_path=3), 1, 8) == BAD_CONFIG
    assert _prefill(_cfg(prefill_path=-1), 1, 8) == BAD_CONFIG
    need = _ws(_cfg(prefill_path=2), 2, 100)
    p = [ctypes.c_void_p(FAKE)] * 16
    lib = kda.lib()

    def call(ws, nbytes, path=2):
        c = _cfg(prefill_path=path)
        return lib.kda_prefill(ctypes.byref(c), 2, 100, *p[:4], 0, *p[4:], ws, nbytes, None)

    assert call(None, 0) == WORKSPACE
    assert call(ctypes.c_void_p(FAKE), need - 1) == WORKSPACE
    assert call(None, need) == WORKSPACE
    assert call(ctypes.c_void_p(FAKE + 16), need) == MISALIGNED
    # the fused layout takes no workspace, so none is checked
    assert _ws(_cfg(prefill_path=1), 2, 100) == 0


def test_launch_size_limits():
    # one workgroup per (sequence, head); a dispatch holds < 2^32 work-items
    assert _decode(_cfg(num_heads=1), 16_777_216) == BAD_SHAPE
    assert _prefill(_cfg(num_heads=1, prefill_path=1), 8_388_608, 0) == BAD_SHAPE
    # chunked: (floor(N/64) + B) * H workgroups; auto falls back to fused past the limit
    big_n = 64 * 8_388_608
    assert _ws(_cfg(num_heads=1, prefill_path=2), 1, big_n) == 0
    assert _prefill(_cfg(num_heads=1, prefill_path=2), 1, big_n) == BAD_SHAPE
    assert _ws(_cfg(num_heads=1), 1, big_n) == 0


def _multi(cfg, B, T, n_tokens=None, ptrs=None, stride=0):
    p = [ctypes.c_void_p(FAKE)] * 15 if ptrs is None else ptrs
    return kda.lib().kda_decode_multi(ctypes.byref(cfg), B, T, n_tokens, *p[:3], stride, *p[3:], None)


def test_decode_multi_rejects_bad_arguments():
    assert _multi(_cfg(head_dim=64), 1, 2) == BAD_CONFIG
    assert _multi(_cfg(), -1, 2) == BAD_SHAPE
    assert _multi(_cfg(), 1, -2) == BAD_SHAPE
    assert _multi(_cfg(), 0, 4) == OK       # empty batch: nothing queued
    assert _multi(_cfg(), 2, 0) == BAD_SHAPE
    assert _multi(_cfg(num_heads=1), 16_777_216, 1) == BAD_SHAPE
    assert _multi(_cfg(num_heads=1), 65_536, 65_536) == BAD_SHAPE  # B*T rows past 2^31-1
    # argument order: q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state_in, state_out,
    # conv_in, conv_out, out -- all required
    for i in range(15):
        p = [ctypes.c_void_p(FAKE)] * 15
        p[i] = None
        assert _multi(_cfg(), 2, 3, ptrs=p) == NULL_ARG, i
        p[i] = ctypes.c_void_p(FAKE + 4)
        assert _multi(_cfg(), 2, 3, ptrs=p) == MISALIGNED, i
    assert _multi(_cfg(), 2, 3, n_tokens=ctypes.c_void_p(FAKE + 2)) == MISALIGNED


def _slots(cfg, B, P, slots=ctypes.c_void_p(FAKE), ptrs=None, stride=0):
    p = [ctypes.c_void_p(FAKE)] * 13 if ptrs is None else ptrs
    return kda.lib().kda_decode_step_slots(ctypes.byref(cfg), B, slots, P, *p[:3], stride, *p[3:], None)


def test_decode_slots_rejects_bad_arguments():
    assert _slots(_cfg(head_dim=64), 1, 4) == BAD_CONFIG
    assert _slots(_cfg(), -1, 4) == BAD_SHAPE
    assert _slots(_cfg(), 1, -4) == BAD_SHAPE
    assert _slots(_cfg(num_heads=1), 16_777_216, 4) == BAD_SHAPE
    assert _slots(_cfg(), 0, 4) == OK   # empty batch: nothing queued
    assert _slots(_cfg(), 3, 0) == OK   # empty pool: every row would be skipped
    assert _slots(_cfg(), 3, 4, slots=None) == NULL_ARG
    assert _slots(_cfg(), 3, 4, slots=ctypes.c_void_p(FAKE + 2)) == MISALIGNED
    # argument order: q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state_pool,
    # conv_pool, out -- all required
    for i in range(13):
        p = [ctypes.c_void_p(FAKE)] * 13
        p[i] = None
        assert _slots(_cfg(), 3, 4, ptrs=p) == NULL_ARG, i
        p[i] = ctypes.c_void_p(FAKE + 4)
        assert _slots(_cfg(), 3, 4, ptrs=p) == MISALIGNED, i


def _copy(cfg, n, src=(FAKE, FAKE), src_entries=4, src_slots=None, dst=(FAKE, FAKE), dst_entries=4, dst_slots=None):
    arr = lambda xs: (ctypes.c_int32 * len(xs))(*xs) if xs is not None else None
    ss = arr(src_slots if src_slots is not None else [0] * max(n, 1))
    ds = arr(dst_slots if dst_slots is not None else [0] * max(n, 1))
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    return kda.lib().kda_state_copy(ctypes.byref(cfg), n, vp(src[0]), vp(src[1]), src_entries, ss,
                                    vp(dst[0]), vp(dst[1]), dst_entries, ds, None)


def test_state_copy_rejects_bad_arguments():
    # every case below is rejected on the host before any copy is queued
    H = 96
    st, cv = H * 128 * 128 * 4, 3 * H * 128 * 3 * 4  # bytes of one entry
    A, B = 0x100000000, 0x200000000  # two far-apart, 16-byte aligned addresses
    src, dst = (A, A + 8 * st), (B, B + 8 * st)
    assert _copy(_cfg(head_dim=64), 1, src, 4, [0], dst, 4, [0]) == BAD_CONFIG
    assert _copy(_cfg(), -1, src, 4, [0], dst, 4, [0]) == BAD_SHAPE
    assert _copy(_cfg(), 1, src, -1, [0], dst, 4, [0]) == BAD_SHAPE
    assert _copy(_cfg(), 0, src, 4, [0], dst, 4, [0]) == OK  # nothing to copy
    assert kda.lib().kda_state_copy(ctypes.byref(_cfg()), 1, ctypes.c_void_p(A), ctypes.c_void_p(A + 8 * st), 4,
                                    None, ctypes.c_void_p(B), ctypes.c_void_p(B + 8 * st), 4,
                                    (ctypes.c_int32 * 1)(0), None) == NULL_ARG
    for i in range(4):
        ptrs = [src[0], src[1], dst[0], dst[1]]
        ptrs[i] = None
        assert _copy(_cfg(), 1, (ptrs[0], ptrs[1]), 4, [0], (ptrs[2], ptrs[3]), 4, [0]) == NULL_ARG, i
        ptrs[i] = [src[0], src[1], dst[0], dst[1]][i] + 4
        assert _copy(_cfg(), 1, (ptrs[0], ptrs[1]), 4, [0], (ptrs[2], ptrs[3]), 4, [0]) == MISALIGNED, i
    # slots outside the buffers, on either side, anywhere in the list
    for ss, ds in (([4], [0]), ([-1], [0]), ([0], [4]), ([0], [-2]), ([0, 1, 9], [0, 1, 2])):
        assert _copy(_cfg(), len(ss), src, 4, ss, dst, 4, ds) == BAD_SHAPE, (ss, ds)
    # distinct source and destination buffers that overlap
    assert _copy(_cfg(), 1, src, 4, [0], (A + st, B), 4, [0]) == OVERLAP
    assert _copy(_cfg(), 1, src, 4, [0], (B, A + 8 * st + 16), 4, [0]) == OVERLAP
    assert _copy(_cfg(), 1, src, 4, [0], (A + 8 * st, B), 4, [0]) == OVERLAP  # dst state on src conv


def _multi_slots(cfg, B, T, P, slots=ctypes.c_void_p(FAKE), n_tokens=None, ptrs=None, stride=0):
    p = [ctypes.c_void_p(FAKE)] * 15 if ptrs is None else ptrs
    return kda.lib().kda_decode_multi_slots(ctypes.byref(cfg), B, T, n_tokens, slots, P, *p[:3], stride, *p[3:],
                                            None)


def test_decode_multi_slots_rejects_bad_arguments():
    assert _multi_slots(_cfg(head_dim=64), 1, 2, 4) == BAD_CONFIG
    assert _multi_slots(_cfg(), -1, 2, 4) == BAD_SHAPE
    assert _multi_slots(_cfg(), 1, 2, -4) == BAD_SHAPE
    assert _multi_slots(_cfg(), 2, 0, 4) == BAD_SHAPE
    assert _multi_slots(_cfg(), 0, 2, 4) == OK   # empty batch: nothing queued
    assert _multi_slots(_cfg(), 2, 2, 0) == OK   # empty pool: every row would be skipped
    assert _multi_slots(_cfg(), 2, 2, 4, slots=None) == NULL_ARG
    assert _multi_slots(_cfg(), 2, 2, 4, slots=ctypes.c_void_p(FAKE + 2)) == MISALIGNED
    assert _multi_slots(_cfg(), 2, 2, 4, n_tokens=ctypes.c_void_p(FAKE + 1)) == MISALIGNED
    for i in range(15):
        p = [ctypes.c_void_p(FAKE)] * 15
        p[i] = None
        assert _multi_slots(_cfg(), 2, 3, 4, ptrs=p) == NULL_ARG, i
        p[i] = ctypes.c_void_p(FAKE + 4)
        assert _multi_slots(_cfg(), 2, 3, 4, ptrs=p) == MISALIGNED, i


def test_qkv_row_stride_rejections():
    H = 96
    HD = H * 128
    # 0 = dense; otherwise >= H*D, a multiple of 8, at most 2^24
    for bad in (HD - 8, HD + 4, -8, (1 << 24) + 8):
        assert _decode(_cfg(), 2, stride=bad) == BAD_SHAPE, bad
        assert _slots(_cfg(), 2, 4, stride=bad) == BAD_SHAPE, bad
        assert _multi(_cfg(), 2, 3, stride=bad) == BAD_SHAPE, bad
        assert _multi_slots(_cfg(), 2, 3, 4, stride=bad) == BAD_SHAPE, bad
        assert _prefill(_cfg(), 2, 100, stride=bad) == BAD_SHAPE, bad


def _spaced(n, gap=1 << 32):
    """n 16-byte aligned addresses, `gap` bytes apart (far enough that no extent overlaps)."""
    return [ctypes.c_void_p((i + 1) * gap) for i in range(n)]


def test_decode_rejects_overlapping_outputs():
    # q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state, conv_state, out
    B, H = 4, 96
    HD = H * 128
    p = _spaced(13)  # (the call with these disjoint buffers would launch: it is not made here)
    out, state, conv = 12, 10, 11
    cases = [
        (out, 0, 0),                      # out on q
        (out, 3, 4 * (B * HD - 4)),       # out's first row on z's last values
        (state, 6, 16),                   # state inside conv_w
        (conv, state, 16),                # conv_state inside state
        (out, conv, 0),                   # out on conv_state
    ]
    for dst, src, off in cases:
        q = list(p)
        q[dst] = ctypes.c_void_p(p[src].value + off)
        assert _decode(_cfg(), B, q) == OVERLAP, (dst, src, off)
        assert _slots(_cfg(), B, 8, ptrs=q) == OVERLAP, (dst, src, off)
    # q, k, v may overlap each other (views of one fused projection): only the outputs count
    q = list(p)
    q[1] = ctypes.c_void_p(p[0].value + 4 * HD)
    q[2] = ctypes.c_void_p(p[0].value + 8 * HD)
    q[out] = ctypes.c_void_p(p[0].value + 4 * ((B - 1) * 3 * HD + HD - 4))  # on q's last row
    assert _decode(_cfg(), B, q, stride=3 * HD) == OVERLAP


def test_decode_multi_overlap_rules():
    # q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, state_in, state_out, conv_in, conv_out, out
    B, T, H = 2, 3, 96
    p = _spaced(15)
    st = B * H * 128 * 128 * 4
    q = list(p)
    q[11] = ctypes.c_void_p(p[10].value + 16)  # state_out partly over state_in
    assert _multi(_cfg(), B, T, ptrs=q) == OVERLAP
    assert _multi_slots(_cfg(), B, T, 4, ptrs=q) == OVERLAP
    q = list(p)
    q[13] = ctypes.c_void_p(p[12].value + 16)  # conv_out partly over conv_in
    assert _multi(_cfg(), B, T, ptrs=q) == OVERLAP
    q = list(p)
    q[14] = ctypes.c_void_p(p[10].value + st - 16)  # out on the end of state_in
    assert _multi(_cfg(), B, T, ptrs=q) == OVERLAP
    q = list(p)
    q[11] = ctypes.c_void_p(p[0].value)  # state_out on q
    assert _multi(_cfg(), B, T, ptrs=q) == OVERLAP


def test_prefill_overlap_rules():
    # cu, q, k, v, z, b, g, conv_w, A_log, dt_bias, norm_w, init_state, init_conv, out,
    # final_state, final_conv
    B, N, H = 2, 100, 96
    HD = H * 128
    p = _spaced(16)
    cases = [
        (14, 11, 16),    # final_state partly over initial_state
        (15, 12, 48),    # final_conv partly over initial_conv
        (13, 1, 0),      # out on q
        (14, 7, 0),      # final_state on conv_w
        (15, 13, 16),    # final_conv inside out
        (13, 0, 0),      # out on cu_seqlens
    ]
    for dst, src, off in cases:
        q = list(p)
        q[dst] = ctypes.c_void_p(p[src].value + off)
        assert _prefill(_cfg(prefill_path=1), B, N, q) == OVERLAP, (dst, src, off)
    # the workspace of the chunked layout counts as an output
    need = _ws(_cfg(prefill_path=2), B, N)
    assert _prefill(_cfg(prefill_path=2), B, N, p, ws_bytes=need, ws=ctypes.c_void_p(p[13].value)) == OVERLAP
    assert _prefill(_cfg(prefill_path=2), B, N, p, ws_bytes=need, ws=ctypes.c_void_p(p[4].value + 256)) == OVERLAP
    # strided q whose last row reaches into out
    q = list(p)
    q[13] = ctypes.c_void_p(p[1].value + 2 * (N - 1) * 3 * HD)
    assert _prefill(_cfg(prefill_path=1), B, N, q, stride=3 * HD) == OVERLAP


def test_state_copy_conv_entry_onto_itself_is_still_checked():
    # the state entry maps onto itself (same buffer, same slot) while the conv windows go
    # to another buffer: accepted (the conv copy is queued on its own); an overlapping
    # conv destination is still rejected
    H = 96
    st, cv = H * 128 * 128 * 4, 3 * H * 128 * 3 * 4
    A, Bc, Cc = 0x100000000, 0x200000000, 0x300000000
    assert _copy(_cfg(), 1, (A, Bc), 4, [0], (A, Bc + cv), 4, [0]) == OVERLAP  # conv buffers overlap


def _noalloc(cfg, B, N, ptrs=None, stride=0):
    p = [ctypes.c_void_p(FAKE)] * 16 if ptrs is None else ptrs
    return kda.lib().kda_prefill_noalloc(ctypes.byref(cfg), B, N, *p[:4], stride, *p[4:], None)


def test_prefill_noalloc_host_rejections():
    # the same argument checks as kda_prefill, before the scratch array is looked up
    assert _noalloc(_cfg(head_dim=64), 1, 8) == BAD_CONFIG
    assert _noalloc(_cfg(), -1, 8) == BAD_SHAPE
    assert _noalloc(_cfg(), 0, 0) == OK
    p = [ctypes.c_void_p(FAKE)] * 16
    p[1] = None
    assert _noalloc(_cfg(), 2, 100, p) == NULL_ARG
    p = _spaced(16)
    q = list(p)
    q[14] = ctypes.c_void_p(p[11].value + 16)
    assert _noalloc(_cfg(prefill_path=1), 2, 100, q) == OVERLAP
    # an explicit chunked layout whose records would not fit the 256 MiB scratch array
    assert _ws(_cfg(prefill_path=2, num_heads=96), 1, 4096) > 256 << 20
    assert _noalloc(_cfg(prefill_path=2, num_heads=96), 1, 4096, p) == WORKSPACE


def test_precision_flag():
    assert kda.lib().kda_config_default().precision == 0
    assert _decode(_cfg(precision=2), 1) == BAD_CONFIG
    assert _prefill(_cfg(precision=-1), 1, 8) == BAD_CONFIG
    # the high-precision records carry the lo parts of W and Q~: 144,384 bytes each (one
    # sequence of 96 heads: the pipelined form, with a ready word per record)
    ready = (129 * 96 * 4 + 255) // 256 * 256
    assert _ws(_cfg(prefill_path=2, num_heads=96, precision=1), 1, 8192) == 256 + ready + (128 + 1) * 96 * 144384
    assert _ws(_cfg(prefill_path=1, precision=1), 1, 8192) == 0


def test_decode_multi_form_flag():
    assert kda.lib().kda_config_default().decode_multi_form == 0  # blocks of eight tokens
    assert _decode(_cfg(decode_multi_form=2), 1) == BAD_CONFIG
    assert _prefill(_cfg(decode_multi_form=-1), 1, 8) == BAD_CONFIG


def _gate_proj(cfg, B, N, ptrs=None, stride=0, ws=None, ws_bytes=0):
    # cu, q, k, v, f, w_fb, b, g, conv_w, A_log, dt_bias, norm_w, init_state, init_conv, out, final_state,
    # final_conv
    p = [ctypes.c_void_p(FAKE)] * 17 if ptrs is None else ptrs
    return kda.lib().kda_prefill_gate_proj(ctypes.byref(cfg), B, N, *p[:4], stride, *p[4:], ws, ws_bytes, None)


def test_prefill_gate_proj_rejections():
    assert _gate_proj(_cfg(head_dim=64), 1, 8) == BAD_CONFIG
    assert _gate_proj(_cfg(), -1, 8) == BAD_SHAPE
    assert _gate_proj(_cfg(), 0, 0) == OK
    for i in (4, 5):  # f and w_fb are required
        p = [ctypes.c_void_p(FAKE)] * 17
        p[i] = None
        assert _gate_proj(_cfg(prefill_path=1), 2, 100, p) == NULL_ARG, i
        p[i] = ctypes.c_void_p(FAKE + 8)
        assert _gate_proj(_cfg(prefill_path=1), 2, 100, p) == MISALIGNED, i
    # w_fb is still required with no tokens; f is not
    p = [ctypes.c_void_p(FAKE)] * 17
    p[5] = None
    assert _gate_proj(_cfg(prefill_path=1), 2, 0, p) == NULL_ARG
    # outputs over the factors
    p = _spaced(17)
    q = list(p)
    q[14] = ctypes.c_void_p(p[5].value + 64)  # out on w_fb
    assert _gate_proj(_cfg(prefill_path=1), 2, 100, q) == OVERLAP
    q = list(p)
    q[15] = ctypes.c_void_p(p[4].value)  # final_state on f
    assert _gate_proj(_cfg(prefill_path=1), 2, 100, q) == OVERLAP
