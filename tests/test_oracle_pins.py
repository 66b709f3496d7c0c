"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Every step the oracle takes is checked here against a closed form, an invariant, a
library routine (numpy.convolve, scipy.special.expit), brute force on tiny sizes, or an
independently derived chunked form.  Each pin is chosen so that a plausible mistake
(a dropped term, a wrong sign or index, a transposed operand, readout from the old
state, eps outside the sqrt, the scale on the wrong operand) fails it.

The recurrence pinned: page "colibri/c/kimi_k3.c", header comment "KDA per-head
recurrence".
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from tests.chunked_ref import chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def unit(x):
    return x / np.linalg.norm(x)


# ----------------------------------------------------------------------------- scalars

@pytest.mark.parametrize("x", [-1e4, -700.0, -40.0, -3.0, -0.5, 0.0, 1e-8, 0.5, 3.0, 40.0, 1e4])
def test_sigmoid_and_silu_match_scipy(x):
    assert oracle.sigmoid(x) == pytest.approx(expit(x), rel=1e-15, abs=1e-300)
    assert oracle.silu(x) == pytest.approx(x * expit(x), rel=1e-15, abs=1e-300)


def test_sigmoid_saturates_exactly():
    # beta = 0 / a closed output gate are reachable only through saturated logits
    assert oracle.sigmoid(-1e4) == 0.0 and oracle.sigmoid(1e4) == 1.0


# ----------------------------------------------------------------------------- conv

def test_conv_matches_numpy_convolve():
    rng = np.random.default_rng(11)
    w = rng.normal(0, 0.5, 4)
    win = rng.normal(size=3)
    x = rng.normal(size=23)
    y, win_out = oracle.conv_sequence(w, win, x)
    full = np.concatenate([win, x])
    np.testing.assert_allclose(y, np.convolve(full, w[::-1], mode="valid"), rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(win_out, full[-3:])


def test_conv_identity_and_delay_taps():
    rng = np.random.default_rng(12)
    win = rng.normal(size=3)
    x = rng.normal(size=9)
    y, _ = oracle.conv_sequence([0, 0, 0, 1], win, x)
    np.testing.assert_array_equal(y, x)
    y, _ = oracle.conv_sequence([1, 0, 0, 0], win, x)  # oldest tap: a 3-token delay
    np.testing.assert_array_equal(y, np.concatenate([win, x])[:9])


def test_conv_short_sequence_shifts_through_window():
    y, win = oracle.conv_sequence([0.1, 0.2, 0.3, 0.4], [1.0, 2.0, 3.0], [5.0])
    assert y[0] == pytest.approx(0.1 * 1 + 0.2 * 2 + 0.3 * 3 + 0.4 * 5)
    np.testing.assert_array_equal(win, [2.0, 3.0, 5.0])


# ----------------------------------------------------------------------------- rmsnorm

def test_rmsnorm_of_constant_vector():
    D, c, eps = 128, 0.3, 1e-5
    out = oracle.rmsnorm_gate(np.full(D, c), np.full(D, 1e4), np.ones(D), eps)
    np.testing.assert_allclose(out, c / np.sqrt(c * c + eps), rtol=1e-14)


def test_rmsnorm_unit_rms_gate_and_weight():
    rng = np.random.default_rng(13)
    o = rng.normal(size=64)
    out = oracle.rmsnorm_gate(o, np.full(64, 1e4), np.ones(64), 1e-300)
    assert np.mean(out ** 2) == pytest.approx(1.0, rel=1e-13)
    np.testing.assert_array_equal(oracle.rmsnorm_gate(o, np.full(64, -1e4), np.ones(64), 1e-5), 0.0)
    g = rng.normal(size=64)
    w = rng.uniform(0.5, 2.0, 64)
    base = oracle.rmsnorm_gate(o, np.full(64, 1e4), np.ones(64), 1e-5)
    np.testing.assert_allclose(oracle.rmsnorm_gate(o, g, w, 1e-5), base * w * expit(g), rtol=1e-14)


# ----------------------------------------------------------------------------- core

def _transition(alpha, beta, k):
    dk = len(k)
    return (np.eye(dk) - beta * np.outer(k, k)) @ np.diag(alpha)


@pytest.mark.parametrize("dk,dv,T", [(4, 4, 1), (4, 4, 7), (8, 8, 16), (16, 16, 11), (8, 5, 9)])
def test_core_matches_brute_force_transition_products(dk, dv, T):
    rng = np.random.default_rng(100 + dk * 7 + T)
    S0 = rng.normal(size=(dk, dv))
    ks = [unit(rng.normal(size=dk)) * rng.uniform(0.5, 1.0) for _ in range(T)]
    qs = [rng.normal(size=dk) for _ in range(T)]
    vs = [rng.normal(size=dv) for _ in range(T)]
    alphas = [rng.uniform(0.05, 1.0, dk) for _ in range(T)]
    betas = rng.uniform(0.0, 1.0, T)
    S = S0
    outs = []
    for t in range(T):
        S, o = oracle.core_step(S, qs[t], ks[t], vs[t], alphas[t], betas[t])
        outs.append(o)
    Ms = [_transition(alphas[t], betas[t], ks[t]) for t in range(T)]
    for t in range(T):
        # S_t = M_t ... M_1 S0 + sum_s M_t ... M_{s+1} beta_s k_s v_s^T
        St = np.eye(dk)
        for s in range(t + 1):
            St = Ms[s] @ St
        St = St @ S0
        for s in range(t + 1):
            P = np.eye(dk)
            for r in range(s + 1, t + 1):
                P = Ms[r] @ P
            St = St + P @ (betas[s] * np.outer(ks[s], vs[s]))
        np.testing.assert_allclose(outs[t], St.T @ qs[t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, St, rtol=1e-12, atol=1e-12)


def test_core_beta0_alpha1_leaves_state_unchanged():
    rng = np.random.default_rng(1)
    S0 = rng.normal(size=(16, 16))
    S, _ = oracle.core_step(S0, rng.normal(size=16), unit(rng.normal(size=16)), rng.normal(size=16),
                            np.ones(16), 0.0)
    np.testing.assert_array_equal(S, S0)


def test_core_alpha1_beta1_unit_key_retrieves_value():
    rng = np.random.default_rng(2)
    S0 = rng.normal(size=(16, 12))
    k = unit(rng.normal(size=16))
    v = rng.normal(size=12)
    S, _ = oracle.core_step(S0, rng.normal(size=16), k, v, np.ones(16), 1.0)
    np.testing.assert_allclose(S.T @ k, v, rtol=1e-13, atol=1e-13)


def test_core_frobenius_bound():
    rng = np.random.default_rng(3)
    S = rng.normal(size=(32, 32))
    for _ in range(200):
        k = unit(rng.normal(size=32))
        v = rng.normal(size=32)
        beta = rng.uniform(0.0, 1.0)
        alpha = rng.uniform(0.0, 1.0, 32)
        n0 = np.linalg.norm(S)
        S, _ = oracle.core_step(S, rng.normal(size=32), k, v, alpha, beta)
        assert np.linalg.norm(S) <= n0 + beta * np.linalg.norm(k) * np.linalg.norm(v) + 1e-12


def test_core_pure_decay_closed_form():
    rng = np.random.default_rng(4)
    S0 = rng.normal(size=(8, 6))
    S = S0
    prod = np.ones(8)
    for _ in range(10):
        a = rng.uniform(0.1, 1.0, 8)
        prod *= a
        S, _ = oracle.core_step(S, rng.normal(size=8), unit(rng.normal(size=8)), rng.normal(size=6), a, 0.0)
    np.testing.assert_allclose(S, prod[:, None] * S0, rtol=1e-13)


def test_core_orthonormal_keys_exact_retrieval():
    rng = np.random.default_rng(5)
    dk, dv, n = 16, 10, 12
    Qm, _ = np.linalg.qr(rng.normal(size=(dk, dk)))
    keys = Qm[:, :n].T
    vals = rng.normal(size=(n, dv))
    S = rng.normal(size=(dk, dv))
    for j in range(n):
        S, _ = oracle.core_step(S, rng.normal(size=dk), keys[j], vals[j], np.ones(dk), 1.0)
    np.testing.assert_allclose(keys @ S, vals, rtol=1e-12, atol=1e-12)


def test_core_one_step_from_zero():
    rng = np.random.default_rng(6)
    q, k, v = rng.normal(size=8), unit(rng.normal(size=8)), rng.normal(size=5)
    S, o = oracle.core_step(np.zeros((8, 5)), q, k, v, rng.uniform(0.1, 1, 8), 0.37)
    np.testing.assert_allclose(S, 0.37 * np.outer(k, v), rtol=1e-14)
    np.testing.assert_allclose(o, 0.37 * (k @ q) * v, rtol=1e-13)  # readout from the updated S


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_core_matches_independent_chunked_form(T):
    """The chunked WY/UT form (a separate derivation) equals the token recurrence."""
    rng = np.random.default_rng(7 + T)
    dk = dv = 32
    q = np.array([unit(rng.normal(size=dk)) * dk ** -0.5 for _ in range(T)])
    k = np.array([unit(rng.normal(size=dk)) for _ in range(T)])
    v = rng.normal(size=(T, dv))
    # decays as the configs draw them, including near-zero and near -5 log-decays
    gk = -5.0 * expit(np.exp(rng.uniform(-2, 1)) * (rng.normal(size=(T, dk)) + rng.uniform(-1, 1, dk)))
    gk[:, 0] = -1e-4
    gk[:, 1] = -4.999
    beta = expit(rng.normal(size=T))
    S0 = rng.normal(0, 0.05, (dk, dv))
    S = S0
    O = np.zeros((T, dv))
    for t in range(T):
        S, O[t] = oracle.core_step(S, q[t], k[t], v[t], np.exp(gk[t]), beta[t])
    Oc, Sc = chunked(S0, q, k, v, gk, beta)
    np.testing.assert_allclose(Oc, O, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------- full mixer

def _one_head(T, D=16, seed=0, **over):
    """Inputs for a single (sequence, head) in the library layouts, H = 1."""
    rng = np.random.default_rng(seed)
    d = dict(
        q=rng.normal(size=(T, D)), k=rng.normal(size=(T, D)), v=rng.normal(size=(T, D)),
        z=rng.normal(size=(T, D)), b=rng.normal(size=(T, 1)), g=rng.normal(size=(T, D)),
        conv_w=rng.normal(0, 0.5, (3 * D, 4)), A_log=rng.uniform(-2, 1, 1), dt_bias=rng.uniform(-1, 1, D),
        norm_w=np.ones(D), state=rng.normal(0, 0.05, (1, 1, D, D)), conv_state=rng.normal(size=(1, 3 * D, 3)),
    )
    d.update(over)
    return d


def _run(d, D=16, **cfg):
    c = oracle.MixerConfig(head_dim=D, **cfg)
    T = d["q"].shape[0]
    r = oracle.forward(c, [0, T], d["q"], d["k"], d["v"], d["z"], d["b"], d["g"], d["conv_w"], d["A_log"],
                       d["dt_bias"], d["norm_w"], d["state"], d["conv_state"])
    return r[(0, 0)]


def test_mixer_one_step_from_zero_closed_form():
    """Identity conv taps and S0 = 0: S = beta k^ v^T, o = beta (k^.q^) v with
    q^ = SiLU(xq)/sqrt(|SiLU(xq)|^2 + 1e-6) * D^-0.5, k^ likewise without the scale,
    v = SiLU(xv), beta = sigmoid(b) -- SiLU and sigmoid from scipy."""
    D = 16
    taps = np.tile([0.0, 0.0, 0.0, 1.0], (3 * D, 1))
    d = _one_head(1, D, seed=21, conv_w=taps, state=np.zeros((1, 1, D, D)))
    r = _run(d, D, rms_eps=1e-5)
    sq, sk, sv = (d[n][0] * expit(d[n][0]) for n in ("q", "k", "v"))
    qh = sq / np.sqrt(sq @ sq + 1e-6) * D ** -0.5
    kh = sk / np.sqrt(sk @ sk + 1e-6)
    beta = expit(d["b"][0, 0])
    np.testing.assert_allclose(r.state, beta * np.outer(kh, sv), rtol=1e-13, atol=1e-16)
    o = beta * (kh @ qh) * sv
    want = expit(d["g"][0]) * o / np.sqrt(np.mean(o * o) + 1e-5)
    np.testing.assert_allclose(r.out[0], want, rtol=1e-12)


def test_mixer_decay_gate_closed_form():
    """beta = 0 (saturated logit): S_T = Diag(prod_t alpha_t) S0 with
    alpha = exp(-5 * sigmoid(exp(A_log) * (z + dt_bias)))."""
    D, T = 16, 6
    d = _one_head(T, D, seed=22, b=np.full((T, 1), -1e4))
    r = _run(d, D)
    loga = -5.0 * expit(np.exp(d["A_log"][0]) * (d["z"] + d["dt_bias"][None, :]))
    np.testing.assert_allclose(r.state, np.exp(loga.sum(0))[:, None] * d["state"][0, 0], rtol=1e-12)


def test_mixer_gate_lower_bound_parameter():
    D, T = 16, 3
    d = _one_head(T, D, seed=23, b=np.full((T, 1), -1e4))
    r = _run(d, D, gate_lower_bound=-2.0)
    loga = -2.0 * expit(np.exp(d["A_log"][0]) * (d["z"] + d["dt_bias"][None, :]))
    np.testing.assert_allclose(r.state, np.exp(loga.sum(0))[:, None] * d["state"][0, 0], rtol=1e-12)


def test_mixer_output_gate_and_rms():
    D, T = 16, 5
    d = _one_head(T, D, seed=24, g=np.full((T, D), -1e4))
    np.testing.assert_array_equal(_run(d, D).out, 0.0)
    d = _one_head(T, D, seed=24, g=np.full((T, D), 1e4))
    r = _run(d, D, rms_eps=1e-300)
    np.testing.assert_allclose(np.mean(r.out ** 2, axis=1), 1.0, rtol=1e-12)


def test_mixer_conv_state_is_last_three_inputs():
    D, T = 16, 5
    d = _one_head(T, D, seed=25)
    r = _run(d, D)
    for blk, name in enumerate("qkv"):
        np.testing.assert_array_equal(r.conv_state[blk], d[name][-3:].T)
    d = _one_head(2, D, seed=26)  # shorter than the window: shifts through it
    r = _run(d, D)
    want = np.concatenate([d["conv_state"][0, D:2 * D, 2:], d["k"].T], axis=1)
    np.testing.assert_array_equal(r.conv_state[1], want)


def test_mixer_empty_sequence_keeps_state():
    D = 16
    d = _one_head(0, D, seed=27)
    r = _run(d, D)
    np.testing.assert_array_equal(r.state, d["state"][0, 0])
    np.testing.assert_array_equal(r.conv_state.reshape(3 * D, 3), d["conv_state"][0])
    assert r.out.shape == (0, D)


def test_mixer_split_invariance():
    """Running T tokens equals running T1 then T - T1 with the state and windows carried."""
    D, T, T1 = 16, 19, 7
    d = _one_head(T, D, seed=28)
    full = _run(d, D)
    first = {n: (a[:T1] if a.shape[0] == T and n in "qkvzbg" else a) for n, a in d.items()}
    r1 = _run(first, D)
    rest = {n: (a[T1:] if a.shape[0] == T and n in "qkvzbg" else a) for n, a in d.items()}
    rest["state"] = r1.state[None, None]
    rest["conv_state"] = r1.conv_state.reshape(1, 3 * D, 3)
    r2 = _run(rest, D)
    np.testing.assert_allclose(np.concatenate([r1.out, r2.out]), full.out, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(r2.state, full.state, rtol=1e-13, atol=1e-16)


def test_mixer_heads_and_sequences_are_independent():
    """A packed 2-sequence, 2-head batch equals each (sequence, head) run alone."""
    D, H = 8, 2
    rng = np.random.default_rng(29)
    lens = [5, 3]
    N = sum(lens)
    arr = {n: rng.normal(size=(N, H * D)) for n in "qkvzg"}
    b = rng.normal(size=(N, H))
    conv_w = rng.normal(0, 0.5, (3 * H * D, 4))
    A_log, dtb = rng.uniform(-2, 1, H), rng.uniform(-1, 1, H * D)
    st = rng.normal(0, 0.05, (2, H, D, D))
    cst = rng.normal(size=(2, 3 * H * D, 3))
    cfg = oracle.MixerConfig(head_dim=D)
    packed = oracle.forward(cfg, [0, 5, 8], arr["q"], arr["k"], arr["v"], arr["z"], b, arr["g"], conv_w,
                            A_log, dtb, np.ones(D), st, cst)
    for s, (t0, t1) in enumerate([(0, 5), (5, 8)]):
        for h in range(H):
            cs = slice(h * D, (h + 1) * D)
            cw = np.concatenate([conv_w[i * H * D + h * D:i * H * D + (h + 1) * D] for i in range(3)])
            cc = np.concatenate([cst[s, i * H * D + h * D:i * H * D + (h + 1) * D] for i in range(3)])
            alone = oracle.forward(cfg, [0, t1 - t0], *(arr[n][t0:t1, cs] for n in "qkvz"),
                                   b[t0:t1, h:h + 1], arr["g"][t0:t1, cs], cw, A_log[h:h + 1], dtb[cs],
                                   np.ones(D), st[s:s + 1, h:h + 1], cc[None])[(0, 0)]
            np.testing.assert_array_equal(alone.out, packed[(s, h)].out)
            np.testing.assert_array_equal(alone.state, packed[(s, h)].state)


# ----------------------------------------------------------------------------- page values

def test_page_constants_and_state_size():
    with open(os.path.join(GOLDEN, "kda_constants.json")) as f:
        g = json.load(f)
    c = oracle.MixerConfig()
    assert c.head_dim == g["head_dim"] and c.conv_size == g["conv_size"]
    assert c.gate_lower_bound == g["gate_lower_bound"] and c.l2_eps == g["l2_eps"]
    assert g["num_heads"] * g["head_dim"] == g["dt_bias_len"]
    # "~434 MB per photo": one fp32 [heads, D, D] state per KDA layer
    photo = g["kda_layers"] * g["num_heads"] * g["head_dim"] ** 2 * 4
    assert round(photo / 1e6) == g["photo_mb_approx"]


def test_gate_projection_one_hot_factor_selects_channels():
    """A one-hot second factor (row h*D + i = unit vector e_{pi_h(i)}, pi_h a permutation
    that differs per head) makes z[t, h*D + i] = f[t, pi_h(i)]: the oracle with the low-rank
    projection equals the oracle given those logits directly, to the bit.  A transposed
    factor, a wrong head slice or a wrong row order would pick other channels."""
    rng = np.random.default_rng(31)
    D, H, T = 16, 2, 7
    HD = H * D
    perms = [rng.permutation(D) for _ in range(H)]
    w_fb = np.zeros((HD, D))
    for h in range(H):
        w_fb[h * D + np.arange(D), perms[h]] = 1.0
    f = rng.standard_normal((T, D))
    z_direct = np.concatenate([f[:, perms[h]] for h in range(H)], axis=1)
    args = dict(q=rng.standard_normal((T, HD)), k=rng.standard_normal((T, HD)), v=rng.standard_normal((T, HD)),
                b=rng.standard_normal((T, H)), g=rng.standard_normal((T, HD)),
                conv_w=rng.standard_normal((3 * HD, 4)) * 0.5, A_log=rng.uniform(-2, 1, H),
                dt_bias=rng.uniform(-1, 1, HD), norm_w=np.ones(D))
    c = oracle.MixerConfig(head_dim=D)
    a = oracle.forward(c, [0, T], args["q"], args["k"], args["v"], z_direct, args["b"], args["g"], args["conv_w"],
                       args["A_log"], args["dt_bias"], args["norm_w"])
    b = oracle.forward(c, [0, T], args["q"], args["k"], args["v"], None, args["b"], args["g"], args["conv_w"],
                       args["A_log"], args["dt_bias"], args["norm_w"], gate_proj=(f, w_fb))
    for h in range(H):
        np.testing.assert_array_equal(a[(0, h)].out, b[(0, h)].out)
        np.testing.assert_array_equal(a[(0, h)].state, b[(0, h)].state)


def test_gate_projection_matches_explicit_sums():
    """A dense factor of rank 8 against logits summed term by term in Python (no matrix
    routine): z[t, h*D + i] = sum_r w_fb[h*D + i, r] f[t, r]."""
    rng = np.random.default_rng(32)
    D, H, T, R = 8, 2, 5, 8
    HD = H * D
    w_fb = rng.standard_normal((HD, R)) / np.sqrt(R)
    f = rng.standard_normal((T, R))
    z = np.zeros((T, HD))
    for t in range(T):
        for c in range(HD):
            acc = 0.0
            for r in range(R):
                acc += w_fb[c, r] * f[t, r]
            z[t, c] = acc
    args = [rng.standard_normal((T, HD)) for _ in range(3)]
    b, g = rng.standard_normal((T, H)), rng.standard_normal((T, HD))
    prm = [rng.standard_normal((3 * HD, 4)) * 0.5, rng.uniform(-2, 1, H), rng.uniform(-1, 1, HD), np.ones(D)]
    c = oracle.MixerConfig(head_dim=D)
    a = oracle.forward(c, [0, T], *args, z, b, g, *prm)
    bb = oracle.forward(c, [0, T], *args, None, b, g, *prm, gate_proj=(f, w_fb))
    for h in range(H):
        np.testing.assert_allclose(bb[(0, h)].out, a[(0, h)].out, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(bb[(0, h)].state, a[(0, h)].state, rtol=1e-12, atol=1e-14)
