"""GPU tests of kda_state_copy: photos of pool entries into host memory (pinned and
pageable) and their restore into other entries are exact copies, copies inside one pool
run in slot-list order, and decoding resumed from a restored photo gives the same bits as
the uninterrupted run."""
import numpy as np
import pytest
import torch

import gated_delta_rule_31_amd as kda
import kda_inputs as ki
from tests.parity import t

pytestmark = pytest.mark.gpu

D = 128


def _pool(seed, P, H, dev):
    rng = np.random.default_rng(seed)
    st = rng.standard_normal((P, H, D, D), dtype=np.float32) * np.float32(0.05)
    cs = rng.standard_normal((P, 3 * H * D, 3), dtype=np.float32)
    return t(st, dev), t(cs, dev)


@pytest.mark.parametrize("pinned", [True, False])
def test_photo_to_host_and_restore(device, pinned):
    H, P = 4, 7
    print(f"[state-copy] photo/restore H={H} P={P} pinned={pinned}", flush=True)
    cfg = kda.KdaConfig(num_heads=H)
    state, conv = _pool(330, P, H, device)
    ref_s, ref_c = state.clone(), conv.clone()
    photo_s = torch.full((3, H, D, D), float("nan"), dtype=torch.float32, pin_memory=pinned)
    photo_c = torch.full((3, 3 * H * D, 3), float("nan"), dtype=torch.float32, pin_memory=pinned)
    kda.kda_state_copy(cfg, state, conv, [4, 1, 5], photo_s, photo_c, [0, 1, 2])
    torch.cuda.synchronize()
    for i, e in enumerate([4, 1, 5]):
        assert torch.equal(photo_s[i], ref_s[e].cpu()) and torch.equal(photo_c[i], ref_c[e].cpu()), e
    state.fill_(7.0)
    conv.fill_(7.0)
    kda.kda_state_copy(cfg, photo_s, photo_c, [2, 0, 1], state, conv, [6, 0, 3])
    torch.cuda.synchronize()
    for src, dst in zip([5, 4, 1], [6, 0, 3]):
        assert torch.equal(state[dst], ref_s[src]) and torch.equal(conv[dst], ref_c[src]), dst
    for e in (1, 2, 4, 5):  # entries not named as destinations are untouched
        assert (state[e] == 7.0).all() and (conv[e] == 7.0).all(), e


def test_copies_inside_one_pool_run_in_order(device):
    H, P = 2, 5
    print(f"[state-copy] in-pool chain H={H} P={P}", flush=True)
    cfg = kda.KdaConfig(num_heads=H)
    state, conv = _pool(331, P, H, device)
    ref_s, ref_c = state.clone(), conv.clone()
    # 0 -> 1, then 1 -> 2 (sees the new entry 1), and an entry onto itself
    kda.kda_state_copy(cfg, state, conv, [0, 1, 3], state, conv, [1, 2, 3])
    torch.cuda.synchronize()
    for e, src in ((0, 0), (1, 0), (2, 0), (3, 3), (4, 4)):
        assert torch.equal(state[e], ref_s[src]) and torch.equal(conv[e], ref_c[src]), e


def test_decode_resumes_from_a_photo(device):
    """A slot's state is photographed after 3 decode steps; the run continues for 3 more
    steps, the photo is restored into another slot and the same 3 steps are decoded from
    there: outputs and final states agree bit for bit."""
    case = ki.decode_case(332, 3, 4, 6, "photo-resume")
    H = case.H
    print(f"[state-copy] resume B={case.B} H={H}", flush=True)
    cfg = kda.KdaConfig(num_heads=H)
    p = case.params
    prm = [t(p.conv_w, device), t(p.A_log, device), t(p.dt_bias, device), t(p.norm_w, device)]
    P = 2 * case.B
    state = torch.zeros((P, H, D, D), dtype=torch.float32, device=device)
    conv = torch.zeros((P, 3 * H * D, 3), dtype=torch.float32, device=device)
    state[:case.B] = t(case.state, device)
    conv[:case.B] = t(case.conv_state, device)
    home = torch.arange(case.B, dtype=torch.int32, device=device)
    twin = home + case.B

    def step(i, slots):
        x = case.step(i)
        xs = [t(getattr(x, n), device) for n in "qkvzbg"]
        return kda.kda_decode_step_slots(cfg, slots, *xs, *prm, state, conv)

    for i in range(3):
        step(i, home)
    photo_s = torch.empty((case.B, H, D, D), dtype=torch.float32, pin_memory=True)
    photo_c = torch.empty((case.B, 3 * H * D, 3), dtype=torch.float32, pin_memory=True)
    kda.kda_state_copy(cfg, state, conv, list(range(case.B)), photo_s, photo_c, list(range(case.B)))
    first = [step(i, home).clone() for i in range(3, 6)]
    kda.kda_state_copy(cfg, photo_s, photo_c, list(range(case.B)), state, conv, list(range(case.B, P)))
    second = [step(i, twin).clone() for i in range(3, 6)]
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a, b)
    assert torch.equal(state[:case.B], state[case.B:]) and torch.equal(conv[:case.B], conv[case.B:])


def test_conv_only_restore_into_a_shared_state_pool(device):
    """The state entry maps onto itself (same buffer, same slot) while the conv windows
    come from another buffer: the windows are still copied, the state left as it is."""
    H, P = 3, 4
    print(f"[state-copy] conv-only restore H={H} P={P}", flush=True)
    cfg = kda.KdaConfig(num_heads=H)
    state, conv = _pool(332, P, H, device)
    _, conv_photo = _pool(333, P, H, device)
    ref_s = state.clone()
    kda.kda_state_copy(cfg, state, conv_photo, [2, 1], state, conv, [2, 1])
    torch.cuda.synchronize()
    assert torch.equal(state, ref_s)
    for e in (1, 2):
        assert torch.equal(conv[e], conv_photo[e]), e
