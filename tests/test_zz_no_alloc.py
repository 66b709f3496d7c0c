"""kda_prefill_noalloc (the chunked layout's workspace in the library's per-device scratch
array) gives exactly the bits of kda_prefill with a caller workspace: two calls in a row,
the second on a smaller batch, on the chunked layout (the scratch in use) and on the
automatic choice, which falls back to the fused layout when the records would not fit."""
import numpy as np
import pytest
import torch

import gated_delta_rule_31_amd as kda
import kda_inputs as ki
from tests.parity import PATH_AUTO, PATH_CHUNKED, t

pytestmark = pytest.mark.gpu


def _both(case, device, path):
    p = case.params
    prm = [t(p.conv_w, device), t(p.A_log, device), t(p.dt_bias, device), t(p.norm_w, device)]
    cfg = kda.KdaConfig(num_heads=case.H, prefill_path=path)
    cu = t(case.cu_seqlens.astype(np.int32), device)
    xs = [t(getattr(case.x, n), device) for n in "qkvzbg"]
    st, cs = t(case.initial_state, device), t(case.initial_conv_state, device)
    ref = kda.kda_prefill(cfg, cu, *xs, *prm, st, cs)
    torch.cuda.synchronize()
    N, HD, B = case.N, case.H * 128, case.B
    out = torch.full((N, HD), float("nan"), device=device)
    fs = torch.full((B, case.H, 128, 128), float("nan"), device=device)
    fcs = torch.full((B, 3 * HD, 3), float("nan"), device=device)
    got = kda.kda_prefill_noalloc(cfg, cu, *xs, *prm, st, cs, out=out, final_state=fs, final_conv_state=fcs)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("path", [pytest.param(PATH_CHUNKED, id="chunked"), pytest.param(PATH_AUTO, id="auto")])
def test_noalloc_matches_prefill_on_two_calls(device, path):
    cases = [ki.prefill_case(700, 8, [700, 300, 129, 0], True, "noalloc-first"),
             ki.prefill_case(701, 8, [100, 64], True, "noalloc-second")]
    for case in cases:
        need = kda.kda_prefill_workspace_bytes(kda.KdaConfig(num_heads=8, prefill_path=PATH_CHUNKED), case.B, case.N)
        print(f"[noalloc] {case.name} path={path} B={case.B} N={case.N} H={case.H} chunked workspace {need}",
              flush=True)
        assert 0 < need <= 256 << 20
        ref, got = _both(case, device, path)
        for a, b in zip(ref, got):
            assert torch.equal(a, b)


def test_noalloc_auto_falls_back_to_fused_past_the_scratch(device):
    # one 4096-token sequence x 96 heads: the chunked layout would need 65 x 96 records
    # (697 MB); the automatic choice runs the fused layout, which gives the same bits
    case = ki.prefill_case(702, 96, [4096], True, "noalloc-large")
    need = kda.kda_prefill_workspace_bytes(kda.KdaConfig(num_heads=96, prefill_path=PATH_CHUNKED), 1, 4096)
    print(f"[noalloc] {case.name} chunked workspace {need}", flush=True)
    assert need > 256 << 20
    ref, got = _both(case, device, PATH_AUTO)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    with pytest.raises(kda.KdaError) as e:
        _both(case, device, PATH_CHUNKED)
    assert e.value.status == 5  # KDA_ERR_WORKSPACE
