"""GPU check of the "auto" attention mode (dark_prf_auto_fwd).

README section "Attention modes": exact attention through exact_threshold,
linear attention beyond it.  On both sides of the threshold the output is
compared with the matching oracle (exact_kernel_attention or attention) and
with the direct call of the path that was taken (same kernels: identical
results).
"""
import numpy as np
import pytest

import oracle
from random_feature_linear_amd import binding as bd
from random_feature_linear_amd.workloads import Workload, make_inputs
from tests.gpu_harness import TOL, device_inputs, host, oracle_omega, say
from tests.metrics import normwise_rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [False, True])
def test_auto_both_sides_of_threshold(causal):
    import torch
    w = Workload(name="auto", B=2, H=4, H_kv=2, L=300, d_h=64, m=256, r=64, dtype="bf16", causal=causal,
                 seed=808, m_kind="eye_noise", m_noise=0.3, mask_kind="tail", max_pad=80)
    inp = make_inputs(w)
    dev = device_inputs(w, inp)
    tag = bd.dark_prf_proj_tag(w.seed, w.m, w.r, w.orthogonal)
    args = (dev["q"], dev["k"], dev["v"], dev["M"], dev["omega"])
    for thr, exact in ((300, True), (4096, True), (299, False), (0, False)):
        say(f"[auto] L=300 threshold={thr} causal={causal}: expect {'exact' if exact else 'linear'}")
        got = bd.auto_attention(*args, exact_threshold=thr, mask=dev["mask"], causal=causal, proj_tag=tag)
        if exact:
            direct = bd.exact_attention(dev["q"], dev["k"], dev["v"], dev["M"], mask=dev["mask"], causal=causal)
            ref = oracle.exact_kernel_attention(inp["q"], inp["k"], inp["v"], inp["M"], mask=inp["mask"],
                                                causal=causal)
        else:
            direct = bd.prf_attention(*args, mask=dev["mask"], causal=causal, proj_tag=tag)
            ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["M"], oracle_omega(w), mask=inp["mask"],
                                   causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(got, direct)
        err = normwise_rel_err(host(got), ref)
        say(f"[auto] threshold={thr}: normwise rel err {err:.3e}")
        assert err <= TOL["bf16"], err
    # the linear and exact results differ (the linear one is the m-feature estimate)
    lin = bd.auto_attention(*args, exact_threshold=0, mask=dev["mask"], causal=causal, proj_tag=tag)
    ex = bd.auto_attention(*args, exact_threshold=300, mask=dev["mask"], causal=causal, proj_tag=tag)
    assert not torch.equal(lin, ex)
    assert np.all(np.isfinite(host(lin))) and np.all(np.isfinite(host(ex)))
