"""The forward that allocates nothing (dark_prf_fwd_noalloc) against dark_prf_fwd.

Both entry points run the same kernels; the no-allocation one takes its
workspace from the library's static per-GPU buffer.  Two calls in a row, the
second on a smaller input, each compared with dark_prf_fwd on the same inputs
(and with the fp64 oracle), through the C ABI.
"""
import numpy as np
import pytest

import oracle
from random_feature_linear_amd import binding as bd
from random_feature_linear_amd.workloads import Workload, make_inputs
from tests.gpu_harness import TOL, device_inputs, host, oracle_omega, say
from tests.metrics import normwise_rel_err

pytestmark = pytest.mark.gpu


def _call_both(w):
    import torch
    inp = make_inputs(w)
    dev = device_inputs(w, inp)
    tag = bd.dark_prf_proj_tag(w.seed, w.m, w.r, w.orthogonal)
    ref_dev = bd.prf_attention(dev["q"], dev["k"], dev["v"], dev["M"], dev["omega"], mask=dev["mask"],
                               causal=w.causal, return_state=w.causal, proj_tag=tag)
    out = torch.full_like(dev["q"], float("nan"))
    B, H = w.B, w.H
    S = torch.full((B, H, w.m, w.d_h), float("nan"), dtype=torch.float32, device="cuda:0") if w.causal else None
    z = torch.full((B, H, w.m), float("nan"), dtype=torch.float32, device="cuda:0") if w.causal else None
    desc = bd.make_desc(dev["q"], dev["k"], dev["v"], out, dev["M"], dev["omega"], w.causal, tag)
    assert bd.dark_prf_workspace_bytes(desc) <= bd.DARK_PRF_SCRATCH_BYTES
    st = bd.dark_prf_fwd_noalloc(desc, dev["q"].data_ptr(), dev["k"].data_ptr(), dev["v"].data_ptr(),
                                 dev["M"].data_ptr(), dev["omega"].data_ptr(),
                                 dev["mask"].data_ptr() if dev["mask"] is not None else 0, out.data_ptr(),
                                 S.data_ptr() if S is not None else 0, z.data_ptr() if z is not None else 0,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == bd.DARK_OK, bd.status_str(st)
    torch.cuda.synchronize()
    got = host(out)
    if w.causal:
        ref_out, ref_S, ref_z = (host(t) for t in ref_dev)
        assert np.array_equal(host(S), ref_S)
        assert np.array_equal(host(z), ref_z)
    else:
        ref_out = host(ref_dev)
    # the same kernels on the same inputs: identical results
    assert np.array_equal(got, ref_out)
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["M"], oracle_omega(w), mask=inp["mask"],
                           causal=w.causal)
    err = normwise_rel_err(got, ref)
    say(f"[noalloc] {w.name}: normwise rel err vs oracle {err:.3e}")
    assert err <= TOL[w.dtype]


def test_noalloc_two_calls_second_smaller():
    big = Workload(name="noalloc_big", B=2, H=8, L=2048, d_h=64, m=256, r=64, dtype="bf16", causal=True,
                   seed=4242, m_kind="eye_noise", m_noise=0.3, mask_kind="tail", max_pad=256)
    small = Workload(name="noalloc_small", B=1, H=2, H_kv=1, L=300, d_h=64, m=128, r=32, dtype="bf16",
                     causal=False, seed=4243, m_kind="eye_noise", m_noise=0.3, mask_kind="random", max_pad=60)
    say("[noalloc] first call: B=2 H=8 L=2048 causal")
    _call_both(big)
    say("[noalloc] second call: B=1 H=2 L=300 non-causal, smaller")
    _call_both(small)


def test_noalloc_rejects_oversize():
    import torch
    w = Workload(name="noalloc_huge", B=64, H=8, L=8192, d_h=64, m=256, r=64, dtype="bf16", causal=True)
    q = torch.empty((1, 1, 16, 64), dtype=torch.bfloat16, device="cuda:0")
    d = bd.make_desc(q, q, q, q, torch.empty((8, 64, 64)), torch.empty((256, 64)), True, 0)
    d.B, d.H, d.H_kv, d.L = w.B, w.H, w.H, w.L
    for name in ("q_str", "k_str", "v_str", "o_str"):
        getattr(d, name)[:] = [w.H * w.L * 64, w.L * 64, 64]
    assert bd.dark_prf_workspace_bytes(d) > bd.DARK_PRF_SCRATCH_BYTES
    st = bd.dark_prf_fwd_noalloc(d, q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), 0,
                                 q.data_ptr(), 0, 0, torch.cuda.current_stream().cuda_stream)
    assert st == bd.DARK_ERR_WORKSPACE
