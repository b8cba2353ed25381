"""GPU parity of cross-attention through the C ABI against the fp64 oracle.

dark_prf_context_state summarises a context (keys and values of length L_k
with a context mask) as (S, z); dark_prf_cross_fwd applies that summary to
queries of length L_q with a separate query mask (package README, section
"Cross-attention"; section "Encoder-decoder model and generation" for the
once-per-layer source summary).  The context and the queries are drawn from
the same seeded workload recipe at two lengths: the geometry M is shared, the
context mask is the key mask of the L_k draw and the query mask is the key
mask of the L_q draw.  Error metric and bounds as in test_gpu_parity.
"""
import zlib

import numpy as np
import pytest

import oracle
from random_feature_linear_amd import binding as bd
from random_feature_linear_amd.workloads import Workload, make_inputs
from tests.gpu_harness import TOL, host, oracle_omega, say, to_dev, torch_dtype
from tests.metrics import normwise_rel_err

pytestmark = pytest.mark.gpu

CASES = [
    # name,                dtype,  B, H, Hkv, Lq,  Lk,   d_h, m,   r,   per_head, orth, cmask,    qmask
    ("cross_pages_example", "bf16", 2, 8, 2,   256, 1024, 64,  256, 64,  True,  True,  "tail",   "random"),
    ("cross_f32_d32",      "f32",  1, 2, 1,   77,  300,  32,  48,  16,  False, False, "random", "random"),
    ("cross_bf16_m512",    "bf16", 1, 4, 4,   130, 700,  64,  512, 64,  True,  True,  "random", "none"),
    ("cross_bf16_step",    "bf16", 3, 4, 2,   1,   200,  64,  256, 64,  True,  True,  "tail",   "none"),
    ("cross_bf16_d256",    "bf16", 1, 2, 1,   100, 150,  256, 64,  200, True,  True,  "random", "random"),
    ("cross_bf16_d128_shared", "bf16", 1, 2, 2, 200, 333, 128, 160, 16, False, False, "none",   "tail"),
    # one query per sequence (a decoder step): the single pass over the fp32 summary,
    # two sequences per workgroup from 64 sequences on
    ("cross_step_B80",     "bf16", 80, 4, 2,  1,   300,  64,  256, 64,  True,  True,  "tail",   "random"),
    ("cross_step_f32_d128", "f32", 66, 2, 1,  1,   90,   128, 96,  100, True,  True,  "random", "random"),
]


def _workload(name, dt, B, H, Hkv, dh, m, r, ph, orth, mask_kind, L):
    return Workload(name=name, B=B, H=H, H_kv=Hkv, L=L, d_h=dh, m=m, r=r, dtype=dt, causal=False,
                    per_head_geometry=ph, orthogonal=orth, seed=zlib.crc32(name.encode()) % 100000,
                    m_kind="eye_noise", m_noise=0.3, x_kind="iid", mask_kind=mask_kind,
                    max_pad=max(1, L // 3))


def _draw(case):
    name, dt, B, H, Hkv, Lq, Lk, dh, m, r, ph, orth, cm, qm = case
    wk = _workload(name, dt, B, H, Hkv, dh, m, r, ph, orth, cm, Lk)
    wq = _workload(name, dt, B, H, Hkv, dh, m, r, ph, orth, qm, Lq)
    ctx = make_inputs(wk)
    qry = make_inputs(wq)
    assert np.array_equal(ctx["M"], qry["M"])
    return wk, ctx, qry


def _run(wk, ctx, qry, context_mask=True, query_mask=True):
    import torch
    dt = torch_dtype(wk.dtype)
    tag = bd.dark_prf_proj_tag(wk.seed, wk.m, wk.r, wk.orthogonal)
    om = to_dev(bd.dark_prf_omega(wk.seed, wk.m, wk.r, wk.orthogonal), torch.float32)
    M = to_dev(ctx["M"], torch.float32)
    cmask = to_dev(ctx["mask"]) if (context_mask and ctx["mask"] is not None) else None
    qmask = to_dev(qry["mask"]) if (query_mask and qry["mask"] is not None) else None
    S, z = bd.context_state(to_dev(ctx["k"], dt), to_dev(ctx["v"], dt), M, om, wk.H, context_mask=cmask,
                            proj_tag=tag)
    out = bd.cross_attention(to_dev(qry["q"], dt), M, om, S, z, state_tag=tag, proj_tag=tag,
                             query_mask=qmask, H_kv=wk.hkv)
    torch.cuda.synchronize()
    return host(S), host(z), host(out)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cross_parity(case):
    wk, ctx, qry = _draw(case)
    say(f"[cross] {case[0]} Lq={case[5]} Lk={case[6]} dtype={wk.dtype}")
    S, z, out = _run(wk, ctx, qry)
    om = oracle_omega(wk)
    S_ref, z_ref = oracle.context_state(ctx["k"], ctx["v"], ctx["M"], om, wk.H, context_mask=ctx["mask"])
    ref = oracle.cross_attention(qry["q"], S_ref, z_ref, ctx["M"], om, query_mask=qry["mask"])
    bound = TOL[wk.dtype]
    e_S = normwise_rel_err(S, S_ref)
    e_z = normwise_rel_err(z[..., None], z_ref[..., None])
    e_o = normwise_rel_err(out, ref)
    say(f"[cross] {case[0]}: S {e_S:.3e}  z {e_z:.3e}  out {e_o:.3e} (bound {bound:.0e})")
    assert np.all(np.isfinite(out))
    assert e_S <= bound and e_z <= bound and e_o <= bound
    if qry["mask"] is not None:   # masked query rows are exactly 0
        rows = out.transpose(0, 2, 1, 3)[qry["mask"] == 0]   # [rows][H][d_h]
        assert np.all(rows == 0.0)


def test_cross_empty_and_fully_masked_context():
    import torch
    case = ("cross_empty", "bf16", 2, 2, 1, 40, 96, 64, 64, 32, True, True, "none", "none")
    wk, ctx, qry = _draw(case)
    ctx["mask"] = np.ones((2, 96), dtype=np.uint8)
    ctx["mask"][1] = 0                         # batch row 1: no valid context token
    S, z, out = _run(wk, ctx, qry)
    assert np.all(S[1] == 0.0) and np.all(z[1] == 0.0) and np.all(out[1] == 0.0)
    assert np.all(np.isfinite(out[0])) and np.any(out[0] != 0.0)
    # L_k = 0: an all-zero summary and outputs of 0
    tag = bd.dark_prf_proj_tag(wk.seed, wk.m, wk.r, wk.orthogonal)
    om = to_dev(bd.dark_prf_omega(wk.seed, wk.m, wk.r, wk.orthogonal), torch.float32)
    M = to_dev(ctx["M"], torch.float32)
    k0 = torch.zeros((2, 1, 0, 64), dtype=torch.bfloat16, device="cuda:0")
    S0, z0 = bd.context_state(k0, k0, M, om, 2, proj_tag=tag)
    out0 = bd.cross_attention(to_dev(qry["q"], torch.bfloat16), M, om, S0, z0, state_tag=tag, proj_tag=tag,
                              H_kv=1)
    torch.cuda.synchronize()
    assert float(S0.abs().max()) == 0.0 and float(z0.abs().max()) == 0.0
    assert float(out0.float().abs().max()) == 0.0


def test_cross_equals_self_attention_on_one_sequence():
    """Queries against the summary of their own sequence: the non-causal forward.
    With one feature slice neither path takes the separate shift pass, and the
    summary reaches the query side through the same roundings, so the outputs
    are bit-identical."""
    import torch
    case = ("cross_self", "bf16", 2, 4, 2, 300, 300, 64, 256, 64, True, True, "tail", "none")
    wk, ctx, _ = _draw(case)
    dt = torch_dtype(wk.dtype)
    tag = bd.dark_prf_proj_tag(wk.seed, wk.m, wk.r, wk.orthogonal)
    om = to_dev(bd.dark_prf_omega(wk.seed, wk.m, wk.r, wk.orthogonal), torch.float32)
    M = to_dev(ctx["M"], torch.float32)
    q, k, v = to_dev(ctx["q"], dt), to_dev(ctx["k"], dt), to_dev(ctx["v"], dt)
    mask = to_dev(ctx["mask"])
    self_out = bd.prf_attention(q, k, v, M, om, mask=mask, causal=False, proj_tag=tag)
    S, z = bd.context_state(k, v, M, om, wk.H, context_mask=mask, proj_tag=tag)
    cross_out = bd.cross_attention(q, M, om, S, z, state_tag=tag, proj_tag=tag, H_kv=wk.hkv)
    torch.cuda.synchronize()
    assert torch.equal(self_out, cross_out)


def test_cross_rejects_stale_summary():
    import torch
    case = ("cross_stale", "bf16", 1, 2, 2, 8, 16, 64, 64, 32, True, True, "none", "none")
    wk, ctx, qry = _draw(case)
    tag = bd.dark_prf_proj_tag(wk.seed, wk.m, wk.r, wk.orthogonal)
    om = to_dev(bd.dark_prf_omega(wk.seed, wk.m, wk.r, wk.orthogonal), torch.float32)
    M = to_dev(ctx["M"], torch.float32)
    S, z = bd.context_state(to_dev(ctx["k"], torch.bfloat16), to_dev(ctx["v"], torch.bfloat16), M, om, 2,
                            proj_tag=tag)
    with pytest.raises(bd.DarkPrfError) as ei:
        bd.cross_attention(to_dev(qry["q"], torch.bfloat16), M, om, S, z, state_tag=tag ^ 1, proj_tag=tag,
                           H_kv=2)
    assert ei.value.status == bd.DARK_ERR_STALE_STATE
