"""GPU parity with one projection omega per query head ([H][m][r]).

Each case gives the device the library's per-head projections
(dark_prf_omega_per_head) and the oracle its own (oracle.omega_per_head); the
two generators are compared on the host in test_abi_host.py.  Covered: the
folded exponent (per-head and shared geometry), the unfolded one, d_h = 16
(element-wise fold), the one-block-at-a-time key side (fp32, d_h = 256), causal
and not, GQA, masks; the state export and decode steps; cross-attention; the
backward.  Error metric and bounds as in test_gpu_parity.py.
"""
import zlib

import numpy as np
import pytest

import oracle
from random_feature_linear_amd import binding as bd
from random_feature_linear_amd.workloads import Workload, make_decode_tokens, make_inputs
from tests.gpu_harness import TOL, host, say, to_dev, torch_dtype
from tests.metrics import normwise_rel_err
from tests.test_gpu_bwd import _compare

pytestmark = pytest.mark.gpu


def _omegas(w):
    dev = bd.dark_prf_omega_per_head(w.seed, w.H, w.m, w.r, w.orthogonal)
    ref = oracle.omega_per_head(w.seed, w.H, w.m, w.r, w.orthogonal)
    return dev, ref


CASES = [
    # name,                dtype,  B, H, Hkv, L,   d_h, m,   r,  causal, per_head_M, mask
    ("fold_c_gqa",         "bf16", 2, 4, 2,   333, 64,  256, 64, True,   True,  "tail"),
    ("fold_nc_sharedM",    "bf16", 1, 4, 4,   300, 64,  128, 64, False,  False, "random"),
    ("fold_c_sharedM",     "bf16", 2, 2, 1,   260, 128, 96,  128, True,  False, "tail"),
    ("unfold_nc",          "bf16", 1, 4, 2,   700, 64,  512, 16, False,  False, "random"),
    ("unfold_c",           "bf16", 2, 2, 2,   200, 64,  64,  16, True,   True,  "none"),
    ("d16_fold_c",         "bf16", 2, 2, 1,   150, 16,  64,  16, True,   True,  "random"),
    ("f32_nc",             "f32",  1, 3, 3,   77,  32,  48,  8,  False,  True,  "random"),
    ("f32_d256_seq_c",     "f32",  1, 2, 1,   70,  256, 32,  64, True,   True,  "none"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_per_head_forward(case):
    name, dt, B, H, Hkv, L, dh, m, r, causal, phM, mk = case
    w = Workload(name=name, B=B, H=H, H_kv=Hkv, L=L, d_h=dh, m=m, r=r, dtype=dt, causal=causal,
                 per_head_geometry=phM, orthogonal=True, seed=zlib.crc32(name.encode()) % 100000,
                 m_kind="eye_noise", m_noise=0.3, mask_kind=mk, max_pad=L // 3)
    say(f"[per-head omega] {name}: B={B} H={H}/{Hkv} L={L} d={dh} m={m} r={r} causal={causal}")
    inp = make_inputs(w)
    om_dev, om_ref = _omegas(w)
    tdt = torch_dtype(dt)
    q, k, v = (to_dev(inp[n], tdt) for n in ("q", "k", "v"))
    M = to_dev(inp["M"])
    om = to_dev(om_dev)
    mask = to_dev(inp["mask"]) if inp["mask"] is not None else None
    tag = bd.dark_prf_proj_tag_per_head(w.seed, H, m, r, True)
    res = bd.prf_attention(q, k, v, M, om, mask=mask, causal=causal, return_state=causal, proj_tag=tag)
    out = res[0] if causal else res
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["M"], om_ref, mask=inp["mask"], causal=causal,
                           return_state=causal)
    ref_out = ref[0] if causal else ref
    err = normwise_rel_err(host(out), ref_out)
    say(f"[per-head omega] {name}: normwise rel err {err:.3e}")
    assert err <= TOL[dt], err
    if causal:
        assert normwise_rel_err(host(res[1]), ref[1]) <= TOL[dt]
        assert normwise_rel_err(host(res[2]), ref[2], axes=(-1,)) <= TOL[dt]
    # with every head given the same projection, the result is the shared-omega one
    rep = to_dev(np.stack([om_dev[0]] * H))
    a = bd.prf_attention(q, k, v, M, rep, mask=mask, causal=causal, proj_tag=tag)
    b = bd.prf_attention(q, k, v, M, to_dev(om_dev[0]), mask=mask, causal=causal, proj_tag=tag)
    assert normwise_rel_err(host(a), host(b)) <= 1e-6


def test_per_head_decode():
    import torch
    w = Workload(name="ph_dec", B=5, H=4, H_kv=2, L=40, d_h=64, m=128, r=32, dtype="bf16", causal=True,
                 seed=313, m_kind="eye_noise", m_noise=0.3)
    say("[per-head omega] prefill 40 + 6 decode steps")
    inp = make_inputs(w)
    om_dev, om_ref = _omegas(w)
    q, k, v = (to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    M, om = to_dev(inp["M"]), to_dev(om_dev)
    tag = bd.dark_prf_proj_tag_per_head(w.seed, w.H, w.m, w.r, True)
    _, S, z = bd.prf_attention(q, k, v, M, om, causal=True, return_state=True, proj_tag=tag)
    T = 6
    tok = make_decode_tokens(w, T)
    outs = []
    for t in range(T):
        step = [torch.from_numpy(tok[n][t]).to(torch.bfloat16).to("cuda:0") for n in ("q", "k", "v")]
        outs.append(bd.decode_step(step[0], step[1], step[2], M, om, S, z, tag, tag))
    o = host(torch.stack(outs, dim=2))
    # a state made with the shared projection's tag is rejected
    with pytest.raises(bd.DarkPrfError):
        bd.decode_step(step[0], step[1], step[2], M, om, S, z, bd.dark_prf_proj_tag(w.seed, w.m, w.r, True), tag)
    full = {n: np.concatenate([inp[n], tok[n].transpose(1, 2, 0, 3)], axis=2) for n in ("q", "k", "v")}
    ref, S_ref, z_ref = oracle.attention(full["q"], full["k"], full["v"], inp["M"], om_ref, causal=True,
                                         return_state=True)
    assert normwise_rel_err(o, ref[:, :, w.L:]) <= TOL["bf16"]
    assert normwise_rel_err(host(S), S_ref) <= TOL["bf16"]
    assert normwise_rel_err(host(z), z_ref, axes=(-1,)) <= TOL["bf16"]


def test_per_head_cross_attention():
    w = Workload(name="ph_cross", B=2, H=4, H_kv=2, L=200, d_h=64, m=256, r=64, dtype="bf16", causal=False,
                 seed=314, m_kind="eye_noise", m_noise=0.3, mask_kind="tail", max_pad=60)
    wq = w.with_(L=77, mask_kind="random", max_pad=20, seed=315)
    say("[per-head omega] cross-attention L_q=77 against L_k=200")
    ctx, qry = make_inputs(w), make_inputs(wq)
    om_dev, om_ref = _omegas(w)
    import torch
    k, v = to_dev(ctx["k"], torch.bfloat16), to_dev(ctx["v"], torch.bfloat16)
    q = to_dev(qry["q"], torch.bfloat16)
    M, om = to_dev(ctx["M"]), to_dev(om_dev)
    tag = bd.dark_prf_proj_tag_per_head(w.seed, w.H, w.m, w.r, True)
    S, z = bd.context_state(k, v, M, om, w.H, context_mask=to_dev(ctx["mask"]), proj_tag=tag)
    out = bd.cross_attention(q, M, om, S, z, tag, tag, query_mask=to_dev(qry["mask"]), H_kv=w.H)
    S_ref, z_ref = oracle.context_state(ctx["k"], ctx["v"], ctx["M"], om_ref, w.H, context_mask=ctx["mask"])
    ref = oracle.cross_attention(qry["q"], S_ref, z_ref, ctx["M"], om_ref, query_mask=qry["mask"])
    assert normwise_rel_err(host(S), S_ref) <= TOL["bf16"]
    assert normwise_rel_err(host(out), ref) <= TOL["bf16"]


def test_per_head_backward():
    w = Workload(name="ph_bwd", B=2, H=4, H_kv=2, L=150, d_h=32, m=64, r=16, dtype="f32", causal=True,
                 seed=316, m_kind="eye_noise", m_noise=0.3, mask_kind="tail", max_pad=30)
    say("[per-head omega] backward, causal, GQA")
    inp = make_inputs(w)
    om_dev, om_ref = _omegas(w)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    M, om = to_dev(inp["M"]), to_dev(om_dev)
    rng = np.random.default_rng(317)
    g = rng.standard_normal(inp["q"].shape).astype(np.float32)
    grads = bd.prf_attention_backward(q, k, v, M, om, to_dev(g), mask=to_dev(inp["mask"]), causal=True)
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["M"], om_ref, g, mask=inp["mask"],
                                    causal=True)
    _compare("per-head omega", [host(a) for a in grads], ref, TOL["f32"])
