"""GPU parity of the exact learned-kernel attention through the C ABI.

dark_prf_exact_fwd evaluates softmax attention on u = d_h^(-1/4) M_h x for
queries and keys (package README, section "Attention modes": the exact mode
applies the learned geometry to q and k and runs softmax attention).  The
reference is the oracle's exact_kernel_attention, itself pinned against
PyTorch's scaled_dot_product_attention in fp64.  Error metric and bounds as in
test_gpu_parity.
"""
import zlib

import numpy as np
import pytest

import oracle
from random_feature_linear_amd import binding as bd
from random_feature_linear_amd.workloads import CONFIGS, Workload, make_inputs
from tests.gpu_harness import TOL, host, say, to_dev, torch_dtype
from tests.metrics import normwise_rel_err

pytestmark = pytest.mark.gpu

CASES = [
    # name,               dtype,  B, H, Hkv, L,   d_h, r,   causal, per_head, mask
    ("exact_f32_d16_nc",  "f32",  1, 2, 2,   77,  16,  16,  False, True,  "random"),
    ("exact_f32_d64_c",   "f32",  1, 2, 1,   150, 64,  64,  True,  True,  "tail"),
    ("exact_bf16_d32_c",  "bf16", 2, 2, 1,   100, 32,  16,  True,  True,  "random"),
    ("exact_bf16_d64_nc", "bf16", 2, 4, 2,   333, 64,  64,  False, True,  "tail"),
    ("exact_bf16_d64_L1", "bf16", 3, 2, 2,   1,   64,  64,  True,  True,  "none"),
    ("exact_bf16_d64_L33", "bf16", 1, 4, 4,  33,  64,  30,  True,  False, "none"),
    ("exact_bf16_d128_nc", "bf16", 1, 2, 2,  260, 128, 128, False, False, "random"),
    ("exact_bf16_d256_c", "bf16", 1, 2, 1,   150, 256, 200, True,  True,  "random"),
    ("exact_bf16_d16_c",  "bf16", 2, 2, 2,   130, 16,  16,  True,  True,  "tail"),
    # few (b, h) x query tiles: the keys of a tile split into runs of 2 key tiles
    # and combined (9 key tiles: runs of 2, 2, 2, 2, 1)
    ("exact_split_nc",    "bf16", 1, 2, 1,   1100, 64, 64,  False, True,  "random"),
    ("exact_split_c",     "bf16", 1, 4, 2,   1500, 64, 48,  True,  True,  "tail"),
    ("exact_split_f32_c", "f32",  1, 1, 1,   700,  32, 16,  True,  False, "random"),
]


def _run(w, inp):
    import torch
    dt = torch_dtype(w.dtype)
    mask = to_dev(inp["mask"]) if inp["mask"] is not None else None
    out = bd.exact_attention(to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
                             to_dev(inp["M"], torch.float32), mask=mask, causal=w.causal)
    torch.cuda.synchronize()
    return host(out)


def _check(w, L=None, heads=None):
    inp = make_inputs(w, L=L)
    out = _run(w, inp)
    if heads is None:
        ref = oracle.exact_kernel_attention(inp["q"], inp["k"], inp["v"], inp["M"], mask=inp["mask"],
                                            causal=w.causal)
        got = out
    else:
        bs, hs = [b for b, _ in heads], [h for _, h in heads]
        q = inp["q"][bs, hs][:, None]
        g = [(h * w.hkv) // w.H for h in hs]
        k, v = inp["k"][bs, g][:, None], inp["v"][bs, g][:, None]
        M = inp["M"][hs][:, None] if inp["M"].ndim == 3 else inp["M"]
        ref = np.concatenate([oracle.exact_kernel_attention(q[i:i + 1], k[i:i + 1], v[i:i + 1],
                                                            M[i] if inp["M"].ndim == 3 else M,
                                                            mask=None if inp["mask"] is None else
                                                            inp["mask"][bs[i]:bs[i] + 1],
                                                            causal=w.causal) for i in range(len(heads))])
        got = out[bs, hs][:, None]
    err = normwise_rel_err(got, ref)
    bound = TOL[w.dtype]
    say(f"[exact] {w.name}: normwise rel err {err:.3e} (bound {bound:.0e})")
    assert np.all(np.isfinite(got))
    assert err <= bound, err
    return out, inp


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_exact_parity(case):
    name, dt, B, H, Hkv, L, dh, r, causal, ph, mk = case
    w = Workload(name=name, B=B, H=H, H_kv=Hkv, L=L, d_h=dh, m=16, r=r, dtype=dt, causal=causal,
                 per_head_geometry=ph, seed=zlib.crc32(name.encode()) % 100000, m_kind="eye_noise",
                 m_noise=0.3, x_kind="iid", mask_kind=mk, max_pad=max(1, L // 3))
    _check(w)


def test_exact_c2_shape():
    """The L=2048 causal workload's inputs (padded tails, anisotropic q and k)."""
    _check(CONFIGS["c2_causal_L2048"])


def test_exact_c4_shape_sampled_heads():
    """The L=8192 GQA workload's inputs, d_h = r = 256, on three (batch, head) pairs."""
    _check(CONFIGS["c4_gqa_L8192"], heads=[(0, 0), (1, 3), (3, 7)])


def test_exact_fully_masked_row_is_zero():
    w = Workload(name="exact_masked", B=2, H=2, L=70, d_h=64, m=16, r=64, dtype="bf16", causal=False,
                 seed=5, mask_kind="none")
    inp = make_inputs(w)
    inp["mask"] = np.ones((2, 70), dtype=np.uint8)
    inp["mask"][1] = 0
    out = _run(w, inp)
    assert np.all(out[1] == 0.0) and np.all(np.isfinite(out[0])) and np.any(out[0] != 0.0)
