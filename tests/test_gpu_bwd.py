"""GPU parity of the backward pass through the C ABI against the fp64 oracle.

dark_prf_bwd returns the gradients of sum(dout * out) with respect to q, k, v
and M for the forward dark_prf_fwd computes (package README section "Kernel":
M is learned).  The reference is oracle.attention_backward, itself pinned
against central finite differences of the oracle's forward.  Each gradient is
compared with the normwise relative error of test_gpu_parity (per (b, h)
slice for dq, dk, dv; over the whole tensor for dM) and the same bounds.
"""
import zlib

import numpy as np
import pytest

import oracle
from random_feature_linear_amd import binding as bd
from random_feature_linear_amd.workloads import CONFIGS, Workload, make_inputs
from tests.gpu_harness import TOL, device_inputs, host, oracle_omega, say, to_dev, torch_dtype
from tests.metrics import normwise_rel_err

pytestmark = pytest.mark.gpu

CASES = [
    # name,               dtype,  B, H, Hkv, L,   d_h, m,   r,   causal, per_head, orth,  mask
    ("bwd_bf16_d64_c",    "bf16", 2, 4, 2,   200, 64,  128, 64,  True,  True,  True,  "tail"),
    ("bwd_f32_d32_nc",    "f32",  2, 2, 1,   150, 32,  48,  16,  False, False, False, "random"),
    ("bwd_f32_d64_c",     "f32",  1, 2, 2,   130, 64,  64,  64,  True,  True,  True,  "random"),
    ("bwd_bf16_d16_L1",   "bf16", 3, 2, 2,   1,   16,  32,  16,  True,  True,  True,  "none"),
    ("bwd_f32_d128_c",    "f32",  1, 2, 1,   97,  128, 32,  100, True,  True,  False, "tail"),
    ("bwd_bf16_d256_nc",  "bf16", 1, 4, 1,   100, 256, 64,  200, False, True,  True,  "random"),
    ("bwd_bf16_L700_c",   "bf16", 1, 2, 1,   700, 64,  64,  32,  True,  False, True,  "tail"),
    ("bwd_f32_m512_nc",   "f32",  1, 1, 1,   260, 64,  512, 64,  False, True,  True,  "none"),
    ("bwd_f32_d16_gqa4",  "f32",  1, 8, 2,   90,  16,  32,  8,   True,  False, True,  "random"),
    ("bwd_f32_r1_m16",    "f32",  2, 2, 2,   75,  32,  16,  1,   True,  True,  False, "tail"),
    ("bwd_c1_shape",      "f32",  1, 1, 1,   128, 16,  32,  16,  False, True,  False, "none"),
]


def _dout(w, shape):
    import torch
    rng = np.random.default_rng(zlib.crc32((w.name + "/dout").encode()))
    g = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    return g.to(torch_dtype(w.dtype)).to(torch.float64).numpy()


def _run(w, inp, dout):
    import torch
    dev = device_inputs(w, inp)
    g = to_dev(dout, torch_dtype(w.dtype))
    dq, dk, dv, dM = bd.prf_attention_backward(dev["q"], dev["k"], dev["v"], dev["M"], dev["omega"], g,
                                               mask=dev["mask"], causal=w.causal)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv), host(dM)


def _err(a, b, floor):
    """Normwise relative error, the denominator floored at `floor`: where a
    gradient vanishes analytically (one visible key makes out = v whatever q
    and k are) the oracle's value is rounding noise and the error is measured
    against the largest gradient entry of the call instead."""
    return float(np.max(np.abs(a - b))) / max(float(np.max(np.abs(b))), floor) if a.size else 0.0


def _compare(name, got, ref, bound, per_slice=True):
    floor = 1e-4 * max(float(np.max(np.abs(r))) for r in ref)
    errs = []
    for n, a, b in zip(("dq", "dk", "dv", "dM"), got, ref):
        if per_slice and n != "dM":
            e = max(_err(a[i, j], b[i, j], floor) for i in range(a.shape[0]) for j in range(a.shape[1]))
        else:
            e = _err(a, b, floor)
        errs.append(e)
        assert np.all(np.isfinite(a)), n
    say(f"[bwd] {name}: dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e} dM {errs[3]:.2e} (bound {bound:.0e})")
    assert max(errs) <= bound, errs


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_parity(case):
    name, dt, B, H, Hkv, L, dh, m, r, causal, ph, orth, mk = case
    w = Workload(name=name, B=B, H=H, H_kv=Hkv, L=L, d_h=dh, m=m, r=r, dtype=dt, causal=causal,
                 per_head_geometry=ph, orthogonal=orth, seed=zlib.crc32(name.encode()) % 100000,
                 m_kind="eye_noise", m_noise=0.3, x_kind="iid", mask_kind=mk, max_pad=max(1, L // 3))
    inp = make_inputs(w)
    dout = _dout(w, inp["q"].shape)
    say(f"[bwd] {name} B={B} H={H}/{Hkv} L={L} d_h={dh} m={m} r={r} causal={causal}")
    got = _run(w, inp, dout)
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["M"], oracle_omega(w), dout,
                                    mask=inp["mask"], causal=causal)
    _compare(name, got, ref, TOL[dt])
    if inp["mask"] is not None:   # masked keys get exactly zero dk and dv
        for b in range(B):
            off = inp["mask"][b] == 0
            assert np.all(got[1][b][:, off] == 0) and np.all(got[2][b][:, off] == 0)


def test_bwd_c2_shape_sampled_heads():
    """The L=2048 causal workload's inputs; all (b, h) run on the device, the
    oracle checks heads 0 and 5 over both batch rows (dM of a head sums over b)."""
    w = CONFIGS["c2_causal_L2048"]
    assert w.hkv == w.H and w.per_head_geometry
    inp = make_inputs(w)
    dout = _dout(w, inp["q"].shape)
    got = _run(w, inp, dout)
    om = oracle_omega(w)
    for h in (0, 5):
        sl = lambda x: x[:, h:h + 1]
        ref = oracle.attention_backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), inp["M"][h:h + 1], om,
                                        sl(dout), mask=inp["mask"], causal=True)
        _compare(f"c2 head {h}", [sl(got[0]), sl(got[1]), sl(got[2]), got[3][h:h + 1]], ref, TOL[w.dtype])


def test_bwd_fully_masked_and_empty():
    import torch
    w = Workload(name="bwd_masked", B=2, H=2, L=70, d_h=64, m=64, r=32, dtype="bf16", causal=False,
                 seed=9, mask_kind="none")
    inp = make_inputs(w)
    inp["mask"] = np.ones((2, 70), dtype=np.uint8)
    inp["mask"][1] = 0                       # batch row 1: no valid key, outputs fixed at 0
    dout = _dout(w, inp["q"].shape)
    dq, dk, dv, dM = _run(w, inp, dout)
    assert np.all(dq[1] == 0) and np.all(dk[1] == 0) and np.all(dv[1] == 0)
    assert np.any(dq[0] != 0) and np.all(np.isfinite(dM))
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["M"], oracle_omega(w), dout,
                                    mask=inp["mask"], causal=False)
    assert normwise_rel_err(dM, ref[3]) <= TOL["bf16"]
    # L = 0: nothing to differentiate, dM = 0
    dev = device_inputs(w, inp)
    e = torch.zeros((2, 2, 0, 64), dtype=torch.bfloat16, device="cuda:0")
    g = bd.prf_attention_backward(e, e, e, dev["M"], dev["omega"], e, causal=True)
    torch.cuda.synchronize()
    assert float(g[3].abs().max()) == 0.0 and g[0].numel() == 0
    # B = 0: likewise
    e0 = torch.zeros((0, 2, 70, 64), dtype=torch.bfloat16, device="cuda:0")
    g0 = bd.prf_attention_backward(e0, e0, e0, dev["M"], dev["omega"], e0, causal=False)
    torch.cuda.synchronize()
    assert float(g0[3].abs().max()) == 0.0


def test_bwd_single_token():
    """L = 1: out = v exactly, so dv = dout and dq, dk, dM vanish up to rounding."""
    w = Workload(name="bwd_one", B=3, H=2, H_kv=1, L=1, d_h=64, m=64, r=32, dtype="f32", causal=True, seed=4,
                 mask_kind="none")
    inp = make_inputs(w)
    dout = _dout(w, inp["q"].shape)
    dq, dk, dv, dM = _run(w, inp, dout)
    assert np.max(np.abs(dv - dout.sum(axis=1, keepdims=True))) <= 1e-6 * np.max(np.abs(dout))
    for g in (dq, dk, dM):
        assert np.max(np.abs(g)) <= 1e-4 * np.max(np.abs(dout)), np.max(np.abs(g))


def test_bwd_packed_qkv_strides():
    """q, k and v as views of one packed [B][L][3][H][d_h] tensor: the gradients
    take the views' strides and equal those of the contiguous call bit for bit."""
    import torch
    w = Workload(name="bwd_packed", B=2, H=4, L=150, d_h=64, m=64, r=32, dtype="bf16", causal=True, seed=21,
                 mask_kind="tail", max_pad=40)
    inp = make_inputs(w)
    dev = device_inputs(w, inp)
    packed = torch.empty((2, 150, 3, 4, 64), dtype=torch.bfloat16, device="cuda:0")
    views = [packed[:, :, i].permute(0, 2, 1, 3) for i in range(3)]   # [B][H][L][d_h], rows 3*H*d_h apart
    for vw, n in zip(views, ("q", "k", "v")):
        vw.copy_(dev[n])
    g = to_dev(_dout(w, inp["q"].shape), torch.bfloat16)
    got = bd.prf_attention_backward(*views, dev["M"], dev["omega"], g, mask=dev["mask"], causal=True)
    ref = bd.prf_attention_backward(dev["q"], dev["k"], dev["v"], dev["M"], dev["omega"], g, mask=dev["mask"],
                                    causal=True)
    torch.cuda.synchronize()
    assert got[0].stride() == views[0].stride() and got[2].stride() == views[2].stride()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


def test_bwd_c3_full_size():
    """The L=64K non-causal workload at its full size: every (b, h) on the
    device; the oracle's linear-time form checks dq, dk, dv of heads 0 and 5 and
    the shared dM, which sums all eight heads."""
    w = CONFIGS["c3_long_L64K"]
    assert not w.causal and not w.per_head_geometry and w.hkv == w.H and w.B == 1
    inp = make_inputs(w)
    dout = _dout(w, inp["q"].shape)
    got = _run(w, inp, dout)
    om = oracle_omega(w)
    key_mask = None if inp["mask"] is None else inp["mask"][0]
    dM = np.zeros_like(got[3])
    for h in range(w.H):
        ref = oracle.attention_backward_noncausal_head(inp["q"][0, h], inp["k"][0, h], inp["v"][0, h], inp["M"], om,
                                                       dout[0, h], key_mask=key_mask)
        dM += ref[3]
        if h in (0, 5):
            floor = 1e-4 * max(float(np.max(np.abs(r))) for r in ref[:3])
            errs = [_err(got[i][0, h], ref[i], floor) for i in range(3)]
            say(f"[bwd] c3 head {h}: dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")
            assert max(errs) <= TOL[w.dtype], errs
    e = normwise_rel_err(got[3], dM)
    say(f"[bwd] c3 dM over all heads: {e:.2e}")
    assert e <= TOL[w.dtype]


def test_bwd_c4_batch_row():
    """The L=8192 GQA workload at its full size: all (b, h) on the device; the
    dense oracle checks batch row 0 (its eight query heads share one key/value
    head, so dk and dv of that row sum all eight)."""
    w = CONFIGS["c4_gqa_L8192"]
    assert w.hkv == 1 and w.causal
    inp = make_inputs(w)
    dout = _dout(w, inp["q"].shape)
    got = _run(w, inp, dout)
    sl = lambda x: x[0:1]
    ref = oracle.attention_backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), inp["M"], oracle_omega(w), sl(dout),
                                    mask=None if inp["mask"] is None else sl(inp["mask"]), causal=True)
    floor = 1e-4 * max(float(np.max(np.abs(r))) for r in ref[:3])
    errs = [max(_err(sl(got[i])[0, j], ref[i][0, j], floor) for j in range(ref[i].shape[1])) for i in range(3)]
    say(f"[bwd] c4 batch row 0: dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")
    assert max(errs) <= TOL[w.dtype], errs
    # dM sums the batch: the device backward of batch row 0 alone against the oracle's
    # (the same launch shape per row: r = d_h = 256, 128-token chunks, per-head M)
    one = {n: sl(inp[n]) for n in ("q", "k", "v")}
    one.update(M=inp["M"], mask=None if inp["mask"] is None else sl(inp["mask"]))
    got1 = _run(w.with_(B=1), one, sl(dout))
    e = normwise_rel_err(got1[3], ref[3])
    say(f"[bwd] c4 batch row 0: dM {e:.2e}")
    assert e <= TOL[w.dtype], e
