"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Element-by-element on seeded inputs at sizes the oracle finishes in seconds
(several tiles and ragged tails), and at the five workloads' full sizes on
sampled (batch, head) slices or sampled query rows.  Error metric: per
(batch, head) slice, max |Y - Y_ref| / max |Y_ref|, max over slices; bound
1e-4 for fp32 inputs and 2e-2 for bf16 inputs with fp32 accumulation.
"""
import zlib

import numpy as np
import pytest

import oracle
from random_feature_linear_amd import binding as bd
from random_feature_linear_amd.workloads import CONFIGS, Workload, make_decode_tokens, make_inputs
from tests.gpu_harness import TOL, device_inputs, host, oracle_omega, run_device, say
from tests.metrics import normwise_rel_err

pytestmark = pytest.mark.gpu


def _check(w: Workload, L=None, rows=None, heads=None, qrows=None, tol=None):
    say(f"[parity] {w.name} L={L or w.L} dtype={w.dtype} causal={w.causal}")
    inp = make_inputs(w, L=L, rows=rows)
    dev = device_inputs(w, inp)
    out = host(run_device(w, dev))
    om = oracle_omega(w)
    if qrows is not None:      # non-causal only: query rows are independent
        ref = oracle.attention(inp["q"][:, :, qrows], inp["k"], inp["v"], inp["M"], om,
                               mask=inp["mask"], causal=False)
        got = out[:, :, qrows]
    elif heads is not None:
        ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["M"], om, mask=inp["mask"],
                               causal=w.causal, heads=heads)
        bsel = [b for b, _ in heads]
        hsel = [h for _, h in heads]
        got, ref = out[bsel, hsel], ref[bsel, hsel]
    else:
        ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["M"], om, mask=inp["mask"],
                               causal=w.causal)
        got = out
    err = normwise_rel_err(got, ref)
    bound = TOL[w.dtype] if tol is None else tol
    say(f"[parity] {w.name}: normwise rel err {err:.3e} (bound {bound:.0e})")
    assert np.all(np.isfinite(got))
    assert err <= bound, err
    return err


# ---- small shapes: every tile path, ragged tails, masks, GQA, shared M -------
SMALL = [
    # name,            dtype,  B, H, Hkv, L,   d_h, m,   r,   causal, per_head, orth, mask
    ("f32_d16_nc",     "f32",  1, 1, 1,   128, 16,  32,  16,  False, True,  False, "none"),
    ("f32_d16_c",      "f32",  2, 2, 1,   100, 16,  32,  16,  True,  True,  True,  "random"),
    ("f32_d32_nc_mask", "f32", 2, 3, 3,   77,  32,  48,  8,   False, False, True,  "random"),
    ("f32_d64_c",      "f32",  1, 4, 2,   300, 64,  64,  64,  True,  True,  True,  "tail"),
    ("bf16_d64_nc",    "bf16", 2, 4, 4,   333, 64,  256, 64,  False, True,  True,  "tail"),
    ("bf16_d64_c",     "bf16", 2, 4, 4,   333, 64,  256, 64,  True,  True,  True,  "tail"),
    ("bf16_d64_c_L1",  "bf16", 3, 2, 2,   1,   64,  64,  64,  True,  True,  True,  "none"),
    ("bf16_d64_nc_L5", "bf16", 2, 2, 1,   5,   64,  64,  30,  False, True,  False, "random"),
    ("bf16_d32_c_r100", "bf16", 1, 4, 2,  200, 32,  96,  100, True,  True,  True,  "random"),
    ("bf16_d128_c",    "bf16", 1, 2, 1,   260, 128, 128, 128, True,  True,  True,  "tail"),
    ("bf16_d128_nc",   "bf16", 1, 2, 2,   700, 128, 160, 16,  False, False, False, "none"),
    ("bf16_d256_c",    "bf16", 1, 2, 1,   200, 256, 64,  256, True,  True,  True,  "none"),
    ("bf16_d256_nc",   "bf16", 1, 2, 1,   150, 256, 32,  200, False, True,  True,  "random"),
    ("bf16_d16_c_m16", "bf16", 2, 2, 2,   130, 16,  16,  16,  True,  True,  True,  "random"),
    ("bf16_d64_c_m48", "bf16", 1, 2, 2,   150, 64,  48,  64,  True,  True,  True,  "tail"),
    ("f32_d128_nc",    "f32",  1, 2, 2,   90,  128, 64,  32,  False, True,  True,  "tail"),
    # many heads and chunks, masked tail, two feature slices; the key side takes
    # two chunks per workgroup (11 chunks: the last group holds one)
    ("bf16_d64_c_many", "bf16", 16, 8, 8,  1300, 64,  512, 64,  True,  True,  True,  "tail"),
    # folded exponent with two feature slices: key shifts computed once up front
    ("bf16_d64_nc_m512", "bf16", 1, 2, 1,  300, 64,  512, 64,  False, True,  True,  "random"),
    ("f32_d256_c",     "f32",  1, 1, 1,   70,  256, 32,  64,  True,  True,  True,  "none"),
    # the eight-wave causal query side with 1, 5 and 7 feature steps (each half's
    # first step copied up front, the others staged through registers)
    ("bf16_d64_c_fb1", "bf16", 1, 2, 2,   300, 64,  32,  64,  True,  True,  True,  "tail"),
    ("bf16_d64_c_fb5", "bf16", 2, 2, 1,   260, 64,  160, 64,  True,  True,  True,  "tail"),
    ("bf16_d64_c_fb7", "bf16", 1, 3, 3,   390, 64,  224, 64,  True,  True,  False, "random"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small(case):
    name, dt, B, H, Hkv, L, dh, m, r, causal, ph, orth, mk = case
    w = Workload(name=name, B=B, H=H, H_kv=Hkv, L=L, d_h=dh, m=m, r=r, dtype=dt, causal=causal,
                 per_head_geometry=ph, orthogonal=orth, seed=zlib.crc32(name.encode()) % 100000,
                 m_kind="eye_noise", m_noise=0.3, x_kind="iid", mask_kind=mk, max_pad=L // 3)
    _check(w)


# ---- the five workloads --------------------------------------------------------
def test_c1_tiny_f32():
    _check(CONFIGS["c1_tiny_f32"])


def test_c2_causal_L2048_full():
    _check(CONFIGS["c2_causal_L2048"])


def test_c3_long_reduced_L4096():
    _check(CONFIGS["c3_long_L64K"], L=4096)


def test_c3_long_L64K_sampled_rows():
    rng = np.random.default_rng(3)
    qrows = np.sort(rng.choice(65536, size=384, replace=False))
    qrows[0], qrows[-1] = 0, 65535
    _check(CONFIGS["c3_long_L64K"], qrows=qrows)


def test_c4_gqa_L8192_sampled_heads():
    # eight chunks per key-side workgroup at this size
    _check(CONFIGS["c4_gqa_L8192"], heads=[(0, 0), (1, 3), (3, 7)])


# ---- recurrent state: export, decode, prefill + decode == full causal ----------
def _state_case(dt="bf16", H=4, Hkv=2, L=300, dh=64, m=128, r=32, B=2):
    return Workload(name="state", B=B, H=H, H_kv=Hkv, L=L, d_h=dh, m=m, r=r, dtype=dt, causal=True,
                    seed=77, m_kind="eye_noise", m_noise=0.3, mask_kind="tail", max_pad=40)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_state_export(dt):
    w = _state_case(dt)
    say(f"[state] export dtype={dt}")
    inp = make_inputs(w)
    dev = device_inputs(w, inp)
    out, S, z = run_device(w, dev, return_state=True)
    ref, S_ref, z_ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["M"], oracle_omega(w),
                                         mask=inp["mask"], causal=True, return_state=True)
    assert normwise_rel_err(host(out), ref) <= TOL[dt]
    assert normwise_rel_err(host(S), S_ref) <= TOL[dt]
    assert normwise_rel_err(host(z), z_ref, axes=(-1,)) <= TOL[dt]


def _device_rows(w: Workload, L: int, sample_rows):
    """Device q, k, v for every batch row, uploaded row by row; host copies of `sample_rows`."""
    import torch
    from tests.gpu_harness import torch_dtype
    dt = torch_dtype(w.dtype)
    shape_q = (w.B, w.H, L, w.d_h)
    shape_kv = (w.B, w.hkv, L, w.d_h)
    dev = {"q": torch.empty(shape_q, dtype=dt, device="cuda:0"),
           "k": torch.empty(shape_kv, dtype=dt, device="cuda:0"),
           "v": torch.empty(shape_kv, dtype=dt, device="cuda:0")}
    keep = {"q": [], "k": [], "v": []}
    M = None
    for b in range(w.B):
        row = make_inputs(w, L=L, rows=[b])
        M = row["M"]
        for n in ("q", "k", "v"):
            dev[n][b].copy_(torch.from_numpy(row[n][0]).to(dt))
            if b in sample_rows:
                keep[n].append(row[n][0])
    host_inp = {n: np.stack(keep[n]) for n in keep}
    host_inp["M"] = M
    host_inp["mask"] = None
    dev["M"] = torch.from_numpy(M).to("cuda:0")
    dev["omega"] = torch.from_numpy(bd.dark_prf_omega(w.seed, w.m, w.r, w.orthogonal)).to("cuda:0")
    return dev, host_inp


def _decode_run(w: Workload, P: int, T: int, sample_rows):
    """GPU: prefill P tokens for every sequence with state export, then T decode steps.

    Returns host inputs and decode tokens of `sample_rows` and the device results
    (outputs [N][H][T][d_h], S, z) of those rows."""
    import torch
    dev, inp = _device_rows(w, P, sample_rows)
    tag = bd.dark_prf_proj_tag(w.seed, w.m, w.r, w.orthogonal)
    _, S, z = bd.prf_attention(dev["q"], dev["k"], dev["v"], dev["M"], dev["omega"], mask=None,
                               causal=True, return_state=True, proj_tag=tag)
    tok = make_decode_tokens(w, T)
    dt = dev["q"].dtype
    tq = torch.from_numpy(tok["q"]).to(dt).to("cuda:0")
    tk = torch.from_numpy(tok["k"]).to(dt).to("cuda:0")
    tv = torch.from_numpy(tok["v"]).to(dt).to("cuda:0")
    outs = []
    for t in range(T):
        outs.append(bd.decode_step(tq[t], tk[t], tv[t], dev["M"], dev["omega"], S, z, tag, tag))
    o = torch.stack(outs, dim=2)        # [N][H][T][d_h]
    torch.cuda.synchronize()
    sel = list(sample_rows)
    tok_s = {n: tok[n][:, sel] for n in tok}
    return inp, tok_s, host(o[sel]), host(S[sel]), host(z[sel])


def _decode_ref(w, inp, tok, heads):
    full_q = np.concatenate([inp["q"], tok["q"].transpose(1, 2, 0, 3)], axis=2)
    full_k = np.concatenate([inp["k"], tok["k"].transpose(1, 2, 0, 3)], axis=2)
    full_v = np.concatenate([inp["v"], tok["v"].transpose(1, 2, 0, 3)], axis=2)
    return oracle.attention(full_q, full_k, full_v, inp["M"], oracle_omega(w), causal=True,
                            heads=heads, return_state=True)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_decode_small(dt):
    w = Workload(name="dec", B=3, H=4, H_kv=2, L=0, d_h=32, m=64, r=16, dtype=dt, causal=True,
                 seed=91, m_kind="eye_noise", m_noise=0.3)
    say(f"[decode] small dtype={dt}")
    P, T = 45, 9
    inp, tok, o, S, z = _decode_run(w, P, T, [0, 1, 2])
    heads = [(b, h) for b in range(3) for h in range(4)]
    ref, S_ref, z_ref = _decode_ref(w, inp, tok, heads)
    assert normwise_rel_err(o, ref[:, :, P:]) <= TOL[dt]
    assert normwise_rel_err(S, S_ref) <= TOL[dt]
    assert normwise_rel_err(z, z_ref, axes=(-1,)) <= TOL[dt]


DECODE_SHAPES = {
    # two sequences per workgroup with a ragged last group, a rank that is not a
    # multiple of 4 and m not a multiple of 32
    "bf16_d16_B65_r7_m48": dict(B=65, H=2, H_kv=1, d_h=16, m=48, r=7, dtype="bf16"),
    # d_h = 256: the state is streamed in three 64-row slices, the last one partial
    "bf16_d256_B70_m160": dict(B=70, H=2, H_kv=2, d_h=256, m=160, r=40, dtype="bf16"),
    "f32_d128_B66_m96": dict(B=66, H=1, H_kv=1, d_h=128, m=96, r=100, dtype="f32"),
}


@pytest.mark.parametrize("name", sorted(DECODE_SHAPES))
def test_decode_shapes(name):
    cfg = DECODE_SHAPES[name]
    w = Workload(name="dec_" + name, L=0, causal=True, seed=93, m_kind="eye_noise", m_noise=0.3,
                 **cfg)
    rows = [0, 33, w.B - 1]
    say(f"[decode] {name}: B={w.B} H={w.H} d={w.d_h} m={w.m} r={w.r}; oracle on rows {rows}")
    P, T = 20, 3
    inp, tok, o, S, z = _decode_run(w, P, T, rows)
    heads = [(i, h) for i in range(len(rows)) for h in range(w.H)]
    ref, S_ref, z_ref = _decode_ref(w, inp, tok, heads)
    err_o = normwise_rel_err(o, ref[:, :, P:])
    say(f"[decode] {name}: output err {err_o:.3e}")
    assert err_o <= TOL[w.dtype]
    assert normwise_rel_err(S, S_ref) <= TOL[w.dtype]
    assert normwise_rel_err(z, z_ref, axes=(-1,)) <= TOL[w.dtype]


def test_c5_decode_sampled():
    """Workload 5 in its launch shape: 256 sequences x 8 heads, 4096-token prefill with state
    export, then 512 decode steps; sequences 0, 77 and 255 are checked against the oracle."""
    w = CONFIGS["c5_decode"]
    rows = [0, 77, 255]
    say("[decode] c5: 256 x 8 heads, prefill 4096 + 512 steps; oracle on sequences 0, 77, 255")
    inp, tok, o, S, z = _decode_run(w, w.L, 512, rows)
    heads = [(i, h) for i in range(len(rows)) for h in (0, 3, 7)]
    ref, S_ref, z_ref = _decode_ref(w, inp, tok, heads)
    bsel = [b for b, _ in heads]
    hsel = [h for _, h in heads]
    err_o = normwise_rel_err(o[bsel, hsel], ref[bsel, hsel, w.L:])
    err_s = normwise_rel_err(S[bsel, hsel], S_ref[bsel, hsel])
    err_z = normwise_rel_err(z[bsel, hsel], z_ref[bsel, hsel], axes=(-1,))
    say(f"[decode] c5 output err {err_o:.3e}, S err {err_s:.3e}, z err {err_z:.3e}")
    assert err_o <= TOL["bf16"] and err_s <= TOL["bf16"] and err_z <= TOL["bf16"]


# ---- many causal chunks ---------------------------------------------------------
def test_causal_many_chunks():
    """33 chunks of 128 keys with a masked tail: the chunk-state prefix over many units."""
    w = Workload(name="chunks33", B=1, H=2, H_kv=1, L=4200, d_h=64, m=128, r=64, dtype="bf16", causal=True,
                 seed=99, m_kind="eye_noise", m_noise=0.3, mask_kind="tail", max_pad=300)
    _check(w)


# ---- invariants on the device --------------------------------------------------
def test_deterministic_and_row0():
    import torch
    w = CONFIGS["c2_causal_L2048"].with_(L=512)
    say("[invariant] determinism and causal row 0")
    inp = make_inputs(w)
    dev = device_inputs(w, inp)
    a = run_device(w, dev)
    b = run_device(w, dev)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # causal row 0 sees only key 0: output = v_0 (rounded to the output dtype)
    v0 = dev["v"][:, :, 0]
    assert torch.equal(a[:, :, 0].float(), v0.float())


def test_strided_layout_matches_contiguous():
    import torch
    w = Workload(name="strided", B=2, H=4, L=200, d_h=64, m=128, r=64, dtype="bf16", causal=True,
                 seed=5, m_kind="eye_noise", m_noise=0.3)
    say("[invariant] [B][L][H][d] strided views")
    inp = make_inputs(w)
    dev = device_inputs(w, inp)
    ref = run_device(w, dev)
    # same values stored as [B][L][H][d]; the kernels read through the strides
    blhd = {n: dev[n].transpose(1, 2).contiguous().transpose(1, 2) for n in ("q", "k", "v")}
    out = torch.empty(2, 200, 4, 64, dtype=torch.bfloat16, device="cuda:0").transpose(1, 2)
    tag = bd.dark_prf_proj_tag(w.seed, w.m, w.r, w.orthogonal)
    bd.prf_attention(blhd["q"], blhd["k"], blhd["v"], dev["M"], dev["omega"], causal=True,
                     proj_tag=tag, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_masked_equals_deleted():
    import torch
    w = Workload(name="maskdel", B=1, H=2, L=300, d_h=64, m=128, r=64, dtype="f32", causal=False,
                 seed=6, m_kind="eye_noise", m_noise=0.3)
    say("[invariant] masked key == deleted key")
    inp = make_inputs(w)
    dev = device_inputs(w, inp)
    keep = np.ones(300, dtype=np.uint8)
    keep[[3, 50, 51, 52, 299]] = 0
    dev["mask"] = torch.from_numpy(keep[None]).to("cuda:0")
    a = run_device(w, dev)
    idx = torch.from_numpy(np.nonzero(keep)[0]).to("cuda:0")
    dev2 = dict(dev, k=dev["k"][:, :, idx].contiguous(), v=dev["v"][:, :, idx].contiguous(), mask=None)
    # non-causal: the query count may differ from the key count only through this path,
    # so compare on queries drawn as keys were: rebuild q with the same length as k
    dev2["q"] = dev["q"][:, :, idx].contiguous()
    b = run_device(w.with_(L=int(keep.sum())), dev2)
    torch.cuda.synchronize()
    assert normwise_rel_err(host(a)[:, :, np.nonzero(keep)[0]], host(b)) <= 1e-5


def test_graph_replay_matches_eager():
    """The forward captured in a HIP graph gives the eager result on every replay."""
    import torch
    w = CONFIGS["c2_causal_L2048"].with_(L=700)
    say("[graph] capture + 4 replays vs eager")
    inp = make_inputs(w)
    dev = device_inputs(w, inp)
    eager = run_device(w, dev).clone()
    tag = bd.dark_prf_proj_tag(w.seed, w.m, w.r, w.orthogonal)
    out = torch.empty_like(eager)
    desc = bd.make_desc(dev["q"], dev["k"], dev["v"], out, dev["M"], dev["omega"], True, tag)
    ws = torch.empty(bd.dark_prf_workspace_bytes(desc), dtype=torch.uint8, device="cuda:0")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            st = bd.dark_prf_fwd(desc, dev["q"].data_ptr(), dev["k"].data_ptr(), dev["v"].data_ptr(),
                                 dev["M"].data_ptr(), dev["omega"].data_ptr(), dev["mask"].data_ptr(),
                                 out.data_ptr(), 0, 0, ws.data_ptr(), ws.numel(),
                                 torch.cuda.current_stream().cuda_stream)
            assert st == bd.DARK_OK
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        ws.fill_(0x7F)                      # stale workspace must not leak into results
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        run_device(w, dev)                  # eager work between replays
        torch.cuda.synchronize()


# ---- key rows far outside the fp16 range of the exponent operands ---------------
# The bf16 path holds the exponent's operands in fp16, clamped to +-65504.  A key
# row scaled by 1e6 has |u|^2 / 2 of order 1e12, so its feature is exactly 0 in
# the oracle; the kernels form |u|^2 / 2 in fp32 from the unclamped projection,
# so the key gets weight 0 there too and every output stays finite.
HUGE = [
    # name,              L,   d_h, m,   r,  causal  (r = 64: folded exponent; r = 16: unfolded)
    ("huge_fold_c",      200, 64,  128, 64, True),
    ("huge_fold_nc",     200, 64,  128, 64, False),
    ("huge_unfold_nc",   300, 64,  256, 16, False),
]


@pytest.mark.parametrize("case", HUGE, ids=[c[0] for c in HUGE])
def test_huge_key_rows_get_zero_weight(case):
    from random_feature_linear_amd.workloads import round_bf16
    name, L, dh, m, r, causal = case
    w = Workload(name=name, B=2, H=2, H_kv=2, L=L, d_h=dh, m=m, r=r, dtype="bf16", causal=causal,
                 per_head_geometry=True, orthogonal=True, seed=zlib.crc32(name.encode()) % 100000,
                 m_kind="eye_noise", m_noise=0.3, x_kind="iid", mask_kind="none")
    say(f"[parity] {name} L={L} r={r} causal={causal}: key rows scaled by 1e6")
    inp = make_inputs(w)
    rows = [3, 77, L - 1]
    k = inp["k"].astype(np.float64)
    k[:, :, rows, :] *= 1e6
    inp["k"] = round_bf16(k.astype(np.float32)).astype(inp["k"].dtype)
    assert np.max(np.abs(inp["k"])) > 1e5
    out = host(run_device(w, device_inputs(w, inp)))
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["M"], oracle_omega(w), mask=inp["mask"], causal=causal)
    err = normwise_rel_err(out, ref)
    say(f"[parity] {name}: normwise rel err {err:.3e}")
    assert np.all(np.isfinite(out))
    assert err <= TOL["bf16"], err
