"""Host-side tests of the C ABI: symbols, validation, workspace sizing, Omega.

No kernel runs here: every call below returns before anything is queued.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import omega_gen as oo
from random_feature_linear_amd import binding as bd

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "darkprf.h")
FAKE = 1 << 20          # an aligned, never dereferenced stand-in for a device address


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dark_prf_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) == 27, names
    L = bd.lib()
    for n in names:
        assert hasattr(L, n), n


def _desc(**kw):
    d = bd.DarkPrfDesc()
    base = dict(B=2, H=8, H_kv=8, L=256, d_h=64, m=256, r=64, dtype=bd.DARK_BF16, causal=1, m_per_head=1)
    base.update(kw)
    for k, v in base.items():
        if not k.endswith("_str"):
            setattr(d, k, v)
    L, dh, H = base["L"], base["d_h"], base["H"]
    for name, heads in (("q_str", H), ("k_str", base["H_kv"]), ("v_str", base["H_kv"]), ("o_str", H)):
        getattr(d, name)[:] = kw.get(name, [heads * L * dh, L * dh, dh])
    return d


def _fwd(d, ws_bytes=None, S=0, z=0, mask=0, ws=FAKE):
    nb = bd.dark_prf_workspace_bytes(d) if ws_bytes is None else ws_bytes
    return bd.dark_prf_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, mask, FAKE, S, z, ws, nb, 0)


@pytest.mark.parametrize("kw", [
    dict(H=8, H_kv=3), dict(d_h=48), dict(d_h=512), dict(m=24), dict(m=0), dict(r=0), dict(r=257),
    dict(dtype=7), dict(causal=2), dict(m_per_head=3), dict(B=-1), dict(H=0),
    dict(q_str=[8 * 256 * 64, 256 * 64, 60]),      # rows overlap
    dict(k_str=[8 * 256 * 64, 256 * 64, 68]),      # 136-byte rows: not 16-byte aligned
])
def test_invalid_descriptors(kw):
    d = _desc(**kw)
    assert _fwd(d, ws_bytes=1 << 40) == bd.DARK_ERR_INVALID_ARG
    assert bd.dark_prf_workspace_bytes(d) == 0


def test_null_and_misaligned_pointers():
    d = _desc()
    nb = bd.dark_prf_workspace_bytes(d)
    assert bd.dark_prf_fwd(d, 0, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 0, FAKE, nb, 0) == bd.DARK_ERR_INVALID_ARG
    assert bd.dark_prf_fwd(d, FAKE + 2, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 0, FAKE, nb, 0) == bd.DARK_ERR_INVALID_ARG
    assert bd.dark_prf_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 0, 0, FAKE, nb, 0) == bd.DARK_ERR_INVALID_ARG


def test_workspace_checks():
    d = _desc()
    nb = bd.dark_prf_workspace_bytes(d)
    assert nb > 0
    assert _fwd(d, ws_bytes=nb - 1) == bd.DARK_ERR_WORKSPACE
    assert _fwd(d, ws=0) == bd.DARK_ERR_WORKSPACE
    # more tokens never need less workspace
    assert bd.dark_prf_workspace_bytes(_desc(L=4096)) >= nb


def test_noalloc_rejects_before_touching_a_device():
    # an invalid descriptor, and a call whose workspace exceeds the static buffer,
    # return before the library looks up its buffer or queues anything
    assert bd.dark_prf_fwd_noalloc(_desc(d_h=48), FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 0, 0) == \
        bd.DARK_ERR_INVALID_ARG
    big = _desc(B=64, L=8192)
    assert bd.dark_prf_workspace_bytes(big) > bd.DARK_PRF_SCRATCH_BYTES
    assert bd.dark_prf_fwd_noalloc(big, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 0, 0) == bd.DARK_ERR_WORKSPACE
    # the two L=64K-sized and L=2048-sized workloads fit
    assert bd.dark_prf_workspace_bytes(_desc(B=2, L=2048)) <= bd.DARK_PRF_SCRATCH_BYTES


def test_state_export_rules():
    assert _fwd(_desc(causal=0), S=FAKE, z=FAKE) == bd.DARK_ERR_INVALID_ARG
    assert _fwd(_desc(causal=1), S=FAKE, z=0) == bd.DARK_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op():
    assert _fwd(_desc(B=0), ws=0, ws_bytes=0) == bd.DARK_OK


def _dec_desc(**kw):
    kw.setdefault("L", 1)
    return _desc(**kw)


def test_decode_rejects_stale_state():
    d = _dec_desc()
    d.proj_tag = bd.dark_prf_proj_tag(7, 256, 64, True)
    other = bd.dark_prf_proj_tag(8, 256, 64, True)
    st = bd.dark_prf_decode_step(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, other, FAKE, 0)
    assert st == bd.DARK_ERR_STALE_STATE


def test_decode_argument_checks():
    d = _dec_desc(L=2)
    assert bd.dark_prf_decode_step(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0) == bd.DARK_ERR_INVALID_ARG
    d = _dec_desc()
    d.causal = 0
    assert bd.dark_prf_decode_step(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0) == bd.DARK_ERR_INVALID_ARG
    d = _dec_desc()
    assert bd.dark_prf_decode_step(d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, FAKE, 0) == bd.DARK_ERR_INVALID_ARG


def _ctx(d, S=FAKE, z=FAKE, ws=FAKE, nb=None):
    nb = bd.dark_prf_workspace_bytes(d) if nb is None else nb
    return bd.dark_prf_context_state(d, FAKE, FAKE, FAKE, FAKE, 0, S, z, ws, nb, 0)


def _cross(d, tag=None, q=FAKE, S=FAKE, ws=FAKE, nb=None):
    nb = bd.dark_prf_workspace_bytes(d) if nb is None else nb
    tag = d.proj_tag if tag is None else tag
    return bd.dark_prf_cross_fwd(d, q, FAKE, FAKE, S, FAKE, tag, 0, FAKE, ws, nb, 0)


def test_context_state_argument_checks():
    assert _ctx(_desc(causal=1)) == bd.DARK_ERR_INVALID_ARG           # no causal cross-attention
    assert _ctx(_desc(causal=0), S=0) == bd.DARK_ERR_INVALID_ARG      # the summary is the output
    assert _ctx(_desc(causal=0), z=FAKE + 4) == bd.DARK_ERR_INVALID_ARG
    assert _ctx(_desc(causal=0), nb=0) == bd.DARK_ERR_WORKSPACE
    assert _ctx(_desc(causal=0, B=0), ws=0, nb=0) == bd.DARK_OK
    # the query and output strides are not used by this call
    assert _ctx(_desc(causal=0, q_str=[0, 0, 0], o_str=[0, 0, 0]), nb=0) == bd.DARK_ERR_WORKSPACE
    assert _ctx(_desc(causal=0, k_str=[0, 0, 0])) == bd.DARK_ERR_INVALID_ARG


def test_cross_fwd_argument_checks():
    d = _desc(causal=0, L=100)
    d.proj_tag = bd.dark_prf_proj_tag(7, 256, 64, True)
    other = bd.dark_prf_proj_tag(8, 256, 64, True)
    assert _cross(d, tag=other) == bd.DARK_ERR_STALE_STATE
    assert _cross(_desc(causal=1)) == bd.DARK_ERR_INVALID_ARG
    assert _cross(d, q=0) == bd.DARK_ERR_INVALID_ARG
    assert _cross(d, S=FAKE + 8) == bd.DARK_ERR_INVALID_ARG
    assert _cross(d, nb=0) == bd.DARK_ERR_WORKSPACE
    assert _cross(_desc(causal=0, L=0), ws=0, nb=0) == bd.DARK_OK
    # the key and value strides are not used by this call
    e = _desc(causal=0, L=100, k_str=[0, 0, 0], v_str=[0, 0, 0])
    assert _cross(e, nb=0) == bd.DARK_ERR_WORKSPACE


def test_exact_argument_checks():
    d = _desc(causal=1)
    nb = bd.dark_prf_exact_workspace_bytes(d)
    assert nb > 0
    call = lambda q=FAKE, ws=FAKE, n=nb, dd=d: bd.dark_prf_exact_fwd(dd, q, FAKE, FAKE, FAKE, 0, FAKE, ws, n, 0)
    assert call(q=0) == bd.DARK_ERR_INVALID_ARG
    assert call(q=FAKE + 2) == bd.DARK_ERR_INVALID_ARG
    assert call(n=nb - 1) == bd.DARK_ERR_WORKSPACE
    assert call(ws=0) == bd.DARK_ERR_WORKSPACE
    assert call(dd=_desc(B=0), ws=0, n=0) == bd.DARK_OK
    assert bd.dark_prf_exact_workspace_bytes(_desc(d_h=48)) == 0
    # more tokens never need less workspace
    assert bd.dark_prf_exact_workspace_bytes(_desc(L=4096)) >= nb


def test_omega_device_argument_checks():
    assert bd.dark_prf_omega_device_workspace_bytes(256, 64, False) == 0
    nb = bd.dark_prf_omega_device_workspace_bytes(100, 64, True)
    assert nb == 2 * 3 * 64 * 64 * 8                  # two blocks of G, V and Q in fp64
    assert bd.dark_prf_omega_device_workspace_bytes(16, 257, True) == 0
    call = lambda m=100, r=64, orth=True, om=FAKE, ws=FAKE, n=nb: bd.dark_prf_omega_device(1, m, r, orth, om, ws, n, 0)
    assert call(m=0) == bd.DARK_ERR_INVALID_ARG
    assert call(r=300) == bd.DARK_ERR_INVALID_ARG
    assert call(om=0) == bd.DARK_ERR_INVALID_ARG
    assert call(n=nb - 1) == bd.DARK_ERR_WORKSPACE
    assert call(ws=0) == bd.DARK_ERR_WORKSPACE
    assert call(ws=FAKE + 4) == bd.DARK_ERR_INVALID_ARG


def test_status_strings():
    assert bd.dark_prf_status_str(bd.DARK_OK) == "DARK_OK"
    assert bd.dark_prf_status_str(bd.DARK_ERR_STALE_STATE) == "DARK_ERR_STALE_STATE"
    assert bd.dark_prf_status_str(99) == "DARK_ERR_UNKNOWN"


def test_proj_tag():
    a = bd.dark_prf_proj_tag(5, 256, 64, True)
    assert a == bd.dark_prf_proj_tag(5, 256, 64, True)
    others = {bd.dark_prf_proj_tag(6, 256, 64, True), bd.dark_prf_proj_tag(5, 512, 64, True),
              bd.dark_prf_proj_tag(5, 256, 32, True), bd.dark_prf_proj_tag(5, 256, 64, False)}
    assert a not in others and len(others) == 4


@pytest.mark.parametrize("seed,H,m,r,orth", [(1002, 8, 256, 64, True), (9, 3, 48, 16, False)])
def test_library_per_head_omega_matches_oracle(seed, H, m, r, orth):
    lib_om = bd.dark_prf_omega_per_head(seed, H, m, r, orth)
    ref = oo.omega_per_head(seed, H, m, r, orth)
    assert lib_om.shape == ref.shape == (H, m, r)
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.mean(lib_om == ref) >= 0.999
    assert np.all(np.abs(lib_om - ref) <= ulp)
    for h in range(H):
        assert bd.dark_prf_head_seed(seed, h) == oo.head_seed(seed, h)


def test_per_head_tag_differs_from_shared_and_other_head_counts():
    shared = bd.dark_prf_proj_tag(5, 256, 64, True)
    t8 = bd.dark_prf_proj_tag_per_head(5, 8, 256, 64, True)
    assert t8 == bd.dark_prf_proj_tag_per_head(5, 8, 256, 64, True)
    assert len({shared, t8, bd.dark_prf_proj_tag_per_head(5, 4, 256, 64, True),
                bd.dark_prf_proj_tag_per_head(6, 8, 256, 64, True)}) == 4
    assert bd.lib().dark_prf_omega_per_head(1, 0, 16, 16, 1, None) == bd.DARK_ERR_INVALID_ARG


def test_per_head_omega_flag_is_validated_and_sizes_the_workspace():
    d = _desc(omega_per_head=2)
    assert bd.dark_prf_workspace_bytes(d) == 0
    shared = bd.dark_prf_workspace_bytes(_desc(m_per_head=0, r=16))          # unfolded: omega' once
    per_head = bd.dark_prf_workspace_bytes(_desc(m_per_head=0, r=16, omega_per_head=1))
    assert per_head > shared


def test_auto_mode_choice():
    # exact attention through the threshold (inclusive), linear beyond it
    for L, thr, want in ((256, 256, 1), (257, 256, 0), (1, 0, 0), (2048, 4096, 1), (2048, 1024, 0)):
        d = _desc(L=L)
        assert bd.dark_prf_auto_mode(d, thr) == want, (L, thr)
        ws = bd.dark_prf_exact_workspace_bytes(d) if want else bd.dark_prf_workspace_bytes(d)
        assert bd.dark_prf_auto_workspace_bytes(d, thr) == ws
    assert bd.dark_prf_auto_mode(_desc(), -1) == -1
    assert bd.dark_prf_auto_mode(_desc(d_h=48), 100) == -1
    assert bd.dark_prf_auto_workspace_bytes(_desc(), -1) == 0
    d = _desc(L=300)
    call = lambda thr, q=FAKE, ws=FAKE, n=None: bd.dark_prf_auto_fwd(  # noqa: E731
        d, thr, q, FAKE, FAKE, FAKE, FAKE, 0, FAKE, ws, bd.dark_prf_auto_workspace_bytes(d, thr) if n is None else n, 0)
    assert call(-5) == bd.DARK_ERR_INVALID_ARG
    # argument errors of either path come back before anything is queued
    assert call(1000, q=0) == bd.DARK_ERR_INVALID_ARG          # exact path
    assert call(10, q=0) == bd.DARK_ERR_INVALID_ARG            # linear path
    assert call(1000, n=bd.dark_prf_exact_workspace_bytes(d) - 1) == bd.DARK_ERR_WORKSPACE
    assert call(10, n=bd.dark_prf_workspace_bytes(d) - 1) == bd.DARK_ERR_WORKSPACE


def test_omega_argument_checks():
    buf = np.empty(4, np.float32)
    L = bd.lib()
    assert L.dark_prf_omega(1, 0, 2, 0, buf.ctypes.data_as(ctypes.c_void_p)) == bd.DARK_ERR_INVALID_ARG
    assert L.dark_prf_omega(1, 2, 2, 0, None) == bd.DARK_ERR_INVALID_ARG


@pytest.mark.parametrize("seed,m,r,orth", [
    (1001, 32, 16, False), (1002, 256, 64, True), (1003, 1024, 16, False), (1004, 512, 256, True),
    (1005, 256, 64, True), (42, 100, 16, True), (7, 48, 64, True)])
def test_library_omega_matches_oracle(seed, m, r, orth):
    """The C++ and the numpy generators implement the same published stream."""
    lib_om = bd.dark_prf_omega(seed, m, r, orth)
    ref = oo.omega(seed, m, r, orth)
    assert lib_om.shape == ref.shape and lib_om.dtype == np.float32
    same = np.mean(lib_om == ref)
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert same >= 0.999, same
    assert np.all(np.abs(lib_om - ref) <= ulp), np.max(np.abs(lib_om - ref) / ulp)


def test_timing_end_without_records():
    import ctypes as ct
    L = bd.lib()
    assert L.dark_prf_timing_end(None, None) == bd.DARK_ERR_INVALID_ARG
    bd.dark_prf_timing_begin()
    res = bd.dark_prf_timing_end()
    assert set(res) == set(bd.KERNEL_KINDS) and all(v == (0.0, 0) for v in res.values())


# ---- projection lifecycle (README section "Projection lifecycle") ----------------
def test_projection_initial_draw_is_reproducible():
    a = bd.dark_prf_projection_init(7, 256, 64, True)
    b = bd.dark_prf_projection_init(7, 256, 64, True)
    assert (a.seed, a.tag, a.draw) == (b.seed, b.tag, 0)
    assert a.seed == 7 and a.tag == bd.dark_prf_proj_tag(7, 256, 64, True)
    assert bd.dark_prf_projection_init(8, 256, 64, True).tag != a.tag


def test_projection_stays_unchanged_without_a_schedule():
    p = bd.dark_prf_projection_init(7, 256, 64, True, redraw_interval=0)
    tag = p.tag
    assert all(bd.dark_prf_projection_forward(p, True) == 0 for _ in range(50))
    assert p.tag == tag and p.draw == 0


def test_scheduled_redraw_after_interval_training_forwards():
    p = bd.dark_prf_projection_init(7, 256, 64, True, redraw_interval=3)
    tags, flags = [], []
    for _ in range(10):
        flags.append(bd.dark_prf_projection_forward(p, True))
        tags.append(p.tag)
    # three forwards per draw: the 4th, 7th and 10th forwards start with a redraw
    assert flags == [0, 0, 0, 1, 0, 0, 1, 0, 0, 1]
    assert len(set(tags)) == 4 and p.draw == 3
    assert p.tag == bd.dark_prf_proj_tag(p.seed, 256, 64, True)


def test_evaluation_forwards_do_not_advance_the_schedule():
    p = bd.dark_prf_projection_init(7, 256, 64, True, redraw_interval=2)
    assert bd.dark_prf_projection_forward(p, True) == 0
    for _ in range(20):
        assert bd.dark_prf_projection_forward(p, False) == 0
    assert p.forwards == 1 and p.draw == 0
    assert bd.dark_prf_projection_forward(p, True) == 0
    assert bd.dark_prf_projection_forward(p, True) == 1


def test_fixed_projection_ignores_ordinary_redraws_but_not_forced():
    p = bd.dark_prf_projection_init(7, 256, 64, True, redraw_interval=1)
    bd.dark_prf_projection_fix(p, True)
    tag = p.tag
    assert all(bd.dark_prf_projection_forward(p, True) == 0 for _ in range(5))
    assert bd.dark_prf_projection_redraw(p) == 0 and p.tag == tag
    assert bd.dark_prf_projection_redraw(p, force=True) == 1 and p.tag != tag and p.fixed == 1
    bd.dark_prf_projection_fix(p, False)
    assert bd.dark_prf_projection_redraw(p) == 1


def test_deterministic_fixes_at_construction():
    p = bd.dark_prf_projection_init(7, 256, 64, True, redraw_interval=1, deterministic=True)
    assert p.fixed == 1
    assert all(bd.dark_prf_projection_forward(p, True) == 0 for _ in range(5))


def test_redraw_seeds_are_reproducible_and_distinct():
    a = bd.dark_prf_projection_init(11, 64, 16, False)
    b = bd.dark_prf_projection_init(11, 64, 16, False)
    seeds = set()
    for _ in range(5):
        bd.dark_prf_projection_redraw(a)
        bd.dark_prf_projection_redraw(b)
        assert a.seed == b.seed
        seeds.add(a.seed)
    assert len(seeds) == 5 and 11 not in seeds


def test_projection_argument_checks():
    import ctypes
    L = bd.lib()
    assert L.dark_prf_projection_init(None, 1, 16, 16, 0, 0, 0) == bd.DARK_ERR_INVALID_ARG
    p = bd.DarkPrfProjection()
    assert L.dark_prf_projection_init(ctypes.byref(p), 1, 0, 16, 0, 0, 0) == bd.DARK_ERR_INVALID_ARG
    assert L.dark_prf_projection_forward(None, 1) == -1
    assert L.dark_prf_projection_redraw(None, 1) == -1
    assert L.dark_prf_projection_fix(None, 1) == bd.DARK_ERR_INVALID_ARG


def test_bwd_argument_checks():
    d = _desc(causal=1)
    nb = bd.dark_prf_bwd_workspace_bytes(d)
    # the size the header states for the causal call: per token and head
    # 4*(4m + 4r + 6 d_h + 135) bytes, plus two fp32 m x (d_h + 1) states per 64 tokens
    B, H, L, m, r, dh = 2, 8, 256, 256, 64, 64
    stated = 4 * B * H * L * (4 * m + 4 * r + 6 * dh + 135) + 8 * B * H * (L // 64) * m * (dh + 1)
    stated_max = stated + 4 * B * H * r * dh * (L // 64)
    assert stated <= nb <= 1.01 * stated_max + 64 * 1024, (nb, stated, stated_max)

    def call(q=FAKE, dout=FAKE, dM=FAKE, ws=FAKE, n=nb, dd=d):
        return bd.dark_prf_bwd(dd, q, FAKE, FAKE, FAKE, FAKE, 0, dout, FAKE, FAKE, FAKE, dM, ws, n, 0)
    assert call(q=0) == bd.DARK_ERR_INVALID_ARG
    assert call(q=FAKE + 2) == bd.DARK_ERR_INVALID_ARG
    assert call(dout=0) == bd.DARK_ERR_INVALID_ARG
    assert call(dM=0) == bd.DARK_ERR_INVALID_ARG
    assert call(n=nb - 1) == bd.DARK_ERR_WORKSPACE
    assert call(ws=0) == bd.DARK_ERR_WORKSPACE
    assert call(dd=_desc(o_str=[0, 0, 3])) == bd.DARK_ERR_INVALID_ARG
    assert bd.dark_prf_bwd_workspace_bytes(_desc(d_h=48)) == 0
    assert bd.dark_prf_bwd_workspace_bytes(_desc(L=4096)) >= nb


def test_bwd_workspace_for_empty_calls():
    # an empty batch is sized without dividing by its (zero) tile count: it
    # needs no workspace; neither call below may fault on the host
    for kw in (dict(B=0), dict(B=0, causal=0)):
        assert bd.dark_prf_bwd_workspace_bytes(_desc(**kw)) == 0, kw
    for kw in (dict(L=0), dict(L=0, causal=0)):
        assert bd.dark_prf_bwd_workspace_bytes(_desc(**kw)) > 0, kw
