"""Property-based fuzzing of the C ABI's host-side validation and planning.

Random descriptors (valid and invalid, including extreme sizes and strides)
go through every workspace-sizing call and through the compute entry points in
ways that must return before anything is queued (a missing pointer, a short
workspace).  Properties: a descriptor the library rejects gets a zero
workspace from every sizing call and DARK_ERR_INVALID_ARG (or
DARK_ERR_UNSUPPORTED) from every call; an accepted one gets a positive,
16-byte-multiple workspace that never shrinks as L grows; the auto mode picks
the exact path exactly when L <= threshold.  CPU only: nothing reaches a GPU.
"""
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from random_feature_linear_amd import binding as bd

FAKE = 1 << 20
I32 = st.integers(min_value=-(1 << 31), max_value=(1 << 31) - 1)


def _valid_fields():
    return st.fixed_dictionaries({
        "B": st.integers(0, 64), "H": st.sampled_from([1, 2, 4, 8, 16]),
        "g": st.sampled_from([1, 2, 4, 8]), "L": st.integers(0, 70000),
        "d_h": st.sampled_from([16, 32, 64, 128, 256]), "m": st.integers(1, 80).map(lambda x: 16 * x),
        "r": st.integers(1, 256), "dtype": st.sampled_from([0, 1]), "causal": st.sampled_from([0, 1]),
        "m_per_head": st.sampled_from([0, 1]), "omega_per_head": st.sampled_from([0, 1]),
    })


def _desc(f, pad=0):
    d = bd.DarkPrfDesc()
    H = f["H"]
    Hkv = max(1, H // f["g"]) if H % max(1, H // f["g"]) == 0 else H
    d.B, d.H, d.H_kv, d.L, d.d_h, d.m, d.r = f["B"], H, Hkv, f["L"], f["d_h"], f["m"], f["r"]
    d.dtype, d.causal, d.m_per_head, d.omega_per_head = f["dtype"], f["causal"], f["m_per_head"], f["omega_per_head"]
    row = f["d_h"] + pad
    for name, heads in (("q_str", H), ("k_str", Hkv), ("v_str", Hkv), ("o_str", H)):
        getattr(d, name)[:] = [heads * max(f["L"], 1) * row, max(f["L"], 1) * row, row]
    return d


def _sizes(d):
    return (bd.dark_prf_workspace_bytes(d), bd.dark_prf_exact_workspace_bytes(d), bd.dark_prf_bwd_workspace_bytes(d))


def _reject_all(d):
    """Every entry point must refuse d before queueing anything."""
    ok = (bd.DARK_ERR_INVALID_ARG, bd.DARK_ERR_UNSUPPORTED)
    assert _sizes(d) == (0, 0, 0)
    assert bd.dark_prf_auto_mode(d, 100) == -1 and bd.dark_prf_auto_workspace_bytes(d, 100) == 0
    assert bd.dark_prf_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 0, FAKE, 1 << 40, 0) in ok
    assert bd.dark_prf_fwd_noalloc(d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 0, 0) in ok
    assert bd.dark_prf_exact_fwd(d, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 1 << 40, 0) in ok
    assert bd.dark_prf_auto_fwd(d, 100, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 1 << 40, 0) in ok
    assert bd.dark_prf_bwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, 0) in ok


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(_valid_fields())
def test_valid_descriptors_plan_consistently(f):
    d = _desc(f)
    if (f["B"] * f["H"] * (f["L"] + 255)) > (1 << 31):
        assert bd.dark_prf_workspace_bytes(d) == 0
        return
    ws, ex, bw = _sizes(d)
    if f["B"] == 0:
        assert bw == 0
    for n in (ws, ex):
        assert n > 0 and n % 16 == 0
    # more tokens never need less workspace
    if f["L"] < 60000:
        d2 = _desc(dict(f, L=f["L"] + 257))
        ws2, ex2, _ = _sizes(d2)
        assert ws2 >= ws and ex2 >= ex
    # auto: exact through the threshold, linear beyond
    for thr in (0, f["L"], f["L"] + 1, max(0, f["L"] - 1)):
        mode = bd.dark_prf_auto_mode(d, thr)
        assert mode == (1 if f["L"] <= thr else 0)
        assert bd.dark_prf_auto_workspace_bytes(d, thr) == (ex if mode else ws)
    if f["B"] > 0 and f["L"] > 0:
        # a short workspace, or a missing pointer, is refused before any launch
        assert bd.dark_prf_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 0, FAKE, ws - 1, 0) == \
            bd.DARK_ERR_WORKSPACE
        assert bd.dark_prf_fwd(d, 0, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 0, FAKE, ws, 0) == bd.DARK_ERR_INVALID_ARG
        assert bd.dark_prf_exact_fwd(d, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, ex - 1, 0) == bd.DARK_ERR_WORKSPACE
        assert bd.dark_prf_bwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, bw - 1, 0) == \
            bd.DARK_ERR_WORKSPACE
        if ws > bd.DARK_PRF_SCRATCH_BYTES:
            assert bd.dark_prf_fwd_noalloc(d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 0, 0) == bd.DARK_ERR_WORKSPACE


@settings(max_examples=600, deadline=None)
@given(st.fixed_dictionaries({"B": I32, "H": I32, "H_kv": I32, "L": I32, "d_h": I32, "m": I32, "r": I32,
                              "dtype": I32, "causal": I32, "m_per_head": I32, "omega_per_head": I32,
                              "s": st.lists(st.integers(-(1 << 62), 1 << 62), min_size=12, max_size=12)}))
def test_arbitrary_descriptors_never_crash(f):
    d = bd.DarkPrfDesc()
    for k in ("B", "H", "H_kv", "L", "d_h", "m", "r", "dtype", "causal", "m_per_head", "omega_per_head"):
        setattr(d, k, f[k])
    for i, name in enumerate(("q_str", "k_str", "v_str", "o_str")):
        getattr(d, name)[:] = f["s"][3 * i:3 * i + 3]
    ws, ex, bw = _sizes(d)
    valid = (f["B"] >= 0 and f["L"] >= 0 and f["H"] >= 1 and f["H_kv"] >= 1 and f["H"] % f["H_kv"] == 0
             and f["d_h"] in (16, 32, 64, 128, 256) and f["m"] >= 16 and f["m"] % 16 == 0 and 1 <= f["r"] <= 256
             and f["dtype"] in (0, 1) and f["causal"] in (0, 1) and f["m_per_head"] in (0, 1)
             and f["omega_per_head"] in (0, 1))
    if not valid:
        _reject_all(d)
    else:
        # strides decide the rest; whatever the verdict, the calls return a status
        assert (ws == 0) == (ex == 0)


@pytest.mark.parametrize("extreme", [(1, 2, 1 << 30), (1 << 20, 1, 3000), (1, 1 << 12, 1 << 19)])
def test_size_guard_on_huge_grids(extreme):
    B, H, L = extreme
    d = _desc(dict(B=B, H=H, g=1, L=L, d_h=64, m=256, r=64, dtype=1, causal=1, m_per_head=1, omega_per_head=0))
    assert bd.dark_prf_workspace_bytes(d) == 0
    assert bd.dark_prf_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 0, FAKE, 1 << 50, 0) == \
        bd.DARK_ERR_UNSUPPORTED
