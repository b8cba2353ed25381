"""Seeded synthetic inputs for the DARKFormer positive-random-feature attention path.

This module only draws numbers: it holds none of the method's arithmetic (no
feature map, no attention, no projection of Omega).  Both the HIP path and the
fp64 oracle consume exactly the arrays produced here, so the two sides see
bit-identical q, k, v, M and mask.  Omega is not drawn here: each side builds it
from the same seed with its own implementation of the published generator.

Values that the device receives in bfloat16 are rounded here, once, with
round-to-nearest-even, and returned as float32 arrays that hold bf16-exact
values; converting them to torch.bfloat16 is then exact.

The five workloads follow the shapes and value distributions of the package
README's examples (darkformer-pytorch 0.1.0, sections "Self-attention" and
"Encoder-decoder model and generation") and the synthetic stand-ins for the
Gemma-2B finetuning workload of the paper's Figures 2-5 (the weights and data
behind those figures are not available, so seeded Gaussian inputs of the same
head geometry stand in for them).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32).reshape(x32.shape)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(x32)
    if dtype == "f32":
        return x32
    raise ValueError(dtype)


@dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe for one attention call."""

    name: str
    B: int
    H: int
    L: int
    d_h: int
    m: int
    r: int
    dtype: str = "bf16"          # "bf16" or "f32" for q, k, v and the output
    causal: bool = False
    H_kv: Optional[int] = None   # defaults to H
    per_head_geometry: bool = True
    orthogonal: bool = True      # Omega construction (orthogonal blocks vs i.i.d.)
    seed: int = 0
    m_kind: str = "eye_noise"    # "eye_noise" | "gauss"
    m_noise: float = 0.1         # eye_noise: I + m_noise * N(0,1) * m_noise_scale
    m_noise_scale: Optional[float] = None  # default 1/sqrt(d_h)
    x_kind: str = "iid"          # "iid" | "aniso" | "spike" | "cov"
    mask_kind: str = "none"      # "none" | "ones" | "tail" | "random"
    max_pad: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def hkv(self) -> int:
        return self.H if self.H_kv is None else self.H_kv

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five headline workloads.  Seeds are 1000 + k for workload k (1-based).
CONFIGS = {
    "c1_tiny_f32": Workload(
        name="c1_tiny_f32", B=1, H=1, L=128, d_h=16, m=32, r=16, dtype="f32",
        causal=False, orthogonal=False, seed=1001, m_kind="eye_noise", m_noise=0.1,
        x_kind="iid", mask_kind="none"),
    "c2_causal_L2048": Workload(
        name="c2_causal_L2048", B=2, H=8, L=2048, d_h=64, m=256, r=64, dtype="bf16",
        causal=True, orthogonal=True, seed=1002, m_kind="eye_noise", m_noise=0.1,
        x_kind="aniso", mask_kind="tail", max_pad=256),
    "c3_long_L64K": Workload(
        name="c3_long_L64K", B=1, H=8, L=65536, d_h=64, m=1024, r=16, dtype="bf16",
        causal=False, per_head_geometry=False, orthogonal=False, seed=1003,
        m_kind="gauss", m_noise=0.125, x_kind="spike", mask_kind="ones"),
    "c4_gqa_L8192": Workload(
        name="c4_gqa_L8192", B=4, H=8, H_kv=1, L=8192, d_h=256, m=512, r=256,
        dtype="bf16", causal=True, orthogonal=True, seed=1004, m_kind="eye_noise",
        m_noise=0.05, m_noise_scale=1.0, x_kind="cov", mask_kind="none"),
    "c5_decode": Workload(
        name="c5_decode", B=256, H=8, L=4096, d_h=64, m=256, r=64, dtype="bf16",
        causal=True, orthogonal=True, seed=1005, m_kind="eye_noise", m_noise=0.1,
        x_kind="iid", mask_kind="none", extra={"decode_steps": 512}),
}


def _geometry(w: Workload, rng: np.random.Generator) -> np.ndarray:
    """M: [H][r][d_h] (per-head) or [r][d_h] (shared), float32."""
    shape = (w.H, w.r, w.d_h) if w.per_head_geometry else (w.r, w.d_h)
    noise = rng.standard_normal(shape)
    if w.m_kind == "eye_noise":
        scale = (1.0 / np.sqrt(w.d_h)) if w.m_noise_scale is None else w.m_noise_scale
        eye = np.eye(w.r, w.d_h)
        M = eye + w.m_noise * scale * noise
    elif w.m_kind == "gauss":
        M = w.m_noise * noise
    else:
        raise ValueError(w.m_kind)
    return np.asarray(M, dtype=np.float32)


def _haar(rng: np.random.Generator, n: int) -> np.ndarray:
    """A Haar-random n x n rotation (used only to rotate an input covariance)."""
    g = rng.standard_normal((n, n))
    q, rr = np.linalg.qr(g)
    return q * np.sign(np.diag(rr))[None, :]


def _tokens(w: Workload, rng: np.random.Generator, heads: int, L: int, kind: str,
            ctx: dict) -> np.ndarray:
    """One batch row of a q/k/v tensor: [heads][L][d_h] in float64 before rounding."""
    shape = (heads, L, w.d_h)
    if kind == "iid":
        return rng.standard_normal(shape)
    if kind == "aniso":
        # independent coordinates with variance 4 * 0.9**i
        std = 2.0 * 0.9 ** (0.5 * np.arange(w.d_h))
        return rng.standard_normal(shape) * std
    if kind == "spike":
        # N(0, I) plus U c with U an orthonormal d_h x 8 basis shared by q, k and all
        # heads, and c ~ N(0, 3^2 I_8) drawn per token, head and tensor
        base = rng.standard_normal(shape)
        c = 3.0 * rng.standard_normal((heads, L, 8))
        return base + c @ ctx["spike_basis"].T
    if kind == "cov":
        # N(0, C) with C = R diag(lam) R^T, lam_i = (1+i)^-1.5
        g = rng.standard_normal(shape)
        return (g * ctx["cov_sqrt_lam"]) @ ctx["cov_rot"].T
    raise ValueError(kind)


def _shared(w: Workload):
    """Draws shared by every batch row: extras, then M (stream PCG64(seed))."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    ctx: dict = {}
    if w.x_kind == "spike":
        ctx["spike_basis"], _ = np.linalg.qr(rng.standard_normal((w.d_h, 8)))
    if w.x_kind == "cov":
        ctx["cov_rot"] = _haar(rng, w.d_h)
        ctx["cov_sqrt_lam"] = (1.0 + np.arange(w.d_h)) ** -0.75
    return ctx, _geometry(w, rng)


def _row(w: Workload, ctx: dict, b: int, L: int):
    """q, k, v and mask of batch row b (stream PCG64([seed, b + 1]))."""
    rng = np.random.Generator(np.random.PCG64([w.seed, b + 1]))
    qk_kind = w.x_kind
    v_kind = "iid" if w.x_kind in ("spike", "cov") else w.x_kind
    q = round_to(_tokens(w, rng, w.H, L, qk_kind, ctx), w.dtype)
    k = round_to(_tokens(w, rng, w.hkv, L, qk_kind, ctx), w.dtype)
    v = round_to(_tokens(w, rng, w.hkv, L, v_kind, ctx), w.dtype)
    mask = None
    if w.mask_kind == "ones":
        mask = np.ones(L, dtype=np.uint8)
    elif w.mask_kind == "tail":
        pad = int(rng.integers(0, w.max_pad + 1))
        mask = np.ones(L, dtype=np.uint8)
        if pad > 0:
            mask[L - min(pad, L):] = 0
    elif w.mask_kind == "random":
        mask = (rng.random(L) < 0.7).astype(np.uint8)
    elif w.mask_kind != "none":
        raise ValueError(w.mask_kind)
    return q, k, v, mask


def make_inputs(w: Workload, L: Optional[int] = None, rows: Optional[list] = None) -> dict:
    """Draw M, q, k, v and the key mask for one workload.

    M (and any shared basis) comes from the stream PCG64(seed); batch row b draws
    q, k, v and its mask padding, in that order, from PCG64([seed, b + 1]), so any
    subset of rows can be regenerated alone (`rows`).  Returns float32 arrays
    (bf16-exact when w.dtype == "bf16"): q [B][H][L][d_h], k and v
    [B][H_kv][L][d_h], mask uint8 [B][L] (1 = valid key) or None, and M.
    """
    L = w.L if L is None else L
    rows = list(range(w.B)) if rows is None else list(rows)
    ctx, M = _shared(w)
    qs, ks, vs, ms = [], [], [], []
    for b in rows:
        q, k, v, mk = _row(w, ctx, b, L)
        qs.append(q)
        ks.append(k)
        vs.append(v)
        ms.append(mk)
    mask = None if ms[0] is None else np.stack(ms)
    return {"q": np.stack(qs), "k": np.stack(ks), "v": np.stack(vs), "M": M, "mask": mask}


def make_decode_tokens(w: Workload, steps: int, rows: Optional[list] = None) -> dict:
    """q, k, v for `steps` one-token decode steps: [steps][len(rows)][heads][d_h], N(0,1).

    Batch row b draws from PCG64([seed, 100000 + b]) (q, then k, then v).
    """
    rows = list(range(w.B)) if rows is None else list(rows)
    out = {"q": [], "k": [], "v": []}
    for b in rows:
        rng = np.random.Generator(np.random.PCG64([w.seed, 100000 + b]))
        for name, heads in (("q", w.H), ("k", w.hkv), ("v", w.hkv)):
            out[name].append(round_to(rng.standard_normal((steps, heads, w.d_h)), w.dtype))
    return {k2: np.stack(v2, axis=1) for k2, v2 in out.items()}
