"""Plant plausible mistakes in the oracle (on the CPU) and show that a pin catches each.

Every mutation below is a mistake a reader of the README's section "Kernel"
could plausibly make; the pins in oracle_pins must reject all of them.
"""
import numpy as np
import pytest

from oracle import prf_oracle as po
from tests import oracle_pins as pins


def _feat(scale=lambda d: d ** -0.25, sign=1.0, half=0.5, sqrt_m=True, transpose_m=False):
    def prf_features(X, M_h, omega):
        omega = np.asarray(omega, np.float64)
        M_h = np.asarray(M_h, np.float64)
        Mx = M_h if transpose_m else M_h.T
        U = scale(X.shape[-1]) * (np.asarray(X, np.float64) @ Mx)
        E = sign * (U @ omega.T)
        out = np.exp(E - half * np.sum(U * U, axis=1, keepdims=True))
        return out / np.sqrt(omega.shape[0]) if sqrt_m else out
    return prf_features


def _causal(strict=False, update_first=False):
    def attend_causal_blockwise(PQ, PK, V, block=256):
        L, m = PQ.shape
        S = np.zeros((m, V.shape[1]))
        z = np.zeros(m)
        O = np.zeros((L, V.shape[1]))
        for s in range(0, L, block):
            e = min(L, s + block)
            if update_first:
                S = S + PK[s:e].T @ V[s:e]
                z = z + PK[s:e].sum(0)
            A = np.tril(PQ[s:e] @ PK[s:e].T, -1 if strict else 0)
            if update_first:
                A = 0 * A
            N = PQ[s:e] @ S + A @ V[s:e]
            D = PQ[s:e] @ z + A.sum(1)
            ok = D > 0
            O[s:e][ok] = N[ok] / D[ok, None]
            if not update_first:
                S = S + PK[s:e].T @ V[s:e]
                z = z + PK[s:e].sum(0)
        return O, S, z
    return attend_causal_blockwise


def _ignore_mask(orig):
    def attention(q, k, v, M, omega, mask=None, **kw):
        return orig(q, k, v, M, omega, mask=None, **kw)
    return attention


def _decode_before_update(S, z, q, k, v, M, omega):
    S = np.asarray(S, np.float64).copy()
    z = np.asarray(z, np.float64).copy()
    N, H, d = q.shape
    H_kv = k.shape[1]
    o = np.zeros((N, H, d))
    for h in range(H):
        g = (h * H_kv) // H
        M_h = M[h] if np.asarray(M).ndim == 3 else M
        pq = po.prf_features(np.asarray(q[:, h], np.float64), M_h, omega)
        pk = po.prf_features(np.asarray(k[:, g], np.float64), M_h, omega)
        num = np.einsum("nm,nmd->nd", pq, S[:, h])
        den = np.einsum("nm,nm->n", pq, z[:, h])
        o[:, h] = num / np.where(den > 0, den, 1.0)[:, None]
        S[:, h] += pk[:, :, None] * np.asarray(v[:, g], np.float64)[:, None, :]
        z[:, h] += pk
    return o, S, z


def _context_mask_ignored(orig):
    def context_state(k, v, M, omega, H, context_mask=None):
        return orig(k, v, M, omega, H, context_mask=None)
    return context_state


def _query_mask_ignored(orig):
    def cross_attention(q, S, z, M, omega, query_mask=None):
        return orig(q, S, z, M, omega, query_mask=None)
    return cross_attention


def _bwd(drop_norm=False, dD_sign=-1.0, dpk_untransposed=False, dM_scale=True, gqa_overwrite=False):
    """A copy of the oracle's backward with one planted mistake."""
    def attention_backward(q, k, v, M, omega, dout, mask=None, causal=False):
        q, k, v, dout, omega = (np.asarray(a, np.float64) for a in (q, k, v, dout, omega))
        B, H, L, d = q.shape
        H_kv = k.shape[1]
        s = d ** -0.25
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        dM = np.zeros_like(np.asarray(M, np.float64))
        vis = np.tril(np.ones((L, L))) if causal else np.ones((L, L))
        for b in range(B):
            visb = vis if mask is None else vis * (np.asarray(mask[b]) != 0)[None, :]
            for h in range(H):
                g = (h * H_kv) // H
                M_h = np.asarray(M[h] if np.asarray(M).ndim == 3 else M, np.float64)
                UQ, UK = s * q[b, h] @ M_h.T, s * k[b, g] @ M_h.T
                PQ, PK = po.prf_features(q[b, h], M_h, omega), po.prf_features(k[b, g], M_h, omega)
                W = (PQ @ PK.T) * visb
                D = W.sum(1)
                ok = D > 0
                O = np.zeros((L, d))
                O[ok] = (W @ v[b, g])[ok] / D[ok, None]
                dN, dD = np.zeros((L, d)), np.zeros(L)
                dN[ok] = dout[b, h][ok] / D[ok, None]
                dD[ok] = dD_sign * np.sum(dout[b, h][ok] * O[ok], 1) / D[ok]
                dW = visb * (dN @ v[b, g].T + dD[:, None])
                dv[b, g] += W.T @ dN
                dPK = (dW if dpk_untransposed else dW.T) @ PQ
                out = []
                for P, U, dP in ((PQ, UQ, dW @ PK), (PK, UK, dPK)):
                    dE = dP * P
                    out.append(dE @ omega - (0 if drop_norm else U * dE.sum(1, keepdims=True)))
                dq[b, h] += s * out[0] @ M_h
                if gqa_overwrite:
                    dk[b, g] = s * out[1] @ M_h
                else:
                    dk[b, g] += s * out[1] @ M_h
                dM_h = (s if dM_scale else 1.0) * (out[0].T @ q[b, h] + out[1].T @ k[b, g])
                if dM.ndim == 3:
                    dM[h] += dM_h
                else:
                    dM += dM_h
        return dq, dk, dv, dM
    return attention_backward


MUTATIONS = {
    "scale_d^-1/2": ("prf_features", _feat(scale=lambda d: d ** -0.5)),
    "no_scale": ("prf_features", _feat(scale=lambda d: 1.0)),
    "exponent_sign": ("prf_features", _feat(sign=-1.0)),
    "no_half_norm": ("prf_features", _feat(half=0.0)),
    "full_norm": ("prf_features", _feat(half=1.0)),
    "no_1/sqrt_m": ("prf_features", _feat(sqrt_m=False)),
    "M_transposed": ("prf_features", _feat(transpose_m=True)),
    "causal_strict": ("attend_causal_blockwise", _causal(strict=True)),
    "causal_update_first": ("attend_causal_blockwise", _causal(update_first=True)),
    "mask_ignored": ("attention", None),
    "gqa_modulo": ("kv_head", lambda h, H, H_kv: h % H_kv),
    "decode_pre_update": ("decode_step", _decode_before_update),
    "eps_denominator": ("_ratio", lambda N, D: N / (D + 1e-8)[:, None]),
    "context_mask_ignored": ("context_state", None),
    "query_mask_ignored": ("cross_attention", None),
    "bwd_no_norm_term": ("attention_backward", _bwd(drop_norm=True)),
    "bwd_dD_sign": ("attention_backward", _bwd(dD_sign=1.0)),
    "bwd_dPK_untransposed": ("attention_backward", _bwd(dpk_untransposed=True)),
    "bwd_dM_unscaled": ("attention_backward", _bwd(dM_scale=False)),
    "bwd_gqa_overwrite": ("attention_backward", _bwd(gqa_overwrite=True)),
    "per_head_omega_ignored": ("head_omega", lambda omega, h: np.asarray(omega)[0] if np.ndim(omega) == 3
                               else np.asarray(omega)),
}

QUICK = pins.ALL_CHECKS + [pins.check_mc_kernel]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    attr, repl = MUTATIONS[name]
    if name == "mask_ignored":
        repl = _ignore_mask(po.attention)
    elif name == "context_mask_ignored":
        repl = _context_mask_ignored(po.context_state)
    elif name == "query_mask_ignored":
        repl = _query_mask_ignored(po.cross_attention)
    monkeypatch.setattr(po, attr, repl)
    caught = []
    for check in QUICK:
        try:
            kw = {"ms": (2 ** 8, 2 ** 12)} if check is pins.check_mc_kernel else {}
            check(**kw)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"no pin caught mutation {name}"
