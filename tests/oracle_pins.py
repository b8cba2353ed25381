"""Checks that pin the fp64 oracle to facts other than itself.

Each check raises AssertionError when the oracle disagrees with a closed form,
an algebraic identity of a different evaluation order, a textbook or library
routine, or a statistical law that the package README's section "Kernel"
fixes.  They run against `oracle.prf_oracle` through its module attributes, so
test_oracle_mutations.py can plant a plausible mistake in the oracle and show
that some check here catches it.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import omega_gen as oo
from oracle import prf_oracle as po


def _u(X, M, d_h):
    """u = d_h^(-1/4) M x, written out here (not the oracle's helper)."""
    return (float(d_h) ** -0.25) * (np.asarray(X, np.float64) @ np.asarray(M, np.float64).T)


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(1e-300, float(np.max(np.abs(b))))
    err = float(np.max(np.abs(a - b))) / scale if a.size else 0.0
    assert err <= tol, f"{what}: relative error {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------
# closed forms derived by hand from the section "Kernel" equations
# ----------------------------------------------------------------------------
def check_closed_form_features():
    # Case A: d_h = 4, so the scale is 4^(-1/4) = 2^(-1/2).  r = 1, M = [1 0 0 0],
    # x = [sqrt2 0 0 0]: u = 2^(-1/2) * sqrt2 = 1, |u|^2 / 2 = 1/2.
    # Omega rows 3, -1, 0, 2 (m = 4): phi = exp([3, -1, 0, 2] - 1/2) / sqrt(4).
    M = np.array([[1.0, 0, 0, 0]])
    x = np.array([[math.sqrt(2.0), 0, 0, 0]])
    om = np.array([[3.0], [-1.0], [0.0], [2.0]])
    want = np.array([[math.exp(2.5), math.exp(-1.5), math.exp(-0.5), math.exp(1.5)]]) / 2.0
    _close(po.prf_features(x, M, om), want, 1e-14, "closed form A")

    # Case B: d_h = 16, scale 1/2.  r = 2, M = [e0; 2 e1], x = [2, 1, 0...]:
    # M x = [2, 2], u = [1, 1], |u|^2 / 2 = 1.  Omega = [[1,0],[0,-1],[1,1]] (m = 3):
    # omega.u = [1, -1, 2], phi = exp([0, -2, 1]) / sqrt(3).
    M = np.zeros((2, 16))
    M[0, 0], M[1, 1] = 1.0, 2.0
    x = np.zeros((1, 16))
    x[0, 0], x[0, 1] = 2.0, 1.0
    om = np.array([[1.0, 0.0], [0.0, -1.0], [1.0, 1.0]])
    want = np.exp(np.array([[0.0, -2.0, 1.0]])) / math.sqrt(3.0)
    _close(po.prf_features(x, M, om), want, 1e-14, "closed form B")

    # Case C (orientation of M): d_h = r = 4, M has a single 1 at row 0, column 1,
    # x = [0, sqrt2, 0, 0]: M x = [sqrt2, 0, 0, 0], u = [1, 0, 0, 0] (M^T x would be 0).
    # Omega = [[1, 0, 0, 0]] (m = 1): phi = exp(1 - 1/2) = e^(1/2).
    M = np.zeros((4, 4))
    M[0, 1] = 1.0
    x = np.array([[0.0, math.sqrt(2.0), 0.0, 0.0]])
    om = np.array([[1.0, 0.0, 0.0, 0.0]])
    _close(po.prf_features(x, M, om), np.array([[math.exp(0.5)]]), 1e-14, "closed form C")


def check_closed_form_attention():
    # d_h = 4, r = 1, M = [1 0 0 0], m = 1, Omega = [[1]].  Keys with first
    # coordinates sqrt2, 0, -sqrt2 give u = 1, 0, -1 and phi = e^(1/2), 1, e^(-3/2).
    # Values are the unit vectors e0, e1, e2.  phi(q) cancels in the ratio.
    s2 = math.sqrt(2.0)
    M = np.array([[1.0, 0, 0, 0]])[None]                   # [H=1][r=1][d=4]
    om = np.array([[1.0]])
    k = np.zeros((1, 1, 3, 4))
    k[0, 0, :, 0] = [s2, 0.0, -s2]
    v = np.zeros((1, 1, 3, 4))
    v[0, 0, 0, 0] = v[0, 0, 1, 1] = v[0, 0, 2, 2] = 1.0
    q = np.zeros((1, 1, 3, 4))
    q[0, 0, :, 0] = [0.3, -1.1, 2.0]
    a, b, c = math.exp(0.5), 1.0, math.exp(-1.5)
    # non-causal: every query gets [a, b, c, 0] / (a + b + c)
    want = np.tile(np.array([a, b, c, 0.0]) / (a + b + c), (3, 1))
    _close(po.attention(q, k, v, M, om)[0, 0], want, 1e-14, "closed form non-causal")
    # causal: row 0 = e0, row 1 = [a, b, 0, 0] / (a + b), row 2 as above
    want_c = np.array([[1.0, 0, 0, 0], [a / (a + b), b / (a + b), 0, 0],
                       [a / (a + b + c), b / (a + b + c), c / (a + b + c), 0]])
    _close(po.attention(q, k, v, M, om, causal=True)[0, 0], want_c, 1e-14, "closed form causal")
    # key 1 masked out: rows see {0, 2} (non-causal) or the causal subsets
    mask = np.array([[1, 0, 1]], dtype=np.uint8)
    want_m = np.tile(np.array([a, 0, c, 0.0]) / (a + c), (3, 1))
    _close(po.attention(q, k, v, M, om, mask=mask)[0, 0], want_m, 1e-14, "closed form masked")
    want_mc = np.array([[1.0, 0, 0, 0], [1.0, 0, 0, 0], [a / (a + c), 0, c / (a + c), 0]])
    _close(po.attention(q, k, v, M, om, mask=mask, causal=True)[0, 0], want_mc, 1e-14,
           "closed form masked causal")
    # every key masked: no visible key, output 0
    none = np.zeros((1, 3), dtype=np.uint8)
    _close(po.attention(q, k, v, M, om, mask=none)[0, 0], np.zeros((3, 4)), 0.0, "empty mask")


# ----------------------------------------------------------------------------
# (a) associative evaluation vs the explicit quadratic form
# ----------------------------------------------------------------------------
def _random_case(rng, B=2, H=2, H_kv=2, Lq=17, Lk=None, d=8, m=16, r=8, per_head=True):
    Lk = Lq if Lk is None else Lk
    q = rng.standard_normal((B, H, Lq, d))
    k = rng.standard_normal((B, H_kv, Lk, d))
    v = rng.standard_normal((B, H_kv, Lk, d))
    shape = (H, r, d) if per_head else (r, d)
    M = np.eye(r, d) + 0.3 * rng.standard_normal(shape)
    om = rng.standard_normal((m, r))
    return q, k, v, M, om


def explicit_kernel_matrix(q_bh, k_bg, M_h, om):
    """K[t, j] = (1/m) sum_i exp(omega_i.(u_t + w_j) - |u_t|^2/2 - |w_j|^2/2).

    The product phi(q_t) . phi(k_j) written as one exponent per feature: a
    different evaluation of the same kernel estimate.
    """
    d = q_bh.shape[-1]
    U = _u(q_bh, M_h, d)
    W = _u(k_bg, M_h, d)
    m = om.shape[0]
    K = np.zeros((U.shape[0], W.shape[0]))
    for i in range(m):
        K += np.exp((U @ om[i])[:, None] + (W @ om[i])[None, :]
                    - 0.5 * np.sum(U * U, 1)[:, None] - 0.5 * np.sum(W * W, 1)[None, :])
    return K / m


def explicit_attention(q, k, v, M, om, mask=None, causal=False):
    B, H, L, d = q.shape
    H_kv = k.shape[1]
    O = np.zeros((B, H, L, d))
    for b in range(B):
        for h in range(H):
            g = (h * H_kv) // H
            M_h = M[h] if M.ndim == 3 else M
            om_h = om[h] if np.ndim(om) == 3 else om
            K = explicit_kernel_matrix(q[b, h], k[b, g], M_h, om_h)
            if mask is not None:
                K = K * (np.asarray(mask[b]) != 0)[None, :]
            if causal:
                K = np.tril(K)
            den = K.sum(1)
            num = K @ v[b, g]
            ok = den > 0
            O[b, h][ok] = num[ok] / den[ok, None]
    return O


def check_associative_vs_explicit(seed=0):
    rng = np.random.default_rng(seed)
    for Lq, Lk in ((1, 1), (5, 64), (33, 17)):
        q, k, v, M, om = _random_case(rng, Lq=Lq, Lk=Lk)
        mask = (rng.random((2, Lk)) < 0.6).astype(np.uint8)
        mask[0, 0] = 1
        for mk in (None, mask):
            O = po.attention(q, k, v, M, om, mask=mk)
            _close(O, explicit_attention(q, k, v, M, om, mask=mk), 1e-12,
                   f"associative vs explicit Lq={Lq} Lk={Lk}")


# ----------------------------------------------------------------------------
# (b) causal prefix scan vs the masked quadratic form
# ----------------------------------------------------------------------------
def check_causal_vs_quadratic(seed=1, lengths=(1, 7, 64, 300, 513), blocks=(1, 7, 256)):
    rng = np.random.default_rng(seed)
    for L in lengths:
        q, k, v, M, om = _random_case(rng, B=4, H=1, H_kv=1, Lq=L)
        mask = np.ones((4, L), dtype=np.uint8)
        mask[1, : max(1, L // 3)] = 0                 # leading padding
        mask[2, L - max(1, L // 4):] = 0              # trailing padding
        mask[3, :] = 0                                # fully padded sequence
        if L > 4:
            mask[0, L // 2: L // 2 + 3] = 0           # interior gap
        ref = explicit_attention(q, k, v, M, om, mask=mask, causal=True)
        for blk in blocks:
            O = po.attention(q, k, v, M, om, mask=mask, causal=True, block=blk)
            _close(O, ref, 1e-12, f"causal scan L={L} block={blk}")
        assert np.all(ref[3] == 0.0)


# ----------------------------------------------------------------------------
# (c) Performer special case: M = I, r = d_h
# ----------------------------------------------------------------------------
def performer_positive_features(X, om):
    """Performer's positive softmax-kernel features (Choromanski et al. 2020, FAVOR+):
    phi(x) = exp(w^T x' - |x'|^2 / 2) / sqrt(m) on x' = x / d^(1/4)."""
    d = X.shape[-1]
    Xs = np.asarray(X, np.float64) / d ** 0.25
    return np.exp(Xs @ om.T - 0.5 * np.sum(Xs * Xs, 1, keepdims=True)) / math.sqrt(om.shape[0])


def check_performer_special_case(seed=2):
    rng = np.random.default_rng(seed)
    for d in (4, 16, 64):
        X = rng.standard_normal((23, d))
        om = rng.standard_normal((32, d))
        _close(po.prf_features(X, np.eye(d), om), performer_positive_features(X, om), 1e-13,
               f"Performer special case d={d}")


# ----------------------------------------------------------------------------
# (d) Monte-Carlo law of the estimator
# ----------------------------------------------------------------------------
def check_mc_kernel(seeds=(11, 12, 13), ms=(2 ** 8, 2 ** 12, 2 ** 16, 2 ** 20)):
    """mean_j phi(q)_j phi(k)_j -> exp(q^T Sigma k / sqrt(d_h)) with the stated variance."""
    rng = np.random.default_rng(5)
    d, r = 4, 4
    M = np.eye(r, d) + 0.4 * rng.standard_normal((r, d))
    for pair in range(3):
        qv = 0.5 * rng.standard_normal(d)
        kv = 0.5 * rng.standard_normal(d)
        u = _u(qv[None], M, d)[0]
        w = _u(kv[None], M, d)[0]
        kappa = math.exp(float(qv @ (M.T @ M) @ kv) / math.sqrt(d))
        var = math.exp(2 * float(u @ w)) * (math.exp(float((u + w) @ (u + w))) - 1.0)
        for seed in seeds:
            for m in ms:
                om = oo.omega_iid(seed * 1000 + pair, m, r)
                est = float(po.prf_features(qv[None], M, om)[0] @ po.prf_features(kv[None], M, om)[0])
                assert abs(est - kappa) <= 5.0 * math.sqrt(var / m), (
                    f"MC kernel z-test failed: pair {pair} seed {seed} m={m}: est {est} kappa {kappa}")
    # RMS error falls as m^(-1/2)
    qv = 0.4 * rng.standard_normal(d)
    kv = 0.4 * rng.standard_normal(d)
    kappa = math.exp(float(qv @ (M.T @ M) @ kv) / math.sqrt(d))
    ms2 = [2 ** 6, 2 ** 8, 2 ** 10, 2 ** 12, 2 ** 14]
    rms = []
    for m in ms2:
        errs = []
        for s in range(48):
            om = oo.omega_iid(777 + s, m, r)
            est = float(po.prf_features(qv[None], M, om)[0] @ po.prf_features(kv[None], M, om)[0])
            errs.append(est - kappa)
        rms.append(math.sqrt(float(np.mean(np.square(errs)))))
    slope = float(np.polyfit(np.log(ms2), np.log(rms), 1)[0])
    assert -0.6 <= slope <= -0.4, f"RMS error slope {slope:.3f} not about -1/2"


def check_output_convergence(seed=21):
    """Output error against exact kernel-normalised attention falls like m^(-1/2)."""
    rng = np.random.default_rng(seed)
    B, H, L, d, r = 1, 2, 24, 8, 8
    q = 0.35 * rng.standard_normal((B, H, L, d))
    k = 0.35 * rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    M = np.eye(r, d) + 0.2 * rng.standard_normal((H, r, d))
    exact = po.exact_kernel_attention(q, k, v, M)
    ms = [64, 256, 1024, 4096]
    mean_err = {}
    for orth in (False, True):
        errs = []
        for m in ms:
            e = []
            for s in rng.integers(0, 1 << 62, size=32):
                om = oo.omega(int(s), m, r, orth).astype(np.float64)
                e.append(np.mean((po.attention(q, k, v, M, om) - exact) ** 2))
            errs.append(float(np.sqrt(np.mean(e))))
        slope = float(np.polyfit(np.log(ms), np.log(errs), 1)[0])
        assert -0.7 <= slope <= -0.35, f"output convergence slope {slope:.3f} (orthogonal={orth})"
        mean_err[orth] = float(np.mean(errs))
    assert mean_err[True] <= 1.25 * mean_err[False], f"orthogonal worse than i.i.d.: {mean_err}"


def check_exact_vs_sdpa(seed=31):
    """The exact-limit oracle equals library softmax attention on u = d_h^(-1/4) M x."""
    import torch
    rng = np.random.default_rng(seed)
    B, H, L, d, r = 2, 2, 19, 8, 6
    q, k, v, M, _ = _random_case(rng, B=B, H=H, H_kv=H, Lq=L, d=d, r=r)
    mask = np.ones((B, L), dtype=np.uint8)
    mask[1, 5:9] = 0
    for causal in (False, True):
        O = po.exact_kernel_attention(q, k, v, M, mask=mask, causal=causal)
        uq = np.stack([np.stack([_u(q[b, h], M[h], d) for h in range(H)]) for b in range(B)])
        uk = np.stack([np.stack([_u(k[b, h], M[h], d) for h in range(H)]) for b in range(B)])
        vis = np.ones((B, 1, L, L), dtype=bool) & (mask[:, None, None, :] != 0)
        if causal:
            vis &= np.tril(np.ones((L, L), dtype=bool))[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(uq), torch.from_numpy(uk), torch.from_numpy(v),
            attn_mask=torch.from_numpy(vis), scale=1.0).numpy()
        _close(O, ref, 1e-12, f"exact vs SDPA causal={causal}")
    # grouped K/V heads: query head h reads K/V head h * H_kv / H
    q, k, v, M, _ = _random_case(rng, B=1, H=4, H_kv=2, Lq=L, d=d, r=r)
    O = po.exact_kernel_attention(q, k, v, M, causal=True)
    for h in range(4):
        g = h // 2
        uq, uk = _u(q[0, h], M[h], d), _u(k[0, g], M[h], d)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(uq)[None], torch.from_numpy(uk)[None], torch.from_numpy(v[0, g])[None],
            is_causal=True, scale=1.0).numpy()[0]
        _close(O[0, h], ref, 1e-12, f"exact vs SDPA, GQA head {h}")


# ----------------------------------------------------------------------------
# invariants of normalised positive-feature attention
# ----------------------------------------------------------------------------
def check_invariants(seed=41):
    rng = np.random.default_rng(seed)
    q, k, v, M, om = _random_case(rng, B=2, H=4, H_kv=4, Lq=29)
    # a single valid key gives that key's value exactly
    mask = np.zeros((2, 29), dtype=np.uint8)
    mask[0, 7] = 1
    mask[1, 28] = 1
    O = po.attention(q, k, v, M, om, mask=mask)
    assert np.allclose(O[0], np.broadcast_to(v[0, :, 7][:, None, :], O[0].shape), rtol=1e-13, atol=1e-15)
    assert np.allclose(O[1], np.broadcast_to(v[1, :, 28][:, None, :], O[1].shape), rtol=1e-13, atol=1e-15)
    # causal row 0 is v_0
    Oc = po.attention(q, k, v, M, om, causal=True)
    assert np.allclose(Oc[:, :, 0], v[:, :, 0], rtol=1e-13, atol=1e-15)
    # identical value rows give that row back
    vc = np.broadcast_to(rng.standard_normal(8), v.shape).copy()
    assert np.allclose(po.attention(q, k, vc, M, om), vc[:, :, :1].repeat(29, 2), rtol=1e-12)
    # convex hull of the values, per column
    O = po.attention(q, k, v, M, om)
    lo = v.min(axis=2, keepdims=True)
    hi = v.max(axis=2, keepdims=True)
    assert np.all(O >= lo - 1e-12) and np.all(O <= hi + 1e-12)
    # masked key == deleted key
    mask = np.ones((2, 29), dtype=np.uint8)
    drop = [3, 4, 20]
    mask[:, drop] = 0
    keep = [i for i in range(29) if i not in drop]
    O1 = po.attention(q, k, v, M, om, mask=mask)
    O2 = po.attention(q, k[:, :, keep], v[:, :, keep], M, om)
    _close(O1, O2, 1e-12, "masked == deleted")
    # non-causal output is invariant under a permutation of the keys
    perm = rng.permutation(29)
    _close(po.attention(q, k[:, :, perm], v[:, :, perm], M, om), O, 1e-12, "key permutation")
    # shared geometry == per-head geometry replicated
    Ms = M[0]
    _close(po.attention(q, k, v, Ms, om), po.attention(q, k, v, np.stack([Ms] * 4), om), 1e-13,
           "shared == replicated")
    # grouped K/V heads == K/V repeated to every query head of its group
    q2, k2, v2, M2, om2 = _random_case(rng, B=1, H=4, H_kv=2, Lq=13)
    rep = lambda t: np.repeat(t, 2, axis=1)  # noqa: E731  head h reads kv head h // 2
    _close(po.attention(q2, k2, v2, M2, om2), po.attention(q2, rep(k2), rep(v2), M2, om2), 1e-13,
           "GQA == repeated K/V")
    _close(po.attention(q2, k2, v2, M2, om2, causal=True),
           po.attention(q2, rep(k2), rep(v2), M2, om2, causal=True), 1e-13, "GQA causal")


def check_scaling_rule(seed=51):
    """A positive factor per query row, or one factor on all keys, cancels; one key row does not."""
    rng = np.random.default_rng(seed)
    q, k, v, M, om = _random_case(rng, B=1, H=1, Lq=15)
    PQ = po.prf_features(q[0, 0], M[0], om)
    PK = po.prf_features(k[0, 0], M[0], om)
    O, _, _ = po.attend_noncausal(PQ, PK, v[0, 0])
    c = np.exp(rng.standard_normal((15, 1)))
    _close(po.attend_noncausal(c * PQ, PK, v[0, 0])[0], O, 1e-13, "query-row factor")
    _close(po.attend_noncausal(PQ, 3.7 * PK, v[0, 0])[0], O, 1e-13, "shared key factor")
    PK2 = PK.copy()
    PK2[4] *= 5.0
    assert np.max(np.abs(po.attend_noncausal(PQ, PK2, v[0, 0])[0] - O)) > 1e-6


# ----------------------------------------------------------------------------
# recurrent decoding vs the causal pass
# ----------------------------------------------------------------------------
def check_decode_vs_causal(seed=61, P=37, T=11):
    rng = np.random.default_rng(seed)
    N, H, H_kv, d, m, r = 3, 4, 2, 8, 16, 8
    q, k, v, M, om = _random_case(rng, B=N, H=H, H_kv=H_kv, Lq=P + T, d=d, m=m, r=r)
    full, S_full, z_full = po.attention(q, k, v, M, om, causal=True, return_state=True)
    _, S, z = po.attention(q[:, :, :P], k[:, :, :P], v[:, :, :P], M, om, causal=True,
                           return_state=True)
    outs = []
    for t in range(P, P + T):
        o, S, z = po.decode_step(S, z, q[:, :, t], k[:, :, t], v[:, :, t], M, om)
        outs.append(o)
    _close(np.stack(outs, axis=2), full[:, :, P:], 1e-12, "decode vs causal")
    _close(S, S_full, 1e-12, "decode final S")
    _close(z, z_full, 1e-12, "decode final z")


# ----------------------------------------------------------------------------
# cross-attention (section "Cross-attention"): the context summary written out
# key by key, and the output against the explicit quadratic form
# ----------------------------------------------------------------------------
def check_context_state_explicit(seed=71):
    """S = sum_j phi(k_j) v_j^T and z = sum_j phi(k_j) over valid context keys,
    with phi written out here from the section "Kernel" feature map."""
    rng = np.random.default_rng(seed)
    B, H, H_kv, Lk, d, m, r = 2, 4, 2, 23, 8, 16, 8
    _, k, v, M, om = _random_case(rng, B=B, H=H, H_kv=H_kv, Lq=1, Lk=Lk, d=d, m=m, r=r)
    cmask = (rng.random((B, Lk)) < 0.7).astype(np.uint8)
    S, z = po.context_state(k, v, M, om, H, context_mask=cmask)
    for b in range(B):
        for h in range(H):
            g = (h * H_kv) // H
            S_ref = np.zeros((m, d))
            z_ref = np.zeros(m)
            for j in range(Lk):
                if not cmask[b, j]:
                    continue
                u = _u(k[b, g, j][None, :], M[h], d)[0]
                phi = np.exp(om @ u - 0.5 * float(u @ u)) / math.sqrt(m)
                S_ref += np.outer(phi, v[b, g, j])
                z_ref += phi
            _close(S[b, h], S_ref, 1e-12, f"context S b={b} h={h}")
            _close(z[b, h], z_ref, 1e-12, f"context z b={b} h={h}")


def check_cross_vs_explicit(seed=72):
    """Queries of length L_q against a context of length L_k, GQA, both masks:
    the explicit quadratic form, with masked query rows set to 0."""
    rng = np.random.default_rng(seed)
    B, H, H_kv = 3, 4, 2
    for Lq, Lk in ((1, 9), (13, 40), (29, 5)):
        q, k, v, M, om = _random_case(rng, B=B, H=H, H_kv=H_kv, Lq=Lq, Lk=Lk)
        cmask = (rng.random((B, Lk)) < 0.6).astype(np.uint8)
        cmask[0, 0] = 1
        cmask[2, :] = 0                               # a context with no valid key
        qmask = (rng.random((B, Lq)) < 0.7).astype(np.uint8)
        ref = explicit_attention(q, k, v, M, om, mask=cmask)
        ref = ref * (qmask != 0)[:, None, :, None]
        S, z = po.context_state(k, v, M, om, H, context_mask=cmask)
        O = po.cross_attention(q, S, z, M, om, query_mask=qmask)
        _close(O, ref, 1e-12, f"cross Lq={Lq} Lk={Lk}")
        assert np.all(O[2] == 0.0)


# ----------------------------------------------------------------------------
# backward: the oracle's chain-rule gradients against central finite
# differences of the oracle's forward (pinned above)
# ----------------------------------------------------------------------------
def _fd_case(rng, causal, per_head, H_kv, masked):
    B, H, L, d, m, r = 2, 2, 11, 4, 8, 3
    q, k, v, M, om = _random_case(rng, B=B, H=H, H_kv=H_kv, Lq=L, d=d, m=m, r=r, per_head=per_head)
    q, k = 0.7 * q, 0.7 * k
    mask = None
    if masked:
        mask = np.ones((B, L), np.uint8)
        mask[0, [0, 4, 9]] = 0          # causal: query row 0 of batch 0 sees no key
        mask[1, :] = 0
        mask[1, [3, 7]] = 1
    dout = rng.standard_normal((B, H, L, d))
    return q, k, v, M, om, mask, dout


def check_backward_finite_differences(seed=81, eps=1e-5, n_dir=3):
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        for per_head, H_kv, masked in ((True, 2, False), (True, 1, True), (False, 1, True), (False, 2, False)):
            q, k, v, M, om, mask, dout = _fd_case(rng, causal, per_head, H_kv, masked)
            grads = dict(zip("qkvM", po.attention_backward(q, k, v, M, om, dout, mask=mask, causal=causal)))
            base = dict(q=q, k=k, v=v, M=M)

            def f(**over):
                a = dict(base, **over)
                O = po.attention(a["q"], a["k"], a["v"], a["M"], om, mask=mask, causal=causal)
                return float(np.sum(dout * O))

            for name, x in base.items():
                assert grads[name].shape == x.shape, name
                for _ in range(n_dir):
                    dirn = rng.standard_normal(x.shape)
                    fd = (f(**{name: x + eps * dirn}) - f(**{name: x - eps * dirn})) / (2 * eps)
                    an = float(np.sum(grads[name] * dirn))
                    tol = 1e-6 * max(1.0, abs(fd))
                    assert abs(an - fd) <= tol, (
                        f"d{name} (causal={causal}, per_head={per_head}, H_kv={H_kv}, masked={masked}): "
                        f"analytic {an:.9e} vs finite difference {fd:.9e}")
            if mask is not None:
                # a masked key has no weight anywhere: its k and v rows get no gradient
                for b in range(q.shape[0]):
                    off = np.asarray(mask[b]) == 0
                    assert np.all(grads["k"][b][:, off] == 0) and np.all(grads["v"][b][:, off] == 0)
                if causal:
                    # batch 0, row 0: no visible key, output fixed at 0, so no dq
                    assert np.all(grads["q"][0, :, 0] == 0)


def check_backward_linear_form(seed=82, eps=1e-5):
    """The linear-time non-causal backward of one head: central finite
    differences of the oracle's forward, with a masked key and blocks shorter
    than the sequence; dk and dv of the masked key are exactly 0."""
    rng = np.random.default_rng(seed)
    L, d, m, r = 13, 4, 8, 3
    q, k, v, M, om = _random_case(rng, B=1, H=1, H_kv=1, Lq=L, d=d, m=m, r=r, per_head=False)
    q, k = 0.7 * q, 0.7 * k
    mask = np.ones((1, L), np.uint8)
    mask[0, [2, 8]] = 0
    dout = rng.standard_normal((1, 1, L, d))
    grads = dict(zip("qkvM", po.attention_backward_noncausal_head(q[0, 0], k[0, 0], v[0, 0], M, om, dout[0, 0],
                                                                  key_mask=mask[0], block=5)))
    base = dict(q=q, k=k, v=v, M=M)

    def f(**over):
        a = dict(base, **over)
        return float(np.sum(dout * po.attention(a["q"], a["k"], a["v"], a["M"], om, mask=mask)))

    for name, x in base.items():
        g = grads[name] if name == "M" else grads[name][None, None]
        for _ in range(3):
            dirn = rng.standard_normal(x.shape)
            fd = (f(**{name: x + eps * dirn}) - f(**{name: x - eps * dirn})) / (2 * eps)
            an = float(np.sum(g * dirn))
            assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), f"linear-form d{name}: {an:.9e} vs {fd:.9e}"
    assert np.all(grads["k"][[2, 8]] == 0) and np.all(grads["v"][[2, 8]] == 0)


# ----------------------------------------------------------------------------
# one projection per query head: every head against the explicit form with its
# own omega, a shared omega replicated, the recurrence and the gradients
# ----------------------------------------------------------------------------
def check_per_head_projection(seed=91, eps=1e-5):
    rng = np.random.default_rng(seed)
    B, H, H_kv, L, d, m, r = 2, 4, 2, 19, 8, 16, 8
    q, k, v, M, _ = _random_case(rng, B=B, H=H, H_kv=H_kv, Lq=L, d=d, m=m, r=r)
    om = rng.standard_normal((H, m, r))
    mask = (rng.random((B, L)) < 0.7).astype(np.uint8)
    mask[:, 0] = 1
    for causal in (False, True):
        _close(po.attention(q, k, v, M, om, mask=mask, causal=causal),
               explicit_attention(q, k, v, M, om, mask=mask, causal=causal), 1e-12,
               f"per-head omega vs explicit (causal={causal})")
    # a shared omega equals the same omega given to every head
    _close(po.attention(q, k, v, M, om[1], mask=mask, causal=True),
           po.attention(q, k, v, M, np.stack([om[1]] * H), mask=mask, causal=True), 1e-13,
           "shared omega == replicated")
    # the recurrence with per-head projections
    P = 11
    full, S_full, z_full = po.attention(q, k, v, M, om, causal=True, return_state=True)
    _, S, z = po.attention(q[:, :, :P], k[:, :, :P], v[:, :, :P], M, om, causal=True, return_state=True)
    outs = []
    for t in range(P, L):
        o, S, z = po.decode_step(S, z, q[:, :, t], k[:, :, t], v[:, :, t], M, om)
        outs.append(o)
    _close(np.stack(outs, axis=2), full[:, :, P:], 1e-12, "per-head decode vs causal")
    _close(S, S_full, 1e-12, "per-head decode final S")
    # gradients: central finite differences of the forward
    qs, ks = 0.7 * q[:, :2, :9, :4], 0.7 * k[:, :1, :9, :4]
    vs, Ms, oms = v[:, :1, :9, :4], M[:2, :3, :4], om[:2, :8, :3]
    dout = rng.standard_normal(qs.shape)
    grads = dict(zip("qkvM", po.attention_backward(qs, ks, vs, Ms, oms, dout, causal=True)))
    base = dict(q=qs, k=ks, v=vs, M=Ms)

    def f(**over):
        a = dict(base, **over)
        return float(np.sum(dout * po.attention(a["q"], a["k"], a["v"], a["M"], oms, causal=True)))

    for name, x in base.items():
        dirn = rng.standard_normal(x.shape)
        fd = (f(**{name: x + eps * dirn}) - f(**{name: x - eps * dirn})) / (2 * eps)
        an = float(np.sum(grads[name] * dirn))
        assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), f"per-head d{name}: {an:.9e} vs {fd:.9e}"


ALL_CHECKS = [
    check_per_head_projection,
    check_backward_finite_differences,
    check_backward_linear_form,
    check_closed_form_features,
    check_closed_form_attention,
    check_associative_vs_explicit,
    check_causal_vs_quadratic,
    check_performer_special_case,
    check_invariants,
    check_scaling_rule,
    check_decode_vs_causal,
    check_exact_vs_sdpa,
    check_context_state_explicit,
    check_cross_vs_explicit,
]
