"""fp64 CPU oracle of DARKFormer positive-random-feature (PRF) attention.

TEST INFRASTRUCTURE ONLY.  This is the slow, plain checker that the HIP path is
compared against.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it; the product path never does, and the two share
no code.  Every step is written in the order and notation of the package README
("Data-Aware Random Feature Kernels for Transformers (DARKformer)",
darkformer-pytorch 0.1.0), section "Kernel", with numpy fp64 and matrix
products as the only library primitive.

Notation: x is a query or key row of width d_h; M (r x d_h) is the learned
geometry, Sigma = M^T M; Omega (m x r) holds the feature directions omega_j.

* The attention modules scale q and k by d_h^(-1/4) (section "Kernel",
  scaled-kernel equation), so the kernel is exp(q^T Sigma k / sqrt(d_h)).
* Feature map (section "Kernel", feature-map equation), on the scaled x:
  phi(x)_j = exp(omega_j^T M x - x^T Sigma x / 2) / sqrt(m).
  With u = d_h^(-1/4) M x this is exp(omega_j . u - |u|^2 / 2) / sqrt(m).
* Normalised attention, associative order (section "Kernel", attention
  equation): Phi(Q) (Phi(K)^T V) / Phi(Q) (Phi(K)^T 1).
* Boolean key mask, True = valid token; causal attention combines the mask
  with the causal constraint (section "Self-attention").  Key j is visible to
  query t iff mask[j] and, when causal, j <= t.
* Recurrent decoding keeps the running statistics S = sum phi(k) v^T and
  z = sum phi(k) and updates them per appended token (section "Encoder-decoder
  model and generation").
* Cross-attention (section "Cross-attention"): queries of one sequence attend
  to a context of another length; query and context masks are separate and
  there is no causal option; the context is summarised once as (S, z).

Readings where the README is silent (each is listed with its support in the
design notes): q and k are scaled inside (callers pass unscaled tensors); one
Omega is shared by all heads; M is [H][r][d_h] per head or [r][d_h] shared;
query head h reads key/value head floor(h * H_kv / H); the mask masks keys
only; a query with no visible key gets output 0 (the denominator is positive
otherwise since every feature is positive); the decode output uses the state
after the new token has been added; in cross-attention the context mask masks
context keys and a masked query row gets output 0.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def f64(a) -> np.ndarray:
    """Exact upcast of whatever the device received (fp32 or bf16-valued fp32)."""
    return np.asarray(a, dtype=np.float64)


def qk_scale(d_h: int) -> float:
    """d_h^(-1/4), applied to both queries and keys (section "Kernel")."""
    return float(d_h) ** -0.25


def head_geometry(M: np.ndarray, h: int) -> np.ndarray:
    """M_h: per-head [H][r][d_h] or shared [r][d_h] (per_head_geometry option)."""
    M = f64(M)
    return M[h] if M.ndim == 3 else M


def head_omega(omega: np.ndarray, h: int) -> np.ndarray:
    """Omega_h: one projection per query head [H][m][r], or one [m][r] shared by all heads."""
    omega = np.asarray(omega)
    return omega[h] if omega.ndim == 3 else omega


def kv_head(h: int, H: int, H_kv: int) -> int:
    """Key/value head read by query head h when H_kv heads are shared (GQA)."""
    return (h * H_kv) // H


def project(X: np.ndarray, M_h: np.ndarray) -> np.ndarray:
    """u = d_h^(-1/4) M x for every row x of X: [L][r]."""
    d_h = X.shape[-1]
    return qk_scale(d_h) * (f64(X) @ M_h.T)


def prf_features(X: np.ndarray, M_h: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """phi(x)_j = exp(omega_j^T (M x_s) - x_s^T Sigma x_s / 2) / sqrt(m), x_s = d_h^(-1/4) x.

    Section "Kernel", feature-map equation.  Returns [L][m].
    """
    omega = f64(omega)
    m = omega.shape[0]
    U = project(X, M_h)
    E = U @ omega.T
    half_sq_norm = 0.5 * np.sum(U * U, axis=1, keepdims=True)
    return np.exp(E - half_sq_norm) / np.sqrt(m)


def _ratio(N: np.ndarray, D: np.ndarray) -> np.ndarray:
    """N / D row-wise; rows whose denominator is not positive (no visible key) give 0."""
    out = np.zeros_like(N)
    ok = D > 0
    out[ok] = N[ok] / D[ok, None]
    return out


def attend_noncausal(PQ: np.ndarray, PK: np.ndarray, V: np.ndarray):
    """Phi(Q) (Phi(K)^T V) / Phi(Q) (Phi(K)^T 1) (section "Kernel", attention equation).

    PK rows of masked keys are already zero.  Returns (O, S, z) with
    S = Phi(K)^T V [m][d_h] and z = Phi(K)^T 1 [m].
    """
    S = PK.T @ V
    z = PK.T @ np.ones(PK.shape[0])
    return _ratio(PQ @ S, PQ @ z), S, z


def attend_causal_blockwise(PQ: np.ndarray, PK: np.ndarray, V: np.ndarray, block: int = 256):
    """Causal form: query t sees the keys j <= t, as a block-by-block prefix scan.

    Per block [s, e): A = tril(Phi(Q_blk) Phi(K_blk)^T) with the diagonal kept,
    N = Phi(Q_blk) S + A V_blk, D = Phi(Q_blk) z + A 1, then the running state is
    advanced by S += Phi(K_blk)^T V_blk, z += Phi(K_blk)^T 1.  Returns (O, S, z)
    with (S, z) the state after the last token.
    """
    L, m = PQ.shape
    d = V.shape[1]
    S = np.zeros((m, d))
    z = np.zeros(m)
    O = np.zeros((L, d))
    for s in range(0, L, block):
        e = min(L, s + block)
        A = np.tril(PQ[s:e] @ PK[s:e].T)
        N = PQ[s:e] @ S + A @ V[s:e]
        D = PQ[s:e] @ z + A @ np.ones(e - s)
        O[s:e] = _ratio(N, D)
        S = S + PK[s:e].T @ V[s:e]
        z = z + PK[s:e].T @ np.ones(e - s)
    return O, S, z


def attention(q, k, v, M, omega, mask: Optional[np.ndarray] = None, causal: bool = False,
              block: int = 256, heads: Optional[list] = None, return_state: bool = False):
    """DARKFormer linear-mode attention core.

    q [B][H][L][d_h], k and v [B][H_kv][L][d_h], M [H][r][d_h] or [r][d_h],
    omega [m][r] or [H][m][r] (one projection per query head), mask [B][L]
    (nonzero = valid key) or None.
    `heads` restricts the work to a list of (b, h) pairs (other outputs stay 0).
    Returns O [B][H][L][d_h] (fp64) and, if return_state, S [B][H][m][d_h] and
    z [B][H][m]: the state after the last token.
    """
    q, k, v = f64(q), f64(k), f64(v)
    B, H, L, d = q.shape
    H_kv = k.shape[1]
    m = np.asarray(omega).shape[-2]
    O = np.zeros((B, H, L, d))
    S_all = np.zeros((B, H, m, d)) if return_state else None
    z_all = np.zeros((B, H, m)) if return_state else None
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        g = kv_head(h, H, H_kv)
        M_h, om_h = head_geometry(M, h), head_omega(omega, h)
        PQ = prf_features(q[b, h], M_h, om_h)
        PK = prf_features(k[b, g], M_h, om_h)
        if mask is not None:
            PK = PK * (np.asarray(mask[b]) != 0)[:, None]
        if causal:
            O[b, h], S, z = attend_causal_blockwise(PQ, PK, v[b, g], block)
        else:
            O[b, h], S, z = attend_noncausal(PQ, PK, v[b, g])
        if return_state:
            S_all[b, h], z_all[b, h] = S, z
    if return_state:
        return O, S_all, z_all
    return O


def decode_step(S, z, q, k, v, M, omega):
    """One appended token for every sequence n and head h (recurrent statistics).

    S [N][H][m][d_h], z [N][H][m] (fp64, updated copies are returned),
    q [N][H][d_h], k and v [N][H_kv][d_h].  The new key/value pair is added to the
    state first; the output then reads the updated state:
    S += phi(k) v^T, z += phi(k), o = phi(q)^T S / phi(q)^T z.
    """
    S = f64(S).copy()
    z = f64(z).copy()
    q, k, v = f64(q), f64(k), f64(v)
    N, H, d = q.shape
    H_kv = k.shape[1]
    o = np.zeros((N, H, d))
    for h in range(H):
        g = kv_head(h, H, H_kv)
        M_h = head_geometry(M, h)
        pq = prf_features(q[:, h], M_h, head_omega(omega, h))      # [N][m]
        pk = prf_features(k[:, g], M_h, head_omega(omega, h))      # [N][m]
        S[:, h] += pk[:, :, None] * v[:, g][:, None, :]
        z[:, h] += pk
        num = np.einsum("nm,nmd->nd", pq, S[:, h])
        den = np.einsum("nm,nm->n", pq, z[:, h])
        o[:, h] = _ratio(num, den)
    return o, S, z


def context_state(k, v, M, omega, H: int, context_mask: Optional[np.ndarray] = None):
    """Summary of an encoded source for cross-attention (section "Cross-attention";
    section "Encoder-decoder model and generation": decoder cross-attention
    projects and summarises the source once per layer).

    k and v [B][H_kv][L_k][d_h], context_mask [B][L_k] (nonzero = valid) or None.
    For every batch row b and query head h (geometry M_h, K/V head g(h)):
    S = Phi(K)^T V and z = Phi(K)^T 1 over the valid context keys.
    Returns S [B][H][m][d_h] and z [B][H][m].
    """
    k, v = f64(k), f64(v)
    B, H_kv, L_k, d = k.shape
    m = np.asarray(omega).shape[-2]
    S = np.zeros((B, H, m, d))
    z = np.zeros((B, H, m))
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, H_kv)
            PK = prf_features(k[b, g], head_geometry(M, h), head_omega(omega, h))
            if context_mask is not None:
                PK = PK * (np.asarray(context_mask[b]) != 0)[:, None]
            S[b, h] = PK.T @ v[b, g]
            z[b, h] = PK.T @ np.ones(L_k)
    return S, z


def cross_attention(q, S, z, M, omega, query_mask: Optional[np.ndarray] = None):
    """Queries against a context summary (section "Cross-attention"): query and
    context masks stay separate; there is no causal option.

    q [B][H][L_q][d_h], S [B][H][m][d_h], z [B][H][m] (from context_state),
    query_mask [B][L_q] (nonzero = valid) or None.
    O_t = Phi(q_t) S / Phi(q_t) z; a masked query row, or one whose denominator
    is not positive (no valid context key), gives 0.
    """
    q, S, z = f64(q), f64(S), f64(z)
    B, H, L_q, d = q.shape
    O = np.zeros((B, H, L_q, d))
    for b in range(B):
        for h in range(H):
            PQ = prf_features(q[b, h], head_geometry(M, h), head_omega(omega, h))
            O[b, h] = _ratio(PQ @ S[b, h], PQ @ z[b, h])
            if query_mask is not None:
                O[b, h][np.asarray(query_mask[b]) == 0] = 0.0
    return O


def exact_kernel_attention(q, k, v, M, mask: Optional[np.ndarray] = None, causal: bool = False):
    """Exact normalised attention under the learned kernel exp(q^T Sigma k / sqrt(d_h)).

    The limit m -> infinity of the feature estimator (section "Kernel"; section
    "Attention modes": the exact path applies the geometry to q and k and then
    runs softmax attention).  Textbook softmax with a row-max shift, fp64.
    Query rows with no visible key give 0.
    """
    q, k, v = f64(q), f64(k), f64(v)
    B, H, L, d = q.shape
    Lk = k.shape[2]
    H_kv = k.shape[1]
    O = np.zeros((B, H, L, d))
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, H_kv)
            M_h = head_geometry(M, h)
            logits = project(q[b, h], M_h) @ project(k[b, g], M_h).T
            visible = np.ones((L, Lk), dtype=bool)
            if mask is not None:
                visible &= (np.asarray(mask[b]) != 0)[None, :]
            if causal:
                visible &= np.tril(np.ones((L, Lk), dtype=bool))
            logits = np.where(visible, logits, -np.inf)
            rowmax = np.max(logits, axis=1, keepdims=True)
            has = np.isfinite(rowmax[:, 0])
            w = np.zeros_like(logits)
            w[has] = np.exp(logits[has] - rowmax[has])
            den = w.sum(axis=1)
            O[b, h] = _ratio(w @ v[b, g], den)
    return O


def attention_backward(q, k, v, M, omega, dout, mask: Optional[np.ndarray] = None, causal: bool = False):
    """Gradients of the linear-mode attention core with respect to q, k, v and M.

    The package README (section "Kernel") has M learned, and the DARKFormer
    abstract pages finetune the q-k-v projections together with the
    projection covariance (Figure 4), so the core needs gradients for q, k,
    v and M.  Omega is a fixed random draw and gets none.  The pages give no
    backward formulas: this is the chain rule applied to the forward as
    defined above, written with the quadratic weight matrix
    W[t, j] = phi(q_t) . phi(k_j) * visible(t, j), so O = (W V) / (W 1):

      D_t = sum_j W[t, j], O_t = N_t / D_t with N = W V;
      dN_t = dO_t / D_t,  dD_t = -(dO_t . O_t) / D_t  (both 0 where D_t = 0);
      dW[t, j] = visible(t, j) * (dN_t . v_j + dD_t);   dV = W^T dN;
      dPhi(Q) = dW Phi(K),  dPhi(K) = dW^T Phi(Q);
      phi_j(u) = exp(omega_j . u - |u|^2 / 2) / sqrt(m), so
      dU = (dPhi * Phi) Omega - U * rowsum(dPhi * Phi);
      u = s M x with s = d_h^(-1/4):  dX = s dU M,  dM += s dU^T X.

    With H_kv < H, dk and dv of a key/value head sum over the query heads that
    read it; a shared M ([r][d_h]) sums dM over heads.  Returns fp64
    (dq, dk, dv, dM) shaped like q, k, v and M.
    """
    q, k, v, dout = f64(q), f64(k), f64(v), f64(dout)
    B, H, L, d = q.shape
    H_kv = k.shape[1]
    omega = f64(omega)
    s = qk_scale(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dM = np.zeros_like(f64(M))
    vis = np.tril(np.ones((L, L))) if causal else np.ones((L, L))
    for b in range(B):
        visb = vis if mask is None else vis * (np.asarray(mask[b]) != 0)[None, :]
        for h in range(H):
            g = kv_head(h, H, H_kv)
            M_h, om_h = head_geometry(M, h), head_omega(omega, h)
            UQ, UK = project(q[b, h], M_h), project(k[b, g], M_h)
            PQ = prf_features(q[b, h], M_h, om_h)
            PK = prf_features(k[b, g], M_h, om_h)
            W = (PQ @ PK.T) * visb
            D = W.sum(axis=1)
            O = _ratio(W @ v[b, g], D)
            ok = D > 0
            dN = np.zeros((L, d))
            dD = np.zeros(L)
            dN[ok] = dout[b, h][ok] / D[ok, None]
            dD[ok] = -np.sum(dout[b, h][ok] * O[ok], axis=1) / D[ok]
            dW = visb * (dN @ v[b, g].T + dD[:, None])
            dv[b, g] += W.T @ dN
            grads = []
            for P, U, dP in ((PQ, UQ, dW @ PK), (PK, UK, dW.T @ PQ)):
                dE = dP * P
                grads.append(dE @ om_h - U * dE.sum(axis=1, keepdims=True))
            dUQ, dUK = grads
            dq[b, h] += s * (dUQ @ M_h)
            dk[b, g] += s * (dUK @ M_h)
            dM_h = s * (dUQ.T @ q[b, h] + dUK.T @ k[b, g])
            if dM.ndim == 3:
                dM[h] += dM_h
            else:
                dM += dM_h
    return dq, dk, dv, dM


def attention_backward_noncausal_head(q, k, v, M_h, omega, dout, key_mask=None, block: int = 4096):
    """Gradients of one non-causal (b, h) slice in linear time, for long inputs.

    The same chain rule as attention_backward, with the sums over the other
    side taken through totals instead of the quadratic weights (section
    "Kernel", attention equation, associative order): S = Phi(K)^T V and
    z = Phi(K)^T 1 for the outputs and dPhi(Q) = dN S^T + dD z^T; then
    G = Phi(Q)^T dN and g = Phi(Q)^T dD for dPhi(K) = V G^T + 1 g^T and
    dV = Phi(K) G.  Rows are processed in blocks of `block`.  q, k, v, dout are
    [L][d_h], M_h [r][d_h], key_mask [L] or None.  Returns (dq, dk, dv, dM_h),
    where dk, dv, dM_h are this head's contributions.
    """
    q, k, v, dout, omega, M_h = f64(q), f64(k), f64(v), f64(dout), f64(omega), f64(M_h)
    L, d = q.shape
    m = omega.shape[0]
    s = qk_scale(d)
    valid = np.ones(L) if key_mask is None else (np.asarray(key_mask) != 0).astype(np.float64)

    def feats(X, lo, hi):
        return prf_features(X[lo:hi], M_h, omega), project(X[lo:hi], M_h)

    def through_features(dP, P, U, X):
        dE = dP * P
        dU = dE @ omega - U * dE.sum(axis=1, keepdims=True)
        return s * (dU @ M_h), s * (dU.T @ X)

    S = np.zeros((m, d))
    z = np.zeros(m)
    for lo in range(0, L, block):
        PK, _ = feats(k, lo, lo + block)
        PK = PK * valid[lo:lo + block, None]
        S += PK.T @ v[lo:lo + block]
        z += PK.sum(axis=0)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dM = np.zeros_like(M_h)
    G = np.zeros((m, d))
    g = np.zeros(m)
    for lo in range(0, L, block):
        hi = min(L, lo + block)
        PQ, UQ = feats(q, lo, hi)
        N, D = PQ @ S, PQ @ z
        O = _ratio(N, D)
        ok = D > 0
        dN = np.zeros_like(N)
        dD = np.zeros(hi - lo)
        dN[ok] = dout[lo:hi][ok] / D[ok, None]
        dD[ok] = -np.sum(dout[lo:hi][ok] * O[ok], axis=1) / D[ok]
        G += PQ.T @ dN
        g += PQ.T @ dD
        dq[lo:hi], dMq = through_features(dN @ S.T + dD[:, None] * z[None, :], PQ, UQ, q[lo:hi])
        dM += dMq
    for lo in range(0, L, block):
        hi = min(L, lo + block)
        PK, UK = feats(k, lo, hi)
        PK = PK * valid[lo:hi, None]
        dv[lo:hi] = PK @ G
        dk[lo:hi], dMk = through_features(v[lo:hi] @ G.T + g[None, :], PK, UK, k[lo:hi])
        dM += dMk
    return dq, dk, dv, dM
