"""Oracle-side construction of the random projection Omega (m x r) from a seed.

TEST INFRASTRUCTURE ONLY: this package is the fp64 checker of the device path.
Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import it.
It shares no code with the HIP library, which builds Omega with its own C++ code
from the same published definitions.

What is drawn (darkformer-pytorch README, section "Kernel", feature-map equation:
each omega_j is standard Gaussian; section "Self-attention": orthogonal Gaussian
blocks by default, independent Gaussian features when orthogonal_features=False;
section "Projection lifecycle": a projection seed makes the draw reproducible):

* counter-based uniform stream: SplitMix64 (Steele, Lea and Flood, "Fast
  Splittable Pseudorandom Number Generators", OOPSLA 2014): output i of seed s is
  mix64(s + (i + 1) * 0x9E3779B97F4A7C15) with Stafford's "Mix13" finaliser;
  u_i = ((x_i >> 11) + 1) * 2^-53, a value in (0, 1];
* Gaussians: Box-Muller (Box and Muller, 1958) on the pair (u_2p, u_2p+1):
  n_2p = sqrt(-2 ln u_2p) cos(2 pi u_2p+1), n_2p+1 = sqrt(-2 ln u_2p) sin(2 pi u_2p+1);
* i.i.d. features: Omega[j][c] = n_(j r + c);
* orthogonal blocks: block b (rows b r ... b r + r - 1, the last one truncated to m)
  takes G[a][c] = n_(2 b r^2 + a r + c) and Hn[a][c] = n_(2 b r^2 + r^2 + a r + c);
  Q R = G is the QR factorisation, Q is made Haar-distributed by multiplying each
  column by the sign of the matching diagonal entry of R (Mezzadri, "How to
  generate random matrices from the classical compact groups", Notices AMS 2007),
  and row a of the block is ||Hn[a, :]|| * Q[a, :], so that every row has a
  chi_r-distributed norm like an unconstrained Gaussian row.

All arithmetic is fp64; the result is rounded once to float32.
"""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start ... start+count-1 of the SplitMix64 stream of `seed` (uint64)."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & _MASK64) + idx * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniforms(seed: int, start: int, count: int) -> np.ndarray:
    """u_i in (0, 1] as float64."""
    x = splitmix64(seed, start, count)
    return ((x >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def normals(seed: int, start: int, count: int) -> np.ndarray:
    """Gaussians n_start ... n_(start+count-1) (float64) by Box-Muller pairs."""
    p0 = start // 2
    p1 = (start + count + 1) // 2
    u = uniforms(seed, 2 * p0, 2 * (p1 - p0)).reshape(-1, 2)
    rad = np.sqrt(-2.0 * np.log(u[:, 0]))
    ang = 2.0 * np.pi * u[:, 1]
    pairs = np.stack([rad * np.cos(ang), rad * np.sin(ang)], axis=1).reshape(-1)
    off = start - 2 * p0
    return pairs[off:off + count]


def omega_iid(seed: int, m: int, r: int) -> np.ndarray:
    return normals(seed, 0, m * r).reshape(m, r)


def omega_orthogonal(seed: int, m: int, r: int) -> np.ndarray:
    nblocks = -(-m // r)
    rows = []
    for b in range(nblocks):
        base = 2 * b * r * r
        G = normals(seed, base, r * r).reshape(r, r)
        Hn = normals(seed, base + r * r, r * r).reshape(r, r)
        Q, R = np.linalg.qr(G)
        Q = Q * np.sign(np.diag(R))[None, :]
        norms = np.sqrt(np.sum(Hn * Hn, axis=1))
        keep = min(r, m - b * r)
        rows.append(norms[:keep, None] * Q[:keep, :])
    return np.concatenate(rows, axis=0)


def omega(seed: int, m: int, r: int, orthogonal: bool) -> np.ndarray:
    """Omega as float32 [m][r] (the values both sides feed to the attention)."""
    om = omega_orthogonal(seed, m, r) if orthogonal else omega_iid(seed, m, r)
    return om.astype(np.float32)


def head_seed(seed: int, h: int) -> int:
    """Seed of query head h's projection when every head draws its own: SplitMix64's
    finaliser (the same Mix13 steps as in splitmix64 above) applied to
    seed + (h + 1) * 0xD1B54A32D192ED03 modulo 2^64.  Written with Python integers."""
    z = (seed + (h + 1) * 0xD1B54A32D192ED03) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def omega_per_head(seed: int, H: int, m: int, r: int, orthogonal: bool) -> np.ndarray:
    """Per-head projections [H][m][r] (float32): head h is omega(head_seed(seed, h), m, r, orthogonal)."""
    return np.stack([omega(head_seed(seed, h), m, r, orthogonal) for h in range(H)])
