// Backward pass of the linear-mode attention core: gradients for q, k, v and
// the learned geometry M (package README "Data-Aware Random Feature Kernels
// for Transformers (DARKformer)", section "Kernel": M is learned; the
// DARKFormer abstract pages finetune the q-k-v projections together with the
// projection covariance, Figure 4).  Omega is a fixed draw and gets none.
//
// With u = s M_h x (s = d_h^(-1/4)), phi the feature map, the visible weights
// W[t][j] = phi(q_t).phi(k_j) (j valid under the key mask, and j <= t when
// causal), N = W V, D = W 1 and O = N / D, the chain rule gives
//   Gd_t = [dN_t, dD_t] = [dO_t / D_t, -(dO_t . O_t) / D_t]   (0 when D_t = 0)
//   dW[t][j] = visible * ([V, 1]_j . Gd_t)
//   dPhi(Q) = dW Phi(K),  dPhi(K) = dW^T Phi(Q),  dV = W^T dN
//   dU = (dPhi * Phi) Omega - U * rowsum(dPhi * Phi)
//   dX = s dU M_h,  dM_h += s dU^T X.
// The quadratic products are never formed: as in the forward, the sequence is
// cut into chunks of C tokens and the sums over earlier (or later) chunks go
// through m x (d_h + 1) states, with exclusive prefix sums over chunks:
//   Sx_c = sum_{c' < c} Phi(K_c')^T [V, 1]_c'        (key side, forward scan)
//   Gx_c = sum_{c' > c} Phi(Q_c')^T Gd_c'            (query side, reverse scan)
//   [N, D]_c = Phi(Q_c) Sx_c + tril(Phi(Q_c) Phi(K_c)^T) [V, 1]_c
//   dPhi(Q)_c = Gd_c Sx_c^T + tril(Gd_c [V, 1]_c^T) Phi(K_c)
//   dPhi(K)_c = [V, 1]_c Gx_c^T + tril(Gd_c [V, 1]_c^T)^T Phi(Q_c)
//   dV_c = Phi(K_c) Gx_c[:, :d] + tril(Phi(Q_c) Phi(K_c)^T)^T dN_c.
// Without causality the states are the plain totals and the tril terms vanish.
//
// Every product runs through one batched GEMM kernel: 64 x 64 output tiles,
// 32-deep K slices staged through LDS, operands addressed by strides so that
// transposed operands need no copies.  Features, states and intermediate
// gradients are fp32 in the workspace.  The products run on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32); for bf16 inputs the plain products (not the
// feature exponents or the intra-chunk scores) run on the bf16 matrix cores
// instead, each staged fp32 operand split into a bf16 high part and a bf16
// remainder and the three products hi*hi + lo*hi + hi*lo summed in fp32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>

#include "common.h"

namespace dk {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tokens per chunk.  The causal prefix needs a state per chunk; longer chunks
// write fewer m x (d_h + 1) states but do more intra-chunk work: 128 tokens pay
// off once the state is wide (d_h >= 128), 64 below.
inline int bwd_chunk(const dark_prf_desc& d) { return d.causal && d.d_h >= 128 ? 128 : 64; }
constexpr int kMTarget = 1024; // workgroups the split dM reduction aims for
constexpr int kSTarget = 4096; // workgroups the non-causal state partials aim for

__device__ __forceinline__ float ld_f(const float* p) { return *p; }
__device__ __forceinline__ float ld_f(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ void st_t(float* p, float x) { *p = x; }
__device__ __forceinline__ void st_t(uint16_t* p, float x) {   // round to nearest even
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  *p = (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Operand element (i, k) of batch (b, h, c) sits at
// p + b*sb + (h / hg)*sh + c*sc + i*si + k*sk.
struct GOp {
  const void* p;
  int64_t sb, sh, sc, si, sk;
  int hg;
  const float* p2;   // PROD operands: element (i, k) is p[..] * p2[..] (same offsets)
};
struct GOut {
  float* p;
  int64_t sb, sh, sc, si;
};

enum Epi { kEpiPlain = 0, kEpiTril = 1, kEpiFeature = 2 };

struct GemmArgs {
  GOp A, B;
  GOut C;           // element (i, j) at p + b*sb + h*sh + c*sc + i*si + j
  int M, N, K;      // C (M x N) = alpha * A (M x K) * B (K x N), per batch
  int Ktot;         // > 0: batch c reduces over min(K, Ktot - c*K) terms
  int Arows;        // rows of A at or beyond this read as 0
  int H, NCB;       // batch = (b*H + h)*NCB + c
  int tiles_n, tiles;
  // PROD with k contiguous in A: rowsum[bh*rs_sbh + i] = sum_k A(i, k), written
  // by the workgroups of the first column tile
  float* rowsum;
  int64_t rs_sbh;
  float alpha;
  int accumulate;   // C += result instead of C = result
  int epi;
  // kEpiFeature: C = valid ? exp(acc - nrm[bh*nrm_sbh + i]) * alpha : 0, valid =
  // i < L and (mask == null or b < mask_b0 or mask[(b - mask_b0)*L + i] != 0)
  // (a launch over queries then keys masks the batch rows from mask_b0 on)
  const float* nrm;
  int64_t nrm_sbh;
  const uint8_t* mask;
  int mask_b0;
  int L;
};

constexpr int kKT = 32;   // K depth of one LDS slice

// XC: the last output column N - 1 is not tiled; it is accumulated on the
// vector ALUs from the A values each thread stages (A(i, k) * B(k, N - 1)) and
// reduced at the end, so an odd width such as d_h + 1 needs no extra tile.
// PREC kHiLo (bf16 inputs): the fp32 operands staged in LDS are split into
// bf16 hi + lo parts and multiplied on the bf16 matrix cores (32x32x16), as
// A_hi B_hi + A_lo B_hi + A_hi B_lo with fp32 accumulation: about 16
// significant bits per operand, at a fraction of the fp32 products' cost.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
enum Prec { kF32 = 0, kHiLo = 1 };
template <typename TA, typename TB, bool PROD, bool XC = false, int PREC = kF32>
__global__ __launch_bounds__(256) void bgemm_kernel(GemmArgs a) {
  constexpr int KT = kKT, NE = 64 * KT / 256;   // elements of each operand per thread and slice
  __shared__ float As[64][KT + 1];   // [i][k]
  __shared__ float Bs[KT][65];       // [k][j]
  const int64_t bid = blockIdx.x;
  const int batch = (int)(bid / a.tiles);
  const int tile = (int)(bid - (int64_t)batch * a.tiles);
  const int tm = tile / a.tiles_n, tn = tile - tm * a.tiles_n;
  const int bh = batch / a.NCB, c = batch - bh * a.NCB;
  const int b = bh / a.H, h = bh - b * a.H;
  const int64_t aoff = b * a.A.sb + (int64_t)(h / a.A.hg) * a.A.sh + c * a.A.sc;
  const TA* A = static_cast<const TA*>(a.A.p) + aoff;
  const float* A2 = PROD ? a.A.p2 + aoff : nullptr;
  const TB* Bp = static_cast<const TB*>(a.B.p) + b * a.B.sb + (int64_t)(h / a.B.hg) * a.B.sh + c * a.B.sc;
  float* C = a.C.p + b * a.C.sb + h * a.C.sh + c * a.C.sc;
  const int K = a.Ktot > 0 ? min(a.K, a.Ktot - c * a.K) : a.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int wi = (wave >> 1) * 32, wj = (wave & 1) * 32;
  const int i0 = tm * 64, j0 = tn * 64;
  const bool a_krow = a.A.sk == 1;   // k contiguous in A: threads walk k
  const bool b_jrow = a.B.sk == 1;   // j contiguous in B: threads walk j
  // offsets inside one batch fit in 32 bits (checked on the host)
  const int asi = (int)a.A.si, ask = (int)a.A.sk, bsi = (int)a.B.si, bsk = (int)a.B.sk;
  const int NT = XC ? a.N - 1 : a.N;   // tiled columns
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  // the next K slice is fetched into registers while the current one is
  // multiplied out of LDS
  float ra[NE], rb[NE];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int e8 = 0; e8 < NE; ++e8) {
      const int e = tid + 256 * e8;
      int i, k;
      if (a_krow) { i = e / KT; k = e % KT; } else { i = e & 63; k = e >> 6; }
      const int gi = i0 + i, gk = k0 + k;
      if (gi < a.Arows && gk < K) {
        const int o = gi * asi + gk * ask;
        ra[e8] = PROD ? ld_f(A + o) * A2[o] : ld_f(A + o);
      } else {
        ra[e8] = 0.f;
      }
      int kb, j;
      if (b_jrow) { kb = e >> 6; j = e & 63; } else { kb = e % KT; j = e / KT; }
      const int gkb = k0 + kb, gj = j0 + j;
      rb[e8] = (gkb < K && gj < NT) ? ld_f(Bp + (gkb * bsi + gj * bsk)) : 0.f;
    }
  };
  // the last column: k contiguous in A puts row tid / KT + (256 / KT) e8 and
  // column k = tid % KT in element e8; otherwise row tid & 63 and column
  // tid / 64 + 4 e8.  rbx holds B(k, N - 1) for the thread's columns.
  float xacc[NE], rbx[NE];
#pragma unroll
  for (int e8 = 0; e8 < NE; ++e8) xacc[e8] = rbx[e8] = 0.f;
  auto fetch_x = [&](int k0) {
    if (!XC) return;
#pragma unroll
    for (int e8 = 0; e8 < NE; ++e8) {
      const int k = k0 + (a_krow ? tid % KT : (tid >> 6) + 4 * e8);
      rbx[e8] = k < K ? ld_f(Bp + (k * bsi + (a.N - 1) * bsk)) : 0.f;
      if (a_krow) break;   // one column per thread
    }
  };
  // with k contiguous in A, thread tid holds rows tid / KT + (256 / KT) e8 in every slice
  float rsum[NE];
#pragma unroll
  for (int e8 = 0; e8 < NE; ++e8) rsum[e8] = 0.f;
  fetch(0);
  fetch_x(0);
  for (int k0 = 0; k0 < K; k0 += KT) {
#pragma unroll
    for (int e8 = 0; e8 < NE; ++e8) {
      const int e = tid + 256 * e8;
      if (PROD) rsum[e8] += ra[e8];
      if (XC) xacc[e8] = fmaf(ra[e8], a_krow ? rbx[0] : rbx[e8], xacc[e8]);
      if (a_krow) As[e / KT][e % KT] = ra[e8];
      else As[e & 63][e >> 6] = ra[e8];
      if (b_jrow) Bs[e >> 6][e & 63] = rb[e8];
      else Bs[e % KT][e / KT] = rb[e8];
    }
    __syncthreads();
    if (k0 + KT < K) {
      fetch(k0 + KT);
      fetch_x(k0 + KT);
    }
    if constexpr (PREC == kHiLo) {
      // operand fragments: row (column) l32 of the wave's block at K-slots 8g .. 8g + 7
#pragma unroll
      for (int kk = 0; kk < KT; kk += 16) {
        bf16x8_t ah, al, bh, bl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = As[wi + l32][kk + 8 * g + e], y = Bs[kk + 8 * g + e][wj + l32];
          const __bf16 xh = (__bf16)x, yh = (__bf16)y;
          ah[e] = xh;
          al[e] = (__bf16)(x - (float)xh);
          bh[e] = yh;
          bl[e] = (__bf16)(y - (float)yh);
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KT; kk += 8)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[wi + l32][kk + 4 * g + s], Bs[kk + 4 * g + s][wj + l32],
                                                     acc, 0, 0, 0);
    }
    __syncthreads();
  }
  if (PROD && a.rowsum != nullptr && tn == 0) {   // KT lanes share a row
#pragma unroll
    for (int e8 = 0; e8 < NE; ++e8) {
      float v = rsum[e8];
#pragma unroll
      for (int o = KT / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      const int row = i0 + tid / KT + (256 / KT) * e8;
      if ((tid % KT) == 0 && row < a.M) a.rowsum[bh * a.rs_sbh + row] = v;
    }
  }
  if (XC && tn == 0) {
    // the last column, written like the tiled ones (plain or accumulate)
    auto put = [&](int row, float v) {
      if (row >= a.M) return;
      float* cp = C + row * a.C.si + (a.N - 1);
      const float x = a.alpha * v;
      *cp = a.accumulate ? *cp + x : x;
    };
    if (a_krow) {   // KT lanes share each row
#pragma unroll
      for (int e8 = 0; e8 < NE; ++e8) {
        float v = xacc[e8];
#pragma unroll
        for (int o = KT / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        if ((tid % KT) == 0) put(i0 + tid / KT + (256 / KT) * e8, v);
      }
    } else {        // the four waves share each row: sum through LDS
      float v = 0.f;
#pragma unroll
      for (int e8 = 0; e8 < NE; ++e8) v += xacc[e8];
      float* red = &As[0][0];   // free after the last slice's barrier
      red[tid] = v;
      __syncthreads();
      if (tid < 64) put(i0 + tid, red[tid] + red[tid + 64] + red[tid + 128] + red[tid + 192]);
    }
  }
  const int col = j0 + wj + l32;
  if (col >= NT) return;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = i0 + wi + 8 * (e >> 2) + 4 * g + (e & 3);
    if (row >= a.M) continue;
    float x = a.alpha * acc[e];
    if (a.epi == kEpiTril) {
      if (col > row) x = 0.f;
    } else if (a.epi == kEpiFeature) {
      const bool ok = row < a.L && (a.mask == nullptr || b < a.mask_b0 ||
                                    a.mask[(int64_t)(b - a.mask_b0) * a.L + row] != 0);
      x = ok ? __expf(acc[e] - a.nrm[bh * a.nrm_sbh + row]) * a.alpha : 0.f;
    }
    float* cp = C + row * a.C.si + col;
    if (a.accumulate) x += *cp;
    *cp = x;
  }
}

// [V, 1] rows of query head h (its key/value head), fp32; rows t >= L are 0.
template <typename T>
__global__ void vx_kernel(const T* v, int64_t sb, int64_t sh, int64_t sl, float* Vx, int H, int hg, int L, int Lp,
                          int d, int64_t total) {
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(idx % (d + 1));
    const int64_t row = idx / (d + 1);
    const int t = (int)(row % Lp);
    const int bh = (int)(row / Lp);
    const int b = bh / H, h = bh - b * H;
    float x = 0.f;
    if (t < L) x = e < d ? ld_f(v + b * sb + (int64_t)(h / hg) * sh + t * sl + e) : 1.f;
    Vx[idx] = x;
  }
}

// nrm[row] = |U_row|^2 / 2 (one wave per row)
__global__ __launch_bounds__(256) void halfnorm_kernel(const float* U, float* nrm, int r, int64_t rows) {
  const int64_t row = blockIdx.x * 4LL + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* u = U + row * r;
  float s = 0.f;
  for (int j = lane; j < r; j += 64) s = fmaf(u[j], u[j], s);
  s = wave_sum(s);
  if (lane == 0) nrm[row] = 0.5f * s;
}

// Gd = [dO / D, -(dO . O) / D] per row (one wave per row), 0 when D <= 0 or t >= L.
template <typename T>
__global__ __launch_bounds__(256) void gd_kernel(const T* dout, int64_t sb, int64_t sh, int64_t sl, const float* ND,
                                                 float* Gd, int H, int L, int Lp, int d, int64_t rows) {
  const int64_t row = blockIdx.x * 4LL + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int t = (int)(row % Lp);
  const int bh = (int)(row / Lp);
  const int b = bh / H, h = bh - b * H;
  const float* nd = ND + row * (d + 1);
  float* gd = Gd + row * (d + 1);
  const float D = nd[d];
  const bool ok = t < L && D > 0.f;
  const float inv = ok ? 1.f / D : 0.f;
  float dot = 0.f;
  for (int e = lane; e < d; e += 64) {
    const float go = ok ? ld_f(dout + b * sb + h * sh + t * sl + e) : 0.f;
    dot = fmaf(go, nd[e] * inv, dot);
    gd[e] = go * inv;
  }
  dot = wave_sum(dot);
  if (lane == 0) gd[d] = -dot * inv;
}

// dU -= U * rs (per row)
__global__ void fixdu_kernel(float* dU, const float* U, const float* rs, int r, int64_t total) {
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x)
    dU[idx] -= U[idx] * rs[idx / r];
}

// Exclusive prefix (reverse = 0) or suffix (reverse = 1) sums over the NC
// chunk states of each (b, h), in place; X floats per state.  The states are
// read in groups of 16 whose loads are all in flight together (one memory
// latency per group instead of one per state).
__global__ void chunk_scan_kernel(float* buf, int NC, int64_t X, int64_t total, int reverse) {
  constexpr int G = 16;
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t bh = idx / X, x = idx - bh * X;
  float* p = buf + bh * NC * X + x;
  float run = 0.f;
  for (int i0 = 0; i0 < NC; i0 += G) {
    float v[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int i = i0 + j;
      const int c = reverse ? NC - 1 - i : i;
      v[j] = i < NC ? p[(int64_t)c * X] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int i = i0 + j;
      const int c = reverse ? NC - 1 - i : i;
      if (i < NC) p[(int64_t)c * X] = run;
      run += v[j];
    }
  }
}

// out[bh][x] = sum over the NC chunk states
__global__ void chunk_sum_kernel(const float* buf, float* out, int NC, int64_t X, int64_t total) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t bh = idx / X, x = idx - bh * X;
  const float* p = buf + bh * NC * X + x;
  float s = 0.f;
  for (int c = 0; c < NC; ++c) s += p[c * X];
  out[idx] = s;
}

// dst[b][g][t][e] (strides) = sum over the query heads h of group g of src[b][h][t][e]
template <typename T>
__global__ void head_sum_kernel(const float* src, T* dst, int64_t sb, int64_t sh, int64_t sl, int H, int G, int L,
                                int Lp, int d, int64_t total) {
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(idx % d);
    const int64_t r1 = idx / d;
    const int t = (int)(r1 % L);
    const int64_t r2 = r1 / L;
    const int Hg = H / G;
    const int gidx = (int)(r2 % Hg);
    const int b = (int)(r2 / Hg);
    float s = 0.f;
    for (int i = 0; i < G; ++i) s += src[(((int64_t)b * H + gidx * G + i) * Lp + t) * d + e];
    st_t(dst + b * sb + gidx * sh + t * sl + e, s);
  }
}

// dM = sum of the partials [B][H][NKC][r*d] over b and splits (and heads when shared)
__global__ void dm_sum_kernel(const float* part, float* dM, int B, int H, int NKC, int64_t rd, int per_head) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t n = per_head ? (int64_t)H * rd : rd;
  if (idx >= n) return;
  const int h0 = per_head ? (int)(idx / rd) : 0;
  const int64_t x = idx - (per_head ? h0 * rd : 0);
  const int hn = per_head ? h0 + 1 : H;
  float s = 0.f;
  for (int b = 0; b < B; ++b)
    for (int h = h0; h < hn; ++h)
      for (int c = 0; c < NKC; ++c) s += part[(((int64_t)b * H + h) * NKC + c) * rd + x];
  dM[idx] = s;
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx < n) p[idx] = 0.f;
}

inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  int C, NC, Lp, KC, NKC, D1, CS, NCS;
  size_t Uq, Uk, dUq, dUk, nq, nk, rsq, rsk, Pq, Pk, dPq, dPk, Vx, ND, Gd, Sx, Gx, St, Gt, Wc, A2, dQh, dKh, dVh,
      dMp;
  size_t total;
};

BwdLayout bwd_layout(const dark_prf_desc& d) {
  BwdLayout o;
  o.C = bwd_chunk(d);
  const int L = d.L > 0 ? d.L : 1;
  o.NC = (int)cdiv64(L, o.C);
  o.Lp = o.NC * o.C;
  // dM = s sum_t dU_t^T x_t is split over runs of KC tokens (a multiple of 64)
  // so that the partial products fill about kMTarget workgroups
  const int64_t mtiles = std::max<int64_t>(1, (int64_t)d.B * d.H * cdiv64(d.r, 64) * cdiv64(d.d_h, 64));
  const int64_t nkc = std::max<int64_t>(1, cdiv64(kMTarget, mtiles));
  o.KC = (int)std::max<int64_t>(64, cdiv64(cdiv64(L, nkc), 64) * 64);
  o.NKC = (int)cdiv64(L, o.KC);
  o.D1 = d.d_h + 1;
  // the state partials: per 64-token chunk when causal (the prefix needs them);
  // otherwise per run of CS tokens, sized so the partial products fill about
  // kSTarget workgroups, and summed
  if (d.causal) {
    o.CS = o.C;
  } else {
    const int64_t stiles = std::max<int64_t>(1, (int64_t)d.B * d.H * cdiv64(d.m, 64) * cdiv64(d.d_h + 1, 64));
    const int64_t ncs = std::max<int64_t>(1, cdiv64(kSTarget, stiles));
    o.CS = (int)std::max<int64_t>(64, cdiv64(cdiv64(o.Lp, ncs), 64) * 64);
  }
  o.NCS = (int)cdiv64(o.Lp, o.CS);
  const size_t BH = (size_t)d.B * d.H, Lp = o.Lp, m = d.m, r = d.r, dh = d.d_h, D1 = o.D1;
  size_t off = 0;
  auto take = [&](size_t floats) {
    const size_t at = off;
    off = al256(off + floats * sizeof(float));
    return at;
  };
  o.Uq = take(BH * Lp * r);
  o.Uk = take(BH * Lp * r);
  o.dUq = take(BH * Lp * r);
  o.dUk = take(BH * Lp * r);
  o.nq = take(BH * Lp);
  o.nk = take(BH * Lp);
  o.rsq = take(BH * Lp);
  o.rsk = take(BH * Lp);
  o.Pq = take(BH * Lp * m);
  o.Pk = take(BH * Lp * m);
  o.dPq = take(BH * Lp * m);
  o.dPk = take(BH * Lp * m);
  o.Vx = take(BH * Lp * D1);
  o.ND = take(BH * Lp * D1);
  o.Gd = take(BH * Lp * D1);
  o.Sx = take(BH * o.NCS * m * D1);
  o.Gx = take(BH * o.NCS * m * D1);
  o.St = take(d.causal ? 0 : BH * m * D1);
  o.Gt = take(d.causal ? 0 : BH * m * D1);
  o.Wc = take(d.causal ? BH * Lp * o.C : 0);
  o.A2 = take(d.causal ? BH * Lp * o.C : 0);
  o.dQh = take(BH * Lp * dh);
  o.dKh = take(BH * Lp * dh);
  o.dVh = take(BH * Lp * dh);
  o.dMp = take(BH * o.NKC * r * dh);
  o.total = off;
  return o;
}

GOp op(const void* p, int64_t sb, int64_t sh, int64_t sc, int64_t si, int64_t sk, int hg = 1) {
  GOp o;
  o.p = p;
  o.sb = sb;
  o.sh = sh;
  o.sc = sc;
  o.si = si;
  o.sk = sk;
  o.hg = hg;
  o.p2 = nullptr;
  return o;
}
GOut out(float* p, int64_t sb, int64_t sh, int64_t sc, int64_t si) {
  GOut o;
  o.p = p;
  o.sb = sb;
  o.sh = sh;
  o.sc = sc;
  o.si = si;
  return o;
}

struct Launcher {
  hipStream_t st;
  int H;
  bool hilo = false;   // bf16 inputs: products on the bf16 matrix cores (hi/lo parts)
  double flops = 0.0;
  dark_status status = DARK_OK;

  template <typename TA, typename TB, bool PROD = false, bool XC = false>
  void gemm(GOp A, GOp B, GOut C, int M, int N, int K, int batches, int NCB, float alpha = 1.f, int accumulate = 0,
            int epi = kEpiPlain, int Ktot = 0, int Arows = -1, const float* nrm = nullptr, int64_t nrm_sbh = 0,
            const uint8_t* mask = nullptr, int L = 0, float* rowsum = nullptr, int64_t rs_sbh = 0,
            int mask_b0 = 0) {
    if (status != DARK_OK || M <= 0 || N <= 0 || batches <= 0) return;
    GemmArgs a;
    a.A = A;
    a.B = B;
    a.C = C;
    a.M = M;
    a.N = N;
    a.K = K;
    a.Ktot = Ktot;
    a.Arows = Arows < 0 ? M : Arows;
    a.H = H;
    a.NCB = NCB;
    a.tiles_n = (N - (XC ? 1 : 0) + 63) / 64;
    a.tiles = ((M + 63) / 64) * a.tiles_n;
    a.rowsum = rowsum;
    a.rs_sbh = rs_sbh;
    if ((rowsum != nullptr && (!PROD || A.sk != 1 || NCB != 1)) ||
        (XC && (N < 2 || PROD || epi != kEpiPlain || (A.sk != 1 && A.si != 1)))) {
      status = DARK_ERR_UNSUPPORTED;
      return;
    }
    a.alpha = alpha;
    a.accumulate = accumulate;
    a.epi = epi;
    a.nrm = nrm;
    a.nrm_sbh = nrm_sbh;
    a.mask = mask;
    a.mask_b0 = mask_b0;
    a.L = L;
    const int64_t grid = (int64_t)batches * a.tiles;
    const int64_t amax = (int64_t)(a.Arows - 1) * A.si + (int64_t)(K - 1) * A.sk;
    const int64_t bmax = (int64_t)(K - 1) * B.si + (int64_t)(N - 1) * B.sk;
    if (grid > INT_MAX || amax > INT_MAX || bmax > INT_MAX) {
      status = DARK_ERR_UNSUPPORTED;
      return;
    }
    // multiply-adds of the products as posed (K summed over the splits)
    const int64_t kt = Ktot > 0 ? (int64_t)Ktot * (batches / NCB) : (int64_t)K * batches;
    flops += 2.0 * M * N * (double)kt;
    KernelTimer tm(kBwdGemm, st);
    // bf16 inputs: the plain products from hi/lo parts; the feature exponents
    // and the intra-chunk score gradients (whose sums cancel exactly where the
    // output does not depend on q and k) keep the fp32 products.  (One fp16
    // product for the feature exponents, as in the forward, measured no faster
    // here: this kernel is bound by staging its fp32 operands, not by the
    // products.)
    if (hilo && epi == kEpiPlain)
      hipLaunchKernelGGL((bgemm_kernel<TA, TB, PROD, XC, kHiLo>), dim3((unsigned)grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((bgemm_kernel<TA, TB, PROD, XC>), dim3((unsigned)grid), dim3(256), 0, st, a);
    if (hipGetLastError() != hipSuccess) status = DARK_ERR_HIP;
  }

  template <typename F, typename... Args>
  void aux(F kern, int64_t threads, int block, Args... args) {
    if (status != DARK_OK || threads <= 0) return;
    const int64_t grid = cdiv64(threads, block);
    if (grid > INT_MAX) {
      status = DARK_ERR_UNSUPPORTED;
      return;
    }
    KernelTimer tm(kBwdAux, st);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(block), 0, st, args...);
    if (hipGetLastError() != hipSuccess) status = DARK_ERR_HIP;
  }
};

template <typename T>
dark_status run_bwd(const dark_prf_desc& d, const BwdPtrs& p, char* ws, hipStream_t st, double* flops_out) {
  const BwdLayout o = bwd_layout(d);
  const int H = d.H, G = d.H / d.H_kv, L = d.L, Lp = o.Lp, NC = o.NC, C = o.C, D1 = o.D1;
  const int m = d.m, r = d.r, dh = d.d_h;
  const int64_t BH = (int64_t)d.B * H;
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  float *Uq = F(o.Uq), *Uk = F(o.Uk), *dUq = F(o.dUq), *dUk = F(o.dUk), *nq = F(o.nq), *nk = F(o.nk);
  float *rsq = F(o.rsq), *rsk = F(o.rsk), *Pq = F(o.Pq), *Pk = F(o.Pk), *dPq = F(o.dPq), *dPk = F(o.dPk);
  float *Vx = F(o.Vx), *ND = F(o.ND), *Gd = F(o.Gd), *Sx = F(o.Sx), *Gx = F(o.Gx), *St = F(o.St), *Gt = F(o.Gt);
  float *Wc = F(o.Wc), *A2 = F(o.A2), *dQh = F(o.dQh), *dKh = F(o.dKh), *dVh = F(o.dVh), *dMp = F(o.dMp);
  const float s = 1.0f / sqrtf(sqrtf((float)dh));
  const int64_t hM = d.m_per_head ? (int64_t)r * dh : 0;   // M_h offset per head
  const int64_t hO = d.omega_per_head ? (int64_t)m * r : 0;   // omega_h offset per head
  Launcher ln{st, H};
  ln.hilo = sizeof(T) == 2;   // bf16 inputs

  // per-(b, h) row-major fp32 buffers [BH][Lp][w]: operand and output strides
  auto rows = [&](const float* p, int w) { return op(p, (int64_t)H * Lp * w, (int64_t)Lp * w, (int64_t)C * w, w, 1); };
  auto rowsT = [&](const float* p, int w) { return op(p, (int64_t)H * Lp * w, (int64_t)Lp * w, (int64_t)C * w, 1, w); };
  auto orows = [&](float* p, int w) { return out(p, (int64_t)H * Lp * w, (int64_t)Lp * w, (int64_t)C * w, w); };
  // state partials [BH][NCS][m][D1], one per run of CS tokens (CS = C when causal)
  const int CS = o.CS, NCS = o.NCS;
  const int64_t X = (int64_t)m * D1;
  auto states = [&](const float* p) { return op(p, (int64_t)H * NCS * X, (int64_t)NCS * X, X, D1, 1); };
  auto statesT = [&](const float* p) { return op(p, (int64_t)H * NCS * X, (int64_t)NCS * X, X, 1, D1); };
  auto ostates = [&](float* p) { return out(p, (int64_t)H * NCS * X, (int64_t)NCS * X, X, D1); };
  auto run = [&](const float* p, int w) { return op(p, (int64_t)H * Lp * w, (int64_t)Lp * w, (int64_t)CS * w, w, 1); };
  auto runT = [&](const float* p, int w) { return op(p, (int64_t)H * Lp * w, (int64_t)Lp * w, (int64_t)CS * w, 1, w); };
  // one total state per (b, h) [BH][m][D1]
  auto tot = [&](const float* p) { return op(p, (int64_t)H * X, X, 0, D1, 1); };
  auto totT = [&](const float* p) { return op(p, (int64_t)H * X, X, 0, 1, D1); };
  // intra-chunk C x C blocks [BH][NC][C][C]
  auto blk = [&](const float* p) { return op(p, (int64_t)H * Lp * C, (int64_t)Lp * C, (int64_t)C * C, C, 1); };
  auto blkT = [&](const float* p) { return op(p, (int64_t)H * Lp * C, (int64_t)Lp * C, (int64_t)C * C, 1, C); };
  auto oblk = [&](float* p) { return out(p, (int64_t)H * Lp * C, (int64_t)Lp * C, (int64_t)C * C, C); };

  // 1. projections u = s M_h x (rows t >= L read as 0) and half norms
  const GOp Mt = op(p.M, 0, hM, 0, 1, dh);   // (k, j) = M_h[j][k]
  ln.gemm<T, float>(op(p.q, d.q_str[0], d.q_str[1], 0, d.q_str[2], 1), Mt, orows(Uq, r), Lp, r, dh, (int)BH, 1, s, 0,
                    kEpiPlain, 0, L);
  ln.gemm<T, float>(op(p.k, d.k_str[0], d.k_str[1], 0, d.k_str[2], 1, G), Mt, orows(Uk, r), Lp, r, dh, (int)BH, 1, s,
                    0, kEpiPlain, 0, L);
  // The query and key buffers of each kind are adjacent in the workspace (every
  // size is a multiple of 256 bytes), so one launch over 2 B batch rows covers
  // queries (rows b < B) and keys (rows B + b).
  const bool paired = Uk == Uq + BH * Lp * r && nk == nq + BH * Lp && Pk == Pq + BH * Lp * m &&
                      dPk == dPq + BH * Lp * m && dUk == dUq + BH * Lp * r && rsk == rsq + BH * Lp &&
                      dKh == dQh + BH * Lp * dh;
  if (!paired) return DARK_ERR_UNSUPPORTED;
  const int BH2 = (int)(2 * BH);
  ln.aux(halfnorm_kernel, 2 * BH * Lp * 64, 256, (const float*)Uq, nq, r, 2 * BH * Lp);
  // 2. features phi = exp(u . omega_j - |u|^2 / 2) / sqrt(m); keys masked, rows t >= L zero
  const GOp OmT = op(p.omega, 0, hO, 0, 1, r);   // (k, j) = omega_h[j][k]
  const float inv_sqrt_m = 1.0f / sqrtf((float)m);
  ln.gemm<float, float>(rows(Uq, r), OmT, orows(Pq, m), Lp, m, r, BH2, 1, inv_sqrt_m, 0, kEpiFeature, 0, -1, nq, Lp,
                        p.mask, L, nullptr, 0, p.mask ? d.B : 0);
  // 3. [V, 1] per query head
  ln.aux(vx_kernel<T>, BH * Lp * D1, 256, (const T*)p.v, d.v_str[0], d.v_str[1], d.v_str[2], Vx, H, G, L, Lp, dh,
         BH * Lp * D1);
  // products of width d_h + 1: the last column on the vector ALUs when d_h + 1
  // would otherwise start a 64-wide tile of its own
  auto gemm_d1 = [&](GOp A, GOp B, GOut Cc, int M, int K, int batches, int NCB, int accumulate, int Ktot) {
    if (dh % 64 == 0)
      ln.gemm<float, float, false, true>(A, B, Cc, M, D1, K, batches, NCB, 1.f, accumulate, kEpiPlain, Ktot);
    else
      ln.gemm<float, float>(A, B, Cc, M, D1, K, batches, NCB, 1.f, accumulate, kEpiPlain, Ktot);
  };
  // 4. key-side state partials Phi(K_c)^T [V, 1]_c
  gemm_d1(runT(Pk, m), run(Vx, D1), ostates(Sx), m, CS, (int)(BH * NCS), NCS, 0, Lp);
  const int NB = (int)(BH * NC);
  if (d.causal) {
    ln.aux(chunk_scan_kernel, BH * X, 256, Sx, NC, X, BH * X, 0);
    // 5. [N, D] = Phi(Q_c) Sx_c + tril(Phi(Q_c) Phi(K_c)^T) [V, 1]_c
    ln.gemm<float, float>(rows(Pq, m), rowsT(Pk, m), oblk(Wc), C, C, m, NB, NC, 1.f, 0, kEpiTril);
    gemm_d1(rows(Pq, m), states(Sx), orows(ND, D1), C, m, NB, NC, 0, 0);
    gemm_d1(blk(Wc), rows(Vx, D1), orows(ND, D1), C, C, NB, NC, 1, 0);
  } else {
    ln.aux(chunk_sum_kernel, BH * X, 256, (const float*)Sx, St, NCS, X, BH * X);
    gemm_d1(rows(Pq, m), tot(St), orows(ND, D1), Lp, m, (int)BH, 1, 0, 0);
  }
  // 6. Gd = [dO / D, -(dO . O) / D]
  ln.aux(gd_kernel<T>, BH * Lp * 64, 256, (const T*)p.dout, d.o_str[0], d.o_str[1], d.o_str[2], (const float*)ND, Gd,
         H, L, Lp, dh, BH * Lp);
  // 7. dPhi(Q), the query-side state partials Phi(Q_c)^T Gd_c, dPhi(K) and dV
  gemm_d1(runT(Pq, m), run(Gd, D1), ostates(Gx), m, CS, (int)(BH * NCS), NCS, 0, Lp);
  if (d.causal) {
    ln.aux(chunk_scan_kernel, BH * X, 256, Gx, NC, X, BH * X, 1);
    ln.gemm<float, float>(rows(Gd, D1), rowsT(Vx, D1), oblk(A2), C, C, D1, NB, NC, 1.f, 0, kEpiTril);
    ln.gemm<float, float>(rows(Gd, D1), statesT(Sx), orows(dPq, m), C, m, D1, NB, NC);
    ln.gemm<float, float>(blk(A2), rows(Pk, m), orows(dPq, m), C, m, C, NB, NC, 1.f, 1);
    ln.gemm<float, float>(rows(Vx, D1), statesT(Gx), orows(dPk, m), C, m, D1, NB, NC);
    ln.gemm<float, float>(blkT(A2), rows(Pq, m), orows(dPk, m), C, m, C, NB, NC, 1.f, 1);
    ln.gemm<float, float>(rows(Pk, m), states(Gx), orows(dVh, dh), C, dh, m, NB, NC);
    ln.gemm<float, float>(blkT(Wc), rows(Gd, D1), orows(dVh, dh), C, dh, C, NB, NC, 1.f, 1);
  } else {
    ln.aux(chunk_sum_kernel, BH * X, 256, (const float*)Gx, Gt, NCS, X, BH * X);
    ln.gemm<float, float>(rows(Gd, D1), totT(St), orows(dPq, m), Lp, m, D1, (int)BH, 1);
    ln.gemm<float, float>(rows(Vx, D1), totT(Gt), orows(dPk, m), Lp, m, D1, (int)BH, 1);
    ln.gemm<float, float>(rows(Pk, m), tot(Gt), orows(dVh, dh), Lp, dh, m, (int)BH, 1);
  }
  // 8. through the feature map: dU = (dPhi * Phi) Omega - U * rowsum(dPhi * Phi)
  // (the A operand dPhi * Phi is formed in the loads, which also sum its rows)
  const GOp Om = op(p.omega, 0, hO, 0, r, 1);   // (k, j) = omega_h[k][j]
  GOp dEq = rows(dPq, m);   // and dPk, Pk from batch row B on
  dEq.p2 = Pq;
  ln.gemm<float, float, true>(dEq, Om, orows(dUq, r), Lp, r, m, BH2, 1, 1.f, 0, kEpiPlain, 0, -1, nullptr, 0, nullptr,
                              0, rsq, Lp);
  ln.aux(fixdu_kernel, 2 * BH * Lp * r, 256, dUq, (const float*)Uq, (const float*)rsq, r, 2 * BH * Lp * r);
  // 9. dX = s dU M_h, dM_h = s sum dU^T X
  const GOp Mh = op(p.M, 0, hM, 0, dh, 1);
  ln.gemm<float, float>(rows(dUq, r), Mh, orows(dQh, dh), Lp, dh, r, BH2, 1, s);
  const int KC = o.KC, NKC = o.NKC;
  const int64_t RD = (int64_t)r * dh;
  const GOut oMp = out(dMp, (int64_t)H * NKC * RD, (int64_t)NKC * RD, RD, dh);
  const GOp dUqT = op(dUq, (int64_t)H * Lp * r, (int64_t)Lp * r, (int64_t)KC * r, 1, r);
  const GOp dUkT = op(dUk, (int64_t)H * Lp * r, (int64_t)Lp * r, (int64_t)KC * r, 1, r);
  ln.gemm<float, T>(dUqT, op(p.q, d.q_str[0], d.q_str[1], KC * d.q_str[2], d.q_str[2], 1), oMp, r, dh, KC,
                    (int)(BH * NKC), NKC, s, 0, kEpiPlain, L);
  ln.gemm<float, T>(dUkT, op(p.k, d.k_str[0], d.k_str[1], KC * d.k_str[2], d.k_str[2], 1, G), oMp, r, dh, KC,
                    (int)(BH * NKC), NKC, s, 1, kEpiPlain, L);
  // 10. outputs: dq per head, dk and dv summed over the heads of each group, dM
  ln.aux(head_sum_kernel<T>, (int64_t)d.B * H * L * dh, 256, (const float*)dQh, (T*)p.dq, d.q_str[0], d.q_str[1],
         d.q_str[2], H, 1, L, Lp, dh, (int64_t)d.B * H * L * dh);
  ln.aux(head_sum_kernel<T>, (int64_t)d.B * d.H_kv * L * dh, 256, (const float*)dKh, (T*)p.dk, d.k_str[0],
         d.k_str[1], d.k_str[2], H, G, L, Lp, dh, (int64_t)d.B * d.H_kv * L * dh);
  ln.aux(head_sum_kernel<T>, (int64_t)d.B * d.H_kv * L * dh, 256, (const float*)dVh, (T*)p.dv, d.v_str[0],
         d.v_str[1], d.v_str[2], H, G, L, Lp, dh, (int64_t)d.B * d.H_kv * L * dh);
  const int64_t nM = (d.m_per_head ? H : 1) * RD;
  ln.aux(dm_sum_kernel, nM, 256, (const float*)dMp, p.dM, d.B, H, NKC, RD, d.m_per_head);
  if (flops_out) *flops_out = ln.flops;
  return ln.status;
}

}  // namespace

size_t bwd_ws_bytes(const dark_prf_desc& d) { return bwd_layout(d).total; }

dark_status launch_bwd(const dark_prf_desc& d, const BwdPtrs& p, void* ws, void* stream, double* flops) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (d.L == 0 || d.B == 0) {   // no tokens: every gradient is empty except dM, which is 0
    const int64_t nM = (d.m_per_head ? d.H : 1) * (int64_t)d.r * d.d_h;
    if (flops) *flops = 0.0;
    if (nM > 0) hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)cdiv64(nM, 256)), dim3(256), 0, st, p.dM, nM);
    return hipGetLastError() == hipSuccess ? DARK_OK : DARK_ERR_HIP;
  }
  char* w = static_cast<char*>(ws);
  return d.dtype == DARK_BF16 ? run_bwd<uint16_t>(d, p, w, st, flops) : run_bwd<float>(d, p, w, st, flops);
}

}  // namespace dk
