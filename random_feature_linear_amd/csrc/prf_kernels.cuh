// HIP kernels (gfx950, wave64) of DARKFormer positive-random-feature attention.
//
// Method (package README "Data-Aware Random Feature Kernels for Transformers
// (DARKformer)", section "Kernel"): with u = d_h^(-1/4) M x,
//   phi(x)_j = exp(omega_j . u - |u|^2 / 2) / sqrt(m)          (feature-map equation)
//   out = Phi(Q) (Phi(K)^T V) / Phi(Q) (Phi(K)^T 1)               (attention equation)
// and the causal form of section "Self-attention" (key j visible to query t iff
// j <= t and the key is valid).
//
// Matrix-core layout.  Every product is a 32x32x16 MFMA (bf16 operands, fp32
// accumulate; the fp32 path runs the same code with eight 32x32x2 fp32 MFMAs
// per step).  On gfx950 this shape sustains about twice the rate of the
// 16x16x32 one.  For lane l write c = l % 32 and g = l / 32.  An operand
// fragment holds 8 values per lane: the A operand holds row c and the B operand
// column c, both at K-slots 8g .. 8g+7.  The accumulator (16 floats) holds
// column c at rows R(i, g) = 8 (i / 4) + 4g + i % 4, i = 0..15.  A contraction
// does not care in which order it visits its K index, so registers 8k .. 8k+7
// of an accumulator are directly the K=16 operand fragment k of the next
// product: its slot e carries index 16k + 8 (e / 4) + 4g + e % 4.  Operands
// that come from memory (M, omega, the state, V) are laid out or read in that
// same order.
//
// exp is evaluated as exp2: omega is pre-scaled by log2(e) and the accumulator
// of the exponent product starts at -(log2(e) |u|^2 / 2 + log2(m) / 2), so the
// shift and the 1/sqrt(m) factor cost nothing.  A masked key, and a padding
// feature past m, starts at -inf and gives exactly 0.
//
// Precision of the bf16 path.  The exponent omega_j . u reaches magnitudes of
// ten and more, and a weight error of e per key shows up as a relative output
// error of about e (outputs are averages of zero-mean values), so the operands
// of the exponent cannot be plain bf16.  M', u and omega' are each carried as a
// pair of bf16 values hi + lo (about 16 significant bits): u = M'_hi x + M'_lo x
// and E = u_hi omega'_hi + u_lo omega'_hi + u_hi omega'_lo.
//
// The ones column of [V, 1] rides through the same MFMA as V (column d_h of
// the combined operand), so numerator and denominator see identical rounded
// feature values and the vector ALU is left to the exp.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "common.h"

namespace dk {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;             // waves per workgroup in the attention kernels
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32 * kWaves;    // tokens per key-side tile (one 32-token block per wave)

template <typename T> struct FragOf;
template <> struct FragOf<bf16> { typedef bf16x8 type; };
template <> struct FragOf<float> { typedef f32x8 type; };
template <typename T> constexpr int kParts = sizeof(T) == 2 ? 2 : 1;   // hi (+ lo) parts

__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}
__device__ __forceinline__ f32x16 splat16(float x) {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = x;
  return z;
}
// row of accumulator register i in lane group g
__device__ __forceinline__ constexpr int crow(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// ---- fragments: construction, loads, stores ---------------------------------
__device__ __forceinline__ void make_frag(bf16x8& f, const float* v) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)v[i];
}
__device__ __forceinline__ void make_frag(f32x8& f, const float* v) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = v[i];
}
template <typename F> __device__ __forceinline__ F zero_frag() {
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  F f;
  make_frag(f, v);
  return f;
}
// registers 8k .. 8k+7 of an accumulator as an operand fragment
template <typename F> __device__ __forceinline__ F acc_frag(const f32x16& a, int k) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = a[8 * k + e];
  F f;
  make_frag(f, v);
  return f;
}
__device__ __forceinline__ float bf16_hi(float x) { return (float)(bf16)x; }
// hi and lo parts of registers 8k .. 8k+7 (bf16); the fp32 path has one part
template <typename T>
__device__ __forceinline__ void acc_frag_split(const f32x16& a, int k, typename FragOf<T>::type& hi,
                                               typename FragOf<T>::type& lo) {
  float vh[8], vl[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = a[8 * k + e];
    vh[e] = kParts<T> == 2 ? bf16_hi(x) : x;
    vl[e] = x - vh[e];
  }
  make_frag(hi, vh);
  make_frag(lo, vl);
}

__device__ __forceinline__ bf16x8 ld8(const bf16* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ f32x8 ld8(const float* p) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  f32x8 f = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return f;
}
__device__ __forceinline__ void st8(bf16* p, const bf16x8& f) {
  *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, f);
}
__device__ __forceinline__ void st8(float* p, const f32x8& f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}
// elements p0[0..3] and p1[0..3] as one fragment
__device__ __forceinline__ bf16x8 ld4x2(const bf16* p0, const bf16* p1) {
  uint2 a = *reinterpret_cast<const uint2*>(p0);
  uint2 b = *reinterpret_cast<const uint2*>(p1);
  uint4 u = make_uint4(a.x, a.y, b.x, b.y);
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ f32x8 ld4x2(const float* p0, const float* p1) {
  float4 a = *reinterpret_cast<const float4*>(p0);
  float4 b = *reinterpret_cast<const float4*>(p1);
  f32x8 f = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return f;
}
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ void store_out(bf16* p, float x) { *p = (bf16)x; }
__device__ __forceinline__ void store_out(float* p, float x) { *p = x; }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- the feature map of one 32-token block -----------------------------------
// Token row t as the B-operand fragments X^T of the projection (K-steps of 16
// over d_h); rows at or past the end are zero.
template <typename T, int DH>
__device__ __forceinline__ void load_rows(typename FragOf<T>::type (&xf)[DH / 16], const T* row, bool ok,
                                          int g) {
  typedef typename FragOf<T>::type F;
#pragma unroll
  for (int kd = 0; kd < DH / 16; ++kd) xf[kd] = ok ? ld8(row + kd * 16 + 8 * g) : zero_frag<F>();
}

// u^T = M' x^T for a 32-token block (rank index in rows, token c in the lane),
// returned as hi / lo operand fragments over the rank index (K-steps of 16),
// plus the exp2-domain shift log2(e) |u|^2 / 2 + log2(m) / 2 of token c.
template <typename T, int DH, int R16>
__device__ __forceinline__ float project_block(typename FragOf<T>::type (&uhi)[R16],
                                               typename FragOf<T>::type (&ulo)[R16],
                                               const typename FragOf<T>::type (&xf)[DH / 16],
                                               const T* mfrag, int lane, float half_log2m) {
  constexpr int KD = DH / 16;
  constexpr int R32 = (R16 + 1) / 2;
  constexpr int NM = kParts<T>;
  float ss = 0.f;
#pragma unroll
  for (int rb = 0; rb < R32; ++rb) {
    f32x16 acc = zero16();
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
#pragma unroll
      for (int part = 0; part < NM; ++part)
        acc = mma(ld8(mfrag + (((rb * KD + kd) * NM + part) * 64 + lane) * 8), xf[kd], acc);
#pragma unroll
    for (int i = 0; i < 16; ++i) ss += acc[i] * acc[i];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (2 * rb + h < R16) acc_frag_split<T>(acc, h, uhi[2 * rb + h], ulo[2 * rb + h]);
  }
  ss += __shfl_xor(ss, 32);
  return 0.5f * kLog2e * ss + half_log2m;
}

// e += u . omega' over the rank index: u_hi omega'_hi + u_lo omega'_hi +
// u_hi omega'_lo (bf16), or one fp32 product.  U_IS_A: the u fragments are the
// A operand (result rows = tokens, columns = features); otherwise omega' is
// (result rows = features, columns = tokens).
template <typename T, int R16, bool U_IS_A>
__device__ __forceinline__ f32x16 exponent(const typename FragOf<T>::type* uhi,
                                           const typename FragOf<T>::type* ulo,
                                           const typename FragOf<T>::type* ohi,
                                           const typename FragOf<T>::type* olo, f32x16 e) {
#pragma unroll
  for (int k = 0; k < R16; ++k) {
    if constexpr (U_IS_A) {
      e = mma(uhi[k], ohi[k], e);
      if constexpr (kParts<T> == 2) {
        e = mma(ulo[k], ohi[k], e);
        e = mma(uhi[k], olo[k], e);
      }
    } else {
      e = mma(ohi[k], uhi[k], e);
      if constexpr (kParts<T> == 2) {
        e = mma(ohi[k], ulo[k], e);
        e = mma(olo[k], uhi[k], e);
      }
    }
  }
  return e;
}

// ---------------------------------------------------------------------------
// Preparation: M' = d_h^(-1/4) M and omega' = log2(e) omega in fragment order.
//   mfrag[hm][rb][kd][part][lane][8]: row 32 rb + c of M', columns 16 kd + 8g + e
//   ofrag[fb][k][part][lane][8]: row 32 fb + c of omega', rank index
//                                16k + 8 (e / 4) + 4g + e % 4
// part 0 is the bf16-rounded value, part 1 the rounded remainder (bf16 path).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void prep_kernel(const float* __restrict__ M, const float* __restrict__ omega,
                            T* __restrict__ mfrag, T* __restrict__ ofrag, int HM, int r, int d_h, int m,
                            int R16, int FB, float s) {
  constexpr int NM = kParts<T>;
  const int R32 = (R16 + 1) / 2;
  const int KD = d_h / 16;
  const long nM = (long)HM * R32 * KD * NM * 64;
  const long nO = (long)FB * R16 * NM * 64;
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < nM + nO;
       idx += (long)gridDim.x * blockDim.x) {
    float v[8];
    const bool m_side = idx < nM;
    const long j = m_side ? idx : idx - nM;
    const int lane = (int)(j & 63);
    const long f = j >> 6;
    const int part = (int)(f % NM);
    const int c = lane & 31, g = lane >> 5;
    if (m_side) {
      const int kd = (int)((f / NM) % KD);
      const int rb = (int)((f / ((long)NM * KD)) % R32);
      const int hm = (int)(f / ((long)NM * KD * R32));
      const int row = rb * 32 + c;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = kd * 16 + 8 * g + e;
        const float x = (row < r) ? s * M[((long)hm * r + row) * d_h + col] : 0.f;
        const float hi = NM == 2 ? bf16_hi(x) : x;
        v[e] = part == 0 ? hi : x - hi;
      }
    } else {
      const int k = (int)((f / NM) % R16);
      const int fb = (int)(f / ((long)NM * R16));
      const int row = fb * 32 + c;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int a = 16 * k + 8 * (e >> 2) + 4 * g + (e & 3);
        const float x = (row < m && a < r) ? kLog2e * omega[(long)row * r + a] : 0.f;
        const float hi = NM == 2 ? bf16_hi(x) : x;
        v[e] = part == 0 ? hi : x - hi;
      }
    }
    typename FragOf<T>::type fr;
    make_frag(fr, v);
    st8((m_side ? mfrag : ofrag) + j * 8, fr);
  }
}

// Stage rows t0 .. t0 + TT - 1 of V into LDS transposed, s_vt[d][t] (rows past
// t_end are zero).
template <typename T, int DH, int TT, int VST>
__device__ __forceinline__ void stage_vt(T* s_vt, const T* vb, int64_t vstride, int t0, int t_end, int tid) {
  typedef typename FragOf<T>::type F;
  for (int e = tid; e < TT * (DH / 8); e += kThreads) {
    const int tl = e % TT, d8 = (e / TT) * 8;   // consecutive lanes: consecutive tokens
    const int t = t0 + tl;
    const F x = (t < t_end) ? ld8(vb + (long)t * vstride + d8) : zero_frag<F>();
#pragma unroll
    for (int i = 0; i < 8; ++i) s_vt[(d8 + i) * VST + tl] = x[i];
  }
}

// The same staging in two halves: global loads into registers (issued a tile
// ahead of their use) and the transposed LDS stores.
template <int DH, int TT> constexpr int vloads_per_thread() { return (TT * (DH / 8) + kThreads - 1) / kThreads; }
template <typename T, int DH, int TT>
__device__ __forceinline__ void load_v(typename FragOf<T>::type* vr, const T* vb, int64_t vstride, int t0, int t_end,
                                       int tid) {
  typedef typename FragOf<T>::type F;
#pragma unroll
  for (int p = 0; p < vloads_per_thread<DH, TT>(); ++p) {
    const int e = tid + p * kThreads;
    const int tl = e % TT, d8 = (e / TT) * 8;   // consecutive lanes: consecutive tokens
    const int t = t0 + tl;
    vr[p] = (e < TT * (DH / 8) && t < t_end) ? ld8(vb + (long)t * vstride + d8) : zero_frag<F>();
  }
}
template <typename T, int DH, int TT, int VST>
__device__ __forceinline__ void store_vt(T* s_vt, const typename FragOf<T>::type* vr, int tid) {
#pragma unroll
  for (int p = 0; p < vloads_per_thread<DH, TT>(); ++p) {
    const int e = tid + p * kThreads;
    if (e >= TT * (DH / 8)) break;
    const int tl = e % TT, d8 = (e / TT) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) s_vt[(d8 + i) * VST + tl] = vr[p][i];
  }
}

// [V, 1] operand fragment: column d = 32 db + c (d < d_h: V, d = d_h: ones,
// past that: zero), tokens tb0 + 16k + 8 (e / 4) + 4g + e % 4
template <typename T, int DH, int VST>
__device__ __forceinline__ typename FragOf<T>::type v_frag(const T* s_vt, int db, int tb0, int k, int c, int g) {
  typedef typename FragOf<T>::type F;
  const int d = db * 32 + c;
  if (d >= DH) {
    const float o = d == DH ? 1.0f : 0.0f;
    float v[8] = {o, o, o, o, o, o, o, o};
    F f;
    make_frag(f, v);
    return f;
  }
  const T* base = s_vt + d * VST + tb0 + 16 * k + 4 * g;
  return ld4x2(base, base + 8);
}
// 32-column blocks of [V, 1]
template <int DH> constexpr int vblocks() { return (DH + 1 + 31) / 32; }

// ---------------------------------------------------------------------------
// Key side.  Per unit (a chunk when causal, an L-split otherwise) and feature
// slice:  S[j][d] = sum_t phi(k_t)_j v_t[d]  and  z[j] = sum_t phi(k_t)_j,
// written as bf16 operand fragments of the query side
//   sdelta[bh][unit][db][fk][lane][8]: column d = 32 db + c of [S, z] (column
//                                      d_h is z), feature 16 fk + 8 (e / 4) + 4g + e % 4.
// Workgroup: 4 waves; a tile is 128 tokens; wave w projects token block w and
// publishes its rank-index fragments and shifts in LDS; then every wave maps
// its own FBW x 32 features over the whole tile.
// ---------------------------------------------------------------------------
template <typename T, int DH, int R16, int FBW, bool PAD>
__global__ __launch_bounds__(kThreads) void kstate_kernel(FwdArgs a, Plan pl, const T* __restrict__ mfrag,
                                                           const T* __restrict__ ofrag, T* __restrict__ sdelta) {
  typedef typename FragOf<T>::type F;
  constexpr int KD = DH / 16;
  constexpr int NM = kParts<T>;
  constexpr int DB = vblocks<DH>();
  constexpr int TT = kTile;
  constexpr int VST = TT + 4;   // 4 x odd: 8-byte rows of V^T fall in distinct LDS banks

  constexpr int MFR = ((R16 + 1) / 2) * KD * NM;   // fragments of M' (one head)
  constexpr int VPT = vloads_per_thread<DH, TT>();
  __shared__ __attribute__((aligned(16))) T s_u[kWaves][NM][R16][64 * 8];
  __shared__ __attribute__((aligned(16))) float s_init[TT];
  __shared__ __attribute__((aligned(16))) T s_vt[DH * VST];
  __shared__ __attribute__((aligned(16))) T s_m[MFR * 64 * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int fslice = blockIdx.x % pl.NF;
  const int unit = (blockIdx.x / pl.NF) % pl.NU;
  const int bh = blockIdx.x / (pl.NF * pl.NU);
  const int b = bh / a.H, h = bh % a.H;
  const int hk = (h * a.H_kv) / a.H;
  const T* kbase = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
  const T* vbase = reinterpret_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
  const uint8_t* mrow = a.mask ? a.mask + (long)b * a.L : nullptr;
  const T* mf = mfrag + (long)(a.m_per_head ? h : 0) * ((R16 + 1) / 2) * KD * NM * 64 * 8;
  const float half_log2m = 0.5f * log2f((float)a.m);
  const int t_begin = unit * pl.span1;
  const int t_end = min(a.L, t_begin + pl.span1);
  const int fb0 = (fslice * kWaves + w) * FBW;     // first 32-feature block of this wave

  f32x16 acc[FBW][DB];
#pragma unroll
  for (int f = 0; f < FBW; ++f)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[f][db] = zero16();
  // omega' fragments of this wave's features stay in registers when they are few
  constexpr bool kHoist = FBW * R16 * NM <= 8;
  F ohr[kHoist ? FBW : 1][R16], olr[kHoist ? FBW : 1][R16];
  if constexpr (kHoist) {
#pragma unroll
    for (int f = 0; f < FBW; ++f) {
      const int fb = min(fb0 + f, pl.FB - 1);
#pragma unroll
      for (int k = 0; k < R16; ++k) {
        ohr[f][k] = ld8(ofrag + (((long)(fb * R16 + k) * NM) * 64 + lane) * 8);
        olr[f][k] = ld8(ofrag + (((long)(fb * R16 + k) * NM + NM - 1) * 64 + lane) * 8);
      }
    }
  }

  // M' of this head in LDS: every token block of every tile reads it
  for (int i = tid; i < MFR * 64; i += kThreads) st8(s_m + i * 8, ld8(mf + (long)i * 8));
  // K rows of block w and the V rows of a tile are loaded one tile ahead of their use
  F xpre[KD], vpre[VPT];
  auto prefetch = [&](int tt) {
    const int t = tt + 32 * w + c;
    load_rows<T, DH>(xpre, kbase + (long)t * a.ks[2], t < t_end, g);
    load_v<T, DH, TT>(vpre, vbase, a.vs[2], tt, t_end, tid);
  };
  prefetch(t_begin);
  __syncthreads();

  for (int t0 = t_begin; t0 < t_end; t0 += TT) {
    {  // projection of token block w
      const int t = t0 + 32 * w + c;
      const bool ok = t < t_end;
      F uhi[R16], ulo[R16];
      const float shift = project_block<T, DH, R16>(uhi, ulo, xpre, s_m, lane, half_log2m);
#pragma unroll
      for (int k = 0; k < R16; ++k) {
        st8(&s_u[w][0][k][lane * 8], uhi[k]);
        if constexpr (NM == 2) st8(&s_u[w][NM - 1][k][lane * 8], ulo[k]);
      }
      const bool valid = ok && (mrow == nullptr || mrow[t] != 0);
      if (g == 0) s_init[32 * w + c] = valid ? -shift : -INFINITY;
    }
    store_vt<T, DH, TT, VST>(s_vt, vpre, tid);
    __syncthreads();
    if (t0 + TT < t_end) prefetch(t0 + TT);

#pragma unroll
    for (int tb = 0; tb < kWaves; ++tb) {
      f32x16 ini;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {   // rows 8 jj + 4g .. 8 jj + 4g + 3 are contiguous
        const float4 x = *reinterpret_cast<const float4*>(&s_init[32 * tb + 8 * jj + 4 * g]);
        ini[4 * jj] = x.x;
        ini[4 * jj + 1] = x.y;
        ini[4 * jj + 2] = x.z;
        ini[4 * jj + 3] = x.w;
      }
      F uhi[R16], ulo[R16];
#pragma unroll
      for (int k = 0; k < R16; ++k) {
        uhi[k] = ld8(&s_u[tb][0][k][lane * 8]);
        ulo[k] = ld8(&s_u[tb][NM - 1][k][lane * 8]);
      }
      F vf[DB][2];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int k = 0; k < 2; ++k) vf[db][k] = v_frag<T, DH, VST>(s_vt, db, 32 * tb, k, c, g);
#pragma unroll
      for (int f = 0; f < FBW; ++f) {
        // a block past the last one (last slice only) runs on clamped operands
        // and is never stored: no branch in the loop
        const int fb = fb0 + f;
        const int fbc = min(fb, pl.FB - 1);
        F ohi[R16], olo[R16];
#pragma unroll
        for (int k = 0; k < R16; ++k) {
          if constexpr (kHoist) {
            ohi[k] = ohr[f][k];
            olo[k] = olr[f][k];
          } else {
            ohi[k] = ld8(ofrag + (((long)(fbc * R16 + k) * NM) * 64 + lane) * 8);
            olo[k] = ld8(ofrag + (((long)(fbc * R16 + k) * NM + NM - 1) * 64 + lane) * 8);
          }
        }
        f32x16 e = ini;
        if constexpr (PAD)   // m is not a multiple of 32: features past m give 0
          if (fb * 32 + c >= a.m) e = splat16(-INFINITY);
        e = exponent<T, R16, true>(uhi, ulo, ohi, olo, e);
#pragma unroll
        for (int i = 0; i < 16; ++i) e[i] = fast_exp2(e[i]);
        const F p0 = acc_frag<F>(e, 0), p1 = acc_frag<F>(e, 1);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          acc[f][db] = mma(p0, vf[db][0], acc[f][db]);
          acc[f][db] = mma(p1, vf[db][1], acc[f][db]);
        }
      }
    }
    __syncthreads();
  }

  // ---- write this wave's part of the unit state ----
  const long FK = 2L * pl.FB;     // 16-feature fragments per d-block
  T* sd = sdelta + ((long)bh * pl.NU + unit) * DB * FK * 64 * 8;
#pragma unroll
  for (int f = 0; f < FBW; ++f) {
    const int fb = fb0 + f;
    if (fb >= pl.FB) continue;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int k = 0; k < 2; ++k) st8(sd + ((db * FK + 2 * fb + k) * 64 + lane) * 8, acc_frag<F>(acc[f][db], k));
  }
}

// ---------------------------------------------------------------------------
// Key side for large ranks (the u fragments of a whole tile do not fit in LDS):
// the same result as kstate_kernel, one 32-token block at a time.  The four
// waves split the projection of the block by 32-row slices of M' and meet in
// LDS (fragments plus partial squared norms); V is staged per block.
// ---------------------------------------------------------------------------
template <typename T, int DH, int R16, int FBW, bool PAD>
__global__ __launch_bounds__(kThreads) void kstate_seq_kernel(FwdArgs a, Plan pl, const T* __restrict__ mfrag,
                                                               const T* __restrict__ ofrag,
                                                               T* __restrict__ sdelta) {
  typedef typename FragOf<T>::type F;
  constexpr int KD = DH / 16;
  constexpr int NM = kParts<T>;
  constexpr int DB = vblocks<DH>();
  constexpr int R32 = (R16 + 1) / 2;
  constexpr int VST = 32 + 4;

  __shared__ __attribute__((aligned(16))) T s_u[NM][R16][64 * 8];
  __shared__ __attribute__((aligned(16))) float s_ss[kWaves][32];
  __shared__ __attribute__((aligned(16))) T s_vt[DH * VST];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int fslice = blockIdx.x % pl.NF;
  const int unit = (blockIdx.x / pl.NF) % pl.NU;
  const int bh = blockIdx.x / (pl.NF * pl.NU);
  const int b = bh / a.H, h = bh % a.H;
  const int hk = (h * a.H_kv) / a.H;
  const T* kbase = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
  const T* vbase = reinterpret_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
  const uint8_t* mrow = a.mask ? a.mask + (long)b * a.L : nullptr;
  const T* mf = mfrag + (long)(a.m_per_head ? h : 0) * R32 * KD * NM * 64 * 8;
  const float half_log2m = 0.5f * log2f((float)a.m);
  const int t_begin = unit * pl.span1;
  const int t_end = min(a.L, t_begin + pl.span1);
  const int fb0 = (fslice * kWaves + w) * FBW;

  f32x16 acc[FBW][DB];
#pragma unroll
  for (int f = 0; f < FBW; ++f)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[f][db] = zero16();

  for (int t0 = t_begin; t0 < t_end; t0 += 32) {
    {  // projection slices rb = w, w + 4, ... of this block
      const int t = t0 + c;
      const bool ok = t < t_end;
      F xf[KD];
      load_rows<T, DH>(xf, kbase + (long)t * a.ks[2], ok, g);
      float ss = 0.f;
      for (int rb = w; rb < R32; rb += kWaves) {
        f32x16 u = zero16();
#pragma unroll
        for (int kd = 0; kd < KD; ++kd)
#pragma unroll
          for (int part = 0; part < NM; ++part)
            u = mma(ld8(mf + (((rb * KD + kd) * NM + part) * 64 + lane) * 8), xf[kd], u);
#pragma unroll
        for (int i = 0; i < 16; ++i) ss += u[i] * u[i];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          if (2 * rb + hh < R16) {
            F hi, lo;
            acc_frag_split<T>(u, hh, hi, lo);
            st8(&s_u[0][2 * rb + hh][lane * 8], hi);
            if constexpr (NM == 2) st8(&s_u[NM - 1][2 * rb + hh][lane * 8], lo);
          }
      }
      ss += __shfl_xor(ss, 32);
      if (g == 0) s_ss[w][c] = ss;
    }
    stage_vt<T, DH, 32, VST>(s_vt, vbase, a.vs[2], t0, t_end, tid);
    __syncthreads();

    f32x16 ini;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = crow(i, g);
      const int t = t0 + row;
      const float ss = s_ss[0][row] + s_ss[1][row] + s_ss[2][row] + s_ss[3][row];
      const bool valid = t < t_end && (mrow == nullptr || mrow[t] != 0);
      ini[i] = valid ? -(0.5f * kLog2e * ss + half_log2m) : -INFINITY;
    }
    F uhi[R16], ulo[R16];
#pragma unroll
    for (int k = 0; k < R16; ++k) {
      uhi[k] = ld8(&s_u[0][k][lane * 8]);
      ulo[k] = ld8(&s_u[NM - 1][k][lane * 8]);
    }
#pragma unroll
    for (int f = 0; f < FBW; ++f) {
      const int fb = fb0 + f;
      const int fbc = min(fb, pl.FB - 1);   // past the last block: clamped, never stored
      F ohi[R16], olo[R16];
#pragma unroll
      for (int k = 0; k < R16; ++k) {
        ohi[k] = ld8(ofrag + (((long)(fbc * R16 + k) * NM) * 64 + lane) * 8);
        olo[k] = ld8(ofrag + (((long)(fbc * R16 + k) * NM + NM - 1) * 64 + lane) * 8);
      }
      f32x16 e = ini;
      if constexpr (PAD)
        if (fb * 32 + c >= a.m) e = splat16(-INFINITY);
      e = exponent<T, R16, true>(uhi, ulo, ohi, olo, e);
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = fast_exp2(e[i]);
      const F p0 = acc_frag<F>(e, 0), p1 = acc_frag<F>(e, 1);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        acc[f][db] = mma(p0, v_frag<T, DH, VST>(s_vt, db, 0, 0, c, g), acc[f][db]);
        acc[f][db] = mma(p1, v_frag<T, DH, VST>(s_vt, db, 0, 1, c, g), acc[f][db]);
      }
    }
    __syncthreads();
  }

  const long FK = 2L * pl.FB;
  T* sd = sdelta + ((long)bh * pl.NU + unit) * DB * FK * 64 * 8;
#pragma unroll
  for (int f = 0; f < FBW; ++f) {
    const int fb = fb0 + f;
    if (fb >= pl.FB) continue;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int k = 0; k < 2; ++k) st8(sd + ((db * FK + 2 * fb + k) * 64 + lane) * 8, acc_frag<F>(acc[f][db], k));
  }
}

// ---------------------------------------------------------------------------
// State combination.  Non-causal: the sum over the L-splits.  Causal: the
// exclusive prefix over chunks (the state before each chunk) and, if asked, the
// state after the last token as S[b][h][j][d], z[b][h][j] (fp32).  Sums run in
// fp32; the per-unit states the query side reads are written in the operand
// order of the key side's output.  One thread per fragment lane (8 elements).
// ---------------------------------------------------------------------------
template <typename T, int DH>
__global__ void scan_kernel(FwdArgs a, Plan pl, const T* __restrict__ sdelta, T* __restrict__ sfrag) {
  typedef typename FragOf<T>::type F;
  constexpr int DB = vblocks<DH>();
  const long FK = 2L * pl.FB;
  const long per_unit = DB * FK * 64;          // fragment lanes per unit
  const long nS = (long)pl.BH * per_unit;
  const int nout = a.causal ? pl.NU : 1;
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < nS; idx += (long)gridDim.x * blockDim.x) {
    const long bh = idx / per_unit;
    const long rem = idx % per_unit;
    const T* src = sdelta + (bh * pl.NU * per_unit + rem) * 8;
    T* dst = sfrag + (bh * nout * per_unit + rem) * 8;
    float run[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int u = 0;
    for (; u + 4 <= pl.NU; u += 4) {       // four loads in flight
      F x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = ld8(src + (long)(u + q) * per_unit * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (a.causal) {
          F o;
          make_frag(o, run);
          st8(dst + (long)(u + q) * per_unit * 8, o);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) run[e] += to_f32(x[q][e]);
      }
    }
    for (; u < pl.NU; ++u) {
      const F x = ld8(src + (long)u * per_unit * 8);
      if (a.causal) {
        F o;
        make_frag(o, run);
        st8(dst + (long)u * per_unit * 8, o);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) run[e] += to_f32(x[e]);
    }
    if (!a.causal) {
      F o;
      make_frag(o, run);
      st8(dst, o);
    } else if (a.S_out) {
      const int lane = (int)(rem & 63);
      const long frag = rem >> 6;
      const int fk = (int)(frag % FK), db = (int)(frag / FK);
      const int c = lane & 31, g = lane >> 5;
      const int d = db * 32 + c;
      if (d <= DH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 16 * fk + 8 * (e >> 2) + 4 * g + (e & 3);
          if (j >= a.m) continue;
          if (d < DH) a.S_out[(bh * a.m + j) * DH + d] = run[e];
          else a.z_out[bh * a.m + j] = run[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Query side.  Per (b, h) and tile of 128 NQB queries (a chunk when causal):
//   [N, D] = Phi(Q) [S, z] (+ tril(Phi(Q) Phi(K_chunk)^T) [V, 1] when causal),
//   out = N / D (0 if D == 0).
// Wave w owns query blocks w NQB .. w NQB + NQB - 1 of the tile; when causal,
// the keys at the same positions are mapped by the same wave and shared with
// the other waves through LDS, one 32-feature step at a time.
// ---------------------------------------------------------------------------
template <typename T, int DH, int R16, int NQB, bool CAUSAL, bool PAD>
__global__ __launch_bounds__(kThreads) void qout_kernel(FwdArgs a, Plan pl, const T* __restrict__ mfrag,
                                                         const T* __restrict__ ofrag, const T* __restrict__ sfrag) {
  typedef typename FragOf<T>::type F;
  constexpr int KD = DH / 16;
  constexpr int NM = kParts<T>;
  constexpr int DB = vblocks<DH>();
  constexpr int NB = kWaves * NQB;         // 32-token blocks per tile
  constexpr int TT = 32 * NB;              // tokens per tile
  constexpr int VST = TT + 4;
  constexpr int NOF = R16 * NM;            // omega' fragments per feature step
  constexpr int NSTEP = NOF + 2 * DB;      // plus state fragments
  constexpr int PERW = (NSTEP + kWaves - 1) / kWaves;
  constexpr int VT_ELEMS = CAUSAL ? DH * VST : 8;
  constexpr size_t kBase = (size_t)VT_ELEMS * sizeof(T);
  constexpr size_t kOpStep = (size_t)NSTEP * 64 * 8 * sizeof(T);
  constexpr size_t kKfStep = CAUSAL ? (size_t)NB * 2 * 64 * 8 * sizeof(T) : 0;
  // Operands staged in LDS when one step buffer fits beside the V^T tile (else
  // each wave reads them from L2 itself); double buffers (one barrier per
  // feature step) unless LDS is short.
  constexpr bool STAGE = kBase + kOpStep + kKfStep <= 160 * 1024;
  constexpr int OPB = !STAGE ? 0 : kBase + 2 * kOpStep + 2 * kKfStep <= 160 * 1024 ? 2 : 1;
  constexpr int KBUF = kBase + OPB * kOpStep + 2 * kKfStep <= 160 * 1024 ? 2 : 1;
  constexpr int KF_ELEMS = CAUSAL ? KBUF * NB * 2 * 64 * 8 : 8;

  __shared__ __attribute__((aligned(16))) T s_vt[VT_ELEMS];
  __shared__ __attribute__((aligned(16))) T s_kf[KF_ELEMS];
  __shared__ __attribute__((aligned(16))) T s_op[STAGE ? OPB * NSTEP * 64 * 8 : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int tile = blockIdx.x % pl.NT2;
  const int bh = blockIdx.x / pl.NT2;
  const int b = bh / a.H, h = bh % a.H;
  const int hk = (h * a.H_kv) / a.H;
  const T* qbase = reinterpret_cast<const T*>(a.q) + b * a.qs[0] + h * a.qs[1];
  const T* kbase = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
  const T* vbase = reinterpret_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
  T* obase = reinterpret_cast<T*>(a.out) + b * a.os[0] + h * a.os[1];
  const uint8_t* mrow = a.mask ? a.mask + (long)b * a.L : nullptr;
  const T* mf = mfrag + (long)(a.m_per_head ? h : 0) * ((R16 + 1) / 2) * KD * NM * 64 * 8;
  const float half_log2m = 0.5f * log2f((float)a.m);
  const int t0 = tile * TT;
  const long FK = 2L * pl.FB;
  const long unit_s = (long)bh * (CAUSAL ? pl.NU : 1) + (CAUSAL ? tile : 0);
  const T* sf = sfrag + unit_s * DB * FK * 64 * 8;

  // ---- projections of this wave's query (and key) blocks ----
  F uqh[NQB][R16], uql[NQB][R16];
  float shq[NQB];
  F ukh[CAUSAL ? NQB : 1][R16], ukl[CAUSAL ? NQB : 1][R16];
  float initk[CAUSAL ? NQB : 1];
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const int t = t0 + 32 * (w * NQB + j) + c;
    const bool ok = t < a.L;
    F xf[KD];
    load_rows<T, DH>(xf, qbase + (long)t * a.qs[2], ok, g);
    shq[j] = project_block<T, DH, R16>(uqh[j], uql[j], xf, mf, lane, half_log2m);
    if constexpr (CAUSAL) {
      load_rows<T, DH>(xf, kbase + (long)t * a.ks[2], ok, g);
      const float sh = project_block<T, DH, R16>(ukh[j], ukl[j], xf, mf, lane, half_log2m);
      const bool valid = ok && (mrow == nullptr || mrow[t] != 0);
      initk[j] = valid ? -sh : -INFINITY;
    }
  }
  if constexpr (CAUSAL) stage_vt<T, DH, TT, VST>(s_vt, vbase, a.vs[2], t0, a.L, tid);

  f32x16 acc[NQB][DB];
#pragma unroll
  for (int j = 0; j < NQB; ++j)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[j][db] = zero16();
  f32x16 at[CAUSAL ? NQB : 1][CAUSAL ? NB : 1];   // A^T[key block][query block of the wave]
  if constexpr (CAUSAL) {
#pragma unroll
    for (int j = 0; j < NQB; ++j)
#pragma unroll
      for (int kb2 = 0; kb2 < NB; ++kb2) at[j][kb2] = zero16();
  }

  // Operands of one 32-feature step (omega' hi/lo fragments, then the state
  // fragments) are the same for the four waves: each wave fetches a quarter of
  // them from L2 one step ahead, and all read them from LDS.
  auto gsrc = [&](int fb, int f) -> const T* {
    if (f < NOF) return ofrag + (((long)(fb * R16 + f / NM) * NM + f % NM) * 64 + lane) * 8;
    f -= NOF;
    return sf + (((f >> 1) * FK + 2 * fb + (f & 1)) * 64 + lane) * 8;
  };
  F pre[STAGE ? PERW : 1];
  auto load_step = [&](int fb) {
    if constexpr (STAGE) {
#pragma unroll
      for (int q = 0; q < PERW; ++q) {
        const int f = w + kWaves * q;
        if (f < NSTEP) pre[q] = ld8(gsrc(fb, f));
      }
    }
  };
  auto store_step = [&](int buf) {
    if constexpr (STAGE) {
#pragma unroll
      for (int q = 0; q < PERW; ++q) {
        const int f = w + kWaves * q;
        if (f < NSTEP) st8(s_op + ((buf * NSTEP + f) * 64 + lane) * 8, pre[q]);
      }
    }
  };
  auto op = [&](int fb, int buf, int f) {
    if constexpr (STAGE) return ld8(s_op + ((buf * NSTEP + f) * 64 + lane) * 8);
    else return ld8(gsrc(fb, f));
  };

  // one 32-feature step; the operands of the next step are fetched before it runs
  auto step = [&](int fb, int buf) {
    F ohi[R16], olo[R16];
#pragma unroll
    for (int k = 0; k < R16; ++k) {
      ohi[k] = op(fb, buf, k * NM);
      olo[k] = op(fb, buf, k * NM + NM - 1);
    }
    const bool partial = PAD && (fb + 1) * 32 > a.m;   // the last block may hold padding features
    F pq[NQB][2];
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      f32x16 e = splat16(-shq[j]);
      if (partial) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (fb * 32 + crow(i, g) >= a.m) e[i] = -INFINITY;
      }
      e = exponent<T, R16, false>(uqh[j], uql[j], ohi, olo, e);
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = fast_exp2(e[i]);
      pq[j][0] = acc_frag<F>(e, 0);
      pq[j][1] = acc_frag<F>(e, 1);
    }
    // inter-chunk (or whole-sequence) state
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const F sv = op(fb, buf, NOF + 2 * db + k);
#pragma unroll
        for (int j = 0; j < NQB; ++j) acc[j][db] = mma(pq[j][k], sv, acc[j][db]);
      }
    if constexpr (CAUSAL) {
      T* kbuf = s_kf + (KBUF == 2 ? (fb & 1) : 0) * NB * 2 * 64 * 8;
#pragma unroll
      for (int j = 0; j < NQB; ++j) {
        f32x16 e = splat16(initk[j]);
        if (partial) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (fb * 32 + crow(i, g) >= a.m) e[i] = -INFINITY;
        }
        e = exponent<T, R16, false>(ukh[j], ukl[j], ohi, olo, e);
#pragma unroll
        for (int i = 0; i < 16; ++i) e[i] = fast_exp2(e[i]);
#pragma unroll
        for (int k = 0; k < 2; ++k) st8(kbuf + (((w * NQB + j) * 2 + k) * 64 + lane) * 8, acc_frag<F>(e, k));
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NQB; ++j) {
        const int gq = w * NQB + j;
#pragma unroll
        for (int kb2 = 0; kb2 < NB; ++kb2)
          if (kb2 <= gq)
#pragma unroll
            for (int k = 0; k < 2; ++k)
              at[j][kb2] = mma(ld8(kbuf + ((kb2 * 2 + k) * 64 + lane) * 8), pq[j][k], at[j][kb2]);
      }
      if constexpr (KBUF == 1) __syncthreads();   // the buffer is rewritten by the next step
    }
  };
  load_step(0);
  store_step(0);
  __syncthreads();
  for (int fb = 0; fb < pl.FB; ++fb) {
    const int buf = OPB == 2 ? (fb & 1) : 0;
    if (fb + 1 < pl.FB) load_step(fb + 1);
    step(fb, buf);
    if constexpr (STAGE) {
      if (fb + 1 < pl.FB) {
        if constexpr (OPB == 1) __syncthreads();   // one buffer: everyone is done reading it
        store_step(OPB == 2 ? ((fb + 1) & 1) : 0);
      }
      __syncthreads();
    }
  }

  if constexpr (CAUSAL) {
    // causal mask inside the diagonal block: key R(i, g) is visible to query c iff R(i, g) <= c
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      const int gq = w * NQB + j;
#pragma unroll
      for (int kb2 = 0; kb2 < NB; ++kb2) {
        if (kb2 > gq) continue;
        if (kb2 == gq) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (crow(i, g) > c) at[j][kb2][i] = 0.f;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const F pf = acc_frag<F>(at[j][kb2], k);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[j][db] = mma(pf, v_frag<T, DH, VST>(s_vt, db, 32 * kb2, k, c, g), acc[j][db]);
        }
      }
    }
  }

  // ---- out = N / D; D is column d_h of [N, D], held by lane d_h % 32 of each half ----
  constexpr int DBLK = DH / 32, DCOL = DH % 32;
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const int blk = w * NQB + j;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float dd = __shfl(acc[j][DBLK][i], (lane & 32) | DCOL);
      const int t = t0 + 32 * blk + crow(i, g);
      const float inv = dd > 0.f ? __builtin_amdgcn_rcpf(dd) : 0.f;
      if (t < a.L) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 32 + c;
          if (d < DH) store_out(obase + (long)t * a.os[2] + d, acc[j][db][i] * inv);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host launch of one forward call for (T, DH, R16).
// ---------------------------------------------------------------------------
constexpr size_t kMaxLds = 160 * 1024;
// LDS of the tiled key-side kernel: u fragments of four blocks, shifts, the V^T tile
template <typename T, int DH, int R16> constexpr size_t kstate_tile_lds_bytes() {
  return (size_t)(kWaves * kParts<T> * R16 * 64 * 8 + DH * (kTile + 8) + ((R16 + 1) / 2) * (DH / 16) * kParts<T> * 64 * 8) *
             sizeof(T) +
         kTile * sizeof(float);
}
// Least LDS of the causal query-side kernel: the V^T tile and one key-feature
// buffer (the operand staging buffers are added only where they fit).
template <typename T, int DH, int R16, int NQB> constexpr size_t causal_lds_bytes() {
  return (size_t)(DH * (128 * NQB + 4) + 4 * NQB * 2 * 64 * 8) * sizeof(T);
}

template <typename T, int DH, int R16, int FBW, bool PAD>
dark_status launch_fwd_pad(const FwdArgs& a, const Plan& pl, void* ws, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(ws);
  T* mfrag = reinterpret_cast<T*>(base + pl.off_mfrag);
  T* ofrag = reinterpret_cast<T*>(base + pl.off_ofrag);
  T* sdelta = reinterpret_cast<T*>(base + pl.off_sdelta);
  T* sfrag = reinterpret_cast<T*>(base + pl.off_sfrag);
  constexpr int NM = kParts<T>;
  {
    const long n = (long)pl.HM * ((R16 + 1) / 2) * (DH / 16) * NM * 64 + (long)pl.FB * R16 * NM * 64;
    const int blocks = (int)((n + 255) / 256);
    KernelTimer tm(kPrep, stream);
    hipLaunchKernelGGL(prep_kernel<T>, dim3(blocks), dim3(256), 0, st, a.M, a.omega, mfrag, ofrag, pl.HM, a.r, DH,
                       a.m, R16, pl.FB, powf((float)DH, -0.25f));
  }
  {
    KernelTimer tm(kKState, stream);
    const dim3 grid1(pl.BH * pl.NU * pl.NF);
    if constexpr (kstate_tile_lds_bytes<T, DH, R16>() <= kMaxLds)
      hipLaunchKernelGGL((kstate_kernel<T, DH, R16, FBW, PAD>), grid1, dim3(kThreads), 0, st, a, pl, mfrag, ofrag,
                         sdelta);
    else
      hipLaunchKernelGGL((kstate_seq_kernel<T, DH, R16, FBW, PAD>), grid1, dim3(kThreads), 0, st, a, pl, mfrag,
                         ofrag, sdelta);
  }
  {
    const long n = (long)pl.BH * vblocks<DH>() * 2 * pl.FB * 64;
    const int blocks = (int)((n + 255) / 256);
    KernelTimer tm(kScan, stream);
    hipLaunchKernelGGL((scan_kernel<T, DH>), dim3(blocks), dim3(256), 0, st, a, pl, sdelta, sfrag);
  }
  const dim3 grid(pl.BH * pl.NT2);
  KernelTimer tm(kQOut, stream);
  if (a.causal) {
    if constexpr (causal_lds_bytes<T, DH, R16, 1>() <= kMaxLds) {
      if (pl.NQB != 1) return DARK_ERR_UNSUPPORTED;
      hipLaunchKernelGGL((qout_kernel<T, DH, R16, 1, true, PAD>), grid, dim3(kThreads), 0, st, a, pl, mfrag, ofrag,
                         sfrag);
    } else {
      return DARK_ERR_UNSUPPORTED;
    }
  } else {
    switch (pl.NQB) {
      case 1: hipLaunchKernelGGL((qout_kernel<T, DH, R16, 1, false, PAD>), grid, dim3(kThreads), 0, st, a, pl, mfrag, ofrag, sfrag); break;
      case 2:
        if constexpr (DH <= 128) {   // the planner takes two query blocks per wave only for d_h <= 64
          hipLaunchKernelGGL((qout_kernel<T, DH, R16, 2, false, PAD>), grid, dim3(kThreads), 0, st, a, pl, mfrag,
                             ofrag, sfrag);
          break;
        } else {
          return DARK_ERR_UNSUPPORTED;
        }
      default: return DARK_ERR_UNSUPPORTED;
    }
  }
  return hipGetLastError() == hipSuccess ? DARK_OK : DARK_ERR_HIP;
}

// Host launch of one forward call for (T, DH, R16); m that is not a multiple of
// 32 takes the variant that masks the padding features of the last block.
template <typename T, int DH, int R16, int FBW>
dark_status launch_fwd_impl(const FwdArgs& a, const Plan& pl, void* ws, void* stream) {
  return (a.m % 32 != 0) ? launch_fwd_pad<T, DH, R16, FBW, true>(a, pl, ws, stream)
                         : launch_fwd_pad<T, DH, R16, FBW, false>(a, pl, ws, stream);
}

}  // namespace dk
