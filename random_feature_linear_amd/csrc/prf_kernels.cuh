// HIP kernels (gfx950, wave64) of DARKFormer positive-random-feature attention.
//
// Method (package README "Data-Aware Random Feature Kernels for Transformers
// (DARKformer)", section "Kernel"): with u = d_h^(-1/4) M x,
//   phi(x)_j = exp(omega_j . u - |u|^2 / 2) / sqrt(m)          (feature-map equation)
//   out = Phi(Q) (Phi(K)^T [V, 1]) split into numerator / denominator
//                                                               (attention equation)
// and the causal form of section "Self-attention" (key j visible to query t iff
// j <= t and the key is valid).
//
// Matrix-core layout.  Every contraction is a 16x16x32 MFMA (bf16 operands,
// fp32 accumulate); the fp32 path runs the same code with eight 16x16x4 fp32
// MFMAs per step.  For lane l write c = l % 16 and g = l / 16.  An operand
// fragment holds 8 values per lane: the A operand holds row c and the B operand
// column c, both at K-slots 8g .. 8g+7; the accumulator holds rows 4g .. 4g+3 of
// column c.  Because a contraction does not care in which order its K index is
// visited, the accumulator of one product is fed to the next product directly,
// register for register: for two accumulators X0 (index 0..15) and X1 (index
// 16..31) of the same column, slot 8g + 4h + i of the fragment carries index
// 16h + 4g + i.  Operands that come from memory (M, omega, the state) are laid
// out by the host-side preparation in that same "fragment order", so a lane
// loads its 16 bytes contiguously.
//
// exp is evaluated as exp2: omega is pre-scaled by log2(e) and the accumulator
// of the exponent product starts at -(log2(e) |u|^2 / 2 + log2(m) / 2), so the
// shift and the 1/sqrt(m) factor cost nothing.  A masked key starts at -inf and
// its features are exactly 0.
//
// Precision of the bf16 path.  The exponent omega_j . u reaches magnitudes of
// ten and more, and a weight error of e per key shows up as a relative output
// error of about e (outputs are averages of zero-mean values), so the operands
// of the exponent cannot be plain bf16.  M' and u are each carried as a pair of
// bf16 values hi + lo (about 16 significant bits): u = M'_hi x + M'_lo x and
// E = u_hi . omega' + u_lo . omega'.  With rank r <= 16 the lo half of u rides
// in the padding slots of the 32-wide K-step at no cost.  Rounding omega' to
// bf16 perturbs each feature independently, which averages out in the
// normalised output only while many features share the weight of a pair; with
// anisotropic inputs a few features dominate each kernel estimate, so every
// exponent product also adds u_hi . omega'_lo (three bf16 products in all).
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.h"

namespace dk {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;             // waves per workgroup in the attention kernels
constexpr int kThreads = 64 * kWaves;

template <typename T> struct FragOf;
template <> struct FragOf<bf16> { typedef bf16x8 type; };
template <> struct FragOf<float> { typedef f32x8 type; };

// Fragment counts of the projection and of the feature exponent.
template <typename T, int R16> struct EShape {
  static constexpr bool split = sizeof(T) == 2;           // bf16: hi + lo pairs
  static constexpr int RK = (R16 + 1) / 2;                // 32-wide K-steps over the rank
  static constexpr bool packed = split && R16 == 1;       // lo half in the padding slots
  static constexpr int NM = split ? 2 : 1;                // parts of M'
  static constexpr int NU = !split ? RK : (packed ? 1 : 2 * RK);   // u fragments
  static constexpr int NO = !split ? RK : (packed ? 2 : 2 * RK);   // omega' fragments stored
};

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

// ---- fragment construction, loads and stores ---------------------------------
__device__ __forceinline__ void make_frag(bf16x8& f, const float* v) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)v[i];
}
__device__ __forceinline__ void make_frag(f32x8& f, const float* v) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = v[i];
}
// two accumulators (index 0..15 and 16..31) -> one fragment (slots 4h + i)
template <typename F>
__device__ __forceinline__ F frag_from_acc(const f32x4& a0, const f32x4& a1) {
  float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  F f;
  make_frag(f, v);
  return f;
}
template <typename F> __device__ __forceinline__ F zero_frag() {
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  F f;
  make_frag(f, v);
  return f;
}
// the "ones" operand of [V, 1]: row (or column) d_h of the last 16-block
template <typename F> __device__ __forceinline__ F ones_frag(int c) {
  float o = (c == 0) ? 1.0f : 0.0f;
  float v[8] = {o, o, o, o, o, o, o, o};
  F f;
  make_frag(f, v);
  return f;
}

// 8 contiguous elements (16-byte aligned for bf16, 16-byte aligned halves for fp32)
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
// two groups of 4 contiguous elements -> one fragment
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

// Row t of a [.., L, d_h] tensor as the B-operand fragments X^T of the
// projection (K-steps of 32 over d_h).  Rows at or past L, and slots past d_h,
// are zero.
template <typename T, int DH>
__device__ __forceinline__ void load_rows(typename FragOf<T>::type (&xf)[(DH + 31) / 32],
                                          const T* row, bool ok, int g) {
  typedef typename FragOf<T>::type F;
#pragma unroll
  for (int kd = 0; kd < (DH + 31) / 32; ++kd) {
    const int col = kd * 32 + 8 * g;
    if (ok && col < DH) xf[kd] = ld8(row + col);
    else xf[kd] = zero_frag<F>();
  }
}

// u^T = M' x^T for one 16-token block: ut[rb] holds rows 16 rb + 4g + i of u^T
// (rank index) at token c.  Returns the exp2-domain shift
// log2(e) |u|^2 / 2 + log2(m) / 2 of token c (identical in the 4 lane groups).
template <typename T, int DH, int R16>
__device__ __forceinline__ float project_block(f32x4 (&ut)[R16],
                                               const typename FragOf<T>::type (&xf)[(DH + 31) / 32],
                                               const T* mfrag, int lane, float half_log2m) {
  constexpr int KD = (DH + 31) / 32;
  constexpr int NM = EShape<T, R16>::NM;
  float ss = 0.f;
#pragma unroll
  for (int rb = 0; rb < R16; ++rb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
#pragma unroll
      for (int part = 0; part < NM; ++part)
        acc = mma(ld8(mfrag + (((rb * KD + kd) * NM + part) * 64 + lane) * 8), xf[kd], acc);
    ut[rb] = acc;
#pragma unroll
    for (int i = 0; i < 4; ++i) ss += acc[i] * acc[i];
  }
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  return 0.5f * kLog2e * ss + half_log2m;
}

__device__ __forceinline__ float bf16_hi(float x) { return (float)(bf16)x; }

// u^T accumulators -> operand fragments over the rank index
template <typename T, int R16>
__device__ __forceinline__ void u_frags(typename FragOf<T>::type* uf, const f32x4 (&ut)[R16]) {
  typedef typename FragOf<T>::type F;
  typedef EShape<T, R16> S;
  if constexpr (!S::split) {
#pragma unroll
    for (int p = 0; p < S::RK; ++p) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      uf[p] = frag_from_acc<F>(ut[2 * p], (2 * p + 1 < R16) ? ut[2 * p + 1] : z);
    }
  } else if constexpr (S::packed) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = bf16_hi(ut[0][i]);
      v[4 + i] = ut[0][i] - v[i];
    }
    make_frag(uf[0], v);
  } else {
#pragma unroll
    for (int p = 0; p < S::RK; ++p) {
      float vh[8], vl[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = (2 * p + hh < R16) ? ut[2 * p + hh][i] : 0.f;
          vh[4 * hh + i] = bf16_hi(x);
          vl[4 * hh + i] = x - vh[4 * hh + i];
        }
      make_frag(uf[p], vh);
      make_frag(uf[S::RK + p], vl);
    }
  }
}

// e += u . omega' over the rank index: u_hi omega'_hi + u_lo omega'_hi +
// u_hi omega'_lo on the bf16 path.  U_IS_A: u fragments are the A operand
// (result rows = tokens); otherwise omega' is (result rows = features).
template <typename T, int R16, bool U_IS_A>
__device__ __forceinline__ f32x4 exponent(const typename FragOf<T>::type* uf,
                                          const typename FragOf<T>::type* of, f32x4 e) {
  typedef EShape<T, R16> S;
  auto mm = [](const typename FragOf<T>::type& u, const typename FragOf<T>::type& o, f32x4 c) {
    if constexpr (U_IS_A) return mma(u, o, c);
    else return mma(o, u, c);
  };
  if constexpr (!S::split) {
#pragma unroll
    for (int p = 0; p < S::RK; ++p) e = mm(uf[p], of[p], e);
  } else if constexpr (S::packed) {
    e = mm(uf[0], of[0], e);
    e = mm(uf[0], of[1], e);
  } else {
#pragma unroll
    for (int p = 0; p < S::RK; ++p) {
      e = mm(uf[p], of[p], e);
      e = mm(uf[S::RK + p], of[p], e);
      e = mm(uf[p], of[S::RK + p], e);
    }
  }
  return e;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Preparation: M' = d_h^(-1/4) M and omega' = log2(e) omega in fragment order.
//   mfrag[hm][rb][kd][part][lane][8]: row 16 rb + c of M' (part 0 = hi, 1 = lo
//                                     on the bf16 path), columns 32 kd + 8g + e
//   ofrag[fb][k][lane][8]: row 16 fb + c of omega'; the rank index of slot e is
//     32 p + 16 (e / 4) + 4g + e % 4 for K-step p.  fp32: k = p.  bf16 with
//     r > 16: k = p (hi) and k = RK + p (lo).  bf16 with r <= 16: k = 0 holds
//     the hi part in both halves (it meets u_hi and u_lo), k = 1 the lo part in
//     the first half.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void prep_kernel(const float* __restrict__ M, const float* __restrict__ omega,
                            T* __restrict__ mfrag, T* __restrict__ ofrag, int HM, int r, int d_h,
                            int m, int R16, int KD, int FB, float s) {
  constexpr bool split = sizeof(T) == 2;
  constexpr int NM = split ? 2 : 1;
  const int RK = (R16 + 1) / 2;
  const bool packed = split && R16 == 1;
  const int NO = !split ? RK : (packed ? 2 : 2 * RK);
  const long nM = (long)HM * R16 * KD * NM * 64;
  const long nO = (long)FB * NO * 64;
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < nM + nO;
       idx += (long)gridDim.x * blockDim.x) {
    float v[8];
    if (idx < nM) {
      const int lane = (int)(idx & 63);
      const long f = idx >> 6;
      const int part = (int)(f % NM);
      const int kd = (int)((f / NM) % KD);
      const int rb = (int)((f / ((long)NM * KD)) % R16);
      const int hm = (int)(f / ((long)NM * KD * R16));
      const int c = lane & 15, g = lane >> 4;
      const int row = rb * 16 + c;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = kd * 32 + 8 * g + e;
        const float x = (row < r && col < d_h) ? s * M[((long)hm * r + row) * d_h + col] : 0.f;
        const float hi = split ? bf16_hi(x) : x;
        v[e] = part == 0 ? hi : x - hi;
      }
      typename FragOf<T>::type fr;
      make_frag(fr, v);
      st8(mfrag + idx * 8, fr);
    } else {
      const long j = idx - nM;
      const int lane = (int)(j & 63);
      const long f = j >> 6;
      const int k = (int)(f % NO);
      const int fb = (int)(f / NO);
      const int c = lane & 15, g = lane >> 4;
      const int row = fb * 16 + c;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int hh = e >> 2, i = e & 3;
        int a;
        bool lo;
        if (packed) {
          a = 4 * g + i;
          lo = k == 1;
          if (lo && hh == 1) a = r;            // u_lo . omega'_lo is dropped
        } else {
          const int p = split ? k % RK : k;
          lo = split && k >= RK;
          a = 32 * p + 16 * hh + 4 * g + i;
        }
        const float x = (row < m && a < r) ? kLog2e * omega[(long)row * r + a] : 0.f;
        const float hi = split ? bf16_hi(x) : x;
        v[e] = lo ? x - hi : hi;
      }
      typename FragOf<T>::type fr;
      make_frag(fr, v);
      st8(ofrag + j * 8, fr);
    }
  }
}

// ---------------------------------------------------------------------------
// Key side: per unit (a chunk or an L-split of one (b, h)) and feature slice,
//   S^T[d][j] = sum_t [V, 1][t][d] phi(k_t)_j   (d = 0..d_h, row d_h is z)
// written in fp32 to spart[bh][unit][d][j].
// Workgroup: 4 waves; a tile is 64 tokens; wave w projects token block w and
// publishes its rank-index fragments and shifts in LDS, then every wave
// handles its own FW features for the whole tile.
// ---------------------------------------------------------------------------
template <typename T, int DH, int R16, int FW>
__global__ __launch_bounds__(kThreads) void kstate_kernel(FwdArgs a, Plan pl, const T* __restrict__ mfrag,
                                                           const T* __restrict__ ofrag,
                                                           float* __restrict__ spart) {
  typedef typename FragOf<T>::type F;
  typedef EShape<T, R16> S;
  constexpr int KD = (DH + 31) / 32;
  constexpr int NU = S::NU;
  constexpr int NOL = S::NO;
  constexpr int DB = DH / 16;          // 16-blocks of V; block DB is the ones column
  constexpr int FBW = FW / 16;         // feature blocks per wave
  constexpr int TT = 16 * kWaves;      // tokens per tile
  constexpr int VST = TT + 8;          // LDS row stride of V^T (elements)

  __shared__ __attribute__((aligned(16))) T s_u[kWaves][NU][64 * 8];
  __shared__ float s_init[TT];
  __shared__ __attribute__((aligned(16))) T s_vt[DH * VST];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int fslice = blockIdx.x % pl.NF;
  const int unit = (blockIdx.x / pl.NF) % pl.NU;
  const int bh = blockIdx.x / (pl.NF * pl.NU);
  const int b = bh / a.H, h = bh % a.H;
  const int hk = (h * a.H_kv) / a.H;
  const T* kb = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
  const T* vb = reinterpret_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
  const uint8_t* mrow = a.mask ? a.mask + (long)b * a.L : nullptr;
  const T* mf = mfrag + (long)(a.m_per_head ? h : 0) * R16 * KD * S::NM * 64 * 8;
  const float half_log2m = 0.5f * log2f((float)a.m);
  const int t_begin = unit * pl.span1;
  const int t_end = min(a.L, t_begin + pl.span1);
  const int fb0 = (fslice * kWaves + w) * FBW;   // first feature block of this wave

  f32x4 acc[DB + 1][FBW];
#pragma unroll
  for (int db = 0; db <= DB; ++db)
#pragma unroll
    for (int f = 0; f < FBW; ++f) acc[db][f] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int t0 = t_begin; t0 < t_end; t0 += TT) {
    // ---- projection of token block w (rows t0 + 16 w + c) ----
    {
      const int t = t0 + 16 * w + c;
      const bool ok = t < t_end;
      F xf[KD];
      load_rows<T, DH>(xf, kb + (long)t * a.ks[2], ok, g);
      f32x4 ut[R16];
      const float shift = project_block<T, DH, R16>(ut, xf, mf, lane, half_log2m);
      F uf[NU];
      u_frags<T, R16>(uf, ut);
#pragma unroll
      for (int p = 0; p < NU; ++p) st8(&s_u[w][p][lane * 8], uf[p]);
      const bool valid = ok && (mrow == nullptr || mrow[t] != 0);
      if (g == 0) s_init[16 * w + c] = valid ? -shift : -INFINITY;
    }
    // ---- V tile, transposed: s_vt[d][token] ----
    for (int e = tid; e < TT * (DH / 8); e += kThreads) {
      const int tl = e / (DH / 8), d8 = (e % (DH / 8)) * 8;
      const int t = t0 + tl;
      float vv[8];
      if (t < t_end) {
        const F x = ld8(vb + (long)t * a.vs[2] + d8);
#pragma unroll
        for (int i = 0; i < 8; ++i) vv[i] = to_f32(x[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) vv[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) s_vt[(d8 + i) * VST + tl] = (T)vv[i];
    }
    __syncthreads();

    // ---- features of this wave's blocks and the contraction over tokens ----
#pragma unroll
    for (int q = 0; q < TT / 32; ++q) {
      F vf[DB + 1];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const T* base = s_vt + (db * 16 + c) * VST + 32 * q + 4 * g;
        vf[db] = ld4x2(base, base + 16);
      }
      vf[DB] = ones_frag<F>(c);
#pragma unroll
      for (int f = 0; f < FBW; ++f) {
        const int fb = fb0 + f;
        if (fb < pl.FB) {
          F of[NOL];
#pragma unroll
          for (int p = 0; p < NOL; ++p) of[p] = ld8(ofrag + ((long)(fb * S::NO + p) * 64 + lane) * 8);
          f32x4 ph[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int tb = 2 * q + hh;
            f32x4 e4;
#pragma unroll
            for (int i = 0; i < 4; ++i) e4[i] = s_init[16 * tb + 4 * g + i];
            F uf[NU];
#pragma unroll
            for (int p = 0; p < NU; ++p) uf[p] = ld8(&s_u[tb][p][lane * 8]);
            e4 = exponent<T, R16, true>(uf, of, e4);
#pragma unroll
            for (int i = 0; i < 4; ++i) ph[hh][i] = fast_exp2(e4[i]);
          }
          const F pf = frag_from_acc<F>(ph[0], ph[1]);
#pragma unroll
          for (int db = 0; db <= DB; ++db) acc[db][f] = mma(vf[db], pf, acc[db][f]);
        }
      }
    }
    __syncthreads();
  }

  // ---- write this wave's part of the unit state ----
  float* dst = spart + ((long)bh * pl.NU + unit) * (long)(DH + 1) * a.m;
#pragma unroll
  for (int f = 0; f < FBW; ++f) {
    const int fb = fb0 + f;
    if (fb < pl.FB) {
#pragma unroll
      for (int db = 0; db <= DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = db * 16 + 4 * g + i;
          if (d <= DH) dst[(long)d * a.m + fb * 16 + c] = acc[db][f][i];
        }
    }
  }
}

// ---------------------------------------------------------------------------
// State combination.  Non-causal: the sum over the L-splits.  Causal: the
// exclusive prefix over chunks (the state before each chunk), and optionally
// the state after the last token exported as S[b][h][j][d], z[b][h][j].
// Output in fragment order as the B operand of the query-side contraction:
//   sfrag[bh][unit][db][pm][lane][8]: column d = 16 db + c, feature
//   32 pm + 16 (e / 4) + 4g + e % 4.
// One thread per (bh, db, pm, lane).
// ---------------------------------------------------------------------------
template <typename T, int DH>
__global__ void scan_kernel(FwdArgs a, Plan pl, const float* __restrict__ spart, T* __restrict__ sfrag) {
  constexpr int DB = DH / 16;
  const long n = (long)pl.BH * (DB + 1) * pl.PM * 64;
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < n;
       idx += (long)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const int pm = (int)((idx >> 6) % pl.PM);
    const int db = (int)((idx >> 6) / pl.PM % (DB + 1));
    const long bh = (idx >> 6) / ((long)pl.PM * (DB + 1));
    const int c = lane & 15, g = lane >> 4;
    const int d = db * 16 + c;
    int jj[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) jj[e] = 32 * pm + 16 * (e >> 2) + 4 * g + (e & 3);
    const bool row_ok = d <= DH;
    float run[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const float* src = spart + bh * pl.NU * (long)(DH + 1) * a.m;
    const long ustride = (long)(DH + 1) * a.m;
    const int nout = a.causal ? pl.NU : 1;
    for (int u = 0; u < pl.NU; ++u) {
      if (a.causal) {
        typename FragOf<T>::type fr;
        make_frag(fr, run);
        st8(sfrag + ((((bh * nout + u) * (DB + 1) + db) * pl.PM + pm) * 64 + lane) * 8, fr);
      }
      if (row_ok) {
        const float* s = src + u * ustride + (long)d * a.m;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (jj[e] < a.m) run[e] += s[jj[e]];
      }
    }
    if (!a.causal) {
      typename FragOf<T>::type fr;
      make_frag(fr, run);
      st8(sfrag + (((bh * (DB + 1) + db) * pl.PM + pm) * 64 + lane) * 8, fr);
    } else if (row_ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (jj[e] >= a.m) continue;
        if (d < DH && a.S_out) a.S_out[(bh * a.m + jj[e]) * DH + d] = run[e];
        if (d == DH && a.z_out) a.z_out[bh * a.m + jj[e]] = run[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Query side: per (b, h) and tile of 64 NQB queries (a chunk when causal),
//   [N, D] = Phi(Q) [S, z] (+ tril(Phi(Q) Phi(K_chunk)^T) [V, 1] when causal),
//   out = N / D (0 where D == 0).
// Wave w owns query blocks w NQB .. w NQB + NQB - 1 of the tile; when causal,
// the keys at the same positions are mapped by the same wave and shared with
// the other waves through LDS, one 32-feature step at a time.
// ---------------------------------------------------------------------------
template <typename T, int DH, int R16, int NQB, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void qout_kernel(FwdArgs a, Plan pl, const T* __restrict__ mfrag,
                                                         const T* __restrict__ ofrag,
                                                         const T* __restrict__ sfrag) {
  typedef typename FragOf<T>::type F;
  typedef EShape<T, R16> S;
  constexpr int KD = (DH + 31) / 32;
  constexpr int NU = S::NU;
  constexpr int NOL = S::NO;
  constexpr int DB = DH / 16;
  constexpr int NB = kWaves * NQB;         // 16-token blocks per tile
  constexpr int TT = 16 * NB;              // tokens per tile
  constexpr int VST = TT + 8;
  constexpr int VT_ELEMS = CAUSAL ? DH * VST : 8;
  constexpr int KF_ELEMS = CAUSAL ? 2 * NB * 64 * 8 : 8;

  __shared__ __attribute__((aligned(16))) T s_vt[VT_ELEMS];
  __shared__ __attribute__((aligned(16))) T s_kf[KF_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x % pl.NT2;
  const int bh = blockIdx.x / pl.NT2;
  const int b = bh / a.H, h = bh % a.H;
  const int hk = (h * a.H_kv) / a.H;
  const T* qb = reinterpret_cast<const T*>(a.q) + b * a.qs[0] + h * a.qs[1];
  const T* kb = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
  const T* vb = reinterpret_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
  T* ob = reinterpret_cast<T*>(a.out) + b * a.os[0] + h * a.os[1];
  const uint8_t* mrow = a.mask ? a.mask + (long)b * a.L : nullptr;
  const T* mf = mfrag + (long)(a.m_per_head ? h : 0) * R16 * KD * S::NM * 64 * 8;
  const float half_log2m = 0.5f * log2f((float)a.m);
  const int t0 = tile * TT;
  const T* sf = sfrag + ((long)bh * (CAUSAL ? pl.NU : 1) + (CAUSAL ? tile : 0)) * (DB + 1) * pl.PM * 64 * 8;

  // ---- projections of this wave's query (and key) blocks ----
  F uq[NQB][NU];
  float shq[NQB];
  F uk[CAUSAL ? NQB : 1][NU];
  float initk[CAUSAL ? NQB : 1];
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const int t = t0 + (w * NQB + j) * 16 + c;
    const bool ok = t < a.L;
    F xf[KD];
    f32x4 ut[R16];
    load_rows<T, DH>(xf, qb + (long)t * a.qs[2], ok, g);
    shq[j] = project_block<T, DH, R16>(ut, xf, mf, lane, half_log2m);
    u_frags<T, R16>(uq[j], ut);
    if constexpr (CAUSAL) {
      load_rows<T, DH>(xf, kb + (long)t * a.ks[2], ok, g);
      const float sh = project_block<T, DH, R16>(ut, xf, mf, lane, half_log2m);
      u_frags<T, R16>(uk[j], ut);
      const bool valid = ok && (mrow == nullptr || mrow[t] != 0);
      initk[j] = valid ? -sh : -INFINITY;
    }
  }
  if constexpr (CAUSAL) {
    for (int e = tid; e < TT * (DH / 8); e += kThreads) {
      const int tl = e / (DH / 8), d8 = (e % (DH / 8)) * 8;
      const int t = t0 + tl;
      float vv[8];
      if (t < a.L) {
        const F x = ld8(vb + (long)t * a.vs[2] + d8);
#pragma unroll
        for (int i = 0; i < 8; ++i) vv[i] = to_f32(x[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) vv[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) s_vt[(d8 + i) * VST + tl] = (T)vv[i];
    }
  }

  f32x4 acc[NQB][DB + 1];
#pragma unroll
  for (int j = 0; j < NQB; ++j)
#pragma unroll
    for (int db = 0; db <= DB; ++db) acc[j][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  f32x4 at[CAUSAL ? NQB : 1][CAUSAL ? NB : 1];   // A^T[key block][query block of the wave]
  if constexpr (CAUSAL) {
#pragma unroll
    for (int j = 0; j < NQB; ++j)
#pragma unroll
      for (int kb2 = 0; kb2 < NB; ++kb2) at[j][kb2] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  for (int pm = 0; pm < pl.PM; ++pm) {
    f32x4 phq[NQB][2];
    f32x4 phk[CAUSAL ? NQB : 1][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int fb = 2 * pm + hh;
      if (fb < pl.FB) {
        F of[NOL];
#pragma unroll
        for (int p = 0; p < NOL; ++p) of[p] = ld8(ofrag + ((long)(fb * S::NO + p) * 64 + lane) * 8);
#pragma unroll
        for (int j = 0; j < NQB; ++j) {
          f32x4 e4 = {-shq[j], -shq[j], -shq[j], -shq[j]};
          e4 = exponent<T, R16, false>(uq[j], of, e4);
#pragma unroll
          for (int i = 0; i < 4; ++i) phq[j][hh][i] = fast_exp2(e4[i]);
          if constexpr (CAUSAL) {
            f32x4 k4 = {initk[j], initk[j], initk[j], initk[j]};
            k4 = exponent<T, R16, false>(uk[j], of, k4);
#pragma unroll
            for (int i = 0; i < 4; ++i) phk[j][hh][i] = fast_exp2(k4[i]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NQB; ++j) {
          phq[j][hh] = (f32x4){0.f, 0.f, 0.f, 0.f};
          if constexpr (CAUSAL) phk[j][hh] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    F pq[NQB];
#pragma unroll
    for (int j = 0; j < NQB; ++j) pq[j] = frag_from_acc<F>(phq[j][0], phq[j][1]);
    // inter-chunk (or whole-sequence) state
#pragma unroll
    for (int db = 0; db <= DB; ++db) {
      const F s = ld8(sf + ((long)(db * pl.PM + pm) * 64 + lane) * 8);
#pragma unroll
      for (int j = 0; j < NQB; ++j) acc[j][db] = mma(pq[j], s, acc[j][db]);
    }
    if constexpr (CAUSAL) {
      T* kbuf = s_kf + (pm & 1) * NB * 64 * 8;
#pragma unroll
      for (int j = 0; j < NQB; ++j) st8(kbuf + ((w * NQB + j) * 64 + lane) * 8, frag_from_acc<F>(phk[j][0], phk[j][1]));
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NQB; ++j) {
        const int gq = w * NQB + j;
#pragma unroll
        for (int kb2 = 0; kb2 < NB; ++kb2)
          if (kb2 <= gq) at[j][kb2] = mma(ld8(kbuf + (kb2 * 64 + lane) * 8), pq[j], at[j][kb2]);
      }
    }
  }

  if constexpr (CAUSAL) {
    // causal mask inside the diagonal block: key 4g + i is visible to query c iff 4g + i <= c
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      const int gq = w * NQB + j;
#pragma unroll
      for (int kb2 = 0; kb2 < NB; ++kb2)
        if (kb2 == gq) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * g + i > c) at[j][kb2][i] = 0.f;
        }
    }
#pragma unroll
    for (int q = 0; q < NB / 2; ++q) {
      F vf[DB + 1];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const T* base = s_vt + (db * 16 + c) * VST + 32 * q + 4 * g;
        vf[db] = ld4x2(base, base + 16);
      }
      vf[DB] = ones_frag<F>(c);
#pragma unroll
      for (int j = 0; j < NQB; ++j) {
        const int gq = w * NQB + j;
        if (2 * q <= gq) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          const F pf = frag_from_acc<F>(at[j][2 * q], (2 * q + 1 <= gq) ? at[j][2 * q + 1] : z);
#pragma unroll
          for (int db = 0; db <= DB; ++db) acc[j][db] = mma(pf, vf[db], acc[j][db]);
        }
      }
    }
  }

  // ---- out = N / D ----
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    float den[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) den[i] = __shfl(acc[j][DB][i], lane & 48);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + (w * NQB + j) * 16 + 4 * g + i;
      if (t < a.L) {
        const float inv = den[i] > 0.f ? 1.0f / den[i] : 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) store_out(ob + (long)t * a.os[2] + db * 16 + c, acc[j][db][i] * inv);
      }
    }
  }
}

constexpr size_t kMaxLds = 160 * 1024;
// LDS of the causal query-side kernel: the V^T tile and two key-feature buffers
template <typename T, int DH, int NQB> constexpr size_t causal_lds_bytes() {
  return (size_t)(DH * (64 * NQB + 8) + 2 * 4 * NQB * 64 * 8) * sizeof(T);
}

// ---------------------------------------------------------------------------
// Host launch of one forward call for (T, DH, R16).
// ---------------------------------------------------------------------------
template <typename T, int DH, int R16, int FW>
dark_status launch_fwd_impl(const FwdArgs& a, const Plan& pl, void* ws, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(ws);
  T* mfrag = reinterpret_cast<T*>(base + pl.off_mfrag);
  T* ofrag = reinterpret_cast<T*>(base + pl.off_ofrag);
  float* spart = reinterpret_cast<float*>(base + pl.off_spart);
  T* sfrag = reinterpret_cast<T*>(base + pl.off_sfrag);
  {
    typedef EShape<T, R16> S;
    const long n = (long)pl.HM * R16 * pl.KD * S::NM * 64 + (long)pl.FB * S::NO * 64;
    const int blocks = (int)((n + 255) / 256);
    KernelTimer tm(kPrep, stream);
    hipLaunchKernelGGL(prep_kernel<T>, dim3(blocks), dim3(256), 0, st, a.M, a.omega, mfrag, ofrag, pl.HM,
                       a.r, DH, a.m, R16, pl.KD, pl.FB, powf((float)DH, -0.25f));
  }
  {
    KernelTimer tm(kKState, stream);
    hipLaunchKernelGGL((kstate_kernel<T, DH, R16, FW>), dim3(pl.BH * pl.NU * pl.NF), dim3(kThreads), 0, st, a,
                       pl, mfrag, ofrag, spart);
  }
  {
    const long n = (long)pl.BH * (DH / 16 + 1) * pl.PM * 64;
    const int blocks = (int)((n + 255) / 256);
    KernelTimer tm(kScan, stream);
    hipLaunchKernelGGL((scan_kernel<T, DH>), dim3(blocks), dim3(256), 0, st, a, pl, spart, sfrag);
  }
  const dim3 grid(pl.BH * pl.NT2);
  KernelTimer tm(kQOut, stream);
  if (a.causal) {
    switch (pl.NQB) {
      case 1: hipLaunchKernelGGL((qout_kernel<T, DH, R16, 1, true>), grid, dim3(kThreads), 0, st, a, pl, mfrag, ofrag, sfrag); break;
      case 2:
        if constexpr (causal_lds_bytes<T, DH, 2>() <= kMaxLds) {
          hipLaunchKernelGGL((qout_kernel<T, DH, R16, 2, true>), grid, dim3(kThreads), 0, st, a, pl, mfrag, ofrag, sfrag);
          break;
        } else {
          return DARK_ERR_UNSUPPORTED;
        }
      default: return DARK_ERR_UNSUPPORTED;
    }
  } else {
    switch (pl.NQB) {
      case 1: hipLaunchKernelGGL((qout_kernel<T, DH, R16, 1, false>), grid, dim3(kThreads), 0, st, a, pl, mfrag, ofrag, sfrag); break;
      case 4: hipLaunchKernelGGL((qout_kernel<T, DH, R16, 4, false>), grid, dim3(kThreads), 0, st, a, pl, mfrag, ofrag, sfrag); break;
      default: return DARK_ERR_UNSUPPORTED;
    }
  }
  return hipGetLastError() == hipSuccess ? DARK_OK : DARK_ERR_HIP;
}

}  // namespace dk
