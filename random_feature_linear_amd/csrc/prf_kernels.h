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
// of a key's exponent product starts at -(log2(e) |u|^2 / 2 + log2(m) / 2), so
// the shift and the 1/sqrt(m) factor cost nothing.  A masked key, and a padding
// feature past m, starts at -inf and gives exactly 0.  A query's features need
// neither term: any factor per query row cancels in N / D (section "Kernel",
// attention equation), so the query side subtracts instead its largest
// exponent over the first 32 features, which keeps the exp2 arguments near 0.
//
// Precision of the bf16 path.  The exponent omega_j . u of the feature map
// reaches magnitudes of ten and more, and a weight error of e per key shows up
// as a relative output error of about e (outputs are averages of zero-mean
// values), so the exponent's operands are not plain bf16 (8 significant
// bits).  Unfolded, u = M' x is formed from M' as a pair of bf16 values hi +
// lo (about 16 significant bits: u = M'_hi x + M'_lo x, fp32 accumulate) with
// the bf16 rows x as they are; then u and omega' enter the exponent as fp16
// values (11 significant bits, range clamped to +-65504) in one fp16 product
// per K-step.  Folded, the token row x (converted once to fp16) meets W' =
// omega' M' in fp16 for the exponent and M' in fp16 for |u|^2 / 2.  The
// exponent's error is then about 2^-12 of its terms, below the 2^-9 rounding
// of the features themselves to bf16 for the contractions.
//
// The normaliser z = Phi(K)^T 1 is kept apart from the state S in fp32, so S
// holds only V's column blocks.  The key side forms z as a column of ones
// beside V in its products (unfolded form, or d_h = 16 where that column is
// free) or sums the rounded bf16 features on the vector ALUs (folded form); the
// query side forms D = Phi(Q) z on the vector ALUs, and the causal part adds
// the row sums of the masked scores as rounded for the products.
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

// ---- fp16 operands of the feature exponent (bf16 path) ----------------------
// One fp16 value per slot, carried in a bf16x8 register or memory slot (the
// bits are fp16) and read by the fp16 32x32x16 MFMA.  Values beyond the fp16
// range are clamped to +-65504 (the exponent is then far outside the range
// exp2 resolves in fp32 anyway).  On the fp32 path (kH16 false) the
// operands stay fp32 and nothing here is used.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <typename T> constexpr bool kH16 = sizeof(T) == 2;
__device__ __forceinline__ bf16x8 make_frag_h(const float* v) {
  f16x8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (_Float16)fminf(fmaxf(v[i], -65504.f), 65504.f);
  return __builtin_bit_cast(bf16x8, h);
}
// a bf16 fragment (a token row) as an fp16 one
__device__ __forceinline__ bf16x8 to_h(const bf16x8& x) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)x[i];
  return make_frag_h(v);
}
__device__ __forceinline__ f32x8 to_h(const f32x8& x) { return x; }
__device__ __forceinline__ f32x16 mma_h(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

__device__ __forceinline__ bf16x8 ld8(const bf16* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, u);
}
// 16-byte loads and stores of data that is touched once (the per-unit states
// between the key side and the sum): non-temporal, so they do not displace
// data that is read again.  Measured for the L=8192 GQA workload: sum 212 ->
// 182 us, key side 413 -> 405 us.  (Non-temporal stores of the sum's output,
// which the query side reads, made the sum slower again: 197 us.)
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 ld8_stream(const bf16* p) {
  const u32x4v u = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ f32x8 ld8_stream(const float* p) {
  const f32x4v a = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
  const f32x4v b = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p + 4));
  f32x8 f = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return f;
}
__device__ __forceinline__ void st8_stream(bf16* p, const bf16x8& f) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4v, f), reinterpret_cast<u32x4v*>(p));
}
__device__ __forceinline__ void st8_stream(float* p, const f32x8& f) {
  const f32x4v a = {f[0], f[1], f[2], f[3]}, b = {f[4], f[5], f[6], f[7]};
  __builtin_nontemporal_store(a, reinterpret_cast<f32x4v*>(p));
  __builtin_nontemporal_store(b, reinterpret_cast<f32x4v*>(p + 4));
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
// The per-unit states between the key side and the sum: streamed past the
// caches (non-temporal) when they are too large to stay in L2, else ordinary
// accesses, so that the sum, which runs on the XCD that wrote them, finds them
// in its L2.
template <typename F, typename T> __device__ __forceinline__ F ld8_state(const T* p, int stream) {
  return stream ? ld8_stream(p) : ld8(p);
}
template <typename T, typename F> __device__ __forceinline__ void st8_state(T* p, const F& f, int stream) {
  if (stream)
    st8_stream(p, f);
  else
    st8(p, f);
}
// One 16-byte element per lane from global memory straight into LDS (the
// global_load_lds path, no registers): lane l writes bytes [16 l, 16 l + 16) of
// the 1 KB at lds_dst, which must be the same for the whole wave.  Counted by
// vmcnt.  (The host pass of the compiler only sees an empty body.)
__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
#else
  (void)src;
  (void)lds_dst;
#endif
}
// Workgroups are dispatched to the 8 XCDs in turn (block b runs on XCD b % 8),
// and each XCD has its own L2.  The logical index returned here gives each XCD
// a contiguous range of logical work items, so that items next to each other
// (the feature slices of one key tile, the tiles of one head) share an L2.
__device__ __forceinline__ int xcd_block() {
  constexpr int NX = 8;
  const int n = gridDim.x, b = blockIdx.x;
  const int per = n / NX, rem = n % NX;   // XCD x runs per + (x < rem) blocks
  const int x = b % NX;
  return x * per + min(x, rem) + b / NX;
}
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ void store_out(bf16* p, float x) { *p = (bf16)x; }
__device__ __forceinline__ void store_out(float* p, float x) { *p = x; }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc += (fragment of M' at p) x.  bf16 path: with MH (the folded exponent's
// and the exact path's form) M' is one fp16 part and x is already fp16, one
// fp16 product; otherwise M' is a bf16 hi part at p and lo part 64 x 8
// elements further, and x is bf16 (exact), two products.  fp32: one product.
template <typename T, bool MH>
__device__ __forceinline__ f32x16 m_product(const T* p, const typename FragOf<T>::type& x, f32x16 acc) {
  if constexpr (kH16<T> && MH) {
    return mma_h(ld8(p), x, acc);
  } else if constexpr (kParts<T> == 2) {
    acc = mma(ld8(p), x, acc);
    return mma(ld8(p + 64 * 8), x, acc);
  } else {
    return mma(ld8(p), x, acc);
  }
}
// the token rows of a projection in place: fp16 on the bf16 path
template <typename F, int N> __device__ __forceinline__ void rows_to_h(F (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = to_h(x[i]);
}

// ---- the feature map of one 32-token block -----------------------------------
// Token row t as the B-operand fragments X^T of the projection (K-steps of 16
// over d_h); rows at or past the end are zero.
template <typename T, int DH>
__device__ __forceinline__ void load_rows(typename FragOf<T>::type (&xf)[DH / 16], const T* row, bool ok,
                                          int g) {
  typedef typename FragOf<T>::type F;
  // loads under the lane mask into zeroed registers: a select after the load
  // would make the code right behind it wait for the load
#pragma unroll
  for (int kd = 0; kd < DH / 16; ++kd) xf[kd] = zero_frag<F>();
  if (ok) {
#pragma unroll
    for (int kd = 0; kd < DH / 16; ++kd) xf[kd] = ld8(row + kd * 16 + 8 * g);
  }
}

// u^T = M' x^T for a 32-token block (rank index in rows, token c in the lane),
// returned as hi / lo operand fragments over the rank index (K-steps of 16),
// or (H16, bf16 path) as one fp16 fragment per K-step in uhi, plus the
// exp2-domain shift log2(e) |u|^2 / 2 + log2(m) / 2 of token c.  MH: M' in
// its one-part fp16 form, the token rows xf already fp16 (see m_product).
template <typename T, int DH, int R16, bool H16 = false, bool MH = false>
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
      acc = m_product<T, MH>(mfrag + ((rb * KD + kd) * NM * 64 + lane) * 8, xf[kd], acc);
#pragma unroll
    for (int i = 0; i < 16; ++i) ss += acc[i] * acc[i];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (2 * rb + h < R16) {
        if constexpr (H16) {   // one fp16 part (the lo fragment is not read)
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = acc[8 * h + e];
          uhi[2 * rb + h] = make_frag_h(v);
        } else {
          acc_frag_split<T>(acc, h, uhi[2 * rb + h], ulo[2 * rb + h]);
        }
      }
    if constexpr (KD * NM > 8) __builtin_amdgcn_sched_barrier(0);
  }
  ss += __shfl_xor(ss, 32);
  return 0.5f * kLog2e * ss + half_log2m;
}

// e += u . omega' over the K-steps of the exponent: u_hi omega'_hi + u_lo
// omega'_hi + u_hi omega'_lo (bf16), or one fp32 product.  In the folded form
// (see fold_exponent) u is the token row x itself, which is exact in bf16
// (ULO false, no u_lo term), and omega' is W'.  H16 (the feature map on the
// bf16 path): u and omega' are one fp16 fragment each, one fp16 product per
// K-step, the lo fragments unused.  U_IS_A: the u fragments are the A operand
// (result rows = tokens, columns = features); otherwise omega' is (result rows
// = features, columns = tokens).
template <typename T, int NK, bool U_IS_A, bool ULO = true, bool H16 = false>
__device__ __forceinline__ f32x16 exponent(const typename FragOf<T>::type* uhi,
                                           const typename FragOf<T>::type* ulo,
                                           const typename FragOf<T>::type* ohi,
                                           const typename FragOf<T>::type* olo, f32x16 e) {
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    if constexpr (H16) {
      static_assert(sizeof(T) == 2, "fp16 exponent operands: bf16 path");
      e = U_IS_A ? mma_h(uhi[k], ohi[k], e) : mma_h(ohi[k], uhi[k], e);
    } else if constexpr (U_IS_A) {
      e = mma(uhi[k], ohi[k], e);
      if constexpr (kParts<T> == 2) {
        if constexpr (ULO) e = mma(ulo[k], ohi[k], e);
        e = mma(uhi[k], olo[k], e);
      }
    } else {
      e = mma(ohi[k], uhi[k], e);
      if constexpr (kParts<T> == 2) {
        if constexpr (ULO) e = mma(ohi[k], ulo[k], e);
        e = mma(olo[k], uhi[k], e);
      }
    }
  }
  return e;
}

// The same sum with the operands fetched step by step: uload(k, part) and
// oload(k, part) return fragment k of the token operand and of omega' (W').
// Long sums (more than 8 K-steps, d_h = 256 folded) run in chunks of 2 steps
// whose operands are fetched one chunk ahead, with scheduling fences between
// chunks so that at most two chunks of operands are live in registers.
template <typename T, int NK, bool U_IS_A, bool ULO, bool H16 = false, typename UL, typename OL>
__device__ __forceinline__ f32x16 exponent_stream(UL uload, OL oload, f32x16 e) {
  typedef typename FragOf<T>::type F;
  constexpr bool LO_U = ULO && !H16, LO_O = !H16;   // lo fragments that are read
  if constexpr (NK <= 8) {
    F uh[NK], ul[NK], oh[NK], ol[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      uh[k] = uload(k, 0);
      if constexpr (LO_U) ul[k] = uload(k, 1);
      oh[k] = oload(k, 0);
      if constexpr (LO_O) ol[k] = oload(k, 1);
    }
    return exponent<T, NK, U_IS_A, ULO, H16>(uh, ul, oh, ol, e);
  } else {
    constexpr int CH = 2;
    static_assert(NK % CH == 0, "chunked exponent");
    F uh[2][CH], ul[2][LO_U ? CH : 1], oh[2][CH], ol[2][LO_O ? CH : 1];
    auto fetch = [&](int b, int k0) {
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        uh[b][k] = uload(k0 + k, 0);
        if constexpr (LO_U) ul[b][k] = uload(k0 + k, 1);
        oh[b][k] = oload(k0 + k, 0);
        if constexpr (LO_O) ol[b][k] = oload(k0 + k, 1);
      }
    };
    fetch(0, 0);
#pragma unroll
    for (int c0 = 0; c0 < NK / CH; ++c0) {
      if (c0 + 1 < NK / CH) fetch((c0 + 1) & 1, (c0 + 1) * CH);
      __builtin_amdgcn_sched_barrier(0);
      e = exponent<T, CH, U_IS_A, ULO, H16>(uh[c0 & 1], ul[c0 & 1], oh[c0 & 1], ol[c0 & 1], e);
      __builtin_amdgcn_sched_barrier(0);
    }
    return e;
  }
}

// Only the exp2-domain shift log2(e) |u|^2 / 2 + log2(m) / 2 of token c of a
// 32-token block (the folded exponent does not need u itself).  MH as in
// project_block.
template <typename T, int DH, int R16, bool MH = false>
__device__ __forceinline__ float project_shift(const typename FragOf<T>::type (&xf)[DH / 16], const T* mfrag,
                                               int lane, float half_log2m) {
  constexpr int KD = DH / 16;
  constexpr int R32 = (R16 + 1) / 2;
  constexpr int NM = kParts<T>;
  float ss = 0.f;
#pragma unroll
  for (int rb = 0; rb < R32; ++rb) {
    f32x16 acc = zero16();
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) acc = m_product<T, MH>(mfrag + ((rb * KD + kd) * NM * 64 + lane) * 8, xf[kd], acc);
#pragma unroll
    for (int i = 0; i < 16; ++i) ss += acc[i] * acc[i];
    // large M' (d_h = 256): one 32-row slice of operands in flight at a time
    if constexpr (KD * NM > 8) __builtin_amdgcn_sched_barrier(0);
  }
  ss += __shfl_xor(ss, 32);
  return 0.5f * kLog2e * ss + half_log2m;
}

// Fragment lane idx of M' = s M (see prep_kernel): fp32; on the bf16 path
// either (h16: the folded exponent and the exact path) one fp16 value in part
// 0 of each fragment, part 1 neither written nor read, or a bf16 high part and
// a bf16 remainder (the unfolded exponent, whose token rows stay bf16).
template <typename T>
__device__ __forceinline__ void mfrag_lane(long idx, const float* __restrict__ M, T* __restrict__ mfrag, int r,
                                           int d_h, int R16, float s, bool h16) {
  constexpr int NM = kParts<T>;
  const int R32 = (R16 + 1) / 2;
  const int KD = d_h / 16;
  const int lane = (int)(idx & 63), c = lane & 31, g = lane >> 5;
  const long f = idx >> 6;
  const int part = (int)(f % NM);
  if (kH16<T> && h16 && part != 0) return;
  const int kd = (int)((f / NM) % KD);
  const int rb = (int)((f / ((long)NM * KD)) % R32);
  const int hm = (int)(f / ((long)NM * KD * R32));
  const int row = rb * 32 + c;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int col = kd * 16 + 8 * g + e;
    const float x = (row < r) ? s * M[((long)hm * r + row) * d_h + col] : 0.f;
    const float hi = NM == 2 ? bf16_hi(x) : x;
    v[e] = part == 0 ? hi : x - hi;
    if (kH16<T> && h16) v[e] = x;
  }
  if constexpr (kH16<T>) {
    if (h16) {
      st8(mfrag + idx * 8, make_frag_h(v));
      return;
    }
  }
  typename FragOf<T>::type fr;
  make_frag(fr, v);
  st8(mfrag + idx * 8, fr);
}

// ---------------------------------------------------------------------------
// Preparation: M' = d_h^(-1/4) M and omega' = log2(e) omega in fragment order.
//   mfrag[hm][rb][kd][part][lane][8]: row 32 rb + c of M', columns 16 kd + 8g + e
//   ofrag[ho][fb][k][lane][8]: row 32 fb + c of omega', rank index
//                                16k + 8 (e / 4) + 4g + e % 4
// or, folded, W'_hm = omega' M'_hm:
//   ofrag[hw][fb][kd][lane][8]: row 32 fb + c of W', columns 16 kd + 8g + e
// For M' (bf16 path) part 0 is the bf16-rounded value and part 1 the rounded
// remainder.  omega' and W' have one part: fp16 on the bf16 path (the
// exponent's operand), fp32 otherwise.
// The M' and omega' ranges take one thread per fragment lane and part; the W'
// range one thread per fragment lane (both parts, r products each).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void prep_kernel(const float* __restrict__ M, const float* __restrict__ omega,
                            T* __restrict__ mfrag, T* __restrict__ ofrag, int HM, int HO, int HW, int r, int d_h,
                            int m, int R16, int FB, float s, int fold) {
  constexpr int NM = kParts<T>;
  const int R32 = (R16 + 1) / 2;
  const int KD = d_h / 16;
  const long nM = (long)HM * R32 * KD * NM * 64;
  // fold: 0 omega' fragments (HO projections), 1 W' fragments here (HW
  // operands), 2 W' fragments by fold_kernel
  const long nO = fold == 2 ? 0 : fold ? (long)HW * FB * KD * 64 : (long)HO * FB * R16 * 64;
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < nM + nO;
       idx += (long)gridDim.x * blockDim.x) {
    float v[8];
    typename FragOf<T>::type fr;
    const bool m_side = idx < nM;
    const long j = m_side ? idx : idx - nM;
    const int lane = (int)(j & 63);
    const long f = j >> 6;
    const int c = lane & 31, g = lane >> 5;
    if (!m_side && fold) {
      const int kd = (int)(f % KD);
      const int fb = (int)((f / KD) % FB);
      const int hw = (int)(f / ((long)KD * FB));   // operand hw: M of head hw (or shared), omega likewise
      const int row = fb * 32 + c;
      const int col0 = kd * 16 + 8 * g;
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (row < m) {
        const float* orow = omega + ((long)(HO > 1 ? hw : 0) * m + row) * r;
        const float* Mh = M + (long)(HM > 1 ? hw : 0) * r * d_h + col0;
        for (int a = 0; a < r; ++a) {
          const float w = orow[a];
          const float4 m0 = *reinterpret_cast<const float4*>(Mh + (long)a * d_h);
          const float4 m1 = *reinterpret_cast<const float4*>(Mh + (long)a * d_h + 4);
          acc[0] += w * m0.x;
          acc[1] += w * m0.y;
          acc[2] += w * m0.z;
          acc[3] += w * m0.w;
          acc[4] += w * m1.x;
          acc[5] += w * m1.y;
          acc[6] += w * m1.z;
          acc[7] += w * m1.w;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = kLog2e * s * acc[e];
      const long base = f * 64 + lane;   // fragment f (fp16 on the bf16 path)
      if constexpr (kH16<T>) {
        st8(ofrag + base * 8, make_frag_h(v));
      } else {   // (the folded form is bf16 only)
        make_frag(fr, v);
        st8(ofrag + base * 8, fr);
      }
      continue;
    }
    if (m_side) {
      mfrag_lane<T>(j, M, mfrag, r, d_h, R16, s, fold != 0);
      continue;
    }
    const int k = (int)(f % R16);
    const int fb = (int)((f / R16) % FB);
    const int ho = (int)(f / ((long)R16 * FB));
    const int row = fb * 32 + c;
    const float* om = omega + (long)ho * m * r;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int a = 16 * k + 8 * (e >> 2) + 4 * g + (e & 3);
      v[e] = (row < m && a < r) ? kLog2e * om[(long)row * r + a] : 0.f;
    }
    if constexpr (kH16<T>) {   // the exponent's fp16 operand
      st8(ofrag + j * 8, make_frag_h(v));
    } else {
      make_frag(fr, v);
      st8(ofrag + j * 8, fr);
    }
  }
}

// ---------------------------------------------------------------------------
// Folded operand W'_hm = omega' M'_hm (m x d_h) for the bf16 path.  The
// products run on the bf16 matrix cores with each fp32 operand split into a
// bf16 high part and a bf16 remainder (hi hi + lo hi + hi lo, about 16
// significant bits per operand), well below the fp16 rounding of the stored
// W' (part 0 of each fragment, the exponent's operand).  Workgroup: 4 waves, one 32-feature block and up to four 32-column
// tiles (one per wave).  The rank index runs in chunks of 64: the chunk's M
// columns and omega rows are fetched into registers one chunk ahead (all loads
// of a chunk in flight together), split, and staged in LDS as bf16 parts.
// Each wave's transposed tile W'^T = M'^T omega'^T (features in the lane
// index) goes back through LDS to the fragment order of prep_kernel's folded
// layout.
// ---------------------------------------------------------------------------
constexpr int kFoldRC = 64;   // rank indices per chunk
template <typename T>
__global__ __launch_bounds__(kThreads) void fold_kernel(const float* __restrict__ M, const float* __restrict__ omega,
                                                        T* __restrict__ ofrag, T* __restrict__ mfrag, int HM, int HO,
                                                        int HW, int R16, int r, int d_h, int m, int FB, float s,
                                                        float scale) {
  static_assert(sizeof(T) == 2, "the folded operands are bf16");
  {  // blocks past the W' tiles write the M' fragments (used for |u|^2)
    const int nW = HW * FB * ((d_h / 32 + 3) / 4);
    if ((int)blockIdx.x >= nW) {
      const long nM = (long)HM * ((R16 + 1) / 2) * (d_h / 16) * kParts<T> * 64;
      const long idx = (long)(blockIdx.x - nW) * kThreads + threadIdx.x;
      if (idx < nM) mfrag_lane<T>(idx, M, mfrag, r, d_h, R16, s, true);
      return;
    }
  }
  constexpr int MST = 4 * 32 + 8;   // row stride of the M parts (bf16)
  constexpr int OST = kFoldRC + 8;  // row stride of the omega parts (bf16; 16-byte aligned rows)
  __shared__ float s_m[32][4 * 32 + 1];                                  // transpose buffer of the result
  __shared__ __attribute__((aligned(16))) bf16 s_mp[2][kFoldRC][MST];   // M[a][col] hi / lo, 128 columns
  __shared__ __attribute__((aligned(16))) bf16 s_op[2][32][OST];        // omega[32 fb + row][a] hi / lo
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int DT = d_h / 32;
  const int NG = (DT + 3) / 4;                 // groups of four column tiles
  const int grp = blockIdx.x % NG;
  const int fb = (blockIdx.x / NG) % FB;
  const int hw = blockIdx.x / (NG * FB);       // operand hw: M and omega of head hw (or the shared ones)
  const int col0 = grp * 128;                  // first column of the group
  const float* Mh = M + (long)(HM > 1 ? hw : 0) * r * d_h;
  omega += (long)(HO > 1 ? hw : 0) * m * r;
  // this thread's loads of one chunk: 8 float4 of M (row a, 4 columns), 2 float4 of omega
  float4 vm[8], vo[2];
  auto fetch = [&](int a0) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int e = tid + p * kThreads;        // 0 .. 2047: row e / 32, float4 column e % 32
      const int a = a0 + (e >> 5), cc = col0 + 4 * (e & 31);
      const float4 x = *reinterpret_cast<const float4*>(Mh + (long)min(a, r - 1) * d_h + min(cc, d_h - 4));
      vm[p] = (a < r && cc < d_h) ? x : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int e = tid + p * kThreads;        // 0 .. 511: row e / 16, four rank indices 4 (e % 16)
      const int row = e >> 4, a = a0 + 4 * (e & 15);
      const int j = min(fb * 32 + row, m - 1);
      float4 x;
      if ((r & 3) == 0) {
        x = *reinterpret_cast<const float4*>(omega + (long)j * r + min(a, r - 4));
      } else {   // rows of omega are not 16-byte aligned
        const float* o = omega + (long)j * r;
        x = make_float4(o[min(a, r - 1)], o[min(a + 1, r - 1)], o[min(a + 2, r - 1)], o[min(a + 3, r - 1)]);
      }
      const bool okr = fb * 32 + row < m;
      vo[p] = make_float4(okr && a < r ? x.x : 0.f, okr && a + 1 < r ? x.y : 0.f, okr && a + 2 < r ? x.z : 0.f,
                          okr && a + 3 < r ? x.w : 0.f);
    }
  };
  // four values as bf16 high parts and remainders at dst_hi / dst_lo
  auto split4 = [](const float4& x, bf16* dst_hi, bf16* dst_lo) {
    typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 h, l;
    h[0] = (bf16)x.x;
    h[1] = (bf16)x.y;
    h[2] = (bf16)x.z;
    h[3] = (bf16)x.w;
    l[0] = (bf16)(x.x - (float)h[0]);
    l[1] = (bf16)(x.y - (float)h[1]);
    l[2] = (bf16)(x.z - (float)h[2]);
    l[3] = (bf16)(x.w - (float)h[3]);
    *reinterpret_cast<bf16x4*>(dst_hi) = h;
    *reinterpret_cast<bf16x4*>(dst_lo) = l;
  };
  f32x16 acc = zero16();
  fetch(0);
  for (int a0 = 0; a0 < r; a0 += kFoldRC) {
    __syncthreads();   // the previous chunk is no longer read
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int e = tid + p * kThreads, row = e >> 5, cc = 4 * (e & 31);
      split4(vm[p], &s_mp[0][row][cc], &s_mp[1][row][cc]);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int e = tid + p * kThreads, row = e >> 4, a = 4 * (e & 15);
      split4(vo[p], &s_op[0][row][a], &s_op[1][row][a]);
    }
    __syncthreads();
    if (a0 + kFoldRC < r) fetch(a0 + kFoldRC);
    // K-step ks: A = M'^T (row = column 32 w + c of the group, rank 16 ks + 8 g + e),
    // B = omega'^T (column = feature c, the same ranks)
#pragma unroll
    for (int ks = 0; ks < kFoldRC / 16; ++ks) {
      bf16x8 ah, al;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ah[e] = s_mp[0][16 * ks + 8 * g + e][32 * w + c];
        al[e] = s_mp[1][16 * ks + 8 * g + e][32 * w + c];
      }
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&s_op[0][c][16 * ks + 8 * g]);
      const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&s_op[1][c][16 * ks + 8 * g]);
      acc = mma(ah, bh, acc);
      acc = mma(al, bh, acc);
      acc = mma(ah, bl, acc);
    }
  }
  __syncthreads();
  // acc[i]: W'^T[column 32 w + 8(i/4) + 4g + i%4 of the group][feature c]; s_m is the transpose buffer
#pragma unroll
  for (int i = 0; i < 16; ++i) s_m[crow(i, g)][32 * w + c] = scale * acc[i];
  __syncthreads();
  const int dt = grp * 4 + w;
  if (dt >= DT) return;
  // fragment (fb, kd = 2 dt + h): lane (c, g) holds feature c, columns 16 h + 8g + e
  const int KD = d_h / 16;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s_m[16 * h + 8 * g + e][32 * w + c];
    const long f = ((long)hw * FB + fb) * KD + 2 * dt + h;
    st8(ofrag + (f * 64 + lane) * 8, make_frag_h(x));   // the exponent's fp16 operand
  }
}

// ---------------------------------------------------------------------------
// Key shifts for the folded path: kshift[bh][t] = -(log2(e) |M'_h k_t|^2 / 2 +
// log2(m) / 2) of every key row as seen by query head h, or -inf for a masked
// key.  They replace the projection in the key-side kernel (once per feature
// slice) and in the causal query side.  (Queries need no such shift: a factor
// per query row cancels in N / D.)  Workgroup: 4 waves over 256 key rows
// (fp32: 128); wave w keeps its two 32-row blocks (fp32: one) in registers
// while M' streams through LDS one 32-row slice at a time (double-buffered,
// the next slice fetched during the products), so that every slice fragment
// read from LDS feeds two products.  The query heads that share a K/V head
// take consecutive workgroups (one L2).
// ---------------------------------------------------------------------------
// 32-row blocks per wave (fp32: one, for registers) and rows per workgroup
template <typename T> constexpr int shift_rb() { return sizeof(T) == 2 ? 2 : 1; }
template <typename T> constexpr int shift_tile() { return shift_rb<T>() * kTile; }
template <typename T, int DH, int R16>
__global__ __launch_bounds__(kThreads, 2) void shift_kernel(FwdArgs a, const T* __restrict__ mfrag,
                                                          float* __restrict__ kshift) {
  typedef typename FragOf<T>::type F;
  constexpr int KD = DH / 16;
  constexpr int NM = kParts<T>;
  constexpr int R32 = (R16 + 1) / 2;
  constexpr int RB = shift_rb<T>();
  constexpr int kShiftTile = shift_tile<T>();
  constexpr int SL = KD * NM;                         // fragments of one 32-row slice of M'
  constexpr int PS = (SL * 64 + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) T s_m[2][SL * 64 * 8];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int ntile = (a.L + kShiftTile - 1) / kShiftTile;
  const int blk = xcd_block();
  const int tile = (blk / a.H) % ntile;
  const int bh = (blk / (a.H * ntile)) * a.H + blk % a.H;
  const int b = bh / a.H, h = bh % a.H;
  const int hk = (h * a.H_kv) / a.H;
  const T* base = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
  const int64_t stride = a.ks[2];
  const T* mf = mfrag + (long)(a.m_per_head ? h : 0) * R32 * SL * 64 * 8;
  const int t0 = tile * kShiftTile + RB * 32 * w + c;   // row of block 0 of this lane
  F stage[PS];
  auto fetch = [&](int rb) {
#pragma unroll
    for (int p = 0; p < PS; ++p)
      stage[p] = ld8(mf + ((long)rb * SL * 64 + min(tid + p * kThreads, SL * 64 - 1)) * 8);
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PS; ++p)
      if (tid + p * kThreads < SL * 64) st8(&s_m[buf][(tid + p * kThreads) * 8], stage[p]);
  };
  fetch(0);
  F xf[RB][KD];
#pragma unroll
  for (int j = 0; j < RB; ++j) load_rows<T, DH>(xf[j], base + (long)(t0 + 32 * j) * stride, t0 + 32 * j < a.L, g);
  if constexpr (kH16<T>) {   // fp16 rows against the one-part fp16 M'
#pragma unroll
    for (int j = 0; j < RB; ++j) rows_to_h(xf[j]);
  }
  put(0);
  __syncthreads();
  float ss[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) ss[j] = 0.f;
#pragma unroll 1   // one slice in registers at a time
  for (int rb = 0; rb < R32; ++rb) {
    if (rb + 1 < R32) fetch(rb + 1);
    const T* sm = s_m[rb & 1];
    f32x16 u[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) u[j] = zero16();
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      {   // part 0 of the slice: M' (fp16 on the bf16 path; part 1 is not read)
        const F mfr = ld8(sm + ((kd * NM) * 64 + lane) * 8);
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          if constexpr (kH16<T>) u[j] = mma_h(mfr, xf[j][kd], u[j]);
          else u[j] = mma(mfr, xf[j][kd], u[j]);
        }
      }
      if constexpr (SL > 8)   // bound the slice fragments in flight
        if (kd % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) ss[j] += u[j][i] * u[j][i];
    if (rb + 1 < R32) put((rb + 1) & 1);
    __syncthreads();
  }
  const float hl = 0.5f * log2f((float)a.m);
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const float sq = ss[j] + __shfl_xor(ss[j], 32);
    const float sh = 0.5f * kLog2e * sq + hl;
    const int t = t0 + 32 * j;
    if (g == 0 && t < a.L) {
      const bool valid = a.mask == nullptr || a.mask[(long)b * a.L + t] != 0;
      kshift[(long)bh * a.L + t] = valid ? -sh : -INFINITY;
    }
  }
}

// Stage rows t0 .. t0 + TT - 1 of V into LDS transposed, s_vt[d][t] (rows past
// t_end are zero).
template <typename T, int DH, int TT, int VST>
__device__ __forceinline__ void stage_vt(T* s_vt, const T* vb, int64_t vstride, int t0, int t_end, int tid);

// The same staging in two halves: global loads into registers (issued a tile
// ahead of their use) and the transposed LDS stores.
template <int DH, int TT, int NT = kThreads> constexpr int vloads_per_thread() { return (TT * (DH / 8) + NT - 1) / NT; }
// Thread tid takes token tid % TT of the tile and the 8-column pieces
// 8 (tid / TT) + p VSTEP, p = 0 .. VPT - 1 (consecutive lanes: consecutive
// tokens); when the thread count is a multiple of TT every piece of a thread
// is one token row, at offsets fixed at compile time.
template <int DH, int TT, int NT> constexpr int vstep() { return NT / TT * 8; }
template <int DH, int TT, int NT> constexpr bool vpieces_in_range() {   // no piece past column DH
  return NT % TT == 0 && (vloads_per_thread<DH, TT, NT>() - 1) * vstep<DH, TT, NT>() + (NT / TT - 1) * 8 < DH;
}
template <typename T, int DH, int TT, int NT = kThreads>
__device__ __forceinline__ void load_v(typename FragOf<T>::type* vr, const T* vb, int64_t vstride, int t0, int t_end,
                                       int tid) {
  typedef typename FragOf<T>::type F;
  constexpr int VPT = vloads_per_thread<DH, TT, NT>();
  // rows past t_end are zero: loads under the lane mask into zeroed registers
  // (a select after an unconditional load would make every use of vr, and the
  // code before it, wait for the load)
  if constexpr (vpieces_in_range<DH, TT, NT>()) {
    const int t = t0 + tid % TT;
    const T* row = vb + (long)t * vstride + (tid / TT) * 8;
#pragma unroll
    for (int p = 0; p < VPT; ++p) vr[p] = zero_frag<F>();
    if (t < t_end) {
#pragma unroll
      for (int p = 0; p < VPT; ++p) vr[p] = ld8(row + p * vstep<DH, TT, NT>());
    }
  } else {
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
      const int e = tid + p * NT;
      const int tl = e % TT, d8 = (e / TT) * 8;
      const int t = t0 + tl;
      F x = zero_frag<F>();
      if (e < TT * (DH / 8) && t < t_end) x = ld8(vb + (long)t * vstride + d8);
      vr[p] = x;
    }
  }
}
// Position of token t in a row of the V^T tile: bits 2 and 3 swapped, so that
// the 8 tokens one lane of a V operand fragment holds (16k + 8(e / 4) + 4g + e % 4,
// the operand order of the feature products) are 8 consecutive elements.
__device__ __forceinline__ int vt_pos(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }
template <typename T, int DH, int TT, int VST, int NT = kThreads>
__device__ __forceinline__ void store_vt(T* s_vt, const typename FragOf<T>::type* vr, int tid) {
  constexpr int VPT = vloads_per_thread<DH, TT, NT>();
  if constexpr (vpieces_in_range<DH, TT, NT>()) {
    T* dst = s_vt + (tid / TT) * 8 * VST + vt_pos(tid % TT);
#pragma unroll
    for (int p = 0; p < VPT; ++p)
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[(p * vstep<DH, TT, NT>() + i) * VST] = vr[p][i];
  } else {
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
      const int e = tid + p * NT;
      if (e >= TT * (DH / 8)) break;
      const int tl = e % TT, d8 = (e / TT) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) s_vt[(d8 + i) * VST + vt_pos(tl)] = vr[p][i];
    }
  }
}

// Stage rows t0 .. t0 + TT - 1 of V into LDS transposed, s_vt[d][t] (rows past
// t_end are zero): all global loads first, then the transposed stores.
template <typename T, int DH, int TT, int VST>
__device__ __forceinline__ void stage_vt(T* s_vt, const T* vb, int64_t vstride, int t0, int t_end, int tid) {
  typename FragOf<T>::type vr[vloads_per_thread<DH, TT>()];
  load_v<T, DH, TT>(vr, vb, vstride, t0, t_end, tid);
  store_vt<T, DH, TT, VST>(s_vt, vr, tid);
}

// V operand fragment: column d = 32 db + c (with ONES, column d_h is all
// ones; zero past that), tokens tb0 + 16k + 8 (e / 4) + 4g + e % 4
template <typename T, int DH, int VST, bool ONES = false>
__device__ __forceinline__ typename FragOf<T>::type v_frag(const T* s_vt, int db, int tb0, int k, int c, int g) {
  typedef typename FragOf<T>::type F;
  const int d = db * 32 + c;
  if ((ONES || DH % 32 != 0) && d >= DH) {
    const float o = ONES && d == DH ? 1.0f : 0.0f;
    float v[8] = {o, o, o, o, o, o, o, o};
    F f;
    make_frag(f, v);
    return f;
  }
  return ld8(s_vt + d * VST + tb0 + 16 * k + 8 * g);   // tokens in vt_pos order
}
// bf16: V staged in its own row layout, s_v[t][d] with rows DH + 16 elements
// apart (16-byte aligned; the eight rows of 64 bytes one transpose load reads
// then cover every 16-byte bank group of a 256-byte bank row exactly twice),
// written as 16-byte pieces and read into operand fragments by
// the LDS transpose loads (ds_read_b64_tr_b16).  Within each group of 16 lanes
// such a load returns to lane 4a + b the b-th 16-bit element of the 8-byte
// pieces addressed by lanes a, a + 4, a + 8 and a + 12 of the group.  So lanes
// 16q + x address row tb0 + 16k + 4g + x / 4 (+ 8 for the second load),
// columns 32 db + 16 (q % 2) + 4 (x % 4) .. + 3, and lane l receives column
// 32 db + l % 32 at tokens tb0 + 16k + 8 (e / 4) + 4g + e % 4: the operand
// order of the feature products.
template <int DH> constexpr int vsn() { return DH + 16; }
template <typename T, int DH, int TT, int NT = kThreads>
__device__ __forceinline__ void store_v(T* s_v, const typename FragOf<T>::type* vr, int tid) {
  static_assert(sizeof(T) == 2 && vpieces_in_range<DH, TT, NT>(), "bf16 row pieces");
  T* dst = s_v + (tid % TT) * vsn<DH>() + (tid / TT) * 8;
#pragma unroll
  for (int p = 0; p < vloads_per_thread<DH, TT, NT>(); ++p)
    *reinterpret_cast<typename FragOf<T>::type*>(dst + p * vstep<DH, TT, NT>()) = vr[p];
}
template <int DH, bool ONES = false>
__device__ __forceinline__ bf16x8 v_frag_tr(const bf16* s_v, int db, int tb0, int k, int lane) {
  const int c = lane & 31;
  const int d = db * 32 + c;
  if ((ONES || DH % 32 != 0) && db * 32 >= DH) {   // the whole block past the columns of V
    const float o = ONES && d == DH ? 1.0f : 0.0f;
    float v[8] = {o, o, o, o, o, o, o, o};
    bf16x8 f;
    make_frag(f, v);
    return f;
  }
  const int x = lane & 15, q = lane >> 4, g = lane >> 5;
  const int row = tb0 + 16 * k + 4 * g + (x >> 2);
  const int col = min(db * 32 + 16 * (q & 1) + 4 * (x & 3), DH - 4);   // groups past DH: any valid address
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const bf16* p0 = s_v + row * vsn<DH>() + col;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(__attribute__((address_space(3))) bf16*)p0);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)(__attribute__((address_space(3))) bf16*)(p0 + 8 * vsn<DH>()));
  typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x8 f = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4,
                                     5, 6, 7);
  if constexpr (ONES || DH % 32 != 0) {   // columns past DH in a partly filled block
    if (d >= DH) {
      const float o = ONES && d == DH ? 1.0f : 0.0f;
      float v[8] = {o, o, o, o, o, o, o, o};
      make_frag(f, v);
    }
  }
  return f;
}

// 32-column blocks of V (of the state S).  The normaliser z (the sums of the
// features) is kept apart in fp32: the key side takes it from a column of
// ones beside V on the matrix cores, or sums the rounded features on the
// vector ALUs; the query side always forms D on the vector ALUs.
template <int DH> constexpr int vblocks() { return (DH + 31) / 32; }
template <int DH> constexpr int vblocks_ones() { return (DH + 1 + 31) / 32; }
// s + the sum of the 8 elements of an operand fragment, in fp32 (bf16: pairwise
// dot products with (1, 1), so the sum sees the rounded values the products use)
__device__ __forceinline__ float frag_sum(const bf16x8& f, float s) {
  typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 0, 1), one, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 2, 3), one, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 4, 5), one, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 6, 7), one, s, false);
}
__device__ __forceinline__ float frag_sum(const f32x8& f, float s) {
#pragma unroll
  for (int i = 0; i < 8; ++i) s += f[i];
  return s;
}

// ---------------------------------------------------------------------------
// Key side.  Per unit (a chunk when causal, an L-split otherwise) and feature
// slice:  S[j][d] = sum_t phi(k_t)_j v_t[d]  and  z[j] = sum_t phi(k_t)_j.
// S is written as operand fragments of the query side (bf16 for bf16 inputs)
//   sdelta[bh][unit][db][fk][lane][8]: column d = 32 db + c of S,
//                                      feature 16 fk + 8 (e / 4) + 4g + e % 4,
// z in fp32, zdelta[bh][unit][j] (32 FB features).  Unfolded (or d_h not a
// multiple of 32): z is the column of ones beside V in the products; folded:
// the rounded features summed on the vector ALUs (the products are fewer, the
// registers tighter).
// Workgroup: 4 waves; a tile is 128 tokens; wave w projects token block w and
// publishes its rank-index fragments and shifts in LDS; then every wave maps
// its own FBW x 32 features over the whole tile.
// ---------------------------------------------------------------------------
// The key side's feature steps run as a software pipeline (see compute_tile)
// in the unfolded bf16 form with few accumulator and omega' registers; there
// the kernel is held to two workgroups per compute unit.  (Elsewhere the extra
// exponent registers cost occupancy or spills.)
template <typename T, int DH, int R16, int FBW> constexpr bool kstate_pipe() {
  return sizeof(T) == 2 && !fold_exponent(sizeof(T), DH, R16) &&
         FBW * vblocks_ones<DH>() * 16 + FBW * R16 * kParts<T> * 4 <= 112;
}
template <typename T, int DH, int R16, int FBW, bool PAD>
__global__ __launch_bounds__(kThreads, (kstate_pipe<T, DH, R16, FBW>() ? 2 : 1)) void kstate_kernel(
    FwdArgs a, Plan pl, const T* __restrict__ mfrag,
                                                           const T* __restrict__ ofrag, T* __restrict__ sdelta,
                                                           float* __restrict__ zdelta) {
  typedef typename FragOf<T>::type F;
  constexpr int KD = DH / 16;
  constexpr int NM = kParts<T>;
  constexpr int DB = vblocks<DH>();
  constexpr int TT = kTile;
  constexpr int VST = TT + 8;   // 16-byte aligned rows, an odd number of 16-byte units apart

  constexpr bool FOLD = fold_exponent(sizeof(T), DH, R16);
  constexpr int UK = FOLD ? KD : R16;              // K-steps of the exponent
  constexpr int UP = FOLD ? 1 : NM;                // parts of its token operand
  constexpr bool ZMMA = !FOLD || DH % 32 != 0;     // z from a column of ones in the products
  constexpr int DBK = ZMMA ? vblocks_ones<DH>() : DB;   // accumulator column blocks
  constexpr int MFR = ((R16 + 1) / 2) * KD * NM;   // fragments of M' (one head)
  constexpr bool M_LDS = MFR * 64 * 8 * sizeof(T) <= 32 * 1024;   // M' staged in LDS
  constexpr int VPT = vloads_per_thread<DH, TT>();
  // Double-buffered tile state (one barrier per tile; the next tile is
  // projected right behind the current tile's products) when it fits.
  // bf16: V in its row layout (transpose loads); fp32: V^T
  constexpr bool VTR = sizeof(T) == 2;
  constexpr int V_ELEMS = VTR ? TT * vsn<DH>() : DH * VST;
  constexpr size_t kTileState = (size_t)(kWaves * UP * UK * 64 * 8 + V_ELEMS) * sizeof(T) + TT * sizeof(float);
  constexpr int NBUF = 2 * kTileState + (M_LDS ? MFR * 64 * 8 * sizeof(T) : 0) <= 160 * 1024 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) T s_u[NBUF][kWaves][UP][UK][64 * 8];
  __shared__ __attribute__((aligned(16))) float s_init[NBUF][TT];
  __shared__ __attribute__((aligned(16))) T s_vt[NBUF][V_ELEMS];
  __shared__ __attribute__((aligned(16))) T s_m[M_LDS ? MFR * 64 * 8 : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  // workgroup: feature slice fslice of units u0 .. u0 + UPW - 1 of (b, h)
  const int lb = xcd_block();
  const int NUG = (pl.NU + pl.UPW - 1) / pl.UPW;
  const int fslice = lb % pl.NF;
  const int u0 = ((lb / pl.NF) % NUG) * pl.UPW;
  const int bh = lb / (pl.NF * NUG);
  const int b = bh / a.H, h = bh % a.H;
  const int hk = (h * a.H_kv) / a.H;
  const T* kbase = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
  const T* vbase = reinterpret_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
  const uint8_t* mrow = a.mask ? a.mask + (long)b * a.L : nullptr;
  const T* mf = mfrag + (long)(a.m_per_head ? h : 0) * ((R16 + 1) / 2) * KD * NM * 64 * 8;
  // omega' of this head's projection (or the shared one), or W' of its folded operand
  const T* of = ofrag + (long)((FOLD ? pl.HW : pl.HO) > 1 ? h : 0) * pl.FB * UK * 64 * 8;
  const float half_log2m = 0.5f * log2f((float)a.m);
  const int t_begin = u0 * pl.span1;   // the tiles of all the workgroup's units, in order
  const int t_end = min(a.L, min(u0 + pl.UPW, pl.NU) * pl.span1);
  const int fb0 = (fslice * kWaves + w) * FBW;     // first 32-feature block of this wave

  f32x16 acc[FBW][DBK];
#pragma unroll
  for (int f = 0; f < FBW; ++f)
#pragma unroll
    for (int db = 0; db < DBK; ++db) acc[f][db] = zero16();
  float zacc[FBW];   // (!ZMMA) this lane's part of z for feature 32 fb + c
#pragma unroll
  for (int f = 0; f < FBW; ++f) zacc[f] = 0.f;
  // omega' (W') fragments of this wave's features stay in registers when they are few
  constexpr bool kHoist = FBW * UK * kParts<T> <= (FOLD ? 32 : 8);
  F ohr[kHoist ? FBW : 1][UK];
  if constexpr (kHoist) {
#pragma unroll
    for (int f = 0; f < FBW; ++f) {
      const int fb = min(fb0 + f, pl.FB - 1);
#pragma unroll
      for (int k = 0; k < UK; ++k) ohr[f][k] = ld8(of + ((long)(fb * UK + k) * 64 + lane) * 8);
    }
  }

  // M' of this head in LDS when it is small (every token block of every tile
  // reads it): copied global -> LDS by the DMA path, 1 KB per wave instruction,
  // issued behind the first tile's K and V loads so that all are in flight
  // together; the caller waits for vmcnt(0) and a barrier.
  auto stage_m = [&]() {
    if constexpr (M_LDS) {
      constexpr int NKB = MFR * 64 * 8 * (int)sizeof(T) / 1024;
      for (int i = w; i < NKB; i += kWaves)
        dma16(reinterpret_cast<const char*>(mf) + i * 1024 + lane * 16, reinterpret_cast<char*>(s_m) + i * 1024);
    }
  };
  const T* msrc = M_LDS ? s_m : mf;
  // K rows of block w and the V rows of a tile are loaded one tile ahead of their use
  // (d_h = 256: no register prefetch, the registers go to the accumulators)
  constexpr bool PREF = KD + VPT <= 16;
  F xpre[KD], vpre[VPT];
  auto prefetch = [&](int tt) {
    const int t = tt + 32 * w + c;
    load_rows<T, DH>(xpre, kbase + (long)t * a.ks[2], t < t_end, g);
    load_v<T, DH, TT>(vpre, vbase, a.vs[2], tt, t_end, tid);
  };
  // projection of token block w of the tile at tt into buffer buf (rows from xpre)
  auto project_tile = [&](int tt, int buf, const T* msrc_t) {
    const int t = tt + 32 * w + c;
    const bool ok = t < t_end;
    float shift = 0.f;
    if constexpr (FOLD) {   // the exponent reads the token rows themselves, as fp16
      rows_to_h(xpre);
      if (!pl.kshift) shift = project_shift<T, DH, R16, true>(xpre, msrc_t, lane, half_log2m);
#pragma unroll
      for (int k = 0; k < UK; ++k) st8(&s_u[buf][w][0][k][lane * 8], xpre[k]);
    } else {
      F uhi[R16], ulo[R16];
      shift = project_block<T, DH, R16, kH16<T>>(uhi, ulo, xpre, msrc_t, lane, half_log2m);
#pragma unroll
      for (int k = 0; k < R16; ++k) {
        st8(&s_u[buf][w][0][k][lane * 8], uhi[k]);
        if constexpr (NM == 2 && !kH16<T>) st8(&s_u[buf][w][NM - 1][k][lane * 8], ulo[k]);
      }
    }
    const bool valid = ok && (mrow == nullptr || mrow[t] != 0);
    if (g == 0)
      s_init[buf][32 * w + c] = (FOLD && pl.kshift) ? (ok ? a.kshift[(long)bh * a.L + t] : -INFINITY)
                                                     : (valid ? -shift : -INFINITY);
    if constexpr (VTR) store_v<T, DH, TT>(s_vt[buf], vpre, tid);
    else store_vt<T, DH, TT, VST>(s_vt[buf], vpre, tid);
  };
  auto vfrag = [&](int buf, int db, int tb0, int k) -> F {
    if constexpr (VTR) return v_frag_tr<DH, ZMMA>(s_vt[buf], db, tb0, k, lane);
    else return v_frag<T, DH, VST, ZMMA>(s_vt[buf], db, tb0, k, c, g);
  };
  // the products of one tile from buffer buf, in (token block, feature block)
  // steps.  Pipelined (kstate_pipe), the exponent products of step s + 1 are
  // issued before the exp2 of step s, so that the matrix cores work on them
  // while the vector ALUs take the exponentials.
  auto compute_tile = [&](int buf, const T* of_t) {
    constexpr int NS = kWaves * FBW;
    constexpr bool PIPE = kstate_pipe<T, DH, R16, FBW>();
    auto exponent_of = [&](int s) -> f32x16 {
      const int tb = s / FBW, f = s % FBW;
      f32x16 e;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {   // rows 8 jj + 4g .. 8 jj + 4g + 3 are contiguous
        const float4 x = *reinterpret_cast<const float4*>(&s_init[buf][32 * tb + 8 * jj + 4 * g]);
        e[4 * jj] = x.x;
        e[4 * jj + 1] = x.y;
        e[4 * jj + 2] = x.z;
        e[4 * jj + 3] = x.w;
      }
      // a block past the last one (last slice only) runs on clamped operands
      // and is never stored: no branch in the loop
      const int fb = fb0 + f;
      const int fbc = min(fb, pl.FB - 1);
      auto uload = [&](int k, int part) -> F { return ld8(&s_u[buf][tb][part ? UP - 1 : 0][k][lane * 8]); };
      auto oload = [&](int k, int) -> F {   // omega' (W') has one part
        if constexpr (kHoist) return ohr[f][k];
        else return ld8(of_t + ((long)(fbc * UK + k) * 64 + lane) * 8);
      };
      if constexpr (PAD)   // m is not a multiple of 32: features past m give 0
        if (fb * 32 + c >= a.m) e = splat16(-INFINITY);
      return exponent_stream<T, UK, true, !FOLD, kH16<T>>(uload, oload, e);
    };
    // V (and ones) fragments of a token block: held across the feature blocks
    // when few, else read from LDS at each use
    constexpr bool VHOLD = DBK <= 4;
    F vf[VHOLD ? DBK : 1][2];
    f32x16 en;
    if constexpr (PIPE) en = exponent_of(0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int tb = s / FBW, f = s % FBW;
      // fp32: feature blocks past the last one are skipped (a wave-uniform
      // branch; on the bf16 path they run on clamped operands, no branch in
      // the loop)
      if constexpr (sizeof(T) == 4)
        if (fb0 + f >= pl.FB) continue;
      f32x16 e;
      if constexpr (PIPE) {
        e = en;
        if (s + 1 < NS) en = exponent_of(s + 1);
      } else {
        e = exponent_of(s);
      }
      if constexpr (VHOLD) {
        if (f == 0) {
#pragma unroll
          for (int db = 0; db < DBK; ++db)
#pragma unroll
            for (int k = 0; k < 2; ++k) vf[db][k] = vfrag(buf, db, 32 * tb, k);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = fast_exp2(e[i]);
      const F p0 = acc_frag<F>(e, 0), p1 = acc_frag<F>(e, 1);
      if constexpr (!ZMMA) zacc[f] = frag_sum(p1, frag_sum(p0, zacc[f]));
#pragma unroll
      for (int db = 0; db < DBK; ++db) {
        const F v0 = VHOLD ? vf[VHOLD ? db : 0][0] : vfrag(buf, db, 32 * tb, 0);
        const F v1 = VHOLD ? vf[VHOLD ? db : 0][1] : vfrag(buf, db, 32 * tb, 1);
        acc[f][db] = mma(p0, v0, acc[f][db]);
        acc[f][db] = mma(p1, v1, acc[f][db]);
      }
    }
  };
  // The omega' (W') and M' fragments are the same for every tile; hiding the
  // pointers from the optimiser keeps their loads in the loop instead of
  // hoisting all of them into registers (and spilling) before it.
  auto opaque = [&](const T* p, bool hide) {
    if (hide) asm volatile("" : "+s"(p));
    return p;
  };
  // ---- write this wave's part of the unit state (the accumulators are then
  // cleared for the workgroup's next unit) ----
  auto store_unit = [&](int unit) {
    const long FK = 2L * pl.FB;     // 16-feature fragments per d-block
    T* sd = sdelta + ((long)bh * pl.NU + unit) * DB * FK * 64 * 8;
    float* zd = zdelta + ((long)bh * pl.NU + unit) * pl.FB * 32;
#pragma unroll
    for (int f = 0; f < FBW; ++f) {
      const int fb = fb0 + f;
      if (fb < pl.FB) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int k = 0; k < 2; ++k)
            st8_state(sd + ((db * FK + 2 * fb + k) * 64 + lane) * 8, acc_frag<F>(acc[f][db], k), pl.stream_states);
        if constexpr (ZMMA) {   // column d_h: lane d_h % 32 of each half holds rows crow(i, g)
          if (c == DH % 32) {
#pragma unroll
            for (int i = 0; i < 16; ++i) zd[fb * 32 + crow(i, g)] = acc[f][DBK - 1][i];
          }
        } else {
          const float z = zacc[f] + __shfl_xor(zacc[f], 32);   // the two token halves
          if (g == 0) zd[fb * 32 + c] = z;
        }
      }
#pragma unroll
      for (int db = 0; db < DBK; ++db) acc[f][db] = zero16();
      zacc[f] = 0.f;
    }
  };
  // after the tile at t0: the unit ends there (units are whole tiles).  Only
  // the folded form takes several units per workgroup (the plan keeps one
  // otherwise); the others store their one unit after the loop, which keeps
  // the store's registers out of the loop.
  auto flush = [&](int t0) {
    if constexpr (FOLD)
      if (t0 + TT >= t_end || (t0 + TT - t_begin) % pl.span1 == 0) store_unit(u0 + (t0 - t_begin) / pl.span1);
  };
  if constexpr (NBUF == 2) {
    prefetch(t_begin);
    stage_m();
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the tile's rows and this wave's copies of M'
    __syncthreads();                      // M' in LDS
    project_tile(t_begin, 0, msrc);
    __syncthreads();
    int it = 0;
    for (int t0 = t_begin; t0 < t_end; t0 += TT, ++it) {
      const T* of_t = opaque(of, !kHoist);
      const T* msrc_t = opaque(msrc, !M_LDS);
      const bool more = t0 + TT < t_end;
      if (more) prefetch(t0 + TT);
      compute_tile(it & 1, of_t);
      if (more) project_tile(t0 + TT, (it + 1) & 1, msrc_t);
      flush(t0);
      __syncthreads();
    }
  } else {
    if constexpr (PREF) prefetch(t_begin);
    stage_m();
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();                      // M' in LDS
    for (int t0 = t_begin; t0 < t_end; t0 += TT) {
      const T* of_t = opaque(of, !kHoist);
      const T* msrc_t = opaque(msrc, !M_LDS);
      if constexpr (!PREF) prefetch(t0);
      project_tile(t0, 0, msrc_t);
      __syncthreads();
      if constexpr (PREF)
        if (t0 + TT < t_end) prefetch(t0 + TT);
      compute_tile(0, of_t);
      flush(t0);
      __syncthreads();
    }
  }
  if constexpr (!FOLD) store_unit(u0);
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
                                                               T* __restrict__ sdelta, float* __restrict__ zdelta) {
  typedef typename FragOf<T>::type F;
  constexpr int KD = DH / 16;
  constexpr int NM = kParts<T>;
  constexpr int DB = vblocks<DH>();
  constexpr int DBK = vblocks_ones<DH>();   // V and the column of ones (z)
  constexpr int R32 = (R16 + 1) / 2;
  constexpr int VST = 32 + 8;

  __shared__ __attribute__((aligned(16))) T s_u[NM][R16][64 * 8];
  __shared__ __attribute__((aligned(16))) float s_ss[kWaves][32];
  __shared__ __attribute__((aligned(16))) T s_vt[DH * VST];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int lb = xcd_block();
  const int fslice = lb % pl.NF;
  const int unit = (lb / pl.NF) % pl.NU;
  const int bh = lb / (pl.NF * pl.NU);
  const int b = bh / a.H, h = bh % a.H;
  const int hk = (h * a.H_kv) / a.H;
  const T* kbase = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
  const T* vbase = reinterpret_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
  const uint8_t* mrow = a.mask ? a.mask + (long)b * a.L : nullptr;
  const T* mf = mfrag + (long)(a.m_per_head ? h : 0) * R32 * KD * NM * 64 * 8;
  const T* of = ofrag + (long)(pl.HO > 1 ? h : 0) * pl.FB * R16 * 64 * 8;   // this head's omega'
  const float half_log2m = 0.5f * log2f((float)a.m);
  const int t_begin = unit * pl.span1;
  const int t_end = min(a.L, t_begin + pl.span1);
  const int fb0 = (fslice * kWaves + w) * FBW;

  f32x16 acc[FBW][DBK];
#pragma unroll
  for (int f = 0; f < FBW; ++f)
#pragma unroll
    for (int db = 0; db < DBK; ++db) acc[f][db] = zero16();

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
          u = m_product<T, false>(mf + ((rb * KD + kd) * NM * 64 + lane) * 8, xf[kd], u);
#pragma unroll
        for (int i = 0; i < 16; ++i) ss += u[i] * u[i];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          if (2 * rb + hh < R16) {
            if constexpr (kH16<T>) {   // the exponent's fp16 operand
              float v[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] = u[8 * hh + e];
              st8(&s_u[0][2 * rb + hh][lane * 8], make_frag_h(v));
            } else {
              F hi, lo;
              acc_frag_split<T>(u, hh, hi, lo);
              st8(&s_u[0][2 * rb + hh][lane * 8], hi);
              if constexpr (NM == 2) st8(&s_u[NM - 1][2 * rb + hh][lane * 8], lo);
            }
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
      if constexpr (!kH16<T>) ulo[k] = ld8(&s_u[NM - 1][k][lane * 8]);
    }
#pragma unroll
    for (int f = 0; f < FBW; ++f) {
      const int fb = fb0 + f;
      const int fbc = min(fb, pl.FB - 1);   // past the last block: clamped, never stored
      F ohi[R16];   // omega' has one part
#pragma unroll
      for (int k = 0; k < R16; ++k) ohi[k] = ld8(of + ((long)(fbc * R16 + k) * 64 + lane) * 8);
      f32x16 e = ini;
      if constexpr (PAD)
        if (fb * 32 + c >= a.m) e = splat16(-INFINITY);
      e = exponent<T, R16, true, true, kH16<T>>(uhi, ulo, ohi, ohi, e);
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = fast_exp2(e[i]);
      const F p0 = acc_frag<F>(e, 0), p1 = acc_frag<F>(e, 1);
#pragma unroll
      for (int db = 0; db < DBK; ++db) {
        acc[f][db] = mma(p0, v_frag<T, DH, VST, true>(s_vt, db, 0, 0, c, g), acc[f][db]);
        acc[f][db] = mma(p1, v_frag<T, DH, VST, true>(s_vt, db, 0, 1, c, g), acc[f][db]);
      }
    }
    __syncthreads();
  }

  const long FK = 2L * pl.FB;
  T* sd = sdelta + ((long)bh * pl.NU + unit) * DB * FK * 64 * 8;
  float* zd = zdelta + ((long)bh * pl.NU + unit) * pl.FB * 32;
#pragma unroll
  for (int f = 0; f < FBW; ++f) {
    const int fb = fb0 + f;
    if (fb >= pl.FB) continue;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int k = 0; k < 2; ++k)
        st8_state(sd + ((db * FK + 2 * fb + k) * 64 + lane) * 8, acc_frag<F>(acc[f][db], k), pl.stream_states);
    if (c == DH % 32) {   // column d_h: lane d_h % 32 of each half holds rows crow(i, g)
#pragma unroll
      for (int i = 0; i < 16; ++i) zd[fb * 32 + crow(i, g)] = acc[f][DBK - 1][i];
    }
  }
}

// ---------------------------------------------------------------------------
// State combination.  Non-causal: the sum over the L-splits.  Causal: the
// exclusive prefix over chunks (the state before each chunk) and, if asked, the
// state after the last token as S[b][h][j][d], z[b][h][j] (fp32).  Sums run in
// fp32; the per-unit S the query side reads is written in the operand order of
// the key side's output, z stays fp32.  One thread per fragment lane of S (8
// elements) or per feature of z.
// ---------------------------------------------------------------------------
template <typename T, int DH>
__global__ void scan_kernel(FwdArgs a, Plan pl, const T* __restrict__ sdelta, T* __restrict__ sfrag,
                            const float* __restrict__ zdelta, float* __restrict__ zsum) {
  typedef typename FragOf<T>::type F;
  constexpr int DB = vblocks<DH>();
  const long FK = 2L * pl.FB;
  const long per_unit = DB * FK * 64;          // fragment lanes per unit
  const long nS = (long)pl.BH * per_unit;
  const long z_unit = 32L * pl.FB;             // z values per unit
  const long nZ = (long)pl.BH * z_unit;
  const int nout = a.causal ? pl.NU : 1;
  constexpr int UB = 16;                       // units whose loads are in flight together
  // Work items in (b, h)-major order, S lanes then z values of each (b, h), and
  // blocks taken in XCD order: the (b, h) ranges that one XCD sums are the ones
  // its key side wrote and its query side reads (one L2).
  (void)nS;
  (void)nZ;
  const long per_bh = per_unit + z_unit;
  const long idx_all = (long)xcd_block() * blockDim.x + threadIdx.x;
  if (idx_all < (long)pl.BH * per_bh) {
    const long bh_i = idx_all / per_bh, r_i = idx_all % per_bh;
    const long idx = r_i < per_unit ? bh_i * per_unit + r_i : nS + bh_i * z_unit + (r_i - per_unit);
    if (idx >= nS) {   // z: one feature per thread
      const long zi = idx - nS;
      const long bh = zi / z_unit, j = zi % z_unit;
      const float* src = zdelta + bh * pl.NU * z_unit + j;
      float* dst = zsum + bh * nout * z_unit + j;
      float run = 0.f;
      for (int u = 0; u < pl.NU; u += UB) {
        const int nb = min(UB, pl.NU - u);
        float x[UB];
#pragma unroll
        for (int q = 0; q < UB; ++q) x[q] = src[(long)(u + min(q, nb - 1)) * z_unit];
#pragma unroll
        for (int q = 0; q < UB; ++q) {
          if (q >= nb) break;
          if (a.causal) dst[(long)(u + q) * z_unit] = run;
          run += x[q];
        }
      }
      if (!a.causal) dst[0] = run;
      if (a.z_out && j < a.m) a.z_out[bh * a.m + j] = run;
      return;
    }
    const long bh = idx / per_unit;
    const long rem = idx % per_unit;
    const T* src = sdelta + (bh * pl.NU * per_unit + rem) * 8;
    T* dst = sfrag + (bh * nout * per_unit + rem) * 8;
    float run[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int u = 0;
    for (; u + UB <= pl.NU; u += UB) {
      F x[UB];
#pragma unroll
      for (int q = 0; q < UB; ++q) x[q] = ld8_state<F>(src + (long)(u + q) * per_unit * 8, pl.stream_states);
#pragma unroll
      for (int q = 0; q < UB; ++q) {
        if (a.causal) {
          F o;
          make_frag(o, run);
          st8(dst + (long)(u + q) * per_unit * 8, o);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) run[e] += to_f32(x[q][e]);
      }
    }
    for (; u + 4 <= pl.NU; u += 4) {       // four loads in flight
      F x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = ld8_state<F>(src + (long)(u + q) * per_unit * 8, pl.stream_states);
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
      const F x = ld8_state<F>(src + (long)u * per_unit * 8, pl.stream_states);
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
    }
    if (a.S_out) {
      const int lane = (int)(rem & 63);
      const long frag = rem >> 6;
      const int fk = (int)(frag % FK), db = (int)(frag / FK);
      const int c = lane & 31, g = lane >> 5;
      const int d = db * 32 + c;
      if (d < DH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 16 * fk + 8 * (e >> 2) + 4 * g + (e & 3);
          if (j < a.m) a.S_out[(bh * a.m + j) * DH + d] = run[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Cross-attention: a context summary S [B][H][m][d_h], z [B][H][m] (fp32, from
// the caller) laid out as the query side's operands, in the order the sum over
// units writes them: fragment (d-block db, 16-feature half-block fk), lane
// (c, g), element e holds S[16 fk + 8 (e / 4) + 4 g + e % 4][32 db + c] (0 past
// m or d_h); z is padded with zeros to whole 32-feature blocks.
// ---------------------------------------------------------------------------
template <typename T, int DH>
__global__ void state_frag_kernel(FwdArgs a, Plan pl, T* __restrict__ sfrag, float* __restrict__ zsum) {
  typedef typename FragOf<T>::type F;
  constexpr int DB = vblocks<DH>();
  const long FK = 2L * pl.FB;
  const long per_unit = DB * FK * 64;
  const long nS = (long)pl.BH * per_unit;
  const long z_unit = 32L * pl.FB;
  const long nZ = (long)pl.BH * z_unit;
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < nS + nZ; idx += (long)gridDim.x * blockDim.x) {
    if (idx >= nS) {
      const long zi = idx - nS;
      const long bh = zi / z_unit, j = zi % z_unit;
      zsum[zi] = j < a.m ? a.z_in[bh * a.m + j] : 0.f;
      continue;
    }
    const long bh = idx / per_unit, rem = idx % per_unit;
    const int lane = (int)(rem & 63);
    const long frag = rem >> 6;
    const int fk = (int)(frag % FK), db = (int)(frag / FK);
    const int c = lane & 31, g = lane >> 5;
    const int d = db * 32 + c;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 16 * fk + 8 * (e >> 2) + 4 * g + (e & 3);
      x[e] = (d < DH && j < a.m) ? a.S_in[(bh * a.m + j) * DH + d] : 0.f;
    }
    F o;
    make_frag(o, x);
    st8(sfrag + idx * 8, o);
  }
}

// ---------------------------------------------------------------------------
// Query side.  Per (b, h) and tile of 128 NQB queries (a chunk when causal):
//   N = Phi(Q) S (+ tril(Phi(Q) Phi(K_chunk)^T) V when causal) on the matrix
//   cores, D = Phi(Q) z (fp32 features and z; + the row sums of the masked
//   scores as rounded for the products) on the vector ALUs, out = N / D
//   (0 if D == 0).
// Wave w owns query blocks w NQB .. w NQB + NQB - 1 of the tile; when causal,
// the keys at the same positions are mapped by the same wave and shared with
// the other waves through LDS, one 32-feature step at a time.
// ---------------------------------------------------------------------------
// Operand slots of one 32-feature step: omega' (W') fragments (one part), the
// state fragments, and one slot whose first 128 bytes hold the step's 32 z values.
template <typename T, int DH, int R16> constexpr int qout_nstep() {
  constexpr int UK = fold_exponent(sizeof(T), DH, R16) ? DH / 16 : R16;
  return UK + 2 * vblocks<DH>() + 1;
}
// Whether the causal query side can stage the operands of all ALLFB feature
// steps in LDS at once (bf16): V^T tile, all steps, double key-feature buffers.
constexpr int kAllFB = 8;
template <typename T, int DH, int R16, int ALLFB> constexpr bool qout_all_fits() {
  constexpr size_t vt = (size_t)DH * (128 + 8) * sizeof(T);
  constexpr size_t op = (size_t)ALLFB * qout_nstep<T, DH, R16>() * 64 * 8 * sizeof(T);
  constexpr size_t kf = 2 * 4 * 2 * 64 * 8 * sizeof(T);
  return sizeof(T) == 2 && vt + op + kf <= 160 * 1024;
}

// Largest number of waves per SIMD the compiler schedules the query side for:
// two where each wave reads its operands from L2 itself (non-causal, few
// operand slots).  Left free, the compiler aims at three waves there and, to
// fit their registers, waits for each operand load before issuing the next
// (L=64K query side 213 against 150 us).
template <typename T, int DH, int R16, bool CAUSAL, int ALLFB> constexpr int qout_max_waves() {
  return (!CAUSAL && ALLFB == 0 && qout_nstep<T, DH, R16>() <= 8) ? 2 : 8;
}
template <typename T, int DH, int R16, int NQB, bool CAUSAL, bool PAD, int ALLFB = 0>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, qout_max_waves<T, DH, R16, CAUSAL, ALLFB>())))
void qout_kernel(FwdArgs a, Plan pl, const T* __restrict__ mfrag,
                                                        const T* __restrict__ ofrag, const T* __restrict__ sfrag,
                                                        const float* __restrict__ zsum) {
  typedef typename FragOf<T>::type F;
  constexpr int KD = DH / 16;
  constexpr int NM = kParts<T>;
  constexpr int DB = vblocks<DH>();
  constexpr int NB = kWaves * NQB;         // 32-token blocks per tile
  constexpr int TT = 32 * NB;              // tokens per tile
  constexpr int VST = TT + 8;
  constexpr bool FOLD = fold_exponent(sizeof(T), DH, R16);
  constexpr int UK = FOLD ? KD : R16;      // K-steps of the exponent
  constexpr int NOF = UK;                  // omega' (W') fragments per feature step (one part)
  constexpr int NSTEP = qout_nstep<T, DH, R16>();
  constexpr int ZS = NSTEP - 1;            // the z slot
  constexpr int ZW = 8 * (int)sizeof(T) / 4;   // z values per lane of a slot copy
  static_assert(NSTEP == NOF + 2 * DB + 1, "step layout");
  constexpr int PERW = (NSTEP + kWaves - 1) / kWaves;
  constexpr int VT_ELEMS = CAUSAL ? DH * VST : 8;
  constexpr size_t kBase = (size_t)VT_ELEMS * sizeof(T);
  constexpr size_t kOpStep = (size_t)NSTEP * 64 * 8 * sizeof(T);
  constexpr size_t kKfStep = CAUSAL ? (size_t)NB * 2 * 64 * 8 * sizeof(T) : 0;
  // Operands staged in LDS when one step buffer fits beside the V^T tile (else
  // each wave reads them from L2 itself); double buffers (one barrier per
  // feature step) unless LDS is short.
  // Non-causal with few operands per step (at most 8 slots): no staging and no
  // barrier per step, each wave reads them from L2 itself (L=64K, 16-rank
  // geometry: 150 against 155 us; a register prefetch one step ahead, 152).
  constexpr bool SELF = !CAUSAL && ALLFB == 0 && NSTEP <= 8;
  static_assert(SELF == (qout_max_waves<T, DH, R16, CAUSAL, ALLFB>() == 2), "wave bound of the unstaged form");
  constexpr bool STAGE = !SELF && kBase + kOpStep + kKfStep <= 160 * 1024;
  constexpr int OPB = !STAGE ? 0 : kBase + 2 * kOpStep + 2 * kKfStep <= 160 * 1024 ? 2 : 1;
  constexpr int KBUF = kBase + OPB * kOpStep + 2 * kKfStep <= 160 * 1024 ? 2 : 1;
  constexpr int KF_ELEMS = CAUSAL ? KBUF * NB * 2 * 64 * 8 : 8;
  // ALLFB > 0 (bf16, at most ALLFB feature blocks): the operands of every step
  // are copied global -> LDS by the DMA path at the start, overlapping the
  // projections, and the step loop has no staging and no extra barriers.
  constexpr bool ALL = ALLFB > 0;
  static_assert(!ALL || sizeof(T) == 2, "all-step staging: bf16");
  constexpr int OP_ELEMS = ALL ? ALLFB * NSTEP * 64 * 8 : STAGE ? OPB * NSTEP * 64 * 8 : 8;

  __shared__ __attribute__((aligned(16))) T s_vt[VT_ELEMS];
  __shared__ __attribute__((aligned(16))) T s_kf[KF_ELEMS];
  __shared__ __attribute__((aligned(16))) T s_op[OP_ELEMS];
  // SELF: the 32 FB values of z in LDS (dynamic, FB * 32 floats), copied by
  // DMA at the start: per step the waves read them from LDS instead of
  // requesting them from L2 (L=64K forward 0.261 -> 0.259 ms, same device)
  extern __shared__ __attribute__((aligned(16))) float s_zall[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, c = lane & 31, g = lane >> 5;
  const int w = tid >> 6;
  const int lb = xcd_block();
  const int tile = lb % pl.NT2;
  const int bh = lb / pl.NT2;
  const int b = bh / a.H, h = bh % a.H;
  const int hk = (h * a.H_kv) / a.H;
  const T* qbase = reinterpret_cast<const T*>(a.q) + b * a.qs[0] + h * a.qs[1];
  const T* kbase = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
  const T* vbase = reinterpret_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
  T* obase = reinterpret_cast<T*>(a.out) + b * a.os[0] + h * a.os[1];
  const uint8_t* mrow = a.mask ? a.mask + (long)b * a.L : nullptr;
  const T* mf = mfrag + (long)(a.m_per_head ? h : 0) * ((R16 + 1) / 2) * KD * NM * 64 * 8;
  const T* of = ofrag + (long)((FOLD ? pl.HW : pl.HO) > 1 ? h : 0) * pl.FB * UK * 64 * 8;
  const float half_log2m = 0.5f * log2f((float)a.m);
  const int t0 = tile * TT;
  const long FK = 2L * pl.FB;
  const long unit_s = (long)bh * (CAUSAL ? pl.NU : 1) + (CAUSAL ? tile : 0);
  const T* sf = sfrag + unit_s * DB * FK * 64 * 8;
  const float* zs = zsum + unit_s * pl.FB * 32;
  if constexpr (SELF) {   // 1 KB per wave instruction, 16 bytes per lane, lanes past FB * 32 values idle
    for (int i = w; i * 256 < pl.FB * 32; i += kWaves)
      if (i * 256 + 4 * lane < pl.FB * 32) dma16(zs + i * 256 + 4 * lane, s_zall + i * 256);
  }

  // Operands of one 32-feature step are the same for the four waves.  The z
  // slot: lanes 0 .. 32 / ZW - 1 copy the 32 values (the others repeat the last
  // part, inside the slot).
  auto gsrc = [&](int fb, int f) -> const T* {
    if (f < NOF) return of + ((long)(fb * UK + f) * 64 + lane) * 8;
    if (f == ZS) return reinterpret_cast<const T*>(zs + fb * 32 + min(lane, 32 / ZW - 1) * ZW);
    f -= NOF;
    return sf + (((f >> 1) * FK + 2 * fb + (f & 1)) * 64 + lane) * 8;
  };
  // All-step staging: the step operands, and M' (in the key-feature buffers,
  // free until the first step), go to LDS by DMA before anything else is loaded.
  constexpr int MFRG = ((R16 + 1) / 2) * KD * NM;
  constexpr bool M_LDS = ALL && CAUSAL && MFRG * 64 * 8 <= KF_ELEMS;
  if constexpr (ALL) {
    for (int idx = w; idx < pl.FB * NSTEP; idx += kWaves) {
      const int fb = idx / NSTEP, f = idx - fb * NSTEP;
      dma16(gsrc(fb, f), s_op + idx * 64 * 8);
    }
    if constexpr (M_LDS)
      for (int idx = w; idx < MFRG; idx += kWaves)
        dma16(mf + ((long)idx * 64 + lane) * 8, s_kf + idx * 64 * 8);
  }

  // ---- exponent operands of this wave's query (and key) blocks: u = M' x as
  // hi/lo fragments, or (folded) the token rows x themselves.  Rows and the
  // V tile are requested first, the projections run once they are in.  The
  // queries need no |u|^2 / 2: any factor per query row cancels in N / D, and
  // the exponent of query t is shifted by shq, its largest exponent over the
  // first 32 features (set before the first feature step). ----
  F uqh[NQB][UK], uql[NQB][FOLD ? 1 : UK];
  float shq[NQB];
  F ukh[CAUSAL ? NQB : 1][UK], ukl[CAUSAL ? NQB : 1][FOLD ? 1 : UK];
  float initk[CAUSAL ? NQB : 1];
  F xq[FOLD ? 1 : NQB][KD], xk[(FOLD || !CAUSAL) ? 1 : NQB][KD];
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const int t = t0 + 32 * (w * NQB + j) + c;
    const bool ok = t < a.L;
    F* xr = FOLD ? uqh[j] : xq[FOLD ? 0 : j];
    load_rows<T, DH>(*reinterpret_cast<F(*)[KD]>(xr), qbase + (long)t * a.qs[2], ok, g);
    if constexpr (CAUSAL) {
      F* kr = FOLD ? ukh[j] : xk[FOLD ? 0 : j];
      load_rows<T, DH>(*reinterpret_cast<F(*)[KD]>(kr), kbase + (long)t * a.ks[2], ok, g);
    }
  }
  constexpr int VPT = vloads_per_thread<DH, TT>();
  F vr[CAUSAL ? VPT : 1];
  if constexpr (CAUSAL) load_v<T, DH, TT>(vr, vbase, a.vs[2], t0, a.L, tid);
  if constexpr (ALL) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies have landed
  if constexpr (CAUSAL) store_vt<T, DH, TT, VST>(s_vt, vr, tid);
  if constexpr (M_LDS) __syncthreads();   // M' (and every wave's copies) visible
  const T* msrc = M_LDS ? s_kf : mf;
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const int t = t0 + 32 * (w * NQB + j) + c;
    const bool ok = t < a.L;
    shq[j] = 0.f;
    if constexpr (FOLD && kH16<T>) {   // the token rows as fp16 operands of the projection and exponent
      rows_to_h(*reinterpret_cast<F(*)[KD]>(uqh[j]));
      if constexpr (CAUSAL) rows_to_h(*reinterpret_cast<F(*)[KD]>(ukh[j]));
    }
    if constexpr (!FOLD)
      (void)project_block<T, DH, R16, kH16<T>>(*reinterpret_cast<F(*)[R16]>(uqh[j]),
                                               *reinterpret_cast<F(*)[R16]>(uql[j]), xq[FOLD ? 0 : j], msrc, lane,
                                               half_log2m);
    if constexpr (CAUSAL) {
      float sh = 0.f;
      if (FOLD && pl.kshift) {
        initk[j] = ok ? a.kshift[(long)bh * a.L + t] : -INFINITY;
      } else {
        if constexpr (FOLD)
          sh = project_shift<T, DH, R16, true>(*reinterpret_cast<F(*)[KD]>(ukh[j]), msrc, lane, half_log2m);
        else
          sh = project_block<T, DH, R16, kH16<T>>(*reinterpret_cast<F(*)[R16]>(ukh[j]),
                                                  *reinterpret_cast<F(*)[R16]>(ukl[j]), xk[FOLD ? 0 : j], msrc, lane,
                                                  half_log2m);
        const bool valid = ok && (mrow == nullptr || mrow[t] != 0);
        initk[j] = valid ? -sh : -INFINITY;
      }
    }
  }

  f32x16 acc[NQB][DB];
  float den[NQB];   // this lane's part of D for query c of block j
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    den[j] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[j][db] = zero16();
  }
  f32x16 at[CAUSAL ? NQB : 1][CAUSAL ? NB : 1];   // A^T[key block][query block of the wave]
  if constexpr (CAUSAL) {
#pragma unroll
    for (int j = 0; j < NQB; ++j)
#pragma unroll
      for (int kb2 = 0; kb2 < NB; ++kb2) at[j][kb2] = zero16();
  }

  // Ring staging: each wave fetches a quarter of a step's operands from L2
  // one step ahead, and all read them from LDS.
  F pre[STAGE && !ALL ? PERW : 1];
  auto load_step = [&](int fb) {
    if constexpr (STAGE && !ALL) {
#pragma unroll
      for (int q = 0; q < PERW; ++q) {
        const int f = w + kWaves * q;
        if (f < NSTEP) pre[q] = ld8(gsrc(fb, f));
      }
    }
  };
  auto store_step = [&](int buf) {
    if constexpr (STAGE && !ALL) {
#pragma unroll
      for (int q = 0; q < PERW; ++q) {
        const int f = w + kWaves * q;
        if (f < NSTEP) st8(s_op + ((buf * NSTEP + f) * 64 + lane) * 8, pre[q]);
      }
    }
  };
  auto op = [&](int fb, int buf, int f) {
    if constexpr (ALL) return ld8(s_op + ((fb * NSTEP + f) * 64 + lane) * 8);
    else if constexpr (STAGE) return ld8(s_op + ((buf * NSTEP + f) * 64 + lane) * 8);
    else return ld8(gsrc(fb, f));
  };
  // z of features 32 fb + 8 jj + 4 g .. + 3 (the rows this lane holds)
  auto zrow4 = [&](int fb, int buf, int jj) -> float4 {
    const float* zb;
    if constexpr (ALL) zb = reinterpret_cast<const float*>(s_op + (fb * NSTEP + ZS) * 64 * 8);
    else if constexpr (STAGE) zb = reinterpret_cast<const float*>(s_op + (buf * NSTEP + ZS) * 64 * 8);
    else if constexpr (SELF) zb = s_zall + fb * 32;
    else zb = zs + fb * 32;   // operands too large to stage: each wave reads z from L2 itself
    return *reinterpret_cast<const float4*>(zb + 8 * jj + 4 * g);
  };

  // shq[j]: the largest exponent of query block j's rows over the first 32
  // features (lanes c and c + 32 hold the two halves of query c's features);
  // the first block always holds at least 16 real features
  auto set_query_shift = [&](int buf) {
    auto oload = [&](int k, int) -> F { return op(0, buf, k); };
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      f32x16 e = zero16();
      if constexpr (PAD) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (crow(i, g) >= a.m) e[i] = -INFINITY;
      }
      if constexpr (FOLD)
        e = exponent_stream<T, UK, false, false, kH16<T>>([&](int k, int) -> F { return uqh[j][k]; }, oload, e);
      else
        e = exponent_stream<T, UK, false, true, kH16<T>>(
            [&](int k, int part) -> F { return part ? uql[j][k] : uqh[j][k]; }, oload, e);
      float mx = e[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, e[i]);
      shq[j] = fmaxf(mx, __shfl_xor(mx, 32));
    }
  };
  // one 32-feature step; the operands of the next step are fetched before it runs
  auto step = [&](int fb, int buf) {
    auto oload = [&](int k, int) -> F { return op(fb, buf, k); };
    // Unfolded: omega' fragments of the step read once into registers and
    // shared by the query and key blocks.  (Fetching them per use with the fp32
    // 32x32x2 products gave a schedule whose first launch in a process
    // returned wrong blocks now and then.)
    F ohi[FOLD ? 1 : UK];
    if constexpr (!FOLD) {
#pragma unroll
      for (int k = 0; k < UK; ++k) ohi[k] = op(fb, buf, k);
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
      if constexpr (FOLD)
        e = exponent_stream<T, UK, false, false, kH16<T>>([&](int k, int) -> F { return uqh[j][k]; }, oload, e);
      else
        e = exponent<T, UK, false, true, kH16<T>>(uqh[j], uql[j], ohi, ohi, e);
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = fast_exp2(e[i]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {   // D += phi(q) . z
        const float4 z = zrow4(fb, buf, jj);
        den[j] += e[4 * jj] * z.x + e[4 * jj + 1] * z.y + e[4 * jj + 2] * z.z + e[4 * jj + 3] * z.w;
      }
      pq[j][0] = acc_frag<F>(e, 0);
      pq[j][1] = acc_frag<F>(e, 1);
    }
    // inter-chunk (or whole-sequence) state; with many column blocks the
    // fragments are read in groups of three blocks (bounded registers)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const F sv = op(fb, buf, NOF + 2 * db + k);
#pragma unroll
        for (int j = 0; j < NQB; ++j) acc[j][db] = mma(pq[j][k], sv, acc[j][db]);
      }
      if constexpr (DB > 4)
        if (db % 3 == 2) __builtin_amdgcn_sched_barrier(0);
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
        if constexpr (FOLD)
          e = exponent_stream<T, UK, false, false, kH16<T>>([&](int k, int) -> F { return ukh[j][k]; }, oload, e);
        else
          e = exponent<T, UK, false, true, kH16<T>>(ukh[j], ukl[j], ohi, ohi, e);
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
  // Many operands per step (d_h = 256): no register prefetch across the step,
  // the registers go to the accumulators; the copy runs between steps.
  constexpr bool EARLY = PERW <= 8;
  if constexpr (ALL) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies have landed
    __syncthreads();                      // and everyone else's
    set_query_shift(0);
    for (int fb = 0; fb < pl.FB; ++fb) step(fb, 0);
  } else {
    load_step(0);
    store_step(0);
    if constexpr (SELF) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of z have landed
    __syncthreads();
    set_query_shift(0);
    for (int fb = 0; fb < pl.FB; ++fb) {
      const int buf = OPB == 2 ? (fb & 1) : 0;
      if constexpr (EARLY)
        if (fb + 1 < pl.FB) load_step(fb + 1);
      step(fb, buf);
      if constexpr (STAGE) {
        if (fb + 1 < pl.FB) {
          if constexpr (OPB == 1) __syncthreads();   // one buffer: everyone is done reading it
          if constexpr (!EARLY) load_step(fb + 1);
          store_step(OPB == 2 ? ((fb + 1) & 1) : 0);
        }
        __syncthreads();
      }
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
          den[j] = frag_sum(pf, den[j]);   // the rounded scores the products use
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[j][db] = mma(pf, v_frag<T, DH, VST>(s_vt, db, 32 * kb2, k, c, g), acc[j][db]);
        }
      }
    }
  }

  // ---- out = N / D; lanes c and c + 32 hold the two halves of D for query c ----
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const int blk = w * NQB + j;
    const float dq = den[j] + __shfl_xor(den[j], 32);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float dd = __shfl(dq, crow(i, g));
      const int t = t0 + 32 * blk + crow(i, g);
      // a masked query row (cross-attention) gives 0
      const bool qvalid = a.qmask == nullptr || (t < a.L && a.qmask[(long)b * a.L + t] != 0);
      const float inv = (dd > 0.f && qvalid) ? __builtin_amdgcn_rcpf(dd) : 0.f;
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
// Causal query side with eight waves per workgroup (bf16, every step's
// operands staged in LDS at once).  The same sums as qout_kernel, with the
// feature steps split in two halves: waves w and w + 4 both own query block
// w % 4 (and key block w % 4 of the chunk); wave w takes the first half of the
// 32-feature steps, wave w + 4 the second.  N and D are sums over features, so
// each half forms its own part of Phi(Q) S, of the masked scores
// Phi(Q) Phi(K_chunk)^T and of their products with V, and the two parts are
// added at the end through LDS.  Both halves shift their queries by the same
// value (the largest exponent over the first 32 features, from the first
// step's operands).  Two waves per SIMD let one wave's exp and LDS latencies
// overlap the other's matrix products.
// ---------------------------------------------------------------------------
constexpr int kWaves8 = 2 * kWaves;
constexpr int kThreads8 = 64 * kWaves8;
template <typename T, int DH, int R16, int ALLFB> constexpr bool qout8_fits() {
  constexpr size_t vt = (size_t)DH * (128 + 8) * sizeof(T);
  constexpr size_t op = (size_t)ALLFB * qout_nstep<T, DH, R16>() * 64 * 8 * sizeof(T);
  constexpr size_t kf = 2 * 2 * kWaves * 2 * 64 * 8 * sizeof(T);
  constexpr size_t xch = (size_t)kWaves * (vblocks<DH>() * 16 + 1) * 64 * sizeof(float);   // the halves' hand-over
  constexpr size_t ost = (size_t)kWaves * 32 * (DH + 8) * sizeof(T);                      // output staging
  return sizeof(T) == 2 && vt + op + kf <= 160 * 1024 && xch <= op && (ost <= kf || ost <= vt);
}
template <typename T, int DH, int R16, bool PAD, int ALLFB>
__global__ __launch_bounds__(kThreads8) void qout8_kernel(FwdArgs a, Plan pl, const T* __restrict__ mfrag,
                                                          const T* __restrict__ ofrag, const T* __restrict__ sfrag,
                                                          const float* __restrict__ zsum) {
  typedef typename FragOf<T>::type F;
  static_assert(sizeof(T) == 2, "bf16 only");
  constexpr int KD = DH / 16;
  constexpr int NM = kParts<T>;
  constexpr int DB = vblocks<DH>();
  constexpr int NB = kWaves;               // 32-token blocks per chunk
  constexpr int TT = 32 * NB;              // tokens per chunk
  constexpr int VST = TT + 8;
  constexpr bool FOLD = fold_exponent(sizeof(T), DH, R16);
  constexpr int UK = FOLD ? KD : R16;      // K-steps of the exponent
  constexpr int NOF = UK;                  // omega' (W') fragments per feature step (one part)
  constexpr int NSTEP = qout_nstep<T, DH, R16>();
  constexpr int ZS = NSTEP - 1;            // the z slot
  constexpr int ZW = 8 * (int)sizeof(T) / 4;
  constexpr int VT_ELEMS = DH * VST;
  constexpr int KFH = 2 * NB * 2 * 64 * 8;   // key-feature buffers of one half (two)
  constexpr int KF_ELEMS = 2 * KFH;
  constexpr int OP_ELEMS = ALLFB * NSTEP * 64 * 8;
  static_assert(qout8_fits<T, DH, R16, ALLFB>(), "LDS");
  __shared__ __attribute__((aligned(16))) T s_vt[VT_ELEMS];
  __shared__ __attribute__((aligned(16))) T s_kf[KF_ELEMS];
  __shared__ __attribute__((aligned(16))) T s_op[OP_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, c = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Waves w and w + 4 share a SIMD.  The causal products grow with the query
  // block (block qb visits qb + 1 key blocks), so the second half takes the
  // blocks in reverse order and every SIMD gets one block of each weight.
  const int half = w / NB;
  const int qb = half == 0 ? (w & (NB - 1)) : NB - 1 - (w & (NB - 1));
  const int lb = xcd_block();
  const int tile = lb % pl.NT2;
  const int bh = lb / pl.NT2;
  const int b = bh / a.H, h = bh % a.H;
  const int hk = (h * a.H_kv) / a.H;
  const T* qbase = reinterpret_cast<const T*>(a.q) + b * a.qs[0] + h * a.qs[1];
  const T* kbase = reinterpret_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
  const T* vbase = reinterpret_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
  T* obase = reinterpret_cast<T*>(a.out) + b * a.os[0] + h * a.os[1];
  const uint8_t* mrow = a.mask ? a.mask + (long)b * a.L : nullptr;
  const T* mf = mfrag + (long)(a.m_per_head ? h : 0) * ((R16 + 1) / 2) * KD * NM * 64 * 8;
  const T* of = ofrag + (long)((FOLD ? pl.HW : pl.HO) > 1 ? h : 0) * pl.FB * UK * 64 * 8;
  const float half_log2m = 0.5f * log2f((float)a.m);
  const int t0 = tile * TT;
  const long FK = 2L * pl.FB;
  const long unit_s = (long)bh * pl.NU + tile;
  const T* sf = sfrag + unit_s * DB * FK * 64 * 8;
  const float* zs = zsum + unit_s * pl.FB * 32;

  // step operands as in qout_kernel: W' (omega') fragments, state fragments, z slot
  auto gsrc = [&](int fb, int f) -> const T* {
    if (f < NOF) return of + ((long)(fb * UK + f) * 64 + lane) * 8;
    if (f == ZS) return reinterpret_cast<const T*>(zs + fb * 32 + min(lane, 32 / ZW - 1) * ZW);
    f -= NOF;
    return sf + (((f >> 1) * FK + 2 * fb + (f & 1)) * 64 + lane) * 8;
  };
  // M' (in the key-feature buffers, free until the first step) and the
  // operands of each half's first step (steps 0 and nit) go to LDS by DMA
  // before the rows are loaded.  The other steps' operands are requested into
  // registers last, PL per wave (a fixed count, so that one explicit counter
  // wait covers everything before them), and written to LDS during the first
  // step: their loads overlap the projections and the first step.
  constexpr int MFRG = ((R16 + 1) / 2) * KD * NM;
  constexpr bool M_LDS = MFRG * 64 * 8 <= KF_ELEMS;
  const int nit = (pl.FB + 1) >> 1;   // steps per half (the second half may have one fewer)
  const int nE = pl.FB > 1 ? 2 : 1;   // early steps: 0 and nit
  const int nLate = (pl.FB - nE) * NSTEP;
  constexpr int PL = ((ALLFB - 2) * NSTEP + kWaves8 - 1) / kWaves8;   // late slots per wave
  static_assert(PL <= 15, "one vmcnt immediate");
  auto late_slot = [&](int l, int& fb, int& f) {   // late slot l: step fb, slot f
    const int j = l / NSTEP;
    f = l - j * NSTEP;
    fb = j < nit - 1 ? 1 + j : nit + 1 + (j - (nit - 1));
  };
  if constexpr (M_LDS)
    for (int idx = w; idx < MFRG; idx += kWaves8) dma16(mf + ((long)idx * 64 + lane) * 8, s_kf + idx * 64 * 8);
  for (int idx = w; idx < nE * NSTEP; idx += kWaves8) {
    const int fb = idx < NSTEP ? 0 : nit, f = idx < NSTEP ? idx : idx - NSTEP;
    dma16(gsrc(fb, f), s_op + (fb * NSTEP + f) * 64 * 8);
  }

  // ---- exponent operands of query block qb and key block qb ----
  const int t = t0 + 32 * qb + c;
  const bool ok = t < a.L;
  F uqh[UK], uql[FOLD ? 1 : UK];
  F ukh[UK], ukl[FOLD ? 1 : UK];
  F xq[FOLD ? 1 : KD], xk[FOLD ? 1 : KD];
  load_rows<T, DH>(*reinterpret_cast<F(*)[KD]>(FOLD ? uqh : xq), qbase + (long)t * a.qs[2], ok, g);
  load_rows<T, DH>(*reinterpret_cast<F(*)[KD]>(FOLD ? ukh : xk), kbase + (long)t * a.ks[2], ok, g);
  constexpr int VPT = vloads_per_thread<DH, TT, kThreads8>();
  F vr[VPT];
  load_v<T, DH, TT, kThreads8>(vr, vbase, a.vs[2], t0, a.L, tid);
  // the key's shift (precomputed) or mask byte, read only once the
  // projections need it (a select here would wait for the load at once)
  float initk = -INFINITY;
  int kmask = 1;
  if (FOLD && pl.kshift) {
    if (ok) initk = a.kshift[(long)bh * a.L + t];
  } else if (mrow != nullptr && ok) {
    kmask = mrow[t];
  }
  // the late steps' operands: PL requests per wave, the ones past the last
  // slot from slot 0's address and never stored
  F late[PL];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < PL; ++p) {
    const int l = w + kWaves8 * p;
    int fb = 0, f = 0;
    if (l < nLate) late_slot(l, fb, f);
    late[p] = ld8(gsrc(fb, f));
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70 | PL);   // vmcnt(PL): rows, V and this wave's copies (not the late requests)
  __builtin_amdgcn_sched_barrier(0);
  store_vt<T, DH, TT, VST, kThreads8>(s_vt, vr, tid);
  __syncthreads();                      // M', V^T and every wave's copies visible
  const T* msrc = M_LDS ? s_kf : mf;
  if constexpr (FOLD && kH16<T>) {   // the token rows as fp16 operands of the projection and exponent
    rows_to_h(*reinterpret_cast<F(*)[KD]>(uqh));
    rows_to_h(*reinterpret_cast<F(*)[KD]>(ukh));
  }
  if constexpr (!FOLD)
    (void)project_block<T, DH, R16, kH16<T>>(*reinterpret_cast<F(*)[R16]>(uqh), *reinterpret_cast<F(*)[R16]>(uql),
                                             xq, msrc, lane, half_log2m);
  if (!(FOLD && pl.kshift)) {
    float sh;
    if constexpr (FOLD)
      sh = project_shift<T, DH, R16, true>(*reinterpret_cast<F(*)[KD]>(ukh), msrc, lane, half_log2m);
    else
      sh = project_block<T, DH, R16, kH16<T>>(*reinterpret_cast<F(*)[R16]>(ukh), *reinterpret_cast<F(*)[R16]>(ukl),
                                              xk, msrc, lane, half_log2m);
    initk = (ok && kmask != 0) ? -sh : -INFINITY;
  }

  auto op = [&](int fb, int f) { return ld8(s_op + ((fb * NSTEP + f) * 64 + lane) * 8); };
  auto zrow4 = [&](int fb, int jj) -> float4 {
    const float* zb = reinterpret_cast<const float*>(s_op + (fb * NSTEP + ZS) * 64 * 8);
    return *reinterpret_cast<const float4*>(zb + 8 * jj + 4 * g);
  };
  // the query shift: largest exponent of query c over the first 32 features
  float shq;
  {
    auto oload = [&](int k, int) -> F { return op(0, k); };
    f32x16 e = zero16();
    if constexpr (PAD) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (crow(i, g) >= a.m) e[i] = -INFINITY;
    }
    if constexpr (FOLD)
      e = exponent_stream<T, UK, false, false, kH16<T>>([&](int k, int) -> F { return uqh[k]; }, oload, e);
    else
      e = exponent_stream<T, UK, false, true, kH16<T>>(
          [&](int k, int part) -> F { return part ? uql[k] : uqh[k]; }, oload, e);
    float mx = e[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, e[i]);
    shq = fmaxf(mx, __shfl_xor(mx, 32));
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero16();
  float den = 0.f;
  f32x16 at[NB];   // A^T[key block][query block qb], this half's features
  // every wave's projections are done reading M' from the key-feature buffers
  // before the first step writes key features there
  if constexpr (M_LDS) __syncthreads();
#pragma unroll
  for (int kb2 = 0; kb2 < NB; ++kb2) at[kb2] = zero16();

  for (int it = 0; it < nit; ++it) {
    const int fb = half * nit + it;
    const bool live = fb < pl.FB;
    T* kbuf = s_kf + half * KFH + (it & 1) * NB * 2 * 64 * 8;
    F pq[2];
    if (live) {
      auto oload = [&](int k, int) -> F { return op(fb, k); };
      F ohi[FOLD ? 1 : UK];
      if constexpr (!FOLD) {
#pragma unroll
        for (int k = 0; k < UK; ++k) ohi[k] = op(fb, k);
      }
      const bool partial = PAD && (fb + 1) * 32 > a.m;
      {
        f32x16 e = splat16(-shq);
        if (partial) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (fb * 32 + crow(i, g) >= a.m) e[i] = -INFINITY;
        }
        if constexpr (FOLD)
          e = exponent_stream<T, UK, false, false, kH16<T>>([&](int k, int) -> F { return uqh[k]; }, oload, e);
        else
          e = exponent<T, UK, false, true, kH16<T>>(uqh, uql, ohi, ohi, e);
#pragma unroll
        for (int i = 0; i < 16; ++i) e[i] = fast_exp2(e[i]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {   // D += phi(q) . z
          const float4 z = zrow4(fb, jj);
          den += e[4 * jj] * z.x + e[4 * jj + 1] * z.y + e[4 * jj + 2] * z.z + e[4 * jj + 3] * z.w;
        }
        pq[0] = acc_frag<F>(e, 0);
        pq[1] = acc_frag<F>(e, 1);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int k = 0; k < 2; ++k) acc[db] = mma(pq[k], op(fb, NOF + 2 * db + k), acc[db]);
      {
        f32x16 e = splat16(initk);
        if (partial) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (fb * 32 + crow(i, g) >= a.m) e[i] = -INFINITY;
        }
        if constexpr (FOLD)
          e = exponent_stream<T, UK, false, false, kH16<T>>([&](int k, int) -> F { return ukh[k]; }, oload, e);
        else
          e = exponent<T, UK, false, true, kH16<T>>(ukh, ukl, ohi, ohi, e);
#pragma unroll
        for (int i = 0; i < 16; ++i) e[i] = fast_exp2(e[i]);
#pragma unroll
        for (int k = 0; k < 2; ++k) st8(kbuf + ((qb * 2 + k) * 64 + lane) * 8, acc_frag<F>(e, k));
      }
    }
    if (it == 0) {   // the late steps' operands, read from the next step on
#pragma unroll
      for (int p = 0; p < PL; ++p) {
        const int l = w + kWaves8 * p;
        if (l < nLate) {
          int fb2, f2;
          late_slot(l, fb2, f2);
          st8(s_op + ((fb2 * NSTEP + f2) * 64 + lane) * 8, late[p]);
        }
      }
    }
    __syncthreads();   // this step's key features of the half's four blocks (and the late operands) are in
    if (live) {
#pragma unroll
      for (int kb2 = 0; kb2 < NB; ++kb2)
        if (kb2 <= qb)
#pragma unroll
          for (int k = 0; k < 2; ++k) at[kb2] = mma(ld8(kbuf + ((kb2 * 2 + k) * 64 + lane) * 8), pq[k], at[kb2]);
    }
  }

  // intra-chunk part with this half's scores: key R(i, g) of the diagonal block
  // is visible to query c iff R(i, g) <= c
#pragma unroll
  for (int kb2 = 0; kb2 < NB; ++kb2) {
    if (kb2 > qb) continue;
    if (kb2 == qb) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (crow(i, g) > c) at[kb2][i] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const F pf = acc_frag<F>(at[kb2], k);
      den = frag_sum(pf, den);   // the rounded scores the products use
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = mma(pf, v_frag<T, DH, VST>(s_vt, db, 32 * kb2, k, c, g), acc[db]);
    }
  }

  // ---- the second half's N and D added to the first's through LDS; out = N / D
  // staged per wave and stored as 16-byte pieces of whole rows ----
  constexpr int XW = DB * 16 + 1;   // floats per lane handed over
  static_assert((size_t)kWaves * XW * 64 * sizeof(float) <= (size_t)OP_ELEMS * sizeof(T), "exchange buffer");
  constexpr int OST = DH + 8;
  constexpr bool OST_KF = kWaves * 32 * OST <= KF_ELEMS;   // else the V^T tile's buffer (d_h >= 128)
  static_assert(OST_KF || kWaves * 32 * OST <= VT_ELEMS, "output staging buffer");
  float* xch = reinterpret_cast<float*>(s_op) + qb * XW * 64;
  // (no barrier needed first: the step operands in s_op were last read before
  // the last key-feature barrier, which every wave has passed)
  if (half == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) xch[(db * 16 + i) * 64 + lane] = acc[db][i];
    xch[DB * 16 * 64 + lane] = den;
  }
  __syncthreads();   // the hand-over is in; s_kf and s_vt are no longer read
  if (half == 1) return;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] += xch[(db * 16 + i) * 64 + lane];
  den += xch[DB * 16 * 64 + lane];
  T* const ostage = (OST_KF ? s_kf : s_vt) + qb * 32 * OST;
  const float dq = den + __shfl_xor(den, 32);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float dd = __shfl(dq, crow(i, g));
    const float inv = dd > 0.f ? __builtin_amdgcn_rcpf(dd) : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = db * 32 + c;
      if (d < DH) store_out(ostage + crow(i, g) * OST + d, acc[db][i] * inv);
    }
  }
  constexpr int CPR = DH / 8;   // 16-byte pieces per row
#pragma unroll
  for (int q = lane; q < 32 * CPR; q += 64) {
    const int row = q / CPR, col = (q - row * CPR) * 8;
    const int tr = t0 + 32 * qb + row;
    if (tr < a.L)
      *reinterpret_cast<uint4*>(obase + (long)tr * a.os[2] + col) = *reinterpret_cast<const uint4*>(ostage + row * OST + col);
  }
}

// ---------------------------------------------------------------------------
// Host launch of one forward call for (T, DH, R16).
// ---------------------------------------------------------------------------
constexpr size_t kMaxLds = 160 * 1024;
// LDS of the tiled key-side kernel: exponent operands of four blocks, shifts,
// the V^T tile and (when small) M'
template <typename T, int DH, int R16> constexpr size_t kstate_tile_lds_bytes() {
  constexpr bool FOLD = fold_exponent(sizeof(T), DH, R16);
  constexpr int UK = FOLD ? DH / 16 : R16;
  constexpr int UP = FOLD ? 1 : kParts<T>;
  constexpr size_t mbytes = (size_t)((R16 + 1) / 2) * (DH / 16) * kParts<T> * 64 * 8 * sizeof(T);
  constexpr size_t v_elems = sizeof(T) == 2 ? (size_t)kTile * vsn<DH>() : (size_t)DH * (kTile + 8);
  return (size_t)(kWaves * UP * UK * 64 * 8 + v_elems) * sizeof(T) + kTile * sizeof(float) +
         (mbytes <= 32 * 1024 ? mbytes : 16);
}
// Least LDS of the causal query-side kernel: the V^T tile and one key-feature
// buffer (the operand staging buffers are added only where they fit).
template <typename T, int DH, int R16, int NQB> constexpr size_t causal_lds_bytes() {
  return (size_t)(DH * (128 * NQB + 8) + 4 * NQB * 2 * 64 * 8) * sizeof(T);
}

template <typename T, int DH, int R16, int FBW, bool PAD>
dark_status launch_fwd_pad(const FwdArgs& a_in, const Plan& pl, void* ws, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(ws);
  FwdArgs a = a_in;
  a.kshift = pl.kshift ? reinterpret_cast<float*>(base + pl.off_kshift) : nullptr;
  T* mfrag = reinterpret_cast<T*>(base + pl.off_mfrag);
  T* ofrag = reinterpret_cast<T*>(base + pl.off_ofrag);
  T* sdelta = reinterpret_cast<T*>(base + pl.off_sdelta);
  T* sfrag = reinterpret_cast<T*>(base + pl.off_sfrag);
  float* zdelta = reinterpret_cast<float*>(base + pl.off_zdelta);
  float* zsum = reinterpret_cast<float*>(base + pl.off_zsum);
  // Non-causal with one key-side unit per (b, h) and no exported state (short
  // sequences, such as the tiny fp32 workload): the sum over units is that
  // unit's state, in the same layout, so the query side reads it where the key
  // side wrote it and the sum's launch is left out.
  const bool one_unit = pl.mode == kPlanForward && !a.causal && pl.NU == 1 && a.S_out == nullptr &&
                        a.z_out == nullptr;
  if (one_unit) {
    sfrag = sdelta;
    zsum = zdelta;
  }
  constexpr int NM = kParts<T>;
  {
    // Folded with d_h >= 32: W' by matrix products and M' in one launch;
    // otherwise M' and omega' (or a d_h = 16 W') elementwise.
    const int fmode = !pl.fold ? 0 : (DH >= 32 ? 2 : 1);
    const float s = powf((float)DH, -0.25f);
    const long nM = (long)pl.HM * ((R16 + 1) / 2) * (DH / 16) * NM * 64;
    KernelTimer tm(kPrep, stream);
    if (fmode == 2) {
      if constexpr (sizeof(T) == 2 && DH >= 32) {
        const int nW = pl.HW * pl.FB * ((DH / 32 + 3) / 4);
        hipLaunchKernelGGL(fold_kernel<T>, dim3(nW + (int)((nM + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                           a.M, a.omega, ofrag, mfrag, pl.HM, pl.HO, pl.HW, R16, a.r, DH, a.m, pl.FB, s,
                           kLog2e * s);
      }
    } else {
      const long n = nM + (fmode ? (long)pl.HW * pl.FB * (DH / 16) * 64 : (long)pl.HO * pl.FB * R16 * 64);
      const int blocks = (int)((n + 255) / 256);
      hipLaunchKernelGGL(prep_kernel<T>, dim3(blocks), dim3(256), 0, st, a.M, a.omega, mfrag, ofrag, pl.HM, pl.HO,
                         pl.HW, a.r, DH, a.m, R16, pl.FB, s, fmode);
    }
  }
  if (pl.mode == kPlanCross) {   // the caller's summary as the query side's operands
    const long n = (long)pl.BH * vblocks<DH>() * 2 * pl.FB * 64 + (long)pl.BH * pl.FB * 32;
    KernelTimer tm(kScan, stream);
    hipLaunchKernelGGL((state_frag_kernel<T, DH>), dim3((int)((n + 255) / 256)), dim3(256), 0, st, a, pl, sfrag, zsum);
  }
  if (pl.kshift) {
    const int ntile = (a.L + shift_tile<T>() - 1) / shift_tile<T>();
    KernelTimer tm(kShift, stream);
    hipLaunchKernelGGL((shift_kernel<T, DH, R16>), dim3(pl.BH * ntile), dim3(kThreads), 0, st, a, mfrag,
                       a.kshift);
  }
  if (pl.mode != kPlanCross) {
    KernelTimer tm(kKState, stream);
    const dim3 grid1(pl.BH * pl.NU * pl.NF);
    static_assert(!fold_exponent(sizeof(T), DH, R16) || kstate_tile_lds_bytes<T, DH, R16>() <= kMaxLds,
                  "the folded key side runs on the tiled kernel");
    if constexpr (kstate_tile_lds_bytes<T, DH, R16>() <= kMaxLds)
      hipLaunchKernelGGL((kstate_kernel<T, DH, R16, FBW, PAD>), dim3(pl.BH * ((pl.NU + pl.UPW - 1) / pl.UPW) * pl.NF),
                         dim3(kThreads), 0, st, a, pl, mfrag, ofrag, sdelta, zdelta);
    else
      hipLaunchKernelGGL((kstate_seq_kernel<T, DH, R16, FBW, PAD>), grid1, dim3(kThreads), 0, st, a, pl, mfrag,
                         ofrag, sdelta, zdelta);
  }
  if (pl.mode != kPlanCross && !one_unit) {
    const long n = (long)pl.BH * vblocks<DH>() * 2 * pl.FB * 64 + (long)pl.BH * pl.FB * 32;   // S lanes, z values
    const int blocks = (int)((n + 255) / 256);
    KernelTimer tm(kScan, stream);
    hipLaunchKernelGGL((scan_kernel<T, DH>), dim3(blocks), dim3(256), 0, st, a, pl, sdelta, sfrag, zdelta, zsum);
  }
  if (pl.mode == kPlanContext) return hipGetLastError() == hipSuccess ? DARK_OK : DARK_ERR_HIP;
  const dim3 grid(pl.BH * pl.NT2);
  KernelTimer tm(kQOut, stream);
  if (a.causal) {
    if constexpr (causal_lds_bytes<T, DH, R16, 1>() <= kMaxLds) {
      if (pl.NQB != 1) return DARK_ERR_UNSUPPORTED;
      if constexpr (qout_all_fits<T, DH, R16, kAllFB>()) {   // few feature blocks: all steps staged at once
        if (pl.FB <= kAllFB) {
          if constexpr (!PAD && qout8_fits<T, DH, R16, kAllFB>())   // eight waves, feature steps in two halves
            hipLaunchKernelGGL((qout8_kernel<T, DH, R16, PAD, kAllFB>), grid, dim3(kThreads8), 0, st, a, pl, mfrag,
                               ofrag, sfrag, zsum);
          else
            hipLaunchKernelGGL((qout_kernel<T, DH, R16, 1, true, PAD, kAllFB>), grid, dim3(kThreads), 0, st, a, pl,
                               mfrag, ofrag, sfrag, zsum);
          return hipGetLastError() == hipSuccess ? DARK_OK : DARK_ERR_HIP;
        }
      }
      hipLaunchKernelGGL((qout_kernel<T, DH, R16, 1, true, PAD>), grid, dim3(kThreads), 0, st, a, pl, mfrag, ofrag,
                         sfrag, zsum);
    } else {
      return DARK_ERR_UNSUPPORTED;
    }
  } else {
    // the unstaged non-causal form keeps z in dynamic LDS
    const size_t zlds = qout_max_waves<T, DH, R16, false, 0>() == 2 ? (size_t)pl.FB * 32 * sizeof(float) : 0;
    switch (pl.NQB) {
      case 1: hipLaunchKernelGGL((qout_kernel<T, DH, R16, 1, false, PAD>), grid, dim3(kThreads), zlds, st, a, pl, mfrag, ofrag, sfrag, zsum); break;
      case 2:
        if constexpr (DH <= 128) {   // the planner takes two query blocks per wave only for d_h <= 64
          hipLaunchKernelGGL((qout_kernel<T, DH, R16, 2, false, PAD>), grid, dim3(kThreads), zlds, st, a, pl, mfrag,
                             ofrag, sfrag, zsum);
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

// ---------------------------------------------------------------------------
// Exact learned-kernel attention (README section "Attention modes": the exact
// path applies the learned geometry to q and k and then runs softmax
// attention):  out_t = sum_j softmax_j(u_t . u_j) v_j over the visible valid
// keys j, with u = d_h^(-1/4) M_h x for queries and keys alike.
//
// Workspace: the M' fragments, then ufrag[tensor][b h][32-token block][R16]
// [lane][8]: the operand fragments of u for q (tensor 0) and for k as seen by
// query head h (tensor 1), in the order project_block leaves them (the same for
// both, so the score sum runs over the same rank permutation).  On the bf16
// path u is rounded once to fp16 (11 significant bits, clamped to +-65504) and
// each score K-step is one fp16 product, as in the feature exponent.
// ---------------------------------------------------------------------------
// M' = d_h^(-1/4) M in fragment order (the projection operand).
template <typename T>
__global__ void mfrag_kernel(const float* __restrict__ M, T* __restrict__ mfrag, long n, int r, int d_h, int R16,
                             float s) {
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < n; idx += (long)gridDim.x * blockDim.x)
    mfrag_lane<T>(idx, M, mfrag, r, d_h, R16, s, true);
}

// u of every 32-token block of q and of k (one wave per block).
template <typename T, int DH, int R16>
__global__ __launch_bounds__(kThreads) void exact_proj_kernel(FwdArgs a, const T* __restrict__ mfrag,
                                                               T* __restrict__ ufrag, int NBLK) {
  typedef typename FragOf<T>::type F;
  constexpr int KD = DH / 16;
  constexpr int NM = kParts<T>;
  constexpr int R32 = (R16 + 1) / 2;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 31, g = lane >> 5;
  const int BH = a.B * a.H;
  const int per = (NBLK + kWaves - 1) / kWaves;
  const int tensor = blockIdx.x / (BH * per);   // 0: queries, 1: keys
  const int rem = blockIdx.x % (BH * per);
  const int bh = rem / per, blk = (rem % per) * kWaves + w;
  if (blk >= NBLK) return;
  const int b = bh / a.H, h = bh % a.H, hk = (h * a.H_kv) / a.H;
  const T* base = tensor == 0 ? reinterpret_cast<const T*>(a.q) + b * a.qs[0] + h * a.qs[1]
                              : reinterpret_cast<const T*>(a.k) + b * a.ks[0] + hk * a.ks[1];
  const int64_t stride = tensor == 0 ? a.qs[2] : a.ks[2];
  const int t = blk * 32 + c;
  F xf[KD];
  load_rows<T, DH>(xf, base + (long)t * stride, t < a.L, g);
  if constexpr (kH16<T>) rows_to_h(xf);
  const T* mf = mfrag + (long)(a.m_per_head ? h : 0) * R32 * KD * NM * 64 * 8;
  F uhi[R16], ulo[R16];   // one part: fp16 on the bf16 path (as the feature exponent), fp32 otherwise
  (void)project_block<T, DH, R16, kH16<T>, true>(uhi, ulo, xf, mf, lane, 0.f);
  T* dst = ufrag + (((long)tensor * BH + bh) * NBLK + blk) * R16 * 64 * 8;
#pragma unroll
  for (int kr = 0; kr < R16; ++kr) st8(dst + (kr * 64 + lane) * 8, uhi[kr]);
}

// Softmax attention on the projected rows.  Workgroup: 128 queries of one (b,
// h), wave w owning the 32-query block 4 tile + w; the keys go by in tiles of
// 128 (V staged transposed in LDS, with an additive 0 / -inf key bias from the
// mask and the sequence end).  Pass 1 finds each query's score maximum over
// its visible keys; pass 2 forms p = exp(s - max) rounded to the operand type,
// the row sums of the rounded weights and the products p V.  Scores are
// computed in transposed form (rows = keys, columns = queries), so a lane holds
// one query and its maximum and sum need no cross-lane reduction but one
// exchange between the two lane halves.
// With KS > 0 the keys of a query tile are split into runs of KS key tiles,
// one workgroup each: the workgroup writes its partial maximum m_s, weight sum
// l_s and unnormalised product O_s per query to `part` (exact_combine_kernel
// then forms the softmax over all runs); with KS == 0 one workgroup takes all
// of a tile's keys and writes out directly.
template <typename T, int DH, int R16, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void exact_kernel(FwdArgs a, const T* __restrict__ ufrag, int NBLK, int KS,
                                                          float* __restrict__ part) {
  typedef typename FragOf<T>::type F;
  constexpr int DB = vblocks<DH>();
  constexpr int TT = kTile;
  constexpr int VST = TT + 8;
  constexpr int VPT = vloads_per_thread<DH, TT>();
  constexpr int UFR = R16 * 64 * 8;   // elements of one block's u fragments (one part)
  // ranks up to 64: a key tile's u fragments are staged in LDS beside V^T (the
  // next tile's fetched into registers during the current one); above, every
  // wave reads them from L2
  constexpr bool KLDS = R16 <= 4 && (size_t)(DH * VST + kWaves * UFR) * sizeof(T) + TT * 4 <= 160 * 1024;
  constexpr int KCH = KLDS ? kWaves * UFR / 8 / kThreads : 1;   // 16-byte pieces per thread and tile
  __shared__ __attribute__((aligned(16))) T s_vt[DH * VST];
  __shared__ __attribute__((aligned(16))) float s_bias[TT];
  __shared__ __attribute__((aligned(16))) T s_uk[KLDS ? kWaves * UFR : 8];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c = lane & 31, g = lane >> 5;
  const int NT = (a.L + TT - 1) / TT;
  const int lb = xcd_block();
  int tile, bh, split = 0, kt0 = 0, kt1;
  long pidx = 0;   // (b h, tile, split) index of this workgroup's partial
  if (KS == 0) {
    tile = CAUSAL ? NT - 1 - lb % NT : lb % NT;   // causal: the longest tiles first
    bh = lb / NT;
    kt1 = CAUSAL ? tile + 1 : NT;
  } else {   // runs of KS = kExactKS key tiles: tile t has ceil(n_t / KS), n_t = t + 1 (causal) or NT
    constexpr int KSC = kExactKS;
    const int nsplit_nc = (NT + KSC - 1) / KSC;
    int per_head = 0;
    for (int t = 0; t < NT; ++t) per_head += CAUSAL ? t / KSC + 1 : nsplit_nc;
    bh = lb / per_head;
    int r0 = lb % per_head;
    tile = 0;
    for (;; ++tile) {
      const int ns = CAUSAL ? tile / KSC + 1 : nsplit_nc;
      if (r0 < ns) break;
      r0 -= ns;
    }
    split = r0;
    pidx = (long)lb;
    kt0 = split * KSC;
    kt1 = min(kt0 + KSC, CAUSAL ? tile + 1 : NT);
  }
  const int b = bh / a.H, h = bh % a.H, hk = (h * a.H_kv) / a.H;
  const int BH = a.B * a.H;
  const int qb = tile * kWaves + w;                     // this wave's query block
  const T* uq = ufrag + ((long)bh * NBLK + min(qb, NBLK - 1)) * UFR;
  const T* uk0 = ufrag + ((long)BH + bh) * NBLK * UFR;
  const uint8_t* mrow = a.mask ? a.mask + (long)b * a.L : nullptr;
  const T* vbase = reinterpret_cast<const T*>(a.v) + b * a.vs[0] + hk * a.vs[1];
  // ranks up to 64: the query block's u fragments stay in registers; above,
  // both operands of the score products stream from memory (L1)
  constexpr bool QREG = R16 <= 4;
  F qh[QREG ? R16 : 1];
  if constexpr (QREG) {
#pragma unroll
    for (int kr = 0; kr < R16; ++kr) qh[kr] = ld8(uq + (kr * 64 + lane) * 8);
  }
  const int tiles = kt1;                                // key tiles kt0 .. kt1 - 1
  // last key block this wave uses (a block past the sequence end holds no query
  // that is stored; it still reads only blocks of this sequence)
  const int kb_last = min(CAUSAL ? qb : NBLK - 1, NBLK - 1);
  // the u fragments of key tile kt: registers, then LDS (blocks past the
  // sequence end are read clamped and never used)
  F kreg[KCH];
  auto fetch_k = [&](int kt) {
    if constexpr (KLDS) {
#pragma unroll
      for (int p = 0; p < KCH; ++p) {
        const int e = tid + p * kThreads;                 // 16-byte piece of the tile
        const int kbl = e / (UFR / 8), within = e % (UFR / 8);
        const int kb = min(kt * kWaves + kbl, NBLK - 1);
        kreg[p] = ld8(uk0 + (long)kb * UFR + within * 8);
      }
    }
  };
  auto put_k = [&]() {
    if constexpr (KLDS) {
#pragma unroll
      for (int p = 0; p < KCH; ++p) st8(s_uk + (tid + p * kThreads) * 8, kreg[p]);
    }
  };
  // scores of key block kb (rows = keys, columns = queries), biased and masked
  auto scores = [&](int kb, int kbl) -> f32x16 {
    const T* uk = KLDS ? s_uk + kbl * UFR : uk0 + (long)kb * UFR;
    f32x16 s;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {   // rows 8 jj + 4g .. 8 jj + 4g + 3 are contiguous
      const float4 x = *reinterpret_cast<const float4*>(&s_bias[32 * kbl + 8 * jj + 4 * g]);
      s[4 * jj] = x.x;
      s[4 * jj + 1] = x.y;
      s[4 * jj + 2] = x.z;
      s[4 * jj + 3] = x.w;
    }
    // one-part operands: one fp16 product per K-step on the bf16 path
    auto kload = [&](int k, int) -> F { return ld8(uk + (k * 64 + lane) * 8); };
    if constexpr (QREG) {
      F kh[R16];
#pragma unroll
      for (int kr = 0; kr < R16; ++kr) kh[kr] = kload(kr, 0);
      s = exponent<T, R16, true, true, kH16<T>>(kh, kh, qh, qh, s);
    } else {
      auto qload = [&](int k, int) -> F { return ld8(uq + (k * 64 + lane) * 8); };
      s = exponent_stream<T, R16, true, true, kH16<T>>(kload, qload, s);
    }
    if (CAUSAL && kb == qb) {   // the diagonal block: key crow(i, g) visible to query c iff crow <= c
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (crow(i, g) > c) s[i] = -INFINITY;
    }
    return s;
  };
  auto put_bias = [&](int t0) {
    if (tid < TT) {
      const int j = t0 + tid;
      s_bias[tid] = (j < a.L && (mrow == nullptr || mrow[j] != 0)) ? 0.f : -INFINITY;
    }
  };
  // ---- pass 1: the score maximum of each query ----
  float mx = -INFINITY;
  fetch_k(kt0);
  for (int kt = kt0; kt < tiles; ++kt) {
    put_bias(kt * TT);
    put_k();
    __syncthreads();
    fetch_k(kt + 1 < tiles ? kt + 1 : kt0);   // pass 2 starts again at the first tile
#pragma unroll 1
    for (int kbl = 0; kbl < kWaves; ++kbl) {
      const int kb = kt * kWaves + kbl;
      if (kb > kb_last) break;
      const f32x16 s = scores(kb, kbl);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    }
    __syncthreads();
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mL = mx == -INFINITY ? 0.f : mx * kLog2e;   // no visible key: every weight is 0
  // ---- pass 2: weights, their sums and the products with V ----
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = zero16();
  float den = 0.f;
  F vr[VPT];
  load_v<T, DH, TT>(vr, vbase, a.vs[2], kt0 * TT, a.L, tid);
  for (int kt = kt0; kt < tiles; ++kt) {
    store_vt<T, DH, TT, VST>(s_vt, vr, tid);
    put_bias(kt * TT);
    put_k();
    __syncthreads();
    if (kt + 1 < tiles) {
      load_v<T, DH, TT>(vr, vbase, a.vs[2], (kt + 1) * TT, a.L, tid);
      fetch_k(kt + 1);
    }
#pragma unroll 1
    for (int kbl = 0; kbl < kWaves; ++kbl) {
      const int kb = kt * kWaves + kbl;
      if (kb > kb_last) break;
      f32x16 s = scores(kb, kbl);
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = fast_exp2(s[i] * kLog2e - mL);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const F pf = acc_frag<F>(s, k);
        den = frag_sum(pf, den);   // the rounded weights the products use
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = mma(pf, v_frag<T, DH, VST>(s_vt, db, 32 * kbl, k, c, g), acc[db]);
      }
    }
    __syncthreads();
  }
  // ---- out = (p V) / sum p; lanes c and c + 32 hold the two halves of the sum ----
  T* obase = reinterpret_cast<T*>(a.out) + b * a.os[0] + h * a.os[1];
  const float dq = den + __shfl_xor(den, 32);
  if (KS > 0) {   // partial: O_s [128][d_h], then m_s and l_s [128] per workgroup
    float* po = part + pidx * (long)(TT * DH + 2 * TT);
    float* pm = po + TT * DH;
    if (g == 0) {
      pm[32 * w + c] = mx;
      pm[TT + 32 * w + c] = dq;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 32 + c;
        if (d < DH) po[(32 * w + crow(i, g)) * DH + d] = acc[db][i];
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float dd = __shfl(dq, crow(i, g));
    const int t = qb * 32 + crow(i, g);
    const float inv = dd > 0.f ? __builtin_amdgcn_rcpf(dd) : 0.f;
    if (t < a.L) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 32 + c;
        if (d < DH) store_out(obase + (long)t * a.os[2] + d, acc[db][i] * inv);
      }
    }
  }
}

// Softmax over the runs: out = sum_s O_s e^(m_s - m) / sum_s l_s e^(m_s - m),
// m = max_s m_s (0 when no run saw a visible key).  One thread per query and
// 4 columns.
template <typename T, int DH, bool CAUSAL>
__global__ void exact_combine_kernel(FwdArgs a, const float* __restrict__ part) {
  constexpr int TT = kTile;
  constexpr int KS = kExactKS;
  const int NT = (a.L + TT - 1) / TT;
  const int nsplit_nc = (NT + KS - 1) / KS;
  const long n = (long)a.B * a.H * a.L * (DH / 4);
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < n; idx += (long)gridDim.x * blockDim.x) {
    const int d4 = (int)(idx % (DH / 4));
    const long row = idx / (DH / 4);
    const int t = (int)(row % a.L);
    const int bh = (int)(row / a.L);
    const int tile = t / TT, q = t % TT;
    // first partial of (bh, tile): the same order as the workgroups
    int per_head = 0, before = 0;
    for (int u = 0; u < NT; ++u) {
      const int ns = CAUSAL ? u / KS + 1 : nsplit_nc;
      if (u < tile) before += ns;
      per_head += ns;
    }
    const int ns = CAUSAL ? tile / KS + 1 : nsplit_nc;
    const float* p0 = part + ((long)bh * per_head + before) * (long)(TT * DH + 2 * TT);
    float m = -INFINITY;
    for (int sp = 0; sp < ns; ++sp) m = fmaxf(m, p0[sp * (long)(TT * DH + 2 * TT) + TT * DH + q]);
    float num[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
    if (m != -INFINITY) {
      for (int sp = 0; sp < ns; ++sp) {
        const float* ps = p0 + sp * (long)(TT * DH + 2 * TT);
        const float ms = ps[TT * DH + q];
        if (ms == -INFINITY) continue;
        const float wgt = exp2f((ms - m) * kLog2e);
        den += ps[TT * DH + TT + q] * wgt;
#pragma unroll
        for (int e = 0; e < 4; ++e) num[e] += ps[q * DH + 4 * d4 + e] * wgt;
      }
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    const int b = bh / a.H, h = bh % a.H;
    T* o = reinterpret_cast<T*>(a.out) + b * a.os[0] + h * a.os[1] + (long)t * a.os[2] + 4 * d4;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out(o + e, num[e] * inv);
  }
}

template <typename T, int DH, int R16>
dark_status launch_exact_impl(const FwdArgs& a, void* ws, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int HM = a.m_per_head ? a.H : 1;
  const ExactLayout lay = exact_layout(a.B, a.H, a.L, DH, R16, HM, (int)sizeof(T), a.causal);
  char* base = reinterpret_cast<char*>(ws);
  T* mfrag = reinterpret_cast<T*>(base + lay.off_mfrag);
  T* ufrag = reinterpret_cast<T*>(base + lay.off_ufrag);
  const long nM = (long)HM * ((R16 + 1) / 2) * (DH / 16) * kParts<T> * 64;
  {
    KernelTimer tm(kPrep, stream);
    hipLaunchKernelGGL(mfrag_kernel<T>, dim3((int)((nM + 255) / 256)), dim3(256), 0, st, a.M, mfrag, nM, a.r, DH,
                       R16, powf((float)DH, -0.25f));
  }
  {
    KernelTimer tm(kShift, stream);
    const int per = (lay.NBLK + kWaves - 1) / kWaves;
    hipLaunchKernelGGL((exact_proj_kernel<T, DH, R16>), dim3(2 * a.B * a.H * per), dim3(kThreads), 0, st, a, mfrag,
                       ufrag, lay.NBLK);
  }
  float* part = reinterpret_cast<float*>(base + lay.off_part);
  const int NT = (a.L + kTile - 1) / kTile;
  const int KS = lay.KS;
  {
    KernelTimer tm(kQOut, stream);
    const dim3 grid(KS == 0 ? a.B * a.H * NT : a.B * a.H * lay.splits_per_head);
    if (a.causal)
      hipLaunchKernelGGL((exact_kernel<T, DH, R16, true>), grid, dim3(kThreads), 0, st, a, ufrag, lay.NBLK, KS, part);
    else
      hipLaunchKernelGGL((exact_kernel<T, DH, R16, false>), grid, dim3(kThreads), 0, st, a, ufrag, lay.NBLK, KS,
                         part);
  }
  if (KS > 0) {
    KernelTimer tm(kScan, stream);
    const long n = (long)a.B * a.H * a.L * (DH / 4);
    const int blocks = (int)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
    if (a.causal)
      hipLaunchKernelGGL((exact_combine_kernel<T, DH, true>), dim3(blocks), dim3(256), 0, st, a, part);
    else
      hipLaunchKernelGGL((exact_combine_kernel<T, DH, false>), dim3(blocks), dim3(256), 0, st, a, part);
  }
  return hipGetLastError() == hipSuccess ? DARK_OK : DARK_ERR_HIP;
}

}  // namespace dk
