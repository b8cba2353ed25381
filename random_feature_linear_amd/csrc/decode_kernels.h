// One-token recurrent decode step (package README "Data-Aware Random Feature
// Kernels for Transformers (DARKformer)", section "Encoder-decoder model and
// generation": recurrent self-attention statistics updated per appended token).
//
// For every sequence n and query head h, with the feature map of section
// "Kernel":  S += phi(k) v^T,  z += phi(k),  out = phi(q)^T S / phi(q)^T z.
// The step is bound by streaming the fp32 state S (m x d_h per (n, h)) through
// HBM once in each direction; the feature maps are small fp32 VALU dot
// products (a rank-one update per sequence leaves no dense contraction for the
// matrix cores).
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.h"

namespace dk {

constexpr float kLog2eDec = 1.4426950408889634f;

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int64_t qs[2], ks[2], vs[2], os[2];   // strides over (n, h)
  const float* M;
  const float* omega;
  float* S;
  float* z;
  const uint8_t* qmask;   // read-only pass: query mask [N] (nonzero = valid), or null
  int N, H, H_kv, m, r, m_per_head, omega_per_head, NS;
};

__device__ __forceinline__ float ld_elem(const __bf16* p, int i) { return (float)p[i]; }
__device__ __forceinline__ float ld_elem(const float* p, int i) { return p[i]; }
__device__ __forceinline__ void st_elem(__bf16* p, int i, float x) { p[i] = (__bf16)x; }
__device__ __forceinline__ void st_elem(float* p, int i, float x) { p[i] = x; }

// Workgroup: 256 threads, one query head h, NS consecutive sequences.  The
// state is streamed in slices of 256 x kDecVec float4 per sequence: a thread
// owns the columns d0 .. d0 + 3 (d0 = 4 (tid % (DH / 4))) of rows
// j = tid / (DH / 4) + i 256 / (DH / 4).  All loads of a slice are issued
// before any of its stores.  The first slice is requested after the
// projections u (their M rows are loaded first: vector-memory loads complete
// in order) and before the feature exponents, so its HBM latency overlaps the
// exponents and the z update (measured 4% faster per step than requesting it
// at the start).
// Dynamic LDS (dec_lds_bytes): x[3][NS][DH] (q, k, v), u[2 NS][r], nrm[2 NS],
// ph[2 NS][m], red[NS][256][4], dred[NS][4].
constexpr int kDecThreads = 256;
// float4 per thread per sequence and slice: the update streams the state in
// one slice of 16 (m = 256, d_h = 64); the read-only form in slices of 8, which
// leaves fewer registers per wave (measured 28.4 against 33.8 us per step for
// 256 sequences x 8 heads; 16 is 2% faster for the update)
template <bool UPD> constexpr int dec_vec() { return UPD ? 16 : 8; }
// float4 of an omega row requested together in the feature exponent: 8 for
// the update (with the M rows in pieces: 53.3 against 54.0 us per step for 256
// sequences x 8 heads, m = 256, r = 64); one at a time in the read-only form,
// where both changes together measured slower (30.0 against 28.5 us)
template <bool UPD> constexpr int dec_om_piece() { return UPD ? 8 : 1; }

// LDS carve-up in floats, each array starting on a 16-byte boundary
__host__ __device__ constexpr int dec_align4(int n) { return (n + 3) & ~3; }
__host__ constexpr size_t dec_lds_bytes(int ns, int dh, int r, int m) {
  return (size_t)(3 * ns * dh + dec_align4(2 * ns * r) + dec_align4(2 * ns) + dec_align4(2 * ns * m) +
                  ns * kDecThreads * 4 + ns * 4) *
         sizeof(float);
}

template <int DH> __device__ __forceinline__ void dec_rows(int tid, int i, int& j, int& d0) {
  constexpr int Q4 = DH / 4;
  j = tid / Q4 + i * (kDecThreads / Q4);
  d0 = (tid % Q4) * 4;
}

// UPD = false is the read-only form for cross-attention against a context
// summary (README section "Cross-attention"): no key or value, S and z are only
// read, and out = phi(q)^T S / phi(q)^T z (0 for a masked query).
template <typename T, int DH, int NS, bool UPD>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeArgs a) {
  constexpr int NV = UPD ? 2 : 1;   // feature vectors per sequence: q (and k)
  constexpr int kDecVec = dec_vec<UPD>();
  extern __shared__ float smem[];
  constexpr int Q4 = DH / 4;
  constexpr int RPS = kDecThreads / Q4;   // rows per slice step
  float* xs = smem;                                 // [3][NS][DH]
  float* us = xs + 3 * NS * DH;                     // [2 NS][r]
  float* nrm = us + dec_align4(2 * NS * a.r);       // [2 NS]
  float* ph = nrm + dec_align4(2 * NS);             // [2 NS][m]
  float* red = ph + dec_align4(2 * NS * a.m);       // [NS][256][4] (16-byte aligned)
  float* dred = red + NS * kDecThreads * 4;         // [NS][4]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int h = blockIdx.x % a.H;
  const int n0 = (blockIdx.x / a.H) * NS;
  const int hk = (h * a.H_kv) / a.H;
  const int ns = min(NS, a.N - n0);
  const float s = powf((float)DH, -0.25f);
  const float* Mh = a.M + (long)(a.m_per_head ? h : 0) * a.r * DH;
  const int nrows_slice = RPS * kDecVec;            // state rows per slice
  const int nslices = (a.m + nrows_slice - 1) / nrows_slice;

  // ---- state slices of every sequence: loaded into registers, updated, stored ----
  float4 sreg[NS][kDecVec];
  auto load_slice = [&](int sl) {
#pragma unroll
    for (int sq = 0; sq < NS; ++sq) {
      const float* Sb = a.S + ((long)(n0 + sq) * a.H + h) * (long)a.m * DH;
#pragma unroll
      for (int i = 0; i < kDecVec; ++i) {
        int j, d0;
        dec_rows<DH>(tid, i, j, d0);
        j += sl * nrows_slice;
        sreg[sq][i] = (sq < ns && j < a.m) ? *reinterpret_cast<const float4*>(Sb + (long)j * DH + d0)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };

  // ---- token rows to LDS (fp32) ----
  for (int e = tid; e < (UPD ? 3 : 1) * NS * DH; e += kDecThreads) {
    const int which = e / (NS * DH), sq = (e / DH) % NS, d = e % DH;
    float x = 0.f;
    if (sq < ns) {
      const int n = n0 + sq;
      if (which == 0) x = ld_elem(reinterpret_cast<const T*>(a.q) + n * a.qs[0] + h * a.qs[1], d);
      else if (which == 1) x = ld_elem(reinterpret_cast<const T*>(a.k) + n * a.ks[0] + hk * a.ks[1], d);
      else x = ld_elem(reinterpret_cast<const T*>(a.v) + n * a.vs[0] + hk * a.vs[1], d);
    }
    xs[e] = x;
  }
  __syncthreads();

  // ---- u = s M x for q and k of every sequence (vector vi: NV sq + {0: q, 1: k}) ----
  for (int p = tid; p < NV * NS * a.r; p += kDecThreads) {
    const int row = p % a.r, vi = p / a.r;
    const float* xr = xs + ((vi % NV) * NS + (vi / NV)) * DH;
    const float* mr = Mh + (long)row * DH;
    float acc = 0.f;
    if constexpr (UPD) {
      // the row of M in pieces of up to 64 columns, each piece's loads in flight together
      constexpr int PC = DH < 64 ? DH : 64;
#pragma unroll
      for (int d0 = 0; d0 < DH; d0 += PC) {
        float4 mv[PC / 4];
#pragma unroll
        for (int q = 0; q < PC / 4; ++q) mv[q] = *reinterpret_cast<const float4*>(mr + d0 + 4 * q);
#pragma unroll
        for (int q = 0; q < PC / 4; ++q) {
          const int d = d0 + 4 * q;
          acc += mv[q].x * xr[d] + mv[q].y * xr[d + 1] + mv[q].z * xr[d + 2] + mv[q].w * xr[d + 3];
        }
      }
    } else {   // read-only form: this loop measured faster there (fewer registers)
#pragma unroll 4
      for (int d = 0; d < DH; d += 4) {
        const float4 mv = *reinterpret_cast<const float4*>(mr + d);
        acc += mv.x * xr[d] + mv.y * xr[d + 1] + mv.z * xr[d + 2] + mv.w * xr[d + 3];
      }
    }
    us[vi * a.r + row] = s * acc;
  }
  __syncthreads();
  // |u|^2 / 2 of each vector: one wave per vector, lanes over the rank index
  for (int vi = wv; vi < NV * NS; vi += kDecThreads / 64) {
    float acc = 0.f;
    for (int i = lane; i < a.r; i += 64) acc += us[vi * a.r + i] * us[vi * a.r + i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) nrm[vi] = 0.5f * acc;
  }
  __syncthreads();

  load_slice(0);

  // ---- phi_j = exp(omega_j . u - |u|^2 / 2) / sqrt(m) for every vector ----
  const float half_log2m = 0.5f * log2f((float)a.m);
  for (int j = tid; j < a.m; j += kDecThreads) {
    const float* om = a.omega + ((long)(a.omega_per_head ? h : 0) * a.m + j) * a.r;
    float e[NV * NS];
#pragma unroll
    for (int vi = 0; vi < NV * NS; ++vi) e[vi] = 0.f;
    if (a.r % 4 == 0) {   // rows of omega are 16-byte aligned
      // the row in pieces of OP float4, each piece's loads in flight together
      // (one L2 round trip per piece, not one per float4)
      constexpr int OP = dec_om_piece<UPD>();
      for (int i0 = 0; i0 < a.r; i0 += 4 * OP) {
        float4 w[OP];
#pragma unroll
        for (int q = 0; q < OP; ++q)
          w[q] = i0 + 4 * q < a.r ? *reinterpret_cast<const float4*>(om + i0 + 4 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int q = 0; q < OP; ++q) {
          const int i = i0 + 4 * q;
          if (i >= a.r) break;
#pragma unroll
          for (int vi = 0; vi < NV * NS; ++vi) {
            const float* u = us + vi * a.r + i;
            e[vi] += w[q].x * u[0] + w[q].y * u[1] + w[q].z * u[2] + w[q].w * u[3];
          }
        }
      }
    } else {
      for (int i = 0; i < a.r; ++i) {
        const float w = om[i];
#pragma unroll
        for (int vi = 0; vi < NV * NS; ++vi) e[vi] += w * us[vi * a.r + i];
      }
    }
#pragma unroll
    for (int vi = 0; vi < NV * NS; ++vi)
      ph[vi * a.m + j] = exp2f(kLog2eDec * (e[vi] - nrm[vi]) - half_log2m);
  }
  __syncthreads();

  // ---- z += phi(k); denominator phi(q) . z ----
  float dp[NS];
#pragma unroll
  for (int sq = 0; sq < NS; ++sq) {
    dp[sq] = 0.f;
    if (sq >= ns) continue;
    const long st = (long)(n0 + sq) * a.H + h;
    const float* pq = ph + (NV * sq) * a.m;
    for (int j = tid; j < a.m; j += kDecThreads) {
      float zj = a.z[st * a.m + j];
      if constexpr (UPD) {
        zj += ph[(NV * sq + 1) * a.m + j];
        a.z[st * a.m + j] = zj;
      }
      dp[sq] += pq[j] * zj;
    }
  }

  // ---- S += phi(k) v^T and the numerator phi(q)^T S, slice by slice ----
  float np[NS][4];
#pragma unroll
  for (int sq = 0; sq < NS; ++sq)
#pragma unroll
    for (int c = 0; c < 4; ++c) np[sq][c] = 0.f;
  for (int sl = 0; sl < nslices; ++sl) {
    if (sl > 0) load_slice(sl);
#pragma unroll
    for (int sq = 0; sq < NS; ++sq) {
      if (sq >= ns) continue;
      float* Sb = a.S + ((long)(n0 + sq) * a.H + h) * (long)a.m * DH;
      const float* pq = ph + (NV * sq) * a.m;
      const float* pk = ph + (NV * sq + (UPD ? 1 : 0)) * a.m;
      const float* vv = xs + (2 * NS + sq) * DH;
      int j0, d0;
      dec_rows<DH>(tid, 0, j0, d0);
      const float4 v4 = UPD ? *reinterpret_cast<const float4*>(vv + d0) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int i = 0; i < kDecVec; ++i) {
        const int j = j0 + i * RPS + sl * nrows_slice;
        if (j >= a.m) break;
        const float qj = pq[j];
        float4 s4 = sreg[sq][i];
        if constexpr (UPD) {
          const float kj = pk[j];
          s4.x += kj * v4.x;
          s4.y += kj * v4.y;
          s4.z += kj * v4.z;
          s4.w += kj * v4.w;
          *reinterpret_cast<float4*>(Sb + (long)j * DH + d0) = s4;
        }
        np[sq][0] += qj * s4.x;
        np[sq][1] += qj * s4.y;
        np[sq][2] += qj * s4.z;
        np[sq][3] += qj * s4.w;
      }
    }
  }

  // ---- reductions: numerator over the row groups, denominator over all threads ----
#pragma unroll
  for (int sq = 0; sq < NS; ++sq) {
    *reinterpret_cast<float4*>(red + (sq * kDecThreads + tid) * 4) =
        make_float4(np[sq][0], np[sq][1], np[sq][2], np[sq][3]);
    float x = dp[sq];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if (lane == 0) dred[sq * 4 + wv] = x;
  }
  __syncthreads();
  for (int p = tid; p < NS * Q4; p += kDecThreads) {
    const int sq = p / Q4, cg = p % Q4;
    if (sq >= ns) continue;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int grp = 0; grp < RPS; ++grp) {
      const float4 x = *reinterpret_cast<const float4*>(red + (sq * kDecThreads + grp * Q4 + cg) * 4);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    const float dd = dred[sq * 4] + dred[sq * 4 + 1] + dred[sq * 4 + 2] + dred[sq * 4 + 3];
    const bool qvalid = a.qmask == nullptr || a.qmask[n0 + sq] != 0;
    const float inv = (dd > 0.f && qvalid) ? 1.0f / dd : 0.f;
    T* o = reinterpret_cast<T*>(a.out) + (n0 + sq) * a.os[0] + h * a.os[1];
    st_elem(o, 4 * cg, acc.x * inv);
    st_elem(o, 4 * cg + 1, acc.y * inv);
    st_elem(o, 4 * cg + 2, acc.z * inv);
    st_elem(o, 4 * cg + 3, acc.w * inv);
  }
}

template <typename T, int DH>
dark_status launch_decode_impl(const dark_prf_desc& d, const void* q, const void* k, const void* v,
                               const float* M, const float* omega, float* S, float* z, void* out,
                               const uint8_t* qmask, int update, void* stream) {
  DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.qs[0] = d.q_str[0]; a.qs[1] = d.q_str[1];
  a.ks[0] = d.k_str[0]; a.ks[1] = d.k_str[1];
  a.vs[0] = d.v_str[0]; a.vs[1] = d.v_str[1];
  a.os[0] = d.o_str[0]; a.os[1] = d.o_str[1];
  a.M = M;
  a.omega = omega;
  a.S = S;
  a.z = z;
  a.qmask = qmask;
  a.N = d.B;
  a.H = d.H;
  a.H_kv = d.H_kv;
  a.m = d.m;
  a.r = d.r;
  a.m_per_head = d.m_per_head;
  a.omega_per_head = d.omega_per_head;
  auto lds = [&](int ns) { return dec_lds_bytes(ns, DH, d.r, d.m); };
  // two sequences per workgroup (the feature maps share the M and omega reads)
  // when there are enough of them and the LDS allows it
  int NS = (d.B >= 64 && lds(2) <= 64 * 1024) ? 2 : 1;
  if (lds(NS) > 64 * 1024) return DARK_ERR_UNSUPPORTED;
  a.NS = NS;
  const int groups = (d.B + NS - 1) / NS;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  KernelTimer tm(kDecode, stream);
  const dim3 grid(groups * d.H), block(kDecThreads);
  if (update) {
    if (NS == 2) hipLaunchKernelGGL((decode_kernel<T, DH, 2, true>), grid, block, lds(NS), st, a);
    else hipLaunchKernelGGL((decode_kernel<T, DH, 1, true>), grid, block, lds(NS), st, a);
  } else {
    if (NS == 2) hipLaunchKernelGGL((decode_kernel<T, DH, 2, false>), grid, block, lds(NS), st, a);
    else hipLaunchKernelGGL((decode_kernel<T, DH, 1, false>), grid, block, lds(NS), st, a);
  }
  return hipGetLastError() == hipSuccess ? DARK_OK : DARK_ERR_HIP;
}

}  // namespace dk
