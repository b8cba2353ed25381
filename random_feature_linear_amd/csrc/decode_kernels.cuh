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
  int N, H, H_kv, m, r, m_per_head, NS;
};

__device__ __forceinline__ float ld_elem(const __bf16* p, int i) { return (float)p[i]; }
__device__ __forceinline__ float ld_elem(const float* p, int i) { return p[i]; }
__device__ __forceinline__ void st_elem(__bf16* p, int i, float x) { p[i] = (__bf16)x; }
__device__ __forceinline__ void st_elem(float* p, int i, float x) { p[i] = x; }

// Workgroup: 256 threads, one query head, NS consecutive sequences.
// Dynamic LDS: x[3][NS][DH] (q, k, v), u[2][NS][256], ph[2][NS][m], red[256][4], nrm[2][NS], den[NS]
template <typename T, int DH>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  const int NS = a.NS;
  float* xs = smem;                          // [3][NS][DH]
  float* us = xs + 3 * NS * DH;              // [2][NS][256]
  float* ph = us + 2 * NS * 256;             // [2][NS][m]
  float* red = ph + 2 * NS * a.m;            // [256][4]
  float* nrm = red + 256 * 4;                // [2][NS]
  float* den = nrm + 2 * NS;                 // [NS]

  const int tid = threadIdx.x;
  const int h = blockIdx.x % a.H;
  const int n0 = (blockIdx.x / a.H) * NS;
  const int hk = (h * a.H_kv) / a.H;
  const int ns = min(NS, a.N - n0);
  const float s = powf((float)DH, -0.25f);
  const float* Mh = a.M + (long)(a.m_per_head ? h : 0) * a.r * DH;

  // ---- token rows to LDS (fp32) ----
  for (int e = tid; e < 3 * NS * DH; e += 256) {
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

  // ---- u = s M x for q and k; thread `row` owns one rank index ----
  for (int row = tid; row < a.r; row += 256) {
    const float* mr = Mh + (long)row * DH;
    for (int sq = 0; sq < NS; ++sq) {
      float uq = 0.f, uk = 0.f;
      for (int d = 0; d < DH; ++d) {
        const float mv = mr[d];
        uq += mv * xs[sq * DH + d];
        uk += mv * xs[(NS + sq) * DH + d];
      }
      us[sq * 256 + row] = s * uq;
      us[(NS + sq) * 256 + row] = s * uk;
    }
  }
  __syncthreads();
  if (tid < 2 * NS) {
    const float* u = us + tid * 256;
    float acc = 0.f;
    for (int i = 0; i < a.r; ++i) acc += u[i] * u[i];
    nrm[tid] = 0.5f * acc;
  }
  __syncthreads();

  // ---- phi_j = exp(omega_j . u - |u|^2 / 2) / sqrt(m) ----
  const float inv_sqrt_m = 1.0f / sqrtf((float)a.m);
  for (int j = tid; j < a.m; j += 256) {
    const float* om = a.omega + (long)j * a.r;
    for (int sq = 0; sq < NS; ++sq) {
      float eq = 0.f, ek = 0.f;
      for (int i = 0; i < a.r; ++i) {
        const float w = om[i];
        eq += w * us[sq * 256 + i];
        ek += w * us[(NS + sq) * 256 + i];
      }
      ph[sq * a.m + j] = exp2f(kLog2eDec * (eq - nrm[sq])) * inv_sqrt_m;
      ph[(NS + sq) * a.m + j] = exp2f(kLog2eDec * (ek - nrm[NS + sq])) * inv_sqrt_m;
    }
  }
  __syncthreads();

  for (int sq = 0; sq < ns; ++sq) {
    const int n = n0 + sq;
    const long st = ((long)n * a.H + h);
    const float* pq = ph + sq * a.m;
    const float* pk = ph + (NS + sq) * a.m;
    const float* vv = xs + (2 * NS + sq) * DH;
    // z and the denominator
    float dp = 0.f;
    for (int j = tid; j < a.m; j += 256) {
      const float zj = a.z[st * a.m + j] + pk[j];
      a.z[st * a.m + j] = zj;
      dp += pq[j] * zj;
    }
    red[tid] = dp;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if (tid < off) red[tid] += red[tid + off];
      __syncthreads();
    }
    if (tid == 0) den[sq] = red[0];
    __syncthreads();
    // S and the numerator; thread owns columns d0 .. d0 + 3
    constexpr int Q4 = DH / 4;
    const int d0 = (tid % Q4) * 4;
    float np[4] = {0.f, 0.f, 0.f, 0.f};
    float* Sb = a.S + st * (long)a.m * DH;
    for (int e = tid; e < a.m * Q4; e += 256) {
      const int j = e / Q4;
      float4 s4 = *reinterpret_cast<float4*>(Sb + (long)j * DH + d0);
      const float kj = pk[j], qj = pq[j];
      s4.x += kj * vv[d0];
      s4.y += kj * vv[d0 + 1];
      s4.z += kj * vv[d0 + 2];
      s4.w += kj * vv[d0 + 3];
      *reinterpret_cast<float4*>(Sb + (long)j * DH + d0) = s4;
      np[0] += qj * s4.x;
      np[1] += qj * s4.y;
      np[2] += qj * s4.z;
      np[3] += qj * s4.w;
    }
    for (int i = 0; i < 4; ++i) red[tid * 4 + i] = np[i];
    __syncthreads();
    if (tid < Q4) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int grp = tid; grp < 256; grp += Q4)
        for (int i = 0; i < 4; ++i) acc[i] += red[grp * 4 + i];
      const float dd = den[sq];
      const float inv = dd > 0.f ? 1.0f / dd : 0.f;
      T* o = reinterpret_cast<T*>(a.out) + n * a.os[0] + h * a.os[1];
      for (int i = 0; i < 4; ++i) st_elem(o, d0 + i, acc[i] * inv);
    }
    __syncthreads();
  }
}

template <typename T, int DH>
dark_status launch_decode_impl(const dark_prf_desc& d, const void* q, const void* k, const void* v,
                               const float* M, const float* omega, float* S, float* z, void* out,
                               void* stream) {
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
  a.N = d.B;
  a.H = d.H;
  a.H_kv = d.H_kv;
  a.m = d.m;
  a.r = d.r;
  a.m_per_head = d.m_per_head;
  int NS = 4;
  auto lds = [&](int ns) {
    return (size_t)(3 * ns * DH + 2 * ns * 256 + 2 * ns * d.m + 256 * 4 + 3 * ns) * sizeof(float);
  };
  while (NS > 1 && lds(NS) > 64 * 1024) NS >>= 1;
  if (lds(NS) > 64 * 1024) return DARK_ERR_UNSUPPORTED;
  a.NS = NS;
  const int groups = (d.B + NS - 1) / NS;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  KernelTimer tm(kDecode, stream);
  hipLaunchKernelGGL((decode_kernel<T, DH>), dim3(groups * d.H), dim3(256), lds(NS), st, a);
  return hipGetLastError() == hipSuccess ? DARK_OK : DARK_ERR_HIP;
}

}  // namespace dk
