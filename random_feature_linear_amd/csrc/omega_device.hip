// The random projection omega [m][r] generated on the device (package README
// section "Kernel": Gaussian feature directions; section "Self-attention":
// orthogonal Gaussian blocks by default; section "Projection lifecycle": a
// seeded projection, redrawn on request).  The same stream and the same
// construction as the host generator dark_prf_omega (omega_stream.h): i.i.d.
// entries are stream values 0 .. m r - 1; orthogonal block b takes G from
// stream values 2 b r^2 .. (its r x r Gaussian), Q of G = Q R by Householder
// reflections in fp64 with column j of Q multiplied by the sign of R[j][j]
// (Haar, Mezzadri 2007), and row a of the block is the norm of stream values
// 2 b r^2 + r^2 + a r .. + r - 1 (a chi_r draw) times row a of Q.
#include "common.h"
#include "omega_stream.h"

namespace dk {

__global__ void omega_iid_kernel(uint64_t seed, long n, float* __restrict__ out) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    out[i] = (float)normal_at(seed, (uint64_t)i);
}

constexpr int kQrThreads = 256;
constexpr int kQrMaxRank = 256;

// One workgroup per block.  The workspace holds G (reduced in place to R),
// the reflectors V (column k from row k down) and Q, each r x r row-major
// fp64; threads own columns in the rank-one updates (consecutive threads,
// consecutive addresses) and rows in the column reductions.
__global__ __launch_bounds__(kQrThreads) void omega_orth_kernel(uint64_t seed, int m, int r, double* __restrict__ ws,
                                                                 float* __restrict__ out) {
  __shared__ double red[kQrThreads];
  __shared__ double s_vn2[kQrMaxRank];
  __shared__ double s_diag[kQrMaxRank];
  const int b = blockIdx.x, tid = threadIdx.x;
  const long rr = (long)r * r;
  double* G = ws + (long)b * 3 * rr;
  double* V = G + rr;
  double* Q = V + rr;
  const uint64_t base = 2ull * (uint64_t)b * (uint64_t)rr;
  auto block_sum = [&](double x) -> double {
    red[tid] = x;
    __syncthreads();
    for (int s = kQrThreads / 2; s > 0; s >>= 1) {
      if (tid < s) red[tid] += red[tid + s];
      __syncthreads();
    }
    const double v = red[0];
    __syncthreads();
    return v;
  };
  for (long e = tid; e < rr; e += kQrThreads) {
    G[e] = normal_at(seed, base + (uint64_t)e);
    V[e] = 0.0;
  }
  __syncthreads();
  for (int k = 0; k < r; ++k) {
    double part = 0.0;
    for (int i = k + tid; i < r; i += kQrThreads) {
      const double x = G[(long)i * r + k];
      part += x * x;
    }
    const double norm = sqrt(block_sum(part));
    const double alpha = G[(long)k * r + k] >= 0.0 ? -norm : norm;
    part = 0.0;
    for (int i = k + tid; i < r; i += kQrThreads) {
      const double vi = G[(long)i * r + k] - (i == k ? alpha : 0.0);
      V[(long)i * r + k] = vi;
      part += vi * vi;
    }
    const double vn2 = block_sum(part);   // also orders the V writes before their reads
    if (tid == 0) s_vn2[k] = vn2;
    if (vn2 > 0.0) {
      for (int j = k + tid; j < r; j += kQrThreads) {
        double dot = 0.0;
        for (int i = k; i < r; ++i) dot += V[(long)i * r + k] * G[(long)i * r + j];
        const double f = 2.0 * dot / vn2;
        for (int i = k; i < r; ++i) G[(long)i * r + j] -= f * V[(long)i * r + k];
      }
    }
    __syncthreads();
    if (tid == 0) s_diag[k] = G[(long)k * r + k];
  }
  // Q = H_0 H_1 ... H_{r-1} applied to the identity, right to left
  for (long e = tid; e < rr; e += kQrThreads) Q[e] = (e / r == e % r) ? 1.0 : 0.0;
  __syncthreads();
  for (int k = r - 1; k >= 0; --k) {
    const double vn2 = s_vn2[k];
    if (vn2 > 0.0) {
      for (int j = tid; j < r; j += kQrThreads) {
        double dot = 0.0;
        for (int i = k; i < r; ++i) dot += V[(long)i * r + k] * Q[(long)i * r + j];
        const double f = 2.0 * dot / vn2;
        for (int i = k; i < r; ++i) Q[(long)i * r + j] -= f * V[(long)i * r + k];
      }
    }
    __syncthreads();
  }
  // the block's rows of omega
  const int keep = min(r, m - b * r);
  for (int a = 0; a < keep; ++a) {
    double part = 0.0;
    for (int c = tid; c < r; c += kQrThreads) {
      const double x = normal_at(seed, base + (uint64_t)rr + (uint64_t)a * r + c);
      part += x * x;
    }
    const double nrm = sqrt(block_sum(part));
    for (int c = tid; c < r; c += kQrThreads) {
      const double q = s_diag[c] < 0.0 ? -Q[(long)a * r + c] : Q[(long)a * r + c];
      out[((long)b * r + a) * r + c] = (float)(nrm * q);
    }
  }
}

size_t omega_device_ws_bytes(int m, int r, int orthogonal) {
  if (!orthogonal) return 0;
  const long blocks = (m + r - 1) / r;
  return (size_t)blocks * 3 * r * r * sizeof(double);
}

dark_status launch_omega_device(uint64_t seed, int m, int r, int orthogonal, float* omega, void* ws,
                                void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  KernelTimer tm(kPrep, stream);
  if (!orthogonal) {
    const long n = (long)m * r;
    const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(omega_iid_kernel, dim3(blocks), dim3(256), 0, st, seed, n, omega);
  } else {
    hipLaunchKernelGGL(omega_orth_kernel, dim3((m + r - 1) / r), dim3(kQrThreads), 0, st, seed, m, r,
                       reinterpret_cast<double*>(ws), omega);
  }
  return hipGetLastError() == hipSuccess ? DARK_OK : DARK_ERR_HIP;
}

}  // namespace dk
