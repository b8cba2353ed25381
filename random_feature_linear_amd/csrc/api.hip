// C ABI of the darkprf library: argument validation, planning and dispatch.
// Every check happens on the host before anything is queued; see darkprf.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <mutex>
#include <utility>
#include <vector>

#include "common.h"
#include "omega_stream.h"

namespace dk {

// launchers defined in the instantiation units
#define DK_DECL(dt, dh)                                                                                \
  dark_status fwd_##dt##_d##dh##_r1(const FwdArgs&, const Plan&, void*, void*);                       \
  dark_status fwd_##dt##_d##dh##_r2(const FwdArgs&, const Plan&, void*, void*);                       \
  dark_status fwd_##dt##_d##dh##_r4(const FwdArgs&, const Plan&, void*, void*);                       \
  dark_status fwd_##dt##_d##dh##_r8(const FwdArgs&, const Plan&, void*, void*);                       \
  dark_status fwd_##dt##_d##dh##_r16(const FwdArgs&, const Plan&, void*, void*);                      \
  dark_status exact_##dt##_d##dh##_r1(const FwdArgs&, void*, void*);                                  \
  dark_status exact_##dt##_d##dh##_r2(const FwdArgs&, void*, void*);                                  \
  dark_status exact_##dt##_d##dh##_r4(const FwdArgs&, void*, void*);                                  \
  dark_status exact_##dt##_d##dh##_r8(const FwdArgs&, void*, void*);                                  \
  dark_status exact_##dt##_d##dh##_r16(const FwdArgs&, void*, void*);                                 \
  dark_status dec_##dt##_d##dh(const dark_prf_desc&, const void*, const void*, const void*,            \
                               const float*, const float*, float*, float*, void*, const uint8_t*, int,  \
                               void*);
DK_DECL(bf16, 16)
DK_DECL(bf16, 32)
DK_DECL(bf16, 64)
DK_DECL(bf16, 128)
DK_DECL(bf16, 256)
DK_DECL(f32, 16)
DK_DECL(f32, 32)
DK_DECL(f32, 64)
DK_DECL(f32, 128)
DK_DECL(f32, 256)
#undef DK_DECL

static int dh_index(int d_h) {
  switch (d_h) {
    case 16: return 0;
    case 32: return 1;
    case 64: return 2;
    case 128: return 3;
    case 256: return 4;
    default: return -1;
  }
}
static int r16_index(int r16) {
  switch (r16) {
    case 1: return 0;
    case 2: return 1;
    case 4: return 2;
    case 8: return 3;
    case 16: return 4;
    default: return -1;
  }
}

#define DK_ROW(dt, dh) {fwd_##dt##_d##dh##_r1, fwd_##dt##_d##dh##_r2, fwd_##dt##_d##dh##_r4, fwd_##dt##_d##dh##_r8, fwd_##dt##_d##dh##_r16}
static const fwd_launcher kFwd[2][5][5] = {
    {DK_ROW(f32, 16), DK_ROW(f32, 32), DK_ROW(f32, 64), DK_ROW(f32, 128), DK_ROW(f32, 256)},
    {DK_ROW(bf16, 16), DK_ROW(bf16, 32), DK_ROW(bf16, 64), DK_ROW(bf16, 128), DK_ROW(bf16, 256)}};
#undef DK_ROW
typedef dark_status (*exact_launcher)(const FwdArgs&, void* ws, void* stream);
#define DK_XROW(dt, dh) {exact_##dt##_d##dh##_r1, exact_##dt##_d##dh##_r2, exact_##dt##_d##dh##_r4, exact_##dt##_d##dh##_r8, exact_##dt##_d##dh##_r16}
static const exact_launcher kExact[2][5][5] = {
    {DK_XROW(f32, 16), DK_XROW(f32, 32), DK_XROW(f32, 64), DK_XROW(f32, 128), DK_XROW(f32, 256)},
    {DK_XROW(bf16, 16), DK_XROW(bf16, 32), DK_XROW(bf16, 64), DK_XROW(bf16, 128), DK_XROW(bf16, 256)}};
#undef DK_XROW
static exact_launcher find_exact_launcher(int dtype, int d_h, int r16) {
  const int i = dh_index(d_h), j = r16_index(r16);
  if (dtype < 0 || dtype > 1 || i < 0 || j < 0) return nullptr;
  return kExact[dtype][i][j];
}
static const decode_launcher kDec[2][5] = {
    {dec_f32_d16, dec_f32_d32, dec_f32_d64, dec_f32_d128, dec_f32_d256},
    {dec_bf16_d16, dec_bf16_d32, dec_bf16_d64, dec_bf16_d128, dec_bf16_d256}};

fwd_launcher find_fwd_launcher(int dtype, int d_h, int r16) {
  const int i = dh_index(d_h), j = r16_index(r16);
  if (dtype < 0 || dtype > 1 || i < 0 || j < 0) return nullptr;
  return kFwd[dtype][i][j];
}
decode_launcher find_decode_launcher(int dtype, int d_h) {
  const int i = dh_index(d_h);
  if (dtype < 0 || dtype > 1 || i < 0) return nullptr;
  return kDec[dtype][i];
}

static int rank_blocks(int r) { return r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : r <= 128 ? 8 : 16; }
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

// 32-feature blocks per wave in the key-side kernel (must match the instantiation units).
static int feature_blocks_per_wave(int d_h) { return d_h <= 64 ? 2 : 1; }

static void make_plan(const dark_prf_desc& d, Plan& p, int mode = kPlanForward) {
  memset(&p, 0, sizeof(p));
  p.DH = d.d_h;
  p.R16 = rank_blocks(d.r);
  p.FB = cdiv(d.m, 32);
  p.HM = d.m_per_head ? d.H : 1;
  p.HO = d.omega_per_head ? d.H : 1;
  p.HW = (d.m_per_head || d.omega_per_head) ? d.H : 1;
  p.fold = fold_exponent(d.dtype == DARK_BF16 ? 2 : 4, d.d_h, p.R16);
  p.BH = d.B * d.H;
  p.elem = d.dtype == DARK_BF16 ? 2 : 4;
  p.FBW = feature_blocks_per_wave(d.d_h);
  int units_ws = 0;   // units the workspace is sized for (>= NU; grows with L, so the workspace never shrinks)
  p.NF = cdiv(p.FB, 4 * p.FBW);
  const int L = d.L > 0 ? d.L : 1;
  const int tile1 = 128;                 // key-side tile: 4 waves x 32 tokens
  if (d.causal) {
    // chunk = 128 tokens: the key-side unit, the query-side tile and the
    // granularity of the materialised chunk states
    p.NQB = 1;
    p.tile2 = 128;
    p.span1 = p.tile2;
    p.NU = cdiv(L, p.span1);
    p.NT2 = p.NU;
    units_ws = p.NU;
    // folded form: up to 8 chunks per key-side workgroup while at least 1024
    // workgroups remain; the W' fragments are fetched once for all of them and
    // each chunk's rows are fetched during the previous chunk's products
    // (GQA, L = 8192: key side 398 us with one chunk, 357 with 4, 354 with 8,
    // 366 with 16)
    p.UPW = 1;
    while (p.fold && p.UPW < 8 && (long)p.BH * p.NF * cdiv(p.NU, 2 * p.UPW) >= 1024) p.UPW *= 2;
  } else {
    // two query blocks per wave (d_h <= 64) when that still leaves at least
    // two workgroups per compute unit
    p.NQB = (d.d_h <= 64 && (long)p.BH * cdiv(L, 256) >= 512) ? 2 : 1;
    p.tile2 = 128 * p.NQB;
    p.NT2 = cdiv(L, p.tile2);
    int splits = cdiv(512, (long)(p.BH > 0 ? p.BH : 1) * p.NF);   // B = 0 plans as B = 1
    splits = splits < 1 ? 1 : splits;
    const int max_splits = cdiv(L, tile1);
    if (splits > max_splits) splits = max_splits;
    p.span1 = cdiv(cdiv(L, splits), tile1) * tile1;
    p.NU = cdiv(L, p.span1);
    p.UPW = 1;
    units_ws = splits;   // NU <= splits, and splits never decreases as L grows
  }
  // operand copies of M' (bf16: hi and lo parts) and omega' (see prf_kernels.h)
  const int NM = d.dtype == DARK_BF16 ? 2 : 1;
  const int R32 = (p.R16 + 1) / 2;
  const int DB = (d.d_h + 31) / 32;      // 32-column blocks of V
  const size_t frag = 64 * 8;            // elements per operand fragment
  const size_t state_frags = (size_t)DB * 2 * p.FB;   // fragments of one unit state S
  const int nout = d.causal ? p.NU : 1;
  const int units = units_ws > p.NU ? units_ws : p.NU;
  size_t off = 0;
  p.off_mfrag = off;
  off = align256(off + (size_t)p.HM * R32 * (d.d_h / 16) * NM * frag * p.elem);
  p.off_ofrag = off;   // one part (the bf16 path's exponent operands are fp16)
  if (p.fold)   // W' fragments per folded operand, K-steps over d_h
    off = align256(off + (size_t)p.HW * p.FB * (d.d_h / 16) * frag * p.elem);
  else          // omega' fragments per projection, K-steps over the rank
    off = align256(off + (size_t)p.HO * p.FB * p.R16 * frag * p.elem);
  p.off_sdelta = off;
  off = align256(off + (size_t)p.BH * units * state_frags * frag * p.elem);
  // the per-unit states stay in L2 between the key side and the sum (same XCD)
  // unless they are larger than about half of the 8 x 4 MB of L2
  p.stream_states = (size_t)p.BH * p.NU * state_frags * frag * p.elem > ((size_t)16 << 20);
  p.off_sfrag = off;
  off = align256(off + (size_t)p.BH * nout * state_frags * frag * p.elem);
  // normaliser states z (fp32, 32 FB per unit): per unit, then combined
  p.off_zdelta = off;
  off = align256(off + (size_t)p.BH * units * p.FB * 32 * sizeof(float));
  p.off_zsum = off;
  off = align256(off + (size_t)p.BH * nout * p.FB * 32 * sizeof(float));
  // keys are projected once up front (for |u|^2) when several feature slices,
  // or the causal query side, would otherwise repeat it (a context summary
  // projects its own keys; queries need no such shift)
  p.mode = mode;
  p.kshift = mode == kPlanForward && p.fold && (p.NF > 1 || (d.causal && d.d_h >= 128));
  p.off_kshift = off;
  if (p.kshift) off = align256(off + (size_t)p.BH * L * sizeof(float));
  p.total = off;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Shape and stride checks shared by every entry point; `tensors` selects the
// stride sets that the call uses (bit 0 q, 1 k, 2 v, 3 out).
static dark_status check_desc(const dark_prf_desc* d, bool decode, int tensors = 15) {
  if (!d) return DARK_ERR_INVALID_ARG;
  if (d->B < 0 || d->L < 0 || d->H < 1 || d->H_kv < 1 || d->H % d->H_kv != 0) return DARK_ERR_INVALID_ARG;
  if (dh_index(d->d_h) < 0) return DARK_ERR_INVALID_ARG;
  if (d->m < 16 || d->m % 16 != 0) return DARK_ERR_INVALID_ARG;
  if (d->r < 1 || d->r > 256) return DARK_ERR_INVALID_ARG;
  if (d->dtype != DARK_F32 && d->dtype != DARK_BF16) return DARK_ERR_INVALID_ARG;
  if (d->causal != 0 && d->causal != 1) return DARK_ERR_INVALID_ARG;
  if (d->m_per_head != 0 && d->m_per_head != 1) return DARK_ERR_INVALID_ARG;
  if (d->omega_per_head != 0 && d->omega_per_head != 1) return DARK_ERR_INVALID_ARG;
  if (decode && (d->L != 1 || d->causal != 1)) return DARK_ERR_INVALID_ARG;
  const int64_t elem = d->dtype == DARK_BF16 ? 2 : 4;
  const int64_t* strides[4] = {d->q_str, d->k_str, d->v_str, d->o_str};
  for (int t = 0; t < 4; ++t) {
    if (!(tensors >> t & 1)) continue;
    for (int i = 0; i < 3; ++i) {
      if (decode && i == 2) continue;
      if (strides[t][i] < 0 || (strides[t][i] * elem) % 16 != 0) return DARK_ERR_INVALID_ARG;
    }
    if (!decode && d->L > 1 && strides[t][2] < d->d_h) return DARK_ERR_INVALID_ARG;
  }
  // element offsets are formed in 64-bit; the grid is formed in 32-bit
  if ((int64_t)d->B * d->H * ((int64_t)d->L + 255) > (int64_t)1 << 31) return DARK_ERR_UNSUPPORTED;
  return DARK_OK;
}

// ---- Omega: the Gaussian stream (omega_stream.h); Householder QR with the sign of R ----

// Q of G = Q R (n x n, row-major, overwritten) by Householder reflections,
// with column j of Q multiplied by the sign of R[j][j] so that Q is Haar.
static void haar_q(std::vector<double>& G, int n, std::vector<double>& Q) {
  std::vector<double> V((size_t)n * n, 0.0);   // reflector k in column k (rows k..n-1)
  std::vector<double> vn2(n, 0.0), diag(n, 0.0);
  for (int k = 0; k < n; ++k) {
    double norm = 0.0;
    for (int i = k; i < n; ++i) norm += G[(size_t)i * n + k] * G[(size_t)i * n + k];
    norm = sqrt(norm);
    const double alpha = G[(size_t)k * n + k] >= 0.0 ? -norm : norm;
    for (int i = k; i < n; ++i) {
      const double vi = G[(size_t)i * n + k] - (i == k ? alpha : 0.0);
      V[(size_t)i * n + k] = vi;
      vn2[k] += vi * vi;
    }
    if (vn2[k] > 0.0) {
      for (int j = k; j < n; ++j) {
        double dot = 0.0;
        for (int i = k; i < n; ++i) dot += V[(size_t)i * n + k] * G[(size_t)i * n + j];
        const double f = 2.0 * dot / vn2[k];
        for (int i = k; i < n; ++i) G[(size_t)i * n + j] -= f * V[(size_t)i * n + k];
      }
    }
    diag[k] = G[(size_t)k * n + k];
  }
  Q.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) Q[(size_t)i * n + i] = 1.0;
  // Q = H_0 H_1 ... H_{n-1} applied to the identity, right to left
  for (int k = n - 1; k >= 0; --k) {
    if (vn2[k] <= 0.0) continue;
    for (int j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int i = k; i < n; ++i) dot += V[(size_t)i * n + k] * Q[(size_t)i * n + j];
      const double f = 2.0 * dot / vn2[k];
      for (int i = k; i < n; ++i) Q[(size_t)i * n + j] -= f * V[(size_t)i * n + k];
    }
  }
  for (int j = 0; j < n; ++j)
    if (diag[j] < 0.0)
      for (int i = 0; i < n; ++i) Q[(size_t)i * n + j] = -Q[(size_t)i * n + j];
}

// ---- optional per-kernel timing ----
struct TimingState {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> recs;
};
static TimingState& timing() {
  static TimingState t;
  return t;
}

KernelTimer::KernelTimer(int k, void* s) : kind(k), stream(s), ev0(nullptr), ev1(nullptr) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on) return;
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess) return;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return;
  }
  (void)hipEventRecord(a, reinterpret_cast<hipStream_t>(s));
  ev0 = a;
  ev1 = b;
}

KernelTimer::~KernelTimer() {
  if (!ev0) return;
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev1), reinterpret_cast<hipStream_t>(stream));
  t.recs.push_back({kind, {reinterpret_cast<hipEvent_t>(ev0), reinterpret_cast<hipEvent_t>(ev1)}});
}

static void drop_records(TimingState& t) {
  for (auto& r : t.recs) {
    (void)hipEventDestroy(r.second.first);
    (void)hipEventDestroy(r.second.second);
  }
  t.recs.clear();
}

// dark_prf_fwd_noalloc: the forward's workspace taken from a static device
// array instead of the caller.  The array exists once per GPU (each device
// holds its own copy at its own address).  Host code never uses its name as an
// address, only the device pointer that hipGetSymbolAddress returns for the
// current device, looked up on the first call on that device and kept.
static __device__ __align__(256) unsigned char scratch[DARK_PRF_SCRATCH_BYTES];

static dark_status scratch_address(void* stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DARK_ERR_HIP;
  if (stream != nullptr) {   // the kernels run on the stream's device: it must be the current one
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev) != hipSuccess) return DARK_ERR_HIP;
    if (sdev != dev) return DARK_ERR_INVALID_ARG;
  }
  static std::mutex mu;
  static std::vector<void*> ptr;   // per device; null until looked up
  std::lock_guard<std::mutex> g(mu);
  if ((int)ptr.size() <= dev) ptr.resize(dev + 1, nullptr);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DARK_ERR_HIP;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return DARK_OK;
}

}  // namespace dk

using namespace dk;

extern "C" {

const char* dark_prf_status_str(dark_status s) {
  switch (s) {
    case DARK_OK: return "DARK_OK";
    case DARK_ERR_INVALID_ARG: return "DARK_ERR_INVALID_ARG";
    case DARK_ERR_UNSUPPORTED: return "DARK_ERR_UNSUPPORTED";
    case DARK_ERR_WORKSPACE: return "DARK_ERR_WORKSPACE";
    case DARK_ERR_STALE_STATE: return "DARK_ERR_STALE_STATE";
    case DARK_ERR_HIP: return "DARK_ERR_HIP";
    default: return "DARK_ERR_UNKNOWN";
  }
}

uint64_t dark_prf_proj_tag(uint64_t seed, int32_t m, int32_t r, int32_t orthogonal) {
  const uint64_t shape = ((uint64_t)(uint32_t)m << 32) ^ ((uint64_t)(uint32_t)r << 1) ^ (orthogonal ? 1u : 0u);
  return mix64(mix64(seed + 0x9E3779B97F4A7C15ULL) ^ mix64(shape + 0x632BE59BD9B4E019ULL));
}

dark_status dark_prf_omega(uint64_t seed, int32_t m, int32_t r, int32_t orthogonal, float* omega_host) {
  if (m < 1 || r < 1 || omega_host == nullptr) return DARK_ERR_INVALID_ARG;
  if (!orthogonal) {
    for (int64_t i = 0; i < (int64_t)m * r; ++i) omega_host[i] = (float)normal_at(seed, (uint64_t)i);
    return DARK_OK;
  }
  const int blocks = (m + r - 1) / r;
  std::vector<double> G((size_t)r * r), Q;
  for (int b = 0; b < blocks; ++b) {
    const uint64_t base = 2ull * (uint64_t)b * r * r;
    for (int i = 0; i < r * r; ++i) G[i] = normal_at(seed, base + i);
    haar_q(G, r, Q);
    const int keep = (m - b * r) < r ? (m - b * r) : r;
    for (int a = 0; a < keep; ++a) {
      double nn = 0.0;
      for (int c = 0; c < r; ++c) {
        const double x = normal_at(seed, base + (uint64_t)r * r + (uint64_t)a * r + c);
        nn += x * x;
      }
      const double norm = sqrt(nn);
      for (int c = 0; c < r; ++c) omega_host[((int64_t)b * r + a) * r + c] = (float)(norm * Q[(size_t)a * r + c]);
    }
  }
  return DARK_OK;
}

uint64_t dark_prf_head_seed(uint64_t seed, int32_t h) {
  return mix64(seed + (uint64_t)((int64_t)h + 1) * 0xD1B54A32D192ED03ULL);
}

dark_status dark_prf_omega_per_head(uint64_t seed, int32_t H, int32_t m, int32_t r, int32_t orthogonal,
                                    float* omega_host) {
  if (H < 1 || m < 1 || r < 1 || omega_host == nullptr) return DARK_ERR_INVALID_ARG;
  for (int32_t h = 0; h < H; ++h) {
    const dark_status st = dark_prf_omega(dark_prf_head_seed(seed, h), m, r, orthogonal,
                                          omega_host + (int64_t)h * m * r);
    if (st != DARK_OK) return st;
  }
  return DARK_OK;
}

uint64_t dark_prf_proj_tag_per_head(uint64_t seed, int32_t H, int32_t m, int32_t r, int32_t orthogonal) {
  return mix64(dark_prf_proj_tag(seed, m, r, orthogonal) ^ mix64((uint64_t)(uint32_t)H + 0x5851F42D4C957F2DULL));
}

static uint64_t draw_seed(uint64_t base, int64_t draw) {
  return draw == 0 ? base : mix64(base + (uint64_t)draw * 0x9E3779B97F4A7C15ULL);
}
static void set_draw(dark_prf_projection* p, int64_t draw) {
  p->draw = draw;
  p->seed = draw_seed(p->base_seed, draw);
  p->tag = dark_prf_proj_tag(p->seed, p->m, p->r, p->orthogonal);
  p->forwards = 0;
}

dark_status dark_prf_projection_init(dark_prf_projection* p, uint64_t seed, int32_t m, int32_t r,
                                     int32_t orthogonal, int32_t redraw_interval, int32_t deterministic) {
  if (!p || m < 1 || r < 1) return DARK_ERR_INVALID_ARG;
  memset(p, 0, sizeof(*p));
  p->base_seed = seed;
  p->m = m;
  p->r = r;
  p->orthogonal = orthogonal != 0;
  p->interval = redraw_interval;
  p->fixed = deterministic != 0;
  set_draw(p, 0);
  return DARK_OK;
}

int32_t dark_prf_projection_forward(dark_prf_projection* p, int32_t training) {
  if (!p) return -1;
  if (!training) return 0;
  int32_t redrawn = 0;
  if (!p->fixed && p->interval > 0 && p->forwards >= p->interval) {
    set_draw(p, p->draw + 1);
    redrawn = 1;
  }
  p->forwards += 1;
  return redrawn;
}

int32_t dark_prf_projection_redraw(dark_prf_projection* p, int32_t force) {
  if (!p) return -1;
  if (p->fixed && !force) return 0;
  set_draw(p, p->draw + 1);
  return 1;
}

dark_status dark_prf_projection_fix(dark_prf_projection* p, int32_t fixed) {
  if (!p) return DARK_ERR_INVALID_ARG;
  p->fixed = fixed != 0;
  return DARK_OK;
}

size_t dark_prf_omega_device_workspace_bytes(int32_t m, int32_t r, int32_t orthogonal) {
  if (m < 1 || r < 1 || r > 256) return 0;
  return omega_device_ws_bytes(m, r, orthogonal != 0);
}

dark_status dark_prf_omega_device(uint64_t seed, int32_t m, int32_t r, int32_t orthogonal, float* omega,
                                  void* workspace, size_t ws_bytes, void* stream) {
  if (m < 1 || r < 1 || r > 256 || omega == nullptr) return DARK_ERR_INVALID_ARG;
  const size_t need = omega_device_ws_bytes(m, r, orthogonal != 0);
  if (need > 0 && (workspace == nullptr || ws_bytes < need)) return DARK_ERR_WORKSPACE;
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 7) != 0) return DARK_ERR_INVALID_ARG;
  (void)hipGetLastError();   // launch errors below are ours, not an earlier caller's
  return launch_omega_device(seed, m, r, orthogonal != 0, omega, workspace, stream);
}

size_t dark_prf_workspace_bytes(const dark_prf_desc* desc) {
  if (check_desc(desc, false) != DARK_OK) return 0;
  Plan p;
  make_plan(*desc, p);
  return p.total;
}

__global__ void dk_fill_zero(float* p, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) p[i] = 0.f;
}

// Arguments common to the forward-chain calls (pointers the call does not use stay null).
static FwdArgs fwd_args(const dark_prf_desc& d) {
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = d.q_str[i];
    a.ks[i] = d.k_str[i];
    a.vs[i] = d.v_str[i];
    a.os[i] = d.o_str[i];
  }
  a.B = d.B;
  a.H = d.H;
  a.H_kv = d.H_kv;
  a.L = d.L;
  a.m = d.m;
  a.r = d.r;
  a.causal = d.causal;
  a.m_per_head = d.m_per_head;
  a.omega_per_head = d.omega_per_head;
  return a;
}

dark_status dark_prf_fwd(const dark_prf_desc* desc, const void* q, const void* k, const void* v,
                         const float* M, const float* omega, const uint8_t* mask, void* out, float* S_out,
                         float* z_out, void* workspace, size_t ws_bytes, void* stream) {
  dark_status st = check_desc(desc, false);
  if (st != DARK_OK) return st;
  const dark_prf_desc& d = *desc;
  if ((S_out == nullptr) != (z_out == nullptr)) return DARK_ERR_INVALID_ARG;
  if (S_out && !d.causal) return DARK_ERR_INVALID_ARG;
  if (d.B == 0) return DARK_OK;
  if (d.L == 0) {
    if (S_out) {
      (void)hipGetLastError();
      hipStream_t s = reinterpret_cast<hipStream_t>(stream);
      const long nS = (long)d.B * d.H * d.m * d.d_h, nz = (long)d.B * d.H * d.m;
      hipLaunchKernelGGL(dk_fill_zero, dim3(256), dim3(256), 0, s, S_out, nS);
      hipLaunchKernelGGL(dk_fill_zero, dim3(64), dim3(256), 0, s, z_out, nz);
      return hipGetLastError() == hipSuccess ? DARK_OK : DARK_ERR_HIP;
    }
    return DARK_OK;
  }
  if (!q || !k || !v || !M || !omega || !out) return DARK_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return DARK_ERR_INVALID_ARG;
  if (!aligned16(M) || !aligned16(omega)) return DARK_ERR_INVALID_ARG;
  if (S_out && (!aligned16(S_out) || !aligned16(z_out))) return DARK_ERR_INVALID_ARG;
  Plan p;
  make_plan(d, p);
  if (workspace == nullptr || ws_bytes < p.total) return DARK_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DARK_ERR_INVALID_ARG;
  fwd_launcher fn = find_fwd_launcher(d.dtype, d.d_h, p.R16);
  if (!fn) return DARK_ERR_UNSUPPORTED;
  (void)hipGetLastError();   // launch errors below are ours, not an earlier caller's
  FwdArgs a = fwd_args(d);   // every field set; kshift comes from the workspace in the launcher
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.mask = mask;
  a.M = M;
  a.omega = omega;
  a.S_out = S_out;
  a.z_out = z_out;
  return fn(a, p, workspace, stream);
}

dark_status dark_prf_fwd_noalloc(const dark_prf_desc* desc, const void* q, const void* k, const void* v,
                                 const float* M, const float* omega, const uint8_t* mask, void* out, float* S_out,
                                 float* z_out, void* stream) {
  dark_status st = check_desc(desc, false);
  if (st != DARK_OK) return st;
  Plan p;
  make_plan(*desc, p);
  if (p.total > (size_t)DARK_PRF_SCRATCH_BYTES) return DARK_ERR_WORKSPACE;   // more than the static buffer holds
  void* ws = nullptr;
  st = scratch_address(stream, &ws);
  if (st != DARK_OK) return st;
  return dark_prf_fwd(desc, q, k, v, M, omega, mask, out, S_out, z_out, ws, (size_t)DARK_PRF_SCRATCH_BYTES,
                      stream);
}

static dark_status zero_state(const dark_prf_desc& d, float* S, float* z, void* stream) {
  (void)hipGetLastError();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const long nS = (long)d.B * d.H * d.m * d.d_h, nz = (long)d.B * d.H * d.m;
  hipLaunchKernelGGL(dk_fill_zero, dim3(256), dim3(256), 0, s, S, nS);
  hipLaunchKernelGGL(dk_fill_zero, dim3(64), dim3(256), 0, s, z, nz);
  return hipGetLastError() == hipSuccess ? DARK_OK : DARK_ERR_HIP;
}

dark_status dark_prf_context_state(const dark_prf_desc* desc, const void* k, const void* v, const float* M,
                                   const float* omega, const uint8_t* context_mask, float* S_out, float* z_out,
                                   void* workspace, size_t ws_bytes, void* stream) {
  dark_status st = check_desc(desc, false, 2 | 4);
  if (st != DARK_OK) return st;
  const dark_prf_desc& d = *desc;
  if (d.causal != 0) return DARK_ERR_INVALID_ARG;
  if (!S_out || !z_out || !aligned16(S_out) || !aligned16(z_out)) return DARK_ERR_INVALID_ARG;
  if (d.B == 0) return DARK_OK;
  if (d.L == 0) return zero_state(d, S_out, z_out, stream);
  if (!k || !v || !M || !omega) return DARK_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(M) || !aligned16(omega)) return DARK_ERR_INVALID_ARG;
  Plan p;
  make_plan(d, p, kPlanContext);
  if (workspace == nullptr || ws_bytes < p.total) return DARK_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DARK_ERR_INVALID_ARG;
  fwd_launcher fn = find_fwd_launcher(d.dtype, d.d_h, p.R16);
  if (!fn) return DARK_ERR_UNSUPPORTED;
  (void)hipGetLastError();   // launch errors below are ours, not an earlier caller's
  FwdArgs a = fwd_args(d);
  a.k = k;
  a.v = v;
  a.mask = context_mask;
  a.M = M;
  a.omega = omega;
  a.S_out = S_out;
  a.z_out = z_out;
  return fn(a, p, workspace, stream);
}

dark_status dark_prf_cross_fwd(const dark_prf_desc* desc, const void* q, const float* M, const float* omega,
                               const float* S, const float* z, uint64_t state_tag, const uint8_t* query_mask,
                               void* out, void* workspace, size_t ws_bytes, void* stream) {
  dark_status st = check_desc(desc, false, 1 | 8);
  if (st != DARK_OK) return st;
  const dark_prf_desc& d = *desc;
  if (d.causal != 0) return DARK_ERR_INVALID_ARG;
  if (state_tag != d.proj_tag) return DARK_ERR_STALE_STATE;
  if (d.B == 0 || d.L == 0) return DARK_OK;
  if (!q || !M || !omega || !S || !z || !out) return DARK_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || !aligned16(M) || !aligned16(omega)) return DARK_ERR_INVALID_ARG;
  if (!aligned16(S) || !aligned16(z)) return DARK_ERR_INVALID_ARG;
  if (d.L == 1) {   // one query per sequence (a decoder step): one pass over the fp32 summary
    decode_launcher fn = find_decode_launcher(d.dtype, d.d_h);
    if (!fn) return DARK_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    return fn(d, q, nullptr, nullptr, M, omega, const_cast<float*>(S), const_cast<float*>(z), out, query_mask, 0,
              stream);
  }
  Plan p;
  make_plan(d, p, kPlanCross);
  if (workspace == nullptr || ws_bytes < p.total) return DARK_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DARK_ERR_INVALID_ARG;
  fwd_launcher fn = find_fwd_launcher(d.dtype, d.d_h, p.R16);
  if (!fn) return DARK_ERR_UNSUPPORTED;
  (void)hipGetLastError();   // launch errors below are ours, not an earlier caller's
  FwdArgs a = fwd_args(d);
  a.q = q;
  a.out = out;
  a.qmask = query_mask;
  a.M = M;
  a.omega = omega;
  a.S_in = S;
  a.z_in = z;
  return fn(a, p, workspace, stream);
}

size_t dark_prf_exact_workspace_bytes(const dark_prf_desc* desc) {
  if (check_desc(desc, false, 1 | 2 | 4 | 8) != DARK_OK) return 0;
  const dark_prf_desc& d = *desc;
  return exact_layout(d.B, d.H, d.L > 0 ? d.L : 1, d.d_h, rank_blocks(d.r), d.m_per_head ? d.H : 1,
                      d.dtype == DARK_BF16 ? 2 : 4, d.causal).total;
}

dark_status dark_prf_exact_fwd(const dark_prf_desc* desc, const void* q, const void* k, const void* v,
                               const float* M, const uint8_t* mask, void* out, void* workspace, size_t ws_bytes,
                               void* stream) {
  dark_status st = check_desc(desc, false, 1 | 2 | 4 | 8);
  if (st != DARK_OK) return st;
  const dark_prf_desc& d = *desc;
  if (d.B == 0 || d.L == 0) return DARK_OK;
  if (!q || !k || !v || !M || !out) return DARK_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(M)) return DARK_ERR_INVALID_ARG;
  if (workspace == nullptr || ws_bytes < dark_prf_exact_workspace_bytes(desc)) return DARK_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DARK_ERR_INVALID_ARG;
  exact_launcher fn = find_exact_launcher(d.dtype, d.d_h, rank_blocks(d.r));
  if (!fn) return DARK_ERR_UNSUPPORTED;
  (void)hipGetLastError();   // launch errors below are ours, not an earlier caller's
  FwdArgs a = fwd_args(d);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.mask = mask;
  a.M = M;
  return fn(a, workspace, stream);
}

int32_t dark_prf_auto_mode(const dark_prf_desc* desc, int32_t exact_threshold) {
  if (exact_threshold < 0 || check_desc(desc, false) != DARK_OK) return -1;
  return desc->L <= exact_threshold ? 1 : 0;
}

size_t dark_prf_auto_workspace_bytes(const dark_prf_desc* desc, int32_t exact_threshold) {
  const int32_t mode = dark_prf_auto_mode(desc, exact_threshold);
  if (mode < 0) return 0;
  return mode == 1 ? dark_prf_exact_workspace_bytes(desc) : dark_prf_workspace_bytes(desc);
}

dark_status dark_prf_auto_fwd(const dark_prf_desc* desc, int32_t exact_threshold, const void* q, const void* k,
                              const void* v, const float* M, const float* omega, const uint8_t* mask, void* out,
                              void* workspace, size_t ws_bytes, void* stream) {
  if (exact_threshold < 0) return DARK_ERR_INVALID_ARG;
  const dark_status st = check_desc(desc, false);
  if (st != DARK_OK) return st;
  if (desc->L <= exact_threshold)
    return dark_prf_exact_fwd(desc, q, k, v, M, mask, out, workspace, ws_bytes, stream);
  return dark_prf_fwd(desc, q, k, v, M, omega, mask, out, nullptr, nullptr, workspace, ws_bytes, stream);
}

size_t dark_prf_bwd_workspace_bytes(const dark_prf_desc* desc) {
  if (check_desc(desc, false) != DARK_OK) return 0;
  return bwd_ws_bytes(*desc);
}

dark_status dark_prf_bwd(const dark_prf_desc* desc, const void* q, const void* k, const void* v, const float* M,
                         const float* omega, const uint8_t* mask, const void* dout, void* dq, void* dk, void* dv,
                         float* dM, void* workspace, size_t ws_bytes, void* stream) {
  dark_status st = check_desc(desc, false);
  if (st != DARK_OK) return st;
  const dark_prf_desc& d = *desc;
  if (!M || !dM || !aligned16(M) || !aligned16(dM)) return DARK_ERR_INVALID_ARG;
  const bool tokens = d.B > 0 && d.L > 0;
  if (tokens) {
    if (!q || !k || !v || !omega || !dout || !dq || !dk || !dv) return DARK_ERR_INVALID_ARG;
    const void* ptrs[8] = {q, k, v, omega, dout, dq, dk, dv};
    for (const void* ptr : ptrs)
      if (!aligned16(ptr)) return DARK_ERR_INVALID_ARG;
    if (workspace == nullptr || ws_bytes < dark_prf_bwd_workspace_bytes(desc)) return DARK_ERR_WORKSPACE;
    if (!aligned16(workspace)) return DARK_ERR_INVALID_ARG;
  }
  (void)hipGetLastError();   // launch errors below are ours, not an earlier caller's
  BwdPtrs p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.M = M;
  p.omega = omega;
  p.mask = mask;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dM = dM;
  return launch_bwd(d, p, workspace, stream, nullptr);
}

dark_status dark_prf_decode_step(const dark_prf_desc* desc, const void* q, const void* k, const void* v,
                                 const float* M, const float* omega, float* S, float* z, uint64_t state_tag,
                                 void* out, void* stream) {
  dark_status st = check_desc(desc, true);
  if (st != DARK_OK) return st;
  const dark_prf_desc& d = *desc;
  if (state_tag != d.proj_tag) return DARK_ERR_STALE_STATE;
  if (d.B == 0) return DARK_OK;
  if (!q || !k || !v || !M || !omega || !S || !z || !out) return DARK_ERR_INVALID_ARG;
  if (!aligned16(S) || !aligned16(z) || !aligned16(M) || !aligned16(omega)) return DARK_ERR_INVALID_ARG;
  decode_launcher fn = find_decode_launcher(d.dtype, d.d_h);
  if (!fn) return DARK_ERR_UNSUPPORTED;
  (void)hipGetLastError();   // launch errors below are ours, not an earlier caller's
  return fn(d, q, k, v, M, omega, S, z, out, nullptr, 1, stream);
}

dark_status dark_prf_timing_begin(void) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  drop_records(t);
  t.on = true;
  return DARK_OK;
}

dark_status dark_prf_timing_end(double* ms, int32_t* launches) {
  if (!ms || !launches) return DARK_ERR_INVALID_ARG;
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  for (int i = 0; i < DARK_KERNEL_KINDS; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  dark_status st = DARK_OK;
  for (auto& r : t.recs) {
    float e = 0.f;
    if (hipEventSynchronize(r.second.second) != hipSuccess ||
        hipEventElapsedTime(&e, r.second.first, r.second.second) != hipSuccess) {
      st = DARK_ERR_HIP;
      continue;
    }
    if (r.first >= 0 && r.first < DARK_KERNEL_KINDS) {
      ms[r.first] += e;
      launches[r.first] += 1;
    }
  }
  drop_records(t);
  t.on = false;
  return st;
}

}  // extern "C"
