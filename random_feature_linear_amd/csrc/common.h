// Shared host/device definitions of the darkprf HIP library (gfx950).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/darkprf.h"

namespace dk {

// Arguments of one dark_prf_fwd call after validation.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int64_t qs[3], ks[3], vs[3], os[3];
  const uint8_t* mask;
  const float* M;
  const float* omega;
  float* S_out;
  float* z_out;
  float* kshift;   // per-key shifts in the workspace (folded path), or null
  const uint8_t* qmask;   // cross-attention query mask [B][L] (nonzero = valid), or null
  const float* S_in;      // cross-attention context summary S [B][H][m][d_h], z [B][H][m]
  const float* z_in;
  int B, H, H_kv, L, m, r, causal, m_per_head, omega_per_head;
};

// The exponent omega_j . u of a feature can be formed from the projected token
// u = M' x (r-dimensional), or with the projection folded into omega, as
// W'_j . x with W' = omega' M' (m x d_h, one per geometry matrix).  With hi/lo
// bf16 operands the folded form costs 4 m d_h flops per token (plus 4 r d_h
// for |u|^2) against 4 r d_h + 6 r m, so it is taken when d_h < 1.5 r.
constexpr bool fold_exponent(int elem_bytes, int d_h, int r16) { return elem_bytes == 2 && 2 * d_h < 3 * 16 * r16; }

// What one call runs: the whole forward; the key side and its sum only, with the
// summary exported (a cross-attention context); or the query side against a
// summary the caller passes in.
enum PlanMode { kPlanForward = 0, kPlanContext = 1, kPlanCross = 2 };

// How one call is cut into kernels; all sizes derived on the host.
struct Plan {
  int DH;      // head dimension (template value)
  int R16;     // geometry rank in 16-wide blocks, rounded up to 1, 2, 4, 8 or 16
  int FB;      // 32-feature blocks (ceil(m / 32))
  int HM;      // number of geometry matrices M (H or 1)
  int HO;      // number of projections omega (H or 1)
  int HW;      // number of folded operands W' = omega' M' (H if either is per head, else 1)
  int fold;    // exponent from W' x (see fold_exponent)
  int kshift;  // folded path with per-key shifts precomputed once (kshift_kernel)
  int mode;    // kPlanForward, kPlanContext (key side and sum only) or kPlanCross (query side on a given state)
  int BH;      // B * H
  // key-side state kernel
  int span1;   // tokens per unit (a chunk when causal, an L-split otherwise)
  int NU;      // units per (b, h)
  int FBW;     // 32-feature blocks per wave
  int NF;      // feature slices per unit (each slice = 4 waves * FBW blocks)
  int UPW;     // consecutive units per key-side workgroup (tiled kernel; states stored unit by unit)
  // query-side output kernel
  int NQB;     // 32-token query blocks per wave
  int tile2;   // queries per workgroup (4 waves * 32 * NQB); equals span1 when causal
  int NT2;     // query tiles per (b, h)
  // workspace (bytes from the base pointer)
  size_t off_mfrag, off_ofrag, off_sdelta, off_sfrag, off_zdelta, off_zsum, off_kshift, total;
  int elem;    // bytes per element of q/k/v (2 or 4)
  int stream_states;   // per-unit states too large for L2: accessed non-temporally
};

// Workspace of the exact-attention path: the M' fragments, the projected rows
// of q and k (hi/lo operand fragments, 32-token blocks), and, when the keys of
// a query tile are split into runs of KS key tiles, the partial results of
// every run (O_s [128][d_h], m_s and l_s [128], fp32).  The keys are split when
// one workgroup per query tile would leave most compute units idle.
// key tiles per run when the keys are split (measured at L = 2048, 16 heads:
// 79 us per forward against 82 with runs of 4, 86 with 8 and 102 unsplit)
constexpr int kExactKS = 2;
struct ExactLayout {
  size_t off_mfrag, off_ufrag, off_part, total;
  int NBLK;             // 32-token blocks per sequence
  int KS;               // key tiles per run (0: no split)
  int splits_per_head;  // runs over all query tiles of one (b, h)
};
inline ExactLayout exact_layout(int B, int H, int L, int d_h, int R16, int HM, int elem, int causal) {
  ExactLayout e;
  const int NM = elem == 2 ? 2 : 1;
  const size_t frag = 64 * 8;
  e.NBLK = (L + 31) / 32;
  e.off_mfrag = 0;
  size_t off = (size_t)HM * ((R16 + 1) / 2) * (d_h / 16) * NM * frag * elem;
  off = (off + 255) & ~(size_t)255;
  e.off_ufrag = off;
  off += (size_t)2 * B * H * e.NBLK * R16 * NM * frag * elem;
  off = (off + 255) & ~(size_t)255;
  const int NT = (L + 127) / 128;
  const long BH = (long)B * H;
  e.KS = (BH * NT < 512 && NT > 4) ? kExactKS : 0;
  auto runs = [&](int nt) {   // runs of kExactKS key tiles over all query tiles of one (b, h)
    int n = 0;
    for (int t = 0; t < nt; ++t) n += causal ? t / kExactKS + 1 : (nt + kExactKS - 1) / kExactKS;
    return n;
  };
  e.splits_per_head = e.KS > 0 ? runs(NT) : 0;
  // partials reserved for the longest split plan up to this length (equal to the
  // plan's own when it splits), so that the workspace never shrinks as L grows
  const long nt_split = BH > 0 ? (511 / BH < NT ? 511 / BH : NT) : 0;
  const int reserve = nt_split > 4 ? runs((int)nt_split) : 0;
  e.off_part = off;
  off += (size_t)BH * (reserve > e.splits_per_head ? reserve : e.splits_per_head) * (128 * d_h + 2 * 128) *
         sizeof(float);
  e.total = (off + 255) & ~(size_t)255;
  return e;
}

// Optional per-kernel timing (dark_prf_timing_begin / _end): records a HIP
// event pair on `stream` around one launch while timing is on.
enum KernelKind { kPrep = 0, kKState = 1, kScan = 2, kQOut = 3, kDecode = 4, kShift = 5, kBwdGemm = 6, kBwdAux = 7 };
struct KernelTimer {
  KernelTimer(int kind, void* stream);
  ~KernelTimer();
  int kind;
  void* stream;
  void* ev0;
  void* ev1;
};

// One launcher per (element type, head dimension, rank blocks); defined in the
// instantiation units.
typedef dark_status (*fwd_launcher)(const FwdArgs&, const Plan&, void* ws, void* stream);
fwd_launcher find_fwd_launcher(int dtype, int d_h, int r16);

// The random projection on the device (omega_device.hip).
size_t omega_device_ws_bytes(int m, int r, int orthogonal);
dark_status launch_omega_device(uint64_t seed, int m, int r, int orthogonal, float* omega, void* ws, void* stream);

// update = 1: one decode step (S and z updated in place); update = 0: the
// read-only cross-attention step (k, v unused; qmask [N] or null).
typedef dark_status (*decode_launcher)(const dark_prf_desc&, const void* q, const void* k,
                                       const void* v, const float* M, const float* omega,
                                       float* S, float* z, void* out, const uint8_t* qmask,
                                       int update, void* stream);
decode_launcher find_decode_launcher(int dtype, int d_h);

// The backward pass (bwd.hip): device pointers of one call.
struct BwdPtrs {
  const void* q;
  const void* k;
  const void* v;
  const float* M;
  const float* omega;
  const uint8_t* mask;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dM;
};
size_t bwd_ws_bytes(const dark_prf_desc& d);
// flops (optional): the multiply-adds of the matrix products queued, times 2
dark_status launch_bwd(const dark_prf_desc& d, const BwdPtrs& p, void* ws, void* stream, double* flops);

}  // namespace dk
