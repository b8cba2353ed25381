// Host-side fuzz driver of the darkprf C ABI, built with AddressSanitizer on
// the host code (tests/test_host_asan.py builds and runs it on the CPU).
//
// Random descriptors, valid and invalid, go through every sizing call and
// through the compute entry points in ways that must return before anything
// is queued; the host generators and the projection lifecycle run on random
// sizes.  Any out-of-bounds access, use after free or overflow trap in the
// host code stops the run with a sanitizer report; a broken property returns 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "darkprf.h"

static uint64_t rng_state = 0x243F6A8885A308D3ULL;
static uint64_t next64() {   // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1DULL;
}
static int32_t pick(const int32_t* v, int n) { return v[next64() % (uint64_t)n]; }
static int32_t any32() {
  static const int32_t edge[] = {0, 1, -1, 2, 16, 64, 255, 256, 257, 4096, 65536, 1 << 20, 1 << 30, 2147483647,
                                 -2147483647 - 1};
  return (next64() & 1) ? pick(edge, 15) : (int32_t)next64();
}

static int fails = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      fprintf(stderr, "property failed at line %d: %s\n", __LINE__, #c); \
      ++fails;                                                          \
    }                                                                   \
  } while (0)

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 20000;
  void* fake = reinterpret_cast<void*>((uintptr_t)1 << 20);
  const float* ff = reinterpret_cast<const float*>(fake);
  for (int it = 0; it < iters; ++it) {
    dark_prf_desc d;
    memset(&d, 0, sizeof(d));
    const bool plausible = (it & 1) == 0;
    if (plausible) {
      static const int32_t dhs[] = {16, 32, 64, 128, 256}, hs[] = {1, 2, 3, 4, 8, 16};
      d.B = (int32_t)(next64() % 65);
      d.H = pick(hs, 6);
      d.H_kv = (next64() & 1) ? d.H : 1;
      d.L = (int32_t)(next64() % 70000);
      d.d_h = pick(dhs, 5);
      d.m = 16 * (int32_t)(1 + next64() % 80);
      d.r = (int32_t)(1 + next64() % 256);
      d.dtype = (int32_t)(next64() % 2);
      d.causal = (int32_t)(next64() % 2);
      d.m_per_head = (int32_t)(next64() % 2);
      d.omega_per_head = (int32_t)(next64() % 2);
      const int64_t L1 = d.L > 0 ? d.L : 1;
      const int64_t q[3] = {(int64_t)d.H * L1 * d.d_h, L1 * d.d_h, d.d_h};
      const int64_t k[3] = {(int64_t)d.H_kv * L1 * d.d_h, L1 * d.d_h, d.d_h};
      memcpy(d.q_str, q, sizeof(q));
      memcpy(d.o_str, q, sizeof(q));
      memcpy(d.k_str, k, sizeof(k));
      memcpy(d.v_str, k, sizeof(k));
    } else {
      d.B = any32();
      d.H = any32();
      d.H_kv = any32();
      d.L = any32();
      d.d_h = any32();
      d.m = any32();
      d.r = any32();
      d.dtype = any32() & 3;
      d.causal = any32() & 3;
      d.m_per_head = any32() & 3;
      d.omega_per_head = any32() & 3;
      for (int i = 0; i < 3; ++i) {
        d.q_str[i] = (int64_t)next64() >> (next64() % 64);
        d.k_str[i] = (int64_t)next64() >> (next64() % 64);
        d.v_str[i] = (int64_t)next64() >> (next64() % 64);
        d.o_str[i] = (int64_t)next64() >> (next64() % 64);
      }
    }
    const size_t ws = dark_prf_workspace_bytes(&d);
    const size_t ex = dark_prf_exact_workspace_bytes(&d);
    const size_t bw = dark_prf_bwd_workspace_bytes(&d);
    const int32_t thr = (int32_t)(next64() % 70000);
    const int32_t mode = dark_prf_auto_mode(&d, thr);
    const size_t aw = dark_prf_auto_workspace_bytes(&d, thr);
    CHECK((ws == 0) == (ex == 0));
    CHECK(ws % 16 == 0 && ex % 16 == 0 && bw % 16 == 0);
    if (ws == 0) {   // rejected: every compute call refuses it too, before any launch
      CHECK(mode == -1 && aw == 0);
      CHECK(dark_prf_fwd(&d, fake, fake, fake, ff, ff, nullptr, fake, nullptr, nullptr, fake, (size_t)1 << 40,
                         nullptr) != DARK_OK);
      CHECK(dark_prf_fwd_noalloc(&d, fake, fake, fake, ff, ff, nullptr, fake, nullptr, nullptr, nullptr) != DARK_OK);
      CHECK(dark_prf_exact_fwd(&d, fake, fake, fake, ff, nullptr, fake, fake, (size_t)1 << 40, nullptr) != DARK_OK);
      CHECK(dark_prf_auto_fwd(&d, thr, fake, fake, fake, ff, ff, nullptr, fake, fake, (size_t)1 << 40, nullptr) !=
            DARK_OK);
      continue;
    }
    CHECK(mode == (d.L <= thr ? 1 : 0));
    CHECK(aw == (mode ? ex : ws));
    if (d.B > 0 && d.L > 0) {   // a short workspace or a missing pointer returns before any launch
      CHECK(dark_prf_fwd(&d, fake, fake, fake, ff, ff, nullptr, fake, nullptr, nullptr, fake, ws - 1, nullptr) ==
            DARK_ERR_WORKSPACE);
      CHECK(dark_prf_fwd(&d, nullptr, fake, fake, ff, ff, nullptr, fake, nullptr, nullptr, fake, ws, nullptr) ==
            DARK_ERR_INVALID_ARG);
      CHECK(dark_prf_exact_fwd(&d, fake, fake, fake, ff, nullptr, fake, fake, ex - 1, nullptr) == DARK_ERR_WORKSPACE);
      CHECK(dark_prf_bwd(&d, fake, fake, fake, ff, ff, nullptr, fake, fake, fake, fake, reinterpret_cast<float*>(fake),
                         fake, bw - 1, nullptr) == DARK_ERR_WORKSPACE);
      CHECK(dark_prf_context_state(&d, fake, fake, ff, ff, nullptr, nullptr, nullptr, fake, ws, nullptr) ==
            DARK_ERR_INVALID_ARG);
      if (ws > DARK_PRF_SCRATCH_BYTES)
        CHECK(dark_prf_fwd_noalloc(&d, fake, fake, fake, ff, ff, nullptr, fake, nullptr, nullptr, nullptr) ==
              DARK_ERR_WORKSPACE);
    }
  }
  // host generators, tags and the projection lifecycle on random sizes
  for (int it = 0; it < 300; ++it) {
    const int32_t m = (int32_t)(1 + next64() % 300), r = (int32_t)(1 + next64() % 70), H = (int32_t)(1 + next64() % 4);
    const int32_t orth = (int32_t)(next64() & 1);
    std::vector<float> om((size_t)H * m * r);
    CHECK(dark_prf_omega(next64(), m, r, orth, om.data()) == DARK_OK);
    CHECK(dark_prf_omega_per_head(next64(), H, m, r, orth, om.data()) == DARK_OK);
    CHECK(dark_prf_omega(1, 0, r, orth, om.data()) == DARK_ERR_INVALID_ARG);
    (void)dark_prf_proj_tag(next64(), m, r, orth);
    (void)dark_prf_proj_tag_per_head(next64(), H, m, r, orth);
    dark_prf_projection p;
    CHECK(dark_prf_projection_init(&p, next64(), m, r, orth, (int32_t)(next64() % 5), (int32_t)(next64() & 1)) ==
          DARK_OK);
    for (int s = 0; s < 20; ++s) {
      (void)dark_prf_projection_forward(&p, (int32_t)(next64() & 1));
      if ((next64() & 7) == 0) (void)dark_prf_projection_redraw(&p, (int32_t)(next64() & 1));
      if ((next64() & 7) == 0) (void)dark_prf_projection_fix(&p, (int32_t)(next64() & 1));
    }
    CHECK(dark_prf_omega_device_workspace_bytes(m, r, orth) % 8 == 0);
  }
  CHECK(dark_prf_status_str((dark_status)77) != nullptr);
  printf("fuzz_host: %d iterations, %d property failures\n", iters, fails);
  return fails ? 1 : 0;
}
