/* Host-side check of libfa's C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitizers.py
 * builds and runs it).  Every entry point is called with problems made of
 * edge values and seeded random fields, and with no device buffers at all
 * (null tensor pointers), so every call ends in host code: a status, a size,
 * or the no-op of an empty problem; none reaches a launch, and no GPU is
 * needed.  The sanitizers abort at the first invalid access or undefined
 * operation (a signed overflow in the size arithmetic, say); the checks below
 * count statuses and sizes that break the contract in fa.h.  Prints "ok" and
 * exits 0 when nothing failed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa.h"

static long fails = 0;
#define EXPECT(cond, ...)                        \
  do {                                           \
    if (!(cond)) {                               \
      if (fails < 20) {                          \
        fprintf(stderr, __VA_ARGS__);            \
        fputc('\n', stderr);                     \
      }                                          \
      ++fails;                                   \
    }                                            \
  } while (0)

/* xorshift64 (Marsaglia, 2003) */
static uint64_t rs = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void) {
  rs ^= rs << 13;
  rs ^= rs >> 7;
  rs ^= rs << 17;
  return rs;
}

static int32_t pick_dim(void) {
  static const int32_t edge[] = {0,     1,       2,       31,      32,           33,
                                 63,    64,      65,      127,     128,          129,
                                 512,   2048,    2049,    65536,   65537,        70000,
                                 1 << 20, 1 << 24, 1 << 30, INT32_MAX - 1, INT32_MAX, -1,
                                 INT32_MIN};
  const uint64_t r = rnd();
  switch (r & 3) {
    case 0: return edge[(r >> 2) % (sizeof edge / sizeof edge[0])];
    case 1: return (int32_t)((r >> 2) % 300);
    case 2: return (int32_t)((r >> 2) % 70000);
    default: return (int32_t)(r >> 32);
  }
}

static float pick_float(void) {
  static const float edge[] = {0.f, 1.f, 0.125f, -0.125f, 1e-30f, 1e30f, 0.5f, 0.999f, -1.f};
  const uint64_t r = rnd();
  switch (r & 3) {
    case 0: return edge[(r >> 2) % (sizeof edge / sizeof edge[0])];
    case 1: return (float)((r >> 8) % 1000) / 999.f;
    case 2: return (r >> 8) & 1 ? INFINITY : NAN;
    default: return 1.f;
  }
}

/* A non-null "device" address for the mask and bias fields: host code only
 * tests these for null and alignment, never reads through them. */
static const void *fake_ptr(void) {
  const uint64_t r = rnd();
  if (r & 1) return NULL;
  return (const void *)(uintptr_t)(0x100000u + ((r >> 1) & 1 ? 16u : 3u));
}

static int is_empty(const fa_problem *p) {
  return p->batch == 0 || p->head_num == 0 || p->seq_q == 0;
}

static void random_problem(fa_problem *p) {
  memset(p, 0, sizeof *p);
  p->batch = pick_dim();
  p->head_num = pick_dim();
  p->seq_q = pick_dim();
  p->seq_k = pick_dim();
  const uint64_t r = rnd();
  p->head_dim = (r & 3) ? (int32_t[]){64, 128, 32, 96}[(r >> 2) & 3] : pick_dim();
  p->layout = (int32_t)((r >> 4) % 3);         /* 2 is invalid */
  p->dtype = (int32_t)((r >> 6) % 5);          /* 4 is invalid */
  p->scale = pick_float();
  p->keep_prob = (r >> 9) & 1 ? 1.f : pick_float();
  p->mask_flags = (uint32_t)((r >> 10) & 1 ? (r >> 11) & 15 : (r >> 11) & 0xff);
  p->num_modalities = (int32_t)((r >> 20) % 11) - 1;
  p->modality_allow_diag = (int32_t)((r >> 24) & 1);
  for (int i = 0; i < 64; ++i) p->modality_allow[i] = (uint8_t)(rnd() & 1);
  p->pse_kind = (int32_t)((r >> 25) % 4);      /* 3 is invalid */
  p->pse_dtype = (int32_t)((r >> 27) % 5);
  p->explicit_mask = (const uint8_t *)fake_ptr();
  p->em_stride_b = (int64_t)rnd() >> ((r >> 30) & 63);
  p->em_stride_h = (r >> 36) & 1 ? 0 : (int64_t)(rnd() % 100000);
  p->em_stride_q = (int64_t)(rnd() % 100000) - 10;
  p->q_modality = (const int8_t *)fake_ptr();
  p->k_modality = (const int8_t *)fake_ptr();
  p->key_valid = (const uint8_t *)fake_ptr();
  p->alibi_slopes = (const float *)fake_ptr();
  p->pse = fake_ptr();
  p->pse_stride_b = (int64_t)rnd() >> ((r >> 40) & 63);
  p->pse_stride_h = (int64_t)(rnd() % 1000) - 1;
  p->pse_stride_q = (int64_t)(rnd() % 1000);
  p->dropout_seed = rnd();
  p->grad_f32 = (int32_t)((r >> 46) % 3);
  p->reserved0 = (r >> 48) % 50 == 0 ? 1 : 0;
  p->dpse = (r >> 54) % 4 == 0 ? (float *)fake_ptr() : NULL;
}

/* A status the call may return without device buffers: never FA_ERR_HIP (no
 * HIP call is reached) and never an unknown code. */
static int plausible(fa_status s) {
  return s == FA_OK || s == FA_ERR_INVALID_ARG || s == FA_ERR_UNSUPPORTED || s == FA_ERR_WORKSPACE;
}

static void check_problem_calls(const fa_problem *p) {
  fa_status s = fa_fwd(p, NULL, NULL, NULL, NULL, NULL, 0);
  EXPECT(plausible(s), "fa_fwd: status %d", (int)s);
  EXPECT(s != FA_OK || is_empty(p), "fa_fwd: ok without tensors on a non-empty problem");

  size_t n = (size_t)-1;
  s = fa_bwd_workspace_size(p, &n);
  EXPECT(plausible(s), "fa_bwd_workspace_size: status %d", (int)s);
  if (s == FA_OK) {
    if (is_empty(p)) {
      EXPECT(n == 0, "workspace of an empty problem: %zu", n);
    } else {
      const double rows = (double)p->batch * p->head_num * p->seq_q;
      EXPECT(n % 256 == 0 && (double)n >= 4.0 * rows && (double)n < 4.0 * rows + 256.0,
             "workspace %zu for %.0f rows", n, rows);
    }
  }
  const fa_status sw = s;

  s = fa_bwd(p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 0);
  EXPECT(plausible(s), "fa_bwd: status %d", (int)s);
  EXPECT(s != FA_OK || is_empty(p), "fa_bwd: ok without tensors on a non-empty problem");
  s = fa_bwd_noalloc(p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0);
  EXPECT(plausible(s), "fa_bwd_noalloc: status %d", (int)s);
  EXPECT(s != FA_OK || is_empty(p), "fa_bwd_noalloc: ok without tensors on a non-empty problem");
  s = fa_bwd_prep(p, NULL, NULL, NULL, n, 0);
  EXPECT(plausible(s), "fa_bwd_prep: status %d", (int)s);
  EXPECT(s != FA_OK || is_empty(p), "fa_bwd_prep: ok without tensors on a non-empty problem");
  s = fa_bwd_main(p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, n, 0);
  EXPECT(plausible(s), "fa_bwd_main: status %d", (int)s);
  EXPECT(s != FA_OK || is_empty(p), "fa_bwd_main: ok without tensors on a non-empty problem");
  s = fa_bwd_post(p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, n, 0);
  EXPECT(plausible(s), "fa_bwd_post: status %d", (int)s);
  EXPECT(s != FA_OK || is_empty(p), "fa_bwd_post: ok without tensors on a non-empty problem");
  /* every entry point validates the problem the same way */
  if (sw == FA_ERR_INVALID_ARG && p->dtype != FA_FP8_E4M3) {
    s = fa_fwd(p, NULL, NULL, NULL, NULL, NULL, 0);
    EXPECT(s == FA_ERR_INVALID_ARG, "fa_fwd %d where the workspace query said invalid", (int)s);
  }

  size_t n8 = (size_t)-1;
  s = fa_fwd_fp8_workspace_size(p, &n8);
  EXPECT(plausible(s), "fa_fwd_fp8_workspace_size: status %d", (int)s);
  EXPECT(s != FA_OK || n8 % 256 == 0, "fp8 workspace %zu", n8);
  s = fa_fwd_fp8(p, NULL, NULL, NULL, 1.f, 1.f, 1.f, NULL, NULL, NULL, 0, 0);
  EXPECT(plausible(s), "fa_fwd_fp8: status %d", (int)s);
  EXPECT(s != FA_OK || is_empty(p), "fa_fwd_fp8: ok without tensors on a non-empty problem");
}

static void check_maxsim(void) {
  fa_maxsim_problem m;
  memset(&m, 0, sizeof m);
  m.batch = pick_dim();
  m.len_q = pick_dim();
  m.len_d = pick_dim();
  const uint64_t r = rnd();
  m.dim = (r & 1) ? (int32_t[]){128, 768, 256, 64}[(r >> 1) & 3] : pick_dim();
  m.dtype = (int32_t)((r >> 3) % 5);
  m.pad0 = (r >> 6) % 40 == 0;
  m.q_valid = (const uint8_t *)fake_ptr();
  m.d_valid = (const uint8_t *)fake_ptr();
  const fa_status s = fa_maxsim(&m, NULL, NULL, NULL, NULL, 0);
  EXPECT(plausible(s), "fa_maxsim: status %d", (int)s);
  EXPECT(s != FA_OK || m.batch == 0, "fa_maxsim: ok without tensors, batch %d", m.batch);
}

int main(int argc, char **argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 200000;
  EXPECT(fa_abi_version() == FA_ABI_VERSION, "ABI version %d", fa_abi_version());
  for (int c = -8; c <= 4; ++c) EXPECT(fa_status_str((fa_status)c) != NULL, "status_str(%d)", c);

  /* a null problem is refused everywhere */
  size_t n = 0;
  EXPECT(fa_fwd(NULL, NULL, NULL, NULL, NULL, NULL, 0) == FA_ERR_INVALID_ARG, "null problem: fwd");
  EXPECT(fa_bwd_workspace_size(NULL, &n) == FA_ERR_INVALID_ARG, "null problem: workspace");
  EXPECT(fa_bwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 0) ==
             FA_ERR_INVALID_ARG, "null problem: bwd");
  EXPECT(fa_maxsim(NULL, NULL, NULL, NULL, NULL, 0) == FA_ERR_INVALID_ARG, "null problem: maxsim");

  /* sizes whose products overflow 64-bit signed arithmetic if taken naively */
  {
    fa_problem p;
    memset(&p, 0, sizeof p);
    p.batch = INT32_MAX;
    p.head_num = INT32_MAX;
    p.seq_q = (1 << 24) - 1;
    p.seq_k = (1 << 24) - 1;
    p.head_dim = 64;
    p.layout = FA_BNSD;
    p.dtype = FA_BF16;
    p.scale = 0.125f;
    p.keep_prob = 1.f;
    EXPECT(fa_bwd_workspace_size(&p, &n) == FA_ERR_UNSUPPORTED, "B = H = 2^31 - 1 accepted");
    p.seq_q = 0;   /* keys without queries: the backward would zero dK and dV */
    EXPECT(fa_bwd(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 0) ==
               FA_ERR_UNSUPPORTED, "B = H = 2^31 - 1 with S_q = 0 accepted");
    p.dtype = FA_FP8_E4M3;
    p.seq_q = 1;
    EXPECT(fa_fwd_fp8_workspace_size(&p, &n) == FA_ERR_UNSUPPORTED, "fp8: B = H = 2^31 - 1 accepted");
  }

  for (long it = 0; it < iters; ++it) {
    fa_problem p;
    random_problem(&p);
    check_problem_calls(&p);
    check_maxsim();
  }
  if (fails) {
    fprintf(stderr, "%ld failed checks\n", fails);
    return 1;
  }
  printf("ok\n");
  return 0;
}
