// Host-side checks of the C ABI for the sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code): every validation path of every
// entry point, with pointers that are never dereferenced on the host and no
// call that reaches a launch.  Exit status = number of failed checks.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "ssmvjp.h"

static int failures = 0;
#define CHECK(expr, want)                                                                       \
  do {                                                                                          \
    const int got_ = (int)(expr);                                                               \
    if (got_ != (int)(want)) {                                                                  \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #expr, got_, (int)(want)); \
      ++failures;                                                                               \
    }                                                                                           \
  } while (0)

static void* fake(int i) { return (void*)(uintptr_t)(0x100000u * (unsigned)(i + 1)); }  // 256-aligned, never read

static void scan_checks() {
  ssmvjp_scan_desc d{2, 64, 4, 8, 16, 2, SSMVJP_DECAY_PER_HEAD, SSMVJP_F32, 0, 0};
  size_t n = 0;
  CHECK(ssm_scan_bwd_workspace(&d, &n), SSMVJP_OK);
  CHECK(n > 0, 1);
  CHECK(ssm_scan_bwd_workspace(nullptr, &n), SSMVJP_EINVAL);
  CHECK(ssm_scan_bwd_workspace(&d, nullptr), SSMVJP_EINVAL);
  ssmvjp_scan_desc bad = d;
  bad.ngroups = 3;
  CHECK(ssm_scan_bwd_workspace(&bad, &n), SSMVJP_EINVAL);
  bad = d;
  bad.headdim = 128;
  bad.dstate = 128;  // LDS limit
  CHECK(ssm_scan_bwd_workspace(&bad, &n), SSMVJP_EUNSUPPORTED);
  bad = d;
  bad.batch = -1;
  CHECK(ssm_scan_bwd_workspace(&bad, &n), SSMVJP_EINVAL);
  size_t need = 0;
  ssm_scan_bwd_workspace(&d, &need);
  void* p[14];
  for (int i = 0; i < 14; ++i) p[i] = fake(i);
  auto call = [&](const ssmvjp_scan_desc* dd, void** q, void* ws, size_t wsb) {
    return ssm_scan_bwd(dd, q[0], (const float*)q[1], (const float*)q[2], q[3], q[4], (const float*)q[5], q[6],
                        (const float*)q[7], q[8], (float*)q[9], q[10], q[11], (float*)q[12], ws, wsb, nullptr);
  };
  CHECK(call(nullptr, p, fake(20), need), SSMVJP_EINVAL);
  void* q[14];
  for (int i = 0; i < 14; ++i) q[i] = p[i];
  q[0] = nullptr;  // x
  CHECK(call(&d, q, fake(20), need), SSMVJP_EINVAL);
  for (int i = 0; i < 14; ++i) q[i] = p[i];
  q[3] = (char*)p[3] + 2;  // misaligned float32 B
  CHECK(call(&d, q, fake(20), need), SSMVJP_EINVAL);
  CHECK(call(&d, p, nullptr, need), SSMVJP_EWORKSPACE);
  CHECK(call(&d, p, fake(20), need - 1), SSMVJP_EWORKSPACE);
  CHECK(call(&d, p, (char*)fake(20) + 16, need), SSMVJP_EWORKSPACE);
  ssmvjp_scan_desc empty = d;
  empty.batch = 0;
  size_t ne = 0;
  CHECK(ssm_scan_bwd_workspace(&empty, &ne), SSMVJP_OK);
  CHECK(call(&empty, p, ne ? fake(20) : nullptr, ne), SSMVJP_OK);  // nothing to do: returns before any launch
  CHECK(ssm_scan_bwd_dA(&d, p[0], (const float*)p[1], (const float*)p[2], p[3], p[4], (const float*)p[5], p[6],
                        (const float*)p[7], p[8], (float*)p[9], p[10], p[11], (float*)p[12], nullptr, fake(20), need,
                        nullptr),
        SSMVJP_EINVAL);  // dA required
}

static void ssd_checks() {
  ssmvjp_ssd_desc d{2, 100, 4, 32, 32, 2, 1, 32, SSMVJP_FORM_MAMBA2, SSMVJP_BF16};
  size_t n = 0;
  CHECK(ssd_chunk_bwd_workspace(&d, &n), SSMVJP_OK);
  ssmvjp_ssd_desc bad = d;
  bad.mimo_rank = 2;  // Mamba-2 form needs M = 1
  CHECK(ssd_chunk_bwd_workspace(&bad, &n), SSMVJP_EINVAL);
  bad = d;
  bad.headdim = 20;  // not a multiple of 16: zero-padded to 32
  CHECK(ssd_chunk_bwd_workspace(&bad, &n), SSMVJP_OK);
  bad.chunk_len = 24;  // the fused chunk length is not padded
  CHECK(ssd_chunk_bwd_workspace(&bad, &n), SSMVJP_EUNSUPPORTED);
  bad = d;
  bad.form = 7;
  CHECK(ssd_chunk_bwd_workspace(&bad, &n), SSMVJP_EINVAL);
  bad = d;
  bad.chunk_len = 0;
  CHECK(ssd_chunk_bwd_workspace(&bad, &n), SSMVJP_EINVAL);
  size_t need = 0;
  ssd_chunk_bwd_workspace(&d, &need);
  void* p[14];
  for (int i = 0; i < 14; ++i) p[i] = fake(i);
  auto call = [&](const ssmvjp_ssd_desc* dd, void** q, void* ws, size_t wsb) {
    return ssd_chunk_bwd(dd, q[0], (const float*)q[1], (const float*)q[2], q[3], q[4], (const float*)q[5], q[6],
                         (const float*)q[7], q[8], (float*)q[9], q[10], q[11], (float*)q[12], ws, wsb, nullptr);
  };
  void* q[14];
  for (int i = 0; i < 14; ++i) q[i] = p[i];
  q[0] = (char*)p[0] + 8;  // x only 8-byte aligned
  CHECK(call(&d, q, fake(20), need), SSMVJP_EINVAL);
  for (int i = 0; i < 14; ++i) q[i] = p[i];
  q[2] = nullptr;  // A required in the Mamba-2 form
  CHECK(call(&d, q, fake(20), need), SSMVJP_EINVAL);
  CHECK(call(&d, p, fake(20), need / 2), SSMVJP_EWORKSPACE);
  ssmvjp_ssd_desc empty = d;
  empty.batch = 0;
  size_t ne = 0;
  CHECK(ssd_chunk_bwd_workspace(&empty, &ne), SSMVJP_OK);
  CHECK(call(&empty, p, ne ? fake(20) : nullptr, ne), SSMVJP_OK);
  CHECK(ssd_chunk_bwd_dA(&d, p[0], (const float*)p[1], (const float*)p[2], p[3], p[4], (const float*)p[5], p[6],
                         (const float*)p[7], p[8], (float*)p[9], p[10], p[11], (float*)p[12], nullptr, fake(20), need,
                         nullptr),
        SSMVJP_EINVAL);
  ssmvjp_ssd_desc raw = d;
  raw.form = SSMVJP_FORM_RAW;
  CHECK(ssd_chunk_bwd_dA(&raw, p[0], (const float*)p[1], nullptr, p[3], p[4], (const float*)p[5], p[6],
                         (const float*)p[7], p[8], (float*)p[9], p[10], p[11], (float*)p[12], (float*)p[13], fake(20),
                         need, nullptr),
        SSMVJP_EINVAL);  // dA needs the Mamba-2 form
  CHECK(ssd_chunk_bwd_states(&d, p[0], (const float*)p[1], (const float*)p[2], p[3], p[4], (const float*)p[5], p[6],
                             (const float*)p[7], nullptr, fake(20), need, nullptr),
        SSMVJP_EINVAL);  // d_s0 required
  CHECK(ssd_chunk_bwd_grads(&d, p[0], (const float*)p[1], (const float*)p[2], p[3], p[4], p[6], nullptr,
                            (float*)p[9], p[10], p[11], fake(20), need, nullptr),
        SSMVJP_EINVAL);  // dx required
  // no-alloc variant: a shape beyond the built-in array is refused up front
  ssmvjp_ssd_desc big{8, 8192, 32, 64, 128, 1, 1, 64, SSMVJP_FORM_MAMBA2, SSMVJP_BF16};
  CHECK(ssd_chunk_bwd_noalloc(&big, p[0], (const float*)p[1], (const float*)p[2], p[3], p[4], (const float*)p[5],
                              p[6], (const float*)p[7], p[8], (float*)p[9], p[10], p[11], (float*)p[12], nullptr),
        SSMVJP_EWORKSPACE);
  bad = d;
  bad.form = 7;
  CHECK(ssd_chunk_bwd_noalloc(&bad, p[0], (const float*)p[1], (const float*)p[2], p[3], p[4], (const float*)p[5],
                              p[6], (const float*)p[7], p[8], (float*)p[9], p[10], p[11], (float*)p[12], nullptr),
        SSMVJP_EINVAL);
  // forward
  size_t nf = 0;
  CHECK(ssd_chunk_fwd_workspace(&d, &nf), SSMVJP_OK);
  CHECK(ssd_chunk_fwd(&d, p[0], (const float*)p[1], (const float*)p[2], p[3], p[4], nullptr, nullptr, nullptr,
                      fake(20), nf, nullptr),
        SSMVJP_EINVAL);  // y required
}

static void delta_checks() {
  ssmvjp_delta_desc d{1, 40, 2, 4, 128, 64, 0.125f, 0};
  size_t n = 0;
  CHECK(delta_rule_bwd_workspace(&d, &n), SSMVJP_OK);
  ssmvjp_delta_desc bad = d;
  bad.nv_heads = 3;
  CHECK(delta_rule_bwd_workspace(&bad, &n), SSMVJP_EINVAL);
  bad = d;
  bad.dk = 64;
  CHECK(delta_rule_bwd_workspace(&bad, &n), SSMVJP_EUNSUPPORTED);
  bad = d;
  bad.reserved = 1;
  CHECK(delta_rule_bwd_workspace(&bad, &n), SSMVJP_EINVAL);
  float* p[14];
  for (int i = 0; i < 14; ++i) p[i] = (float*)fake(i);
  size_t need = 0;
  delta_rule_bwd_workspace(&d, &need);
  CHECK(delta_rule_bwd(&d, p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], p[9], p[10], p[11], nullptr, p[13],
                       fake(20), need, nullptr),
        SSMVJP_EINVAL);  // dbeta required
  CHECK(delta_rule_bwd(&d, p[0], p[1], (float*)((char*)p[2] + 4), p[3], p[4], p[5], p[6], p[7], p[8], p[9], p[10],
                       p[11], p[12], p[13], fake(20), need, nullptr),
        SSMVJP_EINVAL);  // v not 16-byte aligned
  CHECK(delta_rule_bwd_stages(&d, 0, p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], p[9], p[10], p[11], p[12],
                              p[13], fake(20), need, nullptr),
        SSMVJP_EINVAL);  // empty stage mask
  CHECK(delta_rule_bwd_stages(&d, 8, p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], p[9], p[10], p[11], p[12],
                              p[13], fake(20), need, nullptr),
        SSMVJP_EINVAL);  // unknown stage bit
  CHECK(delta_rule_bwd(&d, p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], p[9], p[10], p[11], p[12], p[13],
                       fake(20), need - 256, nullptr),
        SSMVJP_EWORKSPACE);
}

static void misc_checks() {
  CHECK(ssmvjp_version()[0] != 0, 1);
  for (int s = 0; s <= 5; ++s) CHECK(ssmvjp_status_str((ssmvjp_status)s)[0] != 0, 1);
  CHECK(ssmvjp_status_str((ssmvjp_status)99)[0] != 0, 1);
  // debug finiteness mode: the queries grow by the flag's 256 bytes
  ssmvjp_delta_desc d{1, 40, 2, 4, 128, 64, 0.125f, 0};
  size_t off = 0, on = 0;
  unsetenv("SSMVJP_CHECK_FINITE");
  CHECK(delta_rule_bwd_workspace(&d, &off), SSMVJP_OK);
  setenv("SSMVJP_CHECK_FINITE", "1", 1);
  CHECK(delta_rule_bwd_workspace(&d, &on), SSMVJP_OK);
  unsetenv("SSMVJP_CHECK_FINITE");
  CHECK(on == (off + 255) / 256 * 256 + 256, 1);
}

int main() {
  scan_checks();
  ssd_checks();
  delta_checks();
  misc_checks();
  std::printf("abi checks: %d failure(s)\n", failures);
  return failures;
}
