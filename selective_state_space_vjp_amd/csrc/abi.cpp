// abi.cpp -- the C ABI of libssmvjp: argument validation, workspace sizing and
// dispatch to the kernel launchers.  Validation runs on the host and returns
// before anything is enqueued; nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>

#include "../../include/ssmvjp.h"
#include "kernels.h"

using namespace ssmvjp;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t big_elem(int32_t dtype) { return dtype == SSMVJP_BF16 ? 2 : 4; }

bool valid_dtype(int32_t dtype) { return dtype == SSMVJP_F32 || dtype == SSMVJP_BF16; }

ssmvjp_status scan_check(const ssmvjp_scan_desc* d) {
  if (!d) return SSMVJP_EINVAL;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 || d->ngroups <= 0)
    return SSMVJP_EINVAL;
  if (d->nheads % d->ngroups) return SSMVJP_EINVAL;
  if (d->decay != SSMVJP_DECAY_PER_HEAD && d->decay != SSMVJP_DECAY_PER_STATE) return SSMVJP_EINVAL;
  if (!valid_dtype(d->dtype) || d->ckpt_every < 0 || d->reserved != 0) return SSMVJP_EINVAL;
  if (d->dstate > 1024 || d->headdim * d->dstate > 32768) return SSMVJP_EUNSUPPORTED;
  const SeqPlan plan = seq_plan(*d);
  if ((int64_t)plan.NPG * d->dstate > 1024) return SSMVJP_EUNSUPPORTED;
  if (seq_lds_bytes(*d, plan) > 64 * 1024) return SSMVJP_EUNSUPPORTED;
  if (d->batch * d->nheads > 0x7fffffff) return SSMVJP_EUNSUPPORTED;
  return SSMVJP_OK;
}

ssmvjp_status ssd_check(const ssmvjp_ssd_desc* d) {
  if (!d) return SSMVJP_EINVAL;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 || d->ngroups <= 0 ||
      d->mimo_rank <= 0 || d->chunk_len <= 0)
    return SSMVJP_EINVAL;
  if (d->nheads % d->ngroups) return SSMVJP_EINVAL;
  if (d->form != SSMVJP_FORM_MAMBA2 && d->form != SSMVJP_FORM_RAW) return SSMVJP_EINVAL;
  if (d->form == SSMVJP_FORM_MAMBA2 && d->mimo_rank != 1) return SSMVJP_EINVAL;
  if (!valid_dtype(d->dtype)) return SSMVJP_EINVAL;
  if (!ssd_shape_supported(*d) && !ssd_pad_supported(*d)) return SSMVJP_EUNSUPPORTED;
  return SSMVJP_OK;
}

// workspace of the chunked backward: its plan, or the zero-padded problem's
size_t ssd_bytes(const ssmvjp_ssd_desc& d) {
  return ssd_shape_supported(d) ? ssd_plan(d).bytes : ssd_pad_workspace_bytes(d);
}
size_t ssd_fwd_bytes(const ssmvjp_ssd_desc& d) {
  return ssd_fwd_shape_supported(d) ? ssd_fwd_workspace_bytes(d) : ssd_fwd_pad_workspace_bytes(d);
}

ssmvjp_status delta_check(const ssmvjp_delta_desc* d) {
  if (!d) return SSMVJP_EINVAL;
  if (d->batch < 0 || d->seqlen < 0 || d->nqk_heads <= 0 || d->nv_heads <= 0 || d->dk <= 0 || d->dv <= 0)
    return SSMVJP_EINVAL;
  if (d->nv_heads % d->nqk_heads || d->reserved != 0) return SSMVJP_EINVAL;
  if (!delta_shape_supported(*d)) return SSMVJP_EUNSUPPORTED;
  return SSMVJP_OK;
}

ssmvjp_status hip_status(hipError_t e) { return e == hipSuccess ? SSMVJP_OK : SSMVJP_EHIP; }

// ---- debug finiteness mode (SSMVJP_CHECK_FINITE set and not "0") ----
// The flag lives in FLAG_BYTES at the end of the workspace, after the plan's
// own bytes rounded up to 256; the workspace queries include it while the
// mode is on.
constexpr size_t FLAG_BYTES = 256;

bool check_finite_on() {
  const char* e = std::getenv("SSMVJP_CHECK_FINITE");
  return e && e[0] && std::strcmp(e, "0") != 0;
}
size_t round256(size_t n) { return (n + 255) / 256 * 256; }
size_t with_flag(size_t plan_bytes) { return check_finite_on() ? round256(plan_bytes) + FLAG_BYTES : plan_bytes; }

struct OutSpan {
  const void* p;
  int64_t n;
  bool bf16;
};

// After the launches: clear the flag, scan every output, read the flag back
// (this synchronises the stream) and turn a raised flag into ENONFINITE.
template <size_t K>
ssmvjp_status finite_check(void* workspace, size_t plan_bytes, const OutSpan (&outs)[K], hipStream_t stream) {
  unsigned* flag = (unsigned*)((char*)workspace + round256(plan_bytes));
  launch_flag_clear(flag, stream);
  for (const OutSpan& o : outs) launch_nonfinite_check(o.p, o.n, o.bf16, flag, stream);
  unsigned host = 0;
  if (hipMemcpyAsync(&host, flag, sizeof(host), hipMemcpyDeviceToHost, stream) != hipSuccess) return SSMVJP_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return SSMVJP_EHIP;
  return host ? SSMVJP_ENONFINITE : SSMVJP_OK;
}

}  // namespace

extern "C" {

const char* ssmvjp_version(void) { return "0.1.0"; }

const char* ssmvjp_status_str(ssmvjp_status status) {
  // callers (C, ctypes) may pass any int: read the bits as an int, since
  // loading an out-of-range value through the C++ enum type is undefined
  int s;
  std::memcpy(&s, &status, sizeof s);
  switch (s) {
    case SSMVJP_OK: return "ok";
    case SSMVJP_EINVAL: return "invalid argument";
    case SSMVJP_EUNSUPPORTED: return "unsupported shape or option";
    case SSMVJP_EWORKSPACE: return "workspace missing or too small";
    case SSMVJP_EHIP: return "HIP runtime error";
    case SSMVJP_ENONFINITE: return "non-finite value in an output (SSMVJP_CHECK_FINITE)";
  }
  return "unknown status";
}

// ------------------------------- ssm_scan_bwd -------------------------------

ssmvjp_status ssm_scan_bwd_workspace(const ssmvjp_scan_desc* desc, size_t* bytes) {
  if (!bytes) return SSMVJP_EINVAL;
  ssmvjp_status s = scan_check(desc);
  if (s != SSMVJP_OK) return s;
  *bytes = with_flag(seq_plan(*desc).bytes);
  return SSMVJP_OK;
}

static ssmvjp_status scan_run(const ssmvjp_scan_desc* desc, const void* x, const float* dt, const float* A,
                              const void* B, const void* C, const float* s0, const void* dy, const float* ds_final,
                              void* dx, float* d_dt, void* dB, void* dC, float* d_s0, float* dA, void* workspace,
                              size_t workspace_bytes, void* stream) {
  ssmvjp_status s = scan_check(desc);
  if (s != SSMVJP_OK) return s;
  const ssmvjp_scan_desc& d = *desc;
  const size_t be = big_elem(d.dtype);
  const bool has_tokens = d.batch * d.seqlen > 0;
  const bool has_state = d.batch > 0;
  if (has_tokens && (!x || !dt || !B || !C || !dy || !dx || !d_dt || !dB || !dC)) return SSMVJP_EINVAL;
  if (has_state && (!A || !d_s0)) return SSMVJP_EINVAL;
  const void* pa[] = {x, B, C, dy, dx, dB, dC};
  for (const void* p : pa)
    if (p && !aligned(p, be)) return SSMVJP_EINVAL;
  const void* pf[] = {dt, A, s0, ds_final, d_dt, d_s0, dA};
  for (const void* p : pf)
    if (p && !aligned(p, 4)) return SSMVJP_EINVAL;
  const SeqPlan plan = seq_plan(d);
  const size_t need = with_flag(plan.bytes);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return SSMVJP_EWORKSPACE;
  if (!has_state) return SSMVJP_OK;
  SeqPointers ptr{x, dt, A, B, C, s0, dy, ds_final, dx, d_dt, dB, dC, d_s0, workspace, dA};
  s = hip_status(launch_seq_bwd(d, plan, ptr, (hipStream_t)stream));
  if (s != SSMVJP_OK || !check_finite_on()) return s;
  const bool bf = d.dtype == SSMVJP_BF16;
  const int64_t nx = d.batch * d.seqlen * d.nheads * d.headdim, nbc = d.batch * d.seqlen * d.ngroups * d.dstate;
  const OutSpan outs[] = {{dx, nx, bf}, {d_dt, d.batch * d.seqlen * d.nheads, false}, {dB, nbc, bf}, {dC, nbc, bf},
                          {d_s0, d.batch * d.nheads * d.headdim * d.dstate, false},
                          {dA, dA ? d.nheads * (d.decay == SSMVJP_DECAY_PER_STATE ? d.dstate : 1) : 0, false}};
  return finite_check(workspace, plan.bytes, outs, (hipStream_t)stream);
}

ssmvjp_status ssm_scan_bwd(const ssmvjp_scan_desc* desc, const void* x, const float* dt, const float* A,
                           const void* B, const void* C, const float* s0, const void* dy, const float* ds_final,
                           void* dx, float* d_dt, void* dB, void* dC, float* d_s0, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return scan_run(desc, x, dt, A, B, C, s0, dy, ds_final, dx, d_dt, dB, dC, d_s0, nullptr, workspace,
                  workspace_bytes, stream);
}

ssmvjp_status ssm_scan_bwd_dA(const ssmvjp_scan_desc* desc, const void* x, const float* dt, const float* A,
                              const void* B, const void* C, const float* s0, const void* dy, const float* ds_final,
                              void* dx, float* d_dt, void* dB, void* dC, float* d_s0, float* dA, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (desc && desc->batch > 0 && !dA) return SSMVJP_EINVAL;
  return scan_run(desc, x, dt, A, B, C, s0, dy, ds_final, dx, d_dt, dB, dC, d_s0, dA, workspace, workspace_bytes,
                  stream);
}

// ------------------------------- ssd_chunk_bwd ------------------------------

ssmvjp_status ssd_chunk_bwd_workspace(const ssmvjp_ssd_desc* desc, size_t* bytes) {
  if (!bytes) return SSMVJP_EINVAL;
  ssmvjp_status s = ssd_check(desc);
  if (s != SSMVJP_OK) return s;
  *bytes = with_flag(ssd_bytes(*desc));
  return SSMVJP_OK;
}

static ssmvjp_status ssd_run(const ssmvjp_ssd_desc* desc, const void* x_or_v, const float* dt_or_da,
                             const float* A, const void* B, const void* C, const float* s0, const void* dy,
                             const float* ds_final, void* dx_or_dv, float* d_dt_or_dda, void* dB, void* dC,
                             float* d_s0, float* dA, void* workspace, size_t workspace_bytes, void* stream,
                             int stages) {
  ssmvjp_status s = ssd_check(desc);
  if (s != SSMVJP_OK) return s;
  const ssmvjp_ssd_desc& d = *desc;
  const bool has_tokens = d.batch * d.seqlen > 0;
  const bool has_state = d.batch > 0;
  const bool states = stages & SSD_STAGE_STATES, grads = stages & SSD_STAGE_GRADS;
  if (has_tokens && (!x_or_v || !dt_or_da || !B || !C || !dy)) return SSMVJP_EINVAL;
  if (has_tokens && grads && (!dx_or_dv || !d_dt_or_dda || !dB || !dC)) return SSMVJP_EINVAL;
  if (has_state && states && !d_s0) return SSMVJP_EINVAL;
  if (d.form == SSMVJP_FORM_MAMBA2 && has_tokens && !A) return SSMVJP_EINVAL;
  // 16-byte alignment lets the kernels use vector loads on the big tensors
  const void* pa[] = {x_or_v, B, C, dy, dx_or_dv, dB, dC};
  for (const void* p : pa)
    if (p && !aligned(p, 16)) return SSMVJP_EINVAL;
  const void* pf[] = {dt_or_da, A, s0, ds_final, d_dt_or_dda, d_s0, dA};
  for (const void* p : pf)
    if (p && !aligned(p, 4)) return SSMVJP_EINVAL;
  const size_t plan_bytes = ssd_bytes(d), need = with_flag(plan_bytes);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return SSMVJP_EWORKSPACE;
  if (!has_state) return SSMVJP_OK;
  SsdPointers ptr{x_or_v, dt_or_da, A, B, C, s0, dy, ds_final, dx_or_dv, d_dt_or_dda, dB, dC, d_s0, workspace, dA};
  s = hip_status(ssd_shape_supported(d) ? launch_ssd_bwd(d, ssd_plan(d), ptr, (hipStream_t)stream, stages)
                                        : launch_ssd_bwd_padded(d, ptr, (hipStream_t)stream, stages));
  if (s != SSMVJP_OK || !check_finite_on()) return s;
  const bool bf = d.dtype == SSMVJP_BF16;
  const int64_t nx = d.batch * d.seqlen * d.mimo_rank * d.nheads * d.headdim;
  const int64_t nbc = d.batch * d.seqlen * d.mimo_rank * d.ngroups * d.dstate;
  const OutSpan outs[] = {{grads ? dx_or_dv : nullptr, nx, bf},
                          {grads ? d_dt_or_dda : nullptr, d.batch * d.seqlen * d.nheads, false},
                          {grads ? dB : nullptr, nbc, bf}, {grads ? dC : nullptr, nbc, bf},
                          {states ? d_s0 : nullptr, d.batch * d.nheads * d.headdim * d.dstate, false},
                          {grads ? dA : nullptr, dA ? d.nheads : 0, false}};
  return finite_check(workspace, plan_bytes, outs, (hipStream_t)stream);
}

ssmvjp_status ssd_chunk_bwd(const ssmvjp_ssd_desc* desc, const void* x_or_v, const float* dt_or_da,
                            const float* A, const void* B, const void* C, const float* s0, const void* dy,
                            const float* ds_final, void* dx_or_dv, float* d_dt_or_dda, void* dB, void* dC,
                            float* d_s0, void* workspace, size_t workspace_bytes, void* stream) {
  return ssd_run(desc, x_or_v, dt_or_da, A, B, C, s0, dy, ds_final, dx_or_dv, d_dt_or_dda, dB, dC, d_s0, nullptr,
                 workspace, workspace_bytes, stream, SSD_STAGE_ALL);
}

ssmvjp_status ssd_chunk_bwd_dA(const ssmvjp_ssd_desc* desc, const void* x, const float* dt, const float* A,
                               const void* B, const void* C, const float* s0, const void* dy, const float* ds_final,
                               void* dx, float* d_dt, void* dB, void* dC, float* d_s0, float* dA, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (desc && desc->form != SSMVJP_FORM_MAMBA2) return SSMVJP_EINVAL;  // dA needs the (x, dt, A) form
  if (desc && desc->batch > 0 && !dA) return SSMVJP_EINVAL;
  return ssd_run(desc, x, dt, A, B, C, s0, dy, ds_final, dx, d_dt, dB, dC, d_s0, dA, workspace, workspace_bytes,
                 stream, SSD_STAGE_ALL);
}

ssmvjp_status ssd_chunk_bwd_states(const ssmvjp_ssd_desc* desc, const void* x_or_v, const float* dt_or_da,
                                   const float* A, const void* B, const void* C, const float* s0, const void* dy,
                                   const float* ds_final, float* d_s0, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return ssd_run(desc, x_or_v, dt_or_da, A, B, C, s0, dy, ds_final, nullptr, nullptr, nullptr, nullptr, d_s0,
                 nullptr, workspace, workspace_bytes, stream, SSD_STAGE_STATES);
}

ssmvjp_status ssd_chunk_bwd_grads(const ssmvjp_ssd_desc* desc, const void* x_or_v, const float* dt_or_da,
                                  const float* A, const void* B, const void* C, const void* dy, void* dx_or_dv,
                                  float* d_dt_or_dda, void* dB, void* dC, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return ssd_run(desc, x_or_v, dt_or_da, A, B, C, nullptr, dy, nullptr, dx_or_dv, d_dt_or_dda, dB, dC, nullptr,
                 nullptr, workspace, workspace_bytes, stream, SSD_STAGE_GRADS);
}

// ------------------------------- ssd_chunk_fwd ------------------------------

namespace {
ssmvjp_status ssd_fwd_check(const ssmvjp_ssd_desc* desc) {
  if (!desc) return SSMVJP_EINVAL;
  const ssmvjp_ssd_desc& d = *desc;
  if (d.batch < 0 || d.seqlen < 0 || d.nheads <= 0 || d.headdim <= 0 || d.dstate <= 0 || d.ngroups <= 0 ||
      d.mimo_rank <= 0 || d.chunk_len <= 0)
    return SSMVJP_EINVAL;
  if (d.nheads % d.ngroups) return SSMVJP_EINVAL;
  if (d.form != SSMVJP_FORM_MAMBA2 && d.form != SSMVJP_FORM_RAW) return SSMVJP_EINVAL;
  if (d.form == SSMVJP_FORM_MAMBA2 && d.mimo_rank != 1) return SSMVJP_EINVAL;
  if (!valid_dtype(d.dtype)) return SSMVJP_EINVAL;
  if (!ssd_fwd_shape_supported(d) && !ssd_fwd_pad_supported(d)) return SSMVJP_EUNSUPPORTED;
  return SSMVJP_OK;
}
}  // namespace

ssmvjp_status ssd_chunk_fwd_workspace(const ssmvjp_ssd_desc* desc, size_t* bytes) {
  if (!bytes) return SSMVJP_EINVAL;
  ssmvjp_status s = ssd_fwd_check(desc);
  if (s != SSMVJP_OK) return s;
  *bytes = with_flag(ssd_fwd_bytes(*desc));
  return SSMVJP_OK;
}

ssmvjp_status ssd_chunk_fwd(const ssmvjp_ssd_desc* desc, const void* x_or_v, const float* dt_or_da,
                            const float* A, const void* B, const void* C, const float* s0, void* y,
                            float* s_final, void* workspace, size_t workspace_bytes, void* stream) {
  ssmvjp_status s = ssd_fwd_check(desc);
  if (s != SSMVJP_OK) return s;
  const ssmvjp_ssd_desc& d = *desc;
  const bool has_tokens = d.batch * d.seqlen > 0;
  if (has_tokens && (!x_or_v || !dt_or_da || !B || !C || !y)) return SSMVJP_EINVAL;
  if (d.form == SSMVJP_FORM_MAMBA2 && has_tokens && !A) return SSMVJP_EINVAL;
  const void* pa[] = {x_or_v, B, C, y};
  for (const void* p : pa)
    if (p && !aligned(p, 16)) return SSMVJP_EINVAL;
  const void* pf[] = {dt_or_da, A, s0, s_final};
  for (const void* p : pf)
    if (p && !aligned(p, 4)) return SSMVJP_EINVAL;
  const size_t plan_bytes = ssd_fwd_bytes(d), need = with_flag(plan_bytes);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return SSMVJP_EWORKSPACE;
  if (d.batch == 0) return SSMVJP_OK;
  SsdFwdPointers ptr{x_or_v, dt_or_da, A, B, C, s0, y, s_final, workspace};
  s = hip_status(ssd_fwd_shape_supported(d) ? launch_ssd_fwd(d, ptr, (hipStream_t)stream)
                                            : launch_ssd_fwd_padded(d, ptr, (hipStream_t)stream));
  if (s != SSMVJP_OK || !check_finite_on()) return s;
  const OutSpan outs[] = {{y, d.batch * d.seqlen * d.mimo_rank * d.nheads * d.headdim, d.dtype == SSMVJP_BF16},
                          {s_final, d.batch * d.nheads * d.headdim * d.dstate, false}};
  return finite_check(workspace, plan_bytes, outs, (hipStream_t)stream);
}

// ------------------------------- delta_rule_bwd -----------------------------

ssmvjp_status delta_rule_bwd_workspace(const ssmvjp_delta_desc* desc, size_t* bytes) {
  if (!bytes) return SSMVJP_EINVAL;
  ssmvjp_status s = delta_check(desc);
  if (s != SSMVJP_OK) return s;
  *bytes = with_flag(delta_plan(*desc).bytes);
  return SSMVJP_OK;
}

static ssmvjp_status delta_run(const ssmvjp_delta_desc* desc, int32_t stages, const float* q, const float* k,
                               const float* v, const float* beta, const float* g, const float* S0, const float* d_o,
                               const float* dS_final, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                               float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
  ssmvjp_status s = delta_check(desc);
  if (s != SSMVJP_OK) return s;
  if (stages <= 0 || (stages & ~SSMVJP_DELTA_ALL)) return SSMVJP_EINVAL;
  const ssmvjp_delta_desc& d = *desc;
  const bool has_tokens = d.batch * d.seqlen > 0;
  if (has_tokens && (!q || !k || !v || !beta || !g || !d_o || !dq || !dk || !dv || !dg || !dbeta))
    return SSMVJP_EINVAL;
  const void* pf[] = {q, k, v, beta, g, S0, d_o, dS_final, dq, dk, dv, dg, dbeta, dS0};
  for (const void* p : pf)
    if (p && !aligned(p, 16)) return SSMVJP_EINVAL;
  const DeltaPlan plan = delta_plan(d);
  const size_t need = with_flag(plan.bytes);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return SSMVJP_EWORKSPACE;
  if (d.batch == 0) return SSMVJP_OK;
  DeltaPointers ptr{q, k, v, beta, g, S0, d_o, dS_final, dq, dk, dv, dg, dbeta, dS0, workspace};
  s = hip_status(launch_delta_bwd(d, plan, ptr, (hipStream_t)stream, stages));
  if (s != SSMVJP_OK || !check_finite_on()) return s;
  const bool bwd = stages & SSMVJP_DELTA_BWD, red = stages & SSMVJP_DELTA_REDUCE;
  const int64_t bt = d.batch * d.seqlen;
  const OutSpan outs[] = {{red ? dq : nullptr, bt * d.nqk_heads * d.dk, false},
                          {red ? dk : nullptr, bt * d.nqk_heads * d.dk, false},
                          {bwd ? dv : nullptr, bt * d.nv_heads * d.dv, false},
                          {red ? dg : nullptr, bt * d.nv_heads * d.dk, false},
                          {red ? dbeta : nullptr, bt * d.nv_heads, false},
                          {bwd ? dS0 : nullptr, d.batch * d.nv_heads * d.dk * d.dv, false}};
  return finite_check(workspace, plan.bytes, outs, (hipStream_t)stream);
}

ssmvjp_status delta_rule_bwd(const ssmvjp_delta_desc* desc, const float* q, const float* k, const float* v,
                             const float* beta, const float* g, const float* S0, const float* d_o,
                             const float* dS_final, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                             float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
  return delta_run(desc, SSMVJP_DELTA_ALL, q, k, v, beta, g, S0, d_o, dS_final, dq, dk, dv, dg, dbeta, dS0,
                   workspace, workspace_bytes, stream);
}

ssmvjp_status delta_rule_bwd_stages(const ssmvjp_delta_desc* desc, int32_t stages, const float* q, const float* k,
                                    const float* v, const float* beta, const float* g, const float* S0,
                                    const float* d_o, const float* dS_final, float* dq, float* dk, float* dv,
                                    float* dg, float* dbeta, float* dS0, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return delta_run(desc, stages, q, k, v, beta, g, S0, d_o, dS_final, dq, dk, dv, dg, dbeta, dS0, workspace,
                   workspace_bytes, stream);
}

}  // extern "C"
