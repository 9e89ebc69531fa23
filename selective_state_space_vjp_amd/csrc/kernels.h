// kernels.h -- host-side launch interface between the C ABI layer (abi.cpp)
// and the kernel translation units.  Internal to libssmvjp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ssmvjp.h"

namespace ssmvjp {

// ----------------------------- sequential scan -----------------------------
struct SeqPlan {
  int64_t K, J;       // checkpoint interval and count
  int PPT, NPG;       // p values per thread, p groups per workgroup
  int64_t off_delta, off_sig, off_ck, off_seg, off_dBh, off_dCh;
  int64_t off_dA;  // per-(batch, head[, state]) partial sums of dA
  size_t bytes;
};

struct SeqPointers {
  const void* x;
  const float* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* s0;
  const void* dy;
  const float* ds_final;
  void* dx;
  float* d_dt;
  void* dB;
  void* dC;
  float* d_s0;
  void* workspace;
  float* dA;  // NULL: not computed
};

SeqPlan seq_plan(const ssmvjp_scan_desc& d);
size_t seq_lds_bytes(const ssmvjp_scan_desc& d, const SeqPlan& plan);
hipError_t launch_seq_bwd(const ssmvjp_scan_desc& d, const SeqPlan& plan, const SeqPointers& ptr,
                          hipStream_t stream);
// dA[j] = sum over i < R of part[i * J + j], ascending i (one thread per j)
void launch_dA_reduce(const float* part, int64_t R, int64_t J, float* dA, hipStream_t stream);

// ------------------------------ chunked SSD --------------------------------
struct SsdPlan {
  int64_t nc;          // number of chunks (last one may be shorter)
  int64_t LM;          // fused chunk length L*M
  int64_t hsplit;      // head-split factor of the chunk kernel (1 = writes dB/dC directly)
  int64_t state_elem;  // bytes per stored state element (2 for bf16, 4 for f32)
  int64_t off_S, off_dS, off_part;
  int64_t off_rowv, off_dend;  // row-blocked path (L*M > 64): per-row partial sums, d_end
  int64_t off_csv;             // per-chunk step scalars (cumA, delta, sigmoid(dt))
  int64_t off_dA;              // per-(batch, chunk, head) partial sums of dA
  size_t bytes;
};

struct SsdPointers {
  const void* xv;
  const float* dtda;
  const float* A;
  const void* B;
  const void* C;
  const float* s0;
  const void* dy;
  const float* ds_final;
  void* dxv;
  float* d_dtda;
  void* dB;
  void* dC;
  float* d_s0;
  void* workspace;
  float* dA;  // NULL: not computed (FORM_MAMBA2 only)
};

bool ssd_shape_supported(const ssmvjp_ssd_desc& d);
SsdPlan ssd_plan(const ssmvjp_ssd_desc& d);
enum { SSD_STAGE_STATES = 1, SSD_STAGE_GRADS = 2, SSD_STAGE_ALL = 3 };
hipError_t launch_ssd_bwd(const ssmvjp_ssd_desc& d, const SsdPlan& plan, const SsdPointers& ptr,
                          hipStream_t stream, int stages);

struct SsdFwdPointers {
  const void* xv;
  const float* dtda;
  const float* A;
  const void* B;
  const void* C;
  const float* s0;
  void* y;
  float* s_final;
  void* workspace;
};

bool ssd_fwd_shape_supported(const ssmvjp_ssd_desc& d);
size_t ssd_fwd_workspace_bytes(const ssmvjp_ssd_desc& d);
hipError_t launch_ssd_fwd(const ssmvjp_ssd_desc& d, const SsdFwdPointers& ptr, hipStream_t stream);

// P or N not a multiple of 16: the same calls on a zero-padded copy in the
// workspace (ssd_pad.hip); *_supported is true only where the unpadded shape
// is not supported and the padded one is
bool ssd_pad_supported(const ssmvjp_ssd_desc& d);
bool ssd_fwd_pad_supported(const ssmvjp_ssd_desc& d);
size_t ssd_pad_workspace_bytes(const ssmvjp_ssd_desc& d);
size_t ssd_fwd_pad_workspace_bytes(const ssmvjp_ssd_desc& d);
hipError_t launch_ssd_bwd_padded(const ssmvjp_ssd_desc& d, const SsdPointers& ptr, hipStream_t stream, int stages);
hipError_t launch_ssd_fwd_padded(const ssmvjp_ssd_desc& d, const SsdFwdPointers& ptr, hipStream_t stream);

// ------------------------------ delta rule ---------------------------------
struct DeltaPlan {
  int64_t CK;          // checkpoint interval (steps)
  int64_t nck;         // checkpoints per (b, hv)
  int64_t vsplit;      // value-column slices per (b, hv), one workgroup each
  int64_t off_ck, off_r, off_part, off_partb;
  size_t bytes;
};

struct DeltaPointers {
  const float *q, *k, *v, *beta, *g, *S0, *d_o, *dS_final;
  float *dq, *dk, *dv, *dg, *dbeta, *dS0;
  void* workspace;
};

bool delta_shape_supported(const ssmvjp_delta_desc& d);
DeltaPlan delta_plan(const ssmvjp_delta_desc& d);
hipError_t launch_delta_bwd(const ssmvjp_delta_desc& d, const DeltaPlan& plan, const DeltaPointers& ptr,
                            hipStream_t stream, int stages);

// ---------------------------- debug finiteness -----------------------------
// flag = 0; then flag = 1 if any of the n elements at p (bf16 or float) is NaN
// or infinite (finite.hip)
void launch_flag_clear(unsigned* flag, hipStream_t stream);
void launch_nonfinite_check(const void* p, int64_t n, bool is_bf16, unsigned* flag, hipStream_t stream);

}  // namespace ssmvjp
