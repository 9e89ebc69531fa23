// ssd_pad.hip -- the chunked backward and forward for head dims and state
// sizes that are not multiples of 16 (the MFMA tile), by zero padding.
//
// The chunked kernels tile P and N by 16.  For other P or N the library copies
// x (or v), dy, B, C and the states into workspace buffers whose P and N are
// rounded up to multiples of 16, with the added columns (and state rows) set to
// zero, runs the chunked kernels on the padded problem, and copies the real
// columns of the gradients back.  The padding is exact: a zero column of x and
// dy never feeds a state element, a zero column of B and C keeps the added
// state columns at zero (their initial value), and every product or sum over p
// or n only gains zero terms, so the real outputs are those of the unpadded
// problem up to the order of summation.
#include "ssd_common.cuh"

namespace ssmvjp {
namespace {

i64 up16(i64 v) { return (v + 15) / 16 * 16; }

// dst[o][i][j] = src[o][i][j] for i < r, j < c, else 0; dst is [outer][R][C],
// src is [outer][r][c] (NULL: zeros)
template <typename T>
__global__ void __launch_bounds__(256) pad_kernel(const T* src, T* dst, i64 outer, int r, int c, int R, int C) {
  const i64 n = outer * R * C;
  for (i64 e = (i64)blockIdx.x * 256 + threadIdx.x; e < n; e += (i64)gridDim.x * 256) {
    const int j = (int)(e % C), i = (int)((e / C) % R);
    const i64 o = e / ((i64)R * C);
    dst[e] = (src && i < r && j < c) ? src[(o * r + i) * c + j] : (T)0.0f;
  }
}
// dst[o][i][j] = src[o][i][j] for i < r, j < c; src is [outer][R][C], dst [outer][r][c]
template <typename T>
__global__ void __launch_bounds__(256) unpad_kernel(const T* src, T* dst, i64 outer, int r, int c, int R, int C) {
  const i64 n = outer * r * c;
  for (i64 e = (i64)blockIdx.x * 256 + threadIdx.x; e < n; e += (i64)gridDim.x * 256) {
    const int j = (int)(e % c), i = (int)((e / c) % r);
    const i64 o = e / ((i64)r * c);
    dst[e] = src[(o * R + i) * C + j];
  }
}

unsigned grid_for(i64 n) { return (unsigned)(n <= 0 ? 1 : (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096); }

template <typename T>
void pad(const void* src, void* dst, i64 outer, i64 r, i64 c, i64 R, i64 C, hipStream_t s) {
  if (outer * R * C > 0)
    hipLaunchKernelGGL(pad_kernel<T>, dim3(grid_for(outer * R * C)), dim3(256), 0, s, (const T*)src, (T*)dst, outer,
                       (int)r, (int)c, (int)R, (int)C);
}
template <typename T>
void unpad(const void* src, void* dst, i64 outer, i64 r, i64 c, i64 R, i64 C, hipStream_t s) {
  if (dst && outer * r * c > 0)
    hipLaunchKernelGGL(unpad_kernel<T>, dim3(grid_for(outer * r * c)), dim3(256), 0, s, (const T*)src, (T*)dst,
                       outer, (int)r, (int)c, (int)R, (int)C);
}

// workspace layout of the padded path: the padded problem's own workspace,
// then the padded tensors
struct PadLayout {
  ssmvjp_ssd_desc dp;  // the padded descriptor
  i64 off_x, off_dy, off_dx, off_B, off_C, off_dB, off_dC, off_s0, off_dsf, off_ds0, off_y, off_sf;
  size_t inner, bytes;
};

PadLayout pad_layout(const ssmvjp_ssd_desc& d, bool fwd) {
  PadLayout L;
  L.dp = d;
  L.dp.headdim = up16(d.headdim);
  L.dp.dstate = up16(d.dstate);
  const i64 esz = d.dtype == SSMVJP_BF16 ? 2 : 4;
  const i64 nx = d.batch * d.seqlen * d.mimo_rank * d.nheads * L.dp.headdim * esz;
  const i64 nbc = d.batch * d.seqlen * d.mimo_rank * d.ngroups * L.dp.dstate * esz;
  const i64 nst = d.batch * d.nheads * L.dp.headdim * L.dp.dstate * 4;
  L.inner = fwd ? ssd_fwd_workspace_bytes(L.dp) : ssd_plan(L.dp).bytes;
  i64 off = (i64)L.inner;
  auto carve = [&](i64 bytes) {
    off = (off + 255) / 256 * 256;
    const i64 o = off;
    off += bytes;
    return o;
  };
  L.off_x = carve(nx);
  L.off_B = carve(nbc);
  L.off_C = carve(nbc);
  L.off_s0 = carve(nst);
  if (fwd) {
    L.off_y = carve(nx);
    L.off_sf = carve(nst);
    L.off_dy = L.off_dx = L.off_dB = L.off_dC = L.off_dsf = L.off_ds0 = 0;
  } else {
    L.off_dy = carve(nx);
    L.off_dsf = carve(nst);
    L.off_dx = carve(nx);
    L.off_dB = carve(nbc);
    L.off_dC = carve(nbc);
    L.off_ds0 = carve(nst);
    L.off_y = L.off_sf = 0;
  }
  L.bytes = (size_t)((off + 255) / 256 * 256);
  return L;
}

bool pad_candidate(const ssmvjp_ssd_desc& d) { return d.headdim % 16 != 0 || d.dstate % 16 != 0; }

template <typename T>
hipError_t bwd_padded_t(const ssmvjp_ssd_desc& d, const SsdPointers& ptr, hipStream_t s, int stages) {
  const PadLayout L = pad_layout(d, false);
  char* ws = (char*)ptr.workspace;
  const i64 P = d.headdim, N = d.dstate, Pp = L.dp.headdim, Np = L.dp.dstate;
  const i64 rows_x = d.batch * d.seqlen * d.mimo_rank * d.nheads, rows_bc = d.batch * d.seqlen * d.mimo_rank * d.ngroups;
  const i64 nstate = d.batch * d.nheads;
  const bool states = stages & SSD_STAGE_STATES, grads = stages & SSD_STAGE_GRADS;
  // the inputs both stages read
  pad<T>(ptr.xv, ws + L.off_x, rows_x, 1, P, 1, Pp, s);
  pad<T>(ptr.dy, ws + L.off_dy, rows_x, 1, P, 1, Pp, s);
  pad<T>(ptr.B, ws + L.off_B, rows_bc, 1, N, 1, Np, s);
  pad<T>(ptr.C, ws + L.off_C, rows_bc, 1, N, 1, Np, s);
  if (states) {
    pad<float>(ptr.s0, ws + L.off_s0, nstate, P, N, Pp, Np, s);
    pad<float>(ptr.ds_final, ws + L.off_dsf, nstate, P, N, Pp, Np, s);
  }
  SsdPointers pp = ptr;
  pp.xv = ws + L.off_x;
  pp.dy = ws + L.off_dy;
  pp.B = ws + L.off_B;
  pp.C = ws + L.off_C;
  pp.s0 = (const float*)(ws + L.off_s0);
  pp.ds_final = (const float*)(ws + L.off_dsf);
  pp.dxv = ws + L.off_dx;
  pp.dB = ws + L.off_dB;
  pp.dC = ws + L.off_dC;
  pp.d_s0 = (float*)(ws + L.off_ds0);
  pp.workspace = ws;  // the padded problem's workspace comes first
  const hipError_t e = launch_ssd_bwd(L.dp, ssd_plan(L.dp), pp, s, stages);
  if (e != hipSuccess) return e;
  if (states) unpad<float>(ws + L.off_ds0, ptr.d_s0, nstate, P, N, Pp, Np, s);
  if (grads) {
    unpad<T>(ws + L.off_dx, ptr.dxv, rows_x, 1, P, 1, Pp, s);
    unpad<T>(ws + L.off_dB, ptr.dB, rows_bc, 1, N, 1, Np, s);
    unpad<T>(ws + L.off_dC, ptr.dC, rows_bc, 1, N, 1, Np, s);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t fwd_padded_t(const ssmvjp_ssd_desc& d, const SsdFwdPointers& ptr, hipStream_t s) {
  const PadLayout L = pad_layout(d, true);
  char* ws = (char*)ptr.workspace;
  const i64 P = d.headdim, N = d.dstate, Pp = L.dp.headdim, Np = L.dp.dstate;
  const i64 rows_x = d.batch * d.seqlen * d.mimo_rank * d.nheads, rows_bc = d.batch * d.seqlen * d.mimo_rank * d.ngroups;
  const i64 nstate = d.batch * d.nheads;
  pad<T>(ptr.xv, ws + L.off_x, rows_x, 1, P, 1, Pp, s);
  pad<T>(ptr.B, ws + L.off_B, rows_bc, 1, N, 1, Np, s);
  pad<T>(ptr.C, ws + L.off_C, rows_bc, 1, N, 1, Np, s);
  pad<float>(ptr.s0, ws + L.off_s0, nstate, P, N, Pp, Np, s);
  SsdFwdPointers pp = ptr;
  pp.xv = ws + L.off_x;
  pp.B = ws + L.off_B;
  pp.C = ws + L.off_C;
  pp.s0 = (const float*)(ws + L.off_s0);
  pp.y = ws + L.off_y;
  pp.s_final = ptr.s_final ? (float*)(ws + L.off_sf) : nullptr;
  pp.workspace = L.inner > 0 ? ws : nullptr;
  const hipError_t e = launch_ssd_fwd(L.dp, pp, s);
  if (e != hipSuccess) return e;
  unpad<T>(ws + L.off_y, ptr.y, rows_x, 1, P, 1, Pp, s);
  unpad<float>(ws + L.off_sf, ptr.s_final, nstate, P, N, Pp, Np, s);
  return hipGetLastError();
}

}  // namespace

bool ssd_pad_supported(const ssmvjp_ssd_desc& d) {
  return pad_candidate(d) && !ssd_shape_supported(d) && ssd_shape_supported(pad_layout(d, false).dp);
}
bool ssd_fwd_pad_supported(const ssmvjp_ssd_desc& d) {
  return pad_candidate(d) && !ssd_fwd_shape_supported(d) && ssd_fwd_shape_supported(pad_layout(d, true).dp);
}
size_t ssd_pad_workspace_bytes(const ssmvjp_ssd_desc& d) { return pad_layout(d, false).bytes; }
size_t ssd_fwd_pad_workspace_bytes(const ssmvjp_ssd_desc& d) { return pad_layout(d, true).bytes; }

hipError_t launch_ssd_bwd_padded(const ssmvjp_ssd_desc& d, const SsdPointers& ptr, hipStream_t stream, int stages) {
  return d.dtype == SSMVJP_BF16 ? bwd_padded_t<bf16>(d, ptr, stream, stages) : bwd_padded_t<float>(d, ptr, stream, stages);
}
hipError_t launch_ssd_fwd_padded(const ssmvjp_ssd_desc& d, const SsdFwdPointers& ptr, hipStream_t stream) {
  return d.dtype == SSMVJP_BF16 ? fwd_padded_t<bf16>(d, ptr, stream) : fwd_padded_t<float>(d, ptr, stream);
}

}  // namespace ssmvjp
