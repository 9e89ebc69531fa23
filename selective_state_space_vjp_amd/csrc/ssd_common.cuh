// ssd_common.cuh -- pieces shared by the chunked SSD backward kernels
// (ssd_chunk.hip: state scans and the per-chunk backward for fused chunks of at
// most 64 rows; ssd_blocked.hip: the row-blocked per-chunk backward for longer
// fused chunks): the argument block, tensor offsets, staging and store helpers
// and the per-chunk step scalars.
#pragma once

#include "common.cuh"
#include "kernels.h"

namespace ssmvjp {

struct SsdArgs {
  i64 b, T, H, P, N, G, M, L, LM, nc, hpg, hsplit, hph;
  int raw;  // 1: (v, da) inputs; 0: Mamba-2 (x, dt, A)
  const void* xv;
  const float* dtda;
  const float* A;
  const void* B;
  const void* C;
  const float* s0;
  const void* dy;
  const float* dsf;
  void* dxv;
  float* d_dtda;
  void* dB;
  void* dC;
  float* d_s0;
  void* S;      // [b][nc][H][P*N] chunk-input states, native tiles
  void* dS;     // [b][nc][H][P*N] dS_{c+1}, native tiles
  float* part;  // [2][hsplit][b*T*M*G*N] per-split dB / dC partials (hsplit > 1)
  float* csv;   // [b][nc][H][3][64] per-chunk step scalars: cumA, delta, sigmoid(dt) (see ssd_chunk_scalars_kernel)
  // row-blocked path (L*M > 64) only:
  float* rowv;  // [b][nc][H][RV_N][LM] per-row partial sums of d_cumA terms
  float* dend;  // [b][nc][H] sum over (p, n) of S_c * dS_{c+1}
  // dA (Mamba-2 form, when requested): [b][nc][H] sums over the chunk's steps
  // of d_da * delta, else NULL
  float* dA_part;
};

// resource over the dA partial sums of chunk c (empty when dA is not requested:
// every store through it is dropped)
__device__ __forceinline__ brsrc dA_rsrc(const SsdArgs& a, i64 bi, i64 c) {
  return a.dA_part ? make_rsrc(a.dA_part + (bi * a.nc + c) * a.H, (unsigned)(a.H * 4)) : make_rsrc(a.d_dtda, 0u);
}

// per-row partial sums kept by the row-blocked path, in this order
enum { RV_BLUE = 0, RV_OROW, RV_OCOL, RV_DEC, RV_DVX, RV_N };

static inline i64 cdiv(i64 a, i64 b) { return (a + b - 1) / b; }

// Offsets.  Big tensors x/v, dy, dx/dv: [b][T][M][H][P]; B, C, dB, dC: [b][T][M][G][N].
__device__ __forceinline__ i64 ix_xv(const SsdArgs& a, i64 bi, i64 t, i64 m, i64 h, i64 p) {
  return (((bi * a.T + t) * a.M + m) * a.H + h) * a.P + p;
}
__device__ __forceinline__ i64 ix_bc(const SsdArgs& a, i64 bi, i64 t, i64 m, i64 g, i64 n) {
  return (((bi * a.T + t) * a.M + m) * a.G + g) * a.N + n;
}
// native tile offset of state element (p, n) inside one [P x N] state
__device__ __forceinline__ i64 native_off(int N, int pt, int nt, int lane, int j) {
  return ((i64)(pt * (N / 16) + nt) * 64 + lane) * 4 + j;
}

__device__ __forceinline__ void store4(float* p, const f32x4& v) { *(float4*)p = make_float4(v[0], v[1], v[2], v[3]); }
__device__ __forceinline__ void store4(bf16* p, const f32x4& v) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 u = {pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3])};
  *(u32x2*)p = u;
}

// four float results stored as 4 consecutive elements of T through a resource
// (dropped past the resource size)
__device__ __forceinline__ void bstore4(brsrc r, unsigned off, const f32x4& v, const float*) {
  u32x4 u = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
  __builtin_amdgcn_raw_buffer_store_b128(u, r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore4(brsrc r, unsigned off, const f32x4& v, const bf16*) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 u = {pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3])};
  __builtin_amdgcn_raw_buffer_store_b64(u, r, (int)off, 0, 0);
}

// 16-byte global <-> register chunks for staging (8 bf16 or 4 float)
__device__ __forceinline__ u32x4 zero_u4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}
__device__ __forceinline__ u32x4 load16(const void* p) { return *(const u32x4*)p; }
// scale the elements of a 16-byte chunk by s (float math, result in T)
__device__ __forceinline__ u32x4 scale16(u32x4 u, float s, const float*) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(__uint_as_float(u[e]) * s);
  return o;
}
__device__ __forceinline__ u32x4 scale16(u32x4 u, float s, const bf16*) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = __uint_as_float(u[e] << 16) * s, hi = __uint_as_float(u[e] & 0xffff0000u) * s;
    o[e] = pk_bf16(lo, hi);
  }
  return o;
}

// XOR-swizzled bf16 tiles: rows without padding whose length is a multiple of
// 64 elements (whole 128-byte segments).  Within each 128-byte segment of a row
// the 8-byte unit u is stored at u ^ f(row), f(row) = 4 (row % 4) + (row / 4) % 4.
// A fragment read along the rows (16 consecutive rows from a multiple of 16,
// one unit each: ld_colk_xs) and a transposed read (4 consecutive rows from a
// multiple of 4, 4 consecutive units each: ld_rowk_xs) then hit 16 distinct
// 8-byte bank pairs; no plain row pitch serves both.
__device__ __forceinline__ int xsw_off(int row, int col) {  // element offset of column col (col % 4 == 0) in its row
  const int u = col >> 2;
  return ((u & ~15) | ((u & 15) ^ (((row & 3) << 2) | ((row >> 2) & 3)))) << 2;
}
__device__ __forceinline__ Frag<bf16> ld_colk_xs(const bf16* t, int pitch, int c0, int k0, int lane) {
  const int row = c0 + (lane & 15);
  Frag<bf16> f;
  f.v = *(const s16x4*)(t + row * pitch + xsw_off(row, k0 + 4 * (lane >> 4)));
  return f;
}
__device__ __forceinline__ Frag<bf16> ld_rowk_xs(const bf16* t, int pitch, int k0, int c0, int lane) {
  const int m = lane & 15, row = k0 + 4 * (lane >> 4) + (m >> 2);
  return lds_tr_b16(t + row * pitch + xsw_off(row, c0 + 4 * (m & 3)));
}
// a 16-byte chunk (columns col .. col+7 of row `row`) into a swizzled tile
__device__ __forceinline__ void st16_xs(bf16* t, int pitch, int row, int col, const u32x4& u) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 lo = {u[0], u[1]}, hi = {u[2], u[3]};
  *(u32x2*)(t + row * pitch + xsw_off(row, col)) = lo;
  *(u32x2*)(t + row * pitch + xsw_off(row, col + 4)) = hi;
}

// Per-chunk step sizes for one head, one lane per step l < L (lanes >= L and
// steps past T get zeros, which keeps cumA flat over a short last chunk).
// z is this lane's dt (Mamba-2) or da (RAW) value, Ah the head's A (Mamba-2).
struct ChunkScalars {
  float delta;  // softplus(dt) (Mamba-2) or 1 (RAW)
  float sig;    // sigmoid(dt) (Mamba-2)
  float cum;    // inclusive cumsum of da within the chunk
  float end;    // cumsum at the last step of the chunk (same in every lane)
};

__device__ __forceinline__ ChunkScalars chunk_scalars(const SsdArgs& a, float z, bool valid, float Ah, int lane) {
  ChunkScalars s;
  float da;
  if (a.raw) {
    s.delta = 1.0f;
    s.sig = 0.0f;
    da = z;
  } else {
    s.delta = valid ? softplus_f(z) : 0.0f;
    s.sig = sigmoid_f(z);
    da = s.delta * Ah;
  }
  s.cum = wave_incl_scan(valid ? da : 0.0f, lane);
  s.end = __shfl(s.cum, 63, 64);
  return s;
}


// The step scalars of chunk c, head h as stored by ssd_chunk_scalars_kernel,
// one lane per step (lanes past the chunk's end hold zero delta and a flat
// cumsum); `end` is the cumsum at the chunk's last step.
__device__ __forceinline__ const float* csv_at(const SsdArgs& a, i64 bi, i64 c, i64 h) {
  return a.csv + ((bi * a.nc + c) * a.H + h) * 3 * 64;
}
// issue the loads (end not set yet: finish_scalars, once the loads are needed)
__device__ __forceinline__ ChunkScalars issue_scalars(const SsdArgs& a, i64 bi, i64 c, i64 h, int lane) {
  const brsrc r = make_rsrc(csv_at(a, bi, c, h), 3 * 64 * 4);
  ChunkScalars s;
  s.cum = bload_f32(r, (unsigned)lane * 4u);
  s.delta = bload_f32(r, (unsigned)(64 + lane) * 4u);
  s.sig = bload_f32(r, (unsigned)(128 + lane) * 4u);
  s.end = 0.0f;
  return s;
}
__device__ __forceinline__ ChunkScalars finish_scalars(ChunkScalars s) {
  s.end = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s.cum), 63));
  return s;
}
__device__ __forceinline__ ChunkScalars load_scalars(const SsdArgs& a, i64 bi, i64 c, i64 h, int lane) {
  return finish_scalars(issue_scalars(a, bi, c, h, lane));
}

// per-chunk backward with 16 waves for bf16 at P = 64, N = 128 and 64-step
// rank-1 chunks, defined in ssd_chunk16.hip
void launch_ssd_chunk16(const SsdArgs& a, hipStream_t stream);

// row-blocked chunk backward (L*M > 64), defined in ssd_blocked.hip
bool ssd_blocked_supported(const ssmvjp_ssd_desc& d);
void launch_ssd_blocked_grads(const SsdArgs& a, bool is_bf16, hipStream_t stream);

}  // namespace ssmvjp
