// common.cuh -- device helpers shared by the libssmvjp kernels (gfx950 only).
//
// Element I/O for the two storage types of the big tensors (float32 and
// bfloat16, round-to-nearest-even on store), the softplus / sigmoid used for the
// step size, wave64 reductions and scans in a fixed order, and thin wrappers
// around the gfx950 MFMA builtins used by the chunked kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssmvjp {

typedef int64_t i64;
typedef __bf16 bf16;

// ---------------------------------------------------------------------------
// element I/O
// ---------------------------------------------------------------------------
__device__ __forceinline__ float ld(const float* p, i64 i) { return p[i]; }
__device__ __forceinline__ float ld(const bf16* p, i64 i) { return (float)p[i]; }
__device__ __forceinline__ void st(float* p, i64 i, float v) { p[i] = v; }
__device__ __forceinline__ void st(bf16* p, i64 i, float v) { p[i] = (bf16)v; }

// ---------------------------------------------------------------------------
// Range-checked global loads through a raw buffer resource.  A load whose
// 32-bit byte offset (plus its size) lies past the resource size returns zeros
// (the hardware range check), so rows past the end of a sequence need neither a
// branch nor a lane mask, and the loads issue on straight-line code, where the
// compiler can count outstanding loads exactly instead of draining them.
// ---------------------------------------------------------------------------
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t brsrc;
constexpr unsigned BUF_OOB = 0x80000000u;  // past the size of every resource made here (< 2^31 bytes)
__device__ __forceinline__ brsrc make_rsrc(const void* base, unsigned bytes) {
  // dword 3: 32-bit data format, the raw (untyped) form of the gfx9 resource
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(brsrc r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ float bload_f32(brsrc r, unsigned off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
// stores through a resource: a store past the resource size is dropped
__device__ __forceinline__ void bstore_f32(brsrc r, unsigned off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, 0);
}
// n stores that the range check drops.  Issued right after a loop's first
// prefetch, they give the loop entry the same sequence of outstanding memory
// operations as its back edge (next loads, then this iteration's stores), so
// the compiler's wait counts inside the loop cover loads only and never wait
// for stores to be acknowledged.
template <int n>
__device__ __forceinline__ void vmem_pad_stores(brsrc r) {
#pragma unroll
  for (int k = 0; k < n; ++k) bstore_f32(r, BUF_OOB, 0.0f);
}

// ---------------------------------------------------------------------------
// step size: delta = softplus(z) (z > 20 -> z), its derivative sigmoid(z)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float softplus_f(float z) { return z > 20.0f ? z : log1pf(expf(z)); }
__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// wave64 reductions.  All lanes end with the sum; each lane's summation order
// is fixed, so results are identical from run to run.
//   sum16: over the 16 lanes of a DPP row (lanes with the same lane/16), with
//          four row rotations folded into v_add_f32_dpp;
//   sum4q: over the 4 lanes with the same lane%16, with the gfx950
//          v_permlane16_swap / v_permlane32_swap exchanges (no LDS traffic);
//   wave_sum = sum4q(sum16(v)).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f<0x128>(v);  // row_ror:8
  v += dpp_f<0x124>(v);  // row_ror:4
  v += dpp_f<0x122>(v);  // row_ror:2
  v += dpp_f<0x121>(v);  // row_ror:1
  return v;
}
__device__ __forceinline__ float sum4q(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
  v = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
  return __builtin_bit_cast(float, (int)b[0]) + __builtin_bit_cast(float, (int)b[1]);
}
__device__ __forceinline__ float wave_sum(float v) { return sum4q(sum16(v)); }

// exp(x) through the hardware exp2 (v_exp_f32, relative error a few 1e-8)
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// softplus(z) = log(1 + e^z) through the hardware exp2 / log2, with the log1p
// correction of Goldberg, "What every computer scientist should know about
// floating-point arithmetic" (Theorem 4): with u = 1 + e rounded,
// log1p(e) = e * log(u) / (u - 1) to a few ulps, and e itself when u rounds to 1.
__device__ __forceinline__ float softplus_hw(float z) {
  const float e = exp_hw(z);
  const float u = 1.0f + e;
  const float l = __builtin_amdgcn_logf(u) * 0.6931471805599453f;
  const float sp = u == 1.0f ? e : l * (e * __builtin_amdgcn_rcpf(u - 1.0f));
  return z > 20.0f ? z : sp;
}

// inclusive prefix sum over the 64 lanes, all in DPP: Hillis-Steele inside
// each 16-lane row (row_shr 1, 2, 4, 8 with zero fill), then the row totals
// carried across rows with row_bcast:15 (rows 1 and 3) and row_bcast:31
// (rows 2 and 3).  Fixed order, no LDS traffic.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_zero(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, true));
}
__device__ __forceinline__ float wave_incl_scan(float v, int /*lane*/) {
  v += dpp_zero<0x111, 0xF>(v);  // row_shr:1
  v += dpp_zero<0x112, 0xF>(v);  // row_shr:2
  v += dpp_zero<0x114, 0xF>(v);  // row_shr:4
  v += dpp_zero<0x118, 0xF>(v);  // row_shr:8
  v += dpp_zero<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_zero<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// inclusive suffix sum over the 64 lanes: lane l gets sum_{k >= l} v_k,
// formed as total - (inclusive prefix - v) (the K1 backward's own form).
__device__ __forceinline__ float wave_incl_suffix(float v, int lane) {
  const float incl = wave_incl_scan(v, lane);
  const float total = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
  return total - (incl - v);
}

// ---------------------------------------------------------------------------
// MFMA 16x16 tiles.
//
// A 16x16 output tile D of an MFMA lives in 4 VGPRs per lane: lane i holds
// D[4*(i/16) + j][i % 16] for j = 0..3.  Operands are described per 16-wide
// block of the contraction index k: lane i supplies A[i % 16][4*(i/16) + j] and
// B[4*(i/16) + j][i % 16] for j = 0..3 ("frag4": four k values per lane).  The
// same frag4 drives one bf16 16x16x16 MFMA or four f32 16x16x4 MFMAs (in the
// f32 case step j uses k = 4*(i/16) + j: a fixed permutation of k applied to
// both operands, which leaves the product unchanged).
//
// Consequence used throughout: the D layout of a tile is exactly the frag4
// layout of that tile as a B operand whose contraction index is D's row index,
// and as an A operand of the transposed tile.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ short bf16_bits(float f) {
  bf16 b = (bf16)f;
  return __builtin_bit_cast(short, b);
}
// two floats rounded to bf16 (nearest even, as bf16_bits) in one dword, lo in
// bits 0..15: a single two-operand v_cvt_pk_bf16_f32
__device__ __forceinline__ unsigned pk_bf16(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// ---------------------------------------------------------------------------
// Typed MFMA operand fragments (frag4 layout, see above): four k values per
// lane, packed bf16 or plain float.
// ---------------------------------------------------------------------------
template <typename T>
struct Frag;
template <>
struct Frag<float> {
  float v[4];
};
template <>
struct Frag<bf16> {
  s16x4 v;
};

__device__ __forceinline__ float bits_bf16(short s) { return (float)__builtin_bit_cast(bf16, s); }

__device__ __forceinline__ void frag_get(const Frag<float>& f, float o[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = f.v[j];
}
__device__ __forceinline__ void frag_get(const Frag<bf16>& f, float o[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = bits_bf16(f.v[j]);
}
template <typename T>
__device__ __forceinline__ Frag<T> frag_make(const float v[4]);
template <>
__device__ __forceinline__ Frag<float> frag_make<float>(const float v[4]) {
  Frag<float> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) f.v[j] = v[j];
  return f;
}
template <>
__device__ __forceinline__ Frag<bf16> frag_make<bf16>(const float v[4]) {
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t u = {pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3])};
  Frag<bf16> f;
  f.v = __builtin_bit_cast(s16x4, u);
  return f;
}

__device__ __forceinline__ void mma(f32x4& d, const Frag<bf16>& a, const Frag<bf16>& b) {
  d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, d, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& d, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], d, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Fragment reads from LDS tiles.
//
// colk: the contraction index runs along a row of a row-major tile: lane
//       (q = lane/16, c = lane%16) gets tile[(c0 + c) * pitch + k0 + 4q + j].
// rowk: the contraction index runs down the rows: lane gets
//       tile[(k0 + 4q + j) * pitch + c0 + c].  For bf16 this is one gfx950
//       transpose read (ds_read_b64_tr_b16): within each 16-lane group, output
//       lane i, slot j, is element i%4 of the 8-byte chunk addressed by lane
//       i/4 + 4j, so lane m addresses row k0 + 4q + m/4, columns c0 + 4(m%4)...+3.
// native: a 16x16 tile stored in MFMA output order (lane-major, 4 values per
//       lane: element (row 4*(l/16)+j, col l%16) at l*4 + j).  ntv reads it
//       as-is (k = row); ntv_t reads it transposed (lane gets element
//       (row c, col 4q + j)), again one transpose read for bf16.
// All bf16 addresses are 8-byte aligned by construction (pitches and column
// offsets are multiples of 4 elements).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ Frag<bf16> lds_tr_b16(const bf16* p) {
  Frag<bf16> f;
  f.v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<bf16*>(p)));
  return f;
}

__device__ __forceinline__ Frag<bf16> ld_colk(const bf16* tile, int pitch, int c0, int k0, int lane) {
  Frag<bf16> f;
  f.v = *(const s16x4*)(tile + (c0 + (lane & 15)) * pitch + k0 + 4 * (lane >> 4));
  return f;
}
__device__ __forceinline__ Frag<float> ld_colk(const float* tile, int pitch, int c0, int k0, int lane) {
  const float4 u = *(const float4*)(tile + (c0 + (lane & 15)) * pitch + k0 + 4 * (lane >> 4));
  Frag<float> f = {{u.x, u.y, u.z, u.w}};
  return f;
}
__device__ __forceinline__ Frag<bf16> ld_rowk(const bf16* tile, int pitch, int k0, int c0, int lane) {
  const int m = lane & 15;
  return lds_tr_b16(tile + (k0 + 4 * (lane >> 4) + (m >> 2)) * pitch + c0 + 4 * (m & 3));
}
__device__ __forceinline__ Frag<float> ld_rowk(const float* tile, int pitch, int k0, int c0, int lane) {
  Frag<float> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) f.v[j] = tile[(k0 + 4 * (lane >> 4) + j) * pitch + c0 + (lane & 15)];
  return f;
}
__device__ __forceinline__ Frag<bf16> ld_ntv(const bf16* t, int lane) {
  Frag<bf16> f;
  f.v = *(const s16x4*)(t + 4 * lane);
  return f;
}
__device__ __forceinline__ Frag<float> ld_ntv(const float* t, int lane) {
  const float4 u = *(const float4*)(t + 4 * lane);
  Frag<float> f = {{u.x, u.y, u.z, u.w}};
  return f;
}
__device__ __forceinline__ Frag<bf16> ld_ntv_t(const bf16* t, int lane) {
  const int m = lane & 15;
  return lds_tr_b16(t + 4 * ((m & 3) * 16 + 4 * (lane >> 4) + (m >> 2)));
}
__device__ __forceinline__ Frag<float> ld_ntv_t(const float* t, int lane) {
  const int c = lane & 15;
  Frag<float> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) f.v[j] = t[4 * ((c >> 2) * 16 + 4 * (lane >> 4) + j) + (c & 3)];
  return f;
}

}  // namespace ssmvjp
