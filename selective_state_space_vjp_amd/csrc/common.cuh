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
// step size: delta = softplus(z) (z > 20 -> z), its derivative sigmoid(z)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float softplus_f(float z) { return z > 20.0f ? z : log1pf(expf(z)); }
__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// wave64 reductions (butterfly, fixed order: every lane ends with the same bits)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// sum over the 16 lanes that share (lane / 16): xor over bits 0..3
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

// sum over the 4 lanes that share (lane % 16): xor over bits 4..5
__device__ __forceinline__ float sum4q(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// inclusive prefix sum over the 64 lanes (Hillis-Steele, fixed order)
__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// inclusive suffix sum over the 64 lanes: lane l gets sum_{k >= l} v_k
__device__ __forceinline__ float wave_incl_suffix(float v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float o = __shfl_down(v, off, 64);
    if (lane + off < 64) v += o;
  }
  return v;
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

struct frag4 {
  float v[4];
};

__device__ __forceinline__ short bf16_bits(float f) {
  bf16 b = (bf16)f;
  return __builtin_bit_cast(short, b);
}

// D += A * B over one 16-wide k block, with operands rounded to bf16.
__device__ __forceinline__ void mma_bf16(f32x4& d, const frag4& a, const frag4& b) {
  s16x4 av = {bf16_bits(a.v[0]), bf16_bits(a.v[1]), bf16_bits(a.v[2]), bf16_bits(a.v[3])};
  s16x4 bv = {bf16_bits(b.v[0]), bf16_bits(b.v[1]), bf16_bits(b.v[2]), bf16_bits(b.v[3])};
  d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, d, 0, 0, 0);
}

// D += A * B over one 16-wide k block in full float32.
__device__ __forceinline__ void mma_f32(f32x4& d, const frag4& a, const frag4& b) {
  d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[0], b.v[0], d, 0, 0, 0);
  d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[1], b.v[1], d, 0, 0, 0);
  d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[2], b.v[2], d, 0, 0, 0);
  d = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[3], b.v[3], d, 0, 0, 0);
}

template <typename T>
struct Mma;
template <>
struct Mma<float> {
  static __device__ __forceinline__ void run(f32x4& d, const frag4& a, const frag4& b) { mma_f32(d, a, b); }
};
template <>
struct Mma<bf16> {
  static __device__ __forceinline__ void run(f32x4& d, const frag4& a, const frag4& b) { mma_bf16(d, a, b); }
};

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

}  // namespace ssmvjp
