// ssd_chunk.hip -- chunked SSD backward of the selective scan (Mamba-2 and the
// Mamba-3 MIMO rank-M form), after burn-mamba "combined_backward.rs".
//
// The method (burn-mamba combined_backward): recompute the forward's K1 chunk
// cumsum, K2 C.B^T, K3 intra-chunk states and K4 state passing from the saved
// inputs; walk the chunks in reverse fusing the K5 backward (BLUE: the
// inter-chunk term exp(cumA) C.S_c; ORANGE: the causal intra-chunk term
// (CB * decay) v) with the K4 backward; then run the K3, K2 and K1 backwards.
//
// MI355X organisation (three launches on the caller's stream):
//
//  1. ssd_state_scan  one workgroup per (batch, head, direction, n-block).
//     forward:  walks c = 0..nc-1, stores the chunk-input state S_c, then
//               S_{c+1} = exp(end_c) S_c + intra_c with
//               intra_c[p,n] = sum_r exp(end_c - cumA_r) v[r,p] B[r,n]   (K1, K3, K4)
//     reverse:  walks c = nc-1..0, stores dS_{c+1}, then
//               dS_c = exp(end_c) dS_{c+1} + u_c with
//               u_c[p,n] = sum_r C[r,n] exp(cumA_r) dy[r,p]              (BLUE d_state, K4 bwd)
//     d_s0 = dS_0.  The two directions are independent and run side by side.
//     The [P x L*M] x [L*M x N] products run on MFMA from LDS tiles staged
//     time-contiguous; the running state stays in registers in MFMA output
//     layout and is stored in that layout ("native tiles": one 16x16 tile is
//     64 lanes x 4 consecutive elements), so kernel 2 reloads it with one
//     vector load per lane.
//  2. ssd_chunk_bwd   one workgroup per (batch, chunk, group, head split).
//     Loops over the heads of the group: BLUE (dC, d_cumA), K3 backward
//     (dB, d_v, d_cumA), ORANGE (d_v, d_cb, d_cumA), the K4 d_cumA term,
//     the K1 suffix sum and the Mamba-2 chain to (dx, d_dt).  dB and dC are
//     summed over the heads of the group in registers in ascending head order
//     (no float atomics), and the K2 backward runs once on the head-summed d_cb.
//  3. ssd_head_sum    only when the heads of a group are split over several
//     workgroups: dB, dC = sum of the per-split partials in split order.
//
// All products accumulate in float32.  With bf16 storage the MFMA operands are
// bf16 (inputs as given; exp-scaled operands rounded once); decays, cumsums,
// states and all reductions stay float32.
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
};

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

// 8 consecutive elements -> float[8]
__device__ __forceinline__ void load8(const float* p, float* o) {
  const float4 u = *(const float4*)p, v = *(const float4*)(p + 4);
  o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w; o[4] = v.x; o[5] = v.y; o[6] = v.z; o[7] = v.w;
}
__device__ __forceinline__ void load8(const bf16* p, float* o) {
  typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
  const bf16x8 u = *(const bf16x8*)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (float)u[e];
}
// 4 consecutive elements -> frag4
__device__ __forceinline__ frag4 load4(const float* p) {
  const float4 u = *(const float4*)p;
  frag4 f = {{u.x, u.y, u.z, u.w}};
  return f;
}
__device__ __forceinline__ frag4 load4(const bf16* p) {
  typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 u = *(const bf16x4*)p;
  frag4 f = {{(float)u[0], (float)u[1], (float)u[2], (float)u[3]}};
  return f;
}
__device__ __forceinline__ void store4(float* p, const f32x4& v) { *(float4*)p = make_float4(v[0], v[1], v[2], v[3]); }
__device__ __forceinline__ void store4(bf16* p, const f32x4& v) {
  typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 u = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *(bf16x4*)p = u;
}

// Per-chunk step sizes for one head, one lane per step l < L (lanes >= L and
// steps past T get zeros, which keeps cumA flat over a short last chunk).
struct ChunkScalars {
  float delta;  // softplus(dt) (Mamba-2) or 1 (RAW)
  float sig;    // sigmoid(dt) (Mamba-2)
  float cum;    // inclusive cumsum of da within the chunk
  float end;    // cumsum at the last step of the chunk (same in every lane)
};

__device__ __forceinline__ ChunkScalars chunk_scalars(const SsdArgs& a, i64 bi, i64 h, i64 t0, int Lc, int lane) {
  ChunkScalars s;
  const bool valid = lane < Lc;
  const float z = valid ? a.dtda[(bi * a.T + t0 + lane) * a.H + h] : 0.0f;
  float da;
  if (a.raw) {
    s.delta = 1.0f;
    s.sig = 0.0f;
    da = z;
  } else {
    s.delta = valid ? softplus_f(z) : 0.0f;
    s.sig = sigmoid_f(z);
    da = s.delta * a.A[h];
  }
  s.cum = wave_incl_scan(valid ? da : 0.0f, lane);
  s.end = __shfl(s.cum, 63, 64);
  return s;
}

// ===========================================================================
// kernel 1: forward and reverse state scans over chunks
// ===========================================================================
constexpr int SCAN_MAXT = 8;  // state tiles per wave

template <typename T>
__global__ void __launch_bounds__(256) ssd_state_scan_kernel(SsdArgs a, int NB) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int P = (int)a.P, N = (int)a.N, LM = (int)a.LM, L = (int)a.L, M = (int)a.M;
  const int PT = P / 16, NTB = NB / 16, RB = LM / 16;
  const int LDK = LM + (sizeof(T) == 2 ? 8 : 4);  // row pitch (elements) of the time-contiguous tiles
  float* sc = (float*)smem_raw;                    // [64] per-step scale
  float* misc = sc + 64;                           // [4]
  T* opT = (T*)(misc + 4);                         // [P][LDK]   v or dy, scaled, time-contiguous
  T* bcT = opT + P * LDK;                          // [NB][LDK]  B or C, time-contiguous

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int nblk = N / NB;
  i64 bid = blockIdx.x;
  const int nbi = (int)(bid % nblk);
  bid /= nblk;
  const int dir = (int)(bid % 2);  // 0 forward (S), 1 reverse (dS)
  bid /= 2;
  const i64 h = bid % a.H, bi = bid / a.H, g = h / a.hpg;
  const int n0 = nbi * NB;
  const T* op = (const T*)(dir == 0 ? a.xv : a.dy);
  const T* bc = (const T*)(dir == 0 ? a.B : a.C);
  T* out = (T*)(dir == 0 ? a.S : a.dS);
  const float* init = dir == 0 ? a.s0 : a.dsf;

  // tiles of this wave: ti = pt * NTB + nt, ti % 4 == w
  const int ntiles = PT * NTB;
  f32x4 st[SCAN_MAXT];
#pragma unroll
  for (int k = 0; k < SCAN_MAXT; ++k) {
    const int ti = w + 4 * k;
    st[k] = zero4();
    if (ti < ntiles && init) {
      const int pt = ti / NTB, nt = ti % NTB;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st[k][j] = init[((bi * a.H + h) * P + 16 * pt + 4 * q + j) * N + n0 + 16 * nt + r16];
    }
  }

  for (i64 step = 0; step < a.nc; ++step) {
    const i64 c = dir == 0 ? step : a.nc - 1 - step;
    const i64 t0 = c * L;
    const int Lc = (int)((a.T - t0) < L ? (a.T - t0) : L);
    if (w == 0) {
      const ChunkScalars cs = chunk_scalars(a, bi, h, t0, Lc, lane);
      if (lane < L) sc[lane] = dir == 0 ? cs.delta * expf(cs.end - cs.cum) : expf(cs.cum);
      if (lane == 0) misc[0] = expf(cs.end);
    }
    __syncthreads();
    // stage the operand rows (scaled per step) and B/C rows, time-contiguous
    for (int idx = tid; idx < LM * (P / 8); idx += 256) {
      const int r = idx / (P / 8), p0 = (idx % (P / 8)) * 8, l = r / M, m = r % M;
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (l < Lc) load8(op + ix_xv(a, bi, t0 + l, m, h, p0), v);
      const float s = sc[l];
#pragma unroll
      for (int e = 0; e < 8; ++e) opT[(p0 + e) * LDK + r] = (T)(v[e] * s);
    }
    for (int idx = tid; idx < LM * (NB / 8); idx += 256) {
      const int r = idx / (NB / 8), c0 = (idx % (NB / 8)) * 8, l = r / M, m = r % M;
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (l < Lc) load8(bc + ix_bc(a, bi, t0 + l, m, g, n0 + c0), v);
#pragma unroll
      for (int e = 0; e < 8; ++e) bcT[(c0 + e) * LDK + r] = (T)v[e];
    }
    __syncthreads();
    const float e_end = misc[0];
    T* outc = out + ((bi * a.nc + c) * a.H + h) * (i64)P * N;
#pragma unroll
    for (int k = 0; k < SCAN_MAXT; ++k) {
      const int ti = w + 4 * k;
      if (ti >= ntiles) continue;
      const int pt = ti / NTB, nt = ti % NTB;
      store4(outc + native_off(N, pt, n0 / 16 + nt, lane, 0), st[k]);
      f32x4 acc = zero4();
      for (int kb = 0; kb < RB; ++kb) {
        const frag4 fa = load4(opT + (16 * pt + r16) * LDK + 16 * kb + 4 * q);
        const frag4 fb = load4(bcT + (16 * nt + r16) * LDK + 16 * kb + 4 * q);
        Mma<T>::run(acc, fa, fb);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) st[k][j] = e_end * st[k][j] + acc[j];
    }
  }
  if (dir == 1) {
#pragma unroll
    for (int k = 0; k < SCAN_MAXT; ++k) {
      const int ti = w + 4 * k;
      if (ti >= ntiles) continue;
      const int pt = ti / NTB, nt = ti % NTB;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a.d_s0[((bi * a.H + h) * P + 16 * pt + 4 * q + j) * N + n0 + 16 * nt + r16] = st[k][j];
    }
  }
}

// ===========================================================================
// kernel 2: per-chunk backward, heads of a group in a loop
// ===========================================================================
constexpr int MAXRB = 4;  // L*M <= 64
constexpr int MAXNW = 2;  // n tiles per wave (N <= 128)
constexpr int MAXPW = 2;  // p tiles per wave (P <= 128)
constexpr int MAXG = 3;   // lower-triangular (t, s) tile pairs per wave (RB <= 4)

enum { PB_BLUE = 0, PB_OROW, PB_OCOL, PB_DEC, PB_DVX, PB_DEND, PB_N };

template <typename T>
__global__ void __launch_bounds__(256) ssd_chunk_bwd_kernel(SsdArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int P = (int)a.P, N = (int)a.N, LM = (int)a.LM, L = (int)a.L, M = (int)a.M;
  const int PT = P / 16, NT = N / 16, RB = LM / 16;
  const int LDC = LM + 4;                          // CB row pitch (float)
  const int LDP = P + (sizeof(T) == 2 ? 8 : 4);    // x/dy row pitch
  const int LDN = N + (sizeof(T) == 2 ? 8 : 4);    // dS row pitch
  float* CB = (float*)smem_raw;                    // [LM][LDC] C.B^T, later the head-summed d_cb
  float* part = CB + LM * LDC;                     // [2][PB_N][8][64] partial row sums (per wave or per p tile)
  T* xs = (T*)(part + 2 * PB_N * 8 * 64);          // [LM][LDP] x (Mamba-2) or v (RAW)
  T* dys = xs + LM * LDP;                          // [LM][LDP] dy
  T* dSl = dys + LM * LDP;                         // [P][LDN]  dS_{c+1}, row-major

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, q = lane >> 4,
            r16 = lane & 15;
  i64 bid = blockIdx.x;
  const i64 hs = bid % a.hsplit;
  bid /= a.hsplit;
  const i64 g = bid % a.G;
  bid /= a.G;
  const i64 c = bid % a.nc, bi = bid / a.nc;
  const i64 t0 = c * L;
  const int Lc = (int)((a.T - t0) < L ? (a.T - t0) : L);
  const T* Bg = (const T*)a.B;
  const T* Cg = (const T*)a.C;
  const T* xg = (const T*)a.xv;
  const T* dyg = (const T*)a.dy;
  T* dxg = (T*)a.dxv;

  // row r of the chunk's fused L*M length -> (step l, rank m); rows past T are zero
  auto bc_frag = [&](const T* base, int r, int k0) -> frag4 {  // 4 consecutive n of row r
    const int l = r / M, m = r % M;
    if (l >= Lc) {
      frag4 z = {{0.f, 0.f, 0.f, 0.f}};
      return z;
    }
    return load4(base + ix_bc(a, bi, t0 + l, m, g, k0));
  };
  auto bc_elem = [&](const T* base, int r, int n) -> float {
    const int l = r / M, m = r % M;
    return l < Lc ? ld(base, ix_bc(a, bi, t0 + l, m, g, n)) : 0.0f;
  };

  // ---- C.B^T for the chunk (K2 recompute), lower-triangular tile pairs ----
  const int npairs = RB * (RB + 1) / 2;
  for (int pi = w; pi < RB * RB; pi += 4) {
    const int rt = pi / RB, rs = pi % RB;
    f32x4 acc = zero4();
    if (rs <= rt) {
      for (int kb = 0; kb < NT; ++kb) {
        const frag4 fa = bc_frag(Cg, 16 * rt + r16, 16 * kb + 4 * q);
        const frag4 fb = bc_frag(Bg, 16 * rs + r16, 16 * kb + 4 * q);
        Mma<T>::run(acc, fa, fb);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) CB[(16 * rt + 4 * q + j) * LDC + 16 * rs + r16] = acc[j];
  }

  f32x4 dBacc[MAXRB][MAXNW], dCacc[MAXRB][MAXNW], dcbacc[MAXG];
#pragma unroll
  for (int rb = 0; rb < MAXRB; ++rb)
#pragma unroll
    for (int k = 0; k < MAXNW; ++k) {
      dBacc[rb][k] = zero4();
      dCacc[rb][k] = zero4();
    }
#pragma unroll
  for (int k = 0; k < MAXG; ++k) dcbacc[k] = zero4();
  int pair_rt[MAXG], pair_rs[MAXG];
#pragma unroll
  for (int k = 0; k < MAXG; ++k) {
    const int pi = w + 4 * k;
    int rt = 0;
    while (rt < RB && (rt + 1) * (rt + 2) / 2 <= pi) ++rt;
    pair_rt[k] = pi < npairs ? rt : -1;
    pair_rs[k] = pi < npairs ? pi - rt * (rt + 1) / 2 : -1;
  }

  const i64 hbase = g * a.hpg + hs * a.hph;
  for (i64 hh = 0; hh < a.hph; ++hh) {
    const i64 h = hbase + hh;
    float* pb = part + (hh & 1) * PB_N * 8 * 64;
    const ChunkScalars cs = chunk_scalars(a, bi, h, t0, Lc, lane);
    const float Ah = a.raw ? 0.0f : a.A[h];
    auto cum_of = [&](int l) { return __shfl(cs.cum, l, 64); };
    auto delta_of = [&](int l) { return __shfl(cs.delta, l, 64); };

    __syncthreads();  // previous head is done with xs / dys / dSl (and CB writes on entry)
    for (int idx = tid; idx < LM * (P / 8); idx += 256) {
      const int r = idx / (P / 8), p0 = (idx % (P / 8)) * 8, l = r / M, m = r % M;
      float xv8[8] = {0, 0, 0, 0, 0, 0, 0, 0}, dy8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (l < Lc) {
        load8(xg + ix_xv(a, bi, t0 + l, m, h, p0), xv8);
        load8(dyg + ix_xv(a, bi, t0 + l, m, h, p0), dy8);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xs[r * LDP + p0 + e] = (T)xv8[e];
        dys[r * LDP + p0 + e] = (T)dy8[e];
      }
    }
    __syncthreads();

    // ---- BLUE: dC_blue = (dy * exp(cumA)) . S_c ; d_cumA_blue = rowsum(C * dC_blue) ----
    // ---- K3:   dB_k3 += (exp(end - cumA) v) . dS_{c+1}                            ----
    // This wave's n tiles of S_c and dS_{c+1} (all p), read in native layout, one
    // k block at a time; dS_{c+1} is also written row-major to LDS for the
    // contraction over n below.
    const T* Sg = (const T*)a.S + ((bi * a.nc + c) * a.H + h) * (i64)P * N;
    const T* dSg = (const T*)a.dS + ((bi * a.nc + c) * a.H + h) * (i64)P * N;
    float dend = 0.0f;
    {
      float ecum[MAXRB][4], xscale[MAXRB], bluep[MAXRB][4];
#pragma unroll
      for (int rb = 0; rb < MAXRB; ++rb) {
        const int ra = 16 * rb + r16;  // A-fragment row of this lane
        xscale[rb] = delta_of(ra / M) * expf(cs.end - cum_of(ra / M));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ecum[rb][j] = expf(cum_of((16 * rb + 4 * q + j) / M));
          bluep[rb][j] = 0.0f;
        }
      }
#pragma unroll
      for (int k = 0; k < MAXNW; ++k) {
        const int nt = w + 4 * k;
        if (nt >= NT) continue;
        f32x4 acc[MAXRB];
#pragma unroll
        for (int rb = 0; rb < MAXRB; ++rb) acc[rb] = zero4();
        for (int kb = 0; kb < PT; ++kb) {
          const frag4 fS = load4(Sg + native_off(N, kb, nt, lane, 0));
          const frag4 fdS = load4(dSg + native_off(N, kb, nt, lane, 0));
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            dend += fS.v[j] * fdS.v[j];
            dSl[(16 * kb + 4 * q + j) * LDN + 16 * nt + r16] = (T)fdS.v[j];
          }
#pragma unroll
          for (int rb = 0; rb < MAXRB; ++rb) {
            if (rb >= RB) break;
            const int ra = 16 * rb + r16;
            const frag4 fa = load4(dys + ra * LDP + 16 * kb + 4 * q);
            Mma<T>::run(acc[rb], fa, fS);
            frag4 fx = load4(xs + ra * LDP + 16 * kb + 4 * q);
#pragma unroll
            for (int j = 0; j < 4; ++j) fx.v[j] *= xscale[rb];
            Mma<T>::run(dBacc[rb][k], fx, fdS);
          }
        }
#pragma unroll
        for (int rb = 0; rb < MAXRB; ++rb) {
          if (rb >= RB) break;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float val = acc[rb][j] * ecum[rb][j];
            dCacc[rb][k][j] += val;
            bluep[rb][j] += bc_elem(Cg, 16 * rb + 4 * q + j, 16 * nt + r16) * val;
          }
        }
      }
#pragma unroll
      for (int rb = 0; rb < MAXRB; ++rb) {
        if (rb >= RB) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float s = sum16(bluep[rb][j]);
          if (r16 == 0) pb[(PB_BLUE * 8 + w) * 64 + 16 * rb + 4 * q + j] = s;
        }
      }
    }

    // ---- ORANGE: G1 = dy . x^T on lower-triangular tiles; d_cb, row/col sums ----
    {
      float orow[MAXRB][4], ocol[MAXRB];
#pragma unroll
      for (int rb = 0; rb < MAXRB; ++rb) {
        ocol[rb] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) orow[rb][j] = 0.0f;
      }
#pragma unroll
      for (int k = 0; k < MAXG; ++k) {
        const int rt = pair_rt[k], rs = pair_rs[k];
        if (rt < 0) continue;
        f32x4 acc = zero4();
        for (int kb = 0; kb < PT; ++kb) {
          const frag4 fa = load4(dys + (16 * rt + r16) * LDP + 16 * kb + 4 * q);
          const frag4 fb = load4(xs + (16 * rs + r16) * LDP + 16 * kb + 4 * q);
          Mma<T>::run(acc, fa, fb);
        }
        const int s = 16 * rs + r16, ls = s / M;
        const float cs_s = cum_of(ls), dls = delta_of(ls);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * rt + 4 * q + j, lt = t / M;
          const float ct = cum_of(lt);
          const float dec = (ls <= lt && lt < Lc) ? expf(ct - cs_s) : 0.0f;
          const float dcb = acc[j] * dls * dec;  // d_w = dy . v^T with v = delta x (delta = 1 for RAW)
          dcbacc[k][j] += dcb;
          const float dd = dcb * CB[t * LDC + s];
#pragma unroll
          for (int rb = 0; rb < MAXRB; ++rb) {
            if (rb == rt) orow[rb][j] += dd;
            if (rb == rs) ocol[rb] += dd;
          }
        }
      }
#pragma unroll
      for (int rb = 0; rb < MAXRB; ++rb) {
        if (rb >= RB) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float s = sum16(orow[rb][j]);
          if (r16 == 0) pb[(PB_OROW * 8 + w) * 64 + 16 * rb + 4 * q + j] = s;
        }
        const float s2 = sum4q(ocol[rb]);
        if (q == 0) pb[(PB_OCOL * 8 + w) * 64 + 16 * rb + r16] = s2;
      }
    }
    dend = wave_sum(dend);
    if (lane == 0) pb[(PB_DEND * 8 + w) * 64] = dend;
    __syncthreads();  // dSl complete

    // ---- K3: d_dv = B . dS^T ; ORANGE: d_v_or = (CB * decay)^T . dy ; dx ----
    // This wave's p tiles, all row blocks.  Partial row sums over p go to one
    // LDS slot per p tile.
#pragma unroll
    for (int k2 = 0; k2 < MAXPW; ++k2) {
      const int pt = w + 4 * k2;
      if (pt >= PT) continue;
      f32x4 acc3[MAXRB], acc5[MAXRB];
#pragma unroll
      for (int rb = 0; rb < MAXRB; ++rb) acc3[rb] = acc5[rb] = zero4();
#pragma unroll 1
      for (int kb = 0; kb < NT; ++kb) {
        const frag4 fb = load4(dSl + (16 * pt + r16) * LDN + 16 * kb + 4 * q);
#pragma unroll
        for (int rb = 0; rb < MAXRB; ++rb) {
          if (rb >= RB) break;
          Mma<T>::run(acc3[rb], bc_frag(Bg, 16 * rb + r16, 16 * kb + 4 * q), fb);
        }
      }
#pragma unroll
      for (int kb = 0; kb < MAXRB; ++kb) {  // k block of t; rows s of block rb <= kb
        if (kb >= RB) break;
        frag4 fd;
        float ct[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * kb + 4 * q + j;
          fd.v[j] = (float)dys[t * LDP + 16 * pt + r16];
          ct[j] = cum_of(t / M);
        }
#pragma unroll
        for (int rb = 0; rb < MAXRB; ++rb) {
          if (rb > kb) break;
          const int s = 16 * rb + r16, ls = s / M;
          const float cs_s = cum_of(ls);
          frag4 fw;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = 16 * kb + 4 * q + j, lt = t / M;
            fw.v[j] = (ls <= lt && lt < Lc) ? CB[t * LDC + s] * expf(ct[j] - cs_s) : 0.0f;
          }
          Mma<T>::run(acc5[rb], fw, fd);
        }
      }
#pragma unroll
      for (int rb = 0; rb < MAXRB; ++rb) {
        if (rb >= RB) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * rb + 4 * q + j, l = r / M, m = r % M, p = 16 * pt + r16;
          const float dl = delta_of(l);
          const float edec = expf(cs.end - cum_of(l));
          const float xval = (float)xs[r * LDP + p];
          const float dv = acc3[rb][j] * edec + acc5[rb][j];  // d_v = d_v_k3 + d_v_orange
          if (l < Lc) st(dxg, ix_xv(a, bi, t0 + l, m, h, p), a.raw ? dv : dv * dl);
          const float s1 = sum16(acc3[rb][j] * dl * xval);     // d_decay = sum_p d_decayed_v . v
          const float s2 = sum16(dv * xval);
          if (r16 == 0) {
            pb[(PB_DEC * 8 + pt) * 64 + r] = s1;
            pb[(PB_DVX * 8 + pt) * 64 + r] = s2;
          }
        }
      }
    }
    __syncthreads();  // partial row sums complete

    // ---- d_cumA from its four sources, K1 suffix sum, chain to d_dt (wave 0) ----
    if (w == 0) {
      float dc = 0.0f, qv = 0.0f, dvx = 0.0f;
      if (lane < LM) {
        float blue = 0, orow = 0, ocol = 0, dec = 0;
        for (int ww = 0; ww < 4; ++ww) {
          blue += pb[(PB_BLUE * 8 + ww) * 64 + lane];
          orow += pb[(PB_OROW * 8 + ww) * 64 + lane];
          ocol += pb[(PB_OCOL * 8 + ww) * 64 + lane];
        }
        for (int pt = 0; pt < PT; ++pt) {
          dec += pb[(PB_DEC * 8 + pt) * 64 + lane];
          dvx += pb[(PB_DVX * 8 + pt) * 64 + lane];
        }
        qv = dec * expf(cs.end - cum_of(lane / M));
        dc = blue + orow - ocol - qv;
      }
      const float qsum = wave_sum(qv);
      float dendt = 0.0f;
      for (int ww = 0; ww < 4; ++ww) dendt += pb[(PB_DEND * 8 + ww) * 64];
      dendt *= expf(cs.end);
      // reduce the fused rows over the rank m: step l collects rows l*M .. l*M+M-1
      float dcl = 0.0f, dvxl = 0.0f;
      for (int m = 0; m < M; ++m) {
        const int src = (lane * M + m) & 63;
        const float v1 = __shfl(dc, src, 64), v2 = __shfl(dvx, src, 64);
        if (lane < L) {
          dcl += v1;
          dvxl += v2;
        }
      }
      if (lane == Lc - 1) dcl += qsum + dendt;  // K3 d cumA_last and K4 d da_chunk_end
      const float dda = wave_incl_suffix(lane < Lc ? dcl : 0.0f, lane);
      if (lane < Lc) {
        const i64 o = (bi * a.T + t0 + lane) * a.H + h;
        a.d_dtda[o] = a.raw ? dda : (dvxl + dda * Ah) * cs.sig;
      }
    }
  }

  // ---- K2 backward on the head-summed d_cb: dC_k2 = d_cb . B, dB_k2 = d_cb^T . C ----
  __syncthreads();
#pragma unroll
  for (int k = 0; k < MAXG; ++k) {
    const int rt = pair_rt[k], rs = pair_rs[k];
    if (rt < 0) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) CB[(16 * rt + 4 * q + j) * LDC + 16 * rs + r16] = dcbacc[k][j];
  }
  __syncthreads();
  float* partB = a.part;
  float* partC = a.part + a.hsplit * a.b * a.T * a.M * a.G * a.N;
#pragma unroll
  for (int rb = 0; rb < MAXRB; ++rb) {
    if (rb >= RB) break;
#pragma unroll
    for (int k = 0; k < MAXNW; ++k) {
      const int nt = w + 4 * k;
      if (nt >= NT) continue;
      f32x4 accC = dCacc[rb][k], accB = dBacc[rb][k];
      for (int kb = 0; kb <= rb; ++kb) {
        const frag4 fa = load4(CB + (16 * rb + r16) * LDC + 16 * kb + 4 * q);
        frag4 fb;
#pragma unroll
        for (int j = 0; j < 4; ++j) fb.v[j] = bc_elem(Bg, 16 * kb + 4 * q + j, 16 * nt + r16);
        Mma<T>::run(accC, fa, fb);
      }
      for (int kb = rb; kb < RB; ++kb) {
        frag4 fa, fb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          fa.v[j] = CB[(16 * kb + 4 * q + j) * LDC + 16 * rb + r16];
          fb.v[j] = bc_elem(Cg, 16 * kb + 4 * q + j, 16 * nt + r16);
        }
        Mma<T>::run(accB, fa, fb);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * rb + 4 * q + j, l = r / M, m = r % M, n = 16 * nt + r16;
        if (l >= Lc) continue;
        const i64 o = ix_bc(a, bi, t0 + l, m, g, n);
        if (a.hsplit == 1) {
          st((T*)a.dB, o, accB[j]);
          st((T*)a.dC, o, accC[j]);
        } else {
          const i64 stride = a.b * a.T * a.M * a.G * a.N;
          partB[hs * stride + o] = accB[j];
          partC[hs * stride + o] = accC[j];
        }
      }
    }
  }
}

template <typename T>
__global__ void ssd_head_sum_kernel(const float* __restrict__ part, i64 n, i64 hsplit, T* __restrict__ dB,
                                    T* __restrict__ dC) {
  const i64 i = (i64)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float sb = 0.0f, sc = 0.0f;
  for (i64 s = 0; s < hsplit; ++s) {
    sb += part[s * n + i];
    sc += part[(hsplit + s) * n + i];
  }
  st(dB, i, sb);
  st(dC, i, sc);
}

// ===========================================================================
// host side
// ===========================================================================
static int scan_nb(const ssmvjp_ssd_desc& d) {
  // n-block per scan workgroup: at most SCAN_MAXT * 4 state tiles per workgroup
  i64 nb = d.dstate;
  while ((d.headdim / 16) * (nb / 16) > SCAN_MAXT * 4 && nb % 32 == 0) nb /= 2;
  return (int)nb;
}

static i64 pick_hsplit(const ssmvjp_ssd_desc& d, i64 nc) {
  const i64 hpg = d.nheads / d.ngroups;
  const i64 base = d.batch * nc * d.ngroups;
  i64 hs = 1;
  while (base * hs < 512 && hs * 2 <= hpg && hpg % (hs * 2) == 0) hs *= 2;
  return hs;
}

bool ssd_shape_supported(const ssmvjp_ssd_desc& d) {
  if (d.headdim % 16 || d.dstate % 16 || d.headdim > 128 || d.dstate > MAXNW * 4 * 16) return false;
  const i64 LM = d.chunk_len * d.mimo_rank;
  if (LM % 16 || LM > MAXRB * 16) return false;
  return (d.headdim / 16) * (scan_nb(d) / 16) <= SCAN_MAXT * 4;
}

SsdPlan ssd_plan(const ssmvjp_ssd_desc& d) {
  SsdPlan p{};
  p.nc = cdiv(d.seqlen, d.chunk_len);
  p.LM = d.chunk_len * d.mimo_rank;
  p.hsplit = pick_hsplit(d, p.nc);
  p.state_elem = d.dtype == SSMVJP_BF16 ? 2 : 4;
  const i64 states = d.batch * p.nc * d.nheads * d.headdim * d.dstate;
  i64 off = 0;
  auto carve = [&](i64 bytes) {
    const i64 o = off;
    off += cdiv(bytes, 256) * 256;
    return o;
  };
  p.off_S = carve(states * p.state_elem);
  p.off_dS = carve(states * p.state_elem);
  p.off_part = carve(p.hsplit > 1 ? 2 * p.hsplit * d.batch * d.seqlen * d.mimo_rank * d.ngroups * d.dstate * 4 : 0);
  p.bytes = (size_t)off;
  return p;
}

template <typename T>
static SsdArgs make_args(const ssmvjp_ssd_desc& d, const SsdPlan& plan, const SsdPointers& ptr) {
  char* ws = (char*)ptr.workspace;
  SsdArgs a;
  a.b = d.batch; a.T = d.seqlen; a.H = d.nheads; a.P = d.headdim; a.N = d.dstate; a.G = d.ngroups;
  a.M = d.mimo_rank; a.L = d.chunk_len; a.LM = plan.LM; a.nc = plan.nc; a.hpg = d.nheads / d.ngroups;
  a.hsplit = plan.hsplit; a.hph = a.hpg / a.hsplit;
  a.raw = d.form == SSMVJP_FORM_RAW;
  a.xv = ptr.xv; a.dtda = ptr.dtda; a.A = ptr.A; a.B = ptr.B; a.C = ptr.C; a.s0 = ptr.s0; a.dy = ptr.dy;
  a.dsf = ptr.ds_final; a.dxv = ptr.dxv; a.d_dtda = ptr.d_dtda; a.dB = ptr.dB; a.dC = ptr.dC; a.d_s0 = ptr.d_s0;
  a.S = ws + plan.off_S;
  a.dS = ws + plan.off_dS;
  a.part = (float*)(ws + plan.off_part);
  return a;
}

template <typename T>
static void launch_states_t(const SsdArgs& a, hipStream_t stream, int NB) {
  const int LDK = (int)a.LM + (sizeof(T) == 2 ? 8 : 4);
  const size_t lds1 = 68 * sizeof(float) + sizeof(T) * (size_t)LDK * (a.P + NB);
  const i64 grid1 = a.b * a.H * 2 * (a.N / NB);
  hipLaunchKernelGGL(ssd_state_scan_kernel<T>, dim3((unsigned)grid1), dim3(256), lds1, stream, a, NB);
}

template <typename T>
static void launch_grads_t(const SsdArgs& a, hipStream_t stream) {
  if (a.T == 0) return;
  const int LDP = (int)a.P + (sizeof(T) == 2 ? 8 : 4);
  const int LDN = (int)a.N + (sizeof(T) == 2 ? 8 : 4);
  const size_t lds2 = sizeof(float) * ((size_t)a.LM * (a.LM + 4) + 2 * PB_N * 8 * 64) +
                      sizeof(T) * (2 * (size_t)a.LM * LDP + (size_t)a.P * LDN);
  const i64 grid2 = a.b * a.nc * a.G * a.hsplit;
  hipLaunchKernelGGL(ssd_chunk_bwd_kernel<T>, dim3((unsigned)grid2), dim3(256), lds2, stream, a);
  if (a.hsplit > 1) {
    const i64 n = a.b * a.T * a.M * a.G * a.N;
    hipLaunchKernelGGL(ssd_head_sum_kernel<T>, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, stream, a.part, n,
                       a.hsplit, (T*)a.dB, (T*)a.dC);
  }
}

hipError_t launch_ssd_bwd(const ssmvjp_ssd_desc& d, const SsdPlan& plan, const SsdPointers& ptr,
                          hipStream_t stream, int stages) {
  const int NB = scan_nb(d);
  if (d.dtype == SSMVJP_BF16) {
    const SsdArgs a = make_args<bf16>(d, plan, ptr);
    if (stages & SSD_STAGE_STATES) launch_states_t<bf16>(a, stream, NB);
    if (stages & SSD_STAGE_GRADS) launch_grads_t<bf16>(a, stream);
  } else {
    const SsdArgs a = make_args<float>(d, plan, ptr);
    if (stages & SSD_STAGE_STATES) launch_states_t<float>(a, stream, NB);
    if (stages & SSD_STAGE_GRADS) launch_grads_t<float>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace ssmvjp
