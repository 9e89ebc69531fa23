// delta_rule.hip -- backward of the KDA gated delta rule (K3 notes, section
// "反向传播推导": forward F1..F6 and the grouping of value heads under qk heads).
//
// Per (batch b, value head hv) the forward keeps a [K x V] state S and, at
// step t, with the key/query of qk head h = hv / (HV/H):
//   S_dec = exp(g_t) (.) S_{t-1}     (one gate per key channel, F1)
//   r     = v_t - k_t^T S_dec        (F2, F3)
//   S_t   = S_dec + (beta_t k_t) (x) r     (F4, F5)
//   o_t   = (scale q_t)^T S_t        (F6)
// The backward walks t = T-1 .. 0 carrying dS (seeded with dS_final).  With
// one vector per state column, u = dS'^T k_t (dS' = dS after the readout's
// part), every gradient of the step follows (the adjoint of the step written
// as S_t = (I - beta k k^T) S_dec + beta k v^T):
//   dS' = dS + (scale q_t) (x) do_t ;   dq_e = S_t do_t
//   dv = dr = beta_t u ;   dbeta = u . r
//   dk_e = beta_t (dS' r - S_dec u)
//   dS_dec = dS' - k_t (x) dr   (the path through r, summed with the direct one)
//   dg = rowsum(S_dec (.) dS_dec) ;   dS_{t-1} = exp(g_t) (.) dS_dec
//   dq = scale * sum of dq_e, dk = sum of dk_e over the value heads of a qk head.
//
// MI355X organisation (three launches):
//  * Columns of S are independent in the recurrence (r[v] and the update of
//    column v read column v only), so V is cut into 32-column slices and every
//    kernel runs one workgroup (8 waves, two per SIMD) per (batch, value head,
//    slice).  A thread owns a 4 x 2 block of its slice (rows 4kq..4kq+3,
//    columns 2vq, 2vq+1); the 32 threads that share a column block sit in one
//    half wave, so the per-column sums over k (k^T S_dec, k^T dS') are DPP row
//    sums plus one permlane16 swap, with no LDS traffic and no barrier.
//  * delta_fwd_ckpt_kernel walks the sequence forward and stores the state
//    at the start of every NS-step sub-segment (the checkpoints) and the
//    residual r of every step.
//  * delta_bwd_kernel walks the sub-segments in reverse: it recomputes the
//    NS states of a sub-segment from its checkpoint and the stored residuals
//    into registers (elementwise: no column sums), then runs the NS backward
//    steps.  dv is a per-column output and is stored directly.  The per-row
//    outputs (dq_e, dk_e, dg: sums over v) never feed back into the
//    recurrence; each thread folds its 2 columns, half waves are paired with
//    one permlane32 swap, and the 8 waves are summed through LDS once per
//    sub-segment into the slice's partial sums (rows stored in the order the
//    lanes hold them, so that the LDS reads and the stores are contiguous),
//    together with the slice's part of dbeta = sum over the columns of u r.
//  * delta_reduce_kernel adds the slice partials in slice order, applies the
//    sum over the value heads of each qk head (ascending), and forms dq, dk,
//    dg and dbeta.  The walk's dk partials leave out the factor beta_t, which
//    is the same for every column of a value head: the reduction applies it
//    once per value head.  Likewise dq_e = S_t do is taken as
//    S_dec do + beta_t k (r . do), so the walk never rebuilds S_t per element.
// The next sub-segment's inputs and checkpoint are loaded into registers while
// the current one runs.  Everything is float32; every sum runs in a fixed
// order, so results are bitwise reproducible.  No float atomics.
#include "common.cuh"
#include "kernels.h"

namespace ssmvjp {
namespace {

constexpr int DK = 128;          // key dimension: rows of the state
constexpr int NW = 8;            // waves per workgroup
constexpr int NTH = 64 * NW;
constexpr int VT = 2;            // state columns per thread
constexpr int NE = 4 * VT;       // state elements per thread (4 rows x VT columns)
constexpr int VS = NW * 2 * VT;  // columns of the state per workgroup (16 column blocks of 2)
constexpr int NS = 8;            // steps per sub-segment = checkpoint interval
constexpr int NQ = 3;            // per-row outputs: dq_e, dk_e / beta, dg
constexpr int NO = 4 * NQ;       // per-row outputs of one thread (4 rows each)

struct DeltaArgs {
  i64 b, T, H, HV, V, nvs, nck, grp;
  float scale;
  const float *q, *k, *v, *beta, *g, *S0, *d_o, *dSf;
  float *dq, *dk, *dv, *dg, *dbeta, *dS0;
  float* ck;     // [b][HV][nvs][nck][NE/4][NTH] float4: state at the start of each sub-segment
  float* rres;   // [b][HV][nvs][nck*NS][VS] residual r of every step, per slice
  float* part;   // [b][T][HV][nvs][NQ][4][32] per-slice partial sums of the per-row outputs;
                 // row k = 4 kq + i at [i][kq]
  float* partb;  // [b][T][HV][nvs] per-slice partial sums of dbeta
};

// sum over the 32 lanes of a half wave; every lane of the half wave gets the
// same bits (the rotation tree and the pair swap add the same operands)
__device__ __forceinline__ float sum32(float v) {
  v = sum16(v);
  const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), false, false);
  return __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
}

// lanes 0..31 get x[l] + x[l+32] of a, lanes 32..63 get the same sum of b
__device__ __forceinline__ float pair_halves(float a, float b) {
  const auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, a), __builtin_bit_cast(int, b), false, false);
  return __builtin_bit_cast(float, (int)s[0]) + __builtin_bit_cast(float, (int)s[1]);
}

__device__ __forceinline__ f32x4 as_f4(u32x4 u) {
  return f32x4{__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]), __uint_as_float(u[3])};
}
__device__ __forceinline__ f32x4 lds4(const float* p) { return *(const f32x4*)p; }

// Workgroup -> (batch, qk head, value head, slice).  The value heads and
// slices that read the same q/k rows get ids congruent modulo b*H, so they
// land on the same XCD (ids are dealt to the 8 XCDs round robin) when b*H is
// a multiple of 8 and share those rows in its L2.
struct Slot {
  i64 bi, h, hv, vs;
};
__device__ __forceinline__ Slot slot_of(const DeltaArgs& a) {
  const i64 ngrp = a.b * a.H, id = blockIdx.x;
  const i64 grp_id = id % ngrp, member = id / ngrp;
  Slot s;
  s.bi = grp_id / a.H;
  s.h = grp_id % a.H;
  s.hv = s.h * a.grp + member / a.nvs;
  s.vs = member % a.nvs;
  return s;
}

// One forward step on this thread's 4 x VT block (S[VT*i+c]: row 4kq+i,
// column VT*vq+c): sd = exp(g) (.) S, r = v - k^T sd (column sums over the
// half wave), S = sd + (beta k) (x) r, with beta k staged per step (bk).
__device__ __forceinline__ void fwd_step(float S[NE], float sd[NE], f32x4 eg, f32x4 kk, f32x4 bk, const float vv[VT],
                                         float r[VT]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < VT; ++c) sd[VT * i + c] = eg[i] * S[VT * i + c];
#pragma unroll
  for (int c = 0; c < VT; ++c) {
    float p = kk[0] * sd[c];
#pragma unroll
    for (int i = 1; i < 4; ++i) p = fmaf(kk[i], sd[VT * i + c], p);
    r[c] = vv[c] - sum32(p);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < VT; ++c) S[VT * i + c] = fmaf(bk[i], r[c], sd[VT * i + c]);
}

__device__ __forceinline__ void ld_cols(const float* p, float o[VT]) {
  const float2 u = *(const float2*)p;
  o[0] = u.x;
  o[1] = u.y;
}

// byte size of the valid rows of one sub-segment in a [.., T, heads, width] tensor
__device__ __forceinline__ unsigned seg_bytes(int ns, i64 row_stride, int width) {
  return (unsigned)(((i64)(ns - 1) * row_stride + width) * 4);
}

// ===========================================================================
// forward walk: checkpoints at the start of every sub-segment
// ===========================================================================
// this thread's 4 x VT block of a [K x V] state (row stride V), through a
// range-checked resource (NULL base: zeros)
__device__ __forceinline__ void load_block(float S[NE], const float* base, i64 V, int kq, int vq) {
  const brsrc r0 = make_rsrc(base ? base : (const float*)nullptr, base ? (unsigned)(((DK - 1) * V + VS) * 4) : 0u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto u = __builtin_amdgcn_raw_buffer_load_b64(r0, (int)(((4 * kq + i) * V + VT * vq) * 4), 0, 0);
    S[VT * i] = __uint_as_float(u[0]);
    S[VT * i + 1] = __uint_as_float(u[1]);
  }
}

__global__ void __launch_bounds__(NTH) delta_fwd_ckpt_kernel(DeltaArgs a) {
  __shared__ __align__(16) float sk[NS][DK];
  __shared__ __align__(16) float sbk[NS][DK];  // beta k
  __shared__ __align__(16) float se[NS][DK];
  __shared__ __align__(16) float sv[NS][VS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kq = lane & 31, vq = 2 * w + (lane >> 5);
  const Slot sl = slot_of(a);
  const i64 T = a.T, V = a.V;

  float S[NE];
  load_block(S, a.S0 ? a.S0 + (sl.bi * a.HV + sl.hv) * DK * V + sl.vs * VS : nullptr, V, kq, vq);
  // register prefetch of one sub-segment (threads 0..255): k and g rows (one
  // float4 each) and the row's beta, the slice of v (threads 0..63)
  u32x4 pk, pg, pv;
  float pb;
  const int srow = (tid & 255) >> 5, scol = 4 * (tid & 31);
  const bool stager = tid < 256;
  auto issue = [&](i64 j) {
    const i64 t0 = j * NS;
    const int ns = (int)(T - t0 < NS ? T - t0 : NS);
    const brsrc rk = make_rsrc(a.k + ((sl.bi * T + t0) * a.H + sl.h) * DK, seg_bytes(ns, a.H * DK, DK));
    const brsrc rg = make_rsrc(a.g + ((sl.bi * T + t0) * a.HV + sl.hv) * DK, seg_bytes(ns, a.HV * DK, DK));
    const brsrc rv = make_rsrc(a.v + ((sl.bi * T + t0) * a.HV + sl.hv) * V + sl.vs * VS, seg_bytes(ns, a.HV * V, VS));
    const brsrc rb = make_rsrc(a.beta + (sl.bi * T + t0) * a.HV + sl.hv, seg_bytes(ns, a.HV, 1));
    pk = bload16(rk, stager ? (unsigned)((srow * a.H * DK + scol) * 4) : BUF_OOB);
    pg = bload16(rg, stager ? (unsigned)((srow * a.HV * DK + scol) * 4) : BUF_OOB);
    pv = bload16(rv, tid < NS * VS / 4 ? (unsigned)(((tid >> 3) * a.HV * V + 4 * (tid & 7)) * 4) : BUF_OOB);
    pb = bload_f32(rb, stager ? (unsigned)(srow * a.HV * 4) : BUF_OOB);
  };
  float* ckb = a.ck + ((sl.bi * a.HV + sl.hv) * a.nvs + sl.vs) * a.nck * (NE * NTH);
  float* rb = a.rres + ((sl.bi * a.HV + sl.hv) * a.nvs + sl.vs) * a.nck * NS * VS;
  if (a.nck > 0) issue(0);
  for (i64 j = 0; j < a.nck; ++j) {
    const int ns = (int)(T - j * NS < NS ? T - j * NS : NS);
    // checkpoint j: the state before step j*NS
#pragma unroll
    for (int i = 0; i < NE / 4; ++i)
      *(f32x4*)(ckb + (j * (NE / 4) + i) * NTH * 4 + tid * 4) = f32x4{S[4 * i], S[4 * i + 1], S[4 * i + 2], S[4 * i + 3]};
    __syncthreads();  // the previous sub-segment is done with the staged rows
    if (stager) {
      const f32x4 kk = as_f4(pk), gg = as_f4(pg);
      *(f32x4*)&sk[srow][scol] = kk;
      *(f32x4*)&sbk[srow][scol] = f32x4{pb * kk[0], pb * kk[1], pb * kk[2], pb * kk[3]};
      *(f32x4*)&se[srow][scol] = f32x4{expf(gg[0]), expf(gg[1]), expf(gg[2]), expf(gg[3])};
    }
    if (tid < NS * VS / 4) *(f32x4*)&sv[tid >> 3][4 * (tid & 7)] = as_f4(pv);
    if (j + 1 < a.nck) issue(j + 1);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s >= ns) break;
      float sd[NE], r[VT], vv[VT];
      ld_cols(&sv[s][VT * vq], vv);
      fwd_step(S, sd, lds4(&se[s][4 * kq]), lds4(&sk[s][4 * kq]), lds4(&sbk[s][4 * kq]), vv, r);
      // the residual of this step for the backward's recompute (one lane per column block)
      if (kq == 0) *(float2*)(rb + (j * NS + s) * VS + VT * vq) = make_float2(r[0], r[1]);
    }
  }
}

// ===========================================================================
// backward walk over the sub-segments, in reverse
// ===========================================================================
__global__ void __launch_bounds__(NTH) delta_bwd_kernel(DeltaArgs a) {
  __shared__ __align__(16) float sq[NS][DK];  // scale * q
  __shared__ __align__(16) float sk[NS][DK];
  __shared__ __align__(16) float sbk[NS][DK];  // beta k
  __shared__ __align__(16) float se[NS][DK];  // exp(g)
  __shared__ __align__(16) float sdo[NS][VS];
  __shared__ __align__(16) float sr[NS][VS];  // r of each step, per column
  __shared__ float sb[NS];
  __shared__ __align__(16) float red[NS][NW][NO][32];  // per-wave per-row outputs, [4 qd + i][kq]
  __shared__ float redb[NS][NW];                        // per-wave parts of dbeta
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5;
  const int kq = lane & 31, vq = 2 * w + half;
  const Slot sl = slot_of(a);
  const i64 T = a.T, V = a.V;

  float dS[NE];
  load_block(dS, a.dSf ? a.dSf + (sl.bi * a.HV + sl.hv) * DK * V + sl.vs * VS : nullptr, V, kq, vq);

  // register prefetch of one sub-segment: q, k, g rows (threads 0..255, one
  // float4 each), the slices of r (threads 0..63) and do (threads 64..127),
  // beta (threads 0..NS-1, and each stager its row's), and every thread's
  // part of the checkpoint
  u32x4 pq, pk, pg, pr, pd, pc[NE / 4];
  float pb, pbr;
  const int srow = (tid & 255) >> 5, scol = 4 * (tid & 31);
  const bool stager = tid < 256;
  const int vrow = (tid & 63) >> 3, vcol = 4 * (tid & 7);
  const i64 slice = (sl.bi * a.HV + sl.hv) * a.nvs + sl.vs;
  const float* ckb = a.ck + slice * a.nck * (NE * NTH);
  const float* rsb = a.rres + slice * a.nck * NS * VS;
  auto issue = [&](i64 j) {
    const i64 t0 = j * NS;
    const int ns = (int)(T - t0 < NS ? T - t0 : NS);
    const i64 qk0 = ((sl.bi * T + t0) * a.H + sl.h) * DK, hv0 = (sl.bi * T + t0) * a.HV + sl.hv;
    const brsrc rq = make_rsrc(a.q + qk0, seg_bytes(ns, a.H * DK, DK));
    const brsrc rk = make_rsrc(a.k + qk0, seg_bytes(ns, a.H * DK, DK));
    const brsrc rg = make_rsrc(a.g + hv0 * DK, seg_bytes(ns, a.HV * DK, DK));
    const brsrc rr = make_rsrc(rsb + t0 * VS, (unsigned)(ns * VS * 4));
    const brsrc rd = make_rsrc(a.d_o + hv0 * V + sl.vs * VS, seg_bytes(ns, a.HV * V, VS));
    const brsrc rb = make_rsrc(a.beta + hv0, seg_bytes(ns, a.HV, 1));
    const brsrc rc = make_rsrc(ckb + j * NE * NTH, NE * NTH * 4);
    const unsigned qoff = stager ? (unsigned)((srow * a.H * DK + scol) * 4) : BUF_OOB;
    pq = bload16(rq, qoff);
    pk = bload16(rk, qoff);
    pg = bload16(rg, stager ? (unsigned)((srow * a.HV * DK + scol) * 4) : BUF_OOB);
    pr = bload16(rr, tid < 64 ? (unsigned)((vrow * VS + vcol) * 4) : BUF_OOB);
    pd = bload16(rd, tid >= 64 && tid < 128 ? (unsigned)((vrow * a.HV * V + vcol) * 4) : BUF_OOB);
    pb = bload_f32(rb, tid < NS ? (unsigned)(tid * a.HV * 4) : BUF_OOB);
    pbr = bload_f32(rb, stager ? (unsigned)(srow * a.HV * 4) : BUF_OOB);
#pragma unroll
    for (int i = 0; i < NE / 4; ++i) pc[i] = bload16(rc, (unsigned)((i * NTH + tid) * 16));
  };

  if (a.nck > 0) issue(a.nck - 1);
  for (i64 j = a.nck - 1; j >= 0; --j) {
    const i64 t0 = j * NS;
    const int ns = (int)(T - t0 < NS ? T - t0 : NS);
    // stage this sub-segment (the previous one finished reading the staged
    // rows before its last barrier)
    float S[NE];
    {
      if (stager) {
        const f32x4 qq = as_f4(pq), gg = as_f4(pg), kk = as_f4(pk);
        *(f32x4*)&sq[srow][scol] = f32x4{a.scale * qq[0], a.scale * qq[1], a.scale * qq[2], a.scale * qq[3]};
        *(f32x4*)&sk[srow][scol] = kk;
        *(f32x4*)&sbk[srow][scol] = f32x4{pbr * kk[0], pbr * kk[1], pbr * kk[2], pbr * kk[3]};
        *(f32x4*)&se[srow][scol] = f32x4{expf(gg[0]), expf(gg[1]), expf(gg[2]), expf(gg[3])};
      }
      if (tid < 64) *(f32x4*)&sr[vrow][vcol] = as_f4(pr);
      if (tid >= 64 && tid < 128) *(f32x4*)&sdo[vrow][vcol] = as_f4(pd);
      if (tid < NS) sb[tid] = pb;
#pragma unroll
      for (int i = 0; i < NE / 4; ++i) {
        const f32x4 x = as_f4(pc[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) S[4 * i + e] = x[e];
      }
    }
    if (j > 0) issue(j - 1);
    __syncthreads();  // staged rows visible; the previous reduction is done with red

    // recompute the sub-segment's S_dec into registers from the checkpoint and
    // the stored residuals: S_dec = exp(g) (.) S, S = S_dec + (beta k) (x) r
    float sd[NS][NE];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s >= ns) break;
      const f32x4 eg = lds4(&se[s][4 * kq]), bk = lds4(&sbk[s][4 * kq]);
      float rr[VT];
      ld_cols(&sr[s][VT * vq], rr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int c = 0; c < VT; ++c) {
          sd[s][VT * i + c] = eg[i] * S[VT * i + c];
          S[VT * i + c] = fmaf(bk[i], rr[c], sd[s][VT * i + c]);
        }
      }
    }

    // backward steps
#pragma unroll
    for (int s = NS - 1; s >= 0; --s) {
      if (s >= ns) continue;
      const f32x4 qq = lds4(&sq[s][4 * kq]), kk = lds4(&sk[s][4 * kq]), eg = lds4(&se[s][4 * kq]);
      const f32x4 bk = lds4(&sbk[s][4 * kq]);
      float dd[VT], rr[VT];
      ld_cols(&sdo[s][VT * vq], dd);
      ld_cols(&sr[s][VT * vq], rr);
      const float beta = sb[s];
      float o[NO];  // per-row outputs: o[4*qd + i], qd = dq_e, dk_e / beta, dg
      float da[4], up[VT];
      float rd = 0.0f;  // r . do over this thread's columns
#pragma unroll
      for (int c = 0; c < VT; ++c) rd = fmaf(rr[c], dd[c], rd);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float dq_e = 0.0f, dai = 0.0f;
#pragma unroll
        for (int c = 0; c < VT; ++c) {
          const int e = VT * i + c;
          dS[e] = fmaf(qq[i], dd[c], dS[e]);  // dS' = dS + (scale q) (x) do
          dq_e = fmaf(sd[s][e], dd[c], dq_e); // S_dec do
          dai = fmaf(rr[c], dS[e], dai);      // dS' r
          up[c] = i == 0 ? kk[i] * dS[e] : fmaf(kk[i], dS[e], up[c]);  // u = dS'^T k
        }
        o[i] = fmaf(bk[i], rd, dq_e);  // dq_e = S_t do = S_dec do + beta k (r . do)
        da[i] = dai;
      }
      float u[VT], dr[VT];
#pragma unroll
      for (int c = 0; c < VT; ++c) {
        u[c] = sum32(up[c]);
        dr[c] = beta * u[c];
      }
      const float bpart = fmaf(rr[0], u[0], rr[1] * u[1]);  // this column block's u . r
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float dg = 0.0f;
#pragma unroll
        for (int c = 0; c < VT; ++c) {
          const int e = VT * i + c;
          da[i] = fmaf(sd[s][e], -u[c], da[i]);  // dS' r - S_dec u
          dS[e] = fmaf(-kk[i], dr[c], dS[e]);    // dS_dec = dS' - k (x) dr
          dg = fmaf(sd[s][e], dS[e], dg);        // dg = rowsum(S_dec (.) dS_dec)
          dS[e] *= eg[i];                        // dS_{t-1} = exp(g) (.) dS_dec
        }
        o[4 + i] = da[i];  // dk_e / beta (the reduction applies beta per value head)
        o[8 + i] = dg;
      }
      // dv = dr: this column block's values, from one lane per half wave
      if (kq == 0) {
        float* dvp = a.dv + ((sl.bi * T + t0 + s) * a.HV + sl.hv) * V + sl.vs * VS + VT * vq;
        *(float2*)dvp = make_float2(dr[0], dr[1]);
      }
      // per-row outputs: pair the half waves (same rows, other columns); half
      // 0 keeps outputs 0..5, half 1 outputs 6..11
#pragma unroll
      for (int jv = 0; jv < NO / 2; ++jv) red[s][w][(NO / 2) * half + jv][kq] = pair_halves(o[jv], o[NO / 2 + jv]);
      const float bw = pair_halves(bpart, bpart);  // both halves: the wave's 4 columns
      if (lane == 0) redb[s][w] = bw;
    }
    __syncthreads();  // red complete
    // sum the waves: thread (row group kq, output slots p = m*16 + tid/32) reads
    // red[s][.][js][kq] for 32 consecutive kq (one bank each), stores 32
    // consecutive partial sums
    {
      const int pk0 = tid >> 5;
#pragma unroll
      for (int m = 0; m < NS * NO / (NTH / 32); ++m) {
        const int pidx = pk0 + (NTH / 32) * m, s = pidx / NO, js = pidx % NO;
        if (s >= ns) continue;
        float acc = red[s][0][js][kq];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) acc += red[s][ww][js][kq];
        a.part[((((sl.bi * T + t0 + s) * a.HV + sl.hv) * a.nvs + sl.vs) * NQ + js / 4) * DK + (js & 3) * 32 + kq] =
            acc;
      }
      if (tid < ns) {
        float acc = redb[tid][0];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) acc += redb[tid][ww];
        a.partb[((sl.bi * T + t0 + tid) * a.HV + sl.hv) * a.nvs + sl.vs] = acc;
      }
    }
  }
  if (a.dS0) {
    float* o = a.dS0 + (sl.bi * a.HV + sl.hv) * DK * V + sl.vs * VS + VT * vq;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(float2*)(o + (4 * kq + i) * V) = make_float2(dS[VT * i], dS[VT * i + 1]);
  }
}

// ===========================================================================
// slice sums, GVA sum, dq / dk / dg / dbeta: one wave per (batch, t, qk head)
// ===========================================================================
__global__ void __launch_bounds__(256) delta_reduce_kernel(DeltaArgs a) {
  const int lane = threadIdx.x & 63;
  const i64 id = (i64)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (id >= a.b * a.T * a.H) return;  // whole waves
  const i64 h = id % a.H, bt = id / a.H;
  // lane handles stored positions lane and lane + 64, i.e. rows k = 4 (p % 32) + p / 32
  const int k0 = 4 * (lane & 31) + (lane >> 5), k1 = k0 + 2;
  float dq0 = 0.f, dq1 = 0.f, dk0 = 0.f, dk1 = 0.f;
  for (i64 j = 0; j < a.grp; ++j) {
    const i64 hv = h * a.grp + j;
    const float* pp = a.part + (bt * a.HV + hv) * a.nvs * NQ * DK;
    float s[NQ][2];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd) s[qd][0] = s[qd][1] = 0.0f;
    for (i64 vs = 0; vs < a.nvs; ++vs)
#pragma unroll
      for (int qd = 0; qd < NQ; ++qd) {
        s[qd][0] += pp[(vs * NQ + qd) * DK + lane];
        s[qd][1] += pp[(vs * NQ + qd) * DK + 64 + lane];
      }
    float* dgp = a.dg + (bt * a.HV + hv) * DK;
    dgp[k0] = s[2][0];
    dgp[k1] = s[2][1];
    if (lane == 0) {
      const float* pb = a.partb + (bt * a.HV + hv) * a.nvs;
      float db = 0.0f;
      for (i64 vs = 0; vs < a.nvs; ++vs) db += pb[vs];
      a.dbeta[bt * a.HV + hv] = db;
    }
    const float bv = a.beta[bt * a.HV + hv];  // dk_e = beta (dS' r - S_dec u): beta applied here
    dq0 += s[0][0];
    dq1 += s[0][1];
    dk0 = fmaf(bv, s[1][0], dk0);
    dk1 = fmaf(bv, s[1][1], dk1);
  }
  float* dqp = a.dq + (bt * a.H + h) * DK;
  float* dkp = a.dk + (bt * a.H + h) * DK;
  dqp[k0] = a.scale * dq0;
  dqp[k1] = a.scale * dq1;
  dkp[k0] = dk0;
  dkp[k1] = dk1;
}

}  // namespace

// ===========================================================================
// host side
// ===========================================================================
bool delta_shape_supported(const ssmvjp_delta_desc& d) {
  if (d.dk != DK || d.dv % VS != 0) return false;
  // 32-bit byte offsets inside one sub-segment's rows
  return (NS * d.nv_heads * d.dv + d.nqk_heads * DK) * 4 < (1ll << 31);
}

DeltaPlan delta_plan(const ssmvjp_delta_desc& d) {
  DeltaPlan p{};
  p.CK = NS;
  p.nck = (d.seqlen + NS - 1) / NS;
  p.vsplit = d.dv / VS;
  int64_t off = 0;
  auto carve = [&](int64_t bytes) {
    const int64_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  p.off_ck = carve(d.batch * d.nv_heads * p.nck * DK * d.dv * 4);  // NE * NTH floats per (slice, checkpoint)
  p.off_r = carve(d.batch * d.nv_heads * p.nck * NS * d.dv * 4);    // residual of every step
  p.off_part = carve(d.batch * d.seqlen * d.nv_heads * p.vsplit * NQ * DK * 4);
  p.off_partb = carve(d.batch * d.seqlen * d.nv_heads * p.vsplit * 4);
  p.bytes = (size_t)off;
  return p;
}

hipError_t launch_delta_bwd(const ssmvjp_delta_desc& d, const DeltaPlan& plan, const DeltaPointers& ptr,
                            hipStream_t stream, int stages) {
  DeltaArgs a;
  a.b = d.batch; a.T = d.seqlen; a.H = d.nqk_heads; a.HV = d.nv_heads; a.V = d.dv;
  a.nvs = plan.vsplit; a.nck = plan.nck; a.grp = d.nv_heads / d.nqk_heads; a.scale = d.scale;
  a.q = ptr.q; a.k = ptr.k; a.v = ptr.v; a.beta = ptr.beta; a.g = ptr.g; a.S0 = ptr.S0; a.d_o = ptr.d_o;
  a.dSf = ptr.dS_final; a.dq = ptr.dq; a.dk = ptr.dk; a.dv = ptr.dv; a.dg = ptr.dg; a.dbeta = ptr.dbeta;
  a.dS0 = ptr.dS0;
  char* ws = (char*)ptr.workspace;
  a.ck = (float*)(ws + plan.off_ck);
  a.rres = (float*)(ws + plan.off_r);
  a.part = (float*)(ws + plan.off_part);
  a.partb = (float*)(ws + plan.off_partb);
  const i64 nwg = d.batch * d.nv_heads * plan.vsplit;
  if (nwg == 0) return hipSuccess;
  if ((stages & SSMVJP_DELTA_CKPT) && d.seqlen > 0)
    hipLaunchKernelGGL(delta_fwd_ckpt_kernel, dim3((unsigned)nwg), dim3(NTH), 0, stream, a);
  if (stages & SSMVJP_DELTA_BWD) hipLaunchKernelGGL(delta_bwd_kernel, dim3((unsigned)nwg), dim3(NTH), 0, stream, a);
  const i64 nred = d.batch * d.seqlen * d.nqk_heads;
  if ((stages & SSMVJP_DELTA_REDUCE) && nred > 0)
    hipLaunchKernelGGL(delta_reduce_kernel, dim3((unsigned)((nred + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ssmvjp
