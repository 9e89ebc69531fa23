// scan_seq.hip -- sequential reverse recurrence of the selective-scan VJP.
//
// Follows the op of llama.cpp PR "S1-31: SSM_SCAN_BACK": walk t from T-1 down
// to 0 carrying the state gradient dS, seeded at t = T with the final-state
// gradient, and emit dx, d_dt (through the decay path and the softplus), dB,
// dC and d_s0.  Mamba-2 (one decay per head) and Mamba-1 (one per state).
//
// The forward overwrote its states, so they are recomputed; instead of storing
// all T+1 states (the page's store-all), the state before every K-th step is
// checkpointed and each K-step segment is recomputed just before the reverse
// walk reaches it (the page's checkpoint-every-K).  The recompute uses exactly
// the arithmetic of the checkpoint pass, so outputs are bitwise identical for
// every K.
//
// Kernels (one stream, in order):
//   1. seq_prologue   delta = softplus(dt), sigma(dt)               [b*T*H]
//   2. seq_ckpt       one lane per state element (b,h,p,n): forward walk,
//                     stores the state before steps 0, K, 2K, ...
//   3. seq_bwd        one workgroup per (b,h): per segment (last first)
//                     recompute, then the reverse walk; per-step reductions
//                     over n (dx), over p (this head's dB, dC) and over (p,n)
//                     (d_dt) go through LDS in a fixed order.  When one
//                     thread holds a whole column of the state (P <= 16) and
//                     a segment fits in LDS, seq_bwd_lds stages the segment's
//                     inputs and recomputed states there instead.
//   4. seq_group_sum  dB, dC = sum over the heads of each group, ascending h.
#include "common.cuh"
#include "kernels.h"

namespace ssmvjp {

struct SeqArgs {
  i64 b, T, H, P, N, G, K, J;  // J = number of checkpoints = ceil(T / K)
  int per_state;
  const void* x;
  const float* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* s0;
  const void* dy;
  const float* dsf;
  void* dx;
  float* d_dt;
  void* dB;
  void* dC;
  float* d_s0;
  float* delta;  // [b,T,H]
  float* sig;    // [b,T,H]
  float* ck;     // [J][b,H,P,N]
  float* seg;    // [b*H][K][P*N]
  float* dBh;    // [b,T,H,N]
  float* dCh;    // [b,T,H,N]
  float* dA_part;  // [b,H,N] (per state) or [b,H] (per head) partial sums of dA, or NULL
};

__global__ void seq_prologue_kernel(const float* __restrict__ dt, i64 n, float* __restrict__ delta,
                                    float* __restrict__ sig) {
  const i64 i = (i64)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float z = dt[i];
  delta[i] = softplus_f(z);
  sig[i] = sigmoid_f(z);
}

// One step of the forward recurrence.  Written with explicit roundings so the
// checkpoint pass and the segment recompute produce identical bits.
__device__ __forceinline__ float scan_step(float s, float d, float acoef, float xv, float bv) {
  const float a = expf(__fmul_rn(d, acoef));
  const float u = __fmul_rn(__fmul_rn(d, xv), bv);
  return __fmaf_rn(a, s, u);
}

template <typename T>
__global__ void seq_ckpt_kernel(SeqArgs a) {
  const i64 total = a.b * a.H * a.P * a.N;
  const i64 e = (i64)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const i64 n = e % a.N, p = (e / a.N) % a.P, h = (e / (a.N * a.P)) % a.H, bi = e / (a.N * a.P * a.H);
  const i64 g = h / (a.H / a.G);
  const float acoef = a.per_state ? a.A[h * a.N + n] : a.A[h];
  const T* x = (const T*)a.x;
  const T* B = (const T*)a.B;
  float s = a.s0 ? a.s0[e] : 0.0f;
  // the walk stops at the last checkpoint, the state before step (J-1) K:
  // the steps after it are recomputed by the reverse pass from that checkpoint.
  // The inputs of CK_GS steps are loaded together, so that their latencies
  // overlap (indices past the last step reload it; those values go unused).
  constexpr int CK_GS = 8;
  const i64 tlast = (a.J - 1) * a.K;
  for (i64 tb = 0; tb < tlast; tb += CK_GS) {
    float gd[CK_GS], gx[CK_GS], gb[CK_GS];
#pragma unroll
    for (int i = 0; i < CK_GS; ++i) {
      const i64 t = tb + i < tlast ? tb + i : tlast - 1;
      gd[i] = a.delta[(bi * a.T + t) * a.H + h];
      gx[i] = ld(x, ((bi * a.T + t) * a.H + h) * a.P + p);
      gb[i] = ld(B, ((bi * a.T + t) * a.G + g) * a.N + n);
    }
#pragma unroll
    for (int i = 0; i < CK_GS; ++i) {
      const i64 t = tb + i;
      if (t >= tlast) break;
      if (t % a.K == 0) a.ck[(t / a.K) * total + e] = s;
      s = scan_step(s, gd[i], acoef, gx[i], gb[i]);
    }
  }
  if (a.J > 0) a.ck[(a.J - 1) * total + e] = s;
}

// Thread layout of seq_bwd: thread tid = pg * N + n owns column n and the p
// range [pg*PPT, pg*PPT + PPT) of the [P, N] state.  N * NPG threads carry
// state; the launch is rounded up to whole waves and the extra threads only
// join the barriers and contribute zeros to the wave reductions.
template <typename T, int MAXPPT>
__global__ void __launch_bounds__(1024) seq_bwd_kernel(SeqArgs a, int PPT, int NPG) {
  extern __shared__ float smem[];
  const int P = (int)a.P, N = (int)a.N;
  const int NT = N * NPG;        // threads that own state
  const int tid = threadIdx.x;
  const bool active = tid < NT;
  const int n = active ? tid % N : 0;
  const int pg = active ? tid / N : NPG;  // idle threads own no p (pg * PPT >= P)
  const int nw = (int)(blockDim.x / 64);
  float* red = smem;                          // [P][N+1]  dS[p,n] * B[n] for the dx row sums
  float* colB = red + P * (N + 1);            // [NPG][N]  partial sums over this thread's p range
  float* colC = colB + NPG * N;               // [NPG][N]
  float* ddw = colC + NPG * N;                // [nw]      per-wave partials of d(delta)

  const i64 bh = blockIdx.x;
  const i64 bi = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
  const i64 PN = a.P * a.N, total = a.b * a.H * PN;
  const i64 ebase = bh * PN;  // this head's state block in [b,H,P,N]
  const T* x = (const T*)a.x;
  const T* B = (const T*)a.B;
  const T* C = (const T*)a.C;
  const T* dy = (const T*)a.dy;
  T* dx = (T*)a.dx;
  float* seg = a.seg + bh * a.K * PN;
  const float acoef = a.per_state ? a.A[h * a.N + n] : a.A[h];

  float dS[MAXPPT];
#pragma unroll
  for (int k = 0; k < MAXPPT; ++k) {
    const int p = pg * PPT + k;
    dS[k] = (k < PPT && p < P && a.dsf) ? a.dsf[ebase + (i64)p * N + n] : 0.0f;
  }
  // dA: d s_t / d A = delta a s_{t-1}, summed over this thread's p range and
  // over t (reverse order) in one register
  float dAacc = 0.0f;

  for (i64 j = a.J - 1; j >= 0; --j) {
    const i64 t0 = j * a.K;
    const i64 t1 = (t0 + a.K < a.T) ? t0 + a.K : a.T;
    // recompute the segment's states from its checkpoint (own elements only)
#pragma unroll
    for (int k = 0; k < MAXPPT; ++k) {
      const int p = pg * PPT + k;
      if (k >= PPT || p >= P) continue;
      float s = a.ck[j * total + ebase + (i64)p * N + n];
      for (i64 t = t0; t < t1; ++t) {
        const float d = a.delta[(bi * a.T + t) * a.H + h];
        s = scan_step(s, d, acoef, ld(x, ((bi * a.T + t) * a.H + h) * a.P + p), ld(B, ((bi * a.T + t) * a.G + g) * a.N + n));
        seg[(t - t0) * PN + (i64)p * N + n] = s;
      }
    }
    for (i64 t = t1 - 1; t >= t0; --t) {
      const i64 bth = (bi * a.T + t) * a.H + h;
      const float d = a.delta[bth];
      const float av = expf(__fmul_rn(d, acoef));
      const float Bn = ld(B, ((bi * a.T + t) * a.G + g) * a.N + n);
      const float Cn = ld(C, ((bi * a.T + t) * a.G + g) * a.N + n);
      float dbn = 0.0f, dcn = 0.0f, dd = 0.0f, dAs = 0.0f;
      __syncthreads();  // previous step's readers of red/colB/colC/ddw are done
#pragma unroll
      for (int k = 0; k < MAXPPT; ++k) {
        const int p = pg * PPT + k;
        if (k >= PPT || p >= P) continue;
        const float xp = ld(x, bth * a.P + p);
        const float dyp = ld(dy, bth * a.P + p);
        const float s_t = seg[(t - t0) * PN + (i64)p * N + n];
        const float s_prev = (t > t0) ? seg[(t - t0 - 1) * PN + (i64)p * N + n] : a.ck[j * total + ebase + (i64)p * N + n];
        dS[k] += dyp * Cn;                         // y_t = C_t . s_t
        dcn += dyp * s_t;                          // dC_t uses s_t
        dbn += dS[k] * xp;                         // dB_t (before the delta factor)
        dd += dS[k] * (xp * Bn + acoef * av * s_prev);  // input path + decay path
        dAs += dS[k] * s_prev;
        red[p * (N + 1) + n] = dS[k] * Bn;
      }
      dAacc += d * av * dAs;
      if (active) {
        colB[pg * N + n] = dbn;
        colC[pg * N + n] = dcn;
      }
      dd = wave_sum(dd);
      if ((tid & 63) == 0) ddw[tid >> 6] = dd;
      __syncthreads();
      for (int p = tid; p < P; p += (int)blockDim.x) {
        float acc = 0.0f;
        for (int nn = 0; nn < N; ++nn) acc += red[p * (N + 1) + nn];
        st(dx, bth * a.P + p, d * acc);
      }
      if (tid < N) {
        float sb = 0.0f, sc = 0.0f;
        for (int q = 0; q < NPG; ++q) {
          sb += colB[q * N + tid];
          sc += colC[q * N + tid];
        }
        a.dBh[bth * a.N + tid] = d * sb;
        a.dCh[bth * a.N + tid] = sc;
      }
      if (tid == 0) {
        float s = 0.0f;
        for (int w = 0; w < nw; ++w) s += ddw[w];
        a.d_dt[bth] = s * a.sig[bth];
      }
#pragma unroll
      for (int k = 0; k < MAXPPT; ++k) dS[k] *= av;
    }
  }
#pragma unroll
  for (int k = 0; k < MAXPPT; ++k) {
    const int p = pg * PPT + k;
    if (k < PPT && p < P) a.d_s0[ebase + (i64)p * N + n] = dS[k];
  }
  if (a.dA_part) {  // uniform: fixed-order sums over the p groups (per state) or all threads (per head)
    __syncthreads();  // the last step's readers of colB and ddw are done
    if (a.per_state) {
      if (active) colB[pg * N + n] = dAacc;
      __syncthreads();
      if (tid < N) {
        float s = 0.0f;
        for (int q = 0; q < NPG; ++q) s += colB[q * N + tid];
        a.dA_part[bh * a.N + tid] = s;
      }
    } else {
      const float v = wave_sum(active ? dAacc : 0.0f);
      if ((tid & 63) == 0) ddw[tid >> 6] = v;
      __syncthreads();
      if (tid == 0) {
        float s = 0.0f;
        for (int w = 0; w < nw; ++w) s += ddw[w];
        a.dA_part[bh] = s;
      }
    }
  }
}

// The same reverse walk for small states (every p of a column in one thread,
// NPG = 1), with each segment's inputs (delta, B, C, x, dy of its K steps) and
// its recomputed states held in LDS: one cooperative load per segment, so the
// steps themselves read no global memory.  Arithmetic and order are those of
// seq_bwd_kernel, so the two give identical bits.
template <typename T, int MAXP>
__global__ void __launch_bounds__(1024) seq_bwd_lds_kernel(SeqArgs a) {
  extern __shared__ float smem[];
  const int P = (int)a.P, N = (int)a.N, K = (int)a.K;
  const int tid = threadIdx.x, nw = (int)(blockDim.x / 64);
  const bool active = tid < N;
  const int n = active ? tid : 0;
  float* red = smem;                 // [P][N+1]
  float* colB = red + P * (N + 1);   // [N]
  float* colC = colB + N;            // [N]
  float* ddw = colC + N;             // [nw]
  float* sd = ddw + nw;              // [K]        delta
  float* sB = sd + K;                // [K][N]
  float* sC = sB + K * N;            // [K][N]
  float* sx = sC + K * N;            // [K][P]
  float* sdy = sx + K * P;           // [K][P]
  float* sseg = sdy + K * P;         // [K][P][N]  states after each step of the segment

  const i64 bh = blockIdx.x;
  const i64 bi = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
  const i64 PN = a.P * a.N, total = a.b * a.H * PN;
  const i64 ebase = bh * PN;
  const T* x = (const T*)a.x;
  const T* B = (const T*)a.B;
  const T* C = (const T*)a.C;
  const T* dy = (const T*)a.dy;
  T* dx = (T*)a.dx;
  const float acoef = a.per_state ? a.A[h * a.N + n] : a.A[h];

  float dS[MAXP];
#pragma unroll
  for (int p = 0; p < MAXP; ++p) dS[p] = (p < P && active && a.dsf) ? a.dsf[ebase + (i64)p * N + n] : 0.0f;
  float dAacc = 0.0f;

  for (i64 j = a.J - 1; j >= 0; --j) {
    const i64 t0 = j * a.K;
    const int kc = (int)((t0 + a.K < a.T) ? a.K : a.T - t0);  // steps in this segment
    __syncthreads();  // the previous segment is done with the staged rows
    // stage the segment's inputs (every load of the block in flight together)
    const int per = 1 + 2 * N + 2 * P;
    for (int idx = tid; idx < kc * per; idx += (int)blockDim.x) {
      const int k = idx / per, r = idx % per;
      const i64 t = t0 + k;
      if (r == 0) {
        sd[k] = a.delta[(bi * a.T + t) * a.H + h];
      } else if (r <= N) {
        sB[k * N + r - 1] = ld(B, ((bi * a.T + t) * a.G + g) * a.N + r - 1);
      } else if (r <= 2 * N) {
        sC[k * N + r - 1 - N] = ld(C, ((bi * a.T + t) * a.G + g) * a.N + r - 1 - N);
      } else if (r <= 2 * N + P) {
        sx[k * P + r - 1 - 2 * N] = ld(x, ((bi * a.T + t) * a.H + h) * a.P + r - 1 - 2 * N);
      } else {
        sdy[k * P + r - 1 - 2 * N - P] = ld(dy, ((bi * a.T + t) * a.H + h) * a.P + r - 1 - 2 * N - P);
      }
    }
    float ck0[MAXP];  // the checkpoint: the state before step t0
#pragma unroll
    for (int p = 0; p < MAXP; ++p) ck0[p] = (p < P && active) ? a.ck[j * total + ebase + (i64)p * N + n] : 0.0f;
    __syncthreads();
    // recompute the segment's states (own column only)
    if (active) {
#pragma unroll
      for (int p = 0; p < MAXP; ++p) {
        if (p >= P) continue;
        float s = ck0[p];
        for (int k = 0; k < kc; ++k) {
          s = scan_step(s, sd[k], acoef, sx[k * P + p], sB[k * N + n]);
          sseg[(k * P + p) * N + n] = s;
        }
      }
    }
    for (int k = kc - 1; k >= 0; --k) {
      const i64 t = t0 + k;
      const i64 bth = (bi * a.T + t) * a.H + h;
      const float d = sd[k];
      const float av = expf(__fmul_rn(d, acoef));
      const float Bn = sB[k * N + n];
      const float Cn = sC[k * N + n];
      float dbn = 0.0f, dcn = 0.0f, dd = 0.0f, dAs = 0.0f;
      __syncthreads();  // previous step's readers of red/colB/colC/ddw are done
      if (active) {
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {
          if (p >= P) continue;
          const float xp = sx[k * P + p];
          const float dyp = sdy[k * P + p];
          const float s_t = sseg[(k * P + p) * N + n];
          const float s_prev = k > 0 ? sseg[((k - 1) * P + p) * N + n] : ck0[p];
          dS[p] += dyp * Cn;                              // y_t = C_t . s_t
          dcn += dyp * s_t;                               // dC_t uses s_t
          dbn += dS[p] * xp;                              // dB_t (before the delta factor)
          dd += dS[p] * (xp * Bn + acoef * av * s_prev);  // input path + decay path
          dAs += dS[p] * s_prev;
          red[p * (N + 1) + n] = dS[p] * Bn;
        }
        dAacc += d * av * dAs;
        colB[n] = dbn;
        colC[n] = dcn;
      }
      dd = wave_sum(dd);
      if ((tid & 63) == 0) ddw[tid >> 6] = dd;
      __syncthreads();
      // dx row sums over n in order (as seq_bwd_kernel sums them), with the
      // LDS reads of eight terms in flight together
      for (int p = tid; p < P; p += (int)blockDim.x) {
        const float* rp = red + p * (N + 1);
        float acc = 0.0f;
        int nn = 0;
        for (; nn + 8 <= N; nn += 8) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = rp[nn + u];
#pragma unroll
          for (int u = 0; u < 8; ++u) acc += v[u];
        }
        for (; nn < N; ++nn) acc += rp[nn];
        st(dx, bth * a.P + p, d * acc);
      }
      if (tid < N) {
        a.dBh[bth * a.N + tid] = d * (0.0f + colB[tid]);
        a.dCh[bth * a.N + tid] = 0.0f + colC[tid];
      }
      if (tid == 0) {
        float s = 0.0f;
        for (int w = 0; w < nw; ++w) s += ddw[w];
        a.d_dt[bth] = s * a.sig[bth];
      }
#pragma unroll
      for (int p = 0; p < MAXP; ++p) dS[p] *= av;
    }
  }
#pragma unroll
  for (int p = 0; p < MAXP; ++p)
    if (p < P && active) a.d_s0[ebase + (i64)p * N + n] = dS[p];
  if (a.dA_part) {  // uniform: one column per state (per state) or a sum over all threads (per head)
    __syncthreads();  // the last step's readers of colB and ddw are done
    if (a.per_state) {
      if (tid < N) a.dA_part[bh * a.N + tid] = 0.0f + dAacc;
    } else {
      const float v = wave_sum(active ? dAacc : 0.0f);
      if ((tid & 63) == 0) ddw[tid >> 6] = v;
      __syncthreads();
      if (tid == 0) {
        float s = 0.0f;
        for (int w = 0; w < nw; ++w) s += ddw[w];
        a.dA_part[bh] = s;
      }
    }
  }
}

template <typename T>
__global__ void seq_group_sum_kernel(const float* __restrict__ dBh, const float* __restrict__ dCh, i64 bT, i64 H,
                                     i64 G, i64 N, T* __restrict__ dB, T* __restrict__ dC) {
  const i64 i = (i64)blockIdx.x * blockDim.x + threadIdx.x;  // over [b*T, G, N]
  if (i >= bT * G * N) return;
  const i64 n = i % N, g = (i / N) % G, bt = i / (N * G);
  const i64 hpg = H / G;
  float sb = 0.0f, sc = 0.0f;
  for (i64 h = g * hpg; h < (g + 1) * hpg; ++h) {
    sb += dBh[(bt * H + h) * N + n];
    sc += dCh[(bt * H + h) * N + n];
  }
  st(dB, i, sb);
  st(dC, i, sc);
}

__global__ void dA_reduce_kernel(const float* __restrict__ part, i64 R, i64 J, float* __restrict__ dA) {
  const i64 j = (i64)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= J) return;
  float s = 0.0f;
  for (i64 i = 0; i < R; ++i) s += part[i * J + j];
  dA[j] = s;
}

static inline i64 cdiv(i64 a, i64 b) { return (a + b - 1) / b; }

void launch_dA_reduce(const float* part, i64 R, i64 J, float* dA, hipStream_t stream) {
  if (J > 0) hipLaunchKernelGGL(dA_reduce_kernel, dim3((unsigned)cdiv(J, 256)), dim3(256), 0, stream, part, R, J, dA);
}

SeqPlan seq_plan(const ssmvjp_scan_desc& d) {
  SeqPlan p{};
  p.K = d.ckpt_every > 0 ? d.ckpt_every : 64;
  if (d.seqlen > 0 && p.K > d.seqlen) p.K = d.seqlen;
  if (p.K < 1) p.K = 1;
  p.J = cdiv(d.seqlen, p.K);
  p.PPT = (int)(d.headdim < 16 ? d.headdim : 16);
  p.NPG = (int)cdiv(d.headdim, p.PPT);
  const i64 bTH = d.batch * d.seqlen * d.nheads;
  const i64 state = d.batch * d.nheads * d.headdim * d.dstate;
  i64 off = 0;
  auto carve = [&](i64 floats) {
    const i64 o = off;
    off += cdiv(floats * 4, 256) * 256;
    return o;
  };
  p.off_delta = carve(bTH);
  p.off_sig = carve(bTH);
  p.off_ck = carve(p.J * state);
  p.off_seg = carve(d.batch * d.nheads * p.K * d.headdim * d.dstate);
  p.off_dBh = carve(bTH * d.dstate);
  p.off_dCh = carve(bTH * d.dstate);
  p.off_dA = carve(d.batch * d.nheads * d.dstate);
  p.bytes = (size_t)off;
  return p;
}

size_t seq_lds_bytes(const ssmvjp_scan_desc& d, const SeqPlan& plan) {
  const i64 nw = cdiv(d.dstate * plan.NPG, 64);
  return sizeof(float) * ((size_t)d.headdim * (d.dstate + 1) + 2 * (size_t)plan.NPG * d.dstate + nw);
}

// LDS of seq_bwd_lds_kernel: the reduction buffers plus one segment's inputs
// and states
static size_t seq_lds_small_bytes(const ssmvjp_scan_desc& d, const SeqPlan& plan) {
  const i64 nw = cdiv(d.dstate, 64);
  return sizeof(float) * ((size_t)d.headdim * (d.dstate + 1) + 2 * (size_t)d.dstate + nw +
                          (size_t)plan.K * (1 + 2 * d.dstate + 2 * d.headdim + d.headdim * d.dstate));
}

template <typename T>
static hipError_t launch_seq_t(const ssmvjp_scan_desc& d, const SeqPlan& plan, const SeqPointers& ptr,
                               hipStream_t stream) {
  char* ws = (char*)ptr.workspace;
  SeqArgs a;
  a.b = d.batch; a.T = d.seqlen; a.H = d.nheads; a.P = d.headdim; a.N = d.dstate; a.G = d.ngroups;
  a.K = plan.K; a.J = plan.J;
  a.per_state = d.decay == SSMVJP_DECAY_PER_STATE;
  a.x = ptr.x; a.dt = ptr.dt; a.A = ptr.A; a.B = ptr.B; a.C = ptr.C; a.s0 = ptr.s0; a.dy = ptr.dy;
  a.dsf = ptr.ds_final; a.dx = ptr.dx; a.d_dt = ptr.d_dt; a.dB = ptr.dB; a.dC = ptr.dC; a.d_s0 = ptr.d_s0;
  a.delta = (float*)(ws + plan.off_delta);
  a.sig = (float*)(ws + plan.off_sig);
  a.ck = (float*)(ws + plan.off_ck);
  a.seg = (float*)(ws + plan.off_seg);
  a.dBh = (float*)(ws + plan.off_dBh);
  a.dCh = (float*)(ws + plan.off_dCh);
  a.dA_part = ptr.dA ? (float*)(ws + plan.off_dA) : nullptr;

  const i64 bTH = a.b * a.T * a.H;
  if (bTH > 0) {
    hipLaunchKernelGGL(seq_prologue_kernel, dim3((unsigned)cdiv(bTH, 256)), dim3(256), 0, stream, a.dt, bTH,
                       a.delta, a.sig);
    const i64 total = a.b * a.H * a.P * a.N;
    hipLaunchKernelGGL(seq_ckpt_kernel<T>, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, stream, a);
  }
  if (a.b * a.H > 0) {
    const int NT = (int)cdiv(a.N * plan.NPG, 64) * 64;
    const size_t small = seq_lds_small_bytes(d, plan);
    if (plan.NPG == 1 && small <= 64 * 1024) {  // one thread holds a whole column: the LDS-staged walk
      if (a.P <= 4)
        hipLaunchKernelGGL((seq_bwd_lds_kernel<T, 4>), dim3((unsigned)(a.b * a.H)), dim3(NT), small, stream, a);
      else
        hipLaunchKernelGGL((seq_bwd_lds_kernel<T, 16>), dim3((unsigned)(a.b * a.H)), dim3(NT), small, stream, a);
    } else {
      hipLaunchKernelGGL((seq_bwd_kernel<T, 16>), dim3((unsigned)(a.b * a.H)), dim3(NT), seq_lds_bytes(d, plan),
                         stream, a, plan.PPT, plan.NPG);
    }
  }
  if (bTH > 0) {
    const i64 n = a.b * a.T * a.G * a.N;
    hipLaunchKernelGGL(seq_group_sum_kernel<T>, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, stream, a.dBh, a.dCh,
                       a.b * a.T, a.H, a.G, a.N, (T*)a.dB, (T*)a.dC);
  }
  if (ptr.dA) launch_dA_reduce(a.dA_part, a.b, a.per_state ? a.H * a.N : a.H, ptr.dA, stream);
  return hipGetLastError();
}


hipError_t launch_seq_bwd(const ssmvjp_scan_desc& d, const SeqPlan& plan, const SeqPointers& ptr,
                          hipStream_t stream) {
  if (d.dtype == SSMVJP_BF16) return launch_seq_t<bf16>(d, plan, ptr, stream);
  return launch_seq_t<float>(d, plan, ptr, stream);
}

}  // namespace ssmvjp
