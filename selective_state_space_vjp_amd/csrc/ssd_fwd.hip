// ssd_fwd.hip -- chunked SSD forward of the selective scan (Mamba-2 and the
// Mamba-3 MIMO rank-M form): the output y and the final state, in one pass.
//
// The method (burn-mamba's chunked forward, kernels K1..K5): inside a chunk the
// cumulative decay cumA (K1), the scores C.B^T (K2) and the chunk's own state
// contribution (K3); the states passed from chunk to chunk (K4); the output as
// an inter-chunk term exp(cumA_r) C_r.S_c (BLUE) plus the causal intra-chunk
// term sum_s (C_r.B_s) exp(cumA_r - cumA_s) v_s (ORANGE) (K5).
//
// MI355X organisation: one workgroup of 8 waves per (batch, head, block of PB
// p columns) walks the chunks in order and keeps its [N x PB] slice of the
// running state in registers, so no state ever goes to HBM; only x, dt, B, C
// are read and y written.  Per chunk:
//   stage     B, C rows and the two scaled copies of x into LDS (loaded into
//             registers two chunks ahead);
//   phase 1   the causal 16x16 tiles of (C.B^T)^T on MFMA with the decay mask
//             applied -> LDS; the old state (as the operand type) -> LDS; the
//             state update S <- exp(end) S + sum_r exp(end - cumA_r) v_r (x) B_r
//             on MFMA into the registers;
//   phase 2   y^T tiles = ORANGE + exp(cumA_r) BLUE on MFMA, stored as rows of y.
// The state is held transposed ([n][p] tiles), whose MFMA output layout is
// directly the operand layout BLUE needs (contraction over n).
//
// The chunk length is the kernel's own: chunk_len steps when chunk_len * M <= 64,
// else 64 / M steps.  y and the final state do not depend on it (the chunked
// form equals the sequential recurrence for every chunk length) apart from
// rounding.
#include "ssd_common.cuh"

namespace ssmvjp {

namespace {

constexpr int FW_NW = 8;  // waves per workgroup
constexpr int FW_NTH = 64 * FW_NW;

struct FwdArgs {
  i64 T, H, P, N, G, M;
  int Lf;      // steps per chunk (Lf * M <= 64)
  int nc;      // chunks
  int npb;     // p blocks per head
  int raw;     // 1: (v, da) inputs; 0: Mamba-2 (x, dt, A)
  int causal;  // 1: no step straddles a 16-row tile (M divides 16): only tiles with s_t <= r_t are non-zero
  int xcd;     // 1: workgroup ids are remapped so that each XCD walks a contiguous range of (batch, head)
  const void* xv;
  const float* dtda;
  const float* A;
  const void* B;
  const void* C;
  const float* s0;
  void* y;
  float* s_final;
};

// (s_t, r_t) row-tile pairs of the 64x64 score block: the 10 causal pairs
// first, then the 6 above the diagonal (only non-zero when M does not divide 16).
// Two bits per pair packed into immediates, so that the lookup of a
// wave-uniform pair index is scalar arithmetic, not a memory load.
constexpr unsigned pack2(const unsigned char (&v)[16]) {
  unsigned m = 0;
  for (int i = 0; i < 16; ++i) m |= (unsigned)v[i] << (2 * i);
  return m;
}
constexpr unsigned char PAIR_S[16] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3, 1, 2, 3, 2, 3, 3};
constexpr unsigned char PAIR_R[16] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3, 0, 0, 0, 1, 1, 2};
constexpr unsigned PAIR_S_BITS = pack2(PAIR_S), PAIR_R_BITS = pack2(PAIR_R);
__device__ __forceinline__ int pair_s(int i) { return (int)((PAIR_S_BITS >> (2 * i)) & 3u); }
__device__ __forceinline__ int pair_r(int i) { return (int)((PAIR_R_BITS >> (2 * i)) & 3u); }

// two 16-wide contraction blocks: two 16x16x16 bf16 MFMAs, or eight 16x16x4
// f32 MFMAs.  (The gfx950 16x16x32 bf16 MFMA would take both blocks in one
// instruction; with it this kernel gave timing-dependent wrong results where
// the compiler let an LDS load overwrite a source register of an in-flight
// 16x16x32 MFMA, so it is not used.)
template <typename T>
__device__ __forceinline__ void mma2(f32x4& d, const Frag<T>& a0, const Frag<T>& a1, const Frag<T>& b0,
                                     const Frag<T>& b1) {
  mma(d, a0, b0);
  mma(d, a1, b1);
}

template <typename T>
__device__ __forceinline__ void store_frag(T* p, const f32x4& v) {
  store4(p, v);
}

// step sizes of one chunk, one lane per step (lanes past the chunk's valid
// steps get delta = 0 and da = 0, which keeps cumA flat)
struct FwdScalars {
  float delta, cum, end;
};
__device__ __forceinline__ FwdScalars fwd_scalars(int raw, float z, bool valid, float Ah, int lane) {
  FwdScalars s;
  float da;
  if (raw) {
    s.delta = 1.0f;
    da = valid ? z : 0.0f;
  } else {
    s.delta = valid ? softplus_f(z) : 0.0f;
    da = s.delta * Ah;
  }
  s.cum = wave_incl_scan(da, lane);
  s.end = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s.cum), 63));
  return s;
}

__device__ __forceinline__ float shfl_f(float v, int src) { return __shfl(v, src, 64); }

// the same with the hardware softplus (the bf16 walk computes these in every
// wave for every chunk)
__device__ __forceinline__ FwdScalars fwd_scalars_hw(int raw, float z, bool valid, float Ah, int lane) {
  FwdScalars s;
  float da;
  if (raw) {
    s.delta = 1.0f;
    da = valid ? z : 0.0f;
  } else {
    s.delta = valid ? softplus_hw(z) : 0.0f;
    da = s.delta * Ah;
  }
  s.cum = wave_incl_scan(da, lane);
  s.end = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s.cum), 63));
  return s;
}

template <typename T, int NT, int PTB>
__global__ void __launch_bounds__(FW_NTH) ssd_fwd_kernel(FwdArgs a) {
  constexpr int E16 = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int PAD = 32 / sizeof(T);  // row padding of the staged tiles (32 bytes)
  constexpr int N = 16 * NT, PB = 16 * PTB;
  constexpr int PPB = N + PAD, PPX = PB + PAD;  // row pitches (elements)
  constexpr int BUF = 2 * 64 * PPB + 2 * 64 * PPX;
  constexpr int NBUF = sizeof(T) == 2 ? 2 : 1;  // input buffers in LDS
  constexpr int NST = NT * PTB, MAXST = (NST + FW_NW - 1) / FW_NW;   // state tiles (per wave)
  constexpr int NOUT = 4 * PTB, MAXO = (NOUT + FW_NW - 1) / FW_NW;  // output tiles (per wave)
  constexpr int CB_ROW = N / E16, X_ROW = PB / E16;                 // 16-byte chunks per staged row
  constexpr int MAXCB = (64 * CB_ROW + FW_NTH - 1) / FW_NTH;
  constexpr int MAXCX = (64 * X_ROW + FW_NTH - 1) / FW_NTH;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* const buf0 = (T*)smem_raw;
  T* const Gs = buf0 + NBUF * BUF;  // 16 slots of 256: masked, decayed (C.B^T)^T tiles, native order
  T* const Ss = Gs + 16 * 256;      // NST slots of 256: the chunk-input state tiles, native order

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, q = lane >> 4,
            c16 = lane & 15;
  i64 id = blockIdx.x;
  if (a.xcd) id = (id % 8) * (gridDim.x / 8) + id / 8;
  const int pb = (int)(id % a.npb);
  id /= a.npb;
  const i64 h = id % a.H, bi = id / a.H, g = h / (a.H / a.G);
  const int p0 = pb * PB;
  const int M = (int)a.M, Lf = a.Lf, nc = a.nc;
  const int T32 = (int)a.T, H32 = (int)a.H;
  const int rs_x = (int)(a.H * a.P), rs_bc = (int)(a.G * a.N);  // fused-row strides of x/y and B/C
  const unsigned esz = sizeof(T);
  const float Ah = a.raw ? 0.0f : a.A[h];

  // running state, transposed: tile k of this wave is (n_t, p_t) = (kk / PTB, kk % PTB), kk = w + 8k;
  // lane holds S[p = p0 + 16 p_t + c16][n = 16 n_t + 4q + j]
  f32x4 S[MAXST];
  const i64 sbase = (bi * a.H + h) * a.P * a.N;
#pragma unroll
  for (int k = 0; k < MAXST; ++k) {
    const int kk = w + FW_NW * k;
    S[k] = zero4();
    if (kk < NST && a.s0) {
      const int nt = kk / PTB, pt = kk % PTB;
#pragma unroll
      for (int j = 0; j < 4; ++j) S[k][j] = a.s0[sbase + (i64)(p0 + 16 * pt + c16) * N + 16 * nt + 4 * q + j];
    }
  }

  const T* x_b = (const T*)a.xv + ((bi * a.T) * a.M * a.H + h) * a.P + p0;
  const T* B_b = (const T*)a.B + ((bi * a.T) * a.M * a.G + g) * a.N;
  const T* C_b = (const T*)a.C + ((bi * a.T) * a.M * a.G + g) * a.N;
  T* y_b = (T*)a.y + ((bi * a.T) * a.M * a.H + h) * a.P + p0;
  const float* dt_b = a.dtda + bi * a.T * a.H + h;

  struct Pre {
    float z;
    u32x4 b[MAXCB], c[MAXCB], x[MAXCX];
  };
  auto issue = [&](Pre& pr, int ch) {
    const int t0 = ch * Lf;
    const int Lc = T32 - t0 < Lf ? T32 - t0 : Lf;
    const int rows = Lc * M;
    pr.z = bload_f32(make_rsrc(dt_b + (i64)t0 * H32, (unsigned)(((Lc - 1) * H32 + 1) * 4)),
                     lane < Lc ? (unsigned)(lane * H32 * 4) : BUF_OOB);
    const i64 R0 = (i64)t0 * M;
    const brsrc rb = make_rsrc(B_b + R0 * rs_bc, (unsigned)(((rows - 1) * rs_bc + N) * esz));
    const brsrc rc = make_rsrc(C_b + R0 * rs_bc, (unsigned)(((rows - 1) * rs_bc + N) * esz));
    const brsrc rx = make_rsrc(x_b + R0 * rs_x, (unsigned)(((rows - 1) * rs_x + PB) * esz));
#pragma unroll
    for (int it = 0; it < MAXCB; ++it) {
      const int idx = tid + it * FW_NTH;
      const unsigned off =
          idx < 64 * CB_ROW ? (unsigned)(((idx / CB_ROW) * rs_bc + (idx % CB_ROW) * E16) * esz) : BUF_OOB;
      pr.b[it] = bload16(rb, off);
      pr.c[it] = bload16(rc, off);
    }
#pragma unroll
    for (int it = 0; it < MAXCX; ++it) {
      const int idx = tid + it * FW_NTH;
      const unsigned off =
          idx < 64 * X_ROW ? (unsigned)(((idx / X_ROW) * rs_x + (idx % X_ROW) * E16) * esz) : BUF_OOB;
      pr.x[it] = bload16(rx, off);
    }
  };

  auto process = [&](Pre& pr, int ch, T* sb) {
    const int t0 = ch * Lf;
    const int Lc = T32 - t0 < Lf ? T32 - t0 : Lf;
    const int rows = Lc * M;
    const FwdScalars sc = fwd_scalars(a.raw, pr.z, lane < Lc, Ah, lane);
    T* const Bs = sb;
    T* const Cs = Bs + 64 * PPB;
    T* const Xd = Cs + 64 * PPB;
    T* const Xw = Xd + 64 * PPX;
    if (NBUF == 1 && ch > 0) __syncthreads();  // the previous chunk's reads of the single buffer are done
    // stage: B and C rows as loaded; x scaled by delta (ORANGE) and by
    // delta * exp(end - cumA) (state update)
#pragma unroll
    for (int it = 0; it < MAXCB; ++it) {
      const int idx = tid + it * FW_NTH;
      if (idx < 64 * CB_ROW) {
        const int o = (idx / CB_ROW) * PPB + (idx % CB_ROW) * E16;
        *(u32x4*)(Bs + o) = pr.b[it];
        *(u32x4*)(Cs + o) = pr.c[it];
      }
    }
#pragma unroll
    for (int it = 0; it < MAXCX; ++it) {
      const int idx = tid + it * FW_NTH;
      const int r = (idx / X_ROW) & 63, l = r / M;
      const float d = shfl_f(sc.delta, l);
      const float e = exp_hw(sc.end - shfl_f(sc.cum, l));
      if (idx < 64 * X_ROW) {
        const int o = r * PPX + (idx % X_ROW) * E16;
        *(u32x4*)(Xd + o) = scale16(pr.x[it], d, (const T*)0);
        *(u32x4*)(Xw + o) = scale16(pr.x[it], d * e, (const T*)0);
      }
    }
    issue(pr, ch + 2 < nc ? ch + 2 : nc - 1);
    __syncthreads();

    // phase 1a: masked, decayed score tiles G^T[s][r] = (C_r . B_s) exp(cumA_r - cumA_s), step(s) <= step(r)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = w + FW_NW * k;
      if (i >= 10 && a.causal) continue;
      const int st = pair_s(i), rt = pair_r(i);
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb + 1 < NT; kb += 2)
        mma2(acc, ld_colk(Bs, PPB, 16 * st, 16 * kb, lane), ld_colk(Bs, PPB, 16 * st, 16 * kb + 16, lane),
             ld_colk(Cs, PPB, 16 * rt, 16 * kb, lane), ld_colk(Cs, PPB, 16 * rt, 16 * kb + 16, lane));
      if (NT & 1)
        mma(acc, ld_colk(Bs, PPB, 16 * st, 16 * (NT - 1), lane), ld_colk(Cs, PPB, 16 * rt, 16 * (NT - 1), lane));
      const int lr = (16 * rt + c16) / M;
      const float cr = shfl_f(sc.cum, lr);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ls = (16 * st + 4 * q + j) / M;
        const float cs = shfl_f(sc.cum, ls);
        acc[j] = ls <= lr ? acc[j] * exp_hw(cr - cs) : 0.0f;
      }
      store_frag(Gs + (st * 4 + rt) * 256 + lane * 4, acc);
    }
    // phase 1b: the chunk-input state to LDS, then the state update on MFMA
    const float e_end = exp_hw(sc.end);
#pragma unroll
    for (int k = 0; k < MAXST; ++k) {
      const int kk = w + FW_NW * k;
      if (kk >= NST) continue;
      const int nt = kk / PTB, pt = kk % PTB;
      store_frag(Ss + kk * 256 + lane * 4, S[k]);
      f32x4 acc;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = e_end * S[k][j];
#pragma unroll
      for (int kb = 0; kb < 4; kb += 2)
        mma2(acc, ld_rowk(Bs, PPB, 16 * kb, 16 * nt, lane), ld_rowk(Bs, PPB, 16 * kb + 16, 16 * nt, lane),
             ld_rowk(Xw, PPX, 16 * kb, 16 * pt, lane), ld_rowk(Xw, PPX, 16 * kb + 16, 16 * pt, lane));
      S[k] = acc;
    }
    __syncthreads();

    // phase 2: y^T[p][r] = sum_s xd[s][p] G^T[s][r] + exp(cumA_r) sum_n S[p][n] C[r][n]
    const brsrc ry = make_rsrc(y_b + (i64)t0 * M * rs_x, (unsigned)(((rows - 1) * rs_x + PB) * esz));
#pragma unroll
    for (int o = 0; o < MAXO; ++o) {
      const int oo = w + FW_NW * o;
      if (oo >= NOUT) continue;
      const int pt = oo % PTB, rt = oo / PTB;
      f32x4 ao = zero4(), ab = zero4();
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (st > rt && a.causal) continue;
        mma(ao, ld_rowk(Xd, PPX, 16 * st, 16 * pt, lane), ld_ntv(Gs + (st * 4 + rt) * 256, lane));
      }
#pragma unroll
      for (int nt = 0; nt + 1 < NT; nt += 2)
        mma2(ab, ld_ntv(Ss + (nt * PTB + pt) * 256, lane), ld_ntv(Ss + ((nt + 1) * PTB + pt) * 256, lane),
             ld_colk(Cs, PPB, 16 * rt, 16 * nt, lane), ld_colk(Cs, PPB, 16 * rt, 16 * nt + 16, lane));
      if (NT & 1)
        mma(ab, ld_ntv(Ss + ((NT - 1) * PTB + pt) * 256, lane), ld_colk(Cs, PPB, 16 * rt, 16 * (NT - 1), lane));
      const int r = 16 * rt + c16;
      const float er = exp_hw(shfl_f(sc.cum, r / M));
      f32x4 yv;
#pragma unroll
      for (int j = 0; j < 4; ++j) yv[j] = ao[j] + er * ab[j];
      bstore4(ry, r < rows ? (unsigned)((r * rs_x + 16 * pt + 4 * q) * esz) : BUF_OOB, yv, (const T*)0);
    }
  };

  if (nc > 0) {
    T* const buf1 = buf0 + (NBUF - 1) * BUF;
    Pre pa, pb2;
    issue(pa, 0);
    issue(pb2, nc > 1 ? 1 : 0);
    int ch = 0;
    for (; ch + 1 < nc; ch += 2) {
      process(pa, ch, buf0);
      process(pb2, ch + 1, buf1);
    }
    if (ch < nc) process(pa, ch, buf0);
  }

  if (a.s_final) {
#pragma unroll
    for (int k = 0; k < MAXST; ++k) {
      const int kk = w + FW_NW * k;
      if (kk >= NST) continue;
      const int nt = kk / PTB, pt = kk % PTB;
#pragma unroll
      for (int j = 0; j < 4; ++j) a.s_final[sbase + (i64)(p0 + 16 * pt + c16) * N + 16 * nt + 4 * q + j] = S[k][j];
    }
  }
}

// ===========================================================================
// bfloat16: the scores C.B^T of every chunk precomputed by a parallel kernel,
// and a walk with one barrier per chunk
// ===========================================================================

// row pitches (elements) of the staged bf16 tiles.  With 32 banks of 4 bytes
// and 16 lanes per 8-byte read: tiles read along their rows (fragments with
// the contraction index in the row) want rows 2 dwords apart modulo the banks;
// tiles read down their rows (transposed reads of 4 consecutive rows by each
// 16 lanes) want rows 8 or 24 dwords apart.
__host__ __device__ constexpr int pitch_along(int n) { return n + 4; }
__host__ __device__ constexpr int pitch_down(int n) { return n + ((16 - n) & 31); }

// 8-byte LDS stores of a 16-byte chunk (pitch_along rows are 8-byte aligned only)
__device__ __forceinline__ void lds_store16_as8(bf16* p, const u32x4& u) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  u32x2 lo = {u[0], u[1]}, hi = {u[2], u[3]};
  *(u32x2*)p = lo;
  *(u32x2*)(p + 4) = hi;
}

constexpr int CB_NW = 4;

// kernel F1: the scores of one (batch, chunk, group): the 16x16 tiles
// (s_t, r_t) of (C.B^T)^T[s][r] = B_s . C_r that the causal mask leaves
// non-zero, stored as float in MFMA output order,
// cbt[((bi * nc + c) * G + g) * 16 + 4 s_t + r_t][lane][4]
template <int NT>
__global__ void __launch_bounds__(64 * CB_NW) ssd_fwd_scores_kernel(FwdArgs a, float* __restrict__ cbt) {
  constexpr int N = 16 * NT, PP = pitch_along(N), CROW = N / 8;
  constexpr int MAXC = (64 * CROW + 64 * CB_NW - 1) / (64 * CB_NW);
  __shared__ __align__(16) bf16 Bs[64 * PP], Cs[64 * PP];
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const i64 id = blockIdx.x;
  const i64 g = id % a.G, c = (id / a.G) % a.nc, bi = id / (a.G * a.nc);
  const int t0 = (int)c * a.Lf;
  const int Lc = (int)a.T - t0 < a.Lf ? (int)a.T - t0 : a.Lf;
  const int rows = Lc * (int)a.M, rs_bc = (int)(a.G * a.N);
  const i64 base = ((bi * a.T + t0) * a.M * a.G + g) * a.N;
  const brsrc rb = make_rsrc((const bf16*)a.B + base, (unsigned)(((rows - 1) * rs_bc + N) * 2));
  const brsrc rc = make_rsrc((const bf16*)a.C + base, (unsigned)(((rows - 1) * rs_bc + N) * 2));
#pragma unroll
  for (int it = 0; it < MAXC; ++it) {
    const int idx = tid + it * 64 * CB_NW;
    const int r = idx / CROW, col = (idx % CROW) * 8;
    const unsigned off = idx < 64 * CROW ? (unsigned)((r * rs_bc + col) * 2) : BUF_OOB;
    const u32x4 vb = bload16(rb, off), vc = bload16(rc, off);
    if (idx < 64 * CROW) {
      lds_store16_as8(Bs + r * PP + col, vb);
      lds_store16_as8(Cs + r * PP + col, vc);
    }
  }
  __syncthreads();
  float* out = cbt + id * 16 * 256;
#pragma unroll
  for (int k = 0; k < 16 / CB_NW; ++k) {
    const int i = w + CB_NW * k;
    if (i >= 10 && a.causal) continue;
    const int st = pair_s(i), rt = pair_r(i);
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < NT; ++kb)
      mma(acc, ld_colk(Bs, PP, 16 * st, 16 * kb, lane), ld_colk(Cs, PP, 16 * rt, 16 * kb, lane));
    store4(out + ((st * 4 + rt) * 64 + lane) * 4, acc);
  }
}

// kernel F2: the walk over the chunks of one (batch, head, p block), software
// pipelined so that each chunk costs one barrier, with two wave roles that
// share each SIMD: waves 0-3 produce the outputs (one 16-row block of y each,
// all p columns of the block), waves 4-7 hold the running state and update it.
// Interval c (c = 0 .. nc):
//   stage    (all waves) B, x (scaled for the state update) of chunk c+1 and
//            C, x and the per-row cumA and delta of chunk c into their LDS
//            buffers (parity of the chunk), from registers loaded one interval
//            ahead; wave 0 also stages dt of chunk c+2;
//   phase 1  (state waves) chunk c: the state as the operand type -> LDS, then
//            the state update on MFMA;
//   phase 2  (output waves) chunk c-1: the decay mask applied to its score
//            tiles (registers), ORANGE and BLUE on MFMA, y stored;
//   barrier.
// Everything an interval reads was written before the previous barrier, and
// every buffer it writes was last read before it.
template <int NT, int PTB>
__global__ void __launch_bounds__(FW_NTH) ssd_fwd_walk_kernel(FwdArgs a, const float* __restrict__ cbt) {
  typedef bf16 T;
  constexpr int N = 16 * NT, PB = 16 * PTB;
  constexpr int PPB = pitch_down(N), PPC = pitch_along(N), PPX = pitch_down(PB);
  constexpr int SB = 64 * PPB, SC = 64 * PPC, SX = 64 * PPX;
  constexpr int NST = NT * PTB;
  constexpr int NTW = (NT + 3) / 4;  // n tiles per state wave (all PTB p tiles of each)
  constexpr int CROW_B = N / 8, CROW_X = PB / 8;
  constexpr int MAXCB = (64 * CROW_B + FW_NTH - 1) / FW_NTH, MAXCX = (64 * CROW_X + FW_NTH - 1) / FW_NTH;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* const Bs = (T*)smem_raw;  // [2][SB]
  T* const Cs = Bs + 2 * SB;   // [2][SC]
  T* const Xw = Cs + 2 * SC;   // [2][SX]
  T* const Xd = Xw + 2 * SX;   // [2][SX]
  T* const Ss = Xd + 2 * SX;   // [2][NST * 256]
  float* const crow = (float*)(Ss + 2 * NST * 256);  // [2][64] cumA per fused row
  float* const drow = crow + 2 * 64;                 // [2][64] delta per fused row
  float* const zrow = drow + 2 * 64;                 // [2][64] dt (or da) per step

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, q = lane >> 4,
            c16 = lane & 15;
  i64 id = blockIdx.x;
  if (a.xcd) id = (id % 8) * (gridDim.x / 8) + id / 8;
  const int pb = (int)(id % a.npb);
  id /= a.npb;
  const i64 h = id % a.H, bi = id / a.H, g = h / (a.H / a.G);
  const int p0 = pb * PB;
  const int M = (int)a.M, Lf = a.Lf, nc = a.nc;
  const int T32 = (int)a.T, H32 = (int)a.H;
  const int rs_x = (int)(a.H * a.P), rs_bc = (int)(a.G * a.N);
  const float Ah = a.raw ? 0.0f : a.A[h];

  // roles: output wave rt = w (w < 4); state wave sw = w - 4 holding the
  // tiles (n_t, p_t) with n_t = NTW * sw + i (i < NTW, n_t < NT), all p_t
  const bool out_wave = w < 4;
  const int ort = w, sw = w - 4, nt0 = NTW * sw;
  f32x4 S[NTW][PTB];
  const i64 sbase = (bi * a.H + h) * a.P * a.N;
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int pt = 0; pt < PTB; ++pt) {
      S[i][pt] = zero4();
      if (!out_wave && nt0 + i < NT && a.s0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          S[i][pt][j] = a.s0[sbase + (i64)(p0 + 16 * pt + c16) * N + 16 * (nt0 + i) + 4 * q + j];
      }
    }

  const T* x_b = (const T*)a.xv + ((bi * a.T) * a.M * a.H + h) * a.P + p0;
  const T* B_b = (const T*)a.B + ((bi * a.T) * a.M * a.G + g) * a.N;
  const T* C_b = (const T*)a.C + ((bi * a.T) * a.M * a.G + g) * a.N;
  T* y_b = (T*)a.y + ((bi * a.T) * a.M * a.H + h) * a.P + p0;
  const float* dt_b = a.dtda + bi * a.T * a.H + h;
  const float* cb_b = cbt + (bi * a.nc * a.G + g) * 16 * 256;  // chunk c at + c * G * 16 * 256

  // loop-invariant row -> step maps: the last fused row of this lane's output
  // row's step (the causal mask is s <= last), the step of each staged x row
  // and of this lane's row (lane = fused row)
  const int last_r = ((16 * ort + c16) / M) * M + M - 1;
  int lx[MAXCX];
#pragma unroll
  for (int it = 0; it < MAXCX; ++it) lx[it] = (((tid + it * FW_NTH) / CROW_X) & 63) / M;
  const int lrow = lane / M;

  auto steps_of = [&](int ch) {
    const int t0 = ch * Lf;
    return T32 - t0 < Lf ? T32 - t0 : Lf;
  };
  struct Set {
    float z;
    u32x4 b[MAXCB], c[MAXCB], x[MAXCX];
    f32x4 cb[4];
  };
  auto clampc = [&](int ch) { return ch < 0 ? 0 : (ch >= nc ? nc - 1 : ch); };
  auto load_dt = [&](int ch) {
    const int t0 = ch * Lf, Lc = steps_of(ch);
    return bload_f32(make_rsrc(dt_b + (i64)t0 * H32, (unsigned)(((Lc - 1) * H32 + 1) * 4)),
                     lane < Lc ? (unsigned)(lane * H32 * 4) : BUF_OOB);
  };
  // loads for one interval: B and x of chunk cb_ (the state update), dt of
  // chunk cb_ + 1 (wave 0), C of chunk cc, scores of chunk cs (output waves)
  auto issue = [&](Set& s, int cb_, int cc, int cs) {
    const int cz = clampc(cb_ + 1);
    cb_ = clampc(cb_);
    cc = clampc(cc);
    cs = clampc(cs);
    if (w == 0) s.z = load_dt(cz);
    {
      const int rows = steps_of(cb_) * M;
      const i64 R0 = (i64)cb_ * Lf * M;
      const brsrc rb = make_rsrc(B_b + R0 * rs_bc, (unsigned)(((rows - 1) * rs_bc + N) * 2));
      const brsrc rx = make_rsrc(x_b + R0 * rs_x, (unsigned)(((rows - 1) * rs_x + PB) * 2));
#pragma unroll
      for (int it = 0; it < MAXCB; ++it) {
        const int idx = tid + it * FW_NTH;
        s.b[it] = bload16(rb, idx < 64 * CROW_B
                                  ? (unsigned)(((idx / CROW_B) * rs_bc + (idx % CROW_B) * 8) * 2) : BUF_OOB);
      }
#pragma unroll
      for (int it = 0; it < MAXCX; ++it) {
        const int idx = tid + it * FW_NTH;
        s.x[it] = bload16(rx, idx < 64 * CROW_X
                                  ? (unsigned)(((idx / CROW_X) * rs_x + (idx % CROW_X) * 8) * 2) : BUF_OOB);
      }
    }
    {
      const int rows = steps_of(cc) * M;
      const brsrc rc = make_rsrc(C_b + (i64)cc * Lf * M * rs_bc, (unsigned)(((rows - 1) * rs_bc + N) * 2));
#pragma unroll
      for (int it = 0; it < MAXCB; ++it) {
        const int idx = tid + it * FW_NTH;
        s.c[it] = bload16(rc, idx < 64 * CROW_B
                                  ? (unsigned)(((idx / CROW_B) * rs_bc + (idx % CROW_B) * 8) * 2) : BUF_OOB);
      }
    }
    if (out_wave) {
      const brsrc rs = make_rsrc(cb_b + (i64)cs * a.G * 16 * 256, 16 * 256 * 4);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bool live = st <= ort || !a.causal;
        const u32x4 u = bload16(rs, live ? (unsigned)(((st * 4 + ort) * 64 + lane) * 16) : BUF_OOB);
        s.cb[st] = __builtin_bit_cast(f32x4, u);
      }
    }
  };

  // step scalars of chunk ch from the dt staged in zrow slot `slot` (lane = step)
  auto scalars_of = [&](int slot, int ch) {
    return fwd_scalars_hw(a.raw, zrow[slot * 64 + lane], lane < steps_of(ch), Ah, lane);
  };
  // B and x of chunk ch (scalars sc) -> the state-update buffers of its parity
  auto stage_state = [&](const Set& s, const FwdScalars& sc, int ch) {
    T* const bs = Bs + (ch & 1) * SB;
    T* const xw = Xw + (ch & 1) * SX;
#pragma unroll
    for (int it = 0; it < MAXCB; ++it) {
      const int idx = tid + it * FW_NTH;
      if (idx < 64 * CROW_B) *(u32x4*)(bs + (idx / CROW_B) * PPB + (idx % CROW_B) * 8) = s.b[it];
    }
#pragma unroll
    for (int it = 0; it < MAXCX; ++it) {
      const int idx = tid + it * FW_NTH;
      const float f = shfl_f(sc.delta, lx[it]) * exp_hw(sc.end - shfl_f(sc.cum, lx[it]));
      if (idx < 64 * CROW_X)
        *(u32x4*)(xw + (idx / CROW_X) * PPX + (idx % CROW_X) * 8) = scale16(s.x[it], f, (const T*)0);
    }
  };
  // C, x and the per-row cumA and delta of chunk ch -> the output buffers of its parity
  auto stage_out = [&](const Set& s, const Set& sx, const FwdScalars& sc, int ch) {
    T* const cs = Cs + (ch & 1) * SC;
    T* const xd = Xd + (ch & 1) * SX;
#pragma unroll
    for (int it = 0; it < MAXCB; ++it) {
      const int idx = tid + it * FW_NTH;
      if (idx < 64 * CROW_B) lds_store16_as8(cs + (idx / CROW_B) * PPC + (idx % CROW_B) * 8, s.c[it]);
    }
#pragma unroll
    for (int it = 0; it < MAXCX; ++it) {
      const int idx = tid + it * FW_NTH;
      if (idx < 64 * CROW_X) *(u32x4*)(xd + (idx / CROW_X) * PPX + (idx % CROW_X) * 8) = sx.x[it];
    }
    const float cr = shfl_f(sc.cum, lrow), dr = shfl_f(sc.delta, lrow);
    if (w == 0) {
      crow[(ch & 1) * 64 + lane] = cr;
      drow[(ch & 1) * 64 + lane] = dr;
    }
  };
  // all of a wave's LDS fragments are read before its first MFMA waits on them
  auto phase1 = [&](const FwdScalars& sc, int ch) {
    if (out_wave) return;
    const T* bs = Bs + (ch & 1) * SB;
    const T* xw = Xw + (ch & 1) * SX;
    T* const ss = Ss + (ch & 1) * NST * 256;
    const float e_end = exp_hw(sc.end);
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int pt = 0; pt < PTB; ++pt)
        if (nt0 + i < NT) store4(ss + ((nt0 + i) * PTB + pt) * 256 + lane * 4, S[i][pt]);
    Frag<T> fb[NTW][4], fx[PTB][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int i = 0; i < NTW; ++i) fb[i][kb] = ld_rowk(bs, PPB, 16 * kb, 16 * (nt0 + i < NT ? nt0 + i : 0), lane);
#pragma unroll
      for (int pt = 0; pt < PTB; ++pt) fx[pt][kb] = ld_rowk(xw, PPX, 16 * kb, 16 * pt, lane);
    }
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int pt = 0; pt < PTB; ++pt) {
        if (nt0 + i >= NT) continue;
        f32x4 acc;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = e_end * S[i][pt][j];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(acc, fb[i][kb], fx[pt][kb]);
        S[i][pt] = acc;
      }
  };
  auto phase2 = [&](const Set& s, int ch) {
    if (!out_wave) return;
    const T* xd = Xd + (ch & 1) * SX;
    const T* cs = Cs + (ch & 1) * SC;
    const T* ss = Ss + (ch & 1) * NST * 256;
    const float* cr_ = crow + (ch & 1) * 64;
    const float* dr_ = drow + (ch & 1) * 64;
    const int r = 16 * ort + c16;
    const float cr = cr_[r];
    f32x4 ao[PTB], ab[PTB];
#pragma unroll
    for (int pt = 0; pt < PTB; ++pt) ao[pt] = ab[pt] = zero4();
    // ORANGE: G^T[s][r] = (B_s . C_r) delta_s exp(cumA_r - cumA_s) for s <= the last row of r's step
    float4 cs4[4], ds4[4];
    Frag<T> xf[4][PTB];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (st > ort && a.causal) continue;
      cs4[st] = *(const float4*)(cr_ + 16 * st + 4 * q);
      ds4[st] = *(const float4*)(dr_ + 16 * st + 4 * q);
#pragma unroll
      for (int pt = 0; pt < PTB; ++pt) xf[st][pt] = ld_rowk(xd, PPX, 16 * st, 16 * pt, lane);
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (st > ort && a.causal) continue;
      const float csj[4] = {cs4[st].x, cs4[st].y, cs4[st].z, cs4[st].w};
      const float dsj[4] = {ds4[st].x, ds4[st].y, ds4[st].z, ds4[st].w};
      float gv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        gv[j] = 16 * st + 4 * q + j <= last_r ? s.cb[st][j] * dsj[j] * exp_hw(cr - csj[j]) : 0.0f;
      const Frag<T> gf = frag_make<T>(gv);
#pragma unroll
      for (int pt = 0; pt < PTB; ++pt) mma(ao[pt], xf[st][pt], gf);
    }
    // BLUE: sum_n S[p][n] C[r][n], fragments read four n tiles at a time
#pragma unroll
    for (int n0 = 0; n0 < NT; n0 += 4) {
      Frag<T> cf[4], sf[4][PTB];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (n0 + u >= NT) continue;
        cf[u] = ld_colk(cs, PPC, 16 * ort, 16 * (n0 + u), lane);
#pragma unroll
        for (int pt = 0; pt < PTB; ++pt) sf[u][pt] = ld_ntv(ss + ((n0 + u) * PTB + pt) * 256, lane);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (n0 + u >= NT) continue;
#pragma unroll
        for (int pt = 0; pt < PTB; ++pt) mma(ab[pt], sf[u][pt], cf[u]);
      }
    }
    const float er = exp_hw(cr);
    const int rows = steps_of(ch) * M;
    const brsrc ry = make_rsrc(y_b + (i64)ch * Lf * M * rs_x, (unsigned)(((rows - 1) * rs_x + PB) * 2));
#pragma unroll
    for (int pt = 0; pt < PTB; ++pt) {
      f32x4 yv;
#pragma unroll
      for (int j = 0; j < 4; ++j) yv[j] = ao[pt][j] + er * ab[pt][j];
      bstore4(ry, r < rows ? (unsigned)((r * rs_x + 16 * pt + 4 * q) * 2) : BUF_OOB, yv, (const T*)0);
    }
  };

  if (nc > 0) {
    Set sa, sb;
    // prologue: dt of chunks 0 and 1 into zrow, B and x of chunk 0 into the
    // state-update buffers, the loads of interval 0
    issue(sb, 0, 0, 0);
    if (w == 0) {
      zrow[lane] = load_dt(0);
      zrow[64 + lane] = sb.z;
    }
    __syncthreads();
    FwdScalars sc_cur = scalars_of(0, 0);
    stage_state(sb, sc_cur, 0);
    issue(sa, 1, 0, 0);
    __syncthreads();
    auto interval = [&](Set& s, Set& o, int c) {
      // s: B, x of chunk c+1, dt of chunk c+2, C of chunk c, scores of chunk c-1;
      // o: x of chunk c, refilled here for interval c+1
      const FwdScalars sc_next = scalars_of((c + 1) & 1, clampc(c + 1));
      if (w == 0) zrow[(c & 1) * 64 + lane] = s.z;
      stage_state(s, sc_next, c + 1);
      stage_out(s, o, sc_cur, c);
      issue(o, c + 2, c + 1, c);
      if (c < nc) phase1(sc_cur, c);
      if (c > 0) phase2(s, c - 1);
      __syncthreads();
      sc_cur = sc_next;
    };
    for (int c = 0; c <= nc; c += 2) {
      interval(sa, sb, c);
      if (c + 1 <= nc) interval(sb, sa, c + 1);
    }
  }

  if (a.s_final && !out_wave) {
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int pt = 0; pt < PTB; ++pt) {
        if (nt0 + i >= NT) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          a.s_final[sbase + (i64)(p0 + 16 * pt + c16) * N + 16 * (nt0 + i) + 4 * q + j] = S[i][pt][j];
      }
  }
}

template <int NT, int PTB>
size_t walk_lds() {
  constexpr int N = 16 * NT, PB = 16 * PTB;
  return 2 * (64 * (size_t)(pitch_down(N) + pitch_along(N) + 2 * pitch_down(PB)) + (size_t)NT * PTB * 256) * 2 +
         3 * 2 * 64 * 4;
}

template <int NT, int PTB>
void launch_walk_t(const FwdArgs& a, const float* cbt, unsigned grid, i64 grid_cb, hipStream_t stream) {
  if (grid_cb > 0)  // T = 0: no chunk, the walk only copies s0 to s_final
    hipLaunchKernelGGL((ssd_fwd_scores_kernel<NT>), dim3((unsigned)grid_cb), dim3(64 * CB_NW), 0, stream, a,
                       (float*)cbt);
  const size_t lds = walk_lds<NT, PTB>();
  hipLaunchKernelGGL((ssd_fwd_walk_kernel<NT, PTB>), dim3(grid), dim3(FW_NTH), lds, stream, a, cbt);
}

template <int PTB>
void launch_walk_nt(const FwdArgs& a, const float* cbt, unsigned grid, i64 grid_cb, hipStream_t stream) {
  switch (a.N / 16) {
    case 1: launch_walk_t<1, PTB>(a, cbt, grid, grid_cb, stream); break;
    case 2: launch_walk_t<2, PTB>(a, cbt, grid, grid_cb, stream); break;
    case 3: launch_walk_t<3, PTB>(a, cbt, grid, grid_cb, stream); break;
    case 4: launch_walk_t<4, PTB>(a, cbt, grid, grid_cb, stream); break;
    case 5: launch_walk_t<5, PTB>(a, cbt, grid, grid_cb, stream); break;
    case 6: launch_walk_t<6, PTB>(a, cbt, grid, grid_cb, stream); break;
    case 7: launch_walk_t<7, PTB>(a, cbt, grid, grid_cb, stream); break;
    default: launch_walk_t<8, PTB>(a, cbt, grid, grid_cb, stream); break;
  }
}

template <typename T, int NT, int PTB>
size_t fwd_lds() {
  constexpr int PAD = 32 / sizeof(T);
  constexpr int N = 16 * NT, PB = 16 * PTB;
  constexpr int BUF = 2 * 64 * (N + PAD) + 2 * 64 * (PB + PAD);
  constexpr int NBUF = sizeof(T) == 2 ? 2 : 1;
  return sizeof(T) * ((size_t)NBUF * BUF + 16 * 256 + (size_t)NT * PTB * 256);
}

template <typename T, int NT, int PTB>
void launch_fwd_t(const FwdArgs& a, unsigned grid, hipStream_t stream) {
  const size_t lds = fwd_lds<T, NT, PTB>();
  hipLaunchKernelGGL((ssd_fwd_kernel<T, NT, PTB>), dim3(grid), dim3(FW_NTH), lds, stream, a);
}

template <typename T, int PTB>
void launch_fwd_nt(const FwdArgs& a, unsigned grid, hipStream_t stream) {
  switch (a.N / 16) {
    case 1: launch_fwd_t<T, 1, PTB>(a, grid, stream); break;
    case 2: launch_fwd_t<T, 2, PTB>(a, grid, stream); break;
    case 3: launch_fwd_t<T, 3, PTB>(a, grid, stream); break;
    case 4: launch_fwd_t<T, 4, PTB>(a, grid, stream); break;
    case 5: launch_fwd_t<T, 5, PTB>(a, grid, stream); break;
    case 6: launch_fwd_t<T, 6, PTB>(a, grid, stream); break;
    case 7: launch_fwd_t<T, 7, PTB>(a, grid, stream); break;
    default: launch_fwd_t<T, 8, PTB>(a, grid, stream); break;
  }
}

}  // namespace

bool ssd_fwd_shape_supported(const ssmvjp_ssd_desc& d) {
  if (d.headdim % 16 || d.dstate % 16 || d.dstate > 128 || d.mimo_rank > 64) return false;
  // byte offsets inside one chunk are 32-bit
  const i64 esz = d.dtype == SSMVJP_BF16 ? 2 : 4;
  if (64 * d.nheads * d.headdim * esz >= (1ll << 31) || 64 * d.ngroups * d.dstate * esz >= (1ll << 31) ||
      64 * d.nheads * 4 >= (1ll << 31))
    return false;
  return true;
}

size_t ssd_fwd_workspace_bytes(const ssmvjp_ssd_desc& d) {
  if (d.dtype != SSMVJP_BF16) return 0;
  const i64 lmax = 64 / d.mimo_rank;
  const i64 Lf = d.chunk_len < lmax ? d.chunk_len : lmax;
  return (size_t)(d.batch * cdiv(d.seqlen, Lf) * d.ngroups) * 16 * 256 * sizeof(float);
}

hipError_t launch_ssd_fwd(const ssmvjp_ssd_desc& d, const SsdFwdPointers& ptr, hipStream_t stream) {
  FwdArgs a;
  a.T = d.seqlen; a.H = d.nheads; a.P = d.headdim; a.N = d.dstate; a.G = d.ngroups; a.M = d.mimo_rank;
  const i64 lmax = 64 / d.mimo_rank;
  a.Lf = (int)(d.chunk_len < lmax ? d.chunk_len : lmax);
  a.nc = (int)cdiv(d.seqlen, a.Lf);
  const int PTB = d.headdim % 32 == 0 ? 2 : 1;
  a.npb = (int)(d.headdim / (16 * PTB));
  a.raw = d.form == SSMVJP_FORM_RAW;
  a.causal = 16 % d.mimo_rank == 0;
  a.xv = ptr.xv; a.dtda = ptr.dtda; a.A = ptr.A; a.B = ptr.B; a.C = ptr.C; a.s0 = ptr.s0;
  a.y = ptr.y; a.s_final = ptr.s_final;
  const i64 grid = d.batch * d.nheads * a.npb;
  if (grid == 0) return hipGetLastError();
  a.xcd = grid % 8 == 0;
  if (d.dtype == SSMVJP_BF16) {
    const i64 grid_cb = d.batch * a.nc * d.ngroups;
    if (PTB == 2) launch_walk_nt<2>(a, (const float*)ptr.workspace, (unsigned)grid, grid_cb, stream);
    else launch_walk_nt<1>(a, (const float*)ptr.workspace, (unsigned)grid, grid_cb, stream);
  } else {
    if (PTB == 2) launch_fwd_nt<float, 2>(a, (unsigned)grid, stream);
    else launch_fwd_nt<float, 1>(a, (unsigned)grid, stream);
  }
  return hipGetLastError();
}

}  // namespace ssmvjp
