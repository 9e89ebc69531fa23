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
#include "ssd_common.cuh"

namespace ssmvjp {

// ===========================================================================
// kernel 0: the per-chunk step scalars (K1 cumsum, delta, sigmoid(dt)), one
// wave per (batch, chunk, head), stored for the scan and gradient kernels
// ===========================================================================
__global__ void __launch_bounds__(256) ssd_chunk_scalars_kernel(SsdArgs a) {
  const int lane = threadIdx.x & 63;
  const i64 id = (i64)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (id >= a.b * a.nc * a.H) return;  // whole waves
  const i64 h = id % a.H, c = (id / a.H) % a.nc, bi = id / (a.H * a.nc);
  const int L = (int)a.L;
  const i64 t0 = c * L;
  const int Lc = (int)((a.T - t0) < L ? (a.T - t0) : L);
  const float z = bload_f32(make_rsrc(a.dtda + (bi * a.T + t0) * a.H + h, (unsigned)(((Lc - 1) * a.H + 1) * 4)),
                            (unsigned)(lane * a.H * 4));
  const float Ah = a.raw ? 0.0f : a.A[h];
  const ChunkScalars cs = chunk_scalars(a, z, lane < Lc, Ah, lane);
  float* o = a.csv + id * 3 * 64;
  o[lane] = cs.cum;
  o[64 + lane] = cs.delta;
  o[128 + lane] = cs.sig;
}

// ===========================================================================
// kernel 1: forward and reverse state scans over chunks
// ===========================================================================
constexpr int SCAN_NW = 8;                   // waves per workgroup
constexpr int SCAN_NTH = 64 * SCAN_NW;
constexpr int SCAN_TILES = 32;               // state tiles per workgroup (at most)
constexpr int SCAN_MAXT = SCAN_TILES / SCAN_NW;  // state tiles per wave
constexpr int SCAN_SB = 64;                  // fused rows staged per step (at most)
// row padding (elements) of the staged tiles: 32 bytes, so that the 16 rows a
// transposed fragment read touches start 8 banks apart
template <typename T>
constexpr int scan_pad() { return 32 / (int)sizeof(T); }

// Shape parameters CP, CNB (n block), CL, CM: a non-zero value fixes P, the n
// block, the chunk length or the rank at compile time (the workload shapes get
// their own instantiations); zero reads it from the arguments.
//
// A step stages SB = min(L*M, 64) fused rows of one chunk: a whole chunk when
// L*M <= 64, else one of the chunk's L*M/64 row blocks, whose products add up
// in registers until the chunk's last block applies the state update.
//
// Pipeline: the rows of steps s+1 .. s+DEPTH are in flight in registers
// (DEPTH = 4 for the compile-time bf16 shapes, else 2) while step s is staged
// into one of two LDS buffers; with two LDS buffers a single barrier per step
// separates the staging of a buffer from its fragment reads (the reads of that
// buffer two steps back ended before the previous step's barrier).
template <typename T, int CP, int CNB, int CL, int CM>
__global__ void __launch_bounds__(SCAN_NTH) ssd_state_scan_kernel(SsdArgs a, int nb_arg) {
  constexpr int E16 = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr bool FIXED = CP && CNB && CL && CM;
  constexpr int CSB = FIXED ? (CL * CM < SCAN_SB ? CL * CM : SCAN_SB) : 0;
  constexpr int MAXC_O = FIXED ? (CSB * CP / E16 + SCAN_NTH - 1) / SCAN_NTH : SCAN_SB * 128 / E16 / SCAN_NTH;
  constexpr int MAXC_B = FIXED ? (CSB * CNB / E16 + SCAN_NTH - 1) / SCAN_NTH : SCAN_SB * 128 / E16 / SCAN_NTH;
  constexpr int MAXC = MAXC_O > MAXC_B ? MAXC_O : MAXC_B;  // staging chunks per thread
  constexpr int PAD = scan_pad<T>();
  // bf16 with compile-time shapes whose n-tile count divides the wave count:
  // fragments are read ahead of the MFMAs (PRE_RB row blocks per step)
  constexpr bool PRE = sizeof(T) == 2 && FIXED && CNB / 16 <= SCAN_NW && SCAN_NW % (CNB / 16 > 0 ? CNB / 16 : 1) == 0;
  constexpr int PRE_RB = PRE ? CSB / 16 : 0;
  // steps whose rows are in flight in registers (2 or 4)
  constexpr int DEPTH = PRE ? 4 : 2;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int P = CP ? CP : (int)a.P, N = (int)a.N, L = CL ? CL : (int)a.L, M = CM ? CM : (int)a.M;
  const int NB = CNB ? CNB : nb_arg, LM = L * M;
  const int SB = CSB ? CSB : (LM < SCAN_SB ? LM : SCAN_SB);  // fused rows per step
  const int NSUB = LM / SB;                                  // steps per chunk
  const int PT = P / 16, NTB = NB / 16, RB = SB / 16;
  const int PPO = P + PAD, PPB = NB + PAD;  // row pitches (elements) of the staged tiles
  const int BUF = SB * (PPO + PPB);         // elements per LDS buffer
  // buffer k: [SB][PPO] v or dy rows scaled per step, then [SB][PPB] B or C rows (this n block)

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, q = lane >> 4,
            r16 = lane & 15;
  __builtin_assume(w >= 0 && w < SCAN_NW);  // lets the tile loop compile without branches
  const int nblk = N / NB;
  // XCD-aware order: the n blocks of one (batch, head, direction) read the same
  // v or dy rows, and the heads of a batch the same B or C rows, so
  // consecutive ids are given workgroups that land on the same XCD (ids are
  // dealt to the 8 XCDs round robin) and walk their chunks side by side
  i64 bid = blockIdx.x;
  if (gridDim.x % 8 == 0) bid = (bid % 8) * (gridDim.x / 8) + bid / 8;
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

  const int ntiles = PT * NTB;  // tiles of this wave: ti = pt * NTB + nt, ti % SCAN_NW == w
  f32x4 st[SCAN_MAXT], acc[SCAN_MAXT];
#pragma unroll
  for (int k = 0; k < SCAN_MAXT; ++k) {
    const int ti = w + SCAN_NW * k;
    st[k] = acc[k] = zero4();
    if (ti < ntiles && init) {
      const int pt = ti / NTB, nt = ti % NTB;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st[k][j] = init[((bi * a.H + h) * P + 16 * pt + 4 * q + j) * N + n0 + 16 * nt + r16];
    }
  }

  // register prefetch of one step: the chunk's step values, operand rows, B/C rows.
  // Branch-free buffer loads: rows past the end of the sequence read zeros.
  struct Pre {
    float cum, delta;  // the chunk's step scalars (this lane's step)
    u32x4 o[MAXC], b[MAXC];
  };
  const int oc_row = P / E16, bc_row = NB / E16;
  const unsigned esz = sizeof(T);
  const int nsteps = (int)(a.nc * NSUB);
  // loop-invariant bases of this (batch, head, n block); per-step offsets
  // inside one batch element are 32-bit (the shape check bounds them)
  const int rs_op = (int)(a.H * P), rs_bc = (int)(a.G * a.N);  // fused-row strides of x/dy and B/C
  const T* op_b = op + ix_xv(a, bi, 0, 0, h, 0);
  const T* bc_b = bc + ix_bc(a, bi, 0, 0, g, n0);
  const float* csv_b = a.csv + (bi * a.nc * a.H + h) * 3 * 64;
  T* out_b = out + (bi * a.nc * a.H + h) * (i64)P * N;
  const int T32 = (int)a.T, nc32 = (int)a.nc, H32 = (int)a.H;
  auto chunk_of = [&](int step) { const int ci = step / NSUB; return dir == 0 ? ci : nc32 - 1 - ci; };
  auto issue = [&](Pre& pr, int step) {
    const int c = chunk_of(step);
    const int R0 = (step % NSUB) * SB;  // first fused row of this step
    const int t0 = c * L;
    const int Lc = T32 - t0 < L ? T32 - t0 : L;
    const int rows = Lc * M - R0;  // valid fused rows of this step (may be <= 0)
    const int R = t0 * M + R0;     // first fused row in the batch element
    const brsrc rcs = make_rsrc(csv_b + c * H32 * 3 * 64, 3 * 64 * 4);
    pr.cum = bload_f32(rcs, (unsigned)lane * 4u);
    pr.delta = bload_f32(rcs, (unsigned)(64 + lane) * 4u);
    const brsrc ro = make_rsrc(op_b + R * rs_op, rows > 0 ? (unsigned)(((rows - 1) * rs_op + P) * esz) : 0u);
    const brsrc rb = make_rsrc(bc_b + R * rs_bc, rows > 0 ? (unsigned)(((rows - 1) * rs_bc + NB) * esz) : 0u);
#pragma unroll
    for (int it = 0; it < MAXC; ++it) {
      const int idx = tid + it * SCAN_NTH;
      const int r1 = idx / oc_row, c1 = (idx % oc_row) * E16;
      const int r2 = idx / bc_row, c2 = (idx % bc_row) * E16;
      pr.o[it] = bload16(ro, idx < SB * oc_row ? (unsigned)((r1 * rs_op + c1) * esz) : BUF_OOB);
      pr.b[it] = bload16(rb, idx < SB * bc_row ? (unsigned)((r2 * rs_bc + c2) * esz) : BUF_OOB);
    }
  };
  // per-chunk scalars, set on the chunk's first step
  float sc = 0.0f, e_end = 1.0f;
  // one step: (first step of a chunk) step scalars, staging into LDS buffer sb,
  // refill of pr with step + DEPTH (clamped to the last step: loads that are never
  // used keep the issue unconditional), one barrier, then the state tiles; the
  // chunk's last step stores S_c (or dS_{c+1}) and applies the state update
  auto process = [&](Pre& pr, int step, T* sb) {
    const int c = chunk_of(step);
    const int ks = step % NSUB;
    const bool last = ks == NSUB - 1;
    if (ks == 0) {
      const float end = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr.cum), 63));
      sc = dir == 0 ? pr.delta * exp_hw(end - pr.cum) : exp_hw(pr.cum);
      e_end = exp_hw(end);
    }
    T* opS = sb;
    T* bcS = sb + SB * PPO;
#pragma unroll
    for (int it = 0; it < MAXC; ++it) {
      const int idx = tid + it * SCAN_NTH;
      const int r = idx / oc_row;
      const float s_r = __shfl(sc, ((ks * SB + r) / M) & 63, 64);
      if (idx < SB * oc_row) *(u32x4*)(opS + r * PPO + (idx % oc_row) * E16) = scale16(pr.o[it], s_r, (const T*)0);
      if (idx < SB * bc_row) *(u32x4*)(bcS + (idx / bc_row) * PPB + (idx % bc_row) * E16) = pr.b[it];
    }
    issue(pr, step + DEPTH < nsteps ? step + DEPTH : nsteps - 1);
    __syncthreads();
    // state block of this chunk and head; the store is dropped except on the
    // chunk's last step (a range check, so that no store sits in a branch)
    const brsrc rout = make_rsrc(out_b + c * H32 * P * N, (unsigned)(P * N) * esz);
    auto update = [&](int k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        st[k][j] = last ? e_end * st[k][j] + acc[k][j] : st[k][j];
        acc[k][j] = last ? 0.0f : acc[k][j];
      }
    };
    if constexpr (PRE_RB > 0) {
      // all of the step's fragment reads are issued before the first MFMA
      // waits on them.  With the n-tile count dividing the wave count every
      // tile of a wave has the same n tile (nt = w % NTB), so the B or C
      // fragments are read once per wave.
      Frag<T> fa[SCAN_MAXT][PRE_RB], fb[PRE_RB];
      const int nt = w % NTB;
#pragma unroll
      for (int kb = 0; kb < PRE_RB; ++kb) fb[kb] = ld_rowk(bcS, PPB, 16 * kb, 16 * nt, lane);
#pragma unroll
      for (int k = 0; k < SCAN_MAXT; ++k) {
        const int ti = w + SCAN_NW * k;
        if (ti >= ntiles) continue;
#pragma unroll
        for (int kb = 0; kb < PRE_RB; ++kb) fa[k][kb] = ld_rowk(opS, PPO, 16 * kb, 16 * (ti / NTB), lane);
      }
#pragma unroll
      for (int k = 0; k < SCAN_MAXT; ++k) {
        const int ti = w + SCAN_NW * k;
        if (ti >= ntiles) continue;
        bstore4(rout, last ? (unsigned)native_off(N, ti / NTB, n0 / 16 + nt, lane, 0) * esz : BUF_OOB, st[k],
                (const T*)0);
#pragma unroll
        for (int kb = 0; kb < PRE_RB; ++kb) mma(acc[k], fa[k][kb], fb[kb]);
        update(k);
      }
    } else {
#pragma unroll
      for (int k = 0; k < SCAN_MAXT; ++k) {
        const int ti = w + SCAN_NW * k;
        if (ti >= ntiles) continue;
        const int pt = ti / NTB, nt = ti % NTB;
        bstore4(rout, last ? (unsigned)native_off(N, pt, n0 / 16 + nt, lane, 0) * esz : BUF_OOB, st[k], (const T*)0);
        for (int kb = 0; kb < RB; ++kb)
          mma(acc[k], ld_rowk(opS, PPO, 16 * kb, 16 * pt, lane), ld_rowk(bcS, PPB, 16 * kb, 16 * nt, lane));
        update(k);
      }
    }
  };

  T* sb0 = (T*)smem_raw;
  T* sb1 = sb0 + BUF;
  int step = 0;
  if (nsteps > 0) {  // T = 0 has no chunk to prefetch
    // each process() ends with SCAN_MAXT state stores after its refill
    const brsrc pad = make_rsrc(out, 0u);
    auto first = [&](Pre& pr, int s) {
      issue(pr, s < nsteps ? s : nsteps - 1);
      vmem_pad_stores<SCAN_MAXT>(pad);
    };
    if constexpr (DEPTH == 4) {
      Pre p0, p1, p2, p3;
      first(p0, 0);
      first(p1, 1);
      first(p2, 2);
      first(p3, 3);
      for (; step + 3 < nsteps; step += 4) {
        process(p0, step, sb0);
        process(p1, step + 1, sb1);
        process(p2, step + 2, sb0);
        process(p3, step + 3, sb1);
      }
      if (step < nsteps) process(p0, step, sb0);
      if (step + 1 < nsteps) process(p1, step + 1, sb1);
      if (step + 2 < nsteps) process(p2, step + 2, sb0);
    } else {
      Pre p0, p1;
      first(p0, 0);
      first(p1, 1);
      for (; step + 1 < nsteps; step += 2) {
        process(p0, step, sb0);
        process(p1, step + 1, sb1);
      }
      if (step < nsteps) process(p0, step, sb0);
    }
  }
  if (dir == 1) {
#pragma unroll
    for (int k = 0; k < SCAN_MAXT; ++k) {
      const int ti = w + SCAN_NW * k;
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
constexpr int CH_NW = 8;              // waves per workgroup
constexpr int CH_NTH = 64 * CH_NW;
constexpr int MAXRB = 4;              // L*M <= 64
constexpr int MAXG2 = 2;              // lower-triangular (t, s) tile pairs per wave (<= 10 pairs)
constexpr int MAXI2 = 4;              // (p tile, row block) items per wave (<= 32 items)

enum { PB_BLUE = 0, PB_OROW, PB_OCOL, PB_DEC, PB_DVX, PB_DEND, PB_N };

// float tile -> operand fragment of type T
template <typename T>
__device__ __forceinline__ Frag<T> cvt_colk(const float* tile, int pitch, int c0, int k0, int lane) {
  const Frag<float> f = ld_colk(tile, pitch, c0, k0, lane);
  return frag_make<T>(f.v);
}
template <typename T>
__device__ __forceinline__ Frag<T> cvt_rowk(const float* tile, int pitch, int k0, int c0, int lane) {
  const Frag<float> f = ld_rowk(tile, pitch, k0, c0, lane);
  return frag_make<T>(f.v);
}

// DA: also the per-chunk dA partial sums (a separate instantiation, so that
// the plain backward keeps its registers)
template <typename T, int CP, int CN, int CL, int CM, bool DA>
__global__ void __launch_bounds__(CH_NTH) ssd_chunk_bwd_kernel(SsdArgs a) {
  constexpr int E16 = 16 / sizeof(T);
  constexpr bool FIXED = CP && CN && CL && CM;
  // bf16: S_c is staged in LDS and the next head's data is prefetched into
  // registers; float32 (twice the bytes) reads S_c straight from global memory
  // and stages unpadded rows, so that the LDS footprint stays under 160 KiB.
  constexpr bool BF = sizeof(T) == 2;
  constexpr int PAD = BF ? 8 : 0;
  constexpr int MAXX = FIXED ? (CL * CM * CP / E16 + CH_NTH - 1) / CH_NTH : 64 * 128 / E16 / CH_NTH;
  constexpr int MAXS = FIXED ? (CP * CN / E16 + CH_NTH - 1) / CH_NTH : 128 * 128 / E16 / CH_NTH;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int P = CP ? CP : (int)a.P, N = CN ? CN : (int)a.N, L = CL ? CL : (int)a.L, M = CM ? CM : (int)a.M;
  const int LM = L * M;
  const int PT = P / 16, NT = N / 16, RB = LM / 16;
  const int LDC = LM + 4;     // CB pitch (float)
  const int LDN = N + PAD;    // B / C pitch
  const int LDP = P + PAD;    // x / dy pitch
  float* CBs = (float*)smem_raw;                 // [LM][LDC] C.B^T, later the head-summed d_cb
  // partial row sums [PB_N][8][64]; bf16 keeps two sets so that a head's
  // d_cumA assembly can run one head later, overlapped with the next head
  constexpr int NPB = BF ? 2 : 1;
  float* pbase = CBs + LM * LDC;
  T* Bs = (T*)(pbase + NPB * PB_N * 8 * 64);     // [LM][LDN]
  T* Cs = Bs + LM * LDN;                         // [LM][LDN]
  T* xs = Cs + LM * LDN;                         // [LM][LDP] x (Mamba-2) or v (RAW)
  T* dys = xs + LM * LDP;                        // [LM][LDP]
  T* dSs = dys + LM * LDP;                       // [P*N] dS_{c+1}, native tiles
  T* Ss = dSs + P * N;                           // [P*N] S_c, native tiles (bf16 only)
  T* Wt = Ss + P * N;                            // [10][256] masked CB * decay per (t, s) tile pair (bf16 only)

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, q = lane >> 4,
            r16 = lane & 15;
  __builtin_assume(w >= 0 && w < CH_NW);  // lets per-wave item loops compile without branches
  i64 bid = blockIdx.x;
  const i64 hs = bid % a.hsplit;
  bid /= a.hsplit;
  const i64 g = bid % a.G;
  bid /= a.G;
  const i64 c = bid % a.nc, bi = bid / a.nc;
  const i64 t0 = c * L;
  const int Lc = (int)((a.T - t0) < L ? (a.T - t0) : L);
  // per-chunk base pointers; offsets inside a chunk are 32-bit
  const int xrs = (int)(a.H * P), brs = (int)(a.G * N);  // fused-row strides of x/dy/dx and B/C/dB/dC
  const i64 xoff0 = (bi * a.T + t0) * M * a.H * P, boff0 = (bi * a.T + t0) * M * a.G * N + g * N;
  const T* xg = (const T*)a.xv + xoff0;
  const T* dyg = (const T*)a.dy + xoff0;
  T* dxg = (T*)a.dxv + xoff0;
  const T* Bg = (const T*)a.B + boff0;
  const T* Cg = (const T*)a.C + boff0;
  float* ddtg = a.d_dtda + (bi * a.T + t0) * a.H;
  const int xrow = P / E16, nrow = N / E16, PN = P * N;
  auto tile_off = [&](int pt, int nt) { return (pt * NT + nt) * 256; };

  // ---- B and C rows of the chunk (group g) into LDS ----
  for (int idx = tid; idx < LM * nrow; idx += CH_NTH) {
    const int r = idx / nrow, col = (idx % nrow) * E16, l = r / M, m = r % M;
    u32x4 ub = zero_u4(), uc = zero_u4();
    (void)m;
    if (l < Lc) {
      ub = load16(Bg + r * brs + col);
      uc = load16(Cg + r * brs + col);
    }
    *(u32x4*)(Bs + r * LDN + col) = ub;
    *(u32x4*)(Cs + r * LDN + col) = uc;
  }

  // ---- register prefetch of one head: dt/da and A, x/v and dy rows, S_c and dS_{c+1} ----
  // Branch-free buffer loads (rows past the end of the sequence read zeros), so
  // that the next head's loads stay in flight across this head's work.
  u32x4 rx[MAXX], ry[MAXX], rs[MAXS], rd[MAXS];
  ChunkScalars rcs = {0.f, 0.f, 0.f, 0.f};  // the head's stored step scalars
  float rA = 0.0f;
  const i64 hbase = g * a.hpg + hs * a.hph;
  const unsigned esz = sizeof(T);
  const unsigned xbytes = (unsigned)(((i64)(Lc * M - 1) * xrs + P) * esz);  // valid rows of one head
  const brsrc rsA = make_rsrc(a.A, a.raw ? 0u : (unsigned)(a.H * 4));      // RAW: no A, reads zero
  auto issue = [&](i64 h) {
    rcs = issue_scalars(a, bi, c, h, lane);
    rA = bload_f32(rsA, (unsigned)(h * 4));
    const brsrc bx = make_rsrc(xg + (int)h * P, xbytes), by = make_rsrc(dyg + (int)h * P, xbytes);
#pragma unroll
    for (int it = 0; it < MAXX; ++it) {
      const int idx = tid + it * CH_NTH;
      const int r = idx / xrow, col = (idx % xrow) * E16;
      const unsigned off = idx < LM * xrow ? (unsigned)(r * xrs + col) * esz : BUF_OOB;
      rx[it] = bload16(bx, off);
      ry[it] = bload16(by, off);
    }
    const T* Sg = (const T*)a.S + ((bi * a.nc + c) * a.H + h) * (i64)PN;
    const T* dSg = (const T*)a.dS + ((bi * a.nc + c) * a.H + h) * (i64)PN;
    const brsrc bs = make_rsrc(Sg, (unsigned)PN * esz), bd = make_rsrc(dSg, (unsigned)PN * esz);
#pragma unroll
    for (int it = 0; it < MAXS; ++it) {
      const int idx = tid + it * CH_NTH;
      const unsigned off = idx < PN / E16 ? (unsigned)idx * 16u : BUF_OOB;
      if (BF) rs[it] = bload16(bs, off);
      rd[it] = bload16(bd, off);
    }
  };
  if (BF) {
    issue(hbase);
    // a head issues the next head's loads, then the d_dt (and dA) stores and
    // one dx store per (p tile, row block) item of this wave
    if constexpr (FIXED) vmem_pad_stores<(DA ? 2 : 1) + (CP / 16) * (CL * CM / 16) / CH_NW>(make_rsrc(a.dxv, 0u));
  }
  __syncthreads();  // B, C staged

  // ---- C.B^T (K2 recompute) over the lower-triangular tile pairs; upper pairs zero ----
  for (int pi = w; pi < RB * RB; pi += CH_NW) {
    const int rt = pi / RB, rs_ = pi % RB;
    f32x4 acc = zero4();
    if (rs_ <= rt)
      for (int kb = 0; kb < NT; ++kb)
        mma(acc, ld_colk(Cs, LDN, 16 * rt, 16 * kb, lane), ld_colk(Bs, LDN, 16 * rs_, 16 * kb, lane));
#pragma unroll
    for (int j = 0; j < 4; ++j) CBs[(16 * rt + 4 * q + j) * LDC + 16 * rs_ + r16] = acc[j];
  }

  // per-wave work items
  const int npairs = RB * (RB + 1) / 2;
  int pair_rt[MAXG2], pair_rs[MAXG2];
#pragma unroll
  for (int k = 0; k < MAXG2; ++k) {
    const int pi = w + CH_NW * k;
    int rt = 0;
    while (rt < RB && (rt + 1) * (rt + 2) / 2 <= pi) ++rt;
    pair_rt[k] = pi < npairs ? rt : -1;
    pair_rs[k] = pi < npairs ? pi - rt * (rt + 1) / 2 : -1;
  }
  const int nt_own = w;  // the n tile of this wave (N <= 16 * CH_NW)
  f32x4 dBacc[MAXRB], dCacc[MAXRB], dcbacc[MAXG2];
#pragma unroll
  for (int rb = 0; rb < MAXRB; ++rb) dBacc[rb] = dCacc[rb] = zero4();
#pragma unroll
  for (int k = 0; k < MAXG2; ++k) dcbacc[k] = zero4();

  // d_cumA from its four sources, the K1 suffix sum and the chain to d_dt for
  // one head, from the partial row sums in pb; run by a single wave, which gets
  // the d_dt (RAW: d_da) value of step `lane` back, and the head's dA partial
  // sum over the chunk, sum_l d_da_l * delta_l, in every lane.
  auto epilogue = [&](const ChunkScalars& cs, float Ah, const float* pb) -> float2 {
    auto cum_of = [&](int l) { return __shfl(cs.cum, l, 64); };
    float dc = 0.0f, qv = 0.0f, dvx = 0.0f;
    const float c_row = cum_of((lane / M) & 63);  // every lane takes part in the shuffle
    if (lane < LM) {
      float blue = 0, orow = 0, ocol = 0, dec = 0;
      for (int k = 0; k < NT; ++k) blue += pb[(PB_BLUE * 8 + k) * 64 + lane];
      for (int k = 0; k < CH_NW; ++k) {
        orow += pb[(PB_OROW * 8 + k) * 64 + lane];
        ocol += pb[(PB_OCOL * 8 + k) * 64 + lane];
      }
      for (int k = 0; k < PT; ++k) {
        dec += pb[(PB_DEC * 8 + k) * 64 + lane];
        dvx += pb[(PB_DVX * 8 + k) * 64 + lane];
      }
      qv = dec * exp_hw(cs.end - c_row);
      dc = blue + orow - ocol - qv;
    }
    const float qsum = wave_sum(qv);
    float dendt = 0.0f;
    for (int k = 0; k < CH_NW; ++k) dendt += pb[(PB_DEND * 8 + k) * 64];
    dendt *= exp_hw(cs.end);
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
    return make_float2(a.raw ? dda : (dvxl + dda * Ah) * cs.sig, DA ? wave_sum(dda * cs.delta) : 0.0f);
  };
  // every wave stores (dropped unless `on` and lane < Lc): no store sits in a
  // branch, which keeps the compiler's count of outstanding loads exact
  const brsrc bddt = make_rsrc(ddtg, (unsigned)(Lc * a.H * 4));
  auto epi_store = [&](bool on, i64 h, float2 v) {
    bstore_f32(bddt, on && lane < Lc ? (unsigned)((lane * a.H + h) * 4) : BUF_OOB, v.x);
    if constexpr (DA) bstore_f32(dA_rsrc(a, bi, c), on && lane == 0 ? (unsigned)(h * 4) : BUF_OOB, v.y);
  };
  i64 prev_h = 0;
  ChunkScalars prev_cs = {0.f, 0.f, 0.f, 0.f};
  float prev_Ah = 0.0f;

  for (i64 hh = 0; hh < a.hph; ++hh) {
    const i64 h = hbase + hh;
    if (!BF) issue(h);
    float* pb = pbase + (BF ? (hh & 1) * PB_N * 8 * 64 : 0);
    const ChunkScalars cs = finish_scalars(rcs);
    const float Ah = rA;
    const brsrc bdx = make_rsrc(dxg + (int)h * P, xbytes);
    // lane shuffles: call them where every lane of the wave is active (a
    // shuffle under a divergent mask reads zero from inactive source lanes)
    auto cum_of = [&](int l) { return __shfl(cs.cum, l, 64); };
    auto delta_of = [&](int l) { return __shfl(cs.delta, l, 64); };

    __syncthreads();  // previous head is done with xs / dys / Ss / dSs (and CB writes on entry)
#pragma unroll
    for (int it = 0; it < MAXX; ++it) {
      const int idx = tid + it * CH_NTH;
      if (idx < LM * xrow) {
        const int r = idx / xrow, col = (idx % xrow) * E16;
        *(u32x4*)(xs + r * LDP + col) = rx[it];
        *(u32x4*)(dys + r * LDP + col) = ry[it];
      }
    }
#pragma unroll
    for (int it = 0; it < MAXS; ++it) {
      const int idx = tid + it * CH_NTH;
      if (idx < PN / E16) {
        if (BF) *(u32x4*)(Ss + idx * E16) = rs[it];
        *(u32x4*)(dSs + idx * E16) = rd[it];
      }
    }
    if (BF) issue(hh + 1 < a.hph ? h + 1 : h);  // unconditional: the last head reloads its own rows
    __syncthreads();
    // the previous head's partial sums are complete: assemble its d_cumA on a
    // rotating wave while the other waves start on this head
    if (BF) {
      const bool on = hh > 0 && w == (int)((hh - 1) % CH_NW);
      float2 v = make_float2(0.0f, 0.0f);
      if (on) v = epilogue(prev_cs, prev_Ah, pbase + ((hh - 1) & 1) * PB_N * 8 * 64);
      epi_store(on, prev_h, v);
    }

    // ---- ORANGE: G1 = dy . x^T on lower-triangular tile pairs; d_cb, row/col sums ----
    {
      float orow[MAXG2][4], ocol[MAXG2];
#pragma unroll
      for (int k = 0; k < MAXG2; ++k) {
        ocol[k] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) orow[k][j] = 0.0f;
        const int rt = pair_rt[k], rs_ = pair_rs[k];
        if (rt < 0) continue;
        f32x4 acc = zero4();
        float wv[4];
        for (int kb = 0; kb < PT; ++kb)
          mma(acc, ld_colk(dys, LDP, 16 * rt, 16 * kb, lane), ld_colk(xs, LDP, 16 * rs_, 16 * kb, lane));
        const int s_ = 16 * rs_ + r16, ls = s_ / M;
        const float cs_s = cum_of(ls), dls = delta_of(ls);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * rt + 4 * q + j, lt = t / M;
          const float ct = cum_of(lt);  // every lane takes part in the shuffle
          const float dec = (ls <= lt && lt < Lc) ? exp_hw(ct - cs_s) : 0.0f;
          const float dcb = acc[j] * dls * dec;  // d_w = dy . v^T with v = delta x (delta = 1 for RAW)
          dcbacc[k][j] += dcb;
          const float cb = CBs[t * LDC + s_];
          const float dd = dcb * cb;
          orow[k][j] += dd;
          ocol[k] += dd;
          wv[j] = cb * dec;  // w = CB * decay at (t, s): the d_v_orange operand
        }
        // w in native tile order is the B operand (k = t, columns s) of d_v_or^T
        if (BF) store4(Wt + (rt * (rt + 1) / 2 + rs_) * 256 + 4 * lane, f32x4{wv[0], wv[1], wv[2], wv[3]});
      }
      // this wave's slots: row sums for its items' row blocks, column sums for
      // its items' column blocks, zero elsewhere
#pragma unroll
      for (int rb = 0; rb < MAXRB; ++rb) {
        if (rb >= RB) break;
        float rsum[4] = {0.f, 0.f, 0.f, 0.f}, csum = 0.0f;
        bool rtouch = false, ctouch = false;
#pragma unroll
        for (int k = 0; k < MAXG2; ++k) {
          if (pair_rt[k] == rb) {
            rtouch = true;
#pragma unroll
            for (int j = 0; j < 4; ++j) rsum[j] += orow[k][j];
          }
          if (pair_rs[k] == rb) {
            ctouch = true;
            csum += ocol[k];
          }
        }
        if (rtouch) {
#pragma unroll
          for (int j = 0; j < 4; ++j) rsum[j] = sum16(rsum[j]);
        }
        if (r16 == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) pb[(PB_OROW * 8 + w) * 64 + 16 * rb + 4 * q + j] = rsum[j];
        }
        if (ctouch) csum = sum4q(csum);
        if (q == 0) pb[(PB_OCOL * 8 + w) * 64 + 16 * rb + r16] = csum;
      }
    }

    // The [L x N] and [L x P] products are computed transposed (rows n or p,
    // columns the chunk's rows r = l*M + m), so per-row factors are per-lane
    // constants, reductions over n or p are in-lane plus sum4q, and results
    // leave as 4 consecutive n or p per lane (vector stores).

    // ---- BLUE: dC_blue^T = S_c^T . (dy * exp(cumA))^T ; d_cumA_blue = colsum(C^T * dC_blue^T) ----
    // ---- K3:   dB_k3^T  += dS_{c+1}^T . (exp(end - cumA) v)^T ;  d_end = sum S_c * dS_{c+1} ----
    float dend = 0.0f;
    if (nt_own < NT) {
      const T* Scur = BF ? (const T*)Ss : (const T*)a.S + ((bi * a.nc + c) * a.H + h) * (i64)PN;
      float ecol[MAXRB], xcol[MAXRB];
#pragma unroll
      for (int rb = 0; rb < MAXRB; ++rb) {
        const int l = (16 * rb + r16) / M;  // this lane's column r
        const float cl = cum_of(l);
        ecol[rb] = exp_hw(cl);
        xcol[rb] = delta_of(l) * exp_hw(cs.end - cl);
      }
      f32x4 acc1[MAXRB], acc2[MAXRB];
#pragma unroll
      for (int rb = 0; rb < MAXRB; ++rb) acc1[rb] = acc2[rb] = zero4();
      for (int kb = 0; kb < PT; ++kb) {
        const Frag<T> fS = ld_ntv(Scur + tile_off(kb, nt_own), lane);    // A: rows n, k = p
        const Frag<T> fdS = ld_ntv(dSs + tile_off(kb, nt_own), lane);
        float vS[4], vdS[4];
        frag_get(fS, vS);
        frag_get(fdS, vdS);
#pragma unroll
        for (int j = 0; j < 4; ++j) dend += vS[j] * vdS[j];
#pragma unroll
        for (int rb = 0; rb < MAXRB; ++rb) {
          if (rb >= RB) break;
          mma(acc1[rb], fS, ld_colk(dys, LDP, 16 * rb, 16 * kb, lane));  // B: k = p, columns r
          mma(acc2[rb], fdS, ld_colk(xs, LDP, 16 * rb, 16 * kb, lane));
        }
      }
#pragma unroll
      for (int rb = 0; rb < MAXRB; ++rb) {
        if (rb >= RB) break;
        const int r = 16 * rb + r16;
        float cv[4];
        frag_get(ld_colk(Cs, LDN, 16 * rb, 16 * nt_own, lane), cv);  // C[r][n .. n+3], n = 16 nt + 4q
        float bsum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float val = acc1[rb][j] * ecol[rb];
          dCacc[rb][j] += val;
          bsum += cv[j] * val;
          dBacc[rb][j] += acc2[rb][j] * xcol[rb];
        }
        bsum = sum4q(bsum);
        if (q == 0) pb[(PB_BLUE * 8 + nt_own) * 64 + r] = bsum;
      }
    }

    if (BF) __syncthreads();  // w tiles complete

    // ---- K3: d_dv^T = dS_{c+1} . B^T ; ORANGE: d_v_or^T = dy^T . (CB * decay) ; dx ----
#pragma unroll
    for (int k2 = 0; k2 < MAXI2; ++k2) {
      const int it = w + CH_NW * k2;
      if (it >= PT * RB) continue;
      const int pt = it / RB, rb = it % RB;
      f32x4 acc3 = zero4(), acc5 = zero4();
      for (int kb = 0; kb < NT; ++kb)  // A: rows p, k = n (transposed native read); B: k = n, columns r
        mma(acc3, ld_ntv_t(dSs + tile_off(pt, kb), lane), ld_colk(Bs, LDN, 16 * rb, 16 * kb, lane));
      const int s_ = 16 * rb + r16, ls = s_ / M;  // this lane's column
      const float cs_s = cum_of(ls);
      for (int kb = rb; kb < RB; ++kb) {  // A: rows p, k = t (transpose read of dy rows); B: k = t, columns s
        if constexpr (BF) {
          mma(acc5, ld_rowk(dys, LDP, 16 * kb, 16 * pt, lane), ld_ntv(Wt + (kb * (kb + 1) / 2 + rb) * 256, lane));
        } else {  // float32: no LDS room for the shared w tiles; recompute them
          float fw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = 16 * kb + 4 * q + j, lt = t / M;
            const float ct = cum_of(lt);  // every lane takes part in the shuffle
            fw[j] = (ls <= lt && lt < Lc) ? CBs[t * LDC + s_] * exp_hw(ct - cs_s) : 0.0f;
          }
          mma(acc5, ld_rowk(dys, LDP, 16 * kb, 16 * pt, lane), frag_make<T>(fw));
        }
      }
      const int r = s_, l = ls;
      const float dl = delta_of(l);
      const float edec = exp_hw(cs.end - cs_s);
      float xv[4];
      frag_get(ld_colk(xs, LDP, 16 * rb, 16 * pt, lane), xv);  // x[r][p .. p+3], p = 16 pt + 4q
      float dvo[4], s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float dv = acc3[j] * edec + acc5[j];  // d_v = d_v_k3 + d_v_orange
        dvo[j] = a.raw ? dv : dv * dl;
        s1 += acc3[j] * xv[j];                      // d_decay / delta = sum_p d_decayed_v . x
        s2 += dv * xv[j];
      }
      // rows past the end of the sequence fall outside the resource and are dropped
      bstore4(bdx, (unsigned)(r * xrs + 16 * pt + 4 * q) * esz, f32x4{dvo[0], dvo[1], dvo[2], dvo[3]}, (const T*)0);
      s1 = sum4q(s1) * dl;
      s2 = sum4q(s2);
      if (q == 0) {
        pb[(PB_DEC * 8 + pt) * 64 + r] = s1;
        pb[(PB_DVX * 8 + pt) * 64 + r] = s2;
      }
    }
    dend = wave_sum(dend);
    if (lane == 0) pb[(PB_DEND * 8 + w) * 64] = dend;
    __syncthreads();  // partial row sums complete

    // ---- d_cumA assembly: this head now (float32) or one head later (bf16) ----
    if (!BF) {
      __syncthreads();  // partial row sums complete
      float2 v = make_float2(0.0f, 0.0f);
      if (w == 0) v = epilogue(cs, Ah, pbase);
      epi_store(w == 0, h, v);
    } else {
      prev_h = h;
      prev_cs = cs;
      prev_Ah = Ah;
    }
  }
  if (BF && a.hph > 0) {
    __syncthreads();
    const bool on = w == (int)((a.hph - 1) % CH_NW);
    float2 v = make_float2(0.0f, 0.0f);
    if (on) v = epilogue(prev_cs, prev_Ah, pbase + ((a.hph - 1) & 1) * PB_N * 8 * 64);
    epi_store(on, prev_h, v);
  }

  // ---- K2 backward on the head-summed d_cb: dC_k2 = d_cb . B, dB_k2 = d_cb^T . C ----
  __syncthreads();
#pragma unroll
  for (int k = 0; k < MAXG2; ++k) {
    const int rt = pair_rt[k], rs_ = pair_rs[k];
    if (rt < 0) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) CBs[(16 * rt + 4 * q + j) * LDC + 16 * rs_ + r16] = dcbacc[k][j];
  }
  __syncthreads();
  if (nt_own < NT) {
    const i64 stride = a.b * a.T * a.M * a.G * a.N;
#pragma unroll
    for (int rb = 0; rb < MAXRB; ++rb) {
      if (rb >= RB) break;
      // transposed: rows n, columns r
      f32x4 accC = dCacc[rb], accB = dBacc[rb];
      for (int kb = 0; kb <= rb; ++kb)  // dC_k2^T = B^T . d_cb^T
        mma(accC, ld_rowk(Bs, LDN, 16 * kb, 16 * nt_own, lane), cvt_colk<T>(CBs, LDC, 16 * rb, 16 * kb, lane));
      for (int kb = rb; kb < RB; ++kb)  // dB_k2^T = C^T . d_cb
        mma(accB, ld_rowk(Cs, LDN, 16 * kb, 16 * nt_own, lane), cvt_rowk<T>(CBs, LDC, 16 * kb, 16 * rb, lane));
      const int r = 16 * rb + r16, l = r / M;
      if (l >= Lc) continue;
      const int o = r * brs + 16 * nt_own + 4 * q;  // dB[r][n .. n+3], offset from boff0
      if (a.hsplit == 1) {
        store4((T*)a.dB + boff0 + o, accB);
        store4((T*)a.dC + boff0 + o, accC);
      } else {
        store4(a.part + hs * stride + boff0 + o, accB);
        store4(a.part + (a.hsplit + hs) * stride + boff0 + o, accC);
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
  // n block per scan workgroup: at most SCAN_TILES state tiles per workgroup
  // (and halved while the scan has fewer workgroups than CUs)
  i64 nb = d.dstate;
  while ((d.headdim / 16) * (nb / 16) > SCAN_TILES && nb % 32 == 0) nb /= 2;
  while (d.batch * d.nheads * 2 * (d.dstate / nb) < 256 && nb % 32 == 0) nb /= 2;
  return (int)nb;
}

// heads of a group split over workgroups only until there is one workgroup per
// CU: the chunk kernel's LDS footprint admits one resident workgroup per CU, so
// further splits would run back to back and only add the partial-sum pass
static i64 pick_hsplit(const ssmvjp_ssd_desc& d, i64 nc) {
  const i64 hpg = d.nheads / d.ngroups;
  const i64 base = d.batch * nc * d.ngroups;
  i64 hs = 1;
  while (base * hs < 256 && hs * 2 <= hpg && hpg % (hs * 2) == 0) hs *= 2;
  return hs;
}

static size_t grads_lds_bytes(const ssmvjp_ssd_desc& d) {
  const bool bf = d.dtype == SSMVJP_BF16;
  const size_t e = bf ? 2 : 4, pad = bf ? 8 : 0, LM = (size_t)(d.chunk_len * d.mimo_rank);
  return 4 * (LM * (LM + 4) + (bf ? 2 : 1) * PB_N * 8 * 64) +
         e * (2 * LM * (d.dstate + pad) + 2 * LM * (d.headdim + pad) + (bf ? 2 : 1) * (size_t)(d.headdim * d.dstate) +
              (bf ? 10 * 256 : 0));
}

bool ssd_shape_supported(const ssmvjp_ssd_desc& d) {
  if (d.headdim % 16 || d.dstate % 16 || d.headdim > 128 || d.dstate > 16 * CH_NW) return false;
  const i64 LM = d.chunk_len * d.mimo_rank;
  if (LM % 16) return false;
  // byte offsets inside one batch element are 32-bit (buffer loads, int row
  // offsets): rows of x/dy and B/C, the stored states
  const i64 esz = d.dtype == SSMVJP_BF16 ? 2 : 4, nc = cdiv(d.seqlen, d.chunk_len);
  if (d.seqlen * d.mimo_rank * d.nheads * d.headdim * esz >= (1ll << 31) ||
      d.seqlen * d.mimo_rank * d.ngroups * d.dstate * esz >= (1ll << 31) ||
      nc * d.nheads * d.headdim * d.dstate * esz >= (1ll << 31) || nc * d.nheads * 3 * 64 * 4 >= (1ll << 31))
    return false;
  if ((d.headdim / 16) * (scan_nb(d) / 16) > SCAN_TILES) return false;
  if (LM > SCAN_SB) return ssd_blocked_supported(d);  // long fused chunks: row-blocked kernels
  return LM <= MAXRB * 16 && grads_lds_bytes(d) <= 160 * 1024;
}

SsdPlan ssd_plan(const ssmvjp_ssd_desc& d) {
  SsdPlan p{};
  p.nc = cdiv(d.seqlen, d.chunk_len);
  p.LM = d.chunk_len * d.mimo_rank;
  p.hsplit = p.LM > SCAN_SB ? 1 : pick_hsplit(d, p.nc);  // the row-blocked path loops over all heads
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
  const bool blocked = p.LM > SCAN_SB;
  p.off_rowv = carve(blocked ? d.batch * p.nc * d.nheads * RV_N * p.LM * 4 : 0);
  p.off_dend = carve(blocked ? d.batch * p.nc * d.nheads * 4 : 0);
  p.off_csv = carve(d.batch * p.nc * d.nheads * 3 * 64 * 4);
  p.off_dA = carve(d.batch * p.nc * d.nheads * 4);
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
  a.rowv = (float*)(ws + plan.off_rowv);
  a.dend = (float*)(ws + plan.off_dend);
  a.csv = (float*)(ws + plan.off_csv);
  a.dA_part = ptr.dA && !a.raw ? (float*)(ws + plan.off_dA) : nullptr;
  return a;
}

template <typename T>
static size_t states_lds(const SsdArgs& a, int NB) {
  const int PAD = scan_pad<T>();
  const size_t SB = a.LM < SCAN_SB ? a.LM : SCAN_SB;
  return 2 * sizeof(T) * SB * ((a.P + PAD) + (NB + PAD));  // two buffers
}

template <typename T>
static size_t grads_lds(const SsdArgs& a) {
  const bool bf = sizeof(T) == 2;
  const int PAD = bf ? 8 : 0;
  return sizeof(float) * ((size_t)a.LM * (a.LM + 4) + (bf ? 2 : 1) * PB_N * 8 * 64) +
         sizeof(T) * (2 * (size_t)a.LM * (a.N + PAD) + 2 * (size_t)a.LM * (a.P + PAD) + (bf ? 2 : 1) * (size_t)a.P * a.N +
                      (bf ? 10 * 256 : 0));
}

// the Mamba-2 chunked workload shape and the rank-4 MIMO workload shape get
// compile-time sizes
static bool workload_shape(const SsdArgs& a) { return a.P == 64 && a.N == 128 && a.L == 64 && a.M == 1; }
static bool mimo_shape(const SsdArgs& a) { return a.P == 64 && a.N == 128 && a.L == 64 && a.M == 4; }

template <typename T>
static void launch_states_t(const SsdArgs& a, hipStream_t stream, int NB) {
  const i64 nw = a.b * a.nc * a.H;  // one wave per (batch, chunk, head)
  if (nw > 0)
    hipLaunchKernelGGL(ssd_chunk_scalars_kernel, dim3((unsigned)cdiv(nw, 4)), dim3(256), 0, stream, a);
  const i64 grid1 = a.b * a.H * 2 * (a.N / NB);
  if (workload_shape(a) && NB == 128)
    hipLaunchKernelGGL((ssd_state_scan_kernel<T, 64, 128, 64, 1>), dim3((unsigned)grid1), dim3(SCAN_NTH),
                       states_lds<T>(a, NB), stream, a, NB);
  else if (mimo_shape(a) && NB == 64)
    hipLaunchKernelGGL((ssd_state_scan_kernel<T, 64, 64, 64, 4>), dim3((unsigned)grid1), dim3(SCAN_NTH),
                       states_lds<T>(a, NB), stream, a, NB);
  else
    hipLaunchKernelGGL((ssd_state_scan_kernel<T, 0, 0, 0, 0>), dim3((unsigned)grid1), dim3(SCAN_NTH),
                       states_lds<T>(a, NB), stream, a, NB);
}

template <typename T>
static void launch_grads_t(const SsdArgs& a, hipStream_t stream) {
  if (a.T == 0) return;
  if (a.LM > SCAN_SB) {
    launch_ssd_blocked_grads(a, sizeof(T) == 2, stream);
    return;
  }
  const i64 grid2 = a.b * a.nc * a.G * a.hsplit;
  if (sizeof(T) == 2 && workload_shape(a))
    launch_ssd_chunk16(a, stream);  // 16 waves, bf16 at P = 64, N = 128, L = 64, M = 1
  else if (workload_shape(a) && a.dA_part)
    hipLaunchKernelGGL((ssd_chunk_bwd_kernel<T, 64, 128, 64, 1, true>), dim3((unsigned)grid2), dim3(CH_NTH),
                       grads_lds<T>(a), stream, a);
  else if (workload_shape(a))
    hipLaunchKernelGGL((ssd_chunk_bwd_kernel<T, 64, 128, 64, 1, false>), dim3((unsigned)grid2), dim3(CH_NTH),
                       grads_lds<T>(a), stream, a);
  else if (a.dA_part)
    hipLaunchKernelGGL((ssd_chunk_bwd_kernel<T, 0, 0, 0, 0, true>), dim3((unsigned)grid2), dim3(CH_NTH),
                       grads_lds<T>(a), stream, a);
  else
    hipLaunchKernelGGL((ssd_chunk_bwd_kernel<T, 0, 0, 0, 0, false>), dim3((unsigned)grid2), dim3(CH_NTH),
                       grads_lds<T>(a), stream, a);
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
  if ((stages & SSD_STAGE_GRADS) && ptr.dA && d.form == SSMVJP_FORM_MAMBA2)
    launch_dA_reduce((const float*)((char*)ptr.workspace + plan.off_dA), d.batch * plan.nc, d.nheads, ptr.dA, stream);
  return hipGetLastError();
}

}  // namespace ssmvjp
