// ssd_blocked.hip -- per-chunk backward of the chunked SSD for long fused
// chunks (L*M > 64 fused rows, e.g. the rank-4 MIMO form with L = 64), after
// burn-mamba "combined_backward.rs": the same quantities as the chunk kernel of
// ssd_chunk.hip (BLUE, ORANGE, the K3 / K2 / K1 backwards and the Mamba-2
// chain), organised for chunks whose [L*M x L*M] matrices do not fit in LDS.
//
// The chunk's fused rows r = l*M + m are cut into 64-row blocks.  The causal
// intra-chunk terms couple a target block (rows t) with every source block
// (rows s) at or before it; those lower-triangular block pairs are walked by
// two kinds of workgroup, one per (batch, chunk, group, block) each, with the
// heads of the group in a loop (ascending, so group sums are deterministic):
//
//   source role (block = s): per head, the K3 backward (d_dv = dS_{c+1}.B^T,
//     dB_k3 = decayed v^T.dS_{c+1}, d_decay), then for every target block
//     t >= s the recomputed CB and G1 = dy.v^T tiles, the decay, d_cb and
//     w = CB * decay, giving d_v_or += w^T.dy, dB_k2 += d_cb^T.C and the
//     column sums of d_cb * CB.  Stores dx (d_v) per head and dB summed over
//     the group's heads.
//   target role (block = t): per head, BLUE (dC_blue = exp(cumA) dy.S_c and
//     its row sums against C), then for every source block s <= t the same
//     G1 and d_cb (recomputed, transposed), giving dC_k2 += d_cb.B, and the
//     row sums of d_cb * CB.  Stores dC summed over the group's heads.
//     Those row sums need no CB tiles when a group has one head: since
//     CB = C.B^T and dC_k2 = d_cb.B, sum_s d_cb[t,s] CB[t,s] equals
//     sum_n C[t,n] dC_k2[t,n], so BLUE's and ORANGE's row sums are read off
//     together from the finished dC tiles (sum_n C dC), the same refactor as
//     BLUE's own.  With several heads per group the dC tiles hold the sum over
//     heads, and the per-head row sums come from the recomputed CB tiles.
//
// Each wave owns one 16-row tile of its block (an s tile or a t tile), so the
// d_cb and w tiles it computes are already in the MFMA operand layout that its
// next products need (the output layout of a tile is the operand layout of the
// tile with its row index as contraction index): nothing goes through LDS but
// the staged input rows and states.  The per-row partial sums of d_cumA go to
// a small buffer; a third kernel, one wave per (batch, chunk, head), adds them
// up, runs the K1 suffix sum and the chain to d_dt (or d_da).
//
// A workgroup's start-up loads (its own rows, the head's state and step
// scalars, the first pair's rows) are issued together, so their latencies
// overlap; each later pair's rows are prefetched into registers during the
// previous pair.  The transposed-read products are scheduled with their reads
// issued ahead of the MFMAs that consume them.
//
// Products accumulate in float32; with bf16 storage the MFMA operands are bf16
// (inputs as given, d_cb and w rounded once).
#include "ssd_common.cuh"

namespace ssmvjp {

constexpr int BK_NW = 4;             // waves per workgroup: one 16-row tile of the 64-row block each
constexpr int BK_NTH = 64 * BK_NW;
constexpr int BK_R = 64;             // fused rows per block
constexpr int BK_TMAX = 8;           // P / 16 and N / 16 at most

// Swizzled LDS layouts (the bf16 P = 64, N = 128 instantiation): the staged
// input tiles are XOR-swizzled (xsw_off), and the state tiles keep MFMA output
// order with each 128-byte quarter of a 512-byte tile rotated by 32 bytes per
// quarter, so that the transposed read, which takes 8 bytes at the same offset
// of every quarter, hits distinct banks.
__device__ __forceinline__ int bk_qsw(int byte) { return (byte & ~127) | ((byte + 32 * ((byte >> 7) & 3)) & 127); }

template <bool SWZ, typename T>
__device__ __forceinline__ Frag<T> bk_colk(const T* t, int pitch, int c0, int k0, int lane) {
  if constexpr (SWZ) {
    return ld_colk_xs(t, pitch, c0, k0, lane);
  } else {
    return ld_colk(t, pitch, c0, k0, lane);
  }
}
template <bool SWZ, typename T>
__device__ __forceinline__ Frag<T> bk_rowk(const T* t, int pitch, int k0, int c0, int lane) {
  if constexpr (SWZ) {
    return ld_rowk_xs(t, pitch, k0, c0, lane);
  } else {
    return ld_rowk(t, pitch, k0, c0, lane);
  }
}
template <bool SWZ, typename T>
__device__ __forceinline__ Frag<T> bk_ntv(const T* t, int lane) {
  if constexpr (SWZ) {
    Frag<T> f;
    f.v = *(const s16x4*)((const char*)t + bk_qsw(8 * lane));
    return f;
  } else {
    return ld_ntv(t, lane);
  }
}
template <bool SWZ, typename T>
__device__ __forceinline__ Frag<T> bk_ntv_t(const T* t, int lane) {
  if constexpr (SWZ) {
    const int m = lane & 15;
    return lds_tr_b16((const T*)((const char*)t + bk_qsw(8 * ((m & 3) * 16 + 4 * (lane >> 4) + (m >> 2)))));
  } else {
    return ld_ntv_t(t, lane);
  }
}
// a 16-byte chunk (columns col .. col+E16-1 of row `row`) into a staged tile
template <bool SWZ, typename T>
__device__ __forceinline__ void bk_put16(T* dst, int pitch, int row, int col, const u32x4& u) {
  if constexpr (SWZ) {
    st16_xs(dst, pitch, row, col, u);
  } else {
    *(u32x4*)(dst + row * pitch + col) = u;
  }
}
// byte offset of the 16-byte chunk idx of a state in its staged layout
template <bool SWZ>
__device__ __forceinline__ int bk_state_off(int idx) {
  return SWZ ? (idx >> 5) * 512 + bk_qsw((idx & 31) * 16) : idx * 16;
}

// 64 rows of a [rows][stride] tensor (ncol columns from src) into LDS rows of
// `pitch` elements; rows at or past `valid` read zeros (range-checked loads)
template <bool SWZ, typename T>
__device__ __forceinline__ void bk_stage_rows(T* dst, int pitch, const T* src, i64 stride, int ncol, int valid,
                                              int tid) {
  constexpr int E16 = 16 / sizeof(T);
  const int cpr = ncol / E16;
  const brsrc r = make_rsrc(src, valid > 0 ? (unsigned)(((valid - 1) * stride + ncol) * sizeof(T)) : 0u);
  for (int idx = tid; idx < BK_R * cpr; idx += BK_NTH) {
    const int row = idx / cpr, col = (idx % cpr) * E16;
    bk_put16<SWZ>(dst, pitch, row, col, bload16(r, (unsigned)((row * stride + col) * sizeof(T))));
  }
}
// one [P x N] state in native tile order
template <bool SWZ, typename T>
__device__ __forceinline__ void bk_stage_state(T* dst, const T* src, int PN, int tid) {
  constexpr int E16 = 16 / sizeof(T);
  const brsrc r = make_rsrc(src, (unsigned)(PN * sizeof(T)));
  for (int idx = tid; idx < PN / E16; idx += BK_NTH)
    *(u32x4*)((char*)dst + bk_state_off<SWZ>(idx)) = bload16(r, (unsigned)idx * 16u);
}

// 64 rows (ncol columns) or one [P x N] state as 16-byte chunks, loaded into
// registers now and written into LDS later, so that a workgroup's start-up
// loads are all in flight together (compile-time shapes: the register arrays
// are sized exactly)
template <int NR, typename T>
__device__ __forceinline__ void bk_load_rows(u32x4 (&r)[NR], const T* src, i64 stride, int ncol, int valid, int tid) {
  constexpr int E16 = 16 / sizeof(T);
  const int cpr = ncol / E16;
  const brsrc rs = make_rsrc(src, valid > 0 ? (unsigned)(((valid - 1) * stride + ncol) * sizeof(T)) : 0u);
#pragma unroll
  for (int it = 0; it < NR; ++it) {
    const int idx = tid + it * BK_NTH, row = idx / cpr, col = (idx % cpr) * E16;
    r[it] = bload16(rs, idx < BK_R * cpr ? (unsigned)((row * stride + col) * sizeof(T)) : BUF_OOB);
  }
}
template <bool SWZ, int NR, typename T>
__device__ __forceinline__ void bk_put_rows(T* dst, int pitch, const u32x4 (&r)[NR], int ncol, int tid) {
  constexpr int E16 = 16 / sizeof(T);
  const int cpr = ncol / E16;
#pragma unroll
  for (int it = 0; it < NR; ++it) {
    const int idx = tid + it * BK_NTH;
    if (idx < BK_R * cpr) bk_put16<SWZ>(dst, pitch, idx / cpr, (idx % cpr) * E16, r[it]);
  }
}
template <int NR, typename T>
__device__ __forceinline__ void bk_load_state(u32x4 (&r)[NR], const T* src, int PN, int tid) {
  const brsrc rs = make_rsrc(src, (unsigned)(PN * sizeof(T)));
#pragma unroll
  for (int it = 0; it < NR; ++it) r[it] = bload16(rs, (unsigned)(tid + it * BK_NTH) * 16u);
}
template <bool SWZ, int NR, typename T>
__device__ __forceinline__ void bk_put_state(T* dst, const u32x4 (&r)[NR], int PN, int tid) {
  constexpr int E16 = 16 / sizeof(T);
#pragma unroll
  for (int it = 0; it < NR; ++it) {
    const int idx = tid + it * BK_NTH;
    if (idx < PN / E16) *(u32x4*)((char*)dst + bk_state_off<SWZ>(idx)) = r[it];
  }
}

// Scheduling pattern for a run of n MFMAs whose B operands are n LDS reads
// (one each): the first `ahead` reads, then one MFMA per read, so that reads
// stay in flight under the products instead of each product waiting for its
// own read.
template <int n, int ahead>
__device__ __forceinline__ void bk_pipeline_reads() {
  __builtin_amdgcn_sched_group_barrier(0x100, ahead, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < n - ahead; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, ahead, 0);
}

// bf16: two workgroups per CU, at most 256 registers (VGPR + AGPR) per lane.
// CP, CN, CM: compile-time P, N and rank M (0: from the arguments); ONEH: one
// head per group (the target role's row sums from its dC tiles).
template <typename T, int CP, int CN, int CM, bool ONEH>
__global__ void __launch_bounds__(BK_NTH) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1))) ssd_blocked_bwd_kernel(SsdArgs a) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr bool SWZ = BF && CP && CN && CP % 64 == 0 && CN % 64 == 0;  // swizzled, unpadded tiles
  constexpr int PAD = SWZ ? 0 : (BF ? 8 : 4);
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int P = CP ? CP : (int)a.P, N = CN ? CN : (int)a.N, M = CM ? CM : (int)a.M, L = (int)a.L;
  // with a compile-time rank that is a multiple of 4, the 4 rows a lane holds
  // in a 16x16 tile (4q .. 4q+3) belong to one step: one decay per tile and lane
  constexpr bool STEP4 = CM != 0 && CM % 4 == 0;
  // with compile-time P and N, a head's loads (scalars, own rows, state) are
  // issued together into registers; otherwise they are staged one by one
  constexpr bool MERGE = CP != 0 && CN != 0;
  const int PT = P / 16, NT = N / 16, LM = (int)a.LM, nblk = LM / BK_R;
  const int LDN = N + PAD, LDP = P + PAD, PN = P * N;
  T* Bs = (T*)smem_raw;    // [64][LDN] B rows of a source block
  T* Cs = Bs + BK_R * LDN;  // [64][LDN] C rows of a target block
  T* xs = Cs + BK_R * LDN;  // [64][LDP] x / v rows of a source block (one head)
  T* dys = xs + BK_R * LDP; // [64][LDP] dy rows of a target block (one head)
  T* STs = dys + BK_R * LDP; // [P*N] dS_{c+1} (source role) or S_c (target role), native tiles
  float* red = (float*)(STs + PN);  // [BK_NW] cross-wave partial sums

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, q = lane >> 4,
            r16 = lane & 15;
  __builtin_assume(w >= 0 && w < BK_NW);
  __builtin_assume(tid >= 0 && tid < BK_NTH);
  // XCD-aware order: consecutive workgroups of one (batch, chunk, group) share
  // their input rows, so they are given ids that land on the same XCD (ids are
  // dealt to the 8 XCDs round robin)
  // (32-bit unsigned arithmetic: the grid and its factors fit, and 64-bit
  // division is a long scalar routine)
  unsigned id = blockIdx.x;
  if (gridDim.x % 8 == 0) id = (id % 8) * (gridDim.x / 8) + id / 8;
  // (a power-of-two factor is a shift and a mask)
  auto divmod = [](unsigned& n, unsigned d) -> unsigned {
    unsigned r;
    if ((d & (d - 1u)) == 0u) {
      r = n & (d - 1u);
      n >>= __builtin_ctz(d);
    } else {
      const unsigned q = n / d;
      r = n - q * d;
      n = q;
    }
    return r;
  };
  const int blk = (int)divmod(id, (unsigned)nblk);
  const int role = (int)(id & 1u);  // 0 source block, 1 target block
  id >>= 1;
  const i64 g = (i64)divmod(id, (unsigned)a.G);
  const i64 c = (i64)divmod(id, (unsigned)a.nc), bi = (i64)id;
  const i64 t0 = c * L;
  const int Lc = (int)((a.T - t0) < L ? (a.T - t0) : L);
  const int vrows = Lc * M;  // valid fused rows of this chunk
  auto valid_in = [&](int b) { const int v = vrows - b * BK_R; return v < 0 ? 0 : (v > BK_R ? BK_R : v); };
  const unsigned esz = sizeof(T);
  const i64 xstr = a.H * P, bstr = a.G * N;  // fused-row strides
  const T* Bg = (const T*)a.B + ix_bc(a, bi, t0, 0, g, 0);
  const T* Cg = (const T*)a.C + ix_bc(a, bi, t0, 0, g, 0);
  const i64 xrow0 = ix_xv(a, bi, t0, 0, 0, 0);  // x / dy / dx offset of fused row 0, head 0
  auto scalars = [&](i64 h) { return load_scalars(a, bi, c, h, lane); };
  float* rowv_c = a.rowv + (bi * a.nc + c) * a.H * RV_N * LM;
  auto tile_off = [&](int pt, int nt) { return (pt * NT + nt) * 256; };
  // this lane's column: fused row blk*64 + 16w + r16 of the wave's tile
  const int col = blk * BK_R + 16 * w + r16;
  const int l_col = col / M;

  // ---- register prefetch of one block pair's staged rows: 64 rows of a B or C
  // tensor (N wide) and 64 rows of an x or dy tensor (P wide, one head).
  // Branch-free range-checked loads, issued one block pair ahead. ----
  constexpr int E16 = 16 / sizeof(T);
  constexpr int MAXN = CN ? (BK_R * CN / E16 + BK_NTH - 1) / BK_NTH : BK_R * 128 / E16 / BK_NTH;
  constexpr int MAXP = CP ? (BK_R * CP / E16 + BK_NTH - 1) / BK_NTH : BK_R * 128 / E16 / BK_NTH;
  constexpr int MAXS = MERGE ? (CP * CN / E16 + BK_NTH - 1) / BK_NTH : 1;
  u32x4 pn[MAXN], pp[MAXP];
  const int cpn = N / E16, cpp = P / E16;  // 16-byte chunks per row
  auto issue = [&](const T* srcN, const T* srcP, int valid) {
    const brsrc rn = make_rsrc(srcN, valid > 0 ? (unsigned)(((valid - 1) * bstr + N) * esz) : 0u);
    const brsrc rp = make_rsrc(srcP, valid > 0 ? (unsigned)(((valid - 1) * xstr + P) * esz) : 0u);
#pragma unroll
    for (int it = 0; it < MAXN; ++it) {
      const int idx = tid + it * BK_NTH, row = idx / cpn, cc = (idx % cpn) * E16;
      pn[it] = bload16(rn, idx < BK_R * cpn ? (unsigned)((row * bstr + cc) * esz) : BUF_OOB);
    }
#pragma unroll
    for (int it = 0; it < MAXP; ++it) {
      const int idx = tid + it * BK_NTH, row = idx / cpp, cc = (idx % cpp) * E16;
      pp[it] = bload16(rp, idx < BK_R * cpp ? (unsigned)((row * xstr + cc) * esz) : BUF_OOB);
    }
  };
  auto commit = [&](T* dstN, T* dstP) {
#pragma unroll
    for (int it = 0; it < MAXN; ++it) {
      const int idx = tid + it * BK_NTH;
      if (idx < BK_R * cpn) bk_put16<SWZ>(dstN, LDN, idx / cpn, (idx % cpn) * E16, pn[it]);
    }
#pragma unroll
    for (int it = 0; it < MAXP; ++it) {
      const int idx = tid + it * BK_NTH;
      if (idx < BK_R * cpp) bk_put16<SWZ>(dstP, LDP, idx / cpp, (idx % cpp) * E16, pp[it]);
    }
  };

  if (role == 0) {
    // ======================= source block s = blk =========================
    // steps: (head hh, target block tb) for tb = blk .. nblk-1, heads in order
    const int nT = nblk - blk;
    const int nsteps = (int)a.hpg * nT;
    auto issue_step = [&](int hh, int tb) {
      hh = __builtin_amdgcn_readfirstlane(hh);
      tb = __builtin_amdgcn_readfirstlane(tb);
      const i64 h = g * a.hpg + hh;
      issue(Cg + (i64)tb * BK_R * bstr, (const T*)a.dy + xrow0 + (i64)tb * BK_R * xstr + h * P, valid_in(tb));
    };
    f32x4 dBT[BK_TMAX];  // dB^T tiles (rows n, columns s), summed over the group's heads
#pragma unroll
    for (int i = 0; i < BK_TMAX; ++i) dBT[i] = zero4();
    f32x4 dvT[BK_TMAX];  // d_v^T tiles (rows p, columns s) of the current head
    float s1 = 0.0f, ocol = 0.0f, cum_s = 0.0f, delta_s = 0.0f;
    ChunkScalars cs = {0.f, 0.f, 0.f, 0.f};
    u32x4 rown[MAXN];  // the block's own B rows, written with the first head's rows
    if constexpr (MERGE)
      bk_load_rows(rown, Bg + (i64)blk * BK_R * bstr, bstr, N, valid_in(blk), tid);
    else
      bk_stage_rows<SWZ>(Bs, LDN, Bg + (i64)blk * BK_R * bstr, bstr, N, valid_in(blk), tid);
    issue_step(0, blk);
    // step k = (head hh, target block tb), counted without divisions
    for (int k = 0, hh = 0, tb = blk; k < nsteps; ++k, tb = (tb + 1 == nblk) ? blk : tb + 1, hh += (tb == blk)) {
      const i64 h = g * a.hpg + hh;
      if (tb == blk) {
        // ---- a new head: its scalars, x / v rows and dS_{c+1}; then the K3 backward ----
        const T* xg = (const T*)a.xv + xrow0 + (i64)blk * BK_R * xstr + h * P;
        const T* dSg = (const T*)a.dS + ((bi * a.nc + c) * a.H + h) * (i64)PN;
        u32x4 rx[MAXP], rst[MAXS];
        if constexpr (MERGE) {  // all of the head's loads in flight together
          ChunkScalars csn = issue_scalars(a, bi, c, h, lane);
          bk_load_rows(rx, xg, xstr, P, valid_in(blk), tid);
          bk_load_state(rst, dSg, PN, tid);
          cs = finish_scalars(csn);
        } else {
          cs = scalars(h);
        }
        cum_s = __shfl(cs.cum, l_col & 63, 64);
        delta_s = __shfl(cs.delta, l_col & 63, 64);
        const float edec = exp_hw(cs.end - cum_s), xcol = delta_s * edec;
        __syncthreads();  // the previous head is done with xs / STs
        if constexpr (MERGE) {
          if (k == 0) bk_put_rows<SWZ>(Bs, LDN, rown, N, tid);
          bk_put_rows<SWZ>(xs, LDP, rx, P, tid);
          bk_put_state<SWZ>(STs, rst, PN, tid);
        } else {
          bk_stage_rows<SWZ>(xs, LDP, xg, xstr, P, valid_in(blk), tid);
          bk_stage_state<SWZ>(STs, dSg, PN, tid);
        }
        __syncthreads();
        // K3: d_dv^T = dS_{c+1}.B^T (rows p, columns s); dB_k3^T += dS^T . (xcol v)^T
        s1 = 0.0f;
        ocol = 0.0f;
#pragma unroll
        for (int pt = 0; pt < BK_TMAX; ++pt) {
          dvT[pt] = zero4();
          if (pt >= PT) continue;
          f32x4 acc = zero4();
          for (int kb = 0; kb < NT; ++kb)
            mma(acc, bk_ntv_t<SWZ>(STs + tile_off(pt, kb), lane), bk_colk<SWZ>(Bs, LDN, 16 * w, 16 * kb, lane));
          float xv[4];
          frag_get(bk_colk<SWZ>(xs, LDP, 16 * w, 16 * pt, lane), xv);  // x[s][p .. p+3], p = 16 pt + 4q
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            s1 += acc[j] * xv[j];  // d_decay / delta = sum_p d_dv . x
            dvT[pt][j] = acc[j] * edec;
          }
        }
#pragma unroll
        for (int nt = 0; nt < BK_TMAX; ++nt) {
          if (nt >= NT) continue;
          f32x4 acc = zero4();
          for (int kb = 0; kb < PT; ++kb)
            mma(acc, bk_ntv<SWZ>(STs + tile_off(kb, nt), lane), bk_colk<SWZ>(xs, LDP, 16 * w, 16 * kb, lane));
#pragma unroll
          for (int j = 0; j < 4; ++j) dBT[nt][j] += acc[j] * xcol;
        }
      }

      // ---- ORANGE and K2 for the pair (t block tb, s block blk) ----
      __syncthreads();  // the previous pair is done with Cs / dys
      commit(Cs, dys);
      {  // the next step's rows; the last step reloads its own, which keeps the issue unconditional
        const bool more = k + 1 < nsteps, wrap = tb + 1 == nblk;
        issue_step(more && wrap ? hh + 1 : hh, more ? (wrap ? blk : tb + 1) : tb);
      }
      __syncthreads();
      Frag<T> wf[4], df[4];  // w and d_cb tiles (rows t, columns s): operands with k = t
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4 cb = zero4(), g1 = zero4();
        for (int kb = 0; kb < NT; ++kb)
          mma(cb, bk_colk<SWZ>(Cs, LDN, 16 * tt, 16 * kb, lane), bk_colk<SWZ>(Bs, LDN, 16 * w, 16 * kb, lane));
        for (int kb = 0; kb < PT; ++kb)
          mma(g1, bk_colk<SWZ>(dys, LDP, 16 * tt, 16 * kb, lane), bk_colk<SWZ>(xs, LDP, 16 * w, 16 * kb, lane));
        float wv[4], dv[4];
        float dec4 = 0.0f;
        if constexpr (STEP4) {
          const int lt = (tb * BK_R + 16 * tt + 4 * q) / CM;
          const float ct = __shfl(cs.cum, lt & 63, 64);  // every lane takes part in the shuffle
          dec4 = (l_col <= lt && lt < Lc) ? exp_hw(ct - cum_s) : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float dec = dec4;
          if constexpr (!STEP4) {
            const int lt = (tb * BK_R + 16 * tt + 4 * q + j) / M;
            const float ct = __shfl(cs.cum, lt & 63, 64);  // every lane takes part in the shuffle
            dec = (l_col <= lt && lt < Lc) ? exp_hw(ct - cum_s) : 0.0f;
          }
          const float dcb = g1[j] * delta_s * dec;  // d_w = dy.v^T with v = delta x (delta = 1 for RAW)
          ocol += dcb * cb[j];
          wv[j] = cb[j] * dec;
          dv[j] = dcb;
        }
        wf[tt] = frag_make<T>(wv);
        df[tt] = frag_make<T>(dv);
      }
      if constexpr (CP && CN) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int pt = 0; pt < BK_TMAX; ++pt) {  // d_v_or^T += dy^T . w
        if (pt >= PT) continue;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) mma(dvT[pt], bk_rowk<SWZ>(dys, LDP, 16 * tt, 16 * pt, lane), wf[tt]);
      }
#pragma unroll
      for (int nt = 0; nt < BK_TMAX; ++nt) {  // dB_k2^T += C^T . d_cb
        if (nt >= NT) continue;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) mma(dBT[nt], bk_rowk<SWZ>(Cs, LDN, 16 * tt, 16 * nt, lane), df[tt]);
      }
      if constexpr (CP && CN) bk_pipeline_reads<4 * (CP + CN) / 16, 8>();

      if (tb == nblk - 1) {
        // ---- the head's outputs: dx (= d_v, times delta for Mamba-2), the column sums ----
        float dvx = 0.0f;
        const brsrc rdx = make_rsrc((T*)a.dxv + xrow0 + (i64)blk * BK_R * xstr + h * P,
                                    valid_in(blk) > 0 ? (unsigned)(((valid_in(blk) - 1) * xstr + P) * esz) : 0u);
#pragma unroll
        for (int pt = 0; pt < BK_TMAX; ++pt) {
          if (pt >= PT) continue;
          float xv[4];
          frag_get(bk_colk<SWZ>(xs, LDP, 16 * w, 16 * pt, lane), xv);
          f32x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            dvx += dvT[pt][j] * xv[j];
            o[j] = a.raw ? dvT[pt][j] : dvT[pt][j] * delta_s;
          }
          bstore4(rdx, (unsigned)(((16 * w + r16) * xstr + 16 * pt + 4 * q) * esz), o, (const T*)0);
        }
        const float s1w = sum4q(s1) * delta_s, ocw = sum4q(ocol), dvxw = sum4q(dvx);
        float* rv = rowv_c + h * RV_N * LM;
        if (q == 0) {
          rv[RV_DEC * LM + col] = s1w;
          rv[RV_OCOL * LM + col] = ocw;
          rv[RV_DVX * LM + col] = dvxw;
        }
      }
    }
    // dB (rows s, 4 consecutive n per lane), summed over the group's heads
    const brsrc rdB = make_rsrc((T*)a.dB + ix_bc(a, bi, t0, 0, g, 0) + (i64)blk * BK_R * bstr,
                                valid_in(blk) > 0 ? (unsigned)(((valid_in(blk) - 1) * bstr + N) * esz) : 0u);
#pragma unroll
    for (int nt = 0; nt < BK_TMAX; ++nt) {
      if (nt >= NT) continue;
      bstore4(rdB, (unsigned)(((16 * w + r16) * bstr + 16 * nt + 4 * q) * esz), dBT[nt], (const T*)0);
    }
  } else {
    // ======================= target block t = blk =========================
    // steps: (head hh, source block sb) for sb = 0 .. blk, heads in order
    const int nS = blk + 1;
    const int nsteps = (int)a.hpg * nS;
    auto issue_step = [&](int hh, int sb) {
      hh = __builtin_amdgcn_readfirstlane(hh);
      sb = __builtin_amdgcn_readfirstlane(sb);
      const i64 h = g * a.hpg + hh;
      issue(Bg + (i64)sb * BK_R * bstr, (const T*)a.xv + xrow0 + (i64)sb * BK_R * xstr + h * P, valid_in(sb));
    };
    f32x4 dCT[BK_TMAX];  // dC^T tiles (rows n, columns t), summed over the group's heads
#pragma unroll
    for (int i = 0; i < BK_TMAX; ++i) dCT[i] = zero4();
    float blue = 0.0f, orow = 0.0f, cum_t = 0.0f;
    ChunkScalars cs = {0.f, 0.f, 0.f, 0.f};
    u32x4 rown[MAXN];  // the block's own C rows, written with the first head's rows
    if constexpr (MERGE)
      bk_load_rows(rown, Cg + (i64)blk * BK_R * bstr, bstr, N, valid_in(blk), tid);
    else
      bk_stage_rows<SWZ>(Cs, LDN, Cg + (i64)blk * BK_R * bstr, bstr, N, valid_in(blk), tid);
    issue_step(0, 0);
    // step k = (head hh, source block sb), counted without divisions
    for (int k = 0, hh = 0, sb = 0; k < nsteps; ++k, sb = (sb == blk) ? 0 : sb + 1, hh += (sb == 0)) {
      const i64 h = g * a.hpg + hh;
      if (sb == 0) {
        // ---- a new head: its scalars, dy rows and S_c; d_end; BLUE ----
        const T* dyg = (const T*)a.dy + xrow0 + (i64)blk * BK_R * xstr + h * P;
        const T* Sg = (const T*)a.S + ((bi * a.nc + c) * a.H + h) * (i64)PN;
        const T* dSg = (const T*)a.dS + ((bi * a.nc + c) * a.H + h) * (i64)PN;
        u32x4 rdy[MAXP], rst[MAXS], rds[MAXS];
        if constexpr (MERGE) {  // all of the head's loads in flight together (dS_{c+1} only for d_end)
          ChunkScalars csn = issue_scalars(a, bi, c, h, lane);
          bk_load_rows(rdy, dyg, xstr, P, valid_in(blk), tid);
          bk_load_state(rst, Sg, PN, tid);
          if (blk == 0) bk_load_state(rds, dSg, PN, tid);
          cs = finish_scalars(csn);
        } else {
          cs = scalars(h);
        }
        cum_t = __shfl(cs.cum, l_col & 63, 64);
        const float ecol = exp_hw(cum_t);
        __syncthreads();  // the previous head is done with dys / STs
        if constexpr (MERGE) {
          if (k == 0) bk_put_rows<SWZ>(Cs, LDN, rown, N, tid);
          bk_put_rows<SWZ>(dys, LDP, rdy, P, tid);
          bk_put_state<SWZ>(STs, rst, PN, tid);
        } else {
          bk_stage_rows<SWZ>(dys, LDP, dyg, xstr, P, valid_in(blk), tid);
          bk_stage_state<SWZ>(STs, Sg, PN, tid);
        }
        __syncthreads();
        if (blk == 0) {  // d_end = sum_{p,n} S_c * dS_{c+1}, once per chunk and head
          float part = 0.0f;
          auto dot16 = [&](const u32x4& u, const u32x4& v) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if constexpr (BF) {
                part += __uint_as_float(u[e] << 16) * __uint_as_float(v[e] << 16);
                part += __uint_as_float(u[e] & 0xffff0000u) * __uint_as_float(v[e] & 0xffff0000u);
              } else {
                part += __uint_as_float(u[e]) * __uint_as_float(v[e]);
              }
            }
          };
          if constexpr (MERGE) {
#pragma unroll
            for (int it = 0; it < MAXS; ++it)
              if (tid + it * BK_NTH < PN / E16) dot16(rds[it], rst[it]);
          } else {
            const brsrc rdS = make_rsrc(dSg, (unsigned)PN * esz);
            for (int idx = tid; idx < PN / E16; idx += BK_NTH)
              dot16(bload16(rdS, (unsigned)idx * 16u), *(const u32x4*)((const char*)STs + bk_state_off<SWZ>(idx)));
          }
          part = wave_sum(part);
          if (lane == 0) red[w] = part;
          __syncthreads();
          if (tid == 0) {
            float sum = 0.0f;
            for (int kw = 0; kw < BK_NW; ++kw) sum += red[kw];
            a.dend[(bi * a.nc + c) * a.H + h] = sum;
          }
        }
        // BLUE: dC_blue^T = S_c^T . (dy * exp(cumA))^T ; its row sums against C
        blue = 0.0f;
        orow = 0.0f;
#pragma unroll
        for (int nt = 0; nt < BK_TMAX; ++nt) {
          if (nt >= NT) continue;
          f32x4 acc = zero4();
          for (int kb = 0; kb < PT; ++kb)  // A: rows n, k = p (native tile); B: k = p, columns t
            mma(acc, bk_ntv<SWZ>(STs + tile_off(kb, nt), lane), bk_colk<SWZ>(dys, LDP, 16 * w, 16 * kb, lane));
          if constexpr (ONEH) {
#pragma unroll
            for (int j = 0; j < 4; ++j) dCT[nt][j] += acc[j] * ecol;
          } else {
            float cv[4];
            frag_get(bk_colk<SWZ>(Cs, LDN, 16 * w, 16 * nt, lane), cv);  // C[t][n .. n+3], n = 16 nt + 4q
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float val = acc[j] * ecol;
              dCT[nt][j] += val;
              blue += cv[j] * val;
            }
          }
        }
      }

      // ---- ORANGE row sums and K2 for the pair (t block blk, s block sb), transposed tiles ----
      __syncthreads();  // the previous pair is done with Bs / xs
      commit(Bs, xs);
      {  // the next step's rows; the last step reloads its own, which keeps the issue unconditional
        const bool more = k + 1 < nsteps, wrap = sb == blk;
        issue_step(more && wrap ? hh + 1 : hh, more ? (wrap ? 0 : sb + 1) : sb);
      }
      __syncthreads();
      Frag<T> df[4];  // d_cb^T tiles (rows s, columns t): operands with k = s
#pragma unroll
      for (int ss = 0; ss < 4; ++ss) {
        f32x4 cb = zero4(), g1 = zero4();
        if constexpr (!ONEH)
          for (int kb = 0; kb < NT; ++kb)
            mma(cb, bk_colk<SWZ>(Bs, LDN, 16 * ss, 16 * kb, lane), bk_colk<SWZ>(Cs, LDN, 16 * w, 16 * kb, lane));
        for (int kb = 0; kb < PT; ++kb)
          mma(g1, bk_colk<SWZ>(xs, LDP, 16 * ss, 16 * kb, lane), bk_colk<SWZ>(dys, LDP, 16 * w, 16 * kb, lane));
        float dv[4];
        float dd4 = 0.0f;  // delta_s * decay
        if constexpr (STEP4) {
          const int ls = (sb * BK_R + 16 * ss + 4 * q) / CM;
          const float cs_s = __shfl(cs.cum, ls & 63, 64);  // every lane takes part in the shuffles
          const float d_s = __shfl(cs.delta, ls & 63, 64);
          dd4 = (ls <= l_col && l_col < Lc) ? d_s * exp_hw(cum_t - cs_s) : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float dd = dd4;
          if constexpr (!STEP4) {
            const int ls = (sb * BK_R + 16 * ss + 4 * q + j) / M;
            const float cs_s = __shfl(cs.cum, ls & 63, 64);  // every lane takes part in the shuffles
            const float d_s = __shfl(cs.delta, ls & 63, 64);
            dd = (ls <= l_col && l_col < Lc) ? d_s * exp_hw(cum_t - cs_s) : 0.0f;
          }
          const float dcb = g1[j] * dd;
          if constexpr (!ONEH) orow += dcb * cb[j];
          dv[j] = dcb;
        }
        df[ss] = frag_make<T>(dv);
      }
      if constexpr (CP && CN) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < BK_TMAX; ++nt) {  // dC_k2^T += B^T . d_cb^T
        if (nt >= NT) continue;
#pragma unroll
        for (int ss = 0; ss < 4; ++ss) mma(dCT[nt], bk_rowk<SWZ>(Bs, LDN, 16 * ss, 16 * nt, lane), df[ss]);
      }
      if constexpr (CP && CN) bk_pipeline_reads<4 * CN / 16, 8>();

      if (sb == blk) {  // the head's row sums
        if constexpr (ONEH) {  // BLUE + ORANGE: sum_n C[t,n] dC[t,n] over the finished dC tiles
#pragma unroll
          for (int nt = 0; nt < BK_TMAX; ++nt) {
            if (nt >= NT) continue;
            float cv[4];
            frag_get(bk_colk<SWZ>(Cs, LDN, 16 * w, 16 * nt, lane), cv);  // C[t][n .. n+3], n = 16 nt + 4q
#pragma unroll
            for (int j = 0; j < 4; ++j) blue += cv[j] * dCT[nt][j];
          }
        }
        const float bw = sum4q(blue), ow = sum4q(orow);
        float* rv = rowv_c + h * RV_N * LM;
        if (q == 0) {
          rv[RV_BLUE * LM + col] = bw;
          rv[RV_OROW * LM + col] = ow;
        }
      }
    }
    // dC (rows t, 4 consecutive n per lane), summed over the group's heads
    const brsrc rdC = make_rsrc((T*)a.dC + ix_bc(a, bi, t0, 0, g, 0) + (i64)blk * BK_R * bstr,
                                valid_in(blk) > 0 ? (unsigned)(((valid_in(blk) - 1) * bstr + N) * esz) : 0u);
#pragma unroll
    for (int nt = 0; nt < BK_TMAX; ++nt) {
      if (nt >= NT) continue;
      bstore4(rdC, (unsigned)(((16 * w + r16) * bstr + 16 * nt + 4 * q) * esz), dCT[nt], (const T*)0);
    }
  }
}

// d_cumA from its sources, the K1 suffix sum and the chain to d_dt (or d_da):
// one wave per (batch, chunk, head), one lane per step l (rows l*M .. l*M+M-1)
__global__ void __launch_bounds__(64) ssd_blocked_epilogue_kernel(SsdArgs a) {
  const int lane = threadIdx.x;
  i64 id = blockIdx.x;
  const i64 h = id % a.H;
  id /= a.H;
  const i64 c = id % a.nc, bi = id / a.nc;
  const int L = (int)a.L, M = (int)a.M, LM = (int)a.LM;
  const i64 t0 = c * L;
  const int Lc = (int)((a.T - t0) < L ? (a.T - t0) : L);
  const float Ah = a.raw ? 0.0f : a.A[h];
  const ChunkScalars cs = load_scalars(a, bi, c, h, lane);
  const float* rv = a.rowv + ((bi * a.nc + c) * a.H + h) * RV_N * LM;
  float dcl = 0.0f, dvxl = 0.0f, qv = 0.0f;
  if (lane < Lc) {
    const float e = exp_hw(cs.end - cs.cum);
    for (int m = 0; m < M; ++m) {
      const int r = lane * M + m;
      const float q1 = rv[RV_DEC * LM + r] * e;
      dcl += rv[RV_BLUE * LM + r] + rv[RV_OROW * LM + r] - rv[RV_OCOL * LM + r] - q1;
      dvxl += rv[RV_DVX * LM + r];
      qv += q1;
    }
  }
  const float qsum = wave_sum(qv);
  const float dendt = a.dend[(bi * a.nc + c) * a.H + h] * exp_hw(cs.end);
  if (lane == Lc - 1) dcl += qsum + dendt;  // K3 d cumA_last and K4 d da_chunk_end
  const float dda = wave_incl_suffix(lane < Lc ? dcl : 0.0f, lane);
  if (lane < Lc) a.d_dtda[(bi * a.T + t0 + lane) * a.H + h] = a.raw ? dda : (dvxl + dda * Ah) * cs.sig;
}

// ===========================================================================
// host side
// ===========================================================================
// swz: the bf16 instantiation for P = 64, N = 128, whose tiles are unpadded
static size_t blocked_lds_bytes(i64 P, i64 N, bool bf, bool swz = false) {
  const i64 e = bf ? 2 : 4, pad = swz ? 0 : (bf ? 8 : 4);
  return (size_t)(e * (2 * BK_R * (N + pad) + 2 * BK_R * (P + pad) + P * N) + 4 * BK_NW);
}

bool ssd_blocked_supported(const ssmvjp_ssd_desc& d) {
  const i64 LM = d.chunk_len * d.mimo_rank;
  // chunk_len <= 64: one lane per step in the chunk scalars; M divides 64: the
  // rows of a step never straddle two blocks, so the causal pairs are exactly
  // the (target block >= source block) pairs that the two roles walk
  if (LM <= 64 || LM % BK_R || d.chunk_len > 64 || BK_R % d.mimo_rank) return false;
  if (d.headdim % 16 || d.dstate % 16 || d.headdim > 16 * BK_TMAX || d.dstate > 16 * BK_TMAX) return false;
  return blocked_lds_bytes(d.headdim, d.dstate, d.dtype == SSMVJP_BF16) <= 160 * 1024;
}

template <typename T, bool ONEH>
static void launch_blocked_h(const SsdArgs& a, size_t lds, i64 grid, hipStream_t stream) {
  const bool fixed = a.P == 64 && a.N == 128;
  if (fixed && a.M == 4)  // the rank-4 MIMO workload shape
    hipLaunchKernelGGL((ssd_blocked_bwd_kernel<T, 64, 128, 4, ONEH>), dim3((unsigned)grid), dim3(BK_NTH), lds, stream, a);
  else if (fixed)
    hipLaunchKernelGGL((ssd_blocked_bwd_kernel<T, 64, 128, 0, ONEH>), dim3((unsigned)grid), dim3(BK_NTH), lds, stream, a);
  else
    hipLaunchKernelGGL((ssd_blocked_bwd_kernel<T, 0, 0, 0, ONEH>), dim3((unsigned)grid), dim3(BK_NTH), lds, stream, a);
}

template <typename T>
static void launch_blocked_t(const SsdArgs& a, hipStream_t stream) {
  const bool fixed = a.P == 64 && a.N == 128;
  const size_t lds = blocked_lds_bytes(a.P, a.N, sizeof(T) == 2, fixed && sizeof(T) == 2);
  const i64 grid = a.b * a.nc * a.G * 2 * (a.LM / BK_R);
  if (a.hpg == 1)
    launch_blocked_h<T, true>(a, lds, grid, stream);
  else
    launch_blocked_h<T, false>(a, lds, grid, stream);
  hipLaunchKernelGGL(ssd_blocked_epilogue_kernel, dim3((unsigned)(a.b * a.nc * a.H)), dim3(64), 0, stream, a);
}

void launch_ssd_blocked_grads(const SsdArgs& a, bool is_bf16, hipStream_t stream) {
  if (a.T == 0) return;
  if (is_bf16)
    launch_blocked_t<bf16>(a, stream);
  else
    launch_blocked_t<float>(a, stream);
}

}  // namespace ssmvjp
