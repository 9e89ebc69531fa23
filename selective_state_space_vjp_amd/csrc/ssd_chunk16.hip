// ssd_chunk16.hip -- the per-chunk backward of the chunked SSD scan (burn-mamba
// "combined_backward.rs": the BLUE, ORANGE, K3, K2 and K1 backwards and, in the
// Mamba-2 form, the chain to (dx, d_dt)) for bf16 storage at head dim P = 64,
// state size N = 128 and 64-step chunks of rank 1, organised for four waves
// per SIMD.
//
// Same method, data layout and results as ssd_chunk_bwd_kernel in ssd_chunk.hip
// (one workgroup per (batch, chunk, group, head split), the heads of a group in
// a loop, dB / dC summed over the heads in registers in ascending head order,
// K2 once on the head-summed d_cb, no float atomics).  What differs is the
// division of the work: 16 waves with fixed roles and at most 128 registers
// each, so that every SIMD interleaves four instruction streams (MFMA, LDS and
// VALU work of different waves overlap):
//   phase A  waves 0..7   BLUE: dC_blue^T for n tile w (S_c^T . (dy e^cumA)^T),
//                         dC += dC_blue, the BLUE d_cumA row sums;
//            waves 8..15  K3: dB_k3^T for n tile w-8 (dS^T . (x delta e^(end-cumA))^T),
//                         dB += dB_k3, the d_end partial sum of S_c (.) dS_{c+1};
//            waves 15..8, 4, 5  one ORANGE (t, s) tile pair each (10 pairs): G1 = dy x^T,
//                         d_cb (summed over heads), masked w = CB * decay, the
//                         ORANGE d_cumA row and column sums;
//            wave 2 or 3 (alternating) assembles the previous head's d_cumA,
//                         K1 suffix sum and d_dt.
//   phase B  wave w       item (p tile w/4, row block w%4): K3 d_v = dS B^T and
//                         ORANGE d_v = dy^T w, dx, the K3 decay and dvx row sums.
// The per-head step scalars (cumA, delta, the per-step decay factors, sigma(dt)
// and A) sit in LDS so that per-element values are LDS reads rather than lane
// shuffles, and the d_cumA assembly reads them there a head later.  The next
// head's x and dy rows and dS_{c+1} go straight from memory into the LDS
// buffers of the other head parity (LDS-direct loads issued in phase A, after
// the ORANGE products); its S_c goes into Ss the same way once phase A's readers of Ss are
// past the second barrier, and wave 0 loads its step scalars into registers
// and writes them, with the factors, to LDS during phase B: two barriers per
// head.
#include "ssd_common.cuh"

namespace ssmvjp {
namespace {

typedef __attribute__((address_space(3))) char lds_char;
// raw buffer resource words (the form make_rsrc builds), made wave-uniform so
// that they sit in scalar registers
__device__ __forceinline__ u32x4 rsrc_words_u(const void* base, unsigned bytes) {
  const unsigned long long p = (unsigned long long)base;
  u32x4 r;
  r[0] = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)p);
  r[1] = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(p >> 32)) & 0xffffu;
  r[2] = (unsigned)__builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000u;
  return r;
}
// LDS-direct loads (each lane's 4 or 16 bytes written to LDS at M0 + the
// lane's slot), issued as assembly: the compiler neither counts them nor, as
// it does for its own LDS-direct loads, waits for every outstanding load
// before the next transposed LDS read.  The caller waits with vmcnt before the
// barrier that publishes the data.  M0 is named as clobbered; the compiler
// uses it for nothing else in this file (it keeps no value there across these
// statements), so its warning about clobbering a reserved register is muted.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_dword(unsigned lds_addr, unsigned off, u32x4 rs) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(off), "s"(rs)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_dwordx4(unsigned lds_addr, unsigned off, u32x4 rs) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(off), "s"(rs)
               : "memory", "m0");
}
#pragma clang diagnostic pop

constexpr int W16 = 16;          // waves per workgroup
constexpr int NTH16 = 64 * W16;
constexpr int P16 = 64, N16 = 128, LM16 = 64;
constexpr int PT = P16 / 16, NT = N16 / 16, RB = LM16 / 16;
constexpr int NPAIR = RB * (RB + 1) / 2;  // lower-triangular (t, s) tile pairs
constexpr int LDC = LM16 + 4;             // CB pitch (float)
// row pitches of the staged tiles: rows 2 dwords apart modulo the 32 LDS
// banks, so the fragment reads along a row (16 lanes, 8 bytes each, one per
// row) hit 32 distinct banks
constexpr int LDN = N16 + 4;              // B / C pitch (bf16)
// x / dy rows: unpadded, each 8-byte unit u of a row stored at u ^ f(row)
// (xsw_off), which keeps the fragment reads along the rows and the transposed
// ones on distinct banks and lets LDS-direct loads place any 8-byte unit
constexpr int LDP = P16;
constexpr int PN = P16 * N16;

// partial row sums of one head (float offsets inside one set)
constexpr int PB_BLUE = 0;                     // [NT][64]    BLUE, by n tile
constexpr int PB_OROW = PB_BLUE + NT * 64;     // [NPAIR][16] ORANGE row sums, rows of the pair's t block
constexpr int PB_OCOL = PB_OROW + NPAIR * 16;  // [NPAIR][16] ORANGE column sums, columns of the pair's s block
constexpr int PB_DEC = PB_OCOL + NPAIR * 16;   // [PT][64]    K3 decay term, by p tile
constexpr int PB_DVX = PB_DEC + PT * 64;       // [PT][64]    sum_p d_v x, by p tile
constexpr int PB_DEND = PB_DVX + PT * 64;      // [NT]        sum S (.) dS, by n tile
constexpr int PB_SET = PB_DEND + 16;

// LDS layout (bytes)
constexpr int L_CB = 0;                                  // float [64][LDC]
constexpr int L_PB = L_CB + LM16 * LDC * 4;              // float [2][PB_SET]
// x, dy, dS_{c+1} and the step scalars are double buffered by head parity: the
// next head is staged during phase B of the current one, which reads them;
// S_c, read only in phase A, is staged in place during phase B
constexpr int SC_N = 7;                                  // per-step values: cumA, delta, the factors below, sigma(dt); A
constexpr int L_SC = L_PB + 2 * PB_SET * 4;              // float [2][SC_N][64], by head parity
constexpr int L_B = L_SC + 2 * SC_N * 64 * 4;            // bf16 [64][LDN]
constexpr int L_C = L_B + LM16 * LDN * 2;                // bf16 [64][LDN]
constexpr int L_X = L_C + LM16 * LDN * 2;                // bf16 [2][64][LDP]
constexpr int L_DY = L_X + 2 * LM16 * LDP * 2;           // bf16 [2][64][LDP]
constexpr int L_DS = L_DY + 2 * LM16 * LDP * 2;          // bf16 [2][P*N] dS_{c+1}, native tiles
constexpr int L_S = L_DS + 2 * PN * 2;                   // bf16 [P*N] S_c, native tiles
constexpr int L_W = L_S + PN * 2;                        // bf16 [NPAIR][256] w tiles in MFMA output order
constexpr int L_TOTAL = L_W + NPAIR * 256 * 2;

__device__ __forceinline__ int pair_of(int rt, int rs) { return rt * (rt + 1) / 2 + rs; }

// The S_c and dS_{c+1} tiles sit in LDS in MFMA output order with each
// 128-byte quarter of a 512-byte tile rotated by 32 bytes per quarter: the
// transposed read gathers 8 bytes from each of the four quarters at the same
// offset, which without the rotation all fall in the same banks.
__device__ __forceinline__ int swz(int byte) { return (byte & ~127) | ((byte + 32 * ((byte >> 7) & 3)) & 127); }
__device__ __forceinline__ Frag<bf16> ld_ntv_s(const bf16* t, int lane) {
  Frag<bf16> f;
  f.v = *(const s16x4*)((const char*)t + swz(8 * lane));
  return f;
}
__device__ __forceinline__ Frag<bf16> ld_ntv_t_s(const bf16* t, int lane) {
  const int m = lane & 15;
  return lds_tr_b16((const bf16*)((const char*)t + swz(8 * ((m & 3) * 16 + 4 * (lane >> 4) + (m >> 2)))));
}
// two 8-byte LDS stores of a 16-byte chunk (rows of the staged tiles are 8-byte aligned)
__device__ __forceinline__ void st16_as8(bf16* p, const u32x4& u) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 lo = {u[0], u[1]}, hi = {u[2], u[3]};
  *(u32x2*)p = lo;
  *(u32x2*)(p + 4) = hi;
}
__device__ __forceinline__ int tile_off(int pt, int nt) { return (pt * NT + nt) * 256; }
// sum of the four products of two bf16 quadruples, added to c (two packed
// bf16 dot products accumulated in float)
__device__ __forceinline__ float dot2_bf16(s16x4 x, s16x4 y, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  const s16x2 x0 = {x[0], x[1]}, x1 = {x[2], x[3]}, y0 = {y[0], y[1]}, y1 = {y[2], y[3]};
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x0), __builtin_bit_cast(bf16x2, y0), c, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x1), __builtin_bit_cast(bf16x2, y1), c, false);
}

// The four sums of x[0..3] over the 4 rows of 16 lanes (lanes with the same
// lane % 16) at once: two row-pair swaps (odd rows of the first operand with
// even rows of the second) and one half swap.  Row q ends with the sum of x[q].
__device__ __forceinline__ float sum4q_x4(const float x[4]) {
  auto bits = [](float f) { return __builtin_bit_cast(int, f); };
  auto flt = [](unsigned u) { return __builtin_bit_cast(float, u); };
  const auto a = __builtin_amdgcn_permlane16_swap(bits(x[0]), bits(x[1]), false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(bits(x[2]), bits(x[3]), false, false);
  const float u = flt(a[0]) + flt(a[1]), w = flt(b[0]) + flt(b[1]);  // rows: x0, x1, x0, x1 / x2, x3, x2, x3 pair sums
  const auto c = __builtin_amdgcn_permlane32_swap(bits(u), bits(w), false, false);
  return flt(c[0]) + flt(c[1]);
}

// The four sums of v[0..3] over the 16 lanes of a DPP row at once: a butterfly
// that halves the values each lane carries at every exchange (partners r16 ^ 8
// by row rotation, then 7 - r16 within the 8-lane half, then r16 ^ 2 and
// r16 ^ 1 within the quad).  Lane r16 ends with the sum of v[r16 >> 2].
__device__ __forceinline__ float sum16x4(const float v[4], int r16) {
  const bool h8 = (r16 & 8) != 0, h4 = (r16 & 4) != 0;
  const float k0 = h8 ? v[2] : v[0], k1 = h8 ? v[3] : v[1];  // kept
  const float s0 = h8 ? v[0] : v[2], s1 = h8 ? v[1] : v[3];  // handed to the partner
  const float a0 = k0 + dpp_f<0x128>(s0), a1 = k1 + dpp_f<0x128>(s1);  // row_ror:8
  const float k = h4 ? a1 : a0, s = h4 ? a0 : a1;
  float r = k + dpp_f<0x141>(s);  // row_half_mirror
  r += dpp_f<0x4E>(r);            // quad_perm [2, 3, 0, 1]
  r += dpp_f<0xB1>(r);            // quad_perm [1, 0, 3, 2]
  return r;
}

// DA: also the per-chunk dA partial sums (a separate instantiation, so that
// the plain backward keeps its registers); RAW: the raw-decay form (delta = 1,
// d_da out), the selective form otherwise
template <bool DA, bool RAW>
__global__ void __launch_bounds__(NTH16) ssd_chunk16_kernel(SsdArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* CBs = (float*)(smem_raw + L_CB);
  float* pbase = (float*)(smem_raw + L_PB);
  float* scb = (float*)(smem_raw + L_SC);
  bf16* Bs = (bf16*)(smem_raw + L_B);
  bf16* Cs = (bf16*)(smem_raw + L_C);
  bf16* xsb = (bf16*)(smem_raw + L_X);
  bf16* dysb = (bf16*)(smem_raw + L_DY);
  bf16* dSsb = (bf16*)(smem_raw + L_DS);
  bf16* Ss = (bf16*)(smem_raw + L_S);
  bf16* Wt = (bf16*)(smem_raw + L_W);

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, q = lane >> 4,
            r16 = lane & 15;
  __builtin_assume(w >= 0 && w < W16);
  i64 bid = blockIdx.x;
  const i64 hs = bid % a.hsplit;
  bid /= a.hsplit;
  const i64 g = bid % a.G;
  bid /= a.G;
  const i64 c = bid % a.nc, bi = bid / a.nc;
  const i64 t0 = c * LM16;
  const int Lc = (int)((a.T - t0) < LM16 ? (a.T - t0) : LM16);
  const int xrs = (int)(a.H * P16), brs = (int)(a.G * N16);  // row strides of x/dy/dx and B/C/dB/dC
  const i64 xoff0 = (bi * a.T + t0) * a.H * P16, boff0 = (bi * a.T + t0) * a.G * N16 + g * N16;
  const bf16* xg = (const bf16*)a.xv + xoff0;
  const bf16* dyg = (const bf16*)a.dy + xoff0;
  bf16* dxg = (bf16*)a.dxv + xoff0;
  const bf16* Bg = (const bf16*)a.B + boff0;
  const bf16* Cg = (const bf16*)a.C + boff0;
  float* ddtg = a.d_dtda + (bi * a.T + t0) * a.H;

  // ---- B and C rows of the chunk into LDS (rows past the sequence: zeros) ----
  {
    const unsigned bcbytes = (unsigned)(((i64)(Lc - 1) * brs + N16) * 2);
    const brsrc rb_ = make_rsrc(Bg, bcbytes), rc_ = make_rsrc(Cg, bcbytes);
    const int r = tid >> 4, col = (tid & 15) * 8;  // 64 rows x 16 chunks of 16 bytes
    st16_as8(Bs + r * LDN + col, bload16(rb_, (unsigned)(r * brs + col) * 2));
    st16_as8(Cs + r * LDN + col, bload16(rc_, (unsigned)(r * brs + col) * 2));
  }

  // ---- loads of one head ----
  // Wave 0 loads the step scalars and A into registers.  The x and dy rows and
  // dS_{c+1} go straight from memory into LDS (LDS-direct loads into the
  // buffers of the head's parity, free since the barrier before): waves 0..7
  // load x, waves 8..15 dy, 4-byte units, four 256-byte wave loads each; every
  // wave one 1 KiB block of dS_{c+1}.  Rows past the sequence read zeros (the
  // resource covers the valid rows only).
  ChunkScalars rcs = {0.f, 0.f, 0.f, 0.f};
  float rA = 0.0f;
  const i64 hbase = g * a.hpg + hs * a.hph;
  const unsigned xbytes = (unsigned)(((i64)(Lc - 1) * xrs + P16) * 2);
  const brsrc rsA = make_rsrc(a.A, RAW ? 0u : (unsigned)(a.H * 4));
  const int xy_sel = w >> 3, xw = w & 7;  // x or dy, and this wave's quarter of the rows
  // source byte offset (in the head's rows) of this lane's 4 bytes for wave load i:
  // LDS dword D = (4 xw + i) * 64 + lane of the row-major buffer, row D / 32, stored
  // 8-byte unit (D % 32) / 2 = logical unit ^ f(row), half D % 2
  unsigned xy_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (4 * xw + i) * 2 + (lane >> 5), e = lane & 31;
    const int f = ((row & 3) << 2) | ((row >> 2) & 3);
    const int u = (e >> 1) ^ f;
    xy_off[i] = (unsigned)(row * xrs + 4 * u + 2 * (e & 1)) * 2u;
  }
  // dS_{c+1}: LDS 16-byte unit v = lane % 32 of tile 2w + lane / 32 holds the
  // tile's unit u with the same quarter, rotated back by two units per quarter
  const int dsv = lane & 31;
  const unsigned ds_off = (unsigned)((2 * w + (lane >> 5)) * 512 + 16 * ((dsv & 24) | (((dsv & 7) - 2 * (dsv >> 3)) & 7)));
  auto issue_regs = [&](i64 h) {
    if (w == 0) {
      rcs = issue_scalars(a, bi, c, h, lane);
      rA = bload_f32(rsA, (unsigned)(h * 4));
    }
  };
  const unsigned lds0 = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(unsigned long long)(lds_char*)smem_raw);
  auto issue_lds = [&](i64 h, int k) {
    const u32x4 wxy = rsrc_words_u((xy_sel ? dyg : xg) + (int)h * P16, xbytes);
    const unsigned dxy = lds0 + (unsigned)(xy_sel ? L_DY : L_X) + (unsigned)(k * LM16 * LDP + 4 * xw * 128) * 2u;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_dword((unsigned)__builtin_amdgcn_readfirstlane((int)(dxy + 256u * i)), xy_off[i], wxy);
    const i64 so = ((bi * a.nc + c) * a.H + h) * (i64)PN;
    dma_dwordx4((unsigned)__builtin_amdgcn_readfirstlane((int)(lds0 + (unsigned)L_DS + (unsigned)(k * PN + w * 512) * 2u)),
                ds_off, rsrc_words_u((const bf16*)a.dS + so, PN * 2));
  };
  // S_c of head h into Ss by LDS-direct loads (the layout of the dS_{c+1} tiles)
  auto issue_s = [&](i64 h) {
    const i64 so = ((bi * a.nc + c) * a.H + h) * (i64)PN;
    dma_dwordx4((unsigned)__builtin_amdgcn_readfirstlane((int)(lds0 + (unsigned)L_S + (unsigned)(w * 512) * 2u)),
                ds_off, rsrc_words_u((const bf16*)a.S + so, PN * 2));
  };
  issue_regs(hbase);
  issue_lds(hbase, 0);
  issue_s(hbase);
  __syncthreads();  // B, C staged

  // ---- C.B^T (K2 recompute) on the lower-triangular tile pairs, waves 0..9 ----
  if (w < NPAIR) {
    int rt = 0;
    while ((rt + 1) * (rt + 2) / 2 <= w) ++rt;
    const int rs_ = w - rt * (rt + 1) / 2;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < NT; ++kb)
      mma(acc, ld_colk(Cs, LDN, 16 * rt, 16 * kb, lane), ld_colk(Bs, LDN, 16 * rs_, 16 * kb, lane));
#pragma unroll
    for (int j = 0; j < 4; ++j) CBs[(16 * rt + 4 * q + j) * LDC + 16 * rs_ + r16] = acc[j];
  }

  // ---- fixed roles ----
  const bool blue = w < NT;             // phase A product: BLUE (dC) or K3 (dB)
  const int nt_own = blue ? w : w - NT;
  // ORANGE pairs: waves 15..8 and 4, 5, so that each SIMD (waves w % 4) holds
  // two or three pairs, the SIMDs with two also taking the d_cumA assembly
  const int pair = w >= 8 ? W16 - 1 - w : (w == 4 || w == 5) ? w + 4 : -1;
  const bool has_pair = pair >= 0;
  int prt = 0;
  while (has_pair && (prt + 1) * (prt + 2) / 2 <= pair) ++prt;
  const int prs = has_pair ? pair - prt * (prt + 1) / 2 : 0;
  const int ipt = w / RB, irb = w % RB;  // phase B item
  f32x4 xacc[RB];                        // dC (BLUE waves) or dB (K3 waves), transposed, summed over heads
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) xacc[rb] = zero4();
  f32x4 dcbacc = zero4();                // d_cb of this wave's pair, summed over heads

  // d_cumA from its sources, the K1 suffix sum and the chain to d_dt (RAW:
  // d_da) for one head, from the partial sums in pb; lane = step.  Also the
  // head's dA partial sum over the chunk, sum_l d_da_l * delta_l (the same in
  // every lane).
  auto epilogue = [&](const float* sc, const float* pb) -> float2 {
    const float cum = sc[lane], end = sc[63], Ah = sc[384];
    float dc = 0.0f, qv = 0.0f, dvx = 0.0f;
    if (lane < LM16) {
      const int rbl = lane >> 4, rl = lane & 15;
      float bl = 0.f, orow = 0.f, ocol = 0.f, dec = 0.f;
#pragma unroll
      for (int k = 0; k < NT; ++k) bl += pb[PB_BLUE + k * 64 + lane];
      for (int k = 0; k <= rbl; ++k) orow += pb[PB_OROW + pair_of(rbl, k) * 16 + rl];
      for (int k = rbl; k < RB; ++k) ocol += pb[PB_OCOL + pair_of(k, rbl) * 16 + rl];
#pragma unroll
      for (int k = 0; k < PT; ++k) {
        dec += pb[PB_DEC + k * 64 + lane];
        dvx += pb[PB_DVX + k * 64 + lane];
      }
      qv = dec * exp_hw(end - cum);
      dc = bl + orow - ocol - qv;
    }
    const float qsum = wave_sum(qv);
    float dendt = 0.0f;
#pragma unroll
    for (int k = 0; k < NT; ++k) dendt += pb[PB_DEND + k];
    dendt *= exp_hw(end);
    if (lane == Lc - 1) dc += qsum + dendt;  // K3 d cumA_last and K4 d da_chunk_end
    const float dda = wave_incl_suffix(lane < Lc ? dc : 0.0f, lane);
    return make_float2(RAW ? dda : (dvx + dda * Ah) * sc[320 + lane], DA ? wave_sum(dda * sc[64 + lane]) : 0.0f);
  };
  const brsrc bddt = make_rsrc(ddtg, (unsigned)(Lc * a.H * 4));
  // waves 2 and 3 store (dropped unless `on`)
  auto epi_store = [&](bool on, i64 h, float2 v) {
    bstore_f32(bddt, on && lane < Lc ? (unsigned)((lane * a.H + h) * 4) : BUF_OOB, v.x);
    if constexpr (DA) bstore_f32(dA_rsrc(a, bi, c), on && lane == 0 ? (unsigned)(h * 4) : BUF_OOB, v.y);
  };
  i64 prev_h = 0;

  // the prefetched head's step scalars into the buffers of parity k (its x,
  // dy, dS_{c+1} and S_c arrive by LDS-direct loads)
  auto stage = [&](int k) {
    if (w == 0) {
      const ChunkScalars ncs = finish_scalars(rcs);  // per step r: cumA, delta, e^cumA (BLUE), delta e^(end-cumA) (K3), e^(end-cumA)
      float* sc = scb + k * SC_N * 64;
      const float edec = exp_hw(ncs.end - ncs.cum);
      sc[lane] = ncs.cum;
      sc[64 + lane] = ncs.delta;
      sc[128 + lane] = exp_hw(ncs.cum);
      sc[192 + lane] = ncs.delta * edec;
      sc[256 + lane] = edec;
      sc[320 + lane] = ncs.sig;
      sc[384 + lane] = rA;
    }
  };
  stage(0);

  for (i64 hh = 0; hh < a.hph; ++hh) {
    const i64 h = hbase + hh;
    const int k = (int)(hh & 1);
    float* pb = pbase + k * PB_SET;
    const brsrc bdx = make_rsrc(dxg + (int)h * P16, xbytes);
    const float* cumL = scb + k * SC_N * 64;
    const float* delL = cumL + 64;
    const float* fbl = cumL + 128;  // e^cumA
    const float* fk3 = cumL + 192;  // delta e^(end-cumA)
    const float* edl = cumL + 256;  // e^(end-cumA)
    const bf16* xs = xsb + k * LM16 * LDP;
    const bf16* dys = dysb + k * LM16 * LDP;
    const bf16* dSs = dSsb + k * PN;

    // this wave's LDS-direct loads have landed: vmcnt(0) on entry; after a head,
    // vmcnt(1), which leaves its dx store (the newest operation; the vector
    // memory count retires in issue order) in flight
    if (hh == 0)
      __builtin_amdgcn_s_waitcnt(0x0F70);
    else
      __builtin_amdgcn_s_waitcnt(0x0F71);
    __syncthreads();  // this head staged; the previous head's phase B done (and CB on entry)

    // the next head (unconditional: past the last head the last head is
    // reloaded into buffers never read again)
    const i64 hn = hh + 1 < a.hph ? h + 1 : hbase + a.hph - 1;
    issue_regs(hn);

    // the previous head's partial sums are complete: its d_cumA on one of waves 0..3
    {
      const bool on = hh > 0 && w == 2 + (int)((hh - 1) & 1);
      float2 v = make_float2(0.0f, 0.0f);
      if (on) v = epilogue(scb + ((hh - 1) & 1) * SC_N * 64, pbase + ((hh - 1) & 1) * PB_SET);
      if ((w >> 1) == 1) epi_store(on, prev_h, v);
    }

    // ---- phase A (1): ORANGE on this wave's tile pair ----
    if (has_pair) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < PT; ++kb)
        mma(acc, ld_colk_xs(dys, LDP, 16 * prt, 16 * kb, lane), ld_colk_xs(xs, LDP, 16 * prs, 16 * kb, lane));
      const int s_ = 16 * prs + r16;
      const float cs_s = cumL[s_], dls = delL[s_];
      const f32x4 ct = *(const f32x4*)(cumL + 16 * prt + 4 * q);  // rows t = 16 prt + 4q + j
      float orow[4], ocol = 0.0f, wv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * prt + 4 * q + j;
        const float dec = (s_ <= t && t < Lc) ? exp_hw(ct[j] - cs_s) : 0.0f;
        const float dcb = acc[j] * dls * dec;  // d_w = dy . v^T with v = delta x (delta = 1 for RAW)
        dcbacc[j] += dcb;
        const float cb = CBs[t * LDC + s_];
        const float dd = dcb * cb;
        orow[j] = dd;
        ocol += dd;
        wv[j] = cb * dec;  // w = CB * decay: the d_v_orange operand
      }
      store4(Wt + pair * 256 + 4 * lane, f32x4{wv[0], wv[1], wv[2], wv[3]});
      const float osum = sum16x4(orow, r16);  // row 4q + r16 / 4 of the t block
      ocol = sum4q(ocol);
      if ((r16 & 3) == 0) pb[PB_OROW + pair * 16 + 4 * q + (r16 >> 2)] = osum;
      if (q == 0) pb[PB_OCOL + pair * 16 + r16] = ocol;
    }

    // the next head's x, dy and dS_{c+1}, issued after the ORANGE products: at
    // the head's start the waves' loads would queue behind one another and hold
    // the ORANGE waves back
    issue_lds(hn, k ^ 1);

    // ---- phase A (2): BLUE (dC) or K3 (dB) on this wave's n tile, computed
    // transposed (rows n, columns the chunk's rows r) ----
    {
      float fcol[RB];  // per-lane column factor of row r = 16 rb + r16
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        fcol[rb] = (blue ? fbl : fk3)[16 * rb + r16];
      }
      const bf16* opA = blue ? Ss : dSs;  // A: rows n, k = p (native tiles)
      const bf16* opB = blue ? dys : xs;  // B: k = p, columns r
      f32x4 acc[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb] = zero4();
      float dend = 0.0f;
#pragma unroll
      for (int kb = 0; kb < PT; ++kb) {
        const Frag<bf16> fa = ld_ntv_s(opA + tile_off(kb, nt_own), lane);
        Frag<bf16> fb[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) fb[rb] = ld_colk_xs(opB, LDP, 16 * rb, 16 * kb, lane);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) mma(acc[rb], fa, fb[rb]);
        if (!blue) {  // d_end partial: S_c (.) dS_{c+1} over this n tile, two bf16 products per step
          const Frag<bf16> fs = ld_ntv_s(Ss + tile_off(kb, nt_own), lane);
          dend = dot2_bf16(fs.v, fa.v, dend);
        }
      }
      if (blue) {
        float bsum[RB];  // sum_n C dC_blue = fcol * sum_n C acc, this lane's 4 n
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float cv[4];
          frag_get(ld_colk(Cs, LDN, 16 * rb, 16 * nt_own, lane), cv);  // C[r][n .. n+3], n = 16 nt + 4q
          float s = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) s = fmaf(cv[j], acc[rb][j], s);
          bsum[rb] = s * fcol[rb];
        }
        // row q of lanes: the sum over the n tile for row block q
        pb[PB_BLUE + nt_own * 64 + 16 * q + r16] = sum4q_x4(bsum);
      } else {
        dend = wave_sum(dend);
        if (lane == 0) pb[PB_DEND + nt_own] = dend;
      }
      // both roles: the product scaled by the column factor, summed over heads
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < 4; ++j) xacc[rb][j] = fmaf(acc[rb][j], fcol[rb], xacc[rb][j]);
    }

    __syncthreads();  // w tiles complete; Ss free

    // the next head's step values, and its S_c into Ss (read in phase A only)
    stage(k ^ 1);
    issue_s(hn);

    // ---- phase B: K3 d_dv^T = dS_{c+1} . B^T and ORANGE d_v_or^T = dy^T . w for
    // the item (p tile ipt, row block irb); dx; K3 decay and dvx row sums ----
    {
      f32x4 acc3 = zero4(), acc5 = zero4();
      // A: rows p, k = n (transposed native read); B: k = n, columns r -- in two batches of 4 n tiles
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        Frag<bf16> f3a[NT / 2], f3b[NT / 2];
#pragma unroll
        for (int k = 0; k < NT / 2; ++k) {
          const int kb = half * (NT / 2) + k;
          f3a[k] = ld_ntv_t_s(dSs + tile_off(ipt, kb), lane);
          f3b[k] = ld_colk(Bs, LDN, 16 * irb, 16 * kb, lane);
        }
#pragma unroll
        for (int k = 0; k < NT / 2; ++k) mma(acc3, f3a[k], f3b[k]);
      }
      {  // A: rows p, k = t (transpose read of dy rows); B: k = t, columns s
        Frag<bf16> f5a[RB], f5b[RB];
#pragma unroll
        for (int kb = 0; kb < RB; ++kb) {
          if (kb < irb) continue;
          f5a[kb] = ld_rowk_xs(dys, LDP, 16 * kb, 16 * ipt, lane);
          f5b[kb] = ld_ntv(Wt + pair_of(kb, irb) * 256, lane);
        }
#pragma unroll
        for (int kb = 0; kb < RB; ++kb) {
          if (kb < irb) continue;
          mma(acc5, f5a[kb], f5b[kb]);
        }
      }
      const int r = 16 * irb + r16;  // this lane's column
      const float dl = delL[r];
      const float edec = edl[r];
      float xv[4];
      frag_get(ld_colk_xs(xs, LDP, 16 * irb, 16 * ipt, lane), xv);  // x[r][p .. p+3], p = 16 pt + 4q
      float dvo[4], s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float dv = fmaf(acc3[j], edec, acc5[j]);  // d_v = d_v_k3 + d_v_orange
        dvo[j] = RAW ? dv : dv * dl;
        s1 = fmaf(acc3[j], xv[j], s1);  // d_decay / delta = sum_p d_decayed_v . x
        s2 = fmaf(dv, xv[j], s2);
      }
      // rows past the end of the sequence fall outside the resource and are dropped
      bstore4(bdx, (unsigned)(r * xrs + 16 * ipt + 4 * q) * 2, f32x4{dvo[0], dvo[1], dvo[2], dvo[3]},
              (const bf16*)0);
      s1 = sum4q(s1) * dl;
      s2 = sum4q(s2);
      if (q == 0) {
        pb[PB_DEC + ipt * 64 + r] = s1;
        pb[PB_DVX + ipt * 64 + r] = s2;
      }
    }
    prev_h = h;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no LDS-direct load outstanding past the loop
  __syncthreads();  // the last head's partial sums complete
  if (a.hph > 0) {
    const bool on = w == 2 + (int)((a.hph - 1) & 1);
    float2 v = make_float2(0.0f, 0.0f);
    if (on) v = epilogue(scb + ((a.hph - 1) & 1) * SC_N * 64, pbase + ((a.hph - 1) & 1) * PB_SET);
    epi_store(on, prev_h, v);
  }

  // ---- K2 backward on the head-summed d_cb: dC_k2 = d_cb . B, dB_k2 = d_cb^T . C ----
  __syncthreads();
  if (has_pair) {
#pragma unroll
    for (int j = 0; j < 4; ++j) CBs[(16 * prt + 4 * q + j) * LDC + 16 * prs + r16] = dcbacc[j];
  }
  __syncthreads();
  const i64 stride = a.b * a.T * a.G * a.N;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    // transposed: rows n, columns r
    f32x4 acc = xacc[rb];
    if (blue) {
      for (int kb = 0; kb <= rb; ++kb)  // dC_k2^T = B^T . d_cb^T
        mma(acc, ld_rowk(Bs, LDN, 16 * kb, 16 * nt_own, lane), frag_make<bf16>(ld_colk(CBs, LDC, 16 * rb, 16 * kb, lane).v));
    } else {
      for (int kb = rb; kb < RB; ++kb)  // dB_k2^T = C^T . d_cb
        mma(acc, ld_rowk(Cs, LDN, 16 * kb, 16 * nt_own, lane), frag_make<bf16>(ld_rowk(CBs, LDC, 16 * kb, 16 * rb, lane).v));
    }
    const int r = 16 * rb + r16;
    if (r >= Lc) continue;
    const int o = r * brs + 16 * nt_own + 4 * q;  // [r][n .. n+3], offset from boff0
    if (a.hsplit == 1)
      store4((bf16*)(blue ? a.dC : a.dB) + boff0 + o, acc);
    else
      store4(a.part + ((blue ? a.hsplit : 0) + hs) * stride + boff0 + o, acc);
  }
}

}  // namespace

void launch_ssd_chunk16(const SsdArgs& a, hipStream_t stream) {
  const i64 grid = a.b * a.nc * a.G * a.hsplit;
  if (a.raw)  // no dA in the raw-decay form
    hipLaunchKernelGGL((ssd_chunk16_kernel<false, true>), dim3((unsigned)grid), dim3(NTH16), L_TOTAL, stream, a);
  else if (a.dA_part)
    hipLaunchKernelGGL((ssd_chunk16_kernel<true, false>), dim3((unsigned)grid), dim3(NTH16), L_TOTAL, stream, a);
  else
    hipLaunchKernelGGL((ssd_chunk16_kernel<false, false>), dim3((unsigned)grid), dim3(NTH16), L_TOTAL, stream, a);
}

}  // namespace ssmvjp
