// Matrix-core stages of the Newton-Schulz iteration on gfx950.
//
// The quintic step of the Muon synthesis note (papers.chlience.com,
// section 4), X <- aX + b(XX^T)X + c(XX^T)^2 X with (a,b,c) =
// (3.4445, -4.7750, 2.0315), is computed as three grouped GEMM launches per
// iteration:
//
//   GRAM : A  = X_hi X_hi^T             symmetric: upper tiles only
//   POLY : P  = b A + c A A^T           symmetric (A = A^T): upper tiles,
//                                       axpy epilogue
//   BX   : X' = a (X_hi + X_lo) + P X_hi    float32 epilogue, re-split into
//                                       the bf16 pair
//
// Layout.  The iterate is kept once, as X^T (long side major):
//   xt_hi / xt_lo : X^T as n_pad x m_pad bf16 (high part, rounding residual),
//                   ping-pong between iterations; B operand of BX, both
//                   operands of GRAM (read transposed, see below) and the
//                   source of the aX term;
//   gram, poly    : m_pad x m_pad bf16, stored in full (both triangles, bit
//                   identical), so rows can be read as operands.
// BX and the polynomial read K-contiguous operand rows, which is what an
// MFMA lane consumes.  The Gram product contracts over the long side, which
// is the row index of X^T: its stage tiles are 32 k-rows x T columns and
// the fragments come out of LDS through the transposing ds_read_b64_tr_b16
// (4 consecutive k of one column per read, two reads per fragment).
// Every buffer is zero padded to multiples of the tile edge, so the main
// loop never bounds-checks and padding stays exactly zero.
//
// Kernel.  One work-group owns a T x T output tile; its waves form an
// NWM x NWN grid, each wave a (T/NWM) x (T/NWN) block of
// v_mfma_f32_16x16x32_bf16 tiles with float32 accumulators.  K advances 32
// per step through a ring of NSTAGE LDS stages filled by direct-to-LDS
// 16-byte loads (global_load_lds_dwordx4), so no registers stage the
// operands.  The loop is software pipelined: after a step's barrier the slot
// just released is refilled NSTAGE steps ahead and the next step's
// fragments are read in place, each right after its last use by this
// step's products, so LDS reads overlap the matrix work (main_loop16).  Each
// wave waits for its own loads (vmcnt) and a barrier makes a stage visible
// to all.  A row-major LDS row holds the 32 k-values of one operand row as
// four 16-byte chunks whose positions are XOR-swizzled by the row index
// ((r >> 1) ^ (r >> 2), measured free of bank conflicts on gfx950 for these
// fragment reads).
//
// Tile order.  Work-groups are dealt to the 8 XCDs round-robin; the block id
// is remapped so each XCD walks a contiguous range of (matrix, tile) work,
// which keeps the operand panels of neighbouring tiles in that XCD's L2.
//
// Epilogue.  An MFMA accumulator holds four consecutive rows of one column,
// so the BX outputs (rows of xt_*) go straight from registers as 8-byte
// stores.  A symmetric tile goes through the wave's private LDS slice,
// first in mirror layout (stored as the mirror half) and then row-major
// (the direct half), 16 bytes per lane along rows (sym_epilogue).  On
// diagonal tiles each symmetric pair is written from the element with
// i <= j only, so both triangles hold the same bits, and the products that
// would only feed elements below the diagonal are skipped (load_loop16,
// mfma16 with TRI).
#include "muon_internal.h"

namespace muon {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));


enum Mode { GRAM = 0, POLY = 1, BXM = 2 };

template <int T_, int NWM_, int NWN_, int NSTAGE_>
struct Cfg {
  static constexpr int T = T_;
  static constexpr int NWM = NWM_;
  static constexpr int NWN = NWN_;
  static constexpr int NW = NWM * NWN;
  static constexpr int kThreads = NW * 64;
  // Work-groups that must fit on one CU: two waves per SIMD either way.
  static constexpr int MINB = (NW == 4) ? 2 : 1;
  static constexpr int WM = T / NWM;
  static constexpr int WN = T / NWN;
  static constexpr int BMB = WM / 16;
  static constexpr int BNB = WN / 16;
  static constexpr int BK = 32;                      // k per step: 4 chunks of 16 bytes
  static constexpr int ROWB = BK * 2;                // bytes per LDS row
  static constexpr int QN = T / 16;                  // 1 KB load instructions per operand per step
  static constexpr int QMAX = (QN + NW - 1) / NW;    // per wave (some waves one fewer)
  static constexpr int OPB = T * ROWB;               // bytes of one operand in one stage
  static constexpr int STAGEB = 2 * OPB;             // A + B
  static constexpr int NSTAGE = NSTAGE_;            // LDS ring depth; loads run NSTAGE-1 steps ahead
  // Epilogue: each wave stages its own sub-tile (EPI_ROWS rows at a time)
  // in a private LDS slice, so no block-wide barrier is needed.
  static constexpr int EPI_LD = WN + 8;              // staged row stride (elements)
  static constexpr int EPI_ROWS = (WM * EPI_LD * 2 * NW <= NSTAGE * STAGEB) ? WM : WM / 2;
  static constexpr int EPIB = EPI_ROWS * EPI_LD * 2; // bytes per wave
  static constexpr int LDSB = (NSTAGE * STAGEB > EPIB * NW) ? NSTAGE * STAGEB : EPIB * NW;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(T % 16 == 0, "tile edge must be a multiple of 16");
};



#define GAS __attribute__((address_space(1)))
#define LAS __attribute__((address_space(3)))





// Position of chunk c (8 columns) within k-row k of a transposed-operand
// stage of width T (NC = T/8 chunks per row); a bijection on each row,
// chosen so the transposing fragment reads are free of bank conflicts at
// every row-block offset (measured on gfx950).  320-byte rows (T = 160)
// already fall on different banks per k-row and take an XOR inside aligned
// groups of 4 chunks; 256-byte rows (T = 128) alias and take a rotation
// across the row.  chunk_tr inverts pos_tr.
template <int T>
__device__ __forceinline__ int pos_tr(int k, int c) {
  if constexpr (T == 160) return c ^ (((k >> 1) ^ (k >> 2)) & 3);
  else return (c + 2 * (k & 3) + 8 * ((k >> 3) & 1)) & (T / 8 - 1);
}
template <int T>
__device__ __forceinline__ int chunk_tr(int k, int p) {
  if constexpr (T == 160) return p ^ (((k >> 1) ^ (k >> 2)) & 3);
  else return (p - 2 * (k & 3) - 8 * ((k >> 3) & 1)) & (T / 8 - 1);
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// LDS fragment addresses of a lane (bytes within a stage), one per 16-row
// block of the wave's A and B operands.
template <class C>
struct Frag16 {
  int a[C::BMB];
  int b[C::BNB];
  int a1[C::BMB];  // transposed operands: address of the second read (k + 4)
  int b1[C::BNB];
};

// Direct-to-LDS loads of one step into `dst` (both operands; SELF: the A
// operand only, for a diagonal tile of a symmetric product, whose B operand
// is the same panel and is read from the A half of the stage).
template <class C, bool SELF>
__device__ __forceinline__ void issue16(const __bf16* __restrict__ Aop, const __bf16* __restrict__ Bop,
                                        const int (&g_off)[C::QMAX], int wave, int koff,
                                        LAS unsigned char* __restrict__ dst) {
#pragma unroll
  for (int i = 0; i < C::QMAX; ++i) {
    const int q = wave + i * C::NW;
    if (i < C::QMAX - 1 || q < C::QN) {
      __builtin_amdgcn_global_load_lds((const GAS void*)(Aop + g_off[i] + koff), (LAS void*)(dst + q * 1024), 16,
                                       0, 0);
      if constexpr (!SELF)
        __builtin_amdgcn_global_load_lds((const GAS void*)(Bop + g_off[i] + koff),
                                         (LAS void*)(dst + C::OPB + q * 1024), 16, 0, 0);
    }
  }
}

// One fragment: a 16-byte read (row-major), or two transposing 8-byte
// reads (k 0..3 at p, k 4..7 at p1).
template <class C, bool TR>
__device__ __forceinline__ bf16x8_t frag16(const LAS unsigned char* p, const LAS unsigned char* p1) {
  if constexpr (TR) {
    return __builtin_shufflevector(__builtin_amdgcn_ds_read_tr16_b64_v4bf16((LAS bf16x4_t*)p),
                                   __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LAS bf16x4_t*)p1),
                                   0, 1, 2, 3, 4, 5, 6, 7);
  } else {
    return *(const LAS bf16x8_t*)p;
  }
}

// TRI: the wave's sub-tile sits on the diagonal of a symmetric product; the
// 16x16 blocks below the diagonal (i > j) are never stored and skipped.
template <class C, bool TRI>
__device__ __forceinline__ void mfma16(const bf16x8_t (&a)[C::BMB], const bf16x8_t (&b)[C::BNB],
                                       f32x4_t (&acc)[C::BMB][C::BNB]) {
#pragma unroll
  for (int i = 0; i < C::BMB; ++i)
#pragma unroll
    for (int j = 0; j < C::BNB; ++j)
      if (!TRI || j >= i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// The products of one step with the next step's fragments read in place:
// a row block's A fragment is re-read as soon as its row of products is
// issued, and during the last row each B fragment right after its last use,
// so the reads overlap the matrix work with a single set of fragment
// registers.  Optionally queues a future step's loads into `dst` first.
// `dst` (the slot just released) and `src` (the next stage) always differ;
// __restrict__ lets the compiler order the LDS reads against the in-flight
// direct-to-LDS loads without a blanket wait.
// Scheduling groups of mfma_and_read16 (counts must be constants): rows
// 0..BMB-2 as (row of products, A re-read); the last row as (product,
// B re-read) pairs.  With TRI a row i holds BNB - i products.
template <int I, int BMB, int BNB, int RPF, bool TRI>
__device__ __forceinline__ void sched_rows16() {
  if constexpr (I < BMB - 1) {
    __builtin_amdgcn_sched_group_barrier(0x008, TRI ? BNB - I : BNB, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RPF, 0);
    sched_rows16<I + 1, BMB, BNB, RPF, TRI>();
  }
}
template <int J, int BMB, int BNB, int RPF, bool TRI>
__device__ __forceinline__ void sched_last16() {
  if constexpr (J < BNB) {
    if constexpr (!TRI || J >= BMB - 1) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RPF, 0);
    sched_last16<J + 1, BMB, BNB, RPF, TRI>();
  }
}

template <class C, bool TR, bool TRI, bool SELF>
__device__ __forceinline__ void mfma_and_read16(const __bf16* __restrict__ Aop, const __bf16* __restrict__ Bop,
                                                const int (&g_off)[C::QMAX], int wave, int koff, bool queue,
                                                LAS unsigned char* __restrict__ dst,
                                                const LAS unsigned char* __restrict__ src, const Frag16<C>& f,
                                                bf16x8_t (&a)[C::BMB], bf16x8_t (&b)[C::BNB],
                                                f32x4_t (&acc)[C::BMB][C::BNB]) {
  if (queue) issue16<C, SELF>(Aop, Bop, g_off, wave, koff, dst);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < C::BMB - 1; ++i) {
#pragma unroll
    for (int j = 0; j < C::BNB; ++j)
      if (!TRI || j >= i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    a[i] = frag16<C, TR>(src + f.a[i], src + f.a1[i]);
  }
  constexpr int L = C::BMB - 1;
#pragma unroll
  for (int j = 0; j < C::BNB; ++j) {
    if (!TRI || j >= L) acc[L][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[L], b[j], acc[L][j], 0, 0, 0);
    b[j] = frag16<C, TR>(src + f.b[j], src + f.b1[j]);
  }
  a[L] = frag16<C, TR>(src + f.a[L], src + f.a1[L]);
  // Keep that order: a row of products, then the re-read of its A fragment;
  // in the last row one product, then one B re-read.
  constexpr int RPF = TR ? 2 : 1;  // LDS reads per fragment
  sched_rows16<0, C::BMB, C::BNB, RPF, TRI>();
  sched_last16<0, C::BMB, C::BNB, RPF, TRI>();
  __builtin_amdgcn_sched_group_barrier(0x100, RPF, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// One pipelined step kt (fragments of kt in a/b): wait for this wave's loads
// of step kt+1 (NEWER later steps may stay in flight) and for its own reads
// of stage kt, barrier (stage kt+1 visible to all, stage kt free), refill
// stage kt with step kt+NSTAGE, multiply while reading step kt+1's
// fragments.
template <class C, int PER, bool TR, bool TRI, bool SELF>
__device__ __forceinline__ void step16(const __bf16* __restrict__ Aop, const __bf16* __restrict__ Bop,
                                       const int (&g_off)[C::QMAX], int kmul, int nk, int kt, int newer,
                                       LAS unsigned char* lds, int wave, const Frag16<C>& f,
                                       bf16x8_t (&a)[C::BMB], bf16x8_t (&b)[C::BNB],
                                       f32x4_t (&acc)[C::BMB][C::BNB]) {
  if (newer >= 2) MUON_WAIT_VM(2 * PER);
  else if (newer == 1) MUON_WAIT_VM(PER);
  else MUON_WAIT_VM(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const int fut = kt + C::NSTAGE;
  mfma_and_read16<C, TR, TRI, SELF>(Aop, Bop, g_off, wave, fut * C::BK * kmul, fut < nk, lds + (kt % C::NSTAGE) * C::STAGEB,
                         lds + ((kt + 1) % C::NSTAGE) * C::STAGEB, f, a, b, acc);
}

// Main loop: the prologue fills every ring slot; steady steps keep
// NSTAGE-2 later steps in flight with immediate wait counts; draining steps
// stop refilling; the last step only multiplies.
template <class C, int PER, bool TR, bool TRI, bool SELF>
__device__ __forceinline__ void main_loop16(const __bf16* __restrict__ Aop, const __bf16* __restrict__ Bop,
                                            const int (&g_off)[C::QMAX], int kmul, int nk,
                                            LAS unsigned char* lds, int wave, const Frag16<C>& f,
                                            f32x4_t (&acc)[C::BMB][C::BNB]) {
  static_assert(C::NSTAGE >= 3 && C::NSTAGE <= 4, "wait counts assume 3 or 4 stages");
#pragma unroll
  for (int st = 0; st < C::NSTAGE; ++st)
    if (st < nk) issue16<C, SELF>(Aop, Bop, g_off, wave, st * C::BK * kmul, lds + st * C::STAGEB);
  {
    const int newer = nk - 1 < C::NSTAGE - 1 ? nk - 1 : C::NSTAGE - 1;
    if (newer >= 3) MUON_WAIT_VM(3 * PER);
    else if (newer == 2) MUON_WAIT_VM(2 * PER);
    else if (newer == 1) MUON_WAIT_VM(PER);
    else MUON_WAIT_VM(0);
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  bf16x8_t a[C::BMB], b[C::BNB];
#pragma unroll
  for (int i = 0; i < C::BMB; ++i) a[i] = frag16<C, TR>(lds + f.a[i], lds + f.a1[i]);
#pragma unroll
  for (int j = 0; j < C::BNB; ++j) b[j] = frag16<C, TR>(lds + f.b[j], lds + f.b1[j]);
  int kt = 0;
  for (; kt < nk - C::NSTAGE; ++kt)
    step16<C, PER, TR, TRI, SELF>(Aop, Bop, g_off, kmul, nk, kt, C::NSTAGE - 2, lds, wave, f, a, b, acc);
  for (; kt + 1 < nk; ++kt)
    step16<C, PER, TR, TRI, SELF>(Aop, Bop, g_off, kmul, nk, kt, nk - 2 - kt, lds, wave, f, a, b, acc);
  mfma16<C, TRI>(a, b, acc);
}

// The main loop of a wave whose sub-tile lies wholly below the diagonal of a
// diagonal tile of a symmetric product: it does its share of the stage
// loads (A half only, as every wave of a diagonal tile), waits and barriers
// exactly as main_loop16 does, but no fragment
// reads and no products (nothing of its sub-tile is stored), which leaves
// its SIMD to the other work-group on the CU.
template <class C, int PER>
__device__ __forceinline__ void load_loop16(const __bf16* __restrict__ Aop, const __bf16* __restrict__ Bop,
                                            const int (&g_off)[C::QMAX], int kmul, int nk,
                                            LAS unsigned char* lds, int wave) {
#pragma unroll
  for (int st = 0; st < C::NSTAGE; ++st)
    if (st < nk) issue16<C, true>(Aop, Bop, g_off, wave, st * C::BK * kmul, lds + st * C::STAGEB);
  {
    const int newer = nk - 1 < C::NSTAGE - 1 ? nk - 1 : C::NSTAGE - 1;
    if (newer >= 3) MUON_WAIT_VM(3 * PER);
    else if (newer == 2) MUON_WAIT_VM(2 * PER);
    else if (newer == 1) MUON_WAIT_VM(PER);
    else MUON_WAIT_VM(0);
  }
  __builtin_amdgcn_s_barrier();
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int newer = (kt < nk - C::NSTAGE) ? C::NSTAGE - 2 : nk - 2 - kt;
    if (newer >= 2) MUON_WAIT_VM(2 * PER);
    else if (newer == 1) MUON_WAIT_VM(PER);
    else MUON_WAIT_VM(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int fut = kt + C::NSTAGE;
    if (fut < nk) issue16<C, true>(Aop, Bop, g_off, wave, fut * C::BK * kmul, lds + (kt % C::NSTAGE) * C::STAGEB);
  }
}

// Epilogue of a symmetric product (Gram, polynomial) for one wave's sub-tile
// (WM x WN, rows gi0 = wi0.., columns gj0 = wj0..), through the wave's LDS
// slice so that every global access is 16 bytes per lane along a row:
//   1. (polynomial) the input A at the mirror positions, A[gj][gi..], rows
//      of the slice M[jl][il] (A is symmetric, so these are the values the
//      accumulators need);
//   2. the results in accumulator layout (column gj per lane, four
//      consecutive rows gi) rounded to bf16 and written to M[jl][il..il+3]
//      (for the polynomial in place of the A values they use);
//   3. rows of M to the mirror half, P[gj][gi..];
//   4. the same words, kept in registers, to a row-major slice S[il][jl]
//      (same LDS), whose rows go to the direct half, P[gi][gj..].
// On a diagonal tile (DIAG) both halves are written from the elements with
// gi <= gj only, so the two triangles hold bit-identical values.
template <class C, int MODE, bool DIAG>
__device__ __forceinline__ void sym_epilogue(const MatDesc& d, int m_pad, int wi0, int wj0, int lane, __bf16* slice,
                                             const f32x4_t (&acc)[C::BMB][C::BNB], float gscale) {
  static_assert(C::EPI_ROWS == C::WM && C::WM == C::WN, "square wave tiles, staged whole");
  constexpr int LD = C::EPI_LD;
  constexpr int CPR = C::WM / 8;       // 16-byte chunks per slice row
  constexpr int NCH = C::WN * CPR;     // chunks per sub-tile
  constexpr int NIT = (NCH + 63) / 64;
  const int l16 = lane & 15, lq = lane >> 4;
  __bf16* rdst = (MODE == POLY) ? d.poly : d.gram;
  if constexpr (MODE == POLY) {
#pragma unroll
    for (int t = 0; t < NIT; ++t) {
      const int c = t * 64 + lane;
      if (c < NCH) {
        const int jl = c / CPR, ch = c - (c / CPR) * CPR;
        *reinterpret_cast<uint4*>(slice + jl * LD + 8 * ch) =
            gld<uint4>(d.gram + static_cast<int64_t>(wj0 + jl) * m_pad + wi0 + 8 * ch);
      }
    }
    asm volatile("" ::: "memory");
  }
  uint32_t w[C::BMB][C::BNB][2];
#pragma unroll
  for (int i = 0; i < C::BMB; ++i)
#pragma unroll
    for (int j = 0; j < C::BNB; ++j) {
      uint2* mp = reinterpret_cast<uint2*>(slice + (16 * j + l16) * LD + 16 * i + 4 * lq);
      float v[4];
      if constexpr (MODE == POLY) {
        const uint2 av = *mp;  // A[gj][gi..gi+3] == A[gi..gi+3][gj]
        v[0] = fmaf(kCoefC, acc[i][j][0], kCoefB * bf_lo(av.x));
        v[1] = fmaf(kCoefC, acc[i][j][1], kCoefB * bf_hi(av.x));
        v[2] = fmaf(kCoefC, acc[i][j][2], kCoefB * bf_lo(av.y));
        v[3] = fmaf(kCoefC, acc[i][j][3], kCoefB * bf_hi(av.y));
      } else {
        // Gram: the first iteration's operand is the unnormalised pair
        // (gscale = sigma^2), later ones 1.
        v[0] = acc[i][j][0] * gscale; v[1] = acc[i][j][1] * gscale;
        v[2] = acc[i][j][2] * gscale; v[3] = acc[i][j][3] * gscale;
      }
      w[i][j][0] = pack_bf16(v[0], v[1]);
      w[i][j][1] = pack_bf16(v[2], v[3]);
      *mp = make_uint2(w[i][j][0], w[i][j][1]);
    }
  asm volatile("" ::: "memory");
  // Mirror half: row gj of the slice holds P[gj][wi0 ..].
#pragma unroll
  for (int t = 0; t < NIT; ++t) {
    const int c = t * 64 + lane;
    if (c < NCH) {
      const int jl = c / CPR, ch = c - (c / CPR) * CPR;
      const int gj = wj0 + jl, gi = wi0 + 8 * ch;
      const uint4 val = *reinterpret_cast<const uint4*>(slice + jl * LD + 8 * ch);
      __bf16* p = rdst + static_cast<int64_t>(gj) * m_pad + gi;
      if (!DIAG || gi + 7 <= gj) {
        gst(p, val);
      } else if (gi <= gj) {
        uint16_t hv[8];
        __builtin_memcpy(hv, &val, 16);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gi + e <= gj) gst(p + e, hv[e]);
      }
    }
  }
  asm volatile("" ::: "memory");
  // Direct half: the words again, row-major.
#pragma unroll
  for (int i = 0; i < C::BMB; ++i)
#pragma unroll
    for (int j = 0; j < C::BNB; ++j) {
      const int rl = 16 * i + 4 * lq, cl = 16 * j + l16;
      const uint16_t hb[4] = {static_cast<uint16_t>(w[i][j][0]), static_cast<uint16_t>(w[i][j][0] >> 16),
                              static_cast<uint16_t>(w[i][j][1]), static_cast<uint16_t>(w[i][j][1] >> 16)};
#pragma unroll
      for (int r = 0; r < 4; ++r) __builtin_memcpy(slice + (rl + r) * LD + cl, &hb[r], 2);
    }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int t = 0; t < NIT; ++t) {
    const int c = t * 64 + lane;
    if (c < NCH) {
      const int il = c / CPR, ch = c - (c / CPR) * CPR;
      const int gi = wi0 + il, gj = wj0 + 8 * ch;
      const uint4 val = *reinterpret_cast<const uint4*>(slice + il * LD + 8 * ch);
      __bf16* p = rdst + static_cast<int64_t>(gi) * m_pad + gj;
      if (!DIAG || gi <= gj) {
        gst(p, val);
      } else if (gi < gj + 8) {
        uint16_t hv[8];
        __builtin_memcpy(hv, &val, 16);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gi <= gj + e) gst(p + e, hv[e]);
      }
    }
  }
}

template <class C, int MODE>
__global__ __launch_bounds__(C::kThreads, C::MINB) void ns_gemm_kernel(const MatDesc* __restrict__ descs,
                                                              const int32_t* __restrict__ prefix,
                                                              int nmats, XcdSplit split, int buf, int first) {
  constexpr int T = C::T;
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[C::LDSB];
  __bf16* smem = reinterpret_cast<__bf16*>(smem_raw);

  // ---- XCD-aware work: XCD (block id % 8) walks its own cost-balanced
  // contiguous range of (matrix, tile) work.
  const int work = split.begin[blockIdx.x & 7] + static_cast<int>(blockIdx.x >> 3);
  if (work >= split.end[blockIdx.x & 7]) return;
  const int mi = find_mat(prefix, nmats, work);
  const MatDesc d = descs[mi];
  int local = work - prefix[mi];
  const int m_pad = d.m_pad;

  int ti, tj;
  if (MODE == BXM) {
    // Gram-side index fastest: tiles running together share the X^T panels
    // (read once from HBM) and cycle through the small P.
    const int tpc = m_pad / T;
    tj = local / tpc;
    ti = local - tj * tpc;
  } else {
    const int nt = m_pad / T;
    ti = 0;
    while (local >= nt - ti) {
      local -= nt - ti;
      ++ti;
    }
    tj = ti + local;
  }

  const __bf16* __restrict__ Aop;
  const __bf16* __restrict__ Bop;
  int ld, K;
  // The Gram product reads X^T (n_pad x m_pad, the iterate's own layout):
  // its tiles are 32 k-rows x T columns, transposed on the way out of LDS.
  constexpr bool TR = MODE == GRAM;
  if (MODE == GRAM) {
    Aop = pick(d.xt_hi, buf) + static_cast<int64_t>(ti) * T;
    Bop = pick(d.xt_hi, buf) + static_cast<int64_t>(tj) * T;
    ld = m_pad;
    K = d.k_gram;
  } else if (MODE == POLY) {
    Aop = d.gram + static_cast<int64_t>(ti) * T * m_pad;
    Bop = d.gram + static_cast<int64_t>(tj) * T * m_pad;
    ld = K = m_pad;
  } else {
    Aop = d.poly + static_cast<int64_t>(ti) * T * m_pad;
    Bop = pick(d.xt_hi, buf) + static_cast<int64_t>(tj) * T * m_pad;
    ld = K = m_pad;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave / C::NWN;
  const int wc = wave - wr * C::NWN;
  const int l16 = lane & 15;
  const int lq = lane >> 4;

  // Direct-to-LDS load slots of this wave.  Row-major operands: instruction
  // q covers operand rows 16q..16q+15; lane l fills LDS chunk slot (row
  // 16q + l/4, position l%4) with the global k-chunk that the swizzle maps
  // there.  Transposed operands (Gram): a stage holds 32 k-rows of NC = T/8
  // chunks of 8 columns; chunk c of k-row k sits at position pos_tr(k, c),
  // and instruction q fills positions 64q..64q+63 in order.
  int g_off[C::QMAX];
#pragma unroll
  for (int i = 0; i < C::QMAX; ++i) {
    const int q = wave + i * C::NW;
    if constexpr (TR) {
      constexpr int NC = T / 8;
      const int p = q * 64 + lane;
      const int k = p / NC;
      const int c = chunk_tr<T>(k, p % NC);
      g_off[i] = k * ld + c * 8;
    } else {
      const int r = q * 16 + (lane >> 2);
      const int c = swz(r, lane & 3);   // swz is an involution on the chunk index
      g_off[i] = r * ld + c * 8;
    }
  }
  // Element distance between consecutive steps: 32 along a row, or 32 rows.
  const int kmul = TR ? ld : 1;
  // Loads this wave issues per step (both operands).
  const int nq = (C::QN - wave + C::NW - 1) / C::NW;

  f32x4_t acc[C::BMB][C::BNB];
#pragma unroll
  for (int i = 0; i < C::BMB; ++i)
#pragma unroll
    for (int j = 0; j < C::BNB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fragment addresses (bytes within a stage).
  Frag16<C> fr;
  if constexpr (TR) {
    // In each 16-lane group g, lane 4a + j' reads columns 4a.. of k-row
    // 8g + j (j = (lane & 15) >> 2, the source-row index of the transposing
    // read), so output lane l gets row (l & 15) at 4 consecutive k; the
    // second read is 4 k-rows on.
    const int aa = lane & 3, j = (lane & 15) >> 2;
    const int krow = 8 * lq + j;
#pragma unroll
    for (int i = 0; i < C::BMB; ++i) {
      const int c = (wr * C::WM + 16 * i + 4 * aa) >> 3;
      fr.a[i] = krow * 2 * T + pos_tr<T>(krow, c) * 16 + (aa & 1) * 8;
      fr.a1[i] = (krow + 4) * 2 * T + pos_tr<T>(krow + 4, c) * 16 + (aa & 1) * 8;
    }
#pragma unroll
    for (int jb = 0; jb < C::BNB; ++jb) {
      const int c = (wc * C::WN + 16 * jb + 4 * aa) >> 3;
      fr.b[jb] = C::OPB + krow * 2 * T + pos_tr<T>(krow, c) * 16 + (aa & 1) * 8;
      fr.b1[jb] = C::OPB + (krow + 4) * 2 * T + pos_tr<T>(krow + 4, c) * 16 + (aa & 1) * 8;
    }
  } else {
    // Row r of a 16-row block at r*64 + swizzled chunk; the swizzle repeats
    // every 8 rows, so block i is block 0 plus 1024 i bytes.
    const int a_row0 = wr * C::WM + l16;
    const int b_row0 = wc * C::WN + l16;
#pragma unroll
    for (int i = 0; i < C::BMB; ++i) fr.a[i] = a_row0 * C::ROWB + swz(a_row0, lq) * 16 + 1024 * i;
#pragma unroll
    for (int jb = 0; jb < C::BNB; ++jb) fr.b[jb] = C::OPB + b_row0 * C::ROWB + swz(b_row0, lq) * 16 + 1024 * jb;
#pragma unroll
    for (int i = 0; i < C::BMB; ++i) fr.a1[i] = fr.a[i];
#pragma unroll
    for (int jb = 0; jb < C::BNB; ++jb) fr.b1[jb] = fr.b[jb];
  }

  const int nk = K / C::BK;
  LAS unsigned char* lds = (LAS unsigned char*)smem_raw;
  // On a diagonal tile of a symmetric product, a wave whose sub-tile lies
  // wholly below the diagonal only loads (its results are never stored).
  // A diagonal tile of a symmetric product multiplies a panel by itself: its
  // stages hold the panel once (A half) and the B fragments are read there.
  const bool self = (MODE != BXM) && ti == tj;
  if (self) {
#pragma unroll
    for (int jb = 0; jb < C::BNB; ++jb) {
      fr.b[jb] -= C::OPB;
      fr.b1[jb] -= C::OPB;
    }
  }
  const bool below = self && wr * C::WM >= (wc + 1) * C::WN;
  if (below) {
    if (nq == C::QMAX) load_loop16<C, C::QMAX>(Aop, Bop, g_off, kmul, nk, lds, wave);
    else load_loop16<C, C::QMAX - 1>(Aop, Bop, g_off, kmul, nk, lds, wave);
  } else if (self && wr * C::WM == wc * C::WN) {
    // A sub-tile on the diagonal: only its blocks with i <= j are stored.
    if constexpr (C::WM == C::WN) {
      if (nq == C::QMAX) main_loop16<C, C::QMAX, TR, true, true>(Aop, Bop, g_off, kmul, nk, lds, wave, fr, acc);
      else main_loop16<C, C::QMAX - 1, TR, true, true>(Aop, Bop, g_off, kmul, nk, lds, wave, fr, acc);
    }
  } else if (self) {
    if (nq == C::QMAX) main_loop16<C, C::QMAX, TR, false, true>(Aop, Bop, g_off, kmul, nk, lds, wave, fr, acc);
    else main_loop16<C, C::QMAX - 1, TR, false, true>(Aop, Bop, g_off, kmul, nk, lds, wave, fr, acc);
  } else {
    if (nq == C::QMAX) main_loop16<C, 2 * C::QMAX, TR, false, false>(Aop, Bop, g_off, kmul, nk, lds, wave, fr, acc);
    else main_loop16<C, 2 * (C::QMAX - 1), TR, false, false>(Aop, Bop, g_off, kmul, nk, lds, wave, fr, acc);
  }
  __syncthreads();
  if (below) return;

  // ---- epilogue.  16x16 accumulator layout: lane holds column (lane & 15),
  // register r holds row 4 * (lane >> 4) + r.  Each wave works alone on its
  // sub-tile through its private LDS slice.
  const int wi0 = ti * T + wr * C::WM;      // first global row of the wave's sub-tile
  const int wj0 = tj * T + wc * C::WN;      // first global column
  __bf16* slice = smem + wave * (C::EPIB / 2);
  // First iteration: the iterate is the unnormalised pair of M; its Gram
  // product is scaled by s1^2 and the BX result by s1 (s1 = sigma, or 1
  // where the prep pass already normalised).
  const float s1 = first ? gld<float>(d.sigma + kSigFirst) : 1.f;
  if constexpr (MODE != BXM) {
    const float gscale = (MODE == GRAM) ? s1 * s1 : 1.f;
    if (ti == tj)
      sym_epilogue<C, MODE, true>(d, m_pad, wi0, wj0, lane, slice, acc, gscale);
    else
      sym_epilogue<C, MODE, false>(d, m_pad, wi0, wj0, lane, slice, acc, gscale);
    return;
  }
  // BX: X' = a (X_hi + X_lo) + P X_hi, stored as the X^T pair straight from
  // the accumulators (four consecutive Gram-side rows per lane are 8
  // contiguous bytes of a row of X^T).  Global reads are issued a batch of
  // PRE block rows at a time (they are independent and mostly come from
  // HBM), then combined.
  constexpr int PRE = (16 / C::BNB) > 0 ? (16 / C::BNB) : 1;
#pragma unroll
  for (int b0 = 0; b0 < C::BMB; b0 += PRE) {
    uint2 in_a[PRE][C::BNB], in_b[PRE][C::BNB];
#pragma unroll
    for (int ib = b0; ib < b0 + PRE && ib < C::BMB; ++ib) {
#pragma unroll
      for (int j = 0; j < C::BNB; ++j) {
        const int gi = wi0 + ib * 16 + lq * 4;
        const int gj = wj0 + j * 16 + l16;
        const int64_t off = static_cast<int64_t>(gj) * m_pad + gi;
        in_a[ib - b0][j] = gld<uint2>(pick(d.xt_hi, buf) + off);
        in_b[ib - b0][j] = gld<uint2>(pick(d.xt_lo, buf) + off);
      }
    }
#pragma unroll
    for (int ib = b0; ib < b0 + PRE && ib < C::BMB; ++ib) {
#pragma unroll
      for (int j = 0; j < C::BNB; ++j) {
        const int gi = wi0 + ib * 16 + lq * 4;
        const int gj = wj0 + j * 16 + l16;
        const int64_t off = static_cast<int64_t>(gj) * m_pad + gi;
        const uint2 hx = in_a[ib - b0][j];
        const uint2 lx = in_b[ib - b0][j];
        float v[4];
        v[0] = fmaf(kCoefA, bf_lo(hx.x) + bf_lo(lx.x), acc[ib][j][0]);
        v[1] = fmaf(kCoefA, bf_hi(hx.x) + bf_hi(lx.x), acc[ib][j][1]);
        v[2] = fmaf(kCoefA, bf_lo(hx.y) + bf_lo(lx.y), acc[ib][j][2]);
        v[3] = fmaf(kCoefA, bf_hi(hx.y) + bf_hi(lx.y), acc[ib][j][3]);
        if (s1 != 1.f) {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] *= s1;
        }
        const uint32_t w0 = pack_bf16(v[0], v[1]);
        const uint32_t w1 = pack_bf16(v[2], v[3]);
        const uint32_t l0 = pack_bf16(v[0] - bf_lo(w0), v[1] - bf_hi(w0));
        const uint32_t l1 = pack_bf16(v[2] - bf_lo(w1), v[3] - bf_hi(w1));
        gst(pick(d.xt_hi, buf ^ 1) + off, make_uint2(w0, w1));
        gst(pick(d.xt_lo, buf ^ 1) + off, make_uint2(l0, l1));
      }
    }
  }
  (void)slice;
}

// Tile configurations: edge T and wave grid.
using C160 = Cfg<160, 2, 2, 4>;
using C128 = Cfg<128, 2, 2, 4>;

template <class C>
hipError_t launch_mode(int mode, const MatDesc* d, const int32_t* prefix, int nmats, const XcdSplit& sp,
                       int buf, int first, hipStream_t s) {
  if (sp.max_len <= 0) return hipSuccess;
  const dim3 grid(8 * sp.max_len);
  if (mode == GRAM)
    hipLaunchKernelGGL((ns_gemm_kernel<C, GRAM>), grid, dim3(C::kThreads), 0, s, d, prefix, nmats, sp, buf, first);
  else if (mode == POLY)
    hipLaunchKernelGGL((ns_gemm_kernel<C, POLY>), grid, dim3(C::kThreads), 0, s, d, prefix, nmats, sp, buf, first);
  else
    hipLaunchKernelGGL((ns_gemm_kernel<C, BXM>), grid, dim3(C::kThreads), 0, s, d, prefix, nmats, sp, buf, first);
  return hipGetLastError();
}

}  // namespace



hipError_t launch_ns_gemm(int mode, int cfg, const MatDesc* d, const int32_t* prefix, int nmats,
                          const XcdSplit& split, int buf, int first, hipStream_t s) {
  if (cfg == kCfgT160) return launch_mode<C160>(mode, d, prefix, nmats, split, buf, first, s);
  if (cfg == kCfgT128) return launch_mode<C128>(mode, d, prefix, nmats, split, buf, first, s);
  return hipErrorInvalidValue;
}

}  // namespace muon
