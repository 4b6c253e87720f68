// Wide-tile matrix-core kernels of the Newton-Schulz iteration on gfx950
// (v_mfma_f32_32x32x16_bf16, two waves per SIMD).
//
// The quintic step of the Muon synthesis note (papers.chlience.com,
// section 4) is evaluated as A = X_hi X_hi^T, P = b A + c A A^T and
// X' = a (X_hi + X_lo) + P X_hi, exactly as in gemm_kernels.hip (same
// layouts, same epilogue arithmetic, so the two kernel families are
// interchangeable per matrix); this file holds the bigger tiles:
//
//   G256 : 256 x 256 output tile, 8 waves as 2 x 4, wave tile 128 x 64.
//          Gram, polynomial (upper tiles) and BX.
//   W320 : 320 x 256 output tile (320 rows on the Gram side m, 256 columns on
//          the long side n), 8 waves as 2 x 4, wave tile 160 x 64.  BX only,
//          for Gram sides that are multiples of 320 (m = 1600).
//   W160 : 160 x 256 output tile, 4 waves as 1 x 4, wave tile 160 x 64.  BX
//          only, for Gram sides that are multiples of 160 but not of 256 or
//          320.
//
// A 32x32x16 MFMA does twice the work of a 16x16x32 one per instruction
// and keeps the matrix pipe full from two waves per SIMD; wave tiles of
// 128 x 64 / 160 x 64 read 12 / 14 KB of LDS fragments per 32-deep k-step
// for 16 / 20 MFMAs.
//
// Main loop: a ring of NSTAGE LDS stages (32 k each; 4 for G256 and W320,
// 3 for W160) is filled by direct-to-LDS 16-byte loads: the slot a step
// frees is refilled with the step NSTAGE later.  Fragment reads are ordinary LDS loads inside a step
// function whose stage pointers are __restrict__ (the stage being filled
// and the stage being read are always different ring slots), which lets
// the compiler order the reads against the in-flight direct-to-LDS loads
// without a blanket wait.  Each wave waits for its own loads (vmcnt) and a
// barrier publishes a stage.  Operand rows are 64 bytes in LDS with the
// four 16-byte k-chunks XOR-swizzled by row ((r >> 1) ^ (r >> 2)): measured
// conflict-free on gfx950 for the 32x32x16 and 16x16x32 fragment reads (the
// (r >> 1) ^ (r >> 3) form runs at half the LDS rate).  The swizzle repeats
// every 8 rows, so one base address per k16 half serves every fragment of
// a wave (+2048 bytes per 32 rows).
//
// Epilogues: a 32x32 accumulator holds, per lane, column (lane & 31) and
// rows 8g + 4 (lane >> 5) + r (g, r = 0..3): four runs of four consecutive
// rows.  Gram and polynomial tiles go through a private 64 x 64 LDS slice
// per wave, which serves both the mirror half and the direct half of the
// symmetric result (sym_epilogue).  The BX epilogue (bx_epilogue) passes
// the float32 results through a wave-private LDS tile so that the X^T pair
// and W are read and written 16 bytes per lane along contiguous rows.  The
// last BX of a step (mode BXL) applies the parameter update of the
// synthesis note's section 4, W <- W - lr*scale*O, from the float32 values
// directly; the iterate itself is not stored then.
#include "muon_internal.h"

namespace muon {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

#define GAS __attribute__((address_space(1)))
#define LAS __attribute__((address_space(3)))


// BXL: the last BX of a step; instead of storing the iterate it applies the
// parameter update W -= lr * scale * O (or stores O in orthogonalise-only
// mode) straight from the epilogue.  BXD: BXL that also sums the per-matrix
// diagnostics of the W it writes (one DiagPart per wave).
enum Mode { GRAM = 0, POLY = 1, BXM = 2, BXL = 3, BXD = 4 };

template <int BM_, int BN_, int NWM_, int NWN_, int NSTAGE_>
struct G32 {
  static constexpr int BM = BM_, BN = BN_, NWM = NWM_, NWN = NWN_;
  static constexpr int NW = NWM * NWN;
  static constexpr int kThreads = NW * 64;
  static constexpr int WM = BM / NWM, WN = BN / NWN;
  static constexpr int BMB = WM / 32, BNB = WN / 32;
  static constexpr int QA = BM / 16, QB = BN / 16;        // 1 KB load instructions per step
  static constexpr int QAMAX = (QA + NW - 1) / NW;
  static constexpr int QBMAX = (QB + NW - 1) / NW;
  static constexpr int OPA = BM * 64, OPB = BN * 64;      // bytes per stage
  static constexpr int STAGEB = OPA + OPB;
  static constexpr int NSTAGE = NSTAGE_;                  // ring of LDS stages
  static constexpr int SLICE_LD = WN + 8;                 // Gram/poly epilogue slice row stride (bf16)
  static constexpr int TP = 68;                           // BX epilogue tile pitch (floats), see bx_epilogue
  static constexpr int SLICEB_SYM = 64 * SLICE_LD * 2;
  static constexpr int SLICEB_BX = WN * TP * 4;
  static constexpr int SLICEB = SLICEB_SYM > SLICEB_BX ? SLICEB_SYM : SLICEB_BX;  // bytes per wave
  static constexpr int LDSB = (NSTAGE * STAGEB > SLICEB * NW) ? NSTAGE * STAGEB : SLICEB * NW;
  static constexpr int MINB = (NW == 4) ? 2 : 1;          // two waves per SIMD
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(NW == 4 || NW == 8, "swizzle invariance of the load slots assumes 4 or 8 waves");
};




// Waits until at most `newer` later steps of this wave's loads are in flight
// (`per` loads per step, a compile-time count for each wave class).
template <int PER>
__device__ __forceinline__ void wait_newer(int newer) {
  if (newer <= 0) MUON_WAIT_VM(0);
  else if (newer == 1) MUON_WAIT_VM(PER);
  else if (newer == 2) MUON_WAIT_VM(2 * PER);
  else MUON_WAIT_VM(3 * PER);
}

// Direct-to-LDS load slots of one lane: element offsets of its A and B
// loads within a step, and the element distance between steps (32 along a
// row for row-major operands, 32 rows for the transposed Gram operand).
template <class C>
struct Slots {
  int aoff[C::QAMAX];
  int boff[C::QBMAX];
  int kmul;
};

// LDS fragment addresses of a lane (bytes within a stage).  Row-major
// operands: one base per k16 half, +2048 per 32-row block.  Transposed
// (Gram) operands: one base per 32-row block; a k16 half adds 16 k-rows.
template <class C>
struct Frag {
  int a[C::BMB > 2 ? C::BMB : 2];
  int b[C::BNB > 2 ? C::BNB : 2];
};

__device__ __forceinline__ bf16x8_t join4(bf16x4_t lo, bf16x4_t hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Fragments of one k16 half of a stage: A rows of the wave (BMB blocks of
// 32) and B rows (BNB blocks).  Row-major operands: one 16-byte LDS read
// each.  Transposed operands (TR, Gram from X^T): two transposing 8-byte
// reads (ds_read_b64_tr_b16) give the 4 + 4 consecutive k of the lane's row.
template <class C, bool TR>
__device__ __forceinline__ void read_half(const LAS unsigned char* __restrict__ src, int h, const Frag<C>& f,
                                          bf16x8_t (&a)[C::BMB], bf16x8_t (&b)[C::BNB]) {
  if constexpr (TR) {
    constexpr int RP = 2 * C::BM;  // k-row pitch (bytes); A and B are equally wide here
    const int ho = h * 16 * RP;
#pragma unroll
    for (int j = 0; j < C::BNB; ++j) {
      const LAS unsigned char* p = src + f.b[j] + ho;
      b[j] = join4(__builtin_amdgcn_ds_read_tr16_b64_v4bf16((LAS bf16x4_t*)p),
                   __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LAS bf16x4_t*)(p + 4 * RP)));
    }
#pragma unroll
    for (int i = 0; i < C::BMB; ++i) {
      const LAS unsigned char* p = src + f.a[i] + ho;
      a[i] = join4(__builtin_amdgcn_ds_read_tr16_b64_v4bf16((LAS bf16x4_t*)p),
                   __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LAS bf16x4_t*)(p + 4 * RP)));
    }
  } else {
#pragma unroll
    for (int j = 0; j < C::BNB; ++j) b[j] = *(const LAS bf16x8_t*)(src + f.b[h] + j * 2048);
#pragma unroll
    for (int i = 0; i < C::BMB; ++i) a[i] = *(const LAS bf16x8_t*)(src + f.a[h] + i * 2048);
  }
}

// DOFF >= 0: the wave's sub-tile straddles the diagonal of a diagonal tile
// of a symmetric product, its column blocks starting DOFF blocks right of
// its row blocks; block (i, j) lies wholly below the diagonal (never stored)
// when i > j + DOFF, and its products are skipped.  DOFF < 0: every block.
template <int DOFF>
__device__ __forceinline__ constexpr bool tri_keep(int i, int j) {
  return DOFF < 0 || i <= j + DOFF;
}
template <class C, int DOFF>
__device__ __forceinline__ constexpr int tri_products() {
  int n = 0;
  for (int i = 0; i < C::BMB; ++i)
    for (int j = 0; j < C::BNB; ++j) n += tri_keep<DOFF>(i, j) ? 1 : 0;
  return n;
}
template <class C, int DOFF>
__device__ __forceinline__ constexpr int tri_reads() {
  int n = C::BNB;  // block column j is always used (with i = 0)
  for (int i = 0; i < C::BMB; ++i) n += tri_keep<DOFF>(i, C::BNB - 1) ? 1 : 0;
  return n;
}

template <class C, int DOFF>
__device__ __forceinline__ void mfma_half(const bf16x8_t (&a)[C::BMB], const bf16x8_t (&b)[C::BNB],
                                          f32x16_t (&acc)[C::BMB][C::BNB]) {
#pragma unroll
  for (int i = 0; i < C::BMB; ++i)
#pragma unroll
    for (int j = 0; j < C::BNB; ++j)
      if (tri_keep<DOFF>(i, j)) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// Direct-to-LDS loads of one step: loads FROM..TO-1 of this wave's PER
// (1 KB each, one per 16 operand rows), A loads first.  Every configuration
// gives each wave the same number of B loads, so its A loads are
// PER - QBMAX (PER on a diagonal tile of a symmetric product, which loads the
// A half only, SELF); with the counts fixed at compile time the loads are
// issued without branches.
template <class C, bool SELF, int PER, int FROM = 0, int TO = PER>
__device__ __forceinline__ void issue_loads(const __bf16* __restrict__ Aop, const __bf16* __restrict__ Bop,
                                            const Slots<C>& sl, int k0, LAS unsigned char* __restrict__ dst,
                                            int wave) {
  static_assert(C::QB % C::NW == 0, "B loads are spread evenly over the waves");
  constexpr int NA = SELF ? PER : PER - C::QBMAX;
  static_assert(NA >= 1 && NA <= C::QAMAX, "A loads of a wave");
  static_assert(0 <= FROM && FROM <= TO && TO <= PER, "load range");
  constexpr int A0 = FROM < NA ? FROM : NA, A1 = TO < NA ? TO : NA;
  constexpr int B0 = (FROM > NA ? FROM : NA) - NA, B1 = (TO > NA ? TO : NA) - NA;
#pragma unroll
  for (int i = A0; i < A1; ++i)
    __builtin_amdgcn_global_load_lds((const GAS void*)(Aop + sl.aoff[i] + k0 * sl.kmul),
                                     (LAS void*)(dst + (wave + i * C::NW) * 1024), 16, 0, 0);
  if constexpr (!SELF) {
#pragma unroll
    for (int i = B0; i < B1; ++i)
      __builtin_amdgcn_global_load_lds((const GAS void*)(Bop + sl.boff[i] + k0 * sl.kmul),
                                       (LAS void*)(dst + C::OPA + (wave + i * C::NW) * 1024), 16, 0, 0);
  }
}

// After the barrier of a step: the first loads of step kt + NSTAGE into the
// slot just released and the reads of the next stage's first half, one after
// each of the second half's products, so that the matrix core starts right
// after the barrier (the loads' own latency is never waited for: their
// stage is needed NSTAGE - 1 steps later).  The slot being filled and the
// stage being read always differ, so the reads need no wait on the loads.
template <class C, int DOFF, int NLOAD>
__device__ __forceinline__ void interleave_post() {
  constexpr int NR = tri_reads<C, DOFF>();
  constexpr int NM = tri_products<C, DOFF>();
  constexpr int NL = NLOAD < NM ? NLOAD : NM;
  constexpr int NRD = (NM - NL) < NR ? (NM - NL) : NR;
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  }
#pragma unroll
  for (int q = 0; q < NRD; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  if constexpr (NM > NL + NRD) __builtin_amdgcn_sched_group_barrier(0x008, NM - NL - NRD, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Scheduling pattern for a block of first-half products: one second-half
// fragment read after each product, so the reads stream out while the matrix
// core works and the products never wait on them, then NLOAD operand loads,
// one after each remaining product.
template <class C, int DOFF, int NLOAD = 0>
__device__ __forceinline__ void interleave() {
  constexpr int NR = tri_reads<C, DOFF>();     // fragment reads of a half
  constexpr int NM = tri_products<C, DOFF>();  // products of a half
  constexpr int NP = NR < NM ? NR : NM;
  constexpr int NL = (NM - NP) < NLOAD ? (NM - NP) : NLOAD;
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
  }
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one operand load
  }
  if constexpr (NM > NP + NL) __builtin_amdgcn_sched_group_barrier(0x008, NM - NP - NL, 0);
  if constexpr (NR > NP) __builtin_amdgcn_sched_group_barrier(0x100, NR - NP, 0);
  if constexpr (NLOAD > NL) __builtin_amdgcn_sched_group_barrier(0x010, NLOAD - NL, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Main loop, software pipelined by k16 halves.  Step kt: multiply the first
// half of stage kt (read before) while reading its second half, then (after this
// wave's loads of step kt+1 have landed and its own reads of stage kt have
// completed) a barrier publishes stage kt+1 and frees stage kt, which is
// refilled with step kt+NSTAGE; the first half of stage kt+1 is read while
// the second half of step kt is multiplied.  The barrier's wait is thus
// covered by queued matrix-core work and the next step's first reads.
// A wave's loads of a step are issued in two parts: H1 = PER/2 right after
// the barrier that frees their slot, the rest among the first-half products
// of the next step, before the next barrier.  Issued all at once after the
// barrier, they held up the products queued behind them in the wave's
// in-order stream, and the second wave of each SIMD, which the matrix core
// serves after the first, finished its step alone (measured per wave with
// the shader clock: 2040 cycles per step against 1280 of products per SIMD,
// 1840 with the split).  The second part still lands NSTAGE - 2 steps before
// its stage is read.
// PER (this wave's loads per step) is a template parameter and the steady
// phase has a fixed number of steps in flight, so the loop body has no
// branches and every wait count is an immediate.
template <class C, int PER, bool TR, bool SELF, int DOFF>
__device__ __forceinline__ void main_loop(const __bf16* __restrict__ Aop, const __bf16* __restrict__ Bop,
                                          const Slots<C>& sl, int nk, LAS unsigned char* lds, int wave,
                                          const Frag<C>& f, f32x16_t (&acc)[C::BMB][C::BNB]) {
  constexpr int NS = C::NSTAGE;
  constexpr int H1 = PER / 2;  // loads of a step issued right after its slot's barrier
  // Prologue: steps 0..NS-2 whole, the first part of step NS-1 (its second
  // part goes with the first products, as in the steady phase).
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) issue_loads<C, SELF, PER>(Aop, Bop, sl, st * 32, lds + st * C::STAGEB, wave);
  if (NS - 1 < nk) issue_loads<C, SELF, PER, 0, H1>(Aop, Bop, sl, (NS - 1) * 32, lds + (NS - 1) * C::STAGEB, wave);
  if (nk >= NS) MUON_WAIT_VM((NS - 2) * PER + H1);
  else wait_newer<PER>(nk - 1);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  bf16x8_t fa0[C::BMB], fb0[C::BNB], fa1[C::BMB], fb1[C::BNB];
  read_half<C, TR>(lds, 0, f, fa0, fb0);
  int kt = 0;
  // Steady phase: the first products of step kt carry the second part of
  // step kt+NS-1 (into the slot freed at the previous barrier), the barrier
  // is followed by the first part of step kt+NS.  Every wait leaves NS-2
  // whole later steps in flight.
  for (; kt < nk - NS; ++kt) {
    LAS unsigned char* cur = lds + (kt % NS) * C::STAGEB;
    mfma_half<C, DOFF>(fa0, fb0, acc);
    read_half<C, TR>(cur, 1, f, fa1, fb1);
    issue_loads<C, SELF, PER, H1, PER>(Aop, Bop, sl, (kt + NS - 1) * 32, lds + ((kt + NS - 1) % NS) * C::STAGEB,
                                       wave);
    interleave<C, DOFF, PER - H1>();
    MUON_WAIT_VM((NS - 2) * PER);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage kt are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue_loads<C, SELF, PER, 0, H1>(Aop, Bop, sl, (kt + NS) * 32, cur, wave);
    read_half<C, TR>(lds + ((kt + 1) % NS) * C::STAGEB, 0, f, fa0, fb0);
    mfma_half<C, DOFF>(fa1, fb1, acc);
    interleave_post<C, DOFF, H1>();
  }
  // The step that carries the second part of the last step (nk >= NS).
  if (kt + NS - 1 < nk) {
    LAS unsigned char* cur = lds + (kt % NS) * C::STAGEB;
    mfma_half<C, DOFF>(fa0, fb0, acc);
    read_half<C, TR>(cur, 1, f, fa1, fb1);
    issue_loads<C, SELF, PER, H1, PER>(Aop, Bop, sl, (kt + NS - 1) * 32, lds + ((kt + NS - 1) % NS) * C::STAGEB,
                                       wave);
    interleave<C, DOFF, PER - H1>();
    MUON_WAIT_VM((NS - 2) * PER);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_half<C, TR>(lds + ((kt + 1) % NS) * C::STAGEB, 0, f, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_half<C, DOFF>(fa1, fb1, acc);
    __builtin_amdgcn_sched_barrier(0);
    ++kt;
  }
  // Drain phase: no refills; the steps still in flight land one by one.
  for (; kt + 1 < nk; ++kt) {
    LAS unsigned char* cur = lds + (kt % NS) * C::STAGEB;
    mfma_half<C, DOFF>(fa0, fb0, acc);
    read_half<C, TR>(cur, 1, f, fa1, fb1);
    interleave<C, DOFF>();
    wait_newer<PER>(nk - 2 - kt);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_half<C, TR>(lds + ((kt + 1) % NS) * C::STAGEB, 0, f, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_half<C, DOFF>(fa1, fb1, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  read_half<C, TR>(lds + ((nk - 1) % NS) * C::STAGEB, 1, f, fa1, fb1);
  mfma_half<C, DOFF>(fa0, fb0, acc);
  mfma_half<C, DOFF>(fa1, fb1, acc);
}

// The main loop of a wave with nothing to compute: its sub-tile lies wholly
// below the diagonal of a diagonal tile of a symmetric product (SELF: A half
// only), or wholly in the padding rows of a BX tile.  Its share of the stage
// loads (each step's whole, right after the barrier that frees its slot, and
// landed by the barrier that publishes it) and the same barriers as
// main_loop, and nothing else.
template <class C, int PER, bool SELF>
__device__ __forceinline__ void load_loop(const __bf16* __restrict__ Aop, const __bf16* __restrict__ Bop,
                                          const Slots<C>& sl, int nk, LAS unsigned char* lds, int wave) {
#pragma unroll
  for (int st = 0; st < C::NSTAGE; ++st)
    if (st < nk) issue_loads<C, SELF, PER>(Aop, Bop, sl, st * 32, lds + st * C::STAGEB, wave);
  wait_newer<PER>(nk - 1 < C::NSTAGE - 1 ? nk - 1 : C::NSTAGE - 1);
  __builtin_amdgcn_s_barrier();
  int kt = 0;
  for (; kt < nk - C::NSTAGE; ++kt) {
    MUON_WAIT_VM((C::NSTAGE - 2) * PER);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue_loads<C, SELF, PER>(Aop, Bop, sl, (kt + C::NSTAGE) * 32, lds + (kt % C::NSTAGE) * C::STAGEB, wave);
  }
  for (; kt + 1 < nk; ++kt) {
    wait_newer<PER>(nk - 2 - kt);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
}

// ---------------------------------------------------------------- BX epilogue
// X' = a (X_hi + X_lo) + P X_hi for a wave's sub-tile (WM Gram-side rows
// wi0.., WN = 64 long-side columns wj0..), block by block of 32 rows.
//
// The accumulators of a 32x32 product hold, per lane, column (lane & 31)
// and four runs of four rows; they go to a wave-private float32 tile
// T[jl][il] in LDS (jl: long side, 64 rows; il: Gram side, 64 columns;
// pitch TP = 68 floats, so 16-byte accesses of 16 consecutive rows, or of
// two rows of 8 chunks, hit all 64 banks once).  Passes over T then make
// every global access 16 bytes per lane along contiguous memory.
//
// A row of X^T holds bf16 values, so 32 Gram-side columns are only half of
// a 128-byte line.  Blocks are therefore handled in units: two blocks that
// together cover one 64-aligned line of columns ("pair", W = 64: 8 lanes
// read or write one whole line of each X^T array), or a block alone where
// its neighbour belongs to another wave or tile ("single", W = 32).  With
// WM = 160 a wave has two pairs and one single; with WM = 128, two pairs.
//   X^T-major pass: lane (jl, 8 consecutive il) -> the X^T pair, or W's row
//     gj when the matrix is transposed and this is the last iteration
//     (float32: 32 columns already fill a line);
//   X-major pass (last iteration, matrix not transposed): lane (il, 8
//     consecutive jl) -> W's row gi (256 contiguous bytes per row).
// A wave's LDS operations complete in order; the compiler barriers keep the
// cross-lane exchanges through T in program order.

// Inputs of a unit: NG row groups (one 16-byte access of each X^T array
// per lane and group).
template <int NG>
struct XIn {
  uint4 hi[NG], lo[NG];
};

// Lane -> (row jl, first of 8 columns il) of 16-byte access p of a unit of
// W columns; the same map addresses the X^T pair in memory and the tile T.
template <int W>
__device__ __forceinline__ void unit_pos(int p, int lane, int& jl, int& il) {
  if constexpr (W == 64) {
    jl = p * 8 + (lane >> 3);
    il = (lane & 7) * 8;
  } else {
    jl = p * 16 + (lane & 15);
    il = (lane >> 4) * 8;
  }
}

// The descriptor fields the BX epilogue uses, read once into registers.
// Its stores go through pointers the compiler cannot tell apart from the
// descriptor table, so a field read through the table would be loaded
// again after every store, and waited for, which also drains the LDS reads
// in flight.
struct BxArgs {
  const __bf16* hi_in;  // the pair this launch reads (X^T, ping-pong slot buf)
  const __bf16* lo_in;
  __bf16* hi_out;       // the new pair (slot buf ^ 1)
  __bf16* lo_out;
  float* W;
  int64_t cols;
  int32_t m, n, flags;
  float lr_scale, lr_wd;
};
__device__ __forceinline__ BxArgs bx_args(const MatDesc& d, int buf) {
  BxArgs a;
  a.hi_in = pick(d.xt_hi, buf);
  a.lo_in = pick(d.xt_lo, buf);
  a.hi_out = pick(d.xt_hi, buf ^ 1);
  a.lo_out = pick(d.xt_lo, buf ^ 1);
  a.W = d.W;
  a.cols = d.cols;
  a.m = d.m;
  a.n = d.n;
  a.flags = d.flags;
  a.lr_scale = d.lr_scale;
  a.lr_wd = d.lr_wd;
  return a;
}

// Row group p0 + q of a W-column unit at Gram-side column gi0 -> x[q].
template <int W, int NG>
__device__ __forceinline__ void bx_load_group(const BxArgs& d, int m_pad, int gi0, int wj0, int lane,
                                              XIn<NG>& x, int q, int p0) {
  int jl, il;
  unit_pos<W>(p0 + q, lane, jl, il);
  const int64_t off = static_cast<int64_t>(wj0 + jl) * m_pad + gi0 + il;
  x.hi[q] = gld<uint4>(d.hi_in + off);
  x.lo[q] = gld<uint4>(d.lo_in + off);
}

// Accumulators of one 32-row block -> T columns co..co+31.
template <class C>
__device__ __forceinline__ void bx_stage_acc(int lane, const f32x16_t (&acc)[C::BNB], float* T) {
  const int col = lane & 31;
  const int rq = 4 * (lane >> 5);
#pragma unroll
  for (int j = 0; j < C::BNB; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 v = make_float4(acc[j][4 * g], acc[j][4 * g + 1], acc[j][4 * g + 2], acc[j][4 * g + 3]);
      *reinterpret_cast<float4*>(T + (j * 32 + col) * C::TP + 8 * g + rq) = v;
    }
  asm volatile("" ::: "memory");
}

// W <- W - lr*wd*W - lr*scale*O, as fma(-ls, O, fma(-lwd, W, W)), on four
// consecutive elements (16-byte aligned) or one; orthogonalise-only mode
// stores O itself.
template <bool DG>
__device__ __forceinline__ void upd4(float* wp, float4 o, float ls, float lwd, bool ortho, DiagAcc& da) {
  if (ortho) {
    gst(wp, o);
    return;
  }
  const float4 w = gld<float4>(wp);
  const float4 nw = make_float4(fmaf(-ls, o.x, fmaf(-lwd, w.x, w.x)), fmaf(-ls, o.y, fmaf(-lwd, w.y, w.y)),
                                fmaf(-ls, o.z, fmaf(-lwd, w.z, w.z)), fmaf(-ls, o.w, fmaf(-lwd, w.w, w.w)));
  if constexpr (DG) {
    diag_add(da, o.x, w.x, nw.x);
    diag_add(da, o.y, w.y, nw.y);
    diag_add(da, o.z, w.z, nw.z);
    diag_add(da, o.w, w.w, nw.w);
  }
  gst(wp, nw);
}
// upd4 with the old W values already loaded (w).
template <bool DG>
__device__ __forceinline__ void upd4w(float* wp, float4 o, float4 w, float ls, float lwd, DiagAcc& da) {
  const float4 nw = make_float4(fmaf(-ls, o.x, fmaf(-lwd, w.x, w.x)), fmaf(-ls, o.y, fmaf(-lwd, w.y, w.y)),
                                fmaf(-ls, o.z, fmaf(-lwd, w.z, w.z)), fmaf(-ls, o.w, fmaf(-lwd, w.w, w.w)));
  if constexpr (DG) {
    diag_add(da, o.x, w.x, nw.x);
    diag_add(da, o.y, w.y, nw.y);
    diag_add(da, o.z, w.z, nw.z);
    diag_add(da, o.w, w.w, nw.w);
  }
  gst(wp, nw);
}
template <bool DG>
__device__ __forceinline__ void upd1(float* wp, float o, float ls, float lwd, bool ortho, DiagAcc& da) {
  if (ortho) {
    gst(wp, o);
    return;
  }
  const float w = gld<float>(wp);
  const float nw = fmaf(-ls, o, fmaf(-lwd, w, w));
  if constexpr (DG) diag_add(da, o, w, nw);
  gst(wp, nw);
}

// The passes over row groups p0 .. p0 + NG - 1 of a unit of W Gram-side
// columns gi0.. staged in T (all of the unit, or one wave's half of a
// merged unit).  While they are finished, the inputs of the next unit (NG2
// groups of a W2-column unit at gi0n from group p0n; NG2 = 0: none) are
// requested group by group, so about one unit of inputs is in flight at
// any time.  The X-major pass covers Gram-side columns 8 q0 .. 8 (q0 + NG).
template <class C, int MODE, int W, int NG, int W2, int NG2, bool MERGED>
__device__ __forceinline__ void bx_pass(const BxArgs& d, int m_pad, int gi0, int wj0, int lane,
                                        float* T, const XIn<NG>& x, int p0, int q0, DiagAcc& da,
                                        XIn<(NG2 > 0 ? NG2 : 1)>& nx, int gi0n, int p0n, float s1) {
  constexpr bool DG = MODE == BXD;
  const bool tr = d.flags & kTransposed;
  const bool ortho = d.flags & kOrthoOnly;
  const float ls = d.lr_scale;
  const float lwd = d.lr_wd;
  const bool w16 = (d.cols & 3) == 0;  // W rows 16-byte aligned (W itself is, per the API)
  const bool need_xmajor = (MODE >= BXL) && !tr;
  // X^T-major pass
#pragma unroll
  for (int p = 0; p < NG; ++p) {
    if constexpr (NG2 > 0) {
#pragma unroll
      for (int q = p * NG2 / NG; q < (p + 1) * NG2 / NG; ++q)
        bx_load_group<W2>(d, m_pad, gi0n, wj0, lane, nx, q, p0n);
    }
    int jl, il;
    unit_pos<W>(p0 + p, lane, jl, il);
    float* tp = T + jl * C::TP + il;
    const float4 t0 = *reinterpret_cast<const float4*>(tp);
    const float4 t1 = *reinterpret_cast<const float4*>(tp + 4);
    float v[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
    const uint32_t hw[4] = {x.hi[p].x, x.hi[p].y, x.hi[p].z, x.hi[p].w};
    const uint32_t lw[4] = {x.lo[p].x, x.lo[p].y, x.lo[p].z, x.lo[p].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = fmaf(kCoefA, bf_lo(hw[q]) + bf_lo(lw[q]), v[2 * q]);
      v[2 * q + 1] = fmaf(kCoefA, bf_hi(hw[q]) + bf_hi(lw[q]), v[2 * q + 1]);
    }
    if (s1 != 1.f) {  // first iteration on the unnormalised pair
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= s1;
    }
    const int gj = wj0 + jl;
    const int gi = gi0 + il;
    if (MODE == BXM) {
      uint32_t nh[4], nl[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        nh[q] = pack_bf16(v[2 * q], v[2 * q + 1]);
        nl[q] = pack_bf16(v[2 * q] - bf_lo(nh[q]), v[2 * q + 1] - bf_hi(nh[q]));
      }
      // The new pair is read again only by the next iteration's Gram
      // product, after the whole launch: stream it past the caches.
      const int64_t off = static_cast<int64_t>(gj) * m_pad + gi;
      gst_stream(d.hi_out + off, make_uint4(nh[0], nh[1], nh[2], nh[3]));
      gst_stream(d.lo_out + off, make_uint4(nl[0], nl[1], nl[2], nl[3]));
    } else if (tr) {
      // O^T = X'^T has W's orientation: W[gj][gi .. gi+7].
      if (gj < d.n) {
        float* wp = d.W + static_cast<int64_t>(gj) * d.cols + gi;
        if (gi + 7 < d.m && w16) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float4 o = make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
            upd4<DG>(wp + 4 * h, o, ls, lwd, ortho, da);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gi + e < d.m) upd1<DG>(wp + e, v[e], ls, lwd, ortho, da);
        }
      }
    }
    if (need_xmajor) {
      *reinterpret_cast<float4*>(tp) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(tp + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    // Keep the accesses of one row group together: hoisting every group's
    // tile reads ahead would hold W / 8 rows of values at once.
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!need_xmajor) return;
  // The X-major pass reads rows of T that the other wave of a merged unit
  // wrote back (uniform over the work-group: one matrix per tile).
  if constexpr (MERGED) __syncthreads();
  asm volatile("" ::: "memory");
  // X-major pass (non-transposed matrix, last iteration: W[gi][gj .. gj+7]),
  // WB row groups at a time: their rows of W are all requested before the
  // first of them is written (WB = 1 with diagnostics, whose sums take the
  // registers).
  constexpr int WB = DG ? 1 : 2;
  static_assert(NG % WB == 0, "X-major pass in batches of WB row groups");
#pragma unroll
  for (int qb = 0; qb < NG; qb += WB) {
    float4 wv[WB][2];
#pragma unroll
    for (int qq = 0; qq < WB; ++qq) {
      const int il = (q0 + qb + qq) * 8 + (lane & 7);
      const int gi = gi0 + il, gj = wj0 + (lane >> 3) * 8;
      if (!ortho && gi < d.m && gj + 7 < d.n && w16) {
        const float* wp = d.W + static_cast<int64_t>(gi) * d.cols + gj;
        wv[qq][0] = gld<float4>(wp);
        wv[qq][1] = gld<float4>(wp + 4);
      }
    }
#pragma unroll
    for (int qq = 0; qq < WB; ++qq) {
      const int il = (q0 + qb + qq) * 8 + (lane & 7);
      const int jl = (lane >> 3) * 8;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = T[(jl + e) * C::TP + il];
      const int gi = gi0 + il;
      const int gj = wj0 + jl;
      if (gi < d.m) {
        float* wp = d.W + static_cast<int64_t>(gi) * d.cols + gj;
        if (gj + 7 < d.n && w16) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float4 o = make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
            if (ortho)
              gst(wp + 4 * h, o);
            else
              upd4w<DG>(wp + 4 * h, o, wv[qq][h], ls, lwd, da);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gj + e < d.n) upd1<DG>(wp + e, v[e], ls, lwd, ortho, da);
        }
      }
    }
  }
  asm volatile("" ::: "memory");
}

// Units of a wave whose first block starts at an even (PH = 0) or odd
// (PH = 1) multiple of 32 Gram-side rows: the line-aligned pairs first
// (blocks 0-1, 2-3, ... or 1-2, 3-4, ...), then the blocks left alone (the
// last one, then block 0), so the accumulators of a leading single stay in
// registers while the pairs, which need the most input registers, run.
template <class C, int PH>
struct Units {
  static constexpr int NP = PH ? (C::BMB - 1) / 2 : C::BMB / 2;
  static constexpr bool tail = PH ? (C::BMB % 2 == 0) : (C::BMB % 2 == 1);
  static constexpr int N = NP + (tail ? 1 : 0) + PH;
  static constexpr bool pair(int k) { return k < NP; }
  static constexpr int start(int k) { return k < NP ? PH + 2 * k : (k == NP && tail) ? C::BMB - 1 : 0; }
  static constexpr int width(int k) { return pair(k) ? 64 : 32; }
};

template <class C, int PH, int K>
__device__ __forceinline__ void bx_stage_unit(int lane, const f32x16_t (&acc)[C::BMB][C::BNB], float* T) {
  using U = Units<C, PH>;
  bx_stage_acc<C>(lane, acc[U::start(K)], T);
  if constexpr (U::pair(K)) bx_stage_acc<C>(lane, acc[U::start(K) + 1], T + 32);
}

// Row groups of the first unit requested before the barrier that ends the
// main loop (their latency overlaps the last products and the barrier);
// the rest after its accumulators are staged.
constexpr int kEarly = 4;

// Unit K is staged in T and its inputs are requested (or in flight): its
// passes run while the next unit's inputs are requested, then the next
// unit's accumulators go to T (after this unit's last read of T).
template <class C, int MODE, int PH, int K>
__device__ __forceinline__ void bx_units(const BxArgs& d, int m_pad, int wi0, int wj0, int lane, float* T,
                                         const f32x16_t (&acc)[C::BMB][C::BNB],
                                         const XIn<Units<C, PH>::width(K) / 8>& cur, DiagAcc& da, float s1) {
  using U = Units<C, PH>;
  constexpr int W = U::width(K);
  const int gi0 = wi0 + 32 * U::start(K);
  if constexpr (K + 1 < U::N) {
    constexpr int W2 = U::width(K + 1);
    XIn<W2 / 8> nxt;
    bx_pass<C, MODE, W, W / 8, W2, W2 / 8, false>(d, m_pad, gi0, wj0, lane, T, cur, 0, 0, da, nxt,
                                                  wi0 + 32 * U::start(K + 1), 0, s1);
    bx_stage_unit<C, PH, K + 1>(lane, acc, T);
    bx_units<C, MODE, PH, K + 1>(d, m_pad, wi0, wj0, lane, T, acc, nxt, da, s1);
  } else {
    XIn<1> none;
    bx_pass<C, MODE, W, W / 8, 32, 0, false>(d, m_pad, gi0, wj0, lane, T, cur, 0, 0, da, none, 0, 0, s1);
  }
}

// The epilogue of a wave that handles its blocks alone: the first unit's
// accumulators go to T (freeing their registers), its inputs are
// requested, then the units run in turn.
template <class C, int MODE, int PH>
__device__ __forceinline__ void bx_epilogue(const BxArgs& d, int m_pad, int wi0, int wj0, int lane, float* T,
                                            const f32x16_t (&acc)[C::BMB][C::BNB], DiagAcc& da, float s1) {
  using U = Units<C, PH>;
  constexpr int W = U::width(0);
  XIn<W / 8> x0;
  constexpr int E = kEarly < W / 8 ? kEarly : W / 8;
#pragma unroll
  for (int q = 0; q < E; ++q) bx_load_group<W>(d, m_pad, wi0 + 32 * U::start(0), wj0, lane, x0, q, 0);
  __syncthreads();  // every wave is done with the ring that T overlaps
  bx_stage_unit<C, PH, 0>(lane, acc, T);
#pragma unroll
  for (int q = E; q < W / 8; ++q) bx_load_group<W>(d, m_pad, wi0 + 32 * U::start(0), wj0, lane, x0, q, 0);
  bx_units<C, MODE, PH, 0>(d, m_pad, wi0, wj0, lane, T, acc, x0, da, s1);
}

// The epilogue of a wave pair that splits a tile's Gram-side rows at an odd
// multiple of 32 (two waves of WM = 160 rows in a 320-row tile): each wave
// has two pairs of its own, and its remaining block shares a line with the
// other wave's.  That line is merged: both blocks go to the T tile of the
// upper wave (H = 0; the lower wave's block to columns 32..63, after a
// barrier that ends the upper wave's own passes over that tile), and each
// wave finishes half of the line's rows after a second barrier.  H = 0:
// pairs (0,1), (2,3), shared block 4; H = 1: pairs (1,2), (3,4), shared
// block 0.
template <class C, int MODE, int H>
__device__ __forceinline__ void bx_epilogue_merged(const BxArgs& d, int m_pad, int wi0, int wj0, int lane,
                                                   float* T, float* Tm, const f32x16_t (&acc)[C::BMB][C::BNB],
                                                   DiagAcc& da, float s1) {
  static_assert(C::BMB == 5, "merged epilogue: two pairs and one shared block per wave");
  constexpr int I0 = H, I1 = H + 2, MB = H ? 0 : 4;
  const int g0 = wi0 + 32 * I0, g1 = wi0 + 32 * I1;
  const int gm = wi0 + 32 * MB - 32 * H;  // first column of the shared line
  XIn<8> x0, x1;
#pragma unroll
  for (int q = 0; q < kEarly; ++q) bx_load_group<64>(d, m_pad, g0, wj0, lane, x0, q, 0);
  __syncthreads();  // every wave is done with the ring that T overlaps
  bx_stage_acc<C>(lane, acc[I0], T);
  bx_stage_acc<C>(lane, acc[I0 + 1], T + 32);
#pragma unroll
  for (int q = kEarly; q < 8; ++q) bx_load_group<64>(d, m_pad, g0, wj0, lane, x0, q, 0);
  bx_pass<C, MODE, 64, 8, 64, 8, false>(d, m_pad, g0, wj0, lane, T, x0, 0, 0, da, x1, g1, 0, s1);
  bx_stage_acc<C>(lane, acc[I1], T);
  bx_stage_acc<C>(lane, acc[I1 + 1], T + 32);
  XIn<4> xm;
  bx_pass<C, MODE, 64, 8, 64, 4, false>(d, m_pad, g1, wj0, lane, T, x1, 0, 0, da, xm, gm, 4 * H, s1);
  __syncthreads();
  bx_stage_acc<C>(lane, acc[MB], Tm + 32 * H);
  __syncthreads();
  XIn<1> none;
  bx_pass<C, MODE, 64, 4, 32, 0, true>(d, m_pad, gm, wj0, lane, Tm, xm, 4 * H, 4 * H, da, none, 0, 0, s1);
}

// Epilogue of a symmetric product (Gram, polynomial) for one wave's sub-tile
// (WM Gram-side rows wi0.., WN = 64 columns wj0..), two 32-row blocks (one
// 128-byte line of columns of the mirror half) at a time, through the
// wave's LDS slice so that every global access is 16 bytes per lane along
// a row:
//   1. (polynomial) the input A at the mirror positions, A[gj][gi..], as
//      rows of the slice M[jl][il] (A is symmetric: these are the values
//      the accumulators need);
//   2. the results in accumulator layout (column gj per lane, runs of four
//      rows gi) rounded to bf16 and written to M[jl][il..il+3] (for the
//      polynomial in place of the A values they use);
//   3. rows of M to the mirror half, P[gj][gi..] (8 lanes per 128 bytes);
//   4. the same words, kept in registers, to a row-major slice S[il][jl]
//      (same LDS), whose rows go to the direct half, P[gi][gj..].
// On a diagonal tile (DIAG) both halves are written from the elements with
// gi <= gj only, so the two triangles hold bit-identical values.
template <class C, int MODE, bool DIAG>
__device__ __forceinline__ void sym_epilogue(const MatDesc& d, int m_pad, int wi0, int wj0, int lane, __bf16* slice,
                                             const f32x16_t (&acc)[C::BMB][C::BNB], float gscale) {
  static_assert(C::BMB % 2 == 0 && C::WN == 64, "block pairs of 64 rows, 64-column wave tiles");
  constexpr int LD = C::SLICE_LD;
  constexpr int NIT = 64 * 8 / 64;     // 16-byte chunks per lane of a 64 x 64 slice
  __bf16* rdst = (MODE == POLY) ? d.poly : d.gram;
  const int col = lane & 31;
  const int rq = 4 * (lane >> 5);
#pragma unroll
  for (int pr = 0; pr < C::BMB / 2; ++pr) {
    const int gi0 = wi0 + 64 * pr;
    if constexpr (MODE == POLY) {
#pragma unroll
      for (int t = 0; t < NIT; ++t) {
        const int jl = t * 8 + (lane >> 3), ch = lane & 7;
        *reinterpret_cast<uint4*>(slice + jl * LD + 8 * ch) =
            gld<uint4>(d.gram + static_cast<int64_t>(wj0 + jl) * m_pad + gi0 + 8 * ch);
      }
      asm volatile("" ::: "memory");
    }
    uint32_t w[2][C::BNB][4][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < C::BNB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2* mp = reinterpret_cast<uint2*>(slice + (32 * j + col) * LD + 32 * h + 8 * g + rq);
          const f32x16_t& a = acc[2 * pr + h][j];
          float v[4] = {a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
          if constexpr (MODE == GRAM) {
            // The first iteration's operand is the unnormalised pair
            // (gscale = sigma^2), later ones 1.
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] *= gscale;
          }
          if constexpr (MODE == POLY) {
            const uint2 av = *mp;  // A[gj][gi..gi+3] == A[gi..gi+3][gj]
            v[0] = fmaf(kCoefC, v[0], kCoefB * bf_lo(av.x));
            v[1] = fmaf(kCoefC, v[1], kCoefB * bf_hi(av.x));
            v[2] = fmaf(kCoefC, v[2], kCoefB * bf_lo(av.y));
            v[3] = fmaf(kCoefC, v[3], kCoefB * bf_hi(av.y));
          }
          w[h][j][g][0] = pack_bf16(v[0], v[1]);
          w[h][j][g][1] = pack_bf16(v[2], v[3]);
          *mp = make_uint2(w[h][j][g][0], w[h][j][g][1]);
        }
    asm volatile("" ::: "memory");
    // Mirror half: row gj of the slice holds P[gj][gi0 .. gi0 + 63].
#pragma unroll
    for (int t = 0; t < NIT; ++t) {
      const int jl = t * 8 + (lane >> 3), ch = lane & 7;
      const int gj = wj0 + jl, gi = gi0 + 8 * ch;
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
    asm volatile("" ::: "memory");
    // Direct half: the same words, row-major.
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < C::BNB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int rl = 32 * h + 8 * g + rq, cl = 32 * j + col;
          const uint16_t hb[4] = {static_cast<uint16_t>(w[h][j][g][0]), static_cast<uint16_t>(w[h][j][g][0] >> 16),
                                  static_cast<uint16_t>(w[h][j][g][1]), static_cast<uint16_t>(w[h][j][g][1] >> 16)};
#pragma unroll
          for (int r = 0; r < 4; ++r) __builtin_memcpy(slice + (rl + r) * LD + cl, &hb[r], 2);
        }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < NIT; ++t) {
      const int il = t * 8 + (lane >> 3), ch = lane & 7;
      const int gi = gi0 + il, gj = wj0 + 8 * ch;
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
    asm volatile("" ::: "memory");
  }
}

template <class C, int MODE>
__global__ __launch_bounds__(C::kThreads, C::MINB) void ns_gemm32_kernel(
    const MatDesc* __restrict__ descs, const int32_t* __restrict__ prefix, int nmats, XcdSplit split, int buf,
    int first) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDSB];

  // XCD-aware work: XCD (block id % 8) walks its own cost-balanced
  // contiguous range of (matrix, tile) work.
  const int work = split.begin[blockIdx.x & 7] + static_cast<int>(blockIdx.x >> 3);
  if (work >= split.end[blockIdx.x & 7]) return;
  const int mi = find_mat(prefix, nmats, work);
  const MatDesc& dr = descs[mi];  // operands and sizes, read before any store
  int local = work - prefix[mi];
  const int m_pad = dr.m_pad, n_pad = dr.n_pad;

  int ti, tj;
  if (MODE >= BXM) {
    // Grouped order: groups of bx_group Gram-side tile rows; inside a group
    // the long-side index is slow and the Gram-side index fast, so tiles
    // that run together share X^T panels, and the group's rows of P stay
    // in L2 while the group sweeps the long side.
    const int tpc = m_pad / C::BM;
    const int tpr = n_pad / C::BN;
    const int g = dr.bx_group;
    const int grp = local / (g * tpr);
    const int rows = min(g, tpc - grp * g);
    const int rem = local - grp * g * tpr;
    tj = rem / rows;
    ti = grp * g + (rem - tj * rows);
  } else {
    const int nt = m_pad / C::BM;
    ti = 0;
    while (local >= nt - ti) {
      local -= nt - ti;
      ++ti;
    }
    tj = ti + local;
  }

  // Operands.  The Gram product reads X^T (n_pad x m_pad, the iterate's
  // own layout): its tiles are 32 k-rows x BM columns, transposed on the
  // way out of LDS.  The others read row-major rows of A, P and X^T.
  constexpr bool TR = MODE == GRAM;
  const __bf16* __restrict__ Aop;
  const __bf16* __restrict__ Bop;
  int ld, K;
  if (MODE == GRAM) {
    Aop = pick(dr.xt_hi, buf) + static_cast<int64_t>(ti) * C::BM;
    Bop = pick(dr.xt_hi, buf) + static_cast<int64_t>(tj) * C::BN;
    ld = m_pad;
    K = dr.k_gram;
  } else if (MODE == POLY) {
    Aop = dr.gram + static_cast<int64_t>(ti) * C::BM * m_pad;
    Bop = dr.gram + static_cast<int64_t>(tj) * C::BN * m_pad;
    ld = K = m_pad;
  } else {
    Aop = dr.poly + static_cast<int64_t>(ti) * C::BM * m_pad;
    Bop = pick(dr.xt_hi, buf) + static_cast<int64_t>(tj) * C::BN * m_pad;
    ld = K = m_pad;
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int wr = wave / C::NWN, wc = wave - wr * C::NWN;
  // Diagonal tile of a symmetric product (G256, 2 x 4 waves of 128 x 64):
  // two sub-tiles lie wholly below the diagonal (nothing to compute), four
  // straddle it (3 or 7 of their 8 blocks needed) and two lie above it.
  // Waves w and w + 4 share a SIMD, so the sub-tiles are dealt to pair a
  // full one with an empty one and a 7-block one with a 3-block one: every
  // SIMD then has at most 10 of the 16 block products of a full tile.
  if constexpr (MODE < BXM && C::NWM == 2 && C::NWN == 4 && C::BMB == 4 && C::BNB == 2) {
    if (ti == tj) {
      constexpr int kR[8] = {0, 0, 0, 1, 1, 1, 1, 0};
      constexpr int kC[8] = {2, 3, 1, 3, 0, 1, 2, 0};
      wr = kR[wave];
      wc = kC[wave];
    }
  }
  // BX tile (W320) whose last wave columns lie wholly in padding rows of X^T
  // (at or past k_gram, which no valid result reads): those waves only load.
  // With one or two valid wave columns the sub-tiles are dealt so that the
  // valid ones sit on different SIMDs (waves w and w + 4 share one); the
  // wave of sub-tile (0, c) keeps index c, whose LDS tile the merged
  // epilogue uses.
  int bx_valid = C::NWN;
  if constexpr (MODE >= BXM && C::NWM == 2 && C::NWN == 4 && C::WM % 64 == 32 && C::BM % 64 == 0) {
    const int rem = dr.k_gram - tj * C::BN;
    bx_valid = rem >= C::BN ? C::NWN : (rem + C::WN - 1) / C::WN;
    if (bx_valid == 1) {
      constexpr int kR[8] = {0, 1, 0, 0, 0, 1, 1, 1};
      constexpr int kC[8] = {0, 0, 1, 2, 3, 1, 2, 3};
      wr = kR[wave];
      wc = kC[wave];
    } else if (bx_valid == 2) {
      constexpr int kR[8] = {0, 0, 1, 1, 0, 0, 1, 1};
      constexpr int kC[8] = {0, 1, 0, 1, 2, 3, 2, 3};
      wr = kR[wave];
      wc = kC[wave];
    }
  }
  const bool bx_pad = wc >= bx_valid;

  Slots<C> sl;
  Frag<C> fr;
  if constexpr (TR) {
    // Stage layout of a transposed operand: 32 k-rows of NC = BM/8 16-byte
    // chunks (8 consecutive columns each); chunk c of k-row k sits at
    // position (c + 4 (k & 3)) mod NC, which keeps the transposing fragment
    // reads free of bank conflicts (measured on gfx950).  Load instruction q
    // fills positions 64q..64q+63 in order, one 16-byte chunk per lane.
    static_assert(C::BM == C::BN && (C::BM == 128 || C::BM == 256), "transposed operands: 128- or 256-wide tiles");
    constexpr int NC = C::BM / 8;
    constexpr int RP = 2 * C::BM;
#pragma unroll
    for (int i = 0; i < C::QAMAX; ++i) {
      const int p = (wave + i * C::NW) * 64 + lane;
      const int k = p / NC;
      const int c = (p - 4 * (k & 3)) & (NC - 1);
      sl.aoff[i] = k * ld + c * 8;
    }
#pragma unroll
    for (int i = 0; i < C::QBMAX; ++i) {
      const int p = (wave + i * C::NW) * 64 + lane;
      const int k = p / NC;
      const int c = (p - 4 * (k & 3)) & (NC - 1);
      sl.boff[i] = k * ld + c * 8;
    }
    sl.kmul = ld;
    // Fragment reads: in each 16-lane group g, lane 4a + j' reads the 4
    // columns 4a.. of k-row 8 (g >> 1) + j (j = (lane & 15) >> 2, the
    // source-row index of the transposing read) so that output lane l gets
    // row (l & 31) at 4 consecutive k.
    const int g = lane >> 4, aa = lane & 3, j = (lane & 15) >> 2;
    const int krow = 8 * (g >> 1) + j;
#pragma unroll
    for (int ib = 0; ib < C::BMB; ++ib) {
      const int c = (wr * C::WM + 32 * ib + 16 * (g & 1) + 4 * aa) >> 3;
      fr.a[ib] = krow * RP + ((c + 4 * j) & (NC - 1)) * 16 + (aa & 1) * 8;
    }
#pragma unroll
    for (int jb = 0; jb < C::BNB; ++jb) {
      const int c = (wc * C::WN + 32 * jb + 16 * (g & 1) + 4 * aa) >> 3;
      fr.b[jb] = C::OPA + krow * RP + ((c + 4 * j) & (NC - 1)) * 16 + (aa & 1) * 8;
    }
  } else {
    // Load slots: instruction q covers operand rows 16q..16q+15, lane l
    // fills LDS position l%4 of row 16q + l/4 with the k-chunk the swizzle
    // maps there.  Rows of one wave's successive slots are NW*16 apart,
    // which leaves the swizzle unchanged.
    const int r0 = wave * 16 + (lane >> 2);
    const int c0 = swz(r0, lane & 3);
#pragma unroll
    for (int i = 0; i < C::QAMAX; ++i) sl.aoff[i] = (r0 + i * C::NW * 16) * ld + c0 * 8;
#pragma unroll
    for (int i = 0; i < C::QBMAX; ++i) sl.boff[i] = (r0 + i * C::NW * 16) * ld + c0 * 8;
    sl.kmul = 1;
    const int a_row0 = wr * C::WM + (lane & 31), b_row0 = wc * C::WN + (lane & 31);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = h * 2 + (lane >> 5);
      fr.a[h] = a_row0 * 64 + swz(a_row0, c) * 16;
      fr.b[h] = C::OPA + b_row0 * 64 + swz(b_row0, c) * 16;
    }
  }
  const int na = (C::QA - wave + C::NW - 1) / C::NW;
  const int nb = (C::QB - wave + C::NW - 1) / C::NW;
  const int per = na + nb;

  f32x16_t acc[C::BMB][C::BNB];
#pragma unroll
  for (int i = 0; i < C::BMB; ++i)
#pragma unroll
    for (int j = 0; j < C::BNB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = K / 32;
  LAS unsigned char* lds = (LAS unsigned char*)smem;
  constexpr int PER_FULL = C::QAMAX + C::QBMAX;
  // A diagonal tile of a symmetric product multiplies a panel by itself: its
  // stages hold the panel once (A half) and the B fragments are read there.
  const bool self = MODE < BXM && ti == tj;
  // In a diagonal tile: sub-tiles wholly below the diagonal only load;
  // sub-tiles straddling it skip their blocks below it (DOFF = offset of
  // the column blocks from the row blocks, in 32-row blocks).
  bool below = false;
  if constexpr (MODE < BXM) {
    if (self) {
#pragma unroll
      for (int j = 0; j < (C::BNB > 2 ? C::BNB : 2); ++j) fr.b[j] -= C::OPA;
      below = wr * C::WM >= (wc + 1) * C::WN;
      const bool above = wr * C::WM + C::WM - 1 <= wc * C::WN;
      const int doff = (wc * C::WN - wr * C::WM) / 32;
      static_assert(C::QAMAX >= 2, "diagonal-tile loops assume two A loads per wave and step");
      if (below) {
        if (na == C::QAMAX) load_loop<C, C::QAMAX, true>(Aop, Bop, sl, nk, lds, wave);
        else load_loop<C, C::QAMAX - 1, true>(Aop, Bop, sl, nk, lds, wave);
      } else if (above || !(C::BMB == 4 && C::BNB == 2 && (doff == 0 || doff == 2))) {
        if (na == C::QAMAX) main_loop<C, C::QAMAX, TR, true, -1>(Aop, Bop, sl, nk, lds, wave, fr, acc);
        else main_loop<C, C::QAMAX - 1, TR, true, -1>(Aop, Bop, sl, nk, lds, wave, fr, acc);
      } else if (doff == 0) {
        if (na == C::QAMAX) main_loop<C, C::QAMAX, TR, true, 0>(Aop, Bop, sl, nk, lds, wave, fr, acc);
        else main_loop<C, C::QAMAX - 1, TR, true, 0>(Aop, Bop, sl, nk, lds, wave, fr, acc);
      } else {
        if (na == C::QAMAX) main_loop<C, C::QAMAX, TR, true, 2>(Aop, Bop, sl, nk, lds, wave, fr, acc);
        else main_loop<C, C::QAMAX - 1, TR, true, 2>(Aop, Bop, sl, nk, lds, wave, fr, acc);
      }
    }
  }
  // (B loads are spread evenly over the waves: per is PER_FULL or one less.)
  if (!self && bx_pad) {
    if (per == PER_FULL) load_loop<C, PER_FULL, false>(Aop, Bop, sl, nk, lds, wave);
    else load_loop<C, PER_FULL - 1, false>(Aop, Bop, sl, nk, lds, wave);
  } else if (!self) {
    if (per == PER_FULL) main_loop<C, PER_FULL, TR, false, -1>(Aop, Bop, sl, nk, lds, wave, fr, acc);
    else main_loop<C, PER_FULL - 1, TR, false, -1>(Aop, Bop, sl, nk, lds, wave, fr, acc);
  }
  // The epilogue's LDS tiles overlap the ring: a barrier first (the BX
  // epilogues take it themselves, after requesting their first inputs).
  if constexpr (MODE < BXM) __syncthreads();
  if (below) return;  // nothing of its sub-tile is stored
  // The epilogue reads the descriptor through the table: a copy (see
  // MatDesc) measured 1% slower here.
  const MatDesc& d = dr;
  // First iteration: the iterate is the unnormalised pair of M; its Gram
  // product is scaled by s1^2 and the BX result by s1 (s1 = sigma, or 1
  // where the prep pass already normalised).
  const float s1 = first ? gld<float>(d.sigma + kSigFirst) : 1.f;

  // ---- epilogue (wave-local).
  const int wi0 = ti * C::BM + wr * C::WM;   // first global row of the wave's sub-tile
  const int wj0 = tj * C::BN + wc * C::WN;   // first global column
  if constexpr (MODE >= BXM) {
    float* T = reinterpret_cast<float*>(smem) + wave * (C::SLICEB / 4);
    const BxArgs ba = bx_args(d, buf);
    DiagAcc da;
    if constexpr (C::NWM == 2 && C::WM % 64 == 32 && C::BM % 64 == 0) {
      // The two waves of a column share the line at row WM - 32 of the tile.
      float* Tm = reinterpret_cast<float*>(smem) + wc * (C::SLICEB / 4);
      if (bx_pad) {
        // Nothing to store; the barriers of bx_epilogue_merged (the first,
        // the two around the shared line, and the X-major pass's).
        const bool need_xmajor = (MODE >= BXL) && !(d.flags & kTransposed);
        __syncthreads();
        __syncthreads();
        __syncthreads();
        if (need_xmajor) __syncthreads();
      } else if (wr == 0)
        bx_epilogue_merged<C, MODE, 0>(ba, m_pad, wi0, wj0, lane, T, Tm, acc, da, s1);
      else
        bx_epilogue_merged<C, MODE, 1>(ba, m_pad, wi0, wj0, lane, T, Tm, acc, da, s1);
    } else if (((wi0 >> 5) & 1) == 0) {
      // Wave-uniform: whether the wave's first block starts a 64-row line.
      bx_epilogue<C, MODE, 0>(ba, m_pad, wi0, wj0, lane, T, acc, da, s1);
    } else {
      bx_epilogue<C, MODE, 1>(ba, m_pad, wi0, wj0, lane, T, acc, da, s1);
    }
    if constexpr (MODE == BXD) diag_flush(da, d.diag_part + local * C::NW + wave, lane);
    return;
  }
  if constexpr (MODE == GRAM || MODE == POLY) {
    __bf16* slice = reinterpret_cast<__bf16*>(smem) + wave * (C::SLICEB / 2);
    const float gscale = (MODE == GRAM && first) ? s1 * s1 : 1.f;
    if (ti == tj)
      sym_epilogue<C, MODE, true>(d, m_pad, wi0, wj0, lane, slice, acc, gscale);
    else
      sym_epilogue<C, MODE, false>(d, m_pad, wi0, wj0, lane, slice, acc, gscale);
  }
}

using G256 = G32<256, 256, 2, 4, 4>;
using W160 = G32<160, 256, 1, 4, 3>;
using W320 = G32<320, 256, 2, 4, 4>;
// G128: G256's arithmetic (32x32x16 products, same k order and epilogues,
// hence the same bits) on 128 x 128 tiles of 2 x 2 waves of 64 x 64.
using G128 = G32<128, 128, 2, 2, 4>;

template <class C, int MODE>
hipError_t launch(const MatDesc* d, const int32_t* prefix, int nmats, const XcdSplit& sp, int buf, int first,
                  hipStream_t s) {
  if (sp.max_len <= 0) return hipSuccess;
  hipLaunchKernelGGL((ns_gemm32_kernel<C, MODE>), dim3(8 * sp.max_len), dim3(C::kThreads), 0, s, d, prefix, nmats, sp,
                     buf, first);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_gemm32(int mode, int cfg, const MatDesc* d, const int32_t* prefix, int nmats,
                            const XcdSplit& split, int buf, int first, hipStream_t s) {
  if (cfg == kCfgG256) {
    if (mode == GRAM) return launch<G256, GRAM>(d, prefix, nmats, split, buf, first, s);
    if (mode == POLY) return launch<G256, POLY>(d, prefix, nmats, split, buf, first, s);
    if (mode == BXM) return launch<G256, BXM>(d, prefix, nmats, split, buf, first, s);
    if (mode == BXL) return launch<G256, BXL>(d, prefix, nmats, split, buf, first, s);
    if (mode == BXD) return launch<G256, BXD>(d, prefix, nmats, split, buf, first, s);
    return hipErrorInvalidValue;
  }
  if (cfg == kCfgG128) {
    if (mode == GRAM) return launch<G128, GRAM>(d, prefix, nmats, split, buf, first, s);
    if (mode == POLY) return launch<G128, POLY>(d, prefix, nmats, split, buf, first, s);
    if (mode == BXM) return launch<G128, BXM>(d, prefix, nmats, split, buf, first, s);
    if (mode == BXL) return launch<G128, BXL>(d, prefix, nmats, split, buf, first, s);
    if (mode == BXD) return launch<G128, BXD>(d, prefix, nmats, split, buf, first, s);
    return hipErrorInvalidValue;
  }
  if (cfg == kCfgW160 && mode == BXM) return launch<W160, BXM>(d, prefix, nmats, split, buf, first, s);
  if (cfg == kCfgW160 && mode == BXL) return launch<W160, BXL>(d, prefix, nmats, split, buf, first, s);
  if (cfg == kCfgW160 && mode == BXD) return launch<W160, BXD>(d, prefix, nmats, split, buf, first, s);
  if (cfg == kCfgW320 && mode == BXM) return launch<W320, BXM>(d, prefix, nmats, split, buf, first, s);
  if (cfg == kCfgW320 && mode == BXL) return launch<W320, BXL>(d, prefix, nmats, split, buf, first, s);
  if (cfg == kCfgW320 && mode == BXD) return launch<W320, BXD>(d, prefix, nmats, split, buf, first, s);
  return hipErrorInvalidValue;
}

}  // namespace muon
