// Internal definitions shared by the host planner and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// Device memory accesses through the global address space.  The kernels
// reach their buffers through generic pointers held in the descriptors;
// copying through an address_space(1) pointer makes the compiler emit
// global (not flat) loads and stores, which only the vector-memory counter
// tracks, so waits on them do not also drain pending LDS traffic.
template <class T>
__device__ __forceinline__ T gld(const void* p) {
  T v;
  __builtin_memcpy(&v, (const __attribute__((address_space(1))) void*)p, sizeof(T));
  return v;
}
template <class T>
__device__ __forceinline__ void gst(void* p, T v) {
  __builtin_memcpy((__attribute__((address_space(1))) void*)p, &v, sizeof(T));
}

// A 16-byte store that streams past the caches (nontemporal): for results
// the next kernel reads only after gigabytes of other traffic.  Through the
// global address space, as gst.
typedef uint32_t u32x4_nt_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void gst_stream(void* p, uint4 v) {
  __builtin_nontemporal_store((u32x4_nt_t){v.x, v.y, v.z, v.w},
                              (__attribute__((address_space(1))) u32x4_nt_t*)p);
}

// bf16 halves of a 32-bit word as float32 (low half = element 0).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Two float32 values rounded to bf16 (nearest, ties to even) in one word,
// a in the low half: a single packed conversion on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t h = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

// Coefficients of the quintic Newton-Schulz step X <- aX + b(XX^T)X +
// c(XX^T)^2 X, as the Muon synthesis note (papers.chlience.com, section 4)
// prints them; float32 constants on the GPU.
constexpr float kCoefA = 3.4445f;
constexpr float kCoefB = -4.7750f;
constexpr float kCoefC = 2.0315f;

// Matrix of a grouped launch that owns work item `blk`: the last i with
// prefix[i] <= blk (prefix = exclusive prefix sums of work per matrix; a
// matrix with no work has an empty range and is never returned).
__device__ __forceinline__ int find_mat(const int32_t* __restrict__ prefix, int nmats, int blk) {
  int lo = 0, hi = nmats - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= blk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Position of 16-byte k-chunk c (0..3) in a 64-byte LDS operand row r of
// the matrix-core kernels: chunks XOR-swizzled by ((r >> 1) ^ (r >> 2)),
// conflict-free for the 32x32x16 and 16x16x32 fragment reads on gfx950.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (((r >> 1) ^ (r >> 2)) & 3); }

// s_waitcnt with only vmcnt limited (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] in [15:14]).
#define MUON_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x0F70)

// Matrix-core kernel configurations (tile rows x tile columns, MFMA shape):
//   G256: 256 x 256, 32x32x16   (Gram, polynomial, BX)
//   W160: 160 x 256, 32x32x16   (BX only; Gram side a multiple of 160)
//   W320: 320 x 256, 32x32x16   (BX only; Gram side a multiple of 320)
//   T160: 160 x 160, 16x16x32   (Gram, polynomial, BX)
//   T128: 128 x 128, 16x16x32   (Gram, polynomial, BX)
// Every iterate / Gram buffer is zero padded to multiples of its matrix's
// tile edges, so the GEMM kernels never bounds-check.
//   G128: 128 x 128, 32x32x16   (Gram, polynomial, BX; the G256 arithmetic
//         on smaller tiles, for calls too small to fill the GPU with G256)
enum GemmCfg : int32_t {
  kCfgG256 = 0, kCfgW160 = 1, kCfgT160 = 2, kCfgT128 = 3, kCfgW320 = 4, kCfgG128 = 5, kNumCfg = 6
};
constexpr int kCfgRows[kNumCfg] = {256, 160, 160, 128, 320, 128};   // tile rows (Gram side)
constexpr int kCfgCols[kNumCfg] = {256, 256, 160, 128, 256, 128};   // tile columns (long side for BX)
constexpr int kCfgWaves[kNumCfg] = {8, 4, 4, 4, 8, 4};              // waves per work-group
// Configurations served by the 32x32x16 wide-tile kernels.
constexpr bool cfg_wide(int c) { return c == kCfgG256 || c == kCfgW160 || c == kCfgW320 || c == kCfgG128; }
// Tile edge of the layout kernels (normalise/transpose, update).
constexpr int kEwTile = 64;
// Momentum work-group tile: 64 rows x 128 columns of M in its own
// orientation, so each float32 row segment it reads and writes is 512
// contiguous bytes (64 x 64 tiles, 256-byte segments, ran 5% slower).  In
// X's orientation (short side i, long side j) that is mom_tile_i x
// mom_tile_j, which depends on whether M is stored transposed.
constexpr int kMomRows = 64, kMomCols = 128;
__host__ __device__ constexpr int mom_tile_i(bool tr) { return tr ? kMomCols : kMomRows; }
__host__ __device__ constexpr int mom_tile_j(bool tr) { return tr ? kMomRows : kMomCols; }
// Matrices whose Gram side m is at most this take the float32 path: with so
// few singular values the bf16 operand rounding does not average out, and
// the Gram work is small enough for plain float32 arithmetic.
constexpr int kSmallGram = 64;
// Columns per work-group of the float32 small-Gram kernels (n_pad multiple).
constexpr int kSmallChunk = 256;

enum GFlags : int32_t {
  kTransposed = 1,  // rows > cols: iterate on M^T
  kGBf16 = 2,       // gradient stored as bfloat16
  kNesterov = 4,    // orthogonalise G + mu * B
  kOrthoOnly = 8,   // muon_orthogonalize: read M, write O, no momentum/update
  kSmall = 16,      // m <= kSmallGram: float32 iterate and Gram path
  kFusedUpd = 32,   // the last BX launch applies the update (no update_kernel work)
  kDiag = 64,       // collect the per-matrix diagnostics of this call
  kFold = 128,      // the momentum pass writes the unnormalised pair; the
                    // first iteration applies 1 / (||M||_F + eps)
};

// Per-matrix scalars after the norm pass (MatDesc::sigma[]).
constexpr int kSigFirst = 1;  // scale the first iteration applies (sigma, or 1)
constexpr int kSigPrep = 2;   // int bits: 1 = the prep pass writes sigma * M

// Per-wave partial sums of the diagnostics, written by the kernel that
// writes W (fused last BX or update pass); reduced in a fixed order.
struct DiagPart {
  float o2;     // sum of O^2
  float d2;     // sum of (W_new - W_old)^2
  float w2;     // sum of W_new^2
  int32_t bad;  // 1 if some W_new is NaN or infinite
};

// A lane's running diagnostics over the W elements it writes: float32 sums
// of squares of O, of the applied step and of the new weights, and whether
// a new weight is NaN or infinite (exponent field all ones).
struct DiagAcc {
  float o2 = 0.f, d2 = 0.f, w2 = 0.f;
  uint32_t bad = 0;
};
__device__ __forceinline__ void diag_add(DiagAcc& a, float o, float w_old, float w_new) {
  a.o2 = fmaf(o, o, a.o2);
  const float dl = w_new - w_old;
  a.d2 = fmaf(dl, dl, a.d2);
  a.w2 = fmaf(w_new, w_new, a.w2);
  a.bad |= (__float_as_uint(w_new) & 0x7f800000u) == 0x7f800000u;
}
// Sums a wave's accumulators (fixed butterfly order) into one DiagPart.
__device__ __forceinline__ void diag_flush(const DiagAcc& a, DiagPart* dst, int lane) {
  float o2 = a.o2, d2 = a.d2, w2 = a.w2;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    o2 += __shfl_xor(o2, off, 64);
    d2 += __shfl_xor(d2, off, 64);
    w2 += __shfl_xor(w2, off, 64);
  }
  const int bad = __any(a.bad != 0) ? 1 : 0;
  if (lane == 0) gst(dst, DiagPart{o2, d2, w2, bad});
}

// One matrix of a call, as the kernels see it (lives in the workspace).
// Kernels take a copy (const MatDesc d = descs[i]): through a reference,
// every store into a buffer might alias the table, and the compiler would
// reload the fields (and wait on the scalar loads) after each store.  The
// ping-pong pairs are read through pick(): a run-time array index would
// put the copy in scratch memory.
struct MatDesc {
  float* W;          // update target (or O output in orthogonalise-only mode)
  const void* G;     // gradient (or M input in orthogonalise-only mode)
  float* B;          // momentum buffer (unused in orthogonalise-only mode)
  __bf16* xt_hi[2];  // X^T high part, n_pad x m_pad, ping-pong
  __bf16* xt_lo[2];  // X^T rounding residual, n_pad x m_pad, ping-pong
  __bf16* gram;      // A, m_pad x m_pad (both triangles)
  __bf16* poly;      // P, m_pad x m_pad (both triangles)
  float* xf[2];      // float32 iterate (small path), kSmallGram x n_pad
  float* sgram;      // small path: per-chunk partial Gram matrices
  float* spoly;      // small path: P, kSmallGram x kSmallGram float32
  float* partials;   // per-tile sums of squares of M
  float* sigma;      // [0] 1 / (||M||_F + eps), [kSigFirst], [kSigPrep]
  int32_t* mom_bad;  // diagnostics: per momentum block, 1 if M holds a non-finite value
  float* mstat;      // diagnostics: [0] = ||M||_F, [1] = non-finite flag of M (int bits)
  DiagPart* diag_part;  // diagnostics: per-wave partials of the W-writing kernel
  int64_t rows, cols;
  int32_t m, n, m_pad, n_pad;
  int32_t flags;
  int32_t mom_blocks;  // work-groups (64 x 128 tiles of M, covering padded X) of the momentum kernel
  float lr_scale;      // lr * scale, formed in float32 on the host
  float lr_wd;         // lr * weight_decay (float32), 0 in orthogonalise-only mode
  int32_t s_chunks;    // small path: column chunks (n_pad / kSmallChunk)
  int32_t sym_cfg;     // kernel configuration of the Gram / polynomial stages
  int32_t bx_cfg;      // kernel configuration of the BX stage
  int32_t k_gram;      // reduction length of the Gram product: n rounded up to 32
  int32_t bx_group;    // BX tile order: Gram-side tile rows per group (see gemm32)
  int32_t diag_slots;  // entries of diag_part (work-groups x waves of the W writer)
};

// Buffer b (0 or 1) of a ping-pong pair, without a run-time array index.
template <class T>
__device__ __forceinline__ T* pick(T* const (&a)[2], int b) {
  return b ? a[1] : a[0];
}

// Split of one grouped GEMM launch over the 8 XCDs: work-groups are dealt
// to XCDs round-robin (block id % 8), and XCD x runs the contiguous work
// range [begin[x], end[x]), chosen on the host so every XCD gets the same
// estimated cost (tiles differ in reduction length).  Blocks beyond their
// XCD's range exit at once; the grid is 8 * max range length.
struct XcdSplit {
  int32_t begin[8];
  int32_t end[8];
  int32_t max_len;
};

// Host-side launchers (defined in the kernel translation units).  `prefix`
// is the exclusive prefix sum of work-groups per matrix for that launch
// (entry [nmats] = total); a matrix with no work in a launch has an empty
// range, which the device-side search skips.
hipError_t launch_momentum(const MatDesc* d, const int32_t* prefix, int nmats, int total,
                           float mu, hipStream_t s);
// prep_count: one int the norm pass increments per matrix it marks for the
// prep pass (zero at the start of the call).
// Sets one int of device memory to zero (a kernel, not a memset, so that it
// can sit in a recorded graph).
hipError_t launch_zero_counter(int32_t* p, hipStream_t s);
// Descriptor tables of at most kTableArgBytes (calls of a few matrices) are
// written into the workspace by one kernel that takes the table as its
// argument: a launch of a few microseconds instead of a host-to-device copy
// (about 11 us for a table of 512 bytes).  bytes must be a multiple of 4.
constexpr int kTableArgBytes = 3072;
hipError_t launch_table_write(void* dst, const void* src, size_t bytes, hipStream_t s);
hipError_t launch_norm(const MatDesc* d, int nmats, float eps, int32_t* prep_count, hipStream_t s);
hipError_t launch_prep(const MatDesc* d, const int32_t* prefix, int nmats, int total, float mu,
                       const int32_t* prep_count, hipStream_t s);
hipError_t launch_update(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                         bool diag, hipStream_t s);
// Final reduction of the diagnostics: one work-group per matrix writes out[i]
// (a muon_diag_t array).
hipError_t launch_diag(const MatDesc* d, int nmats, void* out, hipStream_t s);
// Matrix-core GEMM stage (mode 0 = Gram, 1 = polynomial, 2 = BX; wide tiles
// also 3 = last BX with the update, 4 = the same with diagnostics) for the
// matrices whose configuration for that stage is `cfg` (16x16 kernels:
// T160, T128; 32x32 kernels: G256, W160).
// `first`: the first iteration, whose Gram product is scaled by
// sigma[kSigFirst]^2 and whose BX result by sigma[kSigFirst].
hipError_t launch_ns_gemm(int mode, int cfg, const MatDesc* d, const int32_t* prefix, int nmats,
                          const XcdSplit& split, int buf, int first, hipStream_t s);
hipError_t launch_ns_gemm32(int mode, int cfg, const MatDesc* d, const int32_t* prefix, int nmats,
                            const XcdSplit& split, int buf, int first, hipStream_t s);
// QK-Clip: one batch of matrices per launch, passed by value (kernel
// arguments), so the call needs no workspace.  Matrix i's heads are
// work-groups prefix[i] .. prefix[i+1]-1; head h of matrix i is the
// contiguous range W + h * head_elems of head_elems floats.
constexpr int kClipBatch = 48;
struct ClipDesc {
  float* W;
  const float* max_logit;   // one entry per head
  int64_t head_elems;       // head_dim * cols
  int32_t vec;              // head_elems % 4 == 0 (16-byte accesses)
  int32_t pad;
};
struct ClipBatch {
  ClipDesc d[kClipBatch];
  int32_t prefix[kClipBatch + 1];
  int32_t n;
  float tau;
};
hipError_t launch_qk_clip(const ClipBatch& b, hipStream_t s);
// Streaming copy of n16 16-byte words (bandwidth yardstick); variant as
// muon_copy_probe documents.
hipError_t launch_copy_probe(const void* src, void* dst, int64_t n16, int variant, hipStream_t s);
hipError_t launch_small_gram(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                             hipStream_t s);
hipError_t launch_small_poly(const MatDesc* d, const int32_t* prefix, int nmats, int total,
                             hipStream_t s);
hipError_t launch_small_bx(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                           hipStream_t s);

}  // namespace muon
