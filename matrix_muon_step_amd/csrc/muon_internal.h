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

// Matrix-core kernel configurations (tile rows x tile columns, MFMA shape):
//   G256: 256 x 256, 32x32x16   (Gram, polynomial, BX)
//   W160: 160 x 256, 32x32x16   (BX only; Gram side a multiple of 160)
//   W320: 320 x 256, 32x32x16   (BX only; Gram side a multiple of 320)
//   T160: 160 x 160, 16x16x32   (Gram, polynomial, BX)
//   T128: 128 x 128, 16x16x32   (Gram, polynomial, BX)
// Every iterate / Gram buffer is zero padded to multiples of its matrix's
// tile edges, so the GEMM kernels never bounds-check.
enum GemmCfg : int32_t { kCfgG256 = 0, kCfgW160 = 1, kCfgT160 = 2, kCfgT128 = 3, kCfgW320 = 4, kNumCfg = 5 };
constexpr int kCfgRows[kNumCfg] = {256, 160, 160, 128, 320};   // tile rows (Gram side)
constexpr int kCfgCols[kNumCfg] = {256, 256, 160, 128, 256};   // tile columns (long side for BX)
// Configurations served by the 32x32x16 wide-tile kernels.
constexpr bool cfg_wide(int c) { return c == kCfgG256 || c == kCfgW160 || c == kCfgW320; }
// Tile edge of the layout kernels (normalise/transpose, update).
constexpr int kEwTile = 64;
// Elements per work-group of the momentum/norm kernel.
constexpr int kMomChunk = 4096;
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
};

// One matrix of a call, as the kernels see it (lives in the workspace).
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
  float* partials;   // per-block sums of squares of M
  float* sigma;      // 1 / (||M||_F + eps)
  int64_t rows, cols;
  int32_t m, n, m_pad, n_pad;
  int32_t flags;
  int32_t mom_blocks;  // work-groups of the momentum kernel for this matrix
  float lr_scale;      // lr * scale, formed in float32 on the host
  float lr_wd;         // lr * weight_decay (float32), 0 in orthogonalise-only mode
  int32_t s_chunks;    // small path: column chunks (n_pad / kSmallChunk)
  int32_t sym_cfg;     // kernel configuration of the Gram / polynomial stages
  int32_t bx_cfg;      // kernel configuration of the BX stage
  int32_t k_gram;      // reduction length of the Gram product: n rounded up to 32
  int32_t bx_group;    // BX tile order: Gram-side tile rows per group (see gemm32)
};

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
hipError_t launch_norm(const MatDesc* d, int nmats, float eps, hipStream_t s);
hipError_t launch_prep(const MatDesc* d, const int32_t* prefix, int nmats, int total, float mu,
                       hipStream_t s);
hipError_t launch_update(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                         hipStream_t s);
// Matrix-core GEMM stage (mode 0 = Gram, 1 = polynomial, 2 = BX) for the
// matrices whose configuration for that stage is `cfg` (16x16 kernels:
// T160, T128; 32x32 kernels: G256, W160).
hipError_t launch_ns_gemm(int mode, int cfg, const MatDesc* d, const int32_t* prefix, int nmats,
                          const XcdSplit& split, int buf, hipStream_t s);
hipError_t launch_ns_gemm32(int mode, int cfg, const MatDesc* d, const int32_t* prefix, int nmats,
                            const XcdSplit& split, int buf, hipStream_t s);
hipError_t launch_small_gram(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                             hipStream_t s);
hipError_t launch_small_poly(const MatDesc* d, const int32_t* prefix, int nmats, int total,
                             hipStream_t s);
hipError_t launch_small_bx(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                           hipStream_t s);

}  // namespace muon
