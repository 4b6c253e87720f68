// Internal definitions shared by the host planner and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// Output tile edge of the matrix-core kernels; every iterate / Gram buffer is
// zero padded to a multiple of it, so the GEMM kernels never bounds-check.
constexpr int kTile = 128;
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
};

// One matrix of a call, as the kernels see it (lives in the workspace).
struct MatDesc {
  float* W;          // update target (or O output in orthogonalise-only mode)
  const void* G;     // gradient (or M input in orthogonalise-only mode)
  float* B;          // momentum buffer (unused in orthogonalise-only mode)
  __bf16* xhi[2];    // iterate high parts, m_pad x n_pad, ping-pong
  __bf16* xlo[2];    // iterate residual parts
  __bf16* gram;      // A, m_pad x m_pad
  __bf16* poly;      // P, m_pad x m_pad
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
  int32_t s_chunks;    // small path: column chunks (n_pad / kSmallChunk)
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
hipError_t launch_gram(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                       hipStream_t s);
hipError_t launch_poly(const MatDesc* d, const int32_t* prefix, int nmats, int total,
                       hipStream_t s);
hipError_t launch_bx(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                     hipStream_t s);
hipError_t launch_small_gram(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                             hipStream_t s);
hipError_t launch_small_poly(const MatDesc* d, const int32_t* prefix, int nmats, int total,
                             hipStream_t s);
hipError_t launch_small_bx(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                           hipStream_t s);

}  // namespace muon
