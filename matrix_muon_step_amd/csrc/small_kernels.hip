// Float32 Newton-Schulz path for matrices whose Gram side m <= kSmallGram.
//
// The quintic step of the Muon synthesis note (papers.chlience.com,
// section 4) is computed exactly as in the matrix-core path, A = X X^T,
// P = b A + c A A, X' = a X + P X, but every operand and result stays
// float32.  With few singular values the bf16 operand rounding of the
// matrix-core path does not average out, while the work here is at most
// 2 * 64^2 * n multiply-adds per iteration and per matrix.
//
// The iterate lives as a float32 kSmallGram x n_pad array (rows >= m are
// zero).  Three grouped launches per iteration:
//   small_gram: per 256-column chunk, the partial Gram of the chunk
//   small_poly: per matrix, fixed-order sum of the partials, then P
//   small_bx  : per 256-column chunk, X' = a X + P X
#include "muon_internal.h"

namespace muon {

namespace {

constexpr int SM = kSmallGram;     // 64
constexpr int SC = kSmallChunk;    // 256
constexpr int XS = SM + 4;         // LDS row stride of the transposed chunk


// Partial Gram of one 256-column chunk: G_c[i][j] = sum_k X[i][k] X[j][k].
// Thread t owns the 4x4 block (rows 4*(t/16).., cols 4*(t%16)..).
__global__ __launch_bounds__(256) void small_gram_kernel(const MatDesc* __restrict__ descs,
                                                         const int32_t* __restrict__ prefix,
                                                         int nmats, int buf) {
  const int blk = blockIdx.x;
  const int mi = find_mat(prefix, nmats, blk);
  const MatDesc d = descs[mi];
  const int chunk = blk - prefix[mi];
  const int n_pad = d.n_pad;
  const float* __restrict__ X = pick(d.xf, buf) + static_cast<int64_t>(chunk) * SC;
  __shared__ __attribute__((aligned(16))) float xs[SC][XS];  // [k][i]
  const int t = threadIdx.x;
  // Load X[0:64][chunk] transposed into xs.
  for (int i = 0; i < SM; ++i) xs[t][i] = gld<float>(X + static_cast<int64_t>(i) * n_pad + t);
  __syncthreads();
  const int ib = (t >> 4) * 4;
  const int jb = (t & 15) * 4;
  float acc[4][4] = {};
  for (int k = 0; k < SC; ++k) {
    const float4 xi = *reinterpret_cast<const float4*>(&xs[k][ib]);
    const float4 xj = *reinterpret_cast<const float4*>(&xs[k][jb]);
    const float a[4] = {xi.x, xi.y, xi.z, xi.w};
    const float b[4] = {xj.x, xj.y, xj.z, xj.w};
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(a[r], b[c], acc[r][c]);
  }
  float* __restrict__ out = d.sgram + static_cast<int64_t>(chunk) * SM * SM;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    gst(out + (ib + r) * SM + jb,
        make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]));
}

// A = sum of the chunk partials (fixed order), P = b A + c A A.
__global__ __launch_bounds__(256) void small_poly_kernel(const MatDesc* __restrict__ descs,
                                                         const int32_t* __restrict__ prefix,
                                                         int nmats) {
  const int mi = find_mat(prefix, nmats, blockIdx.x);
  const MatDesc d = descs[mi];
  __shared__ float A[SM][SM + 1];
  const int t = threadIdx.x;
  const int nc = d.s_chunks;
  for (int e = t; e < SM * SM; e += 256) {
    float s = 0.f;
    for (int c = 0; c < nc; ++c) s += gld<float>(d.sgram + static_cast<int64_t>(c) * SM * SM + e);
    A[e / SM][e % SM] = s;
  }
  __syncthreads();
  for (int e = t; e < SM * SM; e += 256) {
    const int i = e / SM, j = e % SM;
    float s = 0.f;
    for (int k = 0; k < SM; ++k) s = fmaf(A[i][k], A[k][j], s);
    gst(d.spoly + e, fmaf(kCoefC, s, kCoefB * A[i][j]));
  }
}

// X' = a X + P X on one 256-column chunk; thread t owns column t.
__global__ __launch_bounds__(256) void small_bx_kernel(const MatDesc* __restrict__ descs,
                                                       const int32_t* __restrict__ prefix,
                                                       int nmats, int buf) {
  const int blk = blockIdx.x;
  const int mi = find_mat(prefix, nmats, blk);
  const MatDesc d = descs[mi];
  const int chunk = blk - prefix[mi];
  const int n_pad = d.n_pad;
  __shared__ __attribute__((aligned(16))) float P[SM * SM];
  const int t = threadIdx.x;
  for (int e = t; e < SM * SM; e += 256) P[e] = gld<float>(d.spoly + e);
  __syncthreads();
  const int64_t col = static_cast<int64_t>(chunk) * SC + t;
  const float* __restrict__ X = pick(d.xf, buf) + col;
  float* __restrict__ Y = pick(d.xf, buf ^ 1) + col;
  float x[SM];
#pragma unroll
  for (int k = 0; k < SM; ++k) x[k] = gld<float>(X + static_cast<int64_t>(k) * n_pad);
#pragma unroll
  for (int i = 0; i < SM; ++i) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < SM; k += 4) {
      const float4 p = *reinterpret_cast<const float4*>(&P[i * SM + k]);
      s = fmaf(p.x, x[k], s);
      s = fmaf(p.y, x[k + 1], s);
      s = fmaf(p.z, x[k + 2], s);
      s = fmaf(p.w, x[k + 3], s);
    }
    gst(Y + static_cast<int64_t>(i) * n_pad, fmaf(kCoefA, x[i], s));
  }
}

}  // namespace

hipError_t launch_small_gram(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                             hipStream_t s) {
  hipLaunchKernelGGL(small_gram_kernel, dim3(total), dim3(256), 0, s, d, prefix, nmats, buf);
  return hipGetLastError();
}

hipError_t launch_small_poly(const MatDesc* d, const int32_t* prefix, int nmats, int total,
                             hipStream_t s) {
  hipLaunchKernelGGL(small_poly_kernel, dim3(total), dim3(256), 0, s, d, prefix, nmats);
  return hipGetLastError();
}

hipError_t launch_small_bx(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                           hipStream_t s) {
  hipLaunchKernelGGL(small_bx_kernel, dim3(total), dim3(256), 0, s, d, prefix, nmats, buf);
  return hipGetLastError();
}

}  // namespace muon
