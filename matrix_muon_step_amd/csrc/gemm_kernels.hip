// Matrix-core stages of the Newton-Schulz iteration on gfx950.
//
// The quintic step of the Muon synthesis note (papers.chlience.com,
// section 4), X <- aX + b(XX^T)X + c(XX^T)^2 X with (a,b,c) =
// (3.4445, -4.7750, 2.0315), is computed as three grouped GEMM launches:
//
//   GRAM : A = X_hi X_hi^T          symmetric: upper 128x128 tiles, mirrored
//   POLY : P = b A + c A A          symmetric (A A = A A^T): upper tiles,
//                                   axpy epilogue, mirrored
//   BX   : X' = a (X_hi + X_lo) + P X_hi   epilogue re-splits X' into the
//                                   bf16 pair (ping-pong buffers)
//
// All operands are bf16 and go through v_mfma_f32_32x32x16_bf16 with float32
// accumulation.  One work-group (4 waves, 256 threads) owns a 128x128 output
// tile; each wave owns a 64x64 quarter as 2x2 MFMA blocks.  K advances 64 at
// a time through double-buffered LDS with the next slab prefetched into
// registers while the current one is multiplied.  Every buffer is zero padded
// to multiples of 128 in both dimensions, so no load or store is masked.
//
// Both operands reach LDS as [row][k] with 8 consecutive k per 16 bytes,
// which is what an MFMA lane consumes.  GRAM and POLY read K-contiguous rows
// directly; BX's right operand (X, K x N with N contiguous) is transposed in
// registers (8 k-rows x 4 columns per thread) on its way into LDS.
#include "muon_internal.h"

namespace muon {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kCoefA = 3.4445f;
constexpr float kCoefB = -4.7750f;
constexpr float kCoefC = 2.0315f;

constexpr int BM = kTile;   // 128
constexpr int BK = 64;
constexpr int LDK = BK + 8; // LDS row stride in bf16 elements (144 bytes)
constexpr int kThreads = 256;

enum Mode { GRAM = 0, POLY = 1, BXM = 2 };

__device__ __forceinline__ int find_mat(const int32_t* __restrict__ prefix, int nmats, int blk) {
  int lo = 0, hi = nmats - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= blk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float bf2f(__bf16 h) { return static_cast<float>(h); }

template <int MODE>
__global__ __launch_bounds__(kThreads) void ns_gemm_kernel(const MatDesc* __restrict__ descs,
                                                           const int32_t* __restrict__ prefix,
                                                           int nmats, int buf) {
  __shared__ __attribute__((aligned(16))) __bf16 smem[2][2][BM * LDK];

  const int blk = blockIdx.x;
  const int mi = find_mat(prefix, nmats, blk);
  const MatDesc& d = descs[mi];
  int local = blk - prefix[mi];
  const int m_pad = d.m_pad;
  const int n_pad = d.n_pad;

  int ti, tj;
  if (MODE == BXM) {
    const int tpr = n_pad / BM;
    ti = local / tpr;
    tj = local - ti * tpr;
  } else {
    const int T = m_pad / BM;
    ti = 0;
    while (local >= T - ti) {
      local -= T - ti;
      ++ti;
    }
    tj = ti + local;
  }

  const __bf16* __restrict__ Aop;
  const __bf16* __restrict__ Bop;
  int lda, ldb, K;
  if (MODE == GRAM) {
    Aop = d.xhi[buf] + static_cast<int64_t>(ti) * BM * n_pad;
    Bop = d.xhi[buf] + static_cast<int64_t>(tj) * BM * n_pad;
    lda = ldb = K = n_pad;
  } else if (MODE == POLY) {
    Aop = d.gram + static_cast<int64_t>(ti) * BM * m_pad;
    Bop = d.gram + static_cast<int64_t>(tj) * BM * m_pad;
    lda = ldb = K = m_pad;
  } else {
    Aop = d.poly + static_cast<int64_t>(ti) * BM * m_pad;
    Bop = d.xhi[buf] + static_cast<int64_t>(tj) * BM;  // column offset; rows are k
    lda = K = m_pad;
    ldb = n_pad;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1;
  const int wc = wave & 1;

  // ---- global -> register prefetch
  uint4 ra[4];
  uint4 rb[4];   // NT right operand
  uint2 rn[8];   // NN right operand (BX)

  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + kThreads * r;
      const int row = c >> 3;
      const int kc = c & 7;
      ra[r] = *reinterpret_cast<const uint4*>(Aop + static_cast<int64_t>(row) * lda + k0 + kc * 8);
    }
    if (MODE == BXM) {
      const int jb = tid & 31;
      const int kb = tid >> 5;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int64_t k = k0 + kb * 8 + r;
        rn[r] = *reinterpret_cast<const uint2*>(Bop + k * ldb + jb * 4);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = tid + kThreads * r;
        const int row = c >> 3;
        const int kc = c & 7;
        rb[r] = *reinterpret_cast<const uint4*>(Bop + static_cast<int64_t>(row) * ldb + k0 + kc * 8);
      }
    }
  };

  auto store_tiles = [&](int sb) {
    __bf16* As = smem[sb][0];
    __bf16* Bs = smem[sb][1];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + kThreads * r;
      const int row = c >> 3;
      const int kc = c & 7;
      *reinterpret_cast<uint4*>(As + row * LDK + kc * 8) = ra[r];
    }
    if (MODE == BXM) {
      const int jb = tid & 31;
      const int kb = tid >> 5;
      // rn[r] holds row k = kb*8 + r, columns jb*4 .. jb*4+3 (two per dword).
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t lo = (x < 2) ? rn[2 * p].x : rn[2 * p].y;
          const uint32_t hi = (x < 2) ? rn[2 * p + 1].x : rn[2 * p + 1].y;
          w[p] = (x & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        *reinterpret_cast<uint4*>(Bs + (jb * 4 + x) * LDK + kb * 8) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = tid + kThreads * r;
        const int row = c >> 3;
        const int kc = c & 7;
        *reinterpret_cast<uint4*>(Bs + row * LDK + kc * 8) = rb[r];
      }
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = K / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();

  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int sb = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * BK);
    const __bf16* As = smem[sb][0];
    const __bf16* Bs = smem[sb][1];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ko = ks * 16 + fk;
      bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(As + (wr * 64 + frow) * LDK + ko);
      bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(As + (wr * 64 + 32 + frow) * LDK + ko);
      bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(Bs + (wc * 64 + frow) * LDK + ko);
      bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(Bs + (wc * 64 + 32 + frow) * LDK + ko);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tiles(sb ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  32x32 accumulator layout: lane holds column (lane & 31),
  // register v holds row 8*(v/4) + 4*(lane/32) + (v%4).
  const int half = lane >> 5;
  const int col = lane & 31;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int il = wr * 64 + bi * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
        const int jl = wc * 64 + bj * 32 + col;
        const float val = acc[bi][bj][v];
        const int gi = ti * BM + il;
        const int gj = tj * BM + jl;
        if (MODE == BXM) {
          const int64_t idx = static_cast<int64_t>(gi) * n_pad + gj;
          const float x = bf2f(d.xhi[buf][idx]) + bf2f(d.xlo[buf][idx]);
          const float o = fmaf(kCoefA, x, val);
          const __bf16 h = static_cast<__bf16>(o);
          const __bf16 l = static_cast<__bf16>(o - bf2f(h));
          d.xhi[buf ^ 1][idx] = h;
          d.xlo[buf ^ 1][idx] = l;
        } else {
          // Diagonal tiles write each symmetric pair once, from (i <= j).
          if (ti == tj && gi > gj) continue;
          float out = val;
          __bf16* dst;
          if (MODE == POLY) {
            out = fmaf(kCoefC, val, kCoefB * bf2f(d.gram[static_cast<int64_t>(gi) * m_pad + gj]));
            dst = d.poly;
          } else {
            dst = d.gram;
          }
          const __bf16 h = static_cast<__bf16>(out);
          dst[static_cast<int64_t>(gi) * m_pad + gj] = h;
          dst[static_cast<int64_t>(gj) * m_pad + gi] = h;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gram(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                       hipStream_t s) {
  hipLaunchKernelGGL(ns_gemm_kernel<GRAM>, dim3(total), dim3(kThreads), 0, s, d, prefix, nmats, buf);
  return hipGetLastError();
}

hipError_t launch_poly(const MatDesc* d, const int32_t* prefix, int nmats, int total,
                       hipStream_t s) {
  hipLaunchKernelGGL(ns_gemm_kernel<POLY>, dim3(total), dim3(kThreads), 0, s, d, prefix, nmats, 0);
  return hipGetLastError();
}

hipError_t launch_bx(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                     hipStream_t s) {
  hipLaunchKernelGGL(ns_gemm_kernel<BXM>, dim3(total), dim3(kThreads), 0, s, d, prefix, nmats, buf);
  return hipGetLastError();
}

}  // namespace muon
