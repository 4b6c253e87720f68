// Bandwidth-bound stages of the Muon step on gfx950:
//   momentum + Frobenius partial sums, per-matrix norm, normalise/transpose/
//   split into the bf16 iterate pair, and the final parameter update.
// The method's steps are those of the Muon synthesis note (papers.chlience.com),
// section 4: momentum accumulation, Frobenius normalisation, transpose to the
// smaller Gram side, and W <- W - lr * O; the optional per-matrix diagnostics
// follow the note's practice checklist (update RMS, weight RMS, norms).
#include "muon.h"
#include "muon_internal.h"

namespace muon {

namespace {


__device__ __forceinline__ float bf16_bits_to_float(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// X^T pair of one 64x64 tile of X held in LDS (tile[r][c] = the tile's
// element of M at row r, column c of M's own orientation), each value
// multiplied by `scale`; padding is written as zeros.  A row of X^T (one
// long-side index) holds the tile's 64 short-side values: 128 bytes of each
// array.
__device__ __forceinline__ void write_pair_tile(const MatDesc& d, const float (&tile)[kEwTile][kEwTile + 1], int i0,
                                                int j0, float scale, bool tr) {
  const int tx = threadIdx.x & 15;
  const int ty = threadIdx.x >> 4;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int jl = ty + 16 * k;
    if (j0 + jl >= d.n_pad || i0 + tx * 4 >= d.m_pad) continue;
    float x[4];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int il = tx * 4 + c4;
      x[c4] = scale * (tr ? tile[jl][il] : tile[il][jl]);
    }
    const uint32_t h0 = pack_bf16(x[0], x[1]), h1 = pack_bf16(x[2], x[3]);
    const uint2 hv = make_uint2(h0, h1);
    const uint2 lv = make_uint2(pack_bf16(x[0] - bf_lo(h0), x[1] - bf_hi(h0)),
                                pack_bf16(x[2] - bf_lo(h1), x[3] - bf_hi(h1)));
    const int64_t off = static_cast<int64_t>(j0 + jl) * d.m_pad + i0 + tx * 4;
    gst(d.xt_hi[0] + off, hv);
    gst(d.xt_lo[0] + off, lv);
  }
}

// ---------------------------------------------------------------- momentum
// X^T pair of the unnormalised M from one momentum tile held in LDS
// (tile[r][c] = M at row r0 + r, column c0 + c of its own orientation;
// kMomRows x kMomCols).  A row of X^T (long-side index j) takes the tile's
// mom_tile_i values of the short side: 128 bytes of each array when M is
// not transposed (rows j are M's columns), 256 bytes when it is.  Padding
// (i < m_pad, j < n_pad past M's extent) is written as zeros.
__device__ __forceinline__ void write_pair_mtile(const MatDesc& d, const float (&tile)[kMomRows][kMomCols + 1],
                                                 int i0, int j0, bool tr) {
  // Lanes of a wave: 16 (not transposed) or 32 (transposed) groups of four
  // consecutive i, the rest of the wave on consecutive j; LDS reads of a wave
  // fall on distinct banks (not transposed) or two-way (transposed).
  const int lg = tr ? 5 : 4;
  const int tx = threadIdx.x & ((1 << lg) - 1);
  const int ty = threadIdx.x >> lg;
  const int jstep = 256 >> lg;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int jl = ty + jstep * k;
    if (j0 + jl >= d.n_pad || i0 + tx * 4 >= d.m_pad) continue;
    float x[4];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) x[c4] = tr ? tile[jl][tx * 4 + c4] : tile[tx * 4 + c4][jl];
    const uint32_t h0 = pack_bf16(x[0], x[1]), h1 = pack_bf16(x[2], x[3]);
    const uint2 hv = make_uint2(h0, h1);
    const uint2 lv = make_uint2(pack_bf16(x[0] - bf_lo(h0), x[1] - bf_hi(h0)),
                                pack_bf16(x[2] - bf_lo(h1), x[3] - bf_hi(h1)));
    const int64_t off = static_cast<int64_t>(j0 + jl) * d.m_pad + i0 + tx * 4;
    gst(d.xt_hi[0] + off, hv);
    gst(d.xt_lo[0] + off, lv);
  }
}

// One tile of kMomRows x kMomCols elements of M (its own orientation;
// mom_tile_i x mom_tile_j of the padded short-side-major X) per work-group:
// B <- mu * B + G and M = B (or G + mu * B) for the tile's elements of M,
// their sum of squares (partials[tile]) and, with diagnostics, whether one
// is NaN or infinite (mom_bad[tile]).  For a matrix whose normalisation is
// folded into the first iteration (kFold), the tile also writes the bf16
// pair of the unnormalised M as X^T.  Orthogonalise-only mode: M is read
// from G and nothing else is written.
__global__ __launch_bounds__(256) void momentum_kernel(const MatDesc* __restrict__ descs,
                                                       const int32_t* __restrict__ prefix, int nmats, float mu) {
  const int blk = blockIdx.x;
  const int mi = find_mat(prefix, nmats, blk);
  const MatDesc d = descs[mi];
  const int local = blk - prefix[mi];
  const int flags = d.flags;
  const bool tr = flags & kTransposed;
  const int tpr = (d.n_pad + mom_tile_j(tr) - 1) / mom_tile_j(tr);
  const int i0 = (local / tpr) * mom_tile_i(tr);  // X rows (short side)
  const int j0 = (local % tpr) * mom_tile_j(tr);  // X cols (long side)
  const bool ortho = flags & kOrthoOnly;
  const bool gbf = flags & kGBf16;
  const bool nest = flags & kNesterov;
  const bool fold = flags & kFold;
  const int64_t rows = d.rows, cols = d.cols;
  const int64_t r0 = tr ? j0 : i0;  // region of M (its own orientation)
  const int64_t c0 = tr ? i0 : j0;
  const bool vec = (cols & 3) == 0;  // rows of M start 16-byte aligned
  __shared__ float tile[kMomRows][kMomCols + 1];
  const int tx = threadIdx.x & 31;   // column group of 4 (32 per 512-byte row segment)
  const int ty = threadIdx.x >> 5;   // 0..7
  float acc = 0.f;
  uint32_t bad = 0;
#pragma unroll
  for (int k = 0; k < kMomRows / 8; ++k) {
    const int rl = ty + 8 * k;
    const int64_t r = r0 + rl;
    const int64_t c = c0 + tx * 4;
    float mv[4] = {0.f, 0.f, 0.f, 0.f};
    if (r < rows && c < cols) {
      const int64_t e = r * cols + c;
      const int cnt = (cols - c >= 4) ? 4 : static_cast<int>(cols - c);
      float g[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
      if (vec && cnt == 4) {
        if (gbf) {
          const uint2 gv = gld<uint2>(static_cast<const uint16_t*>(d.G) + e);
          g[0] = bf_lo(gv.x); g[1] = bf_hi(gv.x); g[2] = bf_lo(gv.y); g[3] = bf_hi(gv.y);
        } else {
          const float4 gv = gld<float4>(static_cast<const float*>(d.G) + e);
          g[0] = gv.x; g[1] = gv.y; g[2] = gv.z; g[3] = gv.w;
        }
        if (!ortho) {
          const float4 bv = gld<float4>(d.B + e);
          b[0] = bv.x; b[1] = bv.y; b[2] = bv.z; b[3] = bv.w;
        }
      } else {
        for (int q = 0; q < cnt; ++q) {
          g[q] = gbf ? bf16_bits_to_float(gld<uint16_t>(static_cast<const uint16_t*>(d.G) + e + q))
                     : gld<float>(static_cast<const float*>(d.G) + e + q);
          if (!ortho) b[q] = gld<float>(d.B + e + q);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (ortho) {
          mv[q] = g[q];
        } else {
          b[q] = fmaf(mu, b[q], g[q]);
          mv[q] = nest ? fmaf(mu, b[q], g[q]) : b[q];
        }
      }
      if (!ortho) {
        if (vec && cnt == 4) {
          gst(d.B + e, make_float4(b[0], b[1], b[2], b[3]));
        } else {
          for (int q = 0; q < cnt; ++q) gst(d.B + e + q, b[q]);
        }
      }
      // Elements past the last column stay zero (the loads above left g, b
      // zero there).
      for (int q = cnt; q < 4; ++q) mv[q] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc = fmaf(mv[q], mv[q], acc);
      bad |= (__float_as_uint(mv[q]) & 0x7f800000u) == 0x7f800000u;
      tile[rl][tx * 4 + q] = mv[q];
    }
  }
  __shared__ float red[4];
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  if (flags & kDiag) {
    // Block-uniform branch: the flag comes from the matrix descriptor.
    const int any_bad = __syncthreads_or(bad != 0);
    if (threadIdx.x == 0) gst(d.mom_bad + local, any_bad ? 1 : 0);
  } else {
    __syncthreads();
  }
  if (threadIdx.x == 0) gst(d.partials + local, ((red[0] + red[1]) + red[2]) + red[3]);
  if (fold) write_pair_mtile(d, tile, i0, j0, tr);
}

// ---------------------------------------------------------------- norm
// One work-group per matrix: fixed-order float64 sum of the tile partials,
// then sigma = 1 / (sqrt(sum) + eps).  A folded matrix (kFold) keeps its
// unnormalised pair when ||M||_F lies in [2^-50, 2^50] and the first
// iteration multiplies by sigma (first_scale = sigma); outside that range
// (where the unnormalised Gram product could lose range in float32) or for
// a matrix that is not folded, the prep pass writes sigma * M instead
// (prep = 1, first_scale = 1).  With diagnostics it also keeps ||M||_F and
// the OR of the tiles' non-finite flags in mstat.
__global__ __launch_bounds__(256) void norm_kernel(const MatDesc* __restrict__ descs, float eps,
                                                   int32_t* __restrict__ prep_count) {
  const MatDesc d = descs[blockIdx.x];
  const int nb = d.mom_blocks;
  double s = 0.0;
  for (int i = threadIdx.x; i < nb; i += 256) s += static_cast<double>(gld<float>(d.partials + i));
  __shared__ double red[256];
  red[threadIdx.x] = s;
  __syncthreads();
#pragma unroll
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const bool diag = d.flags & kDiag;
  int any_bad = 0;
  if (diag) {
    int b = 0;
    for (int i = threadIdx.x; i < nb; i += 256) b |= gld<int32_t>(d.mom_bad + i);
    any_bad = __syncthreads_or(b != 0);
  }
  if (threadIdx.x == 0) {
    const double nrm = sqrt(red[0]);
    const float sigma = static_cast<float>(1.0 / (nrm + static_cast<double>(eps)));
    const bool keep = (d.flags & kFold) && nrm >= 0x1p-50 && nrm <= 0x1p50;
    gst(d.sigma, sigma);
    gst(d.sigma + kSigFirst, keep ? sigma : 1.f);
    gst(d.sigma + kSigPrep, __int_as_float(keep ? 0 : 1));
    if (!keep) atomicAdd(prep_count, 1);  // the call's count of marked matrices (zeroed by the upload)
    if (diag) {
      gst(d.mstat, static_cast<float>(nrm));
      gst(d.mstat + 1, __int_as_float(any_bad ? 1 : 0));
    }
  }
}

// ---------------------------------------------------------------- prep
// X = sigma * M in the short-side-major padded layout (transposed when
// rows > cols), split into bf16 high part and bf16 residual (or float32 for
// the small-Gram path); padding is written as zeros.  Only for the matrices
// the norm pass marked (prep = 1): when none is marked (the count the norm
// pass kept is zero) every work-group returns at once; otherwise the
// work-groups stride over the 64x64 tiles of all matrices and skip the
// tiles of unmarked ones.
__global__ __launch_bounds__(256) void prep_kernel(const MatDesc* __restrict__ descs,
                                                   const int32_t* __restrict__ prefix, int nmats, float mu,
                                                   const int32_t* __restrict__ prep_count) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  const int tx = threadIdx.x & 15;   // column group of 4
  const int ty = threadIdx.x >> 4;   // 0..15
  if (gld<int32_t>(prep_count) == 0) return;
  const int total = prefix[nmats];
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int mi = find_mat(prefix, nmats, t);
    if (__float_as_int(gld<float>(descs[mi].sigma + kSigPrep)) == 0) continue;
    const MatDesc d = descs[mi];
    const int local = t - prefix[mi];
    const int tpr = (d.n_pad + kEwTile - 1) / kEwTile;
    const int flags = d.flags;
    const bool tr = flags & kTransposed;
    const bool ortho = flags & kOrthoOnly;
    const bool gbf = flags & kGBf16;
    const bool nest = flags & kNesterov;
    const int64_t rows = d.rows, cols = d.cols;
    const float sigma = gld<float>(d.sigma);
    {
      const int i0 = (local / tpr) * kEwTile;
      const int j0 = (local % tpr) * kEwTile;
      const int64_t r0 = tr ? j0 : i0;
      const int64_t c0 = tr ? i0 : j0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rl = ty + 16 * k;
        const int64_t r = r0 + rl;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (r < rows) {
          for (int c4 = 0; c4 < 4; ++c4) {
            const int64_t c = c0 + tx * 4 + c4;
            if (c < cols) {
              const int64_t e = r * cols + c;
              float mval;
              if (ortho) {
                mval = gld<float>(static_cast<const float*>(d.G) + e);
              } else {
                const float bval = gld<float>(d.B + e);
                if (nest) {
                  const float g = gbf ? bf16_bits_to_float(gld<uint16_t>(static_cast<const uint16_t*>(d.G) + e))
                                      : gld<float>(static_cast<const float*>(d.G) + e);
                  mval = fmaf(mu, bval, g);
                } else {
                  mval = bval;
                }
              }
              v[c4] = mval;
            }
          }
        }
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) tile[rl][tx * 4 + c4] = v[c4];
      }
      __syncthreads();
      if (flags & kSmall) {
        // Float32 iterate for the small-Gram path.
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int il = ty + 16 * k;
          if (i0 + il >= d.m_pad || j0 + tx * 4 >= d.n_pad) continue;
          float v[4];
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const int jl = tx * 4 + c4;
            v[c4] = sigma * (tr ? tile[jl][il] : tile[il][jl]);
          }
          const int64_t off = static_cast<int64_t>(i0 + il) * d.n_pad + j0 + tx * 4;
          gst(d.xf[0] + off, make_float4(v[0], v[1], v[2], v[3]));
        }
      } else {
        write_pair_tile(d, tile, i0, j0, sigma, tr);
      }
      __syncthreads();  // the tile is rewritten by the next iteration
    }
  }
}

// ---------------------------------------------------------------- update
// W <- W - (lr * scale) * O with O = X_hi + X_lo mapped back to rows x cols
// (transposed when rows > cols).  Orthogonalise-only mode stores O instead.
// DG: each wave also sums the diagnostics of the W it writes into
// diag_part[block * 4 + wave].
template <bool DG>
__global__ __launch_bounds__(256) void update_kernel(const MatDesc* __restrict__ descs,
                                                     const int32_t* __restrict__ prefix, int nmats,
                                                     int buf) {
  const int blk = blockIdx.x;
  const int mi = find_mat(prefix, nmats, blk);
  const MatDesc d = descs[mi];
  const int local = blk - prefix[mi];
  const int64_t rows = d.rows, cols = d.cols;
  const int tpr = static_cast<int>((cols + kEwTile - 1) / kEwTile);
  const int64_t r0 = static_cast<int64_t>(local / tpr) * kEwTile;
  const int64_t c0 = static_cast<int64_t>(local % tpr) * kEwTile;
  const bool tr = d.flags & kTransposed;
  const bool ortho = d.flags & kOrthoOnly;
  const bool small = d.flags & kSmall;
  // Source orientation: the big path keeps X^T (n_pad x m_pad), the small
  // path X (kSmallGram x n_pad).  O[r][c] is source[r][c] ("direct") when
  // the source already has W's orientation, else source[c][r].
  const bool direct = small ? !tr : tr;
  const int64_t s0 = direct ? r0 : c0;  // first source row of this tile
  const int64_t s1 = direct ? c0 : r0;  // first source column
  __shared__ float tile[kEwTile][kEwTile + 1];
  const int tx = threadIdx.x & 15;
  const int ty = threadIdx.x >> 4;
  // Source extents (padded); a 64x64 tile may reach past them when the pad
  // is not a multiple of 64, and those cells are never used for W.
  const int64_t src_rows = small ? d.m_pad : d.n_pad;
  const int64_t src_cols = small ? d.n_pad : d.m_pad;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int sl = ty + 16 * k;
    if (s0 + sl >= src_rows || s1 + tx * 4 >= src_cols) continue;
    if (small) {
      const int64_t off = (s0 + sl) * d.n_pad + s1 + tx * 4;
      const float4 v = gld<float4>(pick(d.xf, buf) + off);
      tile[sl][tx * 4 + 0] = v.x;
      tile[sl][tx * 4 + 1] = v.y;
      tile[sl][tx * 4 + 2] = v.z;
      tile[sl][tx * 4 + 3] = v.w;
      continue;
    }
    const int64_t off = (s0 + sl) * d.m_pad + s1 + tx * 4;
    const uint2 hv = gld<uint2>(pick(d.xt_hi, buf) + off);
    const uint2 lv = gld<uint2>(pick(d.xt_lo, buf) + off);
    tile[sl][tx * 4 + 0] = __uint_as_float(hv.x << 16) + __uint_as_float(lv.x << 16);
    tile[sl][tx * 4 + 1] = __uint_as_float(hv.x & 0xffff0000u) + __uint_as_float(lv.x & 0xffff0000u);
    tile[sl][tx * 4 + 2] = __uint_as_float(hv.y << 16) + __uint_as_float(lv.y << 16);
    tile[sl][tx * 4 + 3] = __uint_as_float(hv.y & 0xffff0000u) + __uint_as_float(lv.y & 0xffff0000u);
  }
  __syncthreads();
  const float ls = d.lr_scale;
  const float lwd = d.lr_wd;
  float* __restrict__ W = d.W;
  DiagAcc da;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rl = ty + 16 * k;
    const int64_t r = r0 + rl;
    if (r >= rows) continue;
    for (int c4 = 0; c4 < 4; ++c4) {
      const int cl = tx * 4 + c4;
      const int64_t c = c0 + cl;
      if (c >= cols) continue;
      const float o = direct ? tile[rl][cl] : tile[cl][rl];
      const int64_t e = r * cols + c;
      if (ortho) {
        gst(W + e, o);
      } else {
        const float w = gld<float>(W + e);
        const float nw = fmaf(-ls, o, fmaf(-lwd, w, w));  // W - lr*wd*W - lr*scale*O
        if constexpr (DG) diag_add(da, o, w, nw);
        gst(W + e, nw);
      }
    }
  }
  if constexpr (DG) diag_flush(da, d.diag_part + local * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
}

// ---------------------------------------------------------------- diagnostics
// One work-group per matrix: float64 sums of the per-wave partials in a
// fixed order (strided per thread, then a tree), and the muon_diag_t record.
__global__ __launch_bounds__(256) void diag_kernel(const MatDesc* __restrict__ descs,
                                                   muon_diag_t* __restrict__ out) {
  const MatDesc d = descs[blockIdx.x];
  const int ns = d.diag_slots;
  double o2 = 0.0, d2 = 0.0, w2 = 0.0;
  int bad = 0;
  for (int i = threadIdx.x; i < ns; i += 256) {
    const DiagPart p = gld<DiagPart>(d.diag_part + i);
    o2 += static_cast<double>(p.o2);
    d2 += static_cast<double>(p.d2);
    w2 += static_cast<double>(p.w2);
    bad |= p.bad;
  }
  __shared__ double red[3][256];
  red[0][threadIdx.x] = o2;
  red[1][threadIdx.x] = d2;
  red[2][threadIdx.x] = w2;
  const int any_bad = __syncthreads_or(bad != 0);
#pragma unroll
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) {
      red[0][threadIdx.x] += red[0][threadIdx.x + w];
      red[1][threadIdx.x] += red[1][threadIdx.x + w];
      red[2][threadIdx.x] += red[2][threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double inv = 1.0 / sqrt(static_cast<double>(d.rows) * static_cast<double>(d.cols));
    muon_diag_t r;
    r.momentum_norm = gld<float>(d.mstat);
    r.direction_rms = static_cast<float>(sqrt(red[0][0]) * inv);
    r.update_rms = static_cast<float>(sqrt(red[1][0]) * inv);
    r.weight_rms = static_cast<float>(sqrt(red[2][0]) * inv);
    r.nonfinite = (__float_as_int(gld<float>(d.mstat + 1)) ? 1 : 0) | (any_bad ? 2 : 0);
    r.reserved[0] = r.reserved[1] = r.reserved[2] = 0;
    gst(out + blockIdx.x, r);
  }
}

// ---------------------------------------------------------------- QK-Clip
// After the step, QK-Clip (the Kimi K2 result in the results section of the
// synthesis note) rescales the query and key projections head by head from
// the head's max logit.  One work-group per (matrix, head): a head whose
// max logit S is not above tau returns after reading S; otherwise its rows
// (contiguous, head_dim * cols floats) are multiplied by sqrt(tau / S)
// (float32 division and square root, both correctly rounded).
__global__ __launch_bounds__(256) void qk_clip_kernel(const ClipBatch b) {
  const int blk = blockIdx.x;
  const int mi = find_mat(b.prefix, b.n, blk);
  const ClipDesc& d = b.d[mi];
  const int h = blk - b.prefix[mi];
  const float s = gld<float>(d.max_logit + h);
  if (!(s > b.tau)) return;
  const float f = __fsqrt_rn(__fdiv_rn(b.tau, s));
  float* w = d.W + static_cast<int64_t>(h) * d.head_elems;
  if (d.vec) {
    const int64_t n4 = d.head_elems >> 2;
    for (int64_t i = threadIdx.x; i < n4; i += 256) {
      float4 v = gld<float4>(w + 4 * i);
      v.x *= f; v.y *= f; v.z *= f; v.w *= f;
      gst(w + 4 * i, v);
    }
  } else {
    for (int64_t i = threadIdx.x; i < d.head_elems; i += 256) gst(w + i, gld<float>(w + i) * f);
  }
}

// One counter set to zero (the per-call count of matrices marked for the
// prep pass, when a recorded plan replays a call without its table upload).
__global__ void zero_counter_kernel(int32_t* p) { gst(p, 0); }

// A small descriptor table passed by value (kernel argument) and stored into
// the workspace.
struct TableArg {
  uint32_t w[kTableArgBytes / 4];
};
__global__ __launch_bounds__(256) void table_write_kernel(uint32_t* __restrict__ dst, const TableArg t, int nwords) {
  for (int i = threadIdx.x; i < nwords; i += 256) gst(dst + i, t.w[i]);
}

// ---------------------------------------------------------------- copy probe
// Streaming copy of n16 16-byte words, the yardstick of the bandwidth-bound
// stages (one read and one write per byte, the momentum pass's mix).  Each
// lane keeps U 16-byte loads in flight before storing them; the grid
// strides over the buffer.  NT: nontemporal loads and stores (streamed
// past the caches).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                         int64_t n16) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * 256 * U;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * U + threadIdx.x; base < n16; base += step) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + 256 * u;
      if (i < n16) v[u] = NT ? __builtin_nontemporal_load(src + i) : gld<u32x4_t>(src + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + 256 * u;
      if (i < n16) {
        if (NT) __builtin_nontemporal_store(v[u], dst + i);
        else gst(dst + i, v[u]);
      }
    }
  }
}

}  // namespace

hipError_t launch_momentum(const MatDesc* d, const int32_t* prefix, int nmats, int total, float mu,
                           hipStream_t s) {
  hipLaunchKernelGGL(momentum_kernel, dim3(total), dim3(256), 0, s, d, prefix, nmats, mu);
  return hipGetLastError();
}

hipError_t launch_norm(const MatDesc* d, int nmats, float eps, int32_t* prep_count, hipStream_t s) {
  hipLaunchKernelGGL(norm_kernel, dim3(nmats), dim3(256), 0, s, d, eps, prep_count);
  return hipGetLastError();
}

hipError_t launch_prep(const MatDesc* d, const int32_t* prefix, int nmats, int total, float mu,
                       const int32_t* prep_count, hipStream_t s) {
  // Enough work-groups to fill the chip when every matrix needs the pass.
  const int grid = total < 4096 ? total : 4096;
  hipLaunchKernelGGL(prep_kernel, dim3(grid > 0 ? grid : 1), dim3(256), 0, s, d, prefix, nmats, mu, prep_count);
  return hipGetLastError();
}

hipError_t launch_update(const MatDesc* d, const int32_t* prefix, int nmats, int total, int buf,
                         bool diag, hipStream_t s) {
  if (diag)
    hipLaunchKernelGGL(update_kernel<true>, dim3(total), dim3(256), 0, s, d, prefix, nmats, buf);
  else
    hipLaunchKernelGGL(update_kernel<false>, dim3(total), dim3(256), 0, s, d, prefix, nmats, buf);
  return hipGetLastError();
}

hipError_t launch_diag(const MatDesc* d, int nmats, void* out, hipStream_t s) {
  hipLaunchKernelGGL(diag_kernel, dim3(nmats), dim3(256), 0, s, d, static_cast<muon_diag_t*>(out));
  return hipGetLastError();
}

hipError_t launch_copy_probe(const void* src, void* dst, int64_t n16, int variant, hipStream_t s) {
  // variant: bit 0 = nontemporal; bits 1.. = grid (0: 1024, 1: 4096, 2: 16384 work-groups)
  const int grids[3] = {1024, 4096, 16384};
  const int gi = variant >> 1;
  if (gi < 0 || gi > 2) return hipErrorInvalidValue;
  const dim3 grid(grids[gi]);
  const u32x4_t* a = static_cast<const u32x4_t*>(src);
  u32x4_t* b = static_cast<u32x4_t*>(dst);
  if (variant & 1)
    hipLaunchKernelGGL((copy_probe_kernel<4, true>), grid, dim3(256), 0, s, a, b, n16);
  else
    hipLaunchKernelGGL((copy_probe_kernel<4, false>), grid, dim3(256), 0, s, a, b, n16);
  return hipGetLastError();
}

hipError_t launch_qk_clip(const ClipBatch& b, hipStream_t s) {
  if (b.n <= 0 || b.prefix[b.n] <= 0) return hipSuccess;
  hipLaunchKernelGGL(qk_clip_kernel, dim3(b.prefix[b.n]), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_table_write(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (bytes > static_cast<size_t>(kTableArgBytes) || bytes % 4 != 0) return hipErrorInvalidValue;
  if (bytes == 0) return hipSuccess;
  TableArg t{};
  const uint32_t* w = static_cast<const uint32_t*>(src);
  for (size_t i = 0; i < bytes / 4; ++i) t.w[i] = w[i];
  hipLaunchKernelGGL(table_write_kernel, dim3(1), dim3(256), 0, s, static_cast<uint32_t*>(dst), t,
                     static_cast<int>(bytes / 4));
  return hipGetLastError();
}

hipError_t launch_zero_counter(int32_t* p, hipStream_t s) {
  hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(1), 0, s, p);
  return hipGetLastError();
}

}  // namespace muon
