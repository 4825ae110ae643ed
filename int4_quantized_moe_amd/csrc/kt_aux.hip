// Auxiliary kernels of the routed layer: activation rows to fp16 with a
// power-of-two exponent, zero fill, the per-token slot combine, the
// route-weight gradient, and the codec test hooks.
#include <limits.h>

#include <algorithm>

#include "kt_common.hpp"
#include "kt_internal.hpp"

namespace kt {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// ---------------------------------------------------------------- bf16 rows -> fp16 * 2^p

// One block per row: p = exponent that maps the row's largest magnitude below
// 2^15, then every element is stored as fp16(x * 2^p) (exact for bf16 values
// within 2^-24..2^15 of the scaled range), at its within-8 permuted position.
// Each thread moves 16-byte chunks of 8 values (cols is a multiple of 8; the
// permutation stays inside a chunk).
__global__ __launch_bounds__(256) void k_rows_to_half(const uint16_t* __restrict__ src, int64_t cols,
                                                      uint16_t* __restrict__ dst, int32_t* __restrict__ exps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const u32x4* s = reinterpret_cast<const u32x4*>(src + row * cols);
  u32x4* d = reinterpret_cast<u32x4*>(dst + row * cols);
  const int64_t n8 = cols / 8;
  float mx = 0.f;
  for (int64_t c = threadIdx.x; c < n8; c += blockDim.x) {
    const u32x4 v = s[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      mx = fmaxf(mx, fmaxf(fabsf(bf16_to_float((uint16_t)(w[q] & 0xffffu))), fabsf(bf16_to_float((uint16_t)(w[q] >> 16)))));
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int p = pow2_exponent_for(mx);
  for (int64_t c = threadIdx.x; c < n8; c += blockDim.x) {
    const u32x4 v = s[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint16_t o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint16_t b = (uint16_t)((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xffffu));
      o[perm_pos(k)] = float_to_half_bits(ldexpf(bf16_to_float(b), p));
    }
    d[c] = u32x4{o[0] | ((uint32_t)o[1] << 16), o[2] | ((uint32_t)o[3] << 16), o[4] | ((uint32_t)o[5] << 16),
                 o[6] | ((uint32_t)o[7] << 16)};
  }
  if (threadIdx.x == 0) exps[row] = p;
}

void launch_rows_to_half(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* dst, int32_t* exps,
                         hipStream_t st) {
  if (rows > 0) {
    k_rows_to_half<<<(unsigned)rows, 256, 0, st>>>(src, cols, dst, exps);
    note_launch();
  }
}

// ---------------------------------------------------------------- scales for the expert GEMMs

// One scale tensor [E][rows][G] (bf16, G = K / 32) to [active][G][rows] in
// fp16, rows of every aligned group of 8 in the within-8 permuted order, so that
// a GEMM stage reads the scales of its column (or contraction-row) block as one
// contiguous run in both orientations.  Experts that received no token-slot
// are skipped; the others go to their place among the experts in use.  An
// expert with a scale outside the exact domain is marked (sshift[2 e + grp])
// for k_scales_fix.  64 x 64 tiles pass through LDS so that the reads (along G,
// 16 bytes per lane where G allows) and the writes (along rows, 16 bytes per
// lane) are both coalesced.
__global__ __launch_bounds__(256) void k_scales_t(const uint16_t* __restrict__ s, int64_t rows, int64_t G,
                                                   const int32_t* __restrict__ expert_slot,
                                                   uint16_t* __restrict__ out, int32_t* __restrict__ sshift, int grp,
                                                   int fmt) {
  __shared__ uint16_t t[64][72];  // [row][group], 144-byte pitch
  __shared__ int nbad_w[4];
  const int64_t e = blockIdx.z;
  const int32_t es = expert_slot[e];
  if (es < 0) return;
  const int64_t r0 = (int64_t)blockIdx.x * 64, g0 = (int64_t)blockIdx.y * 64;
  const uint16_t* se = s + e * rows * G;
  uint16_t* oe = out + (int64_t)es * G * rows;
  int nbad = 0;
  {
    const int i = threadIdx.x >> 2, j0 = 16 * (threadIdx.x & 3);  // row r0 + i, groups g0 + j0 .. + 15
    const int64_t r = r0 + i;
    uint16_t v[16];
    if (r < rows && (G & 7) == 0 && g0 + j0 + 16 <= G) {
      const uint4 a = *reinterpret_cast<const uint4*>(se + r * G + g0 + j0);
      const uint4 b = *reinterpret_cast<const uint4*>(se + r * G + g0 + j0 + 8);
      const uint32_t wds[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        v[2 * q] = (uint16_t)(wds[q] & 0xffffu);
        v[2 * q + 1] = (uint16_t)(wds[q] >> 16);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = (r < rows && g0 + j0 + q < G) ? se[r * G + g0 + j0 + q] : 0;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float f = bf16_to_float(v[q]);
      const bool ok = fmt ? scale_in_domain_mxfp4(f) : scale_in_domain(f);
      nbad += (r < rows && g0 + j0 + q < G && !ok) ? 1 : 0;
      t[i][j0 + q] = float_to_half_bits(f);
    }
  }
  __syncthreads();
  {
    const int j = threadIdx.x >> 2, i0 = 16 * (threadIdx.x & 3);  // group g0 + j, positions r0 + i0 .. + 15
    const int64_t g = g0 + j;
    if (g < G) {
      uint16_t v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        // position p of an aligned group of 8 holds logical row (p & ~7) | ((p & 7) >> 1) | ((p & 1) << 2)
        const int pp = i0 + q;
        v[q] = t[(pp & ~7) | ((pp & 7) >> 1) | ((pp & 1) << 2)][j];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (r0 + i0 + 8 * h < rows) {  // rows is a multiple of 8
          uint4 o;
          o.x = v[8 * h + 0] | ((uint32_t)v[8 * h + 1] << 16);
          o.y = v[8 * h + 2] | ((uint32_t)v[8 * h + 3] << 16);
          o.z = v[8 * h + 4] | ((uint32_t)v[8 * h + 5] << 16);
          o.w = v[8 * h + 6] | ((uint32_t)v[8 * h + 7] << 16);
          *reinterpret_cast<uint4*>(oe + g * rows + r0 + i0 + 8 * h) = o;
        }
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) nbad += __shfl_xor(nbad, off);
  if ((threadIdx.x & 63) == 0) nbad_w[threadIdx.x >> 6] = nbad;
  __syncthreads();
  if (threadIdx.x == 0 && nbad_w[0] + nbad_w[1] + nbad_w[2] + nbad_w[3] > 0) atomicOr(&sshift[2 * e + grp], 1);
}

void launch_scales_t(const uint16_t* s, int64_t E, int64_t rows, int64_t G, const int32_t* expert_slot,
                     uint16_t* out, int32_t* sshift, int grp, int fmt, hipStream_t st) {
  if (E <= 0 || rows <= 0 || G <= 0) return;
  dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((G + 63) / 64), (unsigned)E);
  k_scales_t<<<grid, 256, 0, st>>>(s, rows, G, expert_slot, out, sshift, grp, fmt);
  note_launch();
}

// The scales of one expert's projection group (gate and up together, since the
// gate/up dX GEMM contracts over both; down alone) that k_scales_t marked:
// with s the smallest integer for which the largest magnitude times 2^-s lies
// at or below the domain's top (2720, or 2^13 for MXFP4), the tables hold
// scale * 2^-s instead and the GEMMs multiply their sums by 2^s.  The weights
// are then exact again wherever the group's scales span no more than the
// domain's range (about 2^25 for RAWINT4); scales still outside are counted.
// One block per (expert, group); rare, so plain strided loops.
struct ScaleFixArgs {
  const uint16_t* s[3];  // bf16 scales [E][rows][G]: gate, up, down
  uint16_t* out[3];      // fp16 tables [active][G][rows]
  int64_t rows[3], G[3];
  const int32_t* expert_slot;
  int32_t* sshift;
  unsigned long long* bad;
  int fmt;
};

__global__ __launch_bounds__(256) void k_scales_fix(ScaleFixArgs a) {
  __shared__ float red[2][4];
  __shared__ int s_shift;
  const int64_t e = blockIdx.x;
  const int grp = blockIdx.y;
  const int32_t es = a.expert_slot[e];
  if (es < 0) return;
  const int marked = a.sshift[2 * e + grp];  // every thread reads the mark before it is replaced
  if (!marked) return;
  const int first = grp == 0 ? 0 : 2, last = grp == 0 ? 1 : 2;
  // largest magnitude and smallest nonzero magnitude of the group
  float mx = 0.f, mn = INFINITY;
  for (int t = first; t <= last; ++t) {
    const int64_t n = a.rows[t] * a.G[t];
    const uint16_t* se = a.s[t] + e * n;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
      const float v = fabsf(bf16_to_float(se[i]));
      mx = fmaxf(mx, v);
      if (v > 0.f) mn = fminf(mn, v);
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off));
    mn = fminf(mn, __shfl_xor(mn, off));
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = mx;
    red[1][threadIdx.x >> 6] = mn;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    const float top = a.fmt ? 0x1p13f : 2720.f;
    int sh = 0;
    if (mx < INFINITY) {  // (a non-finite scale stays outside whatever the shift)
      while (ldexpf(mx, -sh) > top) ++sh;
      while (sh > -160 && ldexpf(mx, -(sh - 1)) <= top) --sh;
    }
    s_shift = sh;
  }
  __syncthreads();
  const int sh = s_shift;
  int nbad = 0;
  for (int t = first; t <= last; ++t) {
    const int64_t rows = a.rows[t], G = a.G[t], n = rows * G;
    const uint16_t* se = a.s[t] + e * n;
    uint16_t* oe = a.out[t] + (int64_t)es * G * rows;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
      const int64_t r = i / G, g = i % G;
      const float v = ldexpf(bf16_to_float(se[i]), -sh);
      nbad += (a.fmt ? scale_in_domain_mxfp4(v) : scale_in_domain(v)) ? 0 : 1;
      oe[g * rows + perm_pos((int)(r & 7)) + (r & ~(int64_t)7)] = float_to_half_bits(v);
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) nbad += __shfl_xor(nbad, off);
  __syncthreads();  // red[] is reused
  if ((threadIdx.x & 63) == 0) red[0][threadIdx.x >> 6] = __int_as_float(nbad);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int total = __float_as_int(red[0][0]) + __float_as_int(red[0][1]) + __float_as_int(red[0][2]) +
                      __float_as_int(red[0][3]);
    if (total) atomicAdd(a.bad, (unsigned long long)total);
    a.sshift[2 * e + grp] = sh;
  }
}

void launch_scales_fix(const LayerPtrs& L, const Dims& d, const int32_t* expert_slot, int32_t* sshift,
                       uint16_t* sct_g, uint16_t* sct_u, uint16_t* sct_d, unsigned long long* bad, hipStream_t st) {
  if (d.E <= 0) return;
  ScaleFixArgs a;
  a.s[0] = L.sg;
  a.s[1] = L.su;
  a.s[2] = L.sd;
  a.out[0] = sct_g;
  a.out[1] = sct_u;
  a.out[2] = sct_d;
  a.rows[0] = a.rows[1] = d.I;
  a.G[0] = a.G[1] = d.H / kGroup;
  a.rows[2] = d.H;
  a.G[2] = d.I / kGroup;
  a.expert_slot = expert_slot;
  a.sshift = sshift;
  a.bad = bad;
  a.fmt = d.fmt;
  k_scales_fix<<<dim3((unsigned)d.E, 2), 256, 0, st>>>(a);
  note_launch();
}

// ---------------------------------------------------------------- one exponent per row

// h and dG|dU leave their producing GEMM with one exponent per (row, column
// chunk), since no tile sees a whole row.  One wave per row brings every chunk
// to the row's smallest exponent (fp16 times 2^d, d <= 0, rounded to nearest
// even) and records that exponent for every chunk.  Columns at or above `split`
// belong to the second operand, whose chunks start again at `split` and are
// numbered from nch / 2 (dG|dU); split = cols for a single operand (h).
__global__ __launch_bounds__(256) void k_normalize_chunks(uint16_t* __restrict__ buf, int32_t* __restrict__ exps,
                                                          const int32_t* __restrict__ nrows, int64_t cols,
                                                          int64_t split, int nch, int chunkw) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= *nrows) return;
  int32_t* ex = exps + row * nch;
  int mn = INT_MAX;
  for (int c = lane; c < nch; c += 64) mn = min(mn, ex[c]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) mn = min(mn, __shfl_xor(mn, off));
  uint16_t* b = buf + row * cols;
  for (int64_t c8 = (int64_t)lane * 8; c8 < cols; c8 += 512) {
    const int c = c8 < split ? (int)(c8 / chunkw) : nch / 2 + (int)((c8 - split) / chunkw);
    const int d = mn - ex[c];
    if (d == 0) continue;
    const uint16_t sb = half_pow2_bits(d);
    const half2_t s2 = __builtin_bit_cast(half2_t, (uint32_t)sb | ((uint32_t)sb << 16));
    u32x4 v = *reinterpret_cast<const u32x4*>(b + c8);
    v.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, (uint32_t)v.x) * s2);
    v.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, (uint32_t)v.y) * s2);
    v.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, (uint32_t)v.z) * s2);
    v.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, (uint32_t)v.w) * s2);
    *reinterpret_cast<u32x4*>(b + c8) = v;
  }
  // every lane has read the exponents it needs before any is overwritten
  __builtin_amdgcn_wave_barrier();
  for (int c = lane; c < nch; c += 64) ex[c] = mn;
}

void launch_normalize_chunks(uint16_t* buf, int32_t* exps, const int32_t* nrows, int64_t max_rows, int64_t cols,
                             int64_t split, int nch, int chunkw, hipStream_t st) {
  if (max_rows > 0) {
    k_normalize_chunks<<<(unsigned)((max_rows + 3) / 4), 256, 0, st>>>(buf, exps, nrows, cols, split, nch, chunkw);
    note_launch();
  }
}

__global__ void k_fill_zero(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

void launch_fill_zero_f32(float* p, int64_t n, hipStream_t st) {
  if (n > 0) {
    k_fill_zero<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n);
    note_launch();
  }
}

// ---------------------------------------------------------------- combine and dRoute

// out[t, c] = sum over valid slots s of stage[t*k + s, c] * 2^-p(t*k + s, c / 64), in slot
// order, in fp32, then to bf16 (round to nearest even); staged values are fp16.  Each
// thread sums 8 columns (one 16-byte staged chunk per slot); a block covers whole
// rows of one token.  The slots are read eight at a time, all eight requests out
// before the first sum (a dropped slot's row is read but not added).
__global__ __launch_bounds__(1024) void k_combine(const uint16_t* __restrict__ stage,
                                                  const int32_t* __restrict__ stexp, int64_t st_nch,
                                                  const int64_t* __restrict__ ids, int topk, int E, int64_t H,
                                                  uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int64_t c = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * 8;
  if (c >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < topk; s0 += 8) {
    u32x4 v[8];
    int ex[8];
    bool ok[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int s = min(s0 + j, topk - 1);
      const int64_t slot = t * topk + s;
      const int64_t e = ids[slot];
      ok[j] = s0 + j < topk && e >= 0 && e < E;
      v[j] = *reinterpret_cast<const u32x4*>(stage + slot * H + c);
      ex[j] = -stexp[slot * st_nch + c / kStageExp];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!ok[j]) continue;
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += ldexpf(half_bits_to_float((uint16_t)(w[q] & 0xffffu)), ex[j]);
        acc[2 * q + 1] += ldexpf(half_bits_to_float((uint16_t)(w[q] >> 16)), ex[j]);
      }
    }
  }
  // two 8-byte stores: the output is only required to be 8-byte aligned
  uint2 o0, o1;
  o0.x = float_to_bf16(acc[0]) | ((uint32_t)float_to_bf16(acc[1]) << 16);
  o0.y = float_to_bf16(acc[2]) | ((uint32_t)float_to_bf16(acc[3]) << 16);
  o1.x = float_to_bf16(acc[4]) | ((uint32_t)float_to_bf16(acc[5]) << 16);
  o1.y = float_to_bf16(acc[6]) | ((uint32_t)float_to_bf16(acc[7]) << 16);
  *reinterpret_cast<uint2*>(out + t * H + c) = o0;
  *reinterpret_cast<uint2*>(out + t * H + c + 4) = o1;
}

void launch_combine(const Dims& d, const uint16_t* stage, const int32_t* stexp, int64_t st_nch, const int64_t* ids,
                    uint16_t* out, hipStream_t st) {
  if (d.qlen == 0) return;
  // one block per token row when it fits (up to 1024 threads of 8 columns)
  const int64_t chunks = d.H / 8;
  const int64_t thr = std::min<int64_t>(1024, (chunks + 63) / 64 * 64);
  dim3 grid((unsigned)d.qlen, (unsigned)((chunks + thr - 1) / thr));
  k_combine<<<grid, (unsigned)thr, 0, st>>>(stage, stexp, st_nch, ids, (int)d.K, (int)d.E, d.H, out);
  note_launch();
}

__global__ void k_droute(const int32_t* __restrict__ row_of_slot, const float* __restrict__ drpart, int64_t Ms,
                         int nt, float* __restrict__ grad_route) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= Ms) return;
  const int m = row_of_slot[s];
  float v = 0.f;
  if (m >= 0)
    for (int j = 0; j < nt; ++j) v += drpart[(int64_t)m * nt + j];
  grad_route[s] = v;
}

void launch_droute(const Dims& d, const WsMap& w, void* ws, float* grad_route, hipStream_t st) {
  if (d.Ms == 0) return;
  k_droute<<<(unsigned)((d.Ms + 255) / 256), 256, 0, st>>>(ws_ptr<int32_t>(ws, w.row_of_slot),
                                                           ws_ptr<float>(ws, w.drpart), d.Ms, (int)w.dr_nt,
                                                           grad_route);
  note_launch();
}

// gate/up pre-activations the forward saved (quad-row layout: row m of expert e
// at position q = qoffsets[e] + m - offsets[e], element (q / 4, col, q % 4)),
// gathered into slot order; a dropped slot's row is zero
__global__ void k_saved_preact(const int32_t* __restrict__ row_of_slot, const int32_t* __restrict__ offsets,
                               const int32_t* __restrict__ qoffsets, int E, const float* __restrict__ g,
                               const float* __restrict__ u, int64_t I, float* __restrict__ gate,
                               float* __restrict__ up) {
  const int64_t s = blockIdx.x;
  const int m = row_of_slot[s];
  int64_t q = 0;
  if (m >= 0) {
    int lo = 0, hi = E - 1;  // the expert e with offsets[e] <= m < offsets[e + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (offsets[mid] <= m)
        lo = mid;
      else
        hi = mid - 1;
    }
    q = (int64_t)qoffsets[lo] + (m - offsets[lo]);
  }
  for (int64_t c = threadIdx.x; c < I; c += blockDim.x) {
    const int64_t at = ((q >> 2) * I + c) * 4 + (q & 3);
    gate[s * I + c] = m >= 0 ? g[at] : 0.f;
    up[s * I + c] = m >= 0 ? u[at] : 0.f;
  }
}

void launch_saved_preact(const Dims& d, const WsMap& w, const void* ws, float* gate, float* up, hipStream_t st) {
  if (d.Ms == 0) return;
  void* base = const_cast<void*>(ws);
  k_saved_preact<<<(unsigned)d.Ms, 256, 0, st>>>(ws_ptr<int32_t>(base, w.row_of_slot),
                                                 ws_ptr<int32_t>(base, w.offsets),
                                                 ws_ptr<int32_t>(base, w.qoffsets), (int)d.E,
                                                 ws_ptr<float>(base, w.g), ws_ptr<float>(base, w.u), d.I, gate,
                                                 up);
  note_launch();
}

// ---------------------------------------------------------------- codec hooks

__global__ void k_unpack(const uint8_t* __restrict__ packed, int64_t nbytes, int8_t* __restrict__ codes) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nbytes) return;
  const uint8_t b = packed[i];
  codes[2 * i] = (int8_t)((int)(b & 15) - 8);
  codes[2 * i + 1] = (int8_t)((int)(b >> 4) - 8);
}

void launch_unpack(const uint8_t* packed, int64_t n, int64_t k, int8_t* codes, hipStream_t st) {
  const int64_t nbytes = n * (k / 2);
  if (nbytes > 0) {
    k_unpack<<<(unsigned)((nbytes + 255) / 256), 256, 0, st>>>(packed, nbytes, codes);
    note_launch();
  }
}

// The 8 fp16 values of two decodes are the same numbers (a zero may differ in
// sign: the two decoders round an exact zero with different signs, which no
// product or sum downstream can tell apart).
__device__ __forceinline__ bool same_values(u32x4 a, u32x4 b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
  bool same = true;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t p = (x[i] >> (16 * h)) & 0xffffu, q = (y[i] >> (16 * h)) & 0xffffu;
      same = same && (p == q || ((p | q) & 0x7fffu) == 0);
    }
  return same;
}

// the matrix kernels' decoders: one packed dword -> 8 fp16 values -> fp32, by
// the stored-orientation decoder and the transposed one (one scale for the
// whole dword here); a dword where they give different values comes out as NaN
__global__ void k_dequant(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales, int64_t n,
                          int64_t k, int fmt, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // dword index
  const int64_t dwords_per_row = k / 8;
  if (i >= n * dwords_per_row) return;
  const int64_t row = i / dwords_per_row, d = i % dwords_per_row;
  const uint32_t wv = reinterpret_cast<const uint32_t*>(packed + row * (k / 2))[d];
  // the decoder of the forward matrix kernels (codes along the packed row)
  const _Float16 s = (_Float16)bf16_to_float(scales[row * (k / kGroup) + (d * 8) / kGroup]);
  const half2_t s2 = {s, s};
  u32x4 r;
  if (fmt) {
    // the MXFP4 decoders of both orientations; a disagreement (none is
    // expected) shows as NaN in every value of the dword
    r = decode_dword_e2m1(wv, (float)s);
    const u32x4 t = decode_dword_perm_e2m1(wv, s2, s2, s2, s2);
    if (!same_values(t, r)) r = u32x4{0x7e007e00u, 0x7e007e00u, 0x7e007e00u, 0x7e007e00u};
  } else {
    // the RAWINT4 decoders of both orientations, likewise
    const DecodeConsts dc = decode_consts();
    r = decode_dword_fma(wv, s2 * (half2_t){16.f16, 16.f16}, s2 * (half2_t){-24.f16, -24.f16}, dc);
    const u32x4 t = decode_dword_perm(wv, s2, s2, s2, s2, dc);
    if (!same_values(t, r)) r = u32x4{0x7e007e00u, 0x7e007e00u, 0x7e007e00u, 0x7e007e00u};
  }
  const uint32_t words[4] = {r.x, r.y, r.z, r.w};  // (k0, k4), (k1, k5), (k2, k6), (k3, k7)
  float* o = out + row * k + d * 8;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[j] = half_bits_to_float((uint16_t)(words[j] & 0xffffu));
    o[j + 4] = half_bits_to_float((uint16_t)(words[j] >> 16));
  }
}

void launch_dequant(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, int fmt, float* out,
                    hipStream_t st) {
  const int64_t total = n * (k / 8);
  if (total > 0) {
    k_dequant<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(packed, scales, n, k, fmt, out);
    note_launch();
  }
}

}  // namespace kt
