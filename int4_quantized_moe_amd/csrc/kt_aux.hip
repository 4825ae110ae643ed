// Auxiliary kernels of the routed layer: activation rows to fp16 with a
// power-of-two exponent, LoRA side products and LoRA gradient reductions in
// fp32, the per-token slot combine, the route-weight gradient, and the codec
// test hooks.
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
__global__ __launch_bounds__(256) void k_rows_to_half(const uint16_t* __restrict__ src, int64_t cols,
                                                      uint16_t* __restrict__ dst, int32_t* __restrict__ exps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* s = src + row * cols;
  float mx = 0.f;
  for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) mx = fmaxf(mx, fabsf(bf16_to_float(s[c])));
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int p = pow2_exponent_for(mx);
  for (int64_t c = threadIdx.x; c < cols; c += blockDim.x)
    dst[row * cols + perm_pos((int)c)] = float_to_half_bits(ldexpf(bf16_to_float(s[c]), p));
  if (threadIdx.x == 0) exps[row] = p;
}

void launch_rows_to_half(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* dst, int32_t* exps,
                         hipStream_t st) {
  if (rows > 0) k_rows_to_half<<<(unsigned)rows, 256, 0, st>>>(src, cols, dst, exps);
}

// ---------------------------------------------------------------- row views

__device__ __forceinline__ float rv_value(const RowView& v, int64_t m, int64_t c, const int32_t* sorted_slot,
                                          int topk) {
  float val;
  if (v.kind == kSrcTokBf16) {
    const int64_t tok = sorted_slot[m] / topk;
    val = bf16_to_float(static_cast<const uint16_t*>(v.ptr)[tok * v.ld + v.col_off + c]);
  } else if (v.kind == kSrcF32) {
    val = static_cast<const float*>(v.ptr)[m * v.ld + v.col_off + c];
  } else {
    val = half_bits_to_float(static_cast<const uint16_t*>(v.ptr)[m * v.ld + perm_pos((int)(v.col_off + c))]);
    val = ldexpf(val, -v.exps[m * v.exp_ld + v.exp_off + c / v.chunk_w]);
  }
  if (v.slot_scale) val *= v.slot_scale[sorted_slot[m]];
  return val;
}

// ---------------------------------------------------------------- LoRA side products

// out[m, q] = sum_k src(m, k) W(e, q, k) for the kMTAux rows of one tile and 32
// values of q; fp32 throughout, k summed in increasing order.
__global__ __launch_bounds__(256) void k_lora_rowproj(RowView src, int64_t kdim, const float* __restrict__ W, int rk,
                                                      float* __restrict__ out, int R, int topk,
                                                      const int32_t* __restrict__ sorted_slot,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ tile_e,
                                                      const int32_t* __restrict__ tile_m0,
                                                      const unsigned long long* __restrict__ counters) {
  __shared__ float S[kMTAux][65];
  __shared__ float Wc[32][65];
  const int tile = blockIdx.x;
  if ((unsigned long long)tile >= counters[kNumTilesAux]) return;
  const int e = tile_e[tile], m0 = tile_m0[tile];
  const int mlen = min(kMTAux, offsets[e + 1] - m0);
  const int q0 = blockIdx.y * 32;
  const int tid = threadIdx.x, row = tid >> 2, qs = (tid & 3) * 8;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int64_t k0 = 0; k0 < kdim; k0 += 64) {
    for (int it = tid; it < kMTAux * 64; it += 256) {
      const int r = it >> 6, kk = it & 63;
      S[r][kk] = (r < mlen && k0 + kk < kdim) ? rv_value(src, m0 + r, k0 + kk, sorted_slot, topk) : 0.f;
    }
    for (int it = tid; it < 32 * 64; it += 256) {
      const int qi = it >> 6, kk = it & 63;
      const int q = q0 + qi;
      const int64_t k = k0 + kk;
      float v = 0.f;
      if (q < R && k < kdim) v = rk ? W[((int64_t)e * R + q) * kdim + k] : W[((int64_t)e * kdim + k) * R + q];
      Wc[qi][kk] = v;
    }
    __syncthreads();
    for (int kk = 0; kk < 64; ++kk) {
      const float s = S[row][kk];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += s * Wc[qs + j][kk];
    }
    __syncthreads();
  }
  if (row < mlen) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = q0 + qs + j;
      if (q < R) out[(int64_t)(m0 + row) * R + q] = acc[j];
    }
  }
}

void launch_lora_rowproj(const Dims& d, const WsMap& w, void* ws, const RowView& src, int64_t kdim, const float* W,
                         bool rk, float* out, hipStream_t st) {
  if (w.max_tiles_aux == 0) return;
  dim3 grid((unsigned)w.max_tiles_aux, (unsigned)((d.R + 31) / 32));
  k_lora_rowproj<<<grid, 256, 0, st>>>(src, kdim, W, rk ? 1 : 0, out, (int)d.R, (int)d.K,
                                       ws_ptr<int32_t>(ws, w.sorted_slot), ws_ptr<int32_t>(ws, w.offsets),
                                       ws_ptr<int32_t>(ws, w.tile_e_aux), ws_ptr<int32_t>(ws, w.tile_m0_aux),
                                       ws_ptr<unsigned long long>(ws, w.counters));
}

// ---------------------------------------------------------------- LoRA gradient reductions

// G[e, p, q] = (accumulate ? G : 0) + scale * sum_{rows m of e} P(m, p) Q(m, q);
// one block per (expert, 64x64 tile); rows summed in sorted (= slot) order.
__global__ __launch_bounds__(256) void k_lora_grad(RowView P, int64_t np, RowView Q, int64_t nq,
                                                   float* __restrict__ G, int accumulate, float scale, int topk,
                                                   const int32_t* __restrict__ sorted_slot,
                                                   const int32_t* __restrict__ offsets) {
  __shared__ float Pc[32][65];
  __shared__ float Qc[32][65];
  const int e = blockIdx.x;
  const int64_t p0 = (int64_t)blockIdx.y * 64, q0 = (int64_t)blockIdx.z * 64;
  const int start = offsets[e], cnt = offsets[e + 1] - start;
  if (cnt == 0 && accumulate) return;
  const int tid = threadIdx.x, pi = (tid >> 4) * 4, qi = (tid & 15) * 4;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
  for (int mm = 0; mm < cnt; mm += 32) {
    for (int it = tid; it < 32 * 64; it += 256) {
      const int r = it >> 6, c = it & 63;
      const int64_t m = start + mm + r;
      const bool vr = mm + r < cnt;
      Pc[r][c] = (vr && p0 + c < np) ? rv_value(P, m, p0 + c, sorted_slot, topk) : 0.f;
      Qc[r][c] = (vr && q0 + c < nq) ? rv_value(Q, m, q0 + c, sorted_slot, topk) : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < 32; ++r) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float pv = Pc[r][pi + a];
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] += pv * Qc[r][qi + b];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t p = p0 + pi + a, q = q0 + qi + b;
      if (p < np && q < nq) {
        const int64_t idx = ((int64_t)e * np + p) * nq + q;
        const float prev = accumulate ? G[idx] : 0.f;
        G[idx] = prev + scale * acc[a][b];
      }
    }
}

void launch_lora_grad(const Dims& d, const WsMap& w, void* ws, const RowView& P, int64_t np, const RowView& Q,
                      int64_t nq, float* G, int accumulate, float scale, hipStream_t st) {
  dim3 grid((unsigned)d.E, (unsigned)((np + 63) / 64), (unsigned)((nq + 63) / 64));
  k_lora_grad<<<grid, 256, 0, st>>>(P, np, Q, nq, G, accumulate, scale, (int)d.K, ws_ptr<int32_t>(ws, w.sorted_slot),
                                    ws_ptr<int32_t>(ws, w.offsets));
}

__global__ void k_fill_zero(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

void launch_fill_zero_f32(float* p, int64_t n, hipStream_t st) {
  if (n > 0) k_fill_zero<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n);
}

// ---------------------------------------------------------------- combine and dRoute

// out[t, c] = sum over valid slots s of stage[t*k + s, c], in slot order, to bf16
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ stage, const int64_t* __restrict__ ids,
                                                 int topk, int E, int64_t H, uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int64_t c = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * 4;
  if (c >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < topk; ++s) {
    const int64_t slot = t * topk + s;
    const int64_t e = ids[slot];
    if (e < 0 || e >= E) continue;
    const float4 v = *reinterpret_cast<const float4*>(stage + slot * H + c);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  uint2 o;
  o.x = float_to_bf16(acc.x) | ((uint32_t)float_to_bf16(acc.y) << 16);
  o.y = float_to_bf16(acc.z) | ((uint32_t)float_to_bf16(acc.w) << 16);
  *reinterpret_cast<uint2*>(out + t * H + c) = o;
}

void launch_combine(const Dims& d, const float* stage, const int64_t* ids, uint16_t* out, hipStream_t st) {
  if (d.qlen == 0) return;
  dim3 grid((unsigned)d.qlen, (unsigned)((d.H / 4 + 255) / 256));
  k_combine<<<grid, 256, 0, st>>>(stage, ids, (int)d.K, (int)d.E, d.H, out);
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
  if (nbytes > 0) k_unpack<<<(unsigned)((nbytes + 255) / 256), 256, 0, st>>>(packed, nbytes, codes);
}

// the matrix kernels' decoder: one packed dword -> 8 fp16 values -> fp32
__global__ void k_dequant(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales, int64_t n,
                          int64_t k, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // dword index
  const int64_t dwords_per_row = k / 8;
  if (i >= n * dwords_per_row) return;
  const int64_t row = i / dwords_per_row, d = i % dwords_per_row;
  const uint32_t wv = reinterpret_cast<const uint32_t*>(packed + row * (k / 2))[d];
  const _Float16 s = (_Float16)bf16_to_float(scales[row * (k / kGroup) + (d * 8) / kGroup]);
  const u32x4 r = decode_dword(wv, half2_t{s, s});
  const uint32_t words[4] = {r.x, r.y, r.z, r.w};
  float* o = out + row * k + d * 8;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[2 * j] = half_bits_to_float((uint16_t)(words[j] & 0xffffu));
    o[2 * j + 1] = half_bits_to_float((uint16_t)(words[j] >> 16));
  }
}

void launch_dequant(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, float* out, hipStream_t st) {
  const int64_t total = n * (k / 8);
  if (total > 0) k_dequant<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(packed, scales, n, k, out);
}

}  // namespace kt
