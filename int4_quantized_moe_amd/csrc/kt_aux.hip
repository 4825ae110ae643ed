// Auxiliary kernels of the routed layer: activation rows to fp16 with a
// power-of-two exponent, zero fill, the per-token slot combine, the
// route-weight gradient, and the codec test hooks.
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
