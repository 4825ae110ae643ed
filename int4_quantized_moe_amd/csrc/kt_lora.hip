// LoRA side products and LoRA gradient reductions on bf16 MFMA.
//
// Both are small grouped matrix products of the page "rawint4_sft_reference.py"
// (_lora_linear inside routed_rawint4_lora, and its gradients):
//   side products   out[m, q] = sum_k a(m, k) W(q, k)   (x A^T, h A_d^T, dY B_d, dG B_g, dU B_u)
//   gradients       G[e, p, q] = sum over the expert's rows m of P(m, p) Q(m, q)
// fp32 operands are split into bf16 hi + lo and each fragment pair takes three
// bf16 MFMAs (hi*hi + hi*lo + lo*hi); exactly-bf16 activations (x, dY) have no
// lo part and take two.
//
// Side products: a workgroup owns one row tile of the expert GEMMs' tile list
// by all 64 * NB output columns, walks the contraction 32 at a time with the
// next step's global loads in flight while the current one is multiplied
// (double-buffered LDS, one barrier per step), and splits each operand element
// once.  The hi/lo split truncates: hi keeps the top 16 bits, lo the top 16 bits
// of the exact remainder (relative error below 2^-14 per element; fp16
// activations split exactly).
//
// Gradients: a workgroup owns a 64 x 64 tile of G and walks the expert's rows
// 32 at a time in a fixed order, so results do not depend on scheduling; both
// operands are staged row-major ([k][column]) and read back with
// ds_read_tr16_b64, which hands each lane 4 consecutive rows of one column.
#include "kt_common.hpp"
#include "kt_internal.hpp"

namespace kt {

constexpr int kLT = 64;       // output tile edge
constexpr int kLK = 32;       // contraction step
constexpr int kLQ = kLT + 8;  // [k][column] pitch in 16-bit elements (144 B)

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t* lds_v4s_ptr;

struct LoraArgs {
  int topk;
  const int32_t* sorted_slot;
  const int32_t* offsets;
  // P(m, p), Q(m, q) over the expert's rows; G[e, p, q]
  RowView P, Q;
  int64_t np_, nq_;
  float* G;
  int accumulate;
  float scale;
};

// Up to 8 consecutive values of a row view starting at column c (c % 8 == 0), in
// stored order (for fp16 rows the within-8 permuted order); `nvalid` columns are
// read, the rest are 0.  bf16 and fp16 rows are H or I wide (multiples of 32),
// so for them nvalid is always 8.
__device__ __forceinline__ void load8(const RowView& v, int64_t m, int64_t c, int32_t tok_or_m, int nvalid,
                                      float* out) {
  if (v.kind == kSrcTokBf16) {
    const uint16_t* p = static_cast<const uint16_t*>(v.ptr) + (int64_t)tok_or_m * v.ld + v.col_off + c;
    u32x4 r;
    __builtin_memcpy(&r, p, 16);
    const uint32_t wds[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(wds[i] << 16);
      out[2 * i + 1] = __uint_as_float(wds[i] & 0xffff0000u);
    }
  } else if (v.kind == kSrcF32) {
    const float* p = static_cast<const float*>(v.ptr) + m * v.ld + v.col_off + c;
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = i < nvalid ? p[i] : 0.f;
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(v.ptr) + m * v.ld + v.col_off + c;
    u32x4 r;
    __builtin_memcpy(&r, p, 16);
    const int ex = v.exps[m * v.exp_ld + v.exp_off + c / v.chunk_w];
    const uint32_t wds[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = ldexpf(half_bits_to_float((uint16_t)(wds[i] & 0xffffu)), -ex);
      out[2 * i + 1] = ldexpf(half_bits_to_float((uint16_t)(wds[i] >> 16)), -ex);
    }
  }
}

__global__ __launch_bounds__(256) void k_lora_grad(LoraArgs a) {
  __shared__ __align__(16) uint16_t Ah[kLK * kLQ], Al[kLK * kLQ], Bh[kLK * kLQ], Bl[kLK * kLQ];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  floatx4 acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int e = blockIdx.x;
  const int m0 = a.offsets[e];
  const int rows = a.offsets[e + 1] - m0;
  if (rows == 0 && a.accumulate) return;
  const int64_t i0 = (int64_t)blockIdx.y * kLT, j0 = (int64_t)blockIdx.z * kLT;
  for (int k0 = 0; k0 < rows; k0 += kLK) {
    // thread -> (token row k, 8 consecutive output columns), stored row-major [k][column]
    const int k = tid >> 3, c = 8 * (tid & 7);
    const bool vk = k0 + k < rows;
    const int64_t m = m0 + k0 + k;
    float pv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float qv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (vk) {
      const int32_t slot = a.sorted_slot[m];
      const int32_t tok = slot / a.topk;
      if (i0 + c < a.np_) {
        load8(a.P, m, i0 + c, a.P.kind == kSrcTokBf16 ? tok : (int32_t)m, (int)min<int64_t>(8, a.np_ - (i0 + c)), pv);
        if (a.P.slot_scale) {
          const float sv = a.P.slot_scale[slot];
#pragma unroll
          for (int t = 0; t < 8; ++t) pv[t] *= sv;
        }
      }
      if (j0 + c < a.nq_) {
        load8(a.Q, m, j0 + c, a.Q.kind == kSrcTokBf16 ? tok : (int32_t)m, (int)min<int64_t>(8, a.nq_ - (j0 + c)), qv);
        if (a.Q.slot_scale) {
          const float sv = a.Q.slot_scale[slot];
#pragma unroll
          for (int t = 0; t < 8; ++t) qv[t] *= sv;
        }
      }
    }
    // fp16 views keep the within-8 permuted column order: put each value at its logical column
    float pl[8], ql[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int src = (t & 4) ? 2 * (t & 3) + 1 : 2 * t;  // stored slot of logical offset t
      pl[t] = a.P.kind == kSrcHalfChunked ? pv[src] : pv[t];
      ql[t] = a.Q.kind == kSrcHalfChunked ? qv[src] : qv[t];
    }
    u32x4 hi, lo;
    split8(pl, hi, lo);
    __builtin_memcpy(&Ah[k * kLQ + c], &hi, 16);
    __builtin_memcpy(&Al[k * kLQ + c], &lo, 16);
    split8(ql, hi, lo);
    __builtin_memcpy(&Bh[k * kLQ + c], &hi, 16);
    __builtin_memcpy(&Bl[k * kLQ + c], &lo, 16);
    __syncthreads();
    // lanes 4r..4r+3 of a 16-lane group address token row (8 lg + r) (+4), columns 4 (lr & 3).. of the block:
    // each lane receives 4 consecutive token rows of its column
    const int rr = lr >> 2, cc = 4 * (lr & 3);
    u32x4 ah, al;
    {
      const int base = (8 * lg + rr) * kLQ + w * 16 + cc;
      const v4s_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(&Ah[base]));
      const v4s_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(&Ah[base + 4 * kLQ]));
      const v4s_t l0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(&Al[base]));
      const v4s_t l1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(&Al[base + 4 * kLQ]));
      ah = u32x4{pack2(h0.x, h0.y), pack2(h0.z, h0.w), pack2(h1.x, h1.y), pack2(h1.z, h1.w)};
      al = u32x4{pack2(l0.x, l0.y), pack2(l0.z, l0.w), pack2(l1.x, l1.y), pack2(l1.z, l1.w)};
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int base = (8 * lg + rr) * kLQ + f * 16 + cc;
      const v4s_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(&Bh[base]));
      const v4s_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(&Bh[base + 4 * kLQ]));
      const v4s_t l0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(&Bl[base]));
      const v4s_t l1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(&Bl[base + 4 * kLQ]));
      const u32x4 bh = {pack2(h0.x, h0.y), pack2(h0.z, h0.w), pack2(h1.x, h1.y), pack2(h1.z, h1.w)};
      const u32x4 bl = {pack2(l0.x, l0.y), pack2(l0.z, l0.w), pack2(l1.x, l1.y), pack2(l1.z, l1.w)};
      acc[f] = mfma_bf16(ah, bh, acc[f]);
      acc[f] = mfma_bf16(ah, bl, acc[f]);
      acc[f] = mfma_bf16(al, bh, acc[f]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t i = i0 + w * 16 + lg * 4 + t;  // output row (p)
      const int64_t j = j0 + f * 16 + lr;          // output column (q)
      if (i >= a.np_ || j >= a.nq_) continue;
      const int64_t idx = ((int64_t)e * a.np_ + i) * a.nq_ + j;
      const float prev = a.accumulate ? a.G[idx] : 0.f;
      a.G[idx] = prev + a.scale * acc[f][t];
    }
}

// ================================================================ side products

constexpr int kSK = 32;  // contraction values per step

struct SideArgs {
  int topk;
  const int32_t* sorted_slot;
  const int32_t* offsets;
  const int32_t* tile_e;
  const int32_t* tile_m0;
  const unsigned long long* counters;
  const uint16_t* src;  // token rows of bf16 (exact) or sorted rows of fp16 with a row exponent
  int64_t ld, col_off;
  const int32_t* exps;  // fp16 rows: exponent of row m at exps[m * exp_ld + exp_off]
  int64_t exp_ld, exp_off;
  const float* W;   // [E, R, kdim] (rk) or [E, kdim, R]
  const float* W2;  // optional second matrix: output columns R .. 2R - 1
  int rk, kdim, R, nq;
  float* out;
  float* out2;
  uint16_t* split;  // bf16 hi/lo planes [Ms][2][split_ld] of the product times split_scale
  int64_t split_ld, split_off, split_off2;
  float split_scale;
};

// 8 fp32 -> bf16 hi (top 16 bits) and lo (top 16 bits of the exact remainder)
__device__ __forceinline__ void split8_trunc(const float* v, u32x4& hi, u32x4& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t u = __float_as_uint(v[i]);
    h[i] = u & 0xffff0000u;
    l[i] = __float_as_uint(v[i] - __uint_as_float(h[i]));
  }
  hi = u32x4{(h[0] >> 16) | h[1], (h[2] >> 16) | h[3], (h[4] >> 16) | h[5], (h[6] >> 16) | h[7]};
  lo = u32x4{(l[0] >> 16) | (l[1] & 0xffff0000u), (l[2] >> 16) | (l[3] & 0xffff0000u),
             (l[4] >> 16) | (l[5] & 0xffff0000u), (l[6] >> 16) | (l[7] & 0xffff0000u)};
}

// slot t of an aligned group of 8 in the within-8 permuted order holds logical offset:
__device__ __forceinline__ int perm_src(int t) { return (t & 1) ? 4 + (t >> 1) : (t >> 1); }

template <int MT, int NB, bool HALF>
__global__ __launch_bounds__(256) void k_lora_side(SideArgs a) {
  constexpr int MB = MT / 16;
  constexpr int NQ = 64 * NB;       // tile columns: four waves of NB 16-column blocks
  constexpr int kBTP = 2 * NQ + 32;  // row pitch (bytes) of the k-major weight layout
  constexpr int kBB = NQ * 64 > kSK * kBTP ? NQ * 64 : kSK * kBTP;
  constexpr int kAC = MT * 4 > 256 ? MT * 4 / 256 : 1;  // activation chunks (8 values) per thread
  __shared__ __align__(16) uint8_t Ah[2][MT * 64], Al[2][HALF ? MT * 64 : 16];
  __shared__ __align__(16) uint8_t Bh[2][kBB], Bl[2][kBB];
  __shared__ int32_t s_src[MT], s_ex[MT];

  const int tile = blockIdx.x;
  if ((unsigned long long)tile >= a.counters[kNumTiles]) return;
  const int e = a.tile_e[tile], m0 = a.tile_m0[tile];
  const int mlen = min(MT, a.offsets[e + 1] - m0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int R = a.R, kdim = a.kdim;
  if (tid < MT) {
    const int m = m0 + min(tid, mlen - 1);  // rows past the tile's end repeat its last row
    s_src[tid] = HALF ? m : a.sorted_slot[m] / a.topk;
    s_ex[tid] = HALF ? a.exps[(int64_t)m * a.exp_ld + a.exp_off] : 0;
  }
  __syncthreads();

  u32x4 areg[kAC];
  float breg[NB][8];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kAC; ++i) {
      const int q = tid + 256 * i, row = (q >> 2) & (MT - 1), c = q & 3;
      areg[i] = *reinterpret_cast<const u32x4*>(a.src + (int64_t)s_src[row] * a.ld + a.col_off + k0 + 8 * c);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = tid + 256 * i;
      if (a.rk) {  // W[e][col][k]: thread -> (column, 8 consecutive k)
        const int col = q >> 2, c = q & 3;
        const bool second = col >= R;
        const float* Wm = second ? a.W2 : a.W;
        const int qq = min(second ? col - R : col, R - 1);
        const bool ok = col < a.nq;
        const float* p = (Wm ? Wm : a.W) + ((int64_t)e * R + qq) * kdim + k0 + 8 * c;
        const float4 x0 = *reinterpret_cast<const float4*>(p), x1 = *reinterpret_cast<const float4*>(p + 4);
        const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) breg[i][t] = ok ? v[t] : 0.f;
      } else {  // W[e][k][col]: thread -> (k, 8 consecutive columns)
        const int kr = q / (NQ / 8), c8 = q % (NQ / 8);
        const float* row = a.W + ((int64_t)e * kdim + k0 + kr) * R;
        const float* row2 = a.W2 ? a.W2 + ((int64_t)e * kdim + k0 + kr) * R : row;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int col = 8 * c8 + t;
          const bool second = col >= R;
          const int qq = min(second ? col - R : col, R - 1);
          const float x = (second ? row2 : row)[qq];
          breg[i][t] = col < a.nq ? x : 0.f;
        }
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kAC; ++i) {
      const int q = tid + 256 * i;
      if (q >= MT * 4) continue;
      const int row = q >> 2, c = q & 3;
      const int off = row * 64 + 16 * (c ^ ((row >> 2) & 3));
      if constexpr (HALF) {  // fp16 -> exact bf16 hi + lo
        const u32x4 v = areg[i];
        const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          f[2 * t] = half_bits_to_float((uint16_t)(wds[t] & 0xffffu));
          f[2 * t + 1] = half_bits_to_float((uint16_t)(wds[t] >> 16));
        }
        u32x4 hi, lo;
        split8_trunc(f, hi, lo);
        *reinterpret_cast<u32x4*>(&Ah[buf][off]) = hi;
        *reinterpret_cast<u32x4*>(&Al[buf][off]) = lo;
      } else {
        *reinterpret_cast<u32x4*>(&Ah[buf][off]) = areg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int q = tid + 256 * i;
      float v[8];
      u32x4 hi, lo;
      if (a.rk) {
        const int col = q >> 2, c = q & 3;
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = breg[i][HALF ? perm_src(t) : t];  // in the activation's order
        split8_trunc(v, hi, lo);
        const int off = col * 64 + 16 * (c ^ ((col >> 2) & 3));
        *reinterpret_cast<u32x4*>(&Bh[buf][off]) = hi;
        *reinterpret_cast<u32x4*>(&Bl[buf][off]) = lo;
      } else {
        const int kr = q / (NQ / 8), c8 = q % (NQ / 8);
        const int sr = HALF ? perm_pos(kr) : kr;  // stored row in the activation's order
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = breg[i][t];
        split8_trunc(v, hi, lo);
        *reinterpret_cast<u32x4*>(&Bh[buf][sr * kBTP + 16 * c8]) = hi;
        *reinterpret_cast<u32x4*>(&Bl[buf][sr * kBTP + 16 * c8]) = lo;
      }
    }
  };

  floatx4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int cw = w * 16 * NB;  // this wave's first column
  const int asw = (lr >> 2) & 3;
  const int nsteps = kdim / kSK;
  load(0);
  store(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    if (s + 1 < nsteps) load((s + 1) * kSK);
    if (cw < a.nq) {
      u32x4 bh[NB], bl[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (a.rk) {
          const int col = cw + 16 * nb + lr;
          bh[nb] = *reinterpret_cast<const u32x4*>(&Bh[cur][col * 64 + 16 * (lg ^ ((col >> 2) & 3))]);
          bl[nb] = *reinterpret_cast<const u32x4*>(&Bl[cur][col * 64 + 16 * (lg ^ ((col >> 2) & 3))]);
        } else {
          // lanes 4r..4r+3 address row 8 lg + r (then + 4), columns 4 (lr & 3)..: each lane
          // receives 4 consecutive rows of its column per read
          const int base = (8 * lg + (lr >> 2)) * kBTP + 2 * (cw + 16 * nb + 4 * (lr & 3));
          const v4s_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(&Bh[cur][base]));
          const v4s_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(&Bh[cur][base + 4 * kBTP]));
          const v4s_t l0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(&Bl[cur][base]));
          const v4s_t l1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(&Bl[cur][base + 4 * kBTP]));
          bh[nb] = u32x4{pack2(h0.x, h0.y), pack2(h0.z, h0.w), pack2(h1.x, h1.y), pack2(h1.z, h1.w)};
          bl[nb] = u32x4{pack2(l0.x, l0.y), pack2(l0.z, l0.w), pack2(l1.x, l1.y), pack2(l1.z, l1.w)};
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int off = (16 * mb + lr) * 64 + 16 * (lg ^ asw);
        const u32x4 ah = *reinterpret_cast<const u32x4*>(&Ah[cur][off]);
        u32x4 al = {0u, 0u, 0u, 0u};
        if constexpr (HALF) al = *reinterpret_cast<const u32x4*>(&Al[cur][off]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          acc[mb][nb] = mfma_bf16(ah, bh[nb], acc[mb][nb]);
          acc[mb][nb] = mfma_bf16(ah, bl[nb], acc[mb][nb]);
          if constexpr (HALF) acc[mb][nb] = mfma_bf16(al, bh[nb], acc[mb][nb]);
        }
      }
    }
    if (s + 1 < nsteps) store(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mb + 4 * lg + i;
      if (row >= mlen) continue;
      const int64_t m = m0 + row;
      const int ex = s_ex[row];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = cw + 16 * nb + lr;
        if (col >= a.nq) continue;
        const float v = HALF ? ldexpf(acc[mb][nb][i], -ex) : acc[mb][nb][i];
        if (col < R)
          a.out[m * R + col] = v;
        else
          a.out2[m * R + (col - R)] = v;
        uint16_t hi, lo;
        split_bf16(v * a.split_scale, hi, lo);
        const int64_t sc = col < R ? a.split_off + col : a.split_off2 + (col - R);
        a.split[m * 2 * a.split_ld + sc] = hi;
        a.split[m * 2 * a.split_ld + a.split_ld + sc] = lo;
      }
    }
}

template <int MT, int NB>
static void launch_side_nb(bool half, unsigned grid, const SideArgs& a, hipStream_t st) {
  if (half)
    k_lora_side<MT, NB, true><<<grid, 256, 0, st>>>(a);
  else
    k_lora_side<MT, NB, false><<<grid, 256, 0, st>>>(a);
}

template <int MT>
static void launch_side_mt(int nb, bool half, unsigned grid, const SideArgs& a, hipStream_t st) {
  if (nb <= 1)
    launch_side_nb<MT, 1>(half, grid, a, st);
  else if (nb == 2)
    launch_side_nb<MT, 2>(half, grid, a, st);
  else
    launch_side_nb<MT, 4>(half, grid, a, st);
}

void launch_lora_rowproj(const Dims& d, const WsMap& w, void* ws, const RowView& src, int64_t kdim, const float* W,
                         const float* W2, bool rk, float* out, float* out2, int64_t split_ld, int64_t split_off,
                         int64_t split_off2, hipStream_t st) {
  if (w.max_tiles == 0) return;
  SideArgs a{};
  a.topk = (int)d.K;
  a.sorted_slot = ws_ptr<int32_t>(ws, w.sorted_slot);
  a.offsets = ws_ptr<int32_t>(ws, w.offsets);
  a.tile_e = ws_ptr<int32_t>(ws, w.tile_e);
  a.tile_m0 = ws_ptr<int32_t>(ws, w.tile_m0);
  a.counters = ws_ptr<unsigned long long>(ws, w.counters);
  a.src = static_cast<const uint16_t*>(src.ptr);
  a.ld = src.ld;
  a.col_off = src.col_off;
  a.exps = src.exps;
  a.exp_ld = src.exp_ld;
  a.exp_off = src.exp_off;
  a.W = W;
  a.W2 = W2;
  a.rk = rk ? 1 : 0;
  a.kdim = (int)kdim;
  a.R = (int)d.R;
  a.nq = (int)(W2 ? 2 * d.R : d.R);
  a.out = out;
  a.out2 = out2;
  a.split = ws_ptr<uint16_t>(ws, w.lsplit);
  a.split_ld = split_ld;
  a.split_off = split_off;
  a.split_off2 = split_off2;
  a.split_scale = d.sc;
  const bool half = src.kind == kSrcHalfChunked;
  const int nb = (a.nq + 63) / 64;
  const unsigned grid = (unsigned)w.max_tiles;
  switch (w.mt) {
    case 16:
      launch_side_mt<16>(nb, half, grid, a, st);
      break;
    case 32:
      launch_side_mt<32>(nb, half, grid, a, st);
      break;
    case 64:
      launch_side_mt<64>(nb, half, grid, a, st);
      break;
    default:
      launch_side_mt<128>(nb, half, grid, a, st);
      break;
  }
}

void launch_lora_grad(const Dims& d, const WsMap& w, void* ws, const RowView& P, int64_t np, const RowView& Q,
                      int64_t nq, float* G, int accumulate, float scale, hipStream_t st) {
  LoraArgs a{};
  a.topk = (int)d.K;
  a.sorted_slot = ws_ptr<int32_t>(ws, w.sorted_slot);
  a.offsets = ws_ptr<int32_t>(ws, w.offsets);
  a.P = P;
  a.Q = Q;
  a.np_ = np;
  a.nq_ = nq;
  a.G = G;
  a.accumulate = accumulate;
  a.scale = scale;
  dim3 grid((unsigned)d.E, (unsigned)((np + kLT - 1) / kLT), (unsigned)((nq + kLT - 1) / kLT));
  k_lora_grad<<<grid, 256, 0, st>>>(a);
}

}  // namespace kt
