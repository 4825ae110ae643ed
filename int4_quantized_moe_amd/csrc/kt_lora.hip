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

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t* lds_v4s_ptr;

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

// Gradient tile: 64 columns of the rank-wide operand (LoRA-A/B side product,
// fp32) by 256 columns of the wide one (x, dY, h, dG, dU); both staged
// row-major in LDS ([token row][column], hi and lo planes).
constexpr int kGU = 64;            // narrow-operand columns per tile
constexpr int kGV = 256;           // wide-operand columns per tile
constexpr int kGK = 32;            // token rows per step
constexpr int kUP = 2 * kGU + 16;  // LDS row pitch in bytes, narrow operand
constexpr int kVP = 2 * kGV + 32;  // LDS row pitch in bytes, wide operand

// 8 values of a view at row m from column c, in logical column order, times the
// slot scale; zeros for an invalid row or past the last column
__device__ __forceinline__ void load_logical8(const RowView& v, int64_t m, int64_t c, int32_t slot, int topk,
                                              bool valid, int64_t ncols, float* out) {
  float t[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (valid && c < ncols) {
    load8(v, m, c, v.kind == kSrcTokBf16 ? slot / topk : (int32_t)m, (int)min<int64_t>(8, ncols - c), t);
    if (v.slot_scale) {
      const float sv = v.slot_scale[slot];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] *= sv;
    }
  }
  // fp16 views keep the within-8 permuted column order: logical offset i sits at perm_pos(i)
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = v.kind == kSrcHalfChunked ? t[(i & 4) ? 2 * (i & 3) + 1 : 2 * i] : t[i];
}

// G[e, p, q] = (accumulate ? G : 0) + scale * sum_m P(m, p) Q(m, q).  The narrow
// operand U is P (TRANS = false) or Q (TRANS = true); with TRANS the MFMA
// operands are swapped so that the tile comes out transposed and the stores
// run along q either way.
template <bool TRANS>
__global__ __launch_bounds__(256) void k_lora_grad(LoraArgs a) {
  __shared__ __align__(16) uint8_t Uh[kGK * kUP], Ul[kGK * kUP], Vh[kGK * kVP], Vl[kGK * kVP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const RowView& U = TRANS ? a.Q : a.P;
  const RowView& V = TRANS ? a.P : a.Q;
  const int64_t nu = TRANS ? a.nq_ : a.np_, nv = TRANS ? a.np_ : a.nq_;
  const int e = blockIdx.x;
  const int m0 = a.offsets[e];
  const int rows = a.offsets[e + 1] - m0;
  if (rows == 0 && a.accumulate) return;
  const int64_t u0 = (int64_t)blockIdx.y * kGU, v0 = (int64_t)blockIdx.z * kGV;

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  float ureg[8], vreg[4][8];
  auto load = [&](int k0) {
    {
      const int r = tid >> 3, c = 8 * (tid & 7);
      const int64_t m = m0 + min(k0 + r, rows - 1);
      load_logical8(U, m, u0 + c, a.sorted_slot[m], a.topk, k0 + r < rows, nu, ureg);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, r = q >> 5, c = 8 * (q & 31);
      const int64_t m = m0 + min(k0 + r, rows - 1);
      load_logical8(V, m, v0 + c, a.sorted_slot[m], a.topk, k0 + r < rows, nv, vreg[i]);
    }
  };
  auto store = [&]() {
    u32x4 hi, lo;
    {
      const int r = tid >> 3, c = 8 * (tid & 7);
      split8_trunc(ureg, hi, lo);
      *reinterpret_cast<u32x4*>(&Uh[r * kUP + 2 * c]) = hi;
      *reinterpret_cast<u32x4*>(&Ul[r * kUP + 2 * c]) = lo;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, r = q >> 5, c = 8 * (q & 31);
      split8_trunc(vreg[i], hi, lo);
      *reinterpret_cast<u32x4*>(&Vh[r * kVP + 2 * c]) = hi;
      *reinterpret_cast<u32x4*>(&Vl[r * kVP + 2 * c]) = lo;
    }
  };
  // lanes 4r..4r+3 of a 16-lane group address token row 8 lg + r (then + 4), columns 4 (lr & 3)..:
  // each lane receives 4 consecutive token rows of its column per read
  auto frag = [&](const uint8_t* plane, int pitch, int col) -> u32x4 {
    const int base = (8 * lg + (lr >> 2)) * pitch + 2 * (col + 4 * (lr & 3));
    const v4s_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(plane + base));
    const v4s_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(plane + base + 4 * pitch));
    return u32x4{pack2(x0.x, x0.y), pack2(x0.z, x0.w), pack2(x1.x, x1.y), pack2(x1.z, x1.w)};
  };

  if (rows > 0) load(0);
  for (int k0 = 0; k0 < rows; k0 += kGK) {
    store();
    __syncthreads();
    if (k0 + kGK < rows) load(k0 + kGK);  // in flight while this step is multiplied
    u32x4 uh[4], ul[4];
#pragma unroll
    for (int ub = 0; ub < 4; ++ub) {
      uh[ub] = frag(Uh, kUP, 16 * ub);
      ul[ub] = frag(Ul, kUP, 16 * ub);
    }
#pragma unroll
    for (int vb = 0; vb < 4; ++vb) {
      const u32x4 vh = frag(Vh, kVP, 64 * w + 16 * vb);
      const u32x4 vl = frag(Vl, kVP, 64 * w + 16 * vb);
#pragma unroll
      for (int ub = 0; ub < 4; ++ub) {
        if constexpr (TRANS) {
          acc[ub][vb] = mfma_bf16(vh, uh[ub], acc[ub][vb]);
          acc[ub][vb] = mfma_bf16(vh, ul[ub], acc[ub][vb]);
          acc[ub][vb] = mfma_bf16(vl, uh[ub], acc[ub][vb]);
        } else {
          acc[ub][vb] = mfma_bf16(uh[ub], vh, acc[ub][vb]);
          acc[ub][vb] = mfma_bf16(uh[ub], vl, acc[ub][vb]);
          acc[ub][vb] = mfma_bf16(ul[ub], vh, acc[ub][vb]);
        }
      }
    }
    __syncthreads();  // every wave is done with this step before the next store
  }

#pragma unroll
  for (int ub = 0; ub < 4; ++ub)
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int64_t p, q;
        if constexpr (TRANS) {  // tile rows run along the wide operand (p), columns along q
          p = v0 + 64 * w + 16 * vb + 4 * lg + i;
          q = u0 + 16 * ub + lr;
        } else {
          p = u0 + 16 * ub + 4 * lg + i;
          q = v0 + 64 * w + 16 * vb + lr;
        }
        if (p >= a.np_ || q >= a.nq_) continue;
        const int64_t idx = ((int64_t)e * a.np_ + p) * a.nq_ + q;
        const float prev = a.accumulate ? a.G[idx] : 0.f;
        a.G[idx] = prev + a.scale * acc[ub][vb][i];
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
        const int col0 = 8 * c8;
        const bool second0 = col0 >= R;
        const int cc = second0 ? col0 - R : col0;
        if ((R & 3) == 0 && cc + 8 <= R && col0 + 8 <= a.nq) {  // 8 columns inside one matrix, 16-byte aligned
          const float* p = (second0 ? row2 : row) + cc;
          const float4 x0 = *reinterpret_cast<const float4*>(p), x1 = *reinterpret_cast<const float4*>(p + 4);
          breg[i][0] = x0.x, breg[i][1] = x0.y, breg[i][2] = x0.z, breg[i][3] = x0.w;
          breg[i][4] = x1.x, breg[i][5] = x1.y, breg[i][6] = x1.z, breg[i][7] = x1.w;
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int col = col0 + t;
            const bool second = col >= R;
            const int qq = min(second ? col - R : col, R - 1);
            const float x = (second ? row2 : row)[qq];
            breg[i][t] = col < a.nq ? x : 0.f;
          }
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
  // the rank-wide operand is the narrow one
  const bool trans = nq < np;
  const int64_t nu = trans ? nq : np, nv = trans ? np : nq;
  dim3 grid((unsigned)d.E, (unsigned)((nu + kGU - 1) / kGU), (unsigned)((nv + kGV - 1) / kGV));
  if (trans)
    k_lora_grad<true><<<grid, 256, 0, st>>>(a);
  else
    k_lora_grad<false><<<grid, 256, 0, st>>>(a);
}

}  // namespace kt
