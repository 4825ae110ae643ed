// LoRA side products and LoRA gradient reductions on bf16 MFMA.
//
// Both are small grouped matrix products of the page "rawint4_sft_reference.py"
// (_lora_linear inside routed_rawint4_lora, and its gradients):
//   side products   out[m, q] = sum_k a(m, k) W(q, k)   (x A^T, h A_d^T, dY B_d, dG B_g, dU B_u)
//   gradients       G[e, p, q] = sum over the expert's rows m of P(m, p) Q(m, q)
// Operands arrive in fp32, bf16 or fp16-with-exponent form; every value is
// widened to fp32 and split into bf16 hi + lo (~16 significant bits) while it
// is staged in LDS, and each fragment pair takes three bf16 MFMAs
// (hi*hi + hi*lo + lo*hi); exactly-bf16 activations (x, dY) have no lo part and
// take two.  A workgroup owns a 64 x 64 output tile and walks the contraction 32
// at a time in a fixed order, so results do not depend on scheduling.
//
// Side products stage both operands contraction-contiguous ([row][k]) with
// 16-byte loads.  Gradients contract over token rows, so both operands are
// staged row-major ([k][column]) and read back with ds_read_tr16_b64, which
// hands each lane 4 consecutive rows of one column.
#include "kt_common.hpp"
#include "kt_internal.hpp"

namespace kt {

constexpr int kLT = 64;       // output tile edge
constexpr int kLK = 32;       // contraction step
constexpr int kLP = kLK + 8;  // [row][k] pitch in 16-bit elements (80 B)
constexpr int kLQ = kLT + 8;  // [k][column] pitch in 16-bit elements (144 B)

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t* lds_v4s_ptr;

struct LoraArgs {
  int mode;  // 0: side product, 1: gradient
  int topk, R;
  const int32_t* sorted_slot;
  const int32_t* offsets;
  const int32_t* tile_e;
  const int32_t* tile_m0;
  const unsigned long long* counters;
  // side product: rows of `src`; weights W ([E, nq, kdim] if rk else [E, kdim, nq]);
  // with W2 set, output columns [nq, 2 nq) use W2 and go to out2
  RowView src;
  const float* W;
  const float* W2;
  int rk;
  int64_t kdim, nq;
  float* out;
  float* out2;
  // the product times split_scale as bf16 hi and lo planes, [rows][2][split_ld]
  // (column j < nq: hi at split_off + j, lo at split_ld + split_off + j; the W2
  // half's column j at split_off2 + j)
  uint16_t* split;
  int64_t split_ld, split_off, split_off2;
  float split_scale;
  // gradient: P(m, p), Q(m, q) over the expert's rows; G[e, p, q]
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

__global__ __launch_bounds__(256) void k_lora_mfma(LoraArgs a) {
  __shared__ __align__(16) uint16_t Ah[kLT * kLQ], Al[kLT * kLQ], Bh[kLT * kLQ], Bl[kLT * kLQ];
  __shared__ int32_t s_row[kLT];  // token (bf16 rows) or sorted row index per tile row
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  floatx4 acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (a.mode == 0) {
    // ------------------------------------------------------------ side product
    const int tile = blockIdx.x;
    if ((unsigned long long)tile >= a.counters[kNumTilesAux]) return;
    const int e = a.tile_e[tile], m0 = a.tile_m0[tile];
    const int rows = min(kLT, a.offsets[e + 1] - m0);
    const int64_t j0 = (int64_t)blockIdx.y * kLT;
    const int64_t ncols = a.W2 ? 2 * a.nq : a.nq;
    const bool exact = a.src.kind == kSrcTokBf16 && a.src.slot_scale == nullptr;
    const bool permuted = a.src.kind == kSrcHalfChunked;
    if (tid < kLT) s_row[tid] = tid < rows ? (a.src.kind == kSrcTokBf16 ? a.sorted_slot[m0 + tid] / a.topk : m0 + tid) : -1;
    __syncthreads();
    for (int64_t k0 = 0; k0 < a.kdim; k0 += kLK) {
      {  // activations: thread -> (row, 8 features)
        const int i = tid >> 2, c = 8 * (tid & 3);
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const int r = s_row[i];
        if (r >= 0 && k0 + c < a.kdim) load8(a.src, m0 + i, k0 + c, r, 8, v);
        if (a.src.slot_scale && r >= 0) {
          const float sv = a.src.slot_scale[a.sorted_slot[m0 + i]];
#pragma unroll
          for (int t = 0; t < 8; ++t) v[t] *= sv;
        }
        u32x4 hi, lo;
        split8(v, hi, lo);
        __builtin_memcpy(&Ah[i * kLP + c], &hi, 16);
        if (!exact) __builtin_memcpy(&Al[i * kLP + c], &lo, 16);
      }
      {  // weights: thread -> (output column, 8 features), in the activation's order
        const int j = tid >> 2, c = 8 * (tid & 3);
        const int64_t col = j0 + j;
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (col < ncols && k0 + c < a.kdim) {
          const bool second = col >= a.nq;
          const float* W = second ? a.W2 : a.W;
          const int64_t q = second ? col - a.nq : col;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            // logical feature of stored slot t
            const int64_t kk = k0 + c + (permuted ? ((t & 1) ? 4 + (t >> 1) : (t >> 1)) : t);
            v[t] = a.rk ? W[((int64_t)e * a.nq + q) * a.kdim + kk] : W[((int64_t)e * a.kdim + kk) * a.nq + q];
          }
        }
        u32x4 hi, lo;
        split8(v, hi, lo);
        __builtin_memcpy(&Bh[j * kLP + c], &hi, 16);
        __builtin_memcpy(&Bl[j * kLP + c], &lo, 16);
      }
      __syncthreads();
      const int aoff = (w * 16 + lr) * kLP + 8 * lg;
      u32x4 ah, al = {0u, 0u, 0u, 0u};
      __builtin_memcpy(&ah, &Ah[aoff], 16);
      if (!exact) __builtin_memcpy(&al, &Al[aoff], 16);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int boff = (f * 16 + lr) * kLP + 8 * lg;
        u32x4 bh, bl;
        __builtin_memcpy(&bh, &Bh[boff], 16);
        __builtin_memcpy(&bl, &Bl[boff], 16);
        acc[f] = mfma_bf16(ah, bh, acc[f]);
        acc[f] = mfma_bf16(ah, bl, acc[f]);
        if (!exact) acc[f] = mfma_bf16(al, bh, acc[f]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = w * 16 + lg * 4 + t;
        const int64_t j = j0 + f * 16 + lr;
        if (i >= rows || j >= ncols) continue;
        const int64_t m = m0 + i;
        uint16_t hi, lo;
        split_bf16(acc[f][t] * a.split_scale, hi, lo);
        const int64_t sc = j < a.nq ? a.split_off + j : a.split_off2 + (j - a.nq);
        a.split[m * 2 * a.split_ld + sc] = hi;
        a.split[m * 2 * a.split_ld + a.split_ld + sc] = lo;
        if (j < a.nq)
          a.out[m * a.nq + j] = acc[f][t];
        else
          a.out2[m * a.nq + (j - a.nq)] = acc[f][t];
      }
    return;
  }

  // ------------------------------------------------------------ gradient
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

static LoraArgs base_args(const Dims& d, const WsMap& w, void* ws) {
  LoraArgs a{};
  a.topk = (int)d.K;
  a.R = (int)d.R;
  a.sorted_slot = ws_ptr<int32_t>(ws, w.sorted_slot);
  a.offsets = ws_ptr<int32_t>(ws, w.offsets);
  a.tile_e = ws_ptr<int32_t>(ws, w.tile_e_aux);
  a.tile_m0 = ws_ptr<int32_t>(ws, w.tile_m0_aux);
  a.counters = ws_ptr<unsigned long long>(ws, w.counters);
  return a;
}

void launch_lora_rowproj(const Dims& d, const WsMap& w, void* ws, const RowView& src, int64_t kdim, const float* W,
                         const float* W2, bool rk, float* out, float* out2, int64_t split_ld, int64_t split_off,
                         int64_t split_off2, hipStream_t st) {
  if (w.max_tiles_aux == 0) return;
  LoraArgs a = base_args(d, w, ws);
  a.split = ws_ptr<uint16_t>(ws, w.lsplit);
  a.split_ld = split_ld;
  a.split_off = split_off;
  a.split_off2 = split_off2;
  a.split_scale = d.sc;
  a.mode = 0;
  a.src = src;
  a.W = W;
  a.W2 = W2;
  a.rk = rk ? 1 : 0;
  a.kdim = kdim;
  a.nq = d.R;
  a.out = out;
  a.out2 = out2;
  const int64_t ncols = W2 ? 2 * d.R : d.R;
  dim3 grid((unsigned)w.max_tiles_aux, (unsigned)((ncols + kLT - 1) / kLT));
  k_lora_mfma<<<grid, 256, 0, st>>>(a);
}

void launch_lora_grad(const Dims& d, const WsMap& w, void* ws, const RowView& P, int64_t np, const RowView& Q,
                      int64_t nq, float* G, int accumulate, float scale, hipStream_t st) {
  LoraArgs a = base_args(d, w, ws);
  a.mode = 1;
  a.P = P;
  a.Q = Q;
  a.np_ = np;
  a.nq_ = nq;
  a.G = G;
  a.accumulate = accumulate;
  a.scale = scale;
  dim3 grid((unsigned)d.E, (unsigned)((np + kLT - 1) / kLT), (unsigned)((nq + kLT - 1) / kLT));
  k_lora_mfma<<<grid, 256, 0, st>>>(a);
}

}  // namespace kt
