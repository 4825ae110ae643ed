// Grouped matrix kernels of the routed layer on gfx950 MFMA.
//
// One template serves the four expert GEMMs of the page "rawint4_sft_reference.py"
// (routed_rawint4_lora and the autograd of run_routed_reference):
//   kGateUp    g, u = x W_g^T, x W_u^T (+ LoRA), then the clamped SwiGLU (rawint4_swiglu)
//   kDown      y = h W_d^T (+ LoRA), times the route weight, into per-slot staging
//   kDownBwd   g_h = dY W_d (+ LoRA), then dRoute = <g_h, h> partials and the
//              SwiGLU/clamp gradient dG, dU
//   kGateUpBwd dx = dG W_g + dU W_u (+ LoRA), into per-slot staging
//
// A work tile is MT token-slot rows of one expert (rows sorted by the grouping)
// by kNT = 256 output columns; the four waves of a workgroup split the columns
// (64 each) and share the activation tile, which is staged in LDS 64 contraction
// values at a time, double buffered.
//
// Weights are decoded on the fly into exact fp16 ((c - 8) * scale fits fp16's
// 11-bit significand) and multiplied on v_mfma_f32_16x16x32_f16 with fp32
// accumulation.  In the stored orientation (kGateUp, kDown: contraction along
// the packed K) every lane loads its 16 nibbles straight into registers.  The
// two gradient GEMMs contract over the weight rows: the raw packed rows are
// copied into LDS as they are and read back with ds_read_tr4_b64, which hands
// each lane 16 consecutive rows of one column; this is the transpose-free dX of
// transpose_free_rawint4_dx with the transpose done by the LDS read.
//
// Activations carry a power-of-two exponent per row (x, dY) or per (row, column
// chunk) (h, dG, dU) so that fp16's range never clips them; chunk exponents are
// brought to the row's smallest exponent while the tile is staged, and the
// epilogue removes it.  LoRA terms ride along as extra K-steps: the fp32 LoRA-A
// side products and the fp32 LoRA matrices are split into bf16 hi + lo and
// multiplied with three bf16 MFMAs (hi*hi + hi*lo + lo*hi).
#include <limits.h>

#include "kt_common.hpp"
#include "kt_internal.hpp"

namespace kt {

constexpr int kKS = 64;       // contraction values per super-step (two quant groups)
constexpr int kAP = kKS + 8;  // activation tile pitch in 16-bit elements (144 B)
constexpr int kWP = 144;      // raw weight tile pitch in bytes (128 B of codes for 256 columns)

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t* lds_v2i_ptr;

struct GemmParams {
  int E, topk, H, I, R;
  float sc, limit;
  const int32_t* sorted_slot;
  const int32_t* offsets;
  const int32_t* tile_e;
  const int32_t* tile_m0;
  const unsigned long long* counters;
  LayerPtrs L;
  const uint16_t* a_src;      // fp16 activation rows (within-8 permuted order)
  const int32_t* a_rowexp;    // per token exponent (x, dY)
  const int32_t* a_chunkexp;  // per (row, chunk) exponent (h, dG|dU)
  int a_nch, a_chunkw;
  int64_t lda;
  const float* la0;  // LoRA-A side products per sorted row, [Ms, R]
  const float* la1;
  const float* rw;  // route weights per flat slot
  float* gsave;
  float* usave;
  uint16_t* hh;
  int32_t* hexp;
  int h_nch;
  float* stage;
  uint16_t* dgu;
  int32_t* dguexp;
  int dg_nch;
  float* drpart;
  int dr_nt;
  unsigned long long* bad_scales;
  int n_ntiles;
};

// local column (0..255 within the tile) of N-block f of wave w
template <int KIND>
__device__ __forceinline__ int local_col(int w, int f) {
  if constexpr (KIND == kGateUp) return f < 2 ? w * 32 + f * 16 : kHChunk + w * 32 + (f - 2) * 16;
  return w * 64 + f * 16;
}

__device__ __forceinline__ uint32_t mul_half2(uint32_t v, half2_t s) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v) * s);
}

__device__ __forceinline__ u32x4 pack_bf16x8(const uint16_t* v) {
  u32x4 r;
  r.x = v[0] | ((uint32_t)v[1] << 16);
  r.y = v[2] | ((uint32_t)v[3] << 16);
  r.z = v[4] | ((uint32_t)v[5] << 16);
  r.w = v[6] | ((uint32_t)v[7] << 16);
  return r;
}

// SwiGLU with the boundary-inclusive clamp; masks are 1 where the gradient passes
__device__ __forceinline__ void clamp_swiglu(float g, float u, float limit, float& gp, float& up, float& mg,
                                             float& mu) {
  gp = g;
  up = u;
  mg = 1.f;
  mu = 1.f;
  if (limit > 0.f) {
    if (!(g <= limit)) {
      gp = limit;
      mg = 0.f;
    }
    if (u < -limit) {
      up = -limit;
      mu = 0.f;
    } else if (u > limit) {
      up = limit;
      mu = 0.f;
    }
  }
}

template <int KIND, int MT>
__global__ __launch_bounds__(256) void k_gemm(GemmParams p) {
  constexpr int MB = MT / 16;
  constexpr bool kT = (KIND == kDownBwd || KIND == kGateUpBwd);
  constexpr bool kChunked = (KIND == kDown || KIND == kGateUpBwd);
  constexpr int kAChunks = (MT * 8 + 255) / 256;  // 16-byte activation pieces per thread per super-step
  __shared__ __align__(16) uint16_t As[2][MT * kAP];
  __shared__ __align__(16) uint8_t Wl[kT ? 2 : 1][kT ? kKS * kWP : 16];
  __shared__ __align__(16) uint16_t Sc[kT ? 2 : 1][kT ? (kNT / 32) * kKS : 8];
  __shared__ int32_t s_src[MT], s_exp[MT], s_slot[MT];

  const int tile = (int)(blockIdx.x / (unsigned)p.n_ntiles);
  const int nt = (int)(blockIdx.x % (unsigned)p.n_ntiles);
  if ((unsigned long long)tile >= p.counters[kNumTiles]) return;
  const int e = p.tile_e[tile], m0 = p.tile_m0[tile];
  const int mlen = min(MT, p.offsets[e + 1] - m0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int H = p.H, I = p.I, R = p.R;
  const int n0 = (KIND == kGateUp) ? nt * kHChunk : nt * kNT;
  const int nout = (KIND == kGateUp || KIND == kDownBwd) ? I : H;
  const int kdim = (KIND == kGateUp || KIND == kDownBwd) ? H : (KIND == kDown ? I : 2 * I);
  const int nss = (kdim + kKS - 1) / kKS;

  if (tid < MT) {
    int src = -1, ex = 0, slot = -1;
    if (tid < mlen) {
      const int m = m0 + tid;
      slot = p.sorted_slot[m];
      if constexpr (kChunked) {
        src = m;
        int mn = INT_MAX;
        for (int c = 0; c < p.a_nch; ++c) mn = min(mn, p.a_chunkexp[(size_t)m * p.a_nch + c]);
        ex = mn;
      } else {
        src = slot / p.topk;
        ex = p.a_rowexp[src];
      }
    }
    s_src[tid] = src;
    s_exp[tid] = ex;
    s_slot[tid] = slot;
  }
  __syncthreads();

  floatx4 acc[MB][4];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  // ---------------------------------------------------------------- staging helpers
  u32x4 areg[kAChunks];
  auto load_a = [&](int k0) {
#pragma unroll
    for (int t = 0; t < kAChunks; ++t) {
      const int q = tid + 256 * t;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (q < MT * 8) {
        const int row = q >> 3, k = k0 + 8 * (q & 7);
        const int src = s_src[row];
        if (src >= 0 && k < kdim) {
          v = *reinterpret_cast<const u32x4*>(p.a_src + (size_t)src * p.lda + k);
          if constexpr (kChunked) {
            int c;
            if constexpr (KIND == kDown)
              c = k / p.a_chunkw;
            else
              c = k < I ? k / p.a_chunkw : p.a_nch / 2 + (k - I) / p.a_chunkw;
            const int d = s_exp[row] - p.a_chunkexp[(size_t)src * p.a_nch + c];
            if (d != 0) {
              const uint16_t sb = half_pow2_bits(d);
              const half2_t s2 = __builtin_bit_cast(half2_t, (uint32_t)sb | ((uint32_t)sb << 16));
              v.x = mul_half2(v.x, s2);
              v.y = mul_half2(v.y, s2);
              v.z = mul_half2(v.z, s2);
              v.w = mul_half2(v.w, s2);
            }
          }
        }
      }
      areg[t] = v;
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int t = 0; t < kAChunks; ++t) {
      const int q = tid + 256 * t;
      if (q < MT * 8) *reinterpret_cast<u32x4*>(&As[buf][(q >> 3) * kAP + 8 * (q & 7)]) = areg[t];
    }
  };

  // stored orientation: each lane's 16 nibbles of its output column for one super-step
  uint32_t breg[4][2];
  uint32_t bscale[4];  // fp16 scale in both halves
  auto load_b = [&](int k0, uint32_t (&bw)[4][2], uint32_t (&bs)[4]) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint8_t* W;
      const uint16_t* S;
      size_t row;
      int rk;
      bool valid;
      if constexpr (KIND == kGateUp) {
        const int col = n0 + w * 32 + (f & 1) * 16 + lr;
        valid = col < I;
        W = f < 2 ? p.L.wg : p.L.wu;
        S = f < 2 ? p.L.sg : p.L.su;
        row = (size_t)e * I + col;
        rk = H;
      } else {
        const int col = n0 + w * 64 + f * 16 + lr;
        valid = col < H;
        W = p.L.wd;
        S = p.L.sd;
        row = (size_t)e * H + col;
        rk = I;
      }
      const int k = k0 + 16 * lg;
      uint2 v = make_uint2(0u, 0u);
      uint32_t sh = 0u;
      if (valid && k < kdim) {
        v = *reinterpret_cast<const uint2*>(W + row * (size_t)(rk / 2) + k / 2);
        const float sf = bf16_to_float(S[row * (size_t)(rk / kGroup) + k / kGroup]);
        if (!scale_in_domain(sf) && (lg & 1) == 0) atomicAdd(p.bad_scales, 1ull);
        sh = float_to_half_bits(sf);
      }
      bw[f][0] = v.x;
      bw[f][1] = v.y;
      bs[f] = sh | (sh << 16);
    }
  };

  // contraction over weight rows: raw packed rows and their scales into LDS
  u32x4 wreg[2];
  uint16_t sreg[2];
  auto load_w = [&](int k0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int q = tid + 256 * t;
      const int row = q >> 3, c16 = q & 7;
      const int kk = k0 + row, c = n0 + 32 * c16;
      u32x4 v = {0u, 0u, 0u, 0u};
      uint16_t sh = 0;
      if (kk < kdim && c < nout) {
        const uint8_t* W;
        const uint16_t* S;
        size_t wrow;
        int rk;
        if constexpr (KIND == kDownBwd) {
          W = p.L.wd;
          S = p.L.sd;
          wrow = (size_t)e * H + kk;
          rk = I;
        } else {
          const bool up = kk >= I;
          W = up ? p.L.wu : p.L.wg;
          S = up ? p.L.su : p.L.sg;
          wrow = (size_t)e * I + (up ? kk - I : kk);
          rk = H;
        }
        v = *reinterpret_cast<const u32x4*>(W + wrow * (size_t)(rk / 2) + c / 2);
        const float sf = bf16_to_float(S[wrow * (size_t)(rk / kGroup) + c / kGroup]);
        if (!scale_in_domain(sf)) atomicAdd(p.bad_scales, 1ull);
        sh = float_to_half_bits(sf);
      }
      wreg[t] = v;
      sreg[t] = sh;
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int q = tid + 256 * t;
      const int row = q >> 3, c16 = q & 7;
      *reinterpret_cast<u32x4*>(&Wl[buf][row * kWP + 16 * c16]) = wreg[t];
      Sc[buf][c16 * kKS + perm_pos(row)] = sreg[t];
    }
  };

  auto compute = [&](int cur) {
    if constexpr (kT) {
      v2i_t tr[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int lc = local_col<KIND>(w, f);
        tr[f] = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_v2i_ptr)(&Wl[cur][(16 * lg + lr) * kWP + lc / 2]));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4 af[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          af[mb] = *reinterpret_cast<const u32x4*>(&As[cur][(mb * 16 + lr) * kAP + 16 * lg + 8 * j]);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int cg = local_col<KIND>(w, f) / 32;
          u32x4 sp;  // 8 fp16 scales written as 16-bit values: copy, do not type-pun
          __builtin_memcpy(&sp, &Sc[cur][cg * kKS + 16 * lg + 8 * j], sizeof(sp));
          const uint32_t word = j ? (uint32_t)tr[f].y : (uint32_t)tr[f].x;
          // bit-cast whole scalars: clang's bit_cast of an ext-vector component reads component 0
          const uint32_t s0 = sp.x, s1 = sp.y, s2 = sp.z, s3 = sp.w;
          const u32x4 bf = decode_dword_perm(word, __builtin_bit_cast(half2_t, s0), __builtin_bit_cast(half2_t, s1),
                                             __builtin_bit_cast(half2_t, s2), __builtin_bit_cast(half2_t, s3));
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb][f] = mfma_f16(af[mb], bf, acc[mb][f]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4 af[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          af[mb] = *reinterpret_cast<const u32x4*>(&As[cur][(mb * 16 + lr) * kAP + 16 * lg + 8 * j]);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const half2_t s2 = __builtin_bit_cast(half2_t, bscale[f]);
          const u32x4 bf = decode_dword_perm(breg[f][j], s2, s2, s2, s2);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb][f] = mfma_f16(af[mb], bf, acc[mb][f]);
        }
      }
    }
  };

  // ---------------------------------------------------------------- main loop (fp16)
  load_a(0);
  if constexpr (kT) {
    load_w(0);
    store_w(0);
  } else {
    load_b(0, breg, bscale);
  }
  store_a(0);
  __syncthreads();
  for (int ss = 0; ss < nss; ++ss) {
    const int cur = ss & 1;
    const bool more = ss + 1 < nss;
    uint32_t bnext[4][2];
    uint32_t snext[4];
    if (more) {
      load_a((ss + 1) * kKS);
      if constexpr (kT)
        load_w((ss + 1) * kKS);
      else
        load_b((ss + 1) * kKS, bnext, snext);
    }
    compute(cur);
    if (more) {
      store_a(cur ^ 1);
      if constexpr (kT) {
        store_w(cur ^ 1);
      } else {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          breg[f][0] = bnext[f][0];
          breg[f][1] = bnext[f][1];
          bscale[f] = snext[f];
        }
      }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- LoRA K-steps (bf16 hi/lo)
  const int KL = (KIND == kGateUp || KIND == kGateUpBwd) ? 2 * R : R;
  for (int q0 = 0; q0 < KL; q0 += kGroup) {
    u32x4 ah[MB], al[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = mb * 16 + lr;
      const float coef = ldexpf(p.sc, s_exp[row]);
      uint16_t hi[8], lo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = q0 + 8 * lg + i;
        float v = 0.f;
        if (row < mlen && q < KL) {
          const size_t m = (size_t)(m0 + row);
          if constexpr (KIND == kGateUp || KIND == kGateUpBwd)
            v = q < R ? p.la0[m * R + q] : p.la1[m * R + (q - R)];
          else
            v = p.la0[m * R + q];
          v *= coef;
        }
        split_bf16(v, hi[i], lo[i]);
      }
      ah[mb] = pack_bf16x8(hi);
      al[mb] = pack_bf16x8(lo);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      uint16_t hi[8], lo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = q0 + 8 * lg + i;
        float v = 0.f;
        if constexpr (KIND == kGateUp) {
          const int n = n0 + w * 32 + (f & 1) * 16 + lr;
          if (n < I) {
            if (f < 2 && q < R) v = p.L.bg[((size_t)e * I + n) * R + q];
            if (f >= 2 && q >= R && q < 2 * R) v = p.L.bu[((size_t)e * I + n) * R + (q - R)];
          }
        } else if constexpr (KIND == kDown) {
          const int n = n0 + w * 64 + f * 16 + lr;
          if (n < H && q < R) v = p.L.bd[((size_t)e * H + n) * R + q];
        } else if constexpr (KIND == kDownBwd) {
          const int c = n0 + w * 64 + f * 16 + lr;
          if (c < I && q < R) v = p.L.ad[((size_t)e * R + q) * I + c];
        } else {
          const int c = n0 + w * 64 + f * 16 + lr;
          if (c < H) {
            if (q < R)
              v = p.L.ag[((size_t)e * R + q) * H + c];
            else if (q < 2 * R)
              v = p.L.au[((size_t)e * R + (q - R)) * H + c];
          }
        }
        split_bf16(v, hi[i], lo[i]);
      }
      const u32x4 bh = pack_bf16x8(hi), bl = pack_bf16x8(lo);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        acc[mb][f] = mfma_bf16(ah[mb], bh, acc[mb][f]);
        acc[mb][f] = mfma_bf16(ah[mb], bl, acc[mb][f]);
        acc[mb][f] = mfma_bf16(al[mb], bh, acc[mb][f]);
      }
    }
  }

  // ---------------------------------------------------------------- epilogues
  // the activation tile is free now: reuse it for the cross-wave row reductions
  float* red = reinterpret_cast<float*>(&As[0][0]);  // [3][4 waves][MT]
  const float limit = p.limit;
  if constexpr (KIND == kGateUp) {
    // pass 1: g, u saved in fp32, row maxima of h over the tile's 128 columns
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mb * 16 + lg * 4 + i;
        const bool vrow = row < mlen;
        const size_t m = (size_t)(m0 + row);
        const int ex = s_exp[row];
        float mx = 0.f;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int col = n0 + w * 32 + f * 16 + lr;
          const bool valid = vrow && col < I;
          const float g = ldexpf(acc[mb][f][i], -ex);
          const float u = ldexpf(acc[mb][f + 2][i], -ex);
          if (valid) {
            p.gsave[m * I + col] = g;
            p.usave[m * I + col] = u;
          }
          float gp, up, mg, mu;
          clamp_swiglu(g, u, limit, gp, up, mg, mu);
          const float h = valid ? gp * sigmoid_f(gp) * up : 0.f;
          mx = fmaxf(mx, fabsf(h));
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if (lr == 0) red[w * MT + row] = mx;
      }
    __syncthreads();
    // pass 2: h in fp16 times 2^p, p per (row, 128-column chunk)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mb * 16 + lg * 4 + i;
        if (row >= mlen) continue;
        const size_t m = (size_t)(m0 + row);
        const int ex = s_exp[row];
        const float mx = fmaxf(fmaxf(red[row], red[MT + row]), fmaxf(red[2 * MT + row], red[3 * MT + row]));
        const int pe = pow2_exponent_for(mx);
        if (w == 0 && lr == 0) p.hexp[m * p.h_nch + nt] = pe;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int col = n0 + w * 32 + f * 16 + lr;
          if (col >= I) continue;
          float gp, up, mg, mu;
          clamp_swiglu(ldexpf(acc[mb][f][i], -ex), ldexpf(acc[mb][f + 2][i], -ex), limit, gp, up, mg, mu);
          p.hh[m * I + perm_pos(col)] = float_to_half_bits(ldexpf(gp * sigmoid_f(gp) * up, pe));
        }
      }
  } else if constexpr (KIND == kDown || KIND == kGateUpBwd) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mb * 16 + lg * 4 + i;
        if (row >= mlen) continue;
        const int slot = s_slot[row];
        const float wgt = (KIND == kDown) ? p.rw[slot] : 1.f;
        const int ex = s_exp[row];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = n0 + w * 64 + f * 16 + lr;
          if (col < H) p.stage[(size_t)slot * H + col] = wgt * ldexpf(acc[mb][f][i], -ex);
        }
      }
  } else {  // kDownBwd
    // pass 1: dRoute partial sums and the row maxima of dG and dU
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mb * 16 + lg * 4 + i;
        const bool vrow = row < mlen;
        const size_t m = (size_t)(m0 + row);
        const float wgt = vrow ? p.rw[s_slot[row]] : 0.f;
        const int ex = s_exp[row];
        float dr = 0.f, mxg = 0.f, mxu = 0.f;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = n0 + w * 64 + f * 16 + lr;
          if (!(vrow && col < I)) continue;
          const float gh = ldexpf(acc[mb][f][i], -ex);
          float gp, up, mg, mu;
          clamp_swiglu(p.gsave[m * I + col], p.usave[m * I + col], limit, gp, up, mg, mu);
          const float sg = sigmoid_f(gp);
          const float si = gp * sg;
          const float dsi = sg * (1.f + gp * (1.f - sg));
          dr += gh * si * up;
          const float dh = wgt * gh;
          mxg = fmaxf(mxg, fabsf(dh * up * dsi * mg));
          mxu = fmaxf(mxu, fabsf(dh * si * mu));
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          dr += __shfl_xor(dr, off);
          mxg = fmaxf(mxg, __shfl_xor(mxg, off));
          mxu = fmaxf(mxu, __shfl_xor(mxu, off));
        }
        if (lr == 0) {
          red[w * MT + row] = dr;
          red[(4 + w) * MT + row] = mxg;
          red[(8 + w) * MT + row] = mxu;
        }
      }
    __syncthreads();
    const int half_nch = p.dg_nch / 2;
    // pass 2: dG, dU in fp16 times 2^p, p per (row, 256-column chunk)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mb * 16 + lg * 4 + i;
        if (row >= mlen) continue;
        const size_t m = (size_t)(m0 + row);
        const float wgt = p.rw[s_slot[row]];
        const int ex = s_exp[row];
        const int pg = pow2_exponent_for(fmaxf(fmaxf(red[4 * MT + row], red[5 * MT + row]),
                                               fmaxf(red[6 * MT + row], red[7 * MT + row])));
        const int pu = pow2_exponent_for(fmaxf(fmaxf(red[8 * MT + row], red[9 * MT + row]),
                                               fmaxf(red[10 * MT + row], red[11 * MT + row])));
        if (w == 0 && lr == 0) {
          p.drpart[m * p.dr_nt + nt] = (red[row] + red[MT + row]) + (red[2 * MT + row] + red[3 * MT + row]);
          p.dguexp[m * p.dg_nch + nt] = pg;
          p.dguexp[m * p.dg_nch + half_nch + nt] = pu;
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = n0 + w * 64 + f * 16 + lr;
          if (col >= I) continue;
          const float gh = ldexpf(acc[mb][f][i], -ex);
          float gp, up, mg, mu;
          clamp_swiglu(p.gsave[m * I + col], p.usave[m * I + col], limit, gp, up, mg, mu);
          const float sg = sigmoid_f(gp);
          const float si = gp * sg;
          const float dsi = sg * (1.f + gp * (1.f - sg));
          const float dh = wgt * gh;
          const int pc = perm_pos(col);
          p.dgu[m * (size_t)(2 * I) + pc] = float_to_half_bits(ldexpf(dh * up * dsi * mg, pg));
          p.dgu[m * (size_t)(2 * I) + I + pc] = float_to_half_bits(ldexpf(dh * si * mu, pu));
        }
      }
  }
}

template <int KIND>
static void launch_kind(int mt, unsigned grid, const GemmParams& p, hipStream_t st) {
  switch (mt) {
    case 16:
      k_gemm<KIND, 16><<<grid, 256, 0, st>>>(p);
      break;
    case 32:
      k_gemm<KIND, 32><<<grid, 256, 0, st>>>(p);
      break;
    case 64:
      k_gemm<KIND, 64><<<grid, 256, 0, st>>>(p);
      break;
    default:
      k_gemm<KIND, 128><<<grid, 256, 0, st>>>(p);
      break;
  }
}

void launch_gemm(GemmKind kind, const Dims& d, const WsMap& w, void* ws, const LayerPtrs& L,
                 const float* route_weights, hipStream_t st) {
  GemmParams p{};
  p.E = (int)d.E;
  p.topk = (int)d.K;
  p.H = (int)d.H;
  p.I = (int)d.I;
  p.R = (int)d.R;
  p.sc = d.sc;
  p.limit = d.limit;
  p.sorted_slot = ws_ptr<int32_t>(ws, w.sorted_slot);
  p.offsets = ws_ptr<int32_t>(ws, w.offsets);
  p.tile_e = ws_ptr<int32_t>(ws, w.tile_e);
  p.tile_m0 = ws_ptr<int32_t>(ws, w.tile_m0);
  p.counters = ws_ptr<unsigned long long>(ws, w.counters);
  p.bad_scales = ws_ptr<unsigned long long>(ws, w.counters) + kBadScales;
  p.L = L;
  p.rw = route_weights;
  p.gsave = ws_ptr<float>(ws, w.g);
  p.usave = ws_ptr<float>(ws, w.u);
  p.hh = ws_ptr<uint16_t>(ws, w.hh);
  p.hexp = ws_ptr<int32_t>(ws, w.hexp);
  p.h_nch = (int)w.h_nch;
  p.stage = ws_ptr<float>(ws, w.stage);
  p.dgu = ws_ptr<uint16_t>(ws, w.dgu);
  p.dguexp = ws_ptr<int32_t>(ws, w.dguexp);
  p.dg_nch = (int)w.dg_nch;
  p.drpart = ws_ptr<float>(ws, w.drpart);
  p.dr_nt = (int)w.dr_nt;
  switch (kind) {
    case kGateUp:
      p.n_ntiles = (int)((d.I + kHChunk - 1) / kHChunk);
      p.a_src = ws_ptr<uint16_t>(ws, w.xh);
      p.a_rowexp = ws_ptr<int32_t>(ws, w.xexp);
      p.lda = d.H;
      p.la0 = ws_ptr<float>(ws, w.ua);
      p.la1 = ws_ptr<float>(ws, w.ub);
      break;
    case kDown:
      p.n_ntiles = (int)((d.H + kNT - 1) / kNT);
      p.a_src = ws_ptr<uint16_t>(ws, w.hh);
      p.a_chunkexp = ws_ptr<int32_t>(ws, w.hexp);
      p.a_nch = (int)w.h_nch;
      p.a_chunkw = kHChunk;
      p.lda = d.I;
      p.la0 = ws_ptr<float>(ws, w.ud);
      break;
    case kDownBwd:
      p.n_ntiles = (int)((d.I + kNT - 1) / kNT);
      p.a_src = ws_ptr<uint16_t>(ws, w.dyh);
      p.a_rowexp = ws_ptr<int32_t>(ws, w.dyexp);
      p.lda = d.H;
      p.la0 = ws_ptr<float>(ws, w.dyb);
      break;
    case kGateUpBwd:
      p.n_ntiles = (int)((d.H + kNT - 1) / kNT);
      p.a_src = ws_ptr<uint16_t>(ws, w.dgu);
      p.a_chunkexp = ws_ptr<int32_t>(ws, w.dguexp);
      p.a_nch = (int)w.dg_nch;
      p.a_chunkw = kNT;
      p.lda = 2 * d.I;
      p.la0 = ws_ptr<float>(ws, w.dgb);
      p.la1 = ws_ptr<float>(ws, w.dub);
      break;
  }
  const unsigned grid = (unsigned)(w.max_tiles * p.n_ntiles);
  if (grid == 0) return;
  switch (kind) {
    case kGateUp:
      launch_kind<kGateUp>((int)w.mt, grid, p, st);
      break;
    case kDown:
      launch_kind<kDown>((int)w.mt, grid, p, st);
      break;
    case kDownBwd:
      launch_kind<kDownBwd>((int)w.mt, grid, p, st);
      break;
    case kGateUpBwd:
      launch_kind<kGateUpBwd>((int)w.mt, grid, p, st);
      break;
  }
}

}  // namespace kt
