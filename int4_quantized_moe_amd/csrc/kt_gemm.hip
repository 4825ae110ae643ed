// Grouped matrix kernels of the routed layer on gfx950 MFMA.
//
// One template serves the four expert GEMMs of the page "rawint4_sft_reference.py"
// (routed_rawint4_lora and the autograd of run_routed_reference):
//   kGateUp    g, u = x W_g^T, x W_u^T (+ LoRA), then the clamped SwiGLU (rawint4_swiglu)
//   kDown      y = h W_d^T (+ LoRA), times the route weight, into per-slot staging
//   kDownBwd   g_h = dY W_d (+ LoRA), then dRoute = <g_h, h> partials and the
//              SwiGLU/clamp gradient dG, dU
//   kGateUpBwd dx = dG W_g + dU W_u (+ LoRA), into per-slot staging
// A work tile is kMT token-slot rows of one expert (sorted by the grouping) by a
// block of output columns.  The int4 weights are decoded on the fly into exact
// fp16 values ((c - 8) * scale fits fp16's 11-bit significand) and multiplied
// with fp16 activations on v_mfma_f32_16x16x32_f16, accumulating in fp32.
// Activations carry a power-of-two exponent per row (x, dY) or per (row, column
// chunk) (h, dG, dU) so that fp16's range never clips them; the chunk
// exponents are brought to the row's common exponent when the tile is staged.
// The two gradient GEMMs read W in its stored [N, K] orientation and contract
// over N: the decode transposes 8x8 nibble blocks while staging, which is the
// transpose-free dX of transpose_free_rawint4_dx (no transposed or dense copy).
// The LoRA terms ride along as extra K-steps: the fp32 LoRA-A products and the
// fp32 LoRA matrices are split into bf16 hi + lo parts and multiplied with
// three bf16 MFMAs (hi*hi + hi*lo + lo*hi), about 16 significant bits each.
#include <limits.h>

#include "kt_common.hpp"
#include "kt_internal.hpp"

namespace kt {

constexpr int KP = 40;  // LDS row pitch in 16-bit elements: 80 bytes keeps 16-byte reads conflict free

struct GemmParams {
  int E, topk, H, I, R;
  float sc, limit;
  const int32_t* sorted_slot;
  const int32_t* offsets;
  const int32_t* tile_e;
  const int32_t* tile_m0;
  const unsigned long long* counters;
  LayerPtrs L;
  const uint16_t* a_src;      // fp16 activation rows
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

template <int KIND>
__device__ __forceinline__ int bcol(int wn, int f) {
  if constexpr (KIND == kGateUp) return f < 2 ? wn * 32 + f * 16 : 64 + wn * 32 + (f - 2) * 16;
  return wn * 64 + f * 16;
}

__device__ __forceinline__ uint32_t mul_half2(uint32_t v, half2_t s) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v) * s);
}

template <int KIND>
__global__ __launch_bounds__(256) void k_gemm(GemmParams p) {
  __shared__ __align__(16) uint16_t As[2][kMT * KP];
  __shared__ __align__(16) uint16_t Bs[2][kNT * KP];
  __shared__ int32_t s_src[kMT], s_exp[kMT], s_slot[kMT];
  __shared__ float s_red[3][2][kMT];

  const int tile = (int)(blockIdx.x / (unsigned)p.n_ntiles);
  const int nt = (int)(blockIdx.x % (unsigned)p.n_ntiles);
  if ((unsigned long long)tile >= p.counters[kNumTiles]) return;
  const int e = p.tile_e[tile], m0 = p.tile_m0[tile];
  const int mlen = min(kMT, p.offsets[e + 1] - m0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int H = p.H, I = p.I, R = p.R;

  constexpr bool kTransB = (KIND == kDownBwd || KIND == kGateUpBwd);
  constexpr bool kChunkedA = (KIND == kDown || KIND == kGateUpBwd);
  const int n0 = (KIND == kGateUp) ? nt * kHChunk : nt * kNT;
  const int nout = (KIND == kGateUp || KIND == kDownBwd) ? I : H;
  const int kdim = (KIND == kGateUp || KIND == kDownBwd) ? H : (KIND == kDown ? I : 2 * I);

  if (tid < kMT) {
    int src = -1, ex = 0, slot = -1;
    if (tid < mlen) {
      const int m = m0 + tid;
      slot = p.sorted_slot[m];
      if constexpr (kChunkedA) {
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

  floatx4 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  // ------------------------------------------------------------ main K loop (fp16)
  for (int k0 = 0; k0 < kdim; k0 += kGroup) {
    {  // A tile: kMT rows x 32 columns, one 16-byte piece per thread
      const int row = tid >> 2, part = tid & 3;
      const int src = s_src[row];
      u32x4 v = {0u, 0u, 0u, 0u};
      if (src >= 0) {
        v = *reinterpret_cast<const u32x4*>(p.a_src + (size_t)src * p.lda + k0 + part * 8);
        if constexpr (kChunkedA) {
          int c;
          if constexpr (KIND == kDown) {
            c = k0 / p.a_chunkw;
          } else {
            c = k0 < I ? k0 / p.a_chunkw : p.a_nch / 2 + (k0 - I) / p.a_chunkw;
          }
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
      *reinterpret_cast<u32x4*>(&As[0][row * KP + part * 8]) = v;
    }
    if constexpr (!kTransB) {
      // B tile, stored orientation: output column = weight row, 32 consecutive k
      for (int it = tid; it < kNT * 4; it += 256) {
        const int j = it >> 2, d = it & 3;
        u32x4 r = {0u, 0u, 0u, 0u};
        const uint8_t* W;
        const uint16_t* S;
        size_t row;
        int rk;
        bool valid;
        if constexpr (KIND == kGateUp) {
          const bool up = j >= kHChunk;
          const int n = n0 + (j & (kHChunk - 1));
          valid = n < I;
          W = up ? p.L.wu : p.L.wg;
          S = up ? p.L.su : p.L.sg;
          row = (size_t)e * I + n;
          rk = H;
        } else {
          const int n = n0 + j;
          valid = n < H;
          W = p.L.wd;
          S = p.L.sd;
          row = (size_t)e * H + n;
          rk = I;
        }
        if (valid) {
          const uint32_t wv = *reinterpret_cast<const uint32_t*>(W + row * (size_t)(rk / 2) + k0 / 2 + d * 4);
          const float sf = bf16_to_float(S[row * (size_t)(rk / kGroup) + k0 / kGroup]);
          if (d == 0 && !scale_in_domain(sf)) atomicAdd(p.bad_scales, 1ull);
          const _Float16 sh = (_Float16)sf;
          r = decode_dword(wv, half2_t{sh, sh});
        }
        *reinterpret_cast<u32x4*>(&Bs[0][j * KP + d * 8]) = r;
      }
    } else {
      // B tile, contraction over the weight rows: 8 rows x 8 columns per task,
      // decoded into column-major 16-byte pieces (8 contraction values each)
      if (tid < 64) {
        const int ro = tid >> 4, co = tid & 15;
        const int c = n0 + co * 8;
        const bool valid = c < nout;
        uint32_t wv[8];
        float sv[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const int kk = k0 + ro * 8 + rr;
          const uint8_t* W;
          const uint16_t* S;
          size_t row;
          int rk;
          if constexpr (KIND == kDownBwd) {
            W = p.L.wd;
            S = p.L.sd;
            row = (size_t)e * H + kk;
            rk = I;
          } else {
            const bool up = kk >= I;
            W = up ? p.L.wu : p.L.wg;
            S = up ? p.L.su : p.L.sg;
            row = (size_t)e * I + (up ? kk - I : kk);
            rk = H;
          }
          wv[rr] = 0u;
          sv[rr] = 0.f;
          if (valid) {
            wv[rr] = *reinterpret_cast<const uint32_t*>(W + row * (size_t)(rk / 2) + c / 2);
            sv[rr] = bf16_to_float(S[row * (size_t)(rk / kGroup) + c / kGroup]);
            if (!scale_in_domain(sv[rr])) atomicAdd(p.bad_scales, 1ull);
          }
        }
        half2_t sp[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) sp[q] = half2_t{(_Float16)sv[2 * q], (_Float16)sv[2 * q + 1]};
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          u32x4 o;
          o.x = decode_pair((wv[0] >> (4 * jj)) & 15u, (wv[1] >> (4 * jj)) & 15u, sp[0]);
          o.y = decode_pair((wv[2] >> (4 * jj)) & 15u, (wv[3] >> (4 * jj)) & 15u, sp[1]);
          o.z = decode_pair((wv[4] >> (4 * jj)) & 15u, (wv[5] >> (4 * jj)) & 15u, sp[2]);
          o.w = decode_pair((wv[6] >> (4 * jj)) & 15u, (wv[7] >> (4 * jj)) & 15u, sp[3]);
          if (!valid) o = u32x4{0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(&Bs[0][(co * 8 + jj) * KP + ro * 8]) = o;
        }
      }
    }
    __syncthreads();
    u32x4 af[2];
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
      af[fm] = *reinterpret_cast<const u32x4*>(&As[0][(wm * 32 + fm * 16 + (lane & 15)) * KP + (lane >> 4) * 8]);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const u32x4 bf = *reinterpret_cast<const u32x4*>(&Bs[0][(bcol<KIND>(wn, f) + (lane & 15)) * KP + (lane >> 4) * 8]);
#pragma unroll
      for (int fm = 0; fm < 2; ++fm) acc[fm][f] = mfma_f16(af[fm], bf, acc[fm][f]);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ LoRA K-steps (bf16 hi/lo)
  const int KL = (KIND == kGateUp || KIND == kGateUpBwd) ? 2 * R : R;
  for (int q0 = 0; q0 < KL; q0 += kGroup) {
    {
      const int row = tid >> 2, qq = (tid & 3) * 8;
      const float coef = ldexpf(p.sc, s_exp[row]);
      uint16_t hi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = q0 + qq + j;
        float v = 0.f;
        if (row < mlen && q < KL) {
          const size_t m = (size_t)(m0 + row);
          if constexpr (KIND == kGateUp || KIND == kGateUpBwd)
            v = q < R ? p.la0[m * R + q] : p.la1[m * R + (q - R)];
          else
            v = p.la0[m * R + q];
          v *= coef;
        }
        split_bf16(v, hi[j], lo[j]);
      }
      u32x4 vh, vl;
      vh.x = hi[0] | ((uint32_t)hi[1] << 16);
      vh.y = hi[2] | ((uint32_t)hi[3] << 16);
      vh.z = hi[4] | ((uint32_t)hi[5] << 16);
      vh.w = hi[6] | ((uint32_t)hi[7] << 16);
      vl.x = lo[0] | ((uint32_t)lo[1] << 16);
      vl.y = lo[2] | ((uint32_t)lo[3] << 16);
      vl.z = lo[4] | ((uint32_t)lo[5] << 16);
      vl.w = lo[6] | ((uint32_t)lo[7] << 16);
      *reinterpret_cast<u32x4*>(&As[0][row * KP + qq]) = vh;
      *reinterpret_cast<u32x4*>(&As[1][row * KP + qq]) = vl;
    }
    {
      const int j = tid >> 1, qq = (tid & 1) * 16;
      for (int jj = 0; jj < 16; ++jj) {
        const int q = q0 + qq + jj;
        float v = 0.f;
        if constexpr (KIND == kGateUp) {
          const bool up = j >= kHChunk;
          const int n = n0 + (j & (kHChunk - 1));
          if (n < I) {
            if (!up && q < R) v = p.L.bg[((size_t)e * I + n) * R + q];
            if (up && q >= R && q < 2 * R) v = p.L.bu[((size_t)e * I + n) * R + (q - R)];
          }
        } else if constexpr (KIND == kDown) {
          const int n = n0 + j;
          if (n < H && q < R) v = p.L.bd[((size_t)e * H + n) * R + q];
        } else if constexpr (KIND == kDownBwd) {
          const int c = n0 + j;
          if (c < I && q < R) v = p.L.ad[((size_t)e * R + q) * I + c];
        } else {
          const int c = n0 + j;
          if (c < H) {
            if (q < R)
              v = p.L.ag[((size_t)e * R + q) * H + c];
            else if (q < 2 * R)
              v = p.L.au[((size_t)e * R + (q - R)) * H + c];
          }
        }
        uint16_t hi, lo;
        split_bf16(v, hi, lo);
        Bs[0][j * KP + qq + jj] = hi;
        Bs[1][j * KP + qq + jj] = lo;
      }
    }
    __syncthreads();
    u32x4 ah[2], al[2];
#pragma unroll
    for (int fm = 0; fm < 2; ++fm) {
      const int off = (wm * 32 + fm * 16 + (lane & 15)) * KP + (lane >> 4) * 8;
      ah[fm] = *reinterpret_cast<const u32x4*>(&As[0][off]);
      al[fm] = *reinterpret_cast<const u32x4*>(&As[1][off]);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int off = (bcol<KIND>(wn, f) + (lane & 15)) * KP + (lane >> 4) * 8;
      const u32x4 bh = *reinterpret_cast<const u32x4*>(&Bs[0][off]);
      const u32x4 bl = *reinterpret_cast<const u32x4*>(&Bs[1][off]);
#pragma unroll
      for (int fm = 0; fm < 2; ++fm) {
        acc[fm][f] = mfma_bf16(ah[fm], bh, acc[fm][f]);
        acc[fm][f] = mfma_bf16(ah[fm], bl, acc[fm][f]);
        acc[fm][f] = mfma_bf16(al[fm], bh, acc[fm][f]);
      }
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogues
  const int lc = lane & 15, lg = lane >> 4;
  const float limit = p.limit;
  if constexpr (KIND == kGateUp) {
    float hv[2][2][4];
    float rmax[2][4];
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 32 + fm * 16 + lg * 4 + i;
        const bool vrow = row < mlen;
        const size_t m = (size_t)(m0 + row);
        const int ex = s_exp[row];
        rmax[fm][i] = 0.f;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int col = n0 + wn * 32 + f * 16 + lc;
          const bool valid = vrow && col < I;
          const float g = ldexpf(acc[fm][f][i], -ex);
          const float u = ldexpf(acc[fm][f + 2][i], -ex);
          if (valid) {
            p.gsave[m * I + col] = g;
            p.usave[m * I + col] = u;
          }
          float gp = g, up = u;
          if (limit > 0.f) {
            if (!(g <= limit)) gp = limit;
            up = fminf(fmaxf(u, -limit), limit);
          }
          const float h = valid ? gp * sigmoid_f(gp) * up : 0.f;
          hv[fm][f][i] = h;
          rmax[fm][i] = fmaxf(rmax[fm][i], fabsf(h));
        }
        float v = rmax[fm][i];
        v = fmaxf(v, __shfl_xor(v, 1));
        v = fmaxf(v, __shfl_xor(v, 2));
        v = fmaxf(v, __shfl_xor(v, 4));
        v = fmaxf(v, __shfl_xor(v, 8));
        if (lc == 0) s_red[0][wn][row] = v;
      }
    __syncthreads();
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 32 + fm * 16 + lg * 4 + i;
        if (row >= mlen) continue;
        const size_t m = (size_t)(m0 + row);
        const int pe = pow2_exponent_for(fmaxf(s_red[0][0][row], s_red[0][1][row]));
        if (wn == 0 && lc == 0) p.hexp[m * p.h_nch + nt] = pe;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int col = n0 + wn * 32 + f * 16 + lc;
          if (col < I) p.hh[m * I + col] = float_to_half_bits(ldexpf(hv[fm][f][i], pe));
        }
      }
  } else if constexpr (KIND == kDown || KIND == kGateUpBwd) {
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 32 + fm * 16 + lg * 4 + i;
        if (row >= mlen) continue;
        const int slot = s_slot[row];
        const float w = (KIND == kDown) ? p.rw[slot] : 1.f;
        const int ex = s_exp[row];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = n0 + wn * 64 + f * 16 + lc;
          if (col < H) p.stage[(size_t)slot * H + col] = w * ldexpf(acc[fm][f][i], -ex);
        }
      }
  } else {  // kDownBwd
    float du[2][4][4];
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 32 + fm * 16 + lg * 4 + i;
        const bool vrow = row < mlen;
        const size_t m = (size_t)(m0 + row);
        const float w = vrow ? p.rw[s_slot[row]] : 0.f;
        const int ex = s_exp[row];
        float dr = 0.f, mg = 0.f, mu = 0.f;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = n0 + wn * 64 + f * 16 + lc;
          const bool valid = vrow && col < I;
          const float gh = ldexpf(acc[fm][f][i], -ex);
          const float g = valid ? p.gsave[m * I + col] : 0.f;
          const float u = valid ? p.usave[m * I + col] : 0.f;
          float gp = g, up = u, mgate = 1.f, mup = 1.f;
          if (limit > 0.f) {
            if (!(g <= limit)) {
              gp = limit;
              mgate = 0.f;
            }
            if (u < -limit) {
              up = -limit;
              mup = 0.f;
            } else if (u > limit) {
              up = limit;
              mup = 0.f;
            }
          }
          const float sg = sigmoid_f(gp);
          const float si = gp * sg;
          const float dsi = sg * (1.f + gp * (1.f - sg));
          dr += valid ? gh * si * up : 0.f;
          const float dh = w * gh;
          const float dgv = valid ? dh * up * dsi * mgate : 0.f;
          const float duv = valid ? dh * si * mup : 0.f;
          acc[fm][f][i] = dgv;
          du[fm][f][i] = duv;
          mg = fmaxf(mg, fabsf(dgv));
          mu = fmaxf(mu, fabsf(duv));
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          dr += __shfl_xor(dr, off);
          mg = fmaxf(mg, __shfl_xor(mg, off));
          mu = fmaxf(mu, __shfl_xor(mu, off));
        }
        if (lc == 0) {
          s_red[0][wn][row] = dr;
          s_red[1][wn][row] = mg;
          s_red[2][wn][row] = mu;
        }
      }
    __syncthreads();
    const int half_nch = p.dg_nch / 2;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 32 + fm * 16 + lg * 4 + i;
        if (row >= mlen) continue;
        const size_t m = (size_t)(m0 + row);
        const int pg = pow2_exponent_for(fmaxf(s_red[1][0][row], s_red[1][1][row]));
        const int pu = pow2_exponent_for(fmaxf(s_red[2][0][row], s_red[2][1][row]));
        if (wn == 0 && lc == 0) {
          p.drpart[m * p.dr_nt + nt] = s_red[0][0][row] + s_red[0][1][row];
          p.dguexp[m * p.dg_nch + nt] = pg;
          p.dguexp[m * p.dg_nch + half_nch + nt] = pu;
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = n0 + wn * 64 + f * 16 + lc;
          if (col < I) {
            p.dgu[m * (size_t)(2 * I) + col] = float_to_half_bits(ldexpf(acc[fm][f][i], pg));
            p.dgu[m * (size_t)(2 * I) + I + col] = float_to_half_bits(ldexpf(du[fm][f][i], pu));
          }
        }
      }
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
      k_gemm<kGateUp><<<grid, 256, 0, st>>>(p);
      break;
    case kDown:
      k_gemm<kDown><<<grid, 256, 0, st>>>(p);
      break;
    case kDownBwd:
      k_gemm<kDownBwd><<<grid, 256, 0, st>>>(p);
      break;
    case kGateUpBwd:
      k_gemm<kGateUpBwd><<<grid, 256, 0, st>>>(p);
      break;
  }
}

}  // namespace kt
