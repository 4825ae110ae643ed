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
#include <limits.h>

#include <algorithm>

#include "kt_common.hpp"
#include "kt_internal.hpp"

namespace kt {

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t* lds_v4s_ptr;


// ================================================================ side products

constexpr int kSK = 32;  // contraction values per step
template <int V>
struct IntTag {
  static constexpr int value = V;
};

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
  int ksplit;   // contraction ranges (blockIdx.y); above 1 the blocks write partial sums
  int sub;      // workgroups per tile of the list (each takes MT consecutive rows of it)
  float* part;  // [ksplit][Ms][nq] partial sums, reduced in order by k_side_reduce
  int64_t Ms;
  const int32_t* nrows;  // rows routed to an expert (offsets[E])
  // The planes go to an expert GEMM whose activation row m carries a power-of-two
  // exponent (the one of its fp16 row): the planes carry it too, so that the
  // GEMM adds them to its scaled sums.  fp16 sources: the source row's own
  // exponent (exps); token rows: tok_exp[token] (nullptr: 0).
  const int32_t* tok_exp;
};

// exponent of the consuming GEMM's activation row m
__device__ __forceinline__ int side_plane_exp(const SideArgs& a, int64_t m) {
  if (a.exps) return a.exps[m * a.exp_ld + a.exp_off];
  return a.tok_exp ? a.tok_exp[a.sorted_slot[m] / a.topk] : 0;
}

// product column col of sorted row m: the fp32 output and its bf16 hi/lo planes
// (times the LoRA scale and 2^pe)
__device__ __forceinline__ void side_store(const SideArgs& a, int64_t m, int col, float v, int pe) {
  const int R = a.R;
  if (col < R)
    a.out[m * R + col] = v;
  else
    a.out2[m * R + (col - R)] = v;
  uint16_t hi, lo;
  split_bf16(ldexpf(v * a.split_scale, pe), hi, lo);
  const int64_t sc = col < R ? a.split_off + col : a.split_off2 + (col - R);
  a.split[m * 2 * a.split_ld + sc] = hi;
  a.split[m * 2 * a.split_ld + a.split_ld + sc] = lo;
}

// sum of the partial products over the contraction ranges, in range order
__global__ __launch_bounds__(256) void k_side_reduce(SideArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t m = i / a.nq;
  const int col = (int)(i % a.nq);
  if (m >= *a.nrows) return;  // only rows routed to an expert were multiplied
  float v = 0.f;
  for (int ks = 0; ks < a.ksplit; ++ks) v += a.part[((int64_t)ks * a.Ms + m) * a.nq + col];
  side_store(a, m, col, v, side_plane_exp(a, m));
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
  __shared__ int32_t s_src[MT], s_ex[MT], s_pex[MT];

  // Work item (tile, contraction range); block b (in dispatch order) runs on
  // XCD b % 8, and each XCD takes a contiguous run of the items in use: the
  // tiles of one expert (consecutive in the list) and the ranges of one tile
  // share an XCD, and so its L2 for the expert's LoRA matrix.  (The grid is a
  // whole number of rounds of 8 blocks, at least the items in use: every XCD
  // has a block for each of its items.)
  const unsigned nitems = (unsigned)a.counters[kNumTiles] * a.sub * gridDim.y;
  const unsigned bid = blockIdx.y * gridDim.x + blockIdx.x, per = (nitems + 7) / 8;
  const unsigned item = (bid % 8) * per + bid / 8;
  if (bid / 8 >= per || item >= nitems) return;
  const unsigned per_tile = (unsigned)a.sub * gridDim.y;
  const int tile = (int)(item / per_tile), sb = (int)(item % per_tile / gridDim.y), ks = (int)(item % gridDim.y);
  const int e = a.tile_e[tile], m0 = a.tile_m0[tile] + MT * sb;
  const int mlen = min(MT, a.offsets[e + 1] - m0);
  if (mlen <= 0) return;  // (a part of a list tile past its expert's rows)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int R = a.R, kdim = a.kdim;
  if (tid < MT) {
    const int m = m0 + min(tid, mlen - 1);  // rows past the tile's end repeat its last row
    s_src[tid] = HALF ? m : a.sorted_slot[m] / a.topk;
    s_ex[tid] = HALF ? a.exps[(int64_t)m * a.exp_ld + a.exp_off] : 0;
    s_pex[tid] = side_plane_exp(a, m);
  }
  __syncthreads();

  // per-thread source pointers of the contraction's start, advanced by k0 (A
  // rows, rk matrices) or k0 rows (k-major matrices) per step
  const uint16_t* pA[kAC];
#pragma unroll
  for (int i = 0; i < kAC; ++i) {
    const int q = tid + 256 * i, row = (q >> 2) & (MT - 1), c = q & 3;
    pA[i] = a.src + (int64_t)s_src[row] * a.ld + a.col_off + 8 * c;
  }
  const float* pB[NB];
  bool okB[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int q = tid + 256 * i;
    if (a.rk) {  // W[e][col][k]: thread -> (column, 8 consecutive k)
      const int col = q >> 2, c = q & 3;
      const bool second = col >= R;
      const float* Wm = second ? a.W2 : a.W;
      const int qq = min(second ? col - R : col, R - 1);
      okB[i] = col < a.nq;
      pB[i] = (Wm ? Wm : a.W) + ((int64_t)e * R + qq) * kdim + 8 * c;
    } else {  // W[e][k][col]: thread -> (k, 8 consecutive columns), whole 16-byte runs where possible
      const int kr = q / (NQ / 8), c8 = q % (NQ / 8);
      const int col0 = 8 * c8;
      const bool second0 = col0 >= R;
      const int cc = second0 ? col0 - R : col0;
      okB[i] = (R & 3) == 0 && cc + 8 <= R && col0 + 8 <= a.nq;
      pB[i] = (second0 && a.W2 ? a.W2 : a.W) + ((int64_t)e * kdim + kr) * R + cc;
    }
  }
  // two register sets: step s + 2's loads are in flight while step s is
  // multiplied and step s + 1 is written to LDS
  u32x4 areg2[2][kAC];
  float breg2[2][NB][8];
  auto load = [&](int k0, auto rs) {
    u32x4(&areg)[kAC] = areg2[decltype(rs)::value];
    float(&breg)[NB][8] = breg2[decltype(rs)::value];
#pragma unroll
    for (int i = 0; i < kAC; ++i) areg[i] = *reinterpret_cast<const u32x4*>(pA[i] + k0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (okB[i]) {
        const float* p = pB[i] + (a.rk ? (int64_t)k0 : (int64_t)k0 * R);
        const float4 x0 = *reinterpret_cast<const float4*>(p), x1 = *reinterpret_cast<const float4*>(p + 4);
        breg[i][0] = x0.x, breg[i][1] = x0.y, breg[i][2] = x0.z, breg[i][3] = x0.w;
        breg[i][4] = x1.x, breg[i][5] = x1.y, breg[i][6] = x1.z, breg[i][7] = x1.w;
      } else if (a.rk) {  // a column past the product's width
#pragma unroll
        for (int t = 0; t < 8; ++t) breg[i][t] = 0.f;
      } else {  // k-major columns one at a time (rank not a multiple of 4, or the run crosses a matrix)
        const int q = tid + 256 * i;
        const int kr = q / (NQ / 8), col0 = 8 * (q % (NQ / 8));
        const float* row = a.W + ((int64_t)e * kdim + k0 + kr) * R;
        const float* row2 = a.W2 ? a.W2 + ((int64_t)e * kdim + k0 + kr) * R : row;
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
  };
  auto store = [&](int buf, auto rs) {
    const u32x4(&areg)[kAC] = areg2[decltype(rs)::value];
    const float(&breg)[NB][8] = breg2[decltype(rs)::value];
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
  // this block's contraction range: steps [s0, s1) of kSK values
  const int ksteps = kdim / kSK;
  const int s0 = (int)((int64_t)ksteps * ks / a.ksplit), s1 = (int)((int64_t)ksteps * (ks + 1) / a.ksplit);
  const int nsteps = s1 - s0;
  const IntTag<0> r0{};
  const IntTag<1> r1{};
  load(s0 * kSK, r0);
  store(0, r0);
  if (nsteps > 1) load((s0 + 1) * kSK, r1);
  __syncthreads();
  // step s: registers rn hold step s + 1, registers rf are free for step s + 2
  auto body = [&](int s, auto rn, auto rf) {
    const int cur = s & 1;
    if (s + 2 < nsteps) load((s0 + s + 2) * kSK, rf);
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
    if (s + 1 < nsteps) store(cur ^ 1, rn);
    __syncthreads();
  };
  for (int s = 0; s < nsteps; s += 2) {
    body(s, r1, r0);
    if (s + 1 < nsteps) body(s + 1, r0, r1);
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
        if (a.ksplit > 1)
          a.part[((int64_t)ks * a.Ms + m) * a.nq + col] = v;
        else
          side_store(a, m, col, v, s_pex[row]);
      }
    }
}

template <int MT, int NB>
static void launch_side_nb(bool half, dim3 grid, const SideArgs& a, hipStream_t st) {
  if (half)
    k_lora_side<MT, NB, true><<<grid, 256, 0, st>>>(a);
  else
    k_lora_side<MT, NB, false><<<grid, 256, 0, st>>>(a);
  note_launch();
}

template <int MT>
static void launch_side_mt(int nb, bool half, dim3 grid, const SideArgs& a, hipStream_t st) {
  if (nb <= 1)
    launch_side_nb<MT, 1>(half, grid, a, st);
  else if (nb == 2)
    launch_side_nb<MT, 2>(half, grid, a, st);
  else
    launch_side_nb<MT, 4>(half, grid, a, st);
}

void launch_lora_rowproj(const Dims& d, const WsMap& w, void* ws, const RowView& src, int64_t kdim, const float* W,
                         const float* W2, bool rk, float* out, float* out2, int64_t split_ld, int64_t split_off,
                         int64_t split_off2, const int32_t* tok_exp, hipStream_t st) {
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
  a.tok_exp = tok_exp;
  const bool half = src.kind == kSrcHalfChunked;
  const int nb = (a.nq + 63) / 64;
  // Short contractions (the intermediate width) run each 128-row tile of the
  // list as two 64-row workgroups: fewer padding rows per workgroup for
  // lightly loaded experts, and twice the workgroups in flight (measured
  // faster there; the hidden-width contractions are not).
  a.sub = (w.mt == 128 && kdim <= 2048) ? 2 : 1;
  // few tiles (small token counts) leave most CUs idle through a long
  // contraction: split it over blocks and reduce the partial sums in order
  // (~4096 workgroups in all, at most the split the workspace is planned for;
  // none once there are 2048 or more workgroups without it)
  const int64_t items = std::max<int64_t>(w.max_tiles * a.sub, 1);
  a.ksplit = items >= 2048 ? 1 : (int)std::min<int64_t>(std::min<int64_t>(w.side_ksplit, (4096 + items - 1) / items), kdim / (4 * kSK));
  if (a.ksplit < 1) a.ksplit = 1;
  a.part = ws_ptr<float>(ws, w.side_part);
  a.Ms = d.Ms;
  a.nrows = a.offsets + d.E;
  // whole rounds of 8 blocks: every XCD then has a block for each of its items
  const dim3 grid((unsigned)((w.max_tiles * a.sub + 7) / 8 * 8), (unsigned)a.ksplit);
  switch (w.mt / a.sub) {
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
  if (a.ksplit > 1) {
    const int64_t n = d.Ms * a.nq;
    k_side_reduce<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(a);
    note_launch();
  }
}

// ================================================================ gradients

struct GradPrepArgs {
  const int32_t* offsets;
  const int32_t* sorted_slot;
  const int32_t* tile_e;
  const int32_t* tile_m0;
  const unsigned long long* counters;
  int mt, R;
  const float* rw;  // route weight per flat slot
  const int32_t* hexp;
  int64_t h_nch;
  const int32_t* dgexp;
  int64_t dg_nch;
  const float *ua, *ub, *ud, *dyb, *dgb, *dub;  // side products [Ms][R]
  uint16_t* planes;                             // [Ms][row]
  int64_t row, r16;
  int64_t off_x, np_x, off_dy, np_dy, off_h, np_h, off_g, np_g;  // np_g: one half
  int32_t* gexp;                                                 // [E][2]: h family, dG|dU family
  int E;
  int32_t* eorder;  // [E]: experts by descending row count (ties: lower index first)
  int32_t* gtmax;   // [tiles][2]: largest exponents of the h and dG|dU families in a row tile
};

// Per row tile (side-product tiles, one expert's rows each), the largest binary
// exponent of each fp16 narrow family: h family rw * dyB * 2^-hexp, dG|dU family
// ua | ub * 2^-dgexp (hexp, dgexp: the wide row's own exponent, so the wide fp16
// values can be used as they are); INT_MIN for a family with no finite nonzero value.
__global__ __launch_bounds__(256) void k_grad_tile_max(GradPrepArgs a) {
  __shared__ int s_max[2];
  const int tile = blockIdx.x;
  if ((unsigned long long)tile >= a.counters[kNumTiles]) return;
  const int e = a.tile_e[tile], m0 = a.tile_m0[tile];
  const int mlen = min(a.mt, a.offsets[e + 1] - m0);
  if (threadIdx.x < 2) s_max[threadIdx.x] = INT_MIN;
  __syncthreads();
  int mh = INT_MIN, mg = INT_MIN;
  for (int idx = threadIdx.x; idx < mlen * a.R; idx += blockDim.x) {
    const int64_t m = m0 + idx / a.R;
    const int pq = idx % a.R;
    const float rw = a.rw[a.sorted_slot[m]];
    const int he = a.hexp[m * a.h_nch], ge = a.dgexp[m * a.dg_nch];
    const int64_t i = m * a.R + pq;
    int ex;
    const float vh = fabsf(a.dyb[i] * rw);
    if (vh > 0.f && vh < INFINITY) {
      (void)frexpf(vh, &ex);
      mh = max(mh, ex - he);
    }
    const float vg = fmaxf(fabsf(a.ua[i]), fabsf(a.ub[i]));
    if (vg > 0.f && vg < INFINITY) {
      (void)frexpf(vg, &ex);
      mg = max(mg, ex - ge);
    }
  }
  atomicMax(&s_max[0], mh);
  atomicMax(&s_max[1], mg);
  __syncthreads();
  if (threadIdx.x < 2) a.gtmax[2 * tile + threadIdx.x] = s_max[threadIdx.x];
}

// Per expert, the power-of-two exponent S of each fp16 narrow family that puts
// its largest magnitude into [2^14, 2^15), from its row tiles' maxima (the
// expert's tiles are the ceil(rows / mt) that follow those of the experts
// before it).  Also the expert's place in the order the gradient kernels deal
// their work out: most rows first, so that a heavily loaded expert's long
// contractions start at once rather than last.  One block per expert.
__global__ __launch_bounds__(256) void k_grad_exps(GradPrepArgs a) {
  __shared__ int s_max[2];
  __shared__ int s_rank, s_t0;
  const int e = blockIdx.x;
  const int n = a.offsets[e + 1] - a.offsets[e];
  if (threadIdx.x < 2) s_max[threadIdx.x] = INT_MIN;
  if (threadIdx.x == 0) s_rank = 0, s_t0 = 0;
  __syncthreads();
  {
    int before = 0, t0 = 0;
    for (int f = threadIdx.x; f < a.E; f += blockDim.x) {
      const int nf = a.offsets[f + 1] - a.offsets[f];
      before += (nf > n || (nf == n && f < e)) ? 1 : 0;
      if (f < e) t0 += (nf + a.mt - 1) / a.mt;
    }
    atomicAdd(&s_rank, before);
    atomicAdd(&s_t0, t0);
  }
  __syncthreads();
  const int t0 = s_t0, nt = (n + a.mt - 1) / a.mt;
  int mh = INT_MIN, mg = INT_MIN;
  for (int t = threadIdx.x; t < nt; t += blockDim.x) {
    mh = max(mh, a.gtmax[2 * (t0 + t)]);
    mg = max(mg, a.gtmax[2 * (t0 + t) + 1]);
  }
  atomicMax(&s_max[0], mh);
  atomicMax(&s_max[1], mg);
  __syncthreads();
  if (threadIdx.x < 2) {
    const int mx = s_max[threadIdx.x];
    a.gexp[2 * e + threadIdx.x] = mx == INT_MIN ? 0 : 15 - mx;
  }
  if (threadIdx.x == 0) a.eorder[s_rank] = e;
}

// The narrow planes of one row tile's rows [16 y, 16 y + 16) (y = blockIdx.y):
// every row's four families as 16-bit hi/lo pairs (bf16 by truncation for the x
// and dY families, fp16 rounded to nearest for the h and dG|dU families after the
// expert's exponent), zero past the rank.
constexpr int kPlaneRows = 16;  // rows of a tile per block

// Values c .. c + 7 of an fp32 row of R values (zero past R), times f: two
// 16-byte loads when R is a multiple of 8 (a run of 8 then lies wholly inside
// the row or wholly past it, and starts 32-byte aligned), else one at a time.
__device__ __forceinline__ void load8_scaled(const float* row, int64_t c, int R, float f, float (&v)[8]) {
  if ((R & 7) == 0) {
    if (c < R) {
      const float4 x0 = *reinterpret_cast<const float4*>(row + c), x1 = *reinterpret_cast<const float4*>(row + c + 4);
      v[0] = x0.x * f, v[1] = x0.y * f, v[2] = x0.z * f, v[3] = x0.w * f;
      v[4] = x1.x * f, v[5] = x1.y * f, v[6] = x1.z * f, v[7] = x1.w * f;
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = 0.f;
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) v[t] = c + t < R ? row[c + t] * f : 0.f;
}
__global__ __launch_bounds__(256) void k_grad_planes(GradPrepArgs a) {
  const int tile = blockIdx.x;
  if ((unsigned long long)tile >= a.counters[kNumTiles]) return;
  const int e = a.tile_e[tile];
  const int m0 = a.tile_m0[tile] + kPlaneRows * (int)blockIdx.y;
  const int mlen = min(kPlaneRows, a.offsets[e + 1] - m0);
  if (mlen <= 0) return;
  const int sh = a.gexp[2 * e], sg = a.gexp[2 * e + 1];
  const int R = a.R;
  const int ux = (int)(a.np_x / 8), ud = (int)(a.np_dy / 8), uh = (int)(a.np_h / 8), ug = (int)(a.np_g / 4);
  const int units = ux + ud + uh + ug;
  for (int idx = threadIdx.x; idx < mlen * units; idx += blockDim.x) {
    const int r = idx / units;
    int j = idx % units;
    const int64_t m = m0 + r;
    float v[8];
    int64_t off, pw;
    bool f16;
    if (j < ux) {  // [dG B_g | dU B_u], each padded to r16
      const int64_t u = 8 * j;
      const bool second = u >= a.r16;
      const float* src = second ? a.dub : a.dgb;
      const int64_t c = second ? u - a.r16 : u;
      load8_scaled(src + m * R, c, R, 1.f, v);
      off = a.off_x + u;
      pw = a.np_x;
      f16 = false;
    } else if ((j -= ux) < ud) {  // rw ud
      const int64_t u = 8 * j;
      const float rw = a.rw[a.sorted_slot[m]];
      load8_scaled(a.ud + m * R, u, R, rw, v);
      off = a.off_dy + u;
      pw = a.np_dy;
      f16 = false;
    } else if ((j -= ud) < uh) {  // rw dyB 2^(S - hexp)
      const int64_t u = 8 * j;
      const float rw = a.rw[a.sorted_slot[m]];
      const int k = sh - a.hexp[m * a.h_nch];
      load8_scaled(a.dyb + m * R, u, R, rw, v);
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = ldexpf(v[t], k);
      off = a.off_h + u;
      pw = a.np_h;
      f16 = true;
    } else {  // ua | ub 2^(S - dgexp), halves np_g apart
      j -= uh;
      const int64_t u = 8 * j;
      const bool second = u >= a.np_g;
      const float* src = second ? a.ub : a.ua;
      const int64_t c = second ? u - a.np_g : u;
      const int k = sg - a.dgexp[m * a.dg_nch];
      load8_scaled(src + m * R, c, R, 1.f, v);
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = ldexpf(v[t], k);
      off = a.off_g + u;
      pw = 2 * a.np_g;
      f16 = true;
    }
    u32x4 hi, lo;
    if (f16) {
      uint16_t h[8], l[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        h[t] = float_to_half_bits(v[t]);
        l[t] = float_to_half_bits(v[t] - half_bits_to_float(h[t]));
      }
      hi = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
      lo = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
    } else {
      split8_trunc(v, hi, lo);
    }
    uint16_t* dst = a.planes + m * a.row + off;
    *reinterpret_cast<u32x4*>(dst) = hi;
    *reinterpret_cast<u32x4*>(dst + pw) = lo;
  }
}

// The window rule for experts no row is routed to, when the call does not
// accumulate: their six gradient slices are zero.  Block (e, g, c) clears chunk c
// of gradient g's slice of expert e (slices are contiguous [E][...] rows).
struct GradZeroArgs {
  const int32_t* offsets;
  float* g[6];
  int64_t n[6];  // floats per expert in each gradient
};
constexpr int kZeroChunk = 32768;  // floats per block
__global__ __launch_bounds__(256) void k_grad_zero_unrouted(GradZeroArgs a) {
  const int e = blockIdx.x, j = blockIdx.y;
  if (a.offsets[e + 1] != a.offsets[e]) return;
  const int64_t n = a.n[j], c0 = (int64_t)blockIdx.z * kZeroChunk;
  if (c0 >= n) return;
  float* p = a.g[j] + (int64_t)e * n;
  const int64_t c1 = min<int64_t>(n, c0 + kZeroChunk);
  for (int64_t i = c0 + threadIdx.x; i < c1; i += blockDim.x) p[i] = 0.f;
}

struct GradArgs {
  int E, R;
  const int32_t* offsets;
  const int32_t* tok_of_row;
  const uint16_t* wide;  // row-major 16-bit rows (token rows, or sorted rows)
  int64_t wld;           // row stride (elements)
  int64_t wcols;         // columns of one half
  int64_t whalf;         // column offset of the second half in a row
  int nhalves, nvh;      // halves, 256-column tiles per half
  const uint16_t* planes;  // this family's first plane column
  int64_t prow, pw;        // plane row stride; hi at 0, lo at pw
  int64_t uhalf;           // narrow plane offset for the second wide half
  int nu;                  // narrow tiles
  int64_t usplit;          // narrow index where the second output starts
  const int32_t* gexp;
  const int32_t* eorder;  // experts, most rows first
  int gexp_sel;  // -1: no exponent
  float* out0;
  float* out1;
  int accumulate;
  float scale;
  const void* zero;  // 16 zero bytes
};

// Families: 0 = x (bf16 token rows, narrow x wide), 1 = dY (bf16 token rows,
// wide x narrow), 2 = h (fp16 sorted rows, narrow x wide), 3 = dG|dU (fp16
// sorted rows in two halves, wide x narrow).  fp16 rows keep the within-8
// permuted column order of the matrix kernels.
template <int NUT, int FAM, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void k_lora_grad(GradArgs a) {
  constexpr bool kF16 = FAM >= 2, kGather = FAM <= 1, kTrans = (FAM & 1) != 0, kPerm = FAM >= 2;
  constexpr int kGK = 32;                // expert rows per step (one MFMA contraction)
  constexpr int kWRow = 512;             // LDS bytes of one wide row (256 columns)
  constexpr int kWBytes = kGK * kWRow;
  constexpr int kNRow = 4 * NUT;         // LDS bytes of one narrow row: NUT hi then NUT lo values
  constexpr int kNC = NUT / 4;           // 16-byte chunks per narrow row
  constexpr int kStage = kWBytes + kGK * kNRow;
  constexpr int kStages = 2;
  constexpr int L = kStages - 1;                    // steps in flight ahead of the one multiplied
  constexpr int kWI = 16 / NW;                      // wide copies (1 KB each) per wave per step
  constexpr int kNCW = 8 * NUT / NW;                // narrow 16-byte chunks per wave per step
  constexpr int kNI = kNCW >= 64 ? kNCW / 64 : 1;   // narrow copies per wave per step
  constexpr int kOps = kWI + kNI + (kGather ? 1 : 0);
  constexpr int WN = NUT < 64 ? NUT : 64;           // narrow columns per wave
  constexpr int WAVES_N = NUT / WN;
  constexpr int WV = 256 * WAVES_N / NW;            // wide columns per wave
  constexpr int NB = WN / 16, VB = WV / 16;
  static_assert(NW == 4 || NW == 8, "waves");
  static_assert(kNCW % 64 == 0 || kNCW == 32, "narrow copy shape");
  __shared__ __align__(16) uint8_t ring[kStages * kStage];
  __shared__ __align__(16) int32_t ridx[kGather ? 4 * kGK : 4];

  // work item (expert, narrow tile, half, wide tile), wide tiles fastest.  The
  // experts, most rows first, are dealt to the eight XCDs in turn (blocks reach
  // them in turn too), and each XCD runs its experts' items in that order: a
  // heavily loaded expert (whose items contract over all its rows) starts with
  // the first blocks, and an expert's items share one XCD's L2
  const unsigned per_e = (unsigned)(a.nu * a.nhalves * a.nvh);
  const unsigned xcd = blockIdx.x % 8u, local = blockIdx.x / 8u;
  const unsigned rank = xcd + 8u * (local / per_e);
  if (rank >= (unsigned)a.E) return;
  const int e = a.eorder[rank];
  const unsigned rem = local % per_e;
  const int ut = (int)(rem / (unsigned)(a.nhalves * a.nvh));
  const int half = (int)((rem / (unsigned)a.nvh) % (unsigned)a.nhalves);
  const int vt = (int)(rem % (unsigned)a.nvh);
  const int m0 = a.offsets[e], rows = a.offsets[e + 1] - m0;
  if (rows == 0) return;  // (an expert without rows: its gradient is zeroed by k_grad_zero_unrouted, or kept)
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t v0 = (int64_t)vt * 256;
  const int vend = (int)min<int64_t>(256, a.wcols - v0);
  const int64_t wcol0 = half * a.whalf + v0;
  const int64_t ncol0 = half * a.uhalf + (int64_t)ut * NUT;
  const int nsteps = (rows + kGK - 1) / kGK;
  const uint32_t ring0 = lds_addr(ring);

  // 16-byte chunk c of LDS row r sits at c ^ swz(r): the 4 rows x 32 bytes that
  // a 16-lane transposed read touches fall on distinct banks
  auto swz_w = [](int r) { return 2 * ((r & 3) | (((r >> 3) & 1) << 2)); };
  auto swz_n = [](int r) {
    return kNC >= 16 ? 2 * ((r & 3) | (((r >> 3) & 1) << 2)) : kNC == 8 ? 2 * (r & 3) : 2 * ((r >> 1) & 1);
  };

  // token ids of step t's rows (clamped to the expert's last row) into ridx slot t % 4
  auto issue_idx = [&](int t) {
    if constexpr (kGather) {
      if (lane < kGK) dma4(a.tok_of_row + m0 + min(t * kGK + lane, rows - 1), lds_addr(&ridx[(t & 3) * kGK]));
    }
  };
  // Step t's copies, kOps per wave: the token ids of step t + L first, then the
  // wide rows (rows past the expert's end repeat its last row) and the narrow
  // rows (zero past the end), so a wait for step t also covers ids of t + L.
  auto issue = [&](int t) {
    issue_idx(t + L);
    const uint32_t st = ring0 + (t % kStages) * kStage;
    const int k0 = t * kGK;
#pragma unroll
    for (int j = 0; j < kWI; ++j) {
      const int q = kWI * w + j;
      const int r = 2 * q + (lane >> 5);
      const int c = (lane & 31) ^ swz_w(r);
      const int col = 8 * c < vend ? 8 * c : 0;
      int64_t rowid;
      if constexpr (kGather)
        rowid = ridx[(t & 3) * kGK + r];
      else
        rowid = m0 + min(k0 + r, rows - 1);
      dma16(a.wide + rowid * a.wld + wcol0 + col, st + 1024 * q);
    }
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      if (kNCW >= 64 || lane < kNCW) {
        const int g = w * kNCW + 64 * i + lane;
        const int r = g / kNC;
        const int c = (g % kNC) ^ swz_n(r);
        const int plane = c / (kNC / 2), cc = c % (kNC / 2);
        const void* src = k0 + r < rows
                              ? (const void*)(a.planes + (int64_t)(m0 + k0 + r) * a.prow + plane * a.pw + ncol0 + 8 * cc)
                              : a.zero;
        dma16(src, st + kWBytes + 16 * (w * kNCW + 64 * i));
      }
    }
  };

  // 8 consecutive rows (8 lg ..) of column col of a row-major LDS block, as the
  // MFMA operand of lane (lr, lg): two transposed reads of 4 rows each
  auto frag = [&](const uint8_t* base, int pitch, int chunk0, int col, bool wide) -> u32x4 {
    const int r0 = 8 * lg + (lr >> 2), cc = col + 4 * (lr & 3);
    const int c = chunk0 + (cc >> 3);
    const int s0 = wide ? swz_w(r0) : swz_n(r0), s1 = wide ? swz_w(r0 + 4) : swz_n(r0 + 4);
    const v4s_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s_ptr)(base + r0 * pitch + 16 * (c ^ s0) + 2 * (cc & 7)));
    const v4s_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s_ptr)(base + (r0 + 4) * pitch + 16 * (c ^ s1) + 2 * (cc & 7)));
    return u32x4{pack2(x0.x, x0.y), pack2(x0.z, x0.w), pack2(x1.x, x1.y), pack2(x1.z, x1.w)};
  };
  auto mma = [](u32x4 x, u32x4 y, floatx4 c) { return kF16 ? mfma_f16(x, y, c) : mfma_bf16(x, y, c); };

  constexpr int A0 = kTrans ? VB : NB, A1 = kTrans ? NB : VB;
  floatx4 acc[A0][A1];
#pragma unroll
  for (int i = 0; i < A0; ++i)
#pragma unroll
    for (int j = 0; j < A1; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int wn0 = (w % WAVES_N) * WN, wv0 = (w / WAVES_N) * WV;

  if (nsteps > 0) {
    if constexpr (kGather) {
#pragma unroll
      for (int t = 0; t < L; ++t) issue_idx(t);
      asm volatile("" ::: "memory");
      wait_vm_lgkm<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int t = 0; t < L; ++t)
      if (t < nsteps) issue(t);
    for (int s = 0; s < nsteps; ++s) {
      // step s has landed once at most the later step's copies are outstanding;
      // the barrier shows every wave's copies and frees the slot refilled next
      // (the empty asm statements keep the compiler from moving LDS accesses
      // across the wait and the barrier, which do not order them for it)
      asm volatile("" ::: "memory");
      if (s + 1 < nsteps)
        wait_vm_lgkm<(L - 1) * kOps>();
      else
        wait_vm_lgkm<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (s + L < nsteps) issue(s + L);
      if (wv0 < vend) {
        const uint8_t* sw = ring + (s % kStages) * kStage;
        const uint8_t* sn = sw + kWBytes;
        u32x4 nh[NB], nl[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          nh[nb] = frag(sn, kNRow, 0, wn0 + 16 * nb, false);
          nl[nb] = frag(sn, kNRow, kNC / 2, wn0 + 16 * nb, false);
        }
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
          const u32x4 wf = frag(sw, kWRow, 0, wv0 + 16 * vb, true);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            if constexpr (kTrans) {
              acc[vb][nb] = mma(wf, nh[nb], acc[vb][nb]);
              acc[vb][nb] = mma(wf, nl[nb], acc[vb][nb]);
            } else {
              acc[nb][vb] = mma(nh[nb], wf, acc[nb][vb]);
              acc[nb][vb] = mma(nl[nb], wf, acc[nb][vb]);
            }
          }
        }
      }
    }
  }

  // G = (accumulate ? G : 0) + scale * 2^-S * acc
  const int S = a.gexp_sel >= 0 ? a.gexp[2 * e + a.gexp_sel] : 0;
  auto logical = [](int j) { return kPerm ? (j & ~7) | perm_src(j & 7) : j; };
#pragma unroll
  for (int i0 = 0; i0 < A0; ++i0)
#pragma unroll
    for (int i1 = 0; i1 < A1; ++i1)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = a.scale * ldexpf(acc[i0][i1][i], -S);
        float* out;
        int64_t idx;
        if constexpr (kTrans) {  // rows along the wide operand, columns along the rank
          const int j = wv0 + 16 * i0 + 4 * lg + i;
          const int64_t q = (int64_t)ut * NUT + wn0 + 16 * i1 + lr;
          if (j >= vend || q >= a.R) continue;
          out = half ? a.out1 : a.out0;
          idx = ((int64_t)e * a.wcols + v0 + logical(j)) * a.R + q;
        } else {  // rows along the rank, columns along the wide operand
          const int64_t ug = (int64_t)ut * NUT + wn0 + 16 * i0 + 4 * lg + i;
          const int j = wv0 + 16 * i1 + lr;
          const bool second = ug >= a.usplit;
          const int64_t p = second ? ug - a.usplit : ug;
          if (j >= vend || p >= a.R) continue;
          out = second ? a.out1 : a.out0;
          idx = ((int64_t)e * a.R + p) * a.wcols + v0 + logical(j);
        }
        out[idx] = (a.accumulate ? out[idx] : 0.f) + v;
      }
}

template <int FAM>
static void launch_grad_family(int nut, unsigned grid, const GradArgs& a, hipStream_t st) {
  switch (nut) {
    case 16:
      k_lora_grad<16, FAM, 4><<<grid, 256, 0, st>>>(a);
      note_launch();
      break;
    case 32:
      k_lora_grad<32, FAM, 4><<<grid, 256, 0, st>>>(a);
      note_launch();
      break;
    case 64:
      k_lora_grad<64, FAM, 4><<<grid, 256, 0, st>>>(a);
      note_launch();
      break;
    default:  // 8 waves: a block of the 128-column narrow width and a two-step ring (64 KB of LDS)
      k_lora_grad<128, FAM, 8><<<grid, 512, 0, st>>>(a);
      note_launch();
      break;
  }
}

void launch_lora_grads(const Dims& d, const WsMap& w, void* ws, const uint16_t* inputs, const uint16_t* grad_output,
                       const float* route_weights, const LoraGradOut& out, int accumulate, float scale,
                       hipStream_t st) {
  const GradGeom G = grad_geom(d.R);
  GradPrepArgs p{};
  p.offsets = ws_ptr<int32_t>(ws, w.offsets);
  p.sorted_slot = ws_ptr<int32_t>(ws, w.sorted_slot);
  p.tile_e = ws_ptr<int32_t>(ws, w.tile_e);
  p.tile_m0 = ws_ptr<int32_t>(ws, w.tile_m0);
  p.counters = ws_ptr<unsigned long long>(ws, w.counters);
  p.mt = (int)w.mt;
  p.R = (int)d.R;
  p.rw = route_weights;
  p.hexp = ws_ptr<int32_t>(ws, w.hexp);
  p.h_nch = w.h_nch;
  p.dgexp = ws_ptr<int32_t>(ws, w.dguexp);
  p.dg_nch = w.dg_nch;
  p.ua = ws_ptr<float>(ws, w.ua);
  p.ub = ws_ptr<float>(ws, w.ub);
  p.ud = ws_ptr<float>(ws, w.ud);
  p.dyb = ws_ptr<float>(ws, w.dyb);
  p.dgb = ws_ptr<float>(ws, w.dgb);
  p.dub = ws_ptr<float>(ws, w.dub);
  p.planes = ws_ptr<uint16_t>(ws, w.gplanes);
  p.row = G.row;
  p.r16 = G.r16;
  p.off_x = G.off_x;
  p.np_x = G.x.np;
  p.off_dy = G.off_dy;
  p.np_dy = G.dy.np;
  p.off_h = G.off_h;
  p.np_h = G.h.np;
  p.off_g = G.off_g;
  p.np_g = G.g.np;
  p.gexp = ws_ptr<int32_t>(ws, w.gexp);
  p.E = (int)d.E;
  p.eorder = ws_ptr<int32_t>(ws, w.eorder);
  p.gtmax = ws_ptr<int32_t>(ws, w.gtmax);
  if (w.max_tiles > 0) {
    k_grad_tile_max<<<(unsigned)w.max_tiles, 256, 0, st>>>(p);
    note_launch();
  }
  k_grad_exps<<<(unsigned)d.E, 256, 0, st>>>(p);
  note_launch();
  if (w.max_tiles > 0) {
    k_grad_planes<<<dim3((unsigned)w.max_tiles, (unsigned)((w.mt + kPlaneRows - 1) / kPlaneRows)), 256, 0, st>>>(p);
    note_launch();
  }

  if (!accumulate) {
    GradZeroArgs z{};
    z.offsets = p.offsets;
    float* gs[6] = {out.ag, out.au, out.bd, out.ad, out.bg, out.bu};
    const int64_t ns[6] = {d.R * d.H, d.R * d.H, d.H * d.R, d.R * d.I, d.I * d.R, d.I * d.R};
    int64_t nmax = 0;
    for (int j = 0; j < 6; ++j) {
      z.g[j] = gs[j];
      z.n[j] = ns[j];
      nmax = std::max(nmax, ns[j]);
    }
    const dim3 zg((unsigned)d.E, 6u, (unsigned)((nmax + kZeroChunk - 1) / kZeroChunk));
    k_grad_zero_unrouted<<<zg, 256, 0, st>>>(z);
    note_launch();
  }

  GradArgs a{};
  a.E = (int)d.E;
  a.R = (int)d.R;
  a.offsets = p.offsets;
  a.tok_of_row = ws_ptr<int32_t>(ws, w.tok_of_row);
  a.prow = G.row;
  a.gexp = p.gexp;
  a.eorder = p.eorder;
  a.accumulate = accumulate;
  a.scale = scale;
  a.zero = ws_ptr<unsigned long long>(ws, w.counters) + kZeroWord;
  const uint16_t* planes = p.planes;
  auto tiles = [](int64_t n) { return (int)((n + 255) / 256); };
  // whole rounds of eight experts (one per XCD); blocks past the last expert return
  auto grid = [&](const GradFam& f) { return (unsigned)((a.E + 7) / 8 * 8 * f.nu * a.nhalves * a.nvh); };
  // dA_g, dA_u = sc sum [dG B_g | dU B_u] (x) x
  a.wide = inputs;
  a.wld = d.H;
  a.wcols = d.H;
  a.whalf = 0;
  a.nhalves = 1;
  a.nvh = tiles(d.H);
  a.planes = planes + G.off_x;
  a.pw = G.x.np;
  a.uhalf = 0;
  a.nu = G.x.nu;
  a.usplit = G.r16;
  a.gexp_sel = -1;
  a.out0 = out.ag;
  a.out1 = out.au;
  launch_grad_family<0>(G.x.nut, grid(G.x), a, st);
  // dB_d = sc sum dY (x) rw ud
  a.wide = grad_output;
  a.planes = planes + G.off_dy;
  a.pw = G.dy.np;
  a.nu = G.dy.nu;
  a.usplit = INT64_MAX;
  a.out0 = out.bd;
  a.out1 = out.bd;
  launch_grad_family<1>(G.dy.nut, grid(G.dy), a, st);
  // dA_d = sc sum rw dyB (x) h
  a.wide = ws_ptr<uint16_t>(ws, w.hh);
  a.wld = d.I;
  a.wcols = d.I;
  a.nvh = tiles(d.I);
  a.planes = planes + G.off_h;
  a.pw = G.h.np;
  a.nu = G.h.nu;
  a.gexp_sel = 0;
  a.out0 = out.ad;
  a.out1 = out.ad;
  launch_grad_family<2>(G.h.nut, grid(G.h), a, st);
  // dB_g, dB_u = sc sum dG (x) ua, dU (x) ub
  a.wide = ws_ptr<uint16_t>(ws, w.dgu);
  a.wld = 2 * d.I;
  a.whalf = d.I;
  a.nhalves = 2;
  a.planes = planes + G.off_g;
  a.pw = 2 * G.g.np;
  a.uhalf = G.g.np;
  a.nu = G.g.nu;
  a.gexp_sel = 1;
  a.out0 = out.bg;
  a.out1 = out.bu;
  launch_grad_family<3>(G.g.nut, grid(G.g), a, st);
}

}  // namespace kt
