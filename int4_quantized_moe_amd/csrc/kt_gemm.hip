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
// (64 each) and share the activation tile.  Each expert's rows take full
// 128-row tiles and one tile of the smallest height (16/32/64/96/128) that
// holds the rest; one launch covers every height.  Operands move through an LDS
// ring of 64 contraction values per stage, filled by direct global-to-LDS 16-byte
// loads (no register staging): three stages for 64/96/128-row tiles, five or six
// for 32/16-row tiles, whose fragments of the next stage are read and decoded
// while the current one is multiplied.  The ring waits are explicit (vmcnt)
// around a bare s_barrier, so the compiler's conservative drain at
// __syncthreads does not serialise the ring.  In the 64/96/128-row tiles each
// wave runs a stage's MFMAs at a raised wave priority, one column block after
// another, decoding the next column block's weights in between (and reading
// the next k-step's activation fragments): the SIMD's other wave (another
// workgroup) decodes or copies in the gaps.  16-row tiles in the stored
// orientation, bound by the weight stream, use no ring: each wave loads its
// own codes, scales and activation values straight into registers, several
// units of 128 contraction values ahead, with no barrier.  Position p of
// the tile list runs on XCD p % 8 (blocks reach the XCDs in turn), each XCD
// running all column tiles of a row tile together: the column tiles of one row
// tile share that XCD's L2 for the activation rows, and the grouping places an
// expert's row tiles on one XCD one after another (a heavily loaded expert's
// spread over all eight), so that they share it for the weights.
//
// Weights are decoded on the fly into exact fp16 ((c - 8) * scale fits fp16's
// 11-bit significand) and multiplied on v_mfma_f32_16x16x32_f16 with fp32
// accumulation.  In the stored orientation (kGateUp, kDown: contraction along
// the packed K) each column's 32 packed bytes of a stage sit in LDS and a lane
// reads its 16 nibbles with one 8-byte read; one fused multiply-add per pair of
// weights decodes them (decode_dword_fma).  The two gradient GEMMs contract over
// the weight rows: the raw packed rows are copied into LDS as they are and read
// back with ds_read_tr4_b64, which hands each lane 16 consecutive rows of one
// column; this is the transpose-free dX of transpose_free_rawint4_dx with the
// transpose done by the LDS read.  The scales come from the forward's fp16
// transposed copy ([E][K/32][N], rows within-8 permuted) by the same copies.
// MXFP4 weights (E2M1 codes, power-of-two scales; template flag MX) are decoded
// by gfx950's fp4 conversion instead (decode_dword_e2m1, decode_dword_perm_e2m1),
// into the same exact fp16 values and the same element order.
//
// LDS tiles are XOR-swizzled in 16-byte units so that the fragment reads of a
// wave spread over the banks: activation row r keeps chunk c in slot
// c ^ ((r & 7) ^ ((r >> 3) & 1)); stored-orientation weight column n keeps its
// half h in slot h ^ ((n >> 3) & 1); transposed weight row k keeps its chunk c
// in slot c ^ ((k >> 1) & 7).
//
// Activations carry one power-of-two exponent per row so that fp16's range never
// clips them (x, dY per token; h and dG|dU per sorted row after their chunk
// exponents are brought to the row's smallest); the epilogue removes it.  LoRA
// terms ride along as extra K-steps: the fp32 LoRA-A side products and the fp32
// LoRA matrices are split into bf16 hi + lo and multiplied with three bf16 MFMAs
// (hi*hi + hi*lo + lo*hi); they run while the ring's first stages are in flight.
#include <limits.h>

#include "kt_common.hpp"
#include "kt_internal.hpp"

namespace kt {

constexpr int kKS = 64;         // contraction values per stage (two quant groups)
constexpr int kWBytes = 8192;   // packed weight bytes per stage (256 columns x 64 values)
constexpr int kScBytes = 1024;  // fp16 scales per stage (256 columns x 2 groups, or 64 rows x 8 groups)
constexpr int kLBP = 544;       // row pitch in bytes of a transposed LoRA matrix group (256 bf16 + 32 B)

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t* lds_v2i_ptr;
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t* lds_v4s_ptr;
typedef const void __attribute__((address_space(1)))* global_ptr;
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};
template <int V>
struct FTag {
  static constexpr int value = V;
};
typedef void __attribute__((address_space(3)))* lds_ptr;

// The ring's wait-and-barrier points are fenced for the compiler as well: the
// s_waitcnt and s_barrier builtins do not order memory accesses for it, so
// without these empty asm statements it could move a fragment read of a stage
// above the barrier that makes the stage visible, or a read of a slot below the
// barrier after which another wave refills the slot.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

struct GemmParams {
  int E, topk, H, I, R;
  float sc, limit;
  const int32_t* sorted_slot;
  const int32_t* offsets;
  const int32_t* tile_e;
  const int32_t* tile_m0;
  const int32_t* tile_mt;
  const int32_t* expert_slot;  // place of an expert in the transposed scale tables
  const int32_t* sshift;       // [E][2] power-of-two shift of an expert's gate/up and down scale tables
  const unsigned long long* counters;
  LayerPtrs L;
  const uint16_t* a_src;      // fp16 activation rows (within-8 permuted order)
  const int32_t* a_rowexp;    // per token exponent (x, dY)
  const int32_t* a_chunkexp;  // per (row, chunk) exponent (h, dG|dU), all chunks of a row equal
  int a_nch;
  int64_t lda;
  const uint16_t* lsplit;  // side product times the LoRA scale, bf16 hi/lo planes [Ms][2][KLP]
  const uint16_t* sct0;    // fp16 scales [active expert][K/32][rows], rows within-8 permuted: gate (or down)
  const uint16_t* sct1;    // up
  const float* rw;  // route weights per flat slot
  const void* zero;  // 16 zero bytes
  // saved pre-activations in quad-row layout: row m of expert e sits at
  // position q = qoffsets[e] + (m - offsets[e]), element (q >> 2, col, q & 3) of
  // [rows / 4][I][4], so a lane's four rows of one column are one 16-byte run
  float* gsave;
  float* usave;
  const int32_t* qoffsets;
  uint16_t* hh;
  int32_t* hexp;
  int h_nch;
  uint16_t* stage;  // per-slot rows in fp16 times 2^p
  int32_t* stexp;   // p per (slot row, kStageExp columns)
  int st_nch;
  uint16_t* dgu;
  int32_t* dguexp;
  int dg_nch;
  float* drpart;
  int dr_nt;
  int n_ntiles;
};

// local column (0..255 within the tile) of N-block f of wave w
template <int KIND>
__device__ __forceinline__ int local_col(int w, int f) {
  if constexpr (KIND == kGateUp) return f < 2 ? w * 32 + f * 16 : kHChunk + w * 32 + (f - 2) * 16;
  return w * 64 + f * 16;
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

// Ring depth of a tile height: the 128-row ring sets the LDS of the kernel
// (two workgroups per CU), and shorter tiles spend the same LDS on more stages
// in flight, which is what keeps memory busy when there are few rows to multiply.
__host__ __device__ constexpr int gemm_stages(int MT) { return MT == 16 ? 6 : MT == 32 ? 5 : 3; }
// LDS bytes of the ring of a tile height (the LoRA K-steps reuse it).
__host__ __device__ constexpr int gemm_ring_bytes(int MT) {
  const int a = MT * 128, st = gemm_stages(MT) * (a + kWBytes + kScBytes), lora = a + 64 * kLBP;
  return st > lora ? st : lora;
}
constexpr int kRingMax = gemm_ring_bytes(128);
static_assert(gemm_ring_bytes(16) <= kRingMax && gemm_ring_bytes(32) <= kRingMax && gemm_ring_bytes(64) <= kRingMax &&
                  gemm_ring_bytes(96) <= kRingMax,
              "the 128-row ring is the largest");

// s_waitcnt vmcnt <= n * D (lgkmcnt 0) for a run-time n in [0, 4]
template <int D>
__device__ __forceinline__ void wait_stages(int n) {
  switch (n) {
    case 0:
      wait_vm_lgkm<0>();
      break;
    case 1:
      wait_vm_lgkm<D>();
      break;
    case 2:
      wait_vm_lgkm<2 * D>();
      break;
    case 3:
      wait_vm_lgkm<3 * D>();
      break;
    default:
      wait_vm_lgkm<4 * D>();
      break;
  }
}

// One work tile of height MT; the LDS belongs to the calling kernel.  LDMA:
// the LoRA matrix is copied by DMA in whole 16-byte runs (rank a multiple of 4).
// MX: the weights are MXFP4 (E2M1 codes, power-of-two scales) instead of RAWINT4.
template <int KIND, int MT, bool LDMA, bool MX>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, int tile, int nt, uint8_t* ring, int32_t* s_src,
                                          int32_t* s_exp, int32_t* s_slot, float* s_rw) {
  constexpr int MB = MT / 16;
  constexpr bool kT = (KIND == kDownBwd || KIND == kGateUpBwd);
  constexpr bool kChunked = (KIND == kDown || KIND == kGateUpBwd);
  constexpr int kABytes = MT * 128;                 // activation tile of one stage
  constexpr int kRowsPerInst = MT == 16 ? 4 : 8;     // activation rows per DMA instruction
  constexpr int kAInst = MT == 16 ? 1 : MT / 32;     // activation DMA instructions per wave per stage
  constexpr int kDmaPerStage = kAInst + 3;           // plus two weight and one scale DMA instructions
  // Up to 32 rows the fragments of the next stage are read and decoded while
  // the current one is multiplied (kPipe; stages s + 2 .. s + kStages - 1 in
  // flight).  Taller tiles need the registers for accumulators: each stage's
  // fragments are decoded one column block ahead of its MFMAs, two workgroups
  // per CU overlap each other, and stages s + 1 .. s + 2 are in flight.
  constexpr bool kPipe = MT <= 32;
  // 16-row tiles of the stored orientation stream their operands into registers (no ring)
  constexpr bool kStream = !kT && MT == 16;
  constexpr int kStages = gemm_stages(MT);
  static_assert(!kPipe || (kStages >= 4 && kStages - 3 <= 4), "pipelined ring depth");
  static_assert(kPipe || kStages == 3, "ring depth");
  static_assert(gemm_ring_bytes(MT) <= kRingMax, "ring");
  // the ring holds the activation tiles of all slots, then their weight tiles,
  // then their scales, so that a slot known at compile time is an immediate offset
  constexpr int kWReg = kStages * kABytes, kSReg = kStages * (kABytes + kWBytes);

  const int e = p.tile_e[tile], m0 = p.tile_m0[tile];
  const int es = p.expert_slot[e];  // the expert's place in the scale tables
  // Values the code after the main loop needs, read here with the tile's set-up
  // (the loop's asm copies keep the compiler from moving these reads above
  // it): the power-of-two shift of the expert's scale table, and the first
  // quad-row position of the tile (the expert's tiles start at multiples of 4 rows)
  const int sshift = p.sshift[2 * e + ((KIND == kGateUp || KIND == kGateUpBwd) ? 0 : 1)];
  const int64_t qb = (int64_t)p.qoffsets[e] + (m0 - p.offsets[e]);
  const int mlen = min(MT, p.offsets[e + 1] - m0);
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, known uniform
  const int H = p.H, I = p.I, R = p.R;
  const int n0 = (KIND == kGateUp) ? nt * kHChunk : nt * kNT;
  const int nout = (KIND == kGateUp || KIND == kDownBwd) ? I : H;
  const int kdim = (KIND == kGateUp || KIND == kDownBwd) ? H : (KIND == kDown ? I : 2 * I);
  const int ngroups = kdim / kGroup;
  const int nss = (kdim + kKS - 1) / kKS;

  if (tid < MT) {
    // rows past the tile's end read the last row again; their results are dropped
    const int m = m0 + min(tid, mlen - 1);
    int src, ex;
    if constexpr (kChunked) {
      src = m;
      ex = p.a_chunkexp[(size_t)m * p.a_nch];
    } else {
      src = p.sorted_slot[m] / p.topk;
      ex = p.a_rowexp[src];
    }
    s_src[tid] = src;
    s_exp[tid] = ex;
    const int slot = p.sorted_slot[m];
    s_slot[tid] = tid < mlen ? slot : -1;
    // the route weights the epilogues of down and down dX scale by, read here
    // once so that their loads do not wait behind the epilogue's stores
    if constexpr (KIND == kDown || KIND == kDownBwd) s_rw[tid] = tid < mlen ? p.rw[slot] : 0.f;
  }
  __syncthreads();

  // ---------------------------------------------------------------- ring fill
  // weight row (stored orientation: output column lc of the tile, clamped)
  auto wrow_stored = [&](int lc) -> const uint8_t* {
    if constexpr (KIND == kGateUp) {
      const int col = min(n0 + (lc & (kHChunk - 1)), I - 1);
      return (lc < kHChunk ? p.L.wg : p.L.wu) + ((size_t)e * I + col) * (size_t)(H / 2);
    } else {
      const int col = min(n0 + lc, H - 1);
      return p.L.wd + ((size_t)e * H + col) * (size_t)(I / 2);
    }
  };
  // weight row (transposed orientation: contraction index kk, clamped)
  auto wrow_t = [&](int kk) -> const uint8_t* {
    if constexpr (KIND == kDownBwd) {
      return p.L.wd + ((size_t)e * H + kk) * (size_t)(I / 2);
    } else {
      const bool up = kk >= I;
      const size_t r = (size_t)e * I + (up ? kk - I : kk);
      return (up ? p.L.wu : p.L.wg) + r * (size_t)(H / 2);
    }
  };

  // Issue one stage: activation, weight and scale DMAs, always kDmaPerStage of
  // them per wave (the ring waits count on it).
  auto issue_any = [&](int ss) {
    const int k0 = ss * kKS;
    const int sl = ss % kStages;
    const uint32_t sa = lds_addr(ring) + sl * kABytes, sw = lds_addr(ring) + kWReg + sl * kWBytes,
                   ssc = lds_addr(ring) + kSReg + sl * kScBytes;
#pragma unroll
    for (int i = 0; i < kAInst; ++i) {
      const int u = w * kAInst + i;
      const int row = kRowsPerInst * u + ((lane >> 3) & (kRowsPerInst - 1));
      const int c = (lane & 7) ^ ((row & 7) ^ ((row >> 3) & 1));
      // activation values past the contraction's end come from the zero chunk,
      // which cancels whatever the clamped weights of the final half stage hold
      const int k = k0 + 8 * c;
      const void* g = k < kdim ? (const void*)(p.a_src + (size_t)s_src[row] * p.lda + k) : p.zero;
      if (MT != 16 || lane < 32) dma16(g, sa + 128 * kRowsPerInst * u);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = w * 2 + i;
      const uint8_t* g;
      if constexpr (kT) {
        const int row = 8 * u + (lane >> 3);
        const int c16 = (lane & 7) ^ ((row >> 1) & 7);
        const int kk = min(k0 + row, kdim - 1);
        int c = n0 + 32 * c16;
        if (c >= nout) c = n0;
        g = wrow_t(kk) + c / 2;
      } else {
        const int lc = 32 * u + (lane >> 1);
        int h = (lane & 1) ^ ((lc >> 3) & 1);
        if (k0 + 32 * h >= kdim) h = 0;
        g = wrow_stored(lc) + k0 / 2 + 16 * h;
      }
      dma16(g, sw + 1024 * u);
    }
    // scales: 1 KB per stage, a quarter per wave (16 lanes x 16 B = 8 fp16 each)
    {
      const int q = w * 16 + (lane & 15);
      const uint16_t* g;
      if constexpr (kT) {
        // column group q >> 3 of the tile, contraction rows 8 (q & 7) .. + 7 of the stage
        const int cg = min(n0 / kGroup + (q >> 3), nout / kGroup - 1);
        const int kk = min(k0 + 8 * (q & 7), kdim - 8);
        if constexpr (KIND == kDownBwd) {
          g = p.sct0 + ((size_t)es * (I / kGroup) + cg) * H + kk;
        } else {
          const bool up = kk >= I;
          g = (up ? p.sct1 : p.sct0) + ((size_t)es * (H / kGroup) + cg) * I + (up ? kk - I : kk);
        }
      } else {
        // group (q >> 5) of the stage, output columns 8 (q & 31) .. + 7 of the tile
        const int gi = min(k0 / kGroup + (q >> 5), ngroups - 1);
        const int lc = 8 * (q & 31);
        if constexpr (KIND == kGateUp) {
          const int n = min(n0 + (lc & (kHChunk - 1)), I - 8);
          g = (lc < kHChunk ? p.sct0 : p.sct1) + ((size_t)es * ngroups + gi) * I + n;
        } else {
          const int n = min(n0 + lc, H - 8);
          g = p.sct0 + ((size_t)es * ngroups + gi) * H + n;
        }
      }
      if (lane < 16) dma16(g, ssc + 256 * w);
    }
  };

  // Per-lane source addresses of the stage-0 DMAs, advanced by a wave-uniform
  // offset per stage (whole stages only; a final half stage takes issue_any).
  const uint16_t* pa[kAInst];
#pragma unroll
  for (int i = 0; i < kAInst; ++i) {
    const int u = w * kAInst + i;
    const int row = kRowsPerInst * u + ((lane >> 3) & (kRowsPerInst - 1));
    const int c = (lane & 7) ^ ((row & 7) ^ ((row >> 3) & 1));
    pa[i] = p.a_src + (size_t)s_src[row] * p.lda + 8 * c;
  }
  const uint8_t* pb[2];
  const uint8_t* pb_up[2];  // gate/up transposed: the up rows (contraction index >= I)
  int brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = w * 2 + i;
    if constexpr (kT) {
      const int row = 8 * u + (lane >> 3);
      const int c16 = (lane & 7) ^ ((row >> 1) & 7);
      int c = n0 + 32 * c16;
      if (c >= nout) c = n0;
      brow[i] = row;
      if constexpr (KIND == kDownBwd) {
        pb[i] = p.L.wd + ((size_t)e * H + row) * (size_t)(I / 2) + c / 2;
        pb_up[i] = pb[i];
      } else {
        pb[i] = p.L.wg + ((size_t)e * I + row) * (size_t)(H / 2) + c / 2;
        // up row (kk - I), addressed from kk: offset by -I rows, used only once kk >= I
        pb_up[i] = p.L.wu + ((int64_t)e * I + row - I) * (int64_t)(H / 2) + c / 2;
      }
    } else {
      const int lc = 32 * u + (lane >> 1);
      const int h = (lane & 1) ^ ((lc >> 3) & 1);
      brow[i] = 0;
      pb[i] = wrow_stored(lc) + 16 * h;
      pb_up[i] = pb[i];
    }
  }
  const uint16_t* ps;
  const uint16_t* ps_up;
  {
    const int q = w * 16 + (lane & 15);
    if constexpr (kT) {
      const int cg = min(n0 / kGroup + (q >> 3), nout / kGroup - 1);
      if constexpr (KIND == kDownBwd) {
        ps = p.sct0 + ((size_t)es * (I / kGroup) + cg) * H + 8 * (q & 7);
        ps_up = ps;
      } else {
        ps = p.sct0 + ((size_t)es * (H / kGroup) + cg) * I + 8 * (q & 7);
        ps_up = p.sct1 + ((int64_t)es * (H / kGroup) + cg) * (int64_t)I + 8 * (q & 7) - I;
      }
    } else {
      const int lc = 8 * (q & 31);
      if constexpr (KIND == kGateUp) {
        const int n = min(n0 + (lc & (kHChunk - 1)), I - 8);
        ps = (lc < kHChunk ? p.sct0 : p.sct1) + ((size_t)es * ngroups + (q >> 5)) * I + n;
      } else {
        const int n = min(n0 + lc, H - 8);
        ps = p.sct0 + ((size_t)es * ngroups + (q >> 5)) * H + n;
      }
      ps_up = ps;
    }
  }
  auto issue = [&](int ss) {
    const int k0 = ss * kKS;
    if (k0 + kKS > kdim) {
      issue_any(ss);
      return;
    }
    const int sl = ss % kStages;
    const uint32_t sa = lds_addr(ring) + sl * kABytes, sw = lds_addr(ring) + kWReg + sl * kWBytes,
                   ssc = lds_addr(ring) + kSReg + sl * kScBytes;
#pragma unroll
    for (int i = 0; i < kAInst; ++i)
      if (MT != 16 || lane < 32) dma16(pa[i] + k0, sa + 128 * kRowsPerInst * (w * kAInst + i));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint8_t* g;
      if constexpr (KIND == kDownBwd) {
        g = pb[i] + (size_t)k0 * (I / 2);
      } else if constexpr (KIND == kGateUpBwd) {
        g = (k0 + brow[i] < I ? pb[i] : pb_up[i]) + (size_t)k0 * (H / 2);
      } else {
        g = pb[i] + k0 / 2;
      }
      dma16(g, sw + 1024 * (w * 2 + i));
    }
    {
      const uint16_t* g;
      if constexpr (KIND == kDownBwd) {
        g = ps + k0;
      } else if constexpr (KIND == kGateUpBwd) {
        g = (k0 + 8 * (lane & 7) < I ? ps : ps_up) + k0;
      } else {
        g = ps + (size_t)(k0 / kGroup) * (KIND == kGateUp ? I : H);
      }
      if (lane < 16) dma16(g, ssc + 256 * w);
    }
  };

  floatx4 acc[MB][4];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int aswz = (lr & 7) ^ ((lr >> 3) & 1);  // activation swizzle of rows 16 * mb + lr
  if constexpr (kStream) {
    // -------------------------------------------------------------- main loop, streamed (16 rows)
    // Short tiles are bound by the weight stream.  Each wave loads its own
    // columns' codes and scales straight into registers, one unit ahead; the
    // activation rows, which every wave needs, are copied into an LDS ring by
    // DMA (each wave an eighth of a unit per copy) and read from there, one
    // barrier per unit.  A unit is 256 contraction values (eight quant groups);
    // in half h of unit u, lane group lg takes quant group 8 u + 4 h + lg of its
    // column: one 16-byte run of codes and one scale.  The two halves' code loads
    // go out back to back, so each weight row's 128-byte line is requested
    // whole.  K-step j of a half multiplies values 8 j .. 8 j + 7 of every lane
    // group's run on both sides, which reorders the contraction but not its
    // terms.
    static_assert(MT == 16, "the streamed path holds one row block");
    constexpr int kNA = 4;              // LDS slots
    constexpr int kSlot = MT * 512;     // one unit of activations: MT rows of 256 fp16 values
    constexpr int kAIW = MT / 8;        // activation copies per wave per unit (two rows each)
    constexpr int kCodeVm = 16;         // vector memory instructions of one unit's codes and scales
    static_assert(kNA * kSlot <= kRingMax, "activation ring");
    const int nunits = (ngroups + 7) / 8;
    const int ncol = KIND == kGateUp ? I : H;  // columns of the projection: the scale table's row length
    const uint8_t* wp[4];
    const uint16_t* sp[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int lc = local_col<KIND>(w, f) + lr;
      wp[f] = wrow_stored(lc);
      int n;
      const uint16_t* tbl;
      if constexpr (KIND == kGateUp) {
        n = min(n0 + (lc & (kHChunk - 1)), I - 1);
        tbl = lc < kHChunk ? p.sct0 : p.sct1;
      } else {
        n = min(n0 + lc, H - 1);
        tbl = p.sct0;
      }
      sp[f] = tbl + (size_t)es * ngroups * ncol + perm_pos(n);  // column n of group 0
    }
    // Activation copies: copy i of wave w covers tile rows 2 (kAIW w + i) and the
    // next; lane l writes slot position 16 l, i.e. row + (l >> 5), position
    // l & 31, which holds chunk (l & 31) ^ (row & 7) of the unit (the XOR spreads
    // a k-step's fragment reads over the banks).  Values past the contraction's
    // end come from the zero chunk.
    const uint16_t* asrc[kAIW];
    int achunk[kAIW];
#pragma unroll
    for (int i = 0; i < kAIW; ++i) {
      const int row = 2 * (kAIW * w + i) + (lane >> 5);
      achunk[i] = (lane & 31) ^ (row & 7);
      asrc[i] = p.a_src + (size_t)s_src[row] * p.lda + 8 * achunk[i];
    }
    auto issue_acts = [&](int u, int slot) {
#pragma unroll
      for (int i = 0; i < kAIW; ++i) {
        const bool ok = 256 * u + 8 * achunk[i] < kdim;
        dma16(ok ? (const void*)(asrc[i] + 256 * u) : p.zero, lds_addr(ring) + slot * kSlot + 1024 * (kAIW * w + i));
      }
    };
    struct Codes {
      u32x4 w[4][2];     // codes of the lane's quant group, per column block and half
      uint32_t s[4][2];  // its scale (fp16 bits), per column block and half
    };
    // Every unit's codes load the same way (no branch, so that the compiler
    // cannot merge or sink them toward the MFMAs that use them): lane groups past
    // the last quant group, and the unit past the contraction's end that the last
    // step loads, read clamped codes and scales (the former meet zero
    // activations and add nothing; the latter are never multiplied).
    auto load_codes = [&](int u, Codes& C) {
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int gc = min(8 * u + 4 * h + lg, ngroups - 1);
          C.w[f][h] = *reinterpret_cast<const u32x4*>(wp[f] + 16 * (size_t)gc);
        }
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int gc = min(8 * u + 4 * h + lg, ngroups - 1);
          C.s[f][h] = sp[f][(size_t)gc * ncol];
        }
    };
    const DecodeConsts dc = decode_consts();
    auto compute = [&](const Codes& C, int slot) {
      const uint8_t* st = ring + slot * kSlot + lr * 512;
      u32x4 a[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          a[h][j] = *reinterpret_cast<const u32x4*>(st + 16 * ((16 * h + 4 * lg + j) ^ (lr & 7)));
      uint32_t s0[4][2], s1[4][2];  // per column block and half: 16 s, -24 s (RAWINT4) or the fp32 scale (MXFP4)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const half2_t s2 = __builtin_bit_cast(half2_t, C.s[f][h] | (C.s[f][h] << 16));
          if constexpr (MX) {
            s0[f][h] = __float_as_uint((float)s2.x);
            s1[f][h] = 0u;
          } else {
            s0[f][h] = __builtin_bit_cast(uint32_t, s2 * (half2_t){16.f16, 16.f16});
            s1[f][h] = __builtin_bit_cast(uint32_t, s2 * (half2_t){-24.f16, -24.f16});
          }
        }
      // per accumulator the terms come in the order (h, j); consecutive MFMAs
      // go to different accumulators
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            u32x4 b;
            if constexpr (MX)
              b = decode_dword_e2m1(C.w[f][h][j], __uint_as_float(s0[f][h]));
            else
              b = decode_dword_fma(C.w[f][h][j], __builtin_bit_cast(half2_t, s0[f][h]),
                                   __builtin_bit_cast(half2_t, s1[f][h]), dc);
            acc[0][f] = mfma_f16(a[h][j], b, acc[0][f]);
          }
    };
    // Unit u (slot u % 4): load the codes of unit u + 1, then wait until only
    // those are in flight: unit u's codes and unit u + 1's activation copies
    // (issued one unit ago) have landed.  The wait is one the compiler sees, so
    // it adds none of its own for the codes (it does not count the copies, which
    // are issued from asm so that it does not drain them before every LDS read).
    // Barrier: every wave's copies of unit u + 1 are visible, and every wave is
    // done with slot u + 2, which is refilled next with unit u + 2's activations.
    // Then unit u is multiplied.
    Codes C[2];
    issue_acts(0, 0);
    load_codes(0, C[0]);
    compiler_fence();
    wait_vm_lgkm<0>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (nunits > 1) issue_acts(1, 1);
    for (int u0 = 0; u0 < nunits; u0 += 2) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int u = u0 + d;
        load_codes(u + 1, C[d ^ 1]);
        compiler_fence();
        wait_vm_lgkm<kCodeVm>();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        if (u + 2 < nunits) issue_acts(u + 2, (u + 2) % kNA);  // (no copy is left in flight at the end)
        __builtin_amdgcn_sched_barrier(0);
        if (u < nunits) compute(C[d], u % kNA);  // (an odd count leaves the loop's last unit empty)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i)
      if (i < nss) issue(i);

    // ---------------------------------------------------------------- main loop (fp16)
    const int a_off0 = lr * 128 + 16 * ((2 * lg) ^ aswz);
    const int a_off1 = lr * 128 + 16 * ((2 * lg + 1) ^ aswz);
    // Weight fragments of one stage: codes and scales read from its slot and
    // decoded to fp16.  (In a final half stage the values past the contraction's
    // end are clamped copies; the zero activations there cancel them.)
    const DecodeConsts dc = decode_consts();
    auto decode = [&](int sl, u32x4 (&bf)[2][4]) {
      const uint8_t* Bs = ring + kWReg + sl * kWBytes;
      const uint16_t* Sc = reinterpret_cast<const uint16_t*>(ring + kSReg + sl * kScBytes);
      if constexpr (kT) {
        v2i_t tr[4];
        u32x4 sp[2][4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int lc = local_col<KIND>(w, f);
          const int slot = (lc >> 5) ^ ((lr >> 1) & 7);
          tr[f] = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
              (lds_v2i_ptr)(Bs + (16 * lg + lr) * 128 + 16 * slot + 8 * ((lc >> 4) & 1)));
#pragma unroll
          for (int j = 0; j < 2; ++j)  // 8 fp16 scales written as 16-bit values: copy, do not type-pun
            __builtin_memcpy(&sp[j][f], &Sc[(lc >> 5) * kKS + 16 * lg + 8 * j], sizeof(u32x4));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            const uint32_t word = j ? (uint32_t)tr[f].y : (uint32_t)tr[f].x;
            // bit-cast whole scalars: clang's bit_cast of an ext-vector component reads component 0
            const uint32_t s0 = sp[j][f].x, s1 = sp[j][f].y, s2 = sp[j][f].z, s3 = sp[j][f].w;
            if constexpr (MX)
              bf[j][f] = decode_dword_perm_e2m1(word, __builtin_bit_cast(half2_t, s0), __builtin_bit_cast(half2_t, s1),
                                                __builtin_bit_cast(half2_t, s2), __builtin_bit_cast(half2_t, s3));
            else
              bf[j][f] = decode_dword_perm(word, __builtin_bit_cast(half2_t, s0), __builtin_bit_cast(half2_t, s1),
                                           __builtin_bit_cast(half2_t, s2), __builtin_bit_cast(half2_t, s3), dc);
          }
      } else {
        uint32_t raw[4][2];
        uint32_t bs[4];
        const int bsw = 16 * ((lg >> 1) ^ ((lr >> 3) & 1)) + 8 * (lg & 1);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int lc = local_col<KIND>(w, f) + lr;
          const uint2 v = *reinterpret_cast<const uint2*>(Bs + lc * 32 + bsw);
          raw[f][0] = v.x;
          raw[f][1] = v.y;
          const uint32_t sh = Sc[(lg >> 1) * kNT + local_col<KIND>(w, f) + perm_pos(lr)];
          bs[f] = sh | (sh << 16);
        }
        if constexpr (MX) {
          float sf[4];
#pragma unroll
          for (int f = 0; f < 4; ++f) sf[f] = (float)__builtin_bit_cast(half2_t, bs[f]).x;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int f = 0; f < 4; ++f) bf[j][f] = decode_dword_e2m1(raw[f][j], sf[f]);
        } else {
          half2_t s16[4], b24[4];
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            const half2_t s2 = __builtin_bit_cast(half2_t, bs[f]);
            s16[f] = s2 * (half2_t){16.f16, 16.f16};
            b24[f] = s2 * (half2_t){-24.f16, -24.f16};
          }
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int f = 0; f < 4; ++f) bf[j][f] = decode_dword_fma(raw[f][j], s16[f], b24[f], dc);
        }
      }
    };
    // Stored orientation, one stage's weight operands split in two: the codes and
    // scales read from the slot (stored_raw), and one fragment decoded from them
    // (stored_dec), so that a fragment can be decoded right before its MFMAs.
    auto stored_raw = [&](int sl, uint32_t (&cw)[4][2], uint32_t (&sw)[4][2]) {
      const uint8_t* Bs = ring + kWReg + sl * kWBytes;
      const uint16_t* Sc = reinterpret_cast<const uint16_t*>(ring + kSReg + sl * kScBytes);
      const int bsw = 16 * ((lg >> 1) ^ ((lr >> 3) & 1)) + 8 * (lg & 1);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int lc = local_col<KIND>(w, f) + lr;
        const uint2 v = *reinterpret_cast<const uint2*>(Bs + lc * 32 + bsw);
        cw[f][0] = v.x;
        cw[f][1] = v.y;
        const uint32_t sh = Sc[(lg >> 1) * kNT + local_col<KIND>(w, f) + perm_pos(lr)];
        const half2_t s2 = __builtin_bit_cast(half2_t, sh | (sh << 16));
        if constexpr (MX) {
          sw[f][0] = __float_as_uint((float)s2.x);
          sw[f][1] = 0u;
        } else {
          sw[f][0] = __builtin_bit_cast(uint32_t, s2 * (half2_t){16.f16, 16.f16});
          sw[f][1] = __builtin_bit_cast(uint32_t, s2 * (half2_t){-24.f16, -24.f16});
        }
      }
    };
    auto stored_dec = [&](const uint32_t (&cw)[4][2], const uint32_t (&sw)[4][2], int j, int f) -> u32x4 {
      if constexpr (MX)
        return decode_dword_e2m1(cw[f][j], __uint_as_float(sw[f][0]));
      else
        return decode_dword_fma(cw[f][j], __builtin_bit_cast(half2_t, sw[f][0]), __builtin_bit_cast(half2_t, sw[f][1]),
                                dc);
    };
    // activation fragments of one stage from its slot
    auto read_a = [&](int sl, u32x4 (&af)[2][MB]) {
      const uint8_t* st = ring + sl * kABytes;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          af[j][mb] = *reinterpret_cast<const u32x4*>(st + mb * 2048 + (j ? a_off1 : a_off0));
    };
    // MFMAs of one stage, both operands already in registers
    auto mma = [&](const u32x4 (&af)[2][MB], const u32x4 (&bf)[2][4]) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[mb][f] = mfma_f16(af[j][mb], bf[j][f], acc[mb][f]);
    };
    // Stage ss: wait until stage ss + 1 has landed (each wave waits for its own
    // DMAs, the barrier for everyone's; it also frees the slot of stage ss - 1),
    // refill that slot with stage ss + kStages - 1, then run stage ss's MFMAs from
    // registers while stage ss + 1's activation fragments and weight codes are
    // read and its weights decoded.
    auto step = [&](int ss, const u32x4 (&acur)[2][MB], const u32x4 (&bcur)[2][4], u32x4 (&anxt)[2][MB],
                    u32x4 (&bnxt)[2][4]) {
      compiler_fence();
      if (ss + 1 < nss) wait_stages<kDmaPerStage>(min(kStages - 3, nss - 2 - ss));  // stages issued after ss + 1
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      if (ss + kStages - 1 < nss) issue(ss + kStages - 1);
      const int sn = min(ss + 1, nss - 1);  // (re-reads the last stage at the end; unused)
      read_a(sn % kStages, anxt);
      decode(sn % kStages, bnxt);
      mma(acur, bcur);
      // keep the next stage's reads and decode in this block, next to these
      // MFMAs, rather than letting them sink into the block that consumes them
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int f = 0; f < 4; ++f) asm volatile("" : "+v"(bnxt[j][f]));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+v"(anxt[j][mb]));
      }
    };

    if constexpr (kPipe) {
      u32x4 afa[2][MB], afb[2][MB], bfa[2][4], bfb[2][4];
      {
        // stage 0 landed: the stages issued after it may still be in flight
        compiler_fence();
        wait_stages<kDmaPerStage>(min(kStages - 2, nss - 1));
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        read_a(0, afa);
        decode(0, bfa);
      }
      int ss = 0;
      for (; ss + 1 < nss; ss += 2) {
        step(ss, afa, bfa, afb, bfb);
        step(ss + 1, afb, bfb, afa, bfa);
      }
      if (ss < nss) step(ss, afa, bfa, afb, bfb);
    } else {
      // unrolled by the ring depth, so that each stage's slot is a constant
      for (int s0 = 0; s0 < nss; s0 += kStages) {
#pragma unroll
        for (int sl = 0; sl < kStages; ++sl) {
          const int ss = s0 + sl;
          if (ss >= nss) break;
          // this wave's loads of stage ss have landed once at most the later
          // stages' DMAs are outstanding; the barrier makes every wave's loads
          // visible and frees the slot that stage ss + kStages - 1 refills
          compiler_fence();
          if (ss + 1 < nss)
            wait_vm_lgkm<kDmaPerStage>();
          else
            wait_vm_lgkm<0>();
          __builtin_amdgcn_s_barrier();
          compiler_fence();
          if (ss + kStages - 1 < nss) issue(ss + kStages - 1);
          if constexpr (kT) {
            // As below for the stored orientation: fragment (j, f) is decoded
            // during the MFMAs of the fragment before it, from codes read once
            // per stage (a transposing read per column block) and its 8 fp16
            // scales, which are read one fragment ahead of their decode.
            const uint8_t* Bs = ring + kWReg + sl * kWBytes;
            const uint16_t* Sc = reinterpret_cast<const uint16_t*>(ring + kSReg + sl * kScBytes);
            v2i_t tr[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
              const int lc = local_col<KIND>(w, f);
              const int slot = (lc >> 5) ^ ((lr >> 1) & 7);
              tr[f] = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                  (lds_v2i_ptr)(Bs + (16 * lg + lr) * 128 + 16 * slot + 8 * ((lc >> 4) & 1)));
            }
            // scales of fragment q = 4 j + f: its column group, contraction rows 16 lg + 8 j ..
            auto scl = [&](int q) {
              u32x4 v;  // 8 fp16 scales written as 16-bit values: copy, do not type-pun
              __builtin_memcpy(&v, &Sc[(local_col<KIND>(w, q & 3) >> 5) * kKS + 16 * lg + 8 * (q >> 2)], sizeof(u32x4));
              return v;
            };
            auto dec = [&](int q, const u32x4 sp) -> u32x4 {
              const uint32_t word = (q >> 2) ? (uint32_t)tr[q & 3].y : (uint32_t)tr[q & 3].x;
              // bit-cast whole scalars: clang's bit_cast of an ext-vector component reads component 0
              const uint32_t s0 = sp.x, s1 = sp.y, s2 = sp.z, s3 = sp.w;
              if constexpr (MX)
                return decode_dword_perm_e2m1(word, __builtin_bit_cast(half2_t, s0), __builtin_bit_cast(half2_t, s1),
                                              __builtin_bit_cast(half2_t, s2), __builtin_bit_cast(half2_t, s3));
              else
                return decode_dword_perm(word, __builtin_bit_cast(half2_t, s0), __builtin_bit_cast(half2_t, s1),
                                         __builtin_bit_cast(half2_t, s2), __builtin_bit_cast(half2_t, s3), dc);
            };
            const uint8_t* st = ring + sl * kABytes;
            u32x4 af[MB], an[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) af[mb] = *reinterpret_cast<const u32x4*>(st + mb * 2048 + a_off0);
            u32x4 b = dec(0, scl(0));
            u32x4 sn = scl(1);
            __builtin_amdgcn_s_setprio(2);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
              for (int f = 0; f < 4; ++f) {
                const int q = 4 * j + f;
                const bool more = q < 7;
                u32x4 bn = b, sn2 = sn;
                if (more) bn = dec(q + 1, sn);
                if (q + 2 < 8) sn2 = scl(q + 2);
                constexpr int kHalf = (MB + 1) / 2;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                  acc[mb][f] = mfma_f16(af[mb], b, acc[mb][f]);
                  const int r = f == 2 ? mb : kHalf + mb;  // activation fragment read in this slot
                  const bool rd = j == 0 && f >= 2 && mb < kHalf && r < MB;
                  if (rd) an[r] = *reinterpret_cast<const u32x4*>(st + r * 2048 + a_off1);
                  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                  if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                  if (mb == 0 && q + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the scales
                  if (more) __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two decode VALU
                }
                b = bn;
                sn = sn2;
              }
              if (j == 0) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) af[mb] = an[mb];
              }
            }
            __builtin_amdgcn_s_setprio(0);
          } else {
            // The stage's codes, scales and first activation fragments are
            // read, then each column block's fragment is decoded while the
            // MFMAs of the one before it run, so that one wave keeps the
            // matrix pipe fed by itself (the other wave on the SIMD fills in;
            // the raised priority gives the MFMAs the SIMD first).  The next
            // k-step's activation fragments are read during the current one's
            // last two column blocks.
            uint32_t cw[4][2], sw[4][2];
            stored_raw(sl, cw, sw);
            const uint8_t* st = ring + sl * kABytes;
            u32x4 af[MB], an[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) af[mb] = *reinterpret_cast<const u32x4*>(st + mb * 2048 + a_off0);
            u32x4 b = stored_dec(cw, sw, 0, 0);
            __builtin_amdgcn_s_setprio(2);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
              for (int f = 0; f < 4; ++f) {
                const bool more = f < 3 || j == 0;
                u32x4 bn = b;
                if (more) bn = stored_dec(cw, sw, f < 3 ? j : 1, f < 3 ? f + 1 : 0);
                constexpr int kHalf = (MB + 1) / 2;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                  acc[mb][f] = mfma_f16(af[mb], b, acc[mb][f]);
                  const int r = f == 2 ? mb : kHalf + mb;  // activation fragment read in this slot
                  const bool rd = j == 0 && f >= 2 && mb < kHalf && r < MB;
                  if (rd) an[r] = *reinterpret_cast<const u32x4*>(st + r * 2048 + a_off1);
                  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                  if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                  if (more) __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two decode VALU
                }
                b = bn;
              }
              if (j == 0) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) af[mb] = an[mb];
              }
            }
            __builtin_amdgcn_s_setprio(0);
          }
        }
      }
    }
  }
  __syncthreads();  // every wave is done with the ring before it is reused

  // The scale tables hold scale * 2^-s for an expert whose scales lie outside
  // the exact domain (s = 0 otherwise): the sums get 2^s back before the LoRA terms.
  {
    const int sh = sshift;
    if (sh != 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mb][f][i] = ldexpf(acc[mb][f][i], sh);
    }
  }

  // ---------------------------------------------------------------- LoRA K-steps (bf16 hi/lo)
  // One group of the LoRA contraction at a time, both operands staged in the
  // (now idle) ring: the side product arrives as bf16 hi/lo planes already
  // times the LoRA scale and the row's exponent and is copied by DMA into the activation
  // layout (hi chunks 0..3, lo chunks 4..7); the fp32 LoRA matrix entries are
  // split into bf16 hi/lo.  For gate/up the two halves of the contraction
  // (x A_g^T | x A_u^T) meet only their own half of the columns.  Rank 0 (an
  // inference of the base alone) has no LoRA steps.
  if (R > 0) {
    constexpr bool kTwoHalves = (KIND == kGateUp || KIND == kGateUpBwd);
    const int RP = (R + kGroup - 1) / kGroup * kGroup;  // one padded half
    const int KLP = kTwoHalves ? 2 * RP : RP;
    // plane columns at or past R within the half hold no product: mask them (they may be stale)
    auto keep_mask = [&](int qh) {
      const int nval = min(max(R - (qh + 8 * lg), 0), 8);
      u32x4 keep;
      keep.x = (nval > 0 ? 0xffffu : 0u) | (nval > 1 ? 0xffff0000u : 0u);
      keep.y = (nval > 2 ? 0xffffu : 0u) | (nval > 3 ? 0xffff0000u : 0u);
      keep.z = (nval > 4 ? 0xffffu : 0u) | (nval > 5 ? 0xffff0000u : 0u);
      keep.w = (nval > 6 ? 0xffffu : 0u) | (nval > 7 ? 0xffff0000u : 0u);
      return keep;
    };
    // the lane index as a value the compiler cannot see through: the copy
    // addresses below are then computed here, not hoisted above the main loop
    // where their registers would compete with its fragments
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    // side-product planes of the group starting at q0 into la (activation layout)
    auto copy_planes = [&](int q0, uint8_t* la) {
#pragma unroll
      for (int i = 0; i < kAInst; ++i) {
        const int u = w * kAInst + i;
        const int row = kRowsPerInst * u + ((lane >> 3) & (kRowsPerInst - 1));
        const int c = (lane & 7) ^ ((row & 7) ^ ((row >> 3) & 1));
        const size_t m = (size_t)(m0 + min(row, mlen - 1));
        const uint16_t* g = p.lsplit + m * (size_t)(2 * KLP) + (c >> 2) * KLP + q0 + 8 * (c & 3);
        if (MT != 16 || lane < 32) dma16(g, lds_addr(la) + 128 * kRowsPerInst * u);
      }
    };
    if constexpr (LDMA) {
      // 16-value sub-groups on 16x16x16 bf16 MFMAs.  Each sub-group's side-product
      // planes and the matching fp32 block of the LoRA matrix (whole 16-byte runs,
      // zeros past the rank or in the other half) are copied by DMA into one of
      // two buffers, so the next sub-group's copies run under this one's MFMAs;
      // the matrix is split into bf16 hi/lo as its fragments are read.
      constexpr int kLA = MT * 64;  // planes of one sub-group: [MT][hi 16 | lo 16] bf16
      constexpr int kLB = 16384;    // fp32 matrix block: [256 columns][16] or [16][256 columns]
      constexpr int kLBuf = 3;      // sub-groups in the ring: s + 1 and s + 2 are in flight while s is multiplied
      static_assert(kLBuf * (kLA + kLB) <= kRingMax, "LoRA staging");
      constexpr int kRPI = MT >= 64 ? 16 : MT / 4;  // rows per plane copy (4 lanes per row)
      constexpr int kPC = MT / kRPI;                // plane copies per sub-group
      constexpr int kPI = (kPC + 3) / 4;            // plane copies per wave per sub-group
      static_assert(kPC * kRPI == MT && kPC <= 4 * kPI && 4 * kPI - kPC <= kPC, "plane copies");
      // only the sub-groups that hold contraction values below the rank: a half
      // is padded to a multiple of 32, and the padding contributes nothing
      const int nsgh = (R + 15) / 16;               // sub-groups per half
      const int nsg = (kTwoHalves ? 2 : 1) * nsgh;  // sub-groups in all
      auto sg_q0 = [&](int sg) { return (sg / nsgh) * RP + 16 * (sg % nsgh); };
      auto issue_lora = [&](int sg) {
        const int q0 = sg_q0(sg), half = q0 >= RP ? 1 : 0, qh = q0 - half * RP;
        const int b = sg % kLBuf;
        const uint32_t la = lds_addr(ring) + b * kLA, lb = lds_addr(ring) + kLBuf * kLA + b * kLB;
        // planes: 4 lanes per row, chunk c (0, 1 hi; 2, 3 lo) at c ^ ((row >> 1) & 3)
#pragma unroll
        for (int i = 0; i < kPI; ++i) {
          // every wave issues kPI copies (the waits count on it); past the last
          // copy a wave repeats one of the final copies (same bytes, same place)
          const int u0 = w * kPI + i, u = u0 < kPC ? u0 : u0 - (4 * kPI - kPC);
          const int row = kRPI * u + (lane >> 2);
          const int c = (lane & 3) ^ ((row >> 1) & 3);
          const size_t m = (size_t)(m0 + min(row, mlen - 1));
          const uint16_t* g = p.lsplit + m * (size_t)(2 * KLP) + (c >> 1) * KLP + q0 + 8 * (c & 1);
          if (lane < 4 * kRPI) dma16(g, la + 64 * kRPI * u);
        }
        // matrix: 4 copies of 1 KB per wave
#pragma unroll 1
        for (int i = 0; i < 4; ++i) {
          const int u = w * 4 + i;
          const void* src;
          if constexpr (!kT) {
            // columns 16u .. 16u + 15, 4 lanes per column, chunk c (values 4c .. 4c + 3) at c ^ (column & 3)
            const int lc = 16 * u + (lane >> 2);
            const int c = (lane & 3) ^ (lc & 3);
            const float* mat;
            int n, nrows;
            bool in_half = true;
            if constexpr (KIND == kGateUp) {
              // copies 0..7 (waves 0, 1) hold gate columns, 8..15 (waves 2, 3) up columns
              const bool up = w >= 2;
              mat = up ? p.L.bu : p.L.bg;
              n = n0 + 16 * (u & 7) + (lane >> 2);
              nrows = I;
              in_half = up == (half == 1);
            } else {
              mat = p.L.bd;
              n = n0 + lc;
              nrows = H;
            }
            const int q = qh + 4 * c;
            src = (in_half && q < R && n < nrows) ? (const void*)(mat + ((size_t)e * nrows + n) * R + q) : p.zero;
          } else {
            // contraction row u of the sub-group, columns 4l .. 4l + 3
            const int q = qh + u, c = n0 + 4 * lane;
            const float* mat;
            int ncols;
            if constexpr (KIND == kDownBwd) {
              mat = p.L.ad;
              ncols = I;
            } else {
              mat = half ? p.L.au : p.L.ag;
              ncols = H;
            }
            src = (q < R && c < nout) ? (const void*)(mat + ((size_t)e * R + q) * ncols + c) : p.zero;
          }
          dma16(src, lb + 1024 * u);
        }
      };
      issue_lora(0);
      if (nsg > 1) issue_lora(1);
      for (int sg = 0; sg < nsg; ++sg) {
        const int q0 = sg_q0(sg), half = q0 >= RP ? 1 : 0, qh = q0 - half * RP;
        // sub-group sg has landed once at most sub-group sg + 1's copies are outstanding
        compiler_fence();
        if (sg + 1 < nsg)
          wait_vm_lgkm<kPI + 4>();
        else
          wait_vm_lgkm<0>();
        __builtin_amdgcn_s_barrier();  // also: every wave is done with the buffers sub-group sg + 2 refills
        compiler_fence();
        if (sg + 2 < nsg) issue_lora(sg + 2);
        const uint8_t* la = ring + (sg % kLBuf) * kLA;
        const uint8_t* lb = ring + kLBuf * kLA + (sg % kLBuf) * kLB;
        // column blocks f in [F0, F1): gate/up's gate half meets only the gate
        // columns (f 0, 1) and its up half only the up columns (f 2, 3), the
        // other half's B entries being zero; every other kind meets all four
        auto steps = [&](auto f0_tag) {
          constexpr int F0 = decltype(f0_tag)::value, F1 = KIND == kGateUp ? F0 + 2 : 4;
          if constexpr (KIND != kGateUp) {
            // One 16x16x32 MFMA per fragment pair: the contraction runs over the
            // sub-group's 16 values twice, [hi | lo] of the side product against
            // the matrix entries rounded to bf16 (nearest) twice, which sums
            // (hi + lo) * m.  Lane group lg holds values 8 (lg & 1) .. + 7, of
            // the hi plane for lg < 2 and of the lo plane otherwise.
            u32x4 bm[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
              const int col = local_col<KIND>(w, f) + lr;
              float v[8];
              if constexpr (!kT) {
                const int c0 = 2 * (lg & 1);
                const float4 x0 = *reinterpret_cast<const float4*>(lb + col * 64 + 16 * (c0 ^ (col & 3)));
                const float4 x1 = *reinterpret_cast<const float4*>(lb + col * 64 + 16 * ((c0 + 1) ^ (col & 3)));
                v[0] = x0.x, v[1] = x0.y, v[2] = x0.z, v[3] = x0.w, v[4] = x1.x, v[5] = x1.y, v[6] = x1.z,
                v[7] = x1.w;
              } else {
                const float* fb = reinterpret_cast<const float*>(lb);
#pragma unroll
                for (int t = 0; t < 8; ++t) v[t] = fb[(8 * (lg & 1) + t) * 256 + col];
              }
              uint32_t pk[4];
#pragma unroll
              for (int t = 0; t < 4; ++t)
                pk[t] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){v[2 * t], v[2 * t + 1]}, bf16x2_t));
              bm[f] = u32x4{pk[0], pk[1], pk[2], pk[3]};
            }
            // plane values at or past R within the half hold no product (they may be stale): mask them
            const int nval = min(max(R - (qh + 8 * (lg & 1)), 0), 8);
            u32x4 keep;
            keep.x = (nval > 0 ? 0xffffu : 0u) | (nval > 1 ? 0xffff0000u : 0u);
            keep.y = (nval > 2 ? 0xffffu : 0u) | (nval > 3 ? 0xffff0000u : 0u);
            keep.z = (nval > 4 ? 0xffffu : 0u) | (nval > 5 ? 0xffff0000u : 0u);
            keep.w = (nval > 6 ? 0xffffu : 0u) | (nval > 7 ? 0xffff0000u : 0u);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              const int row = 16 * mb + lr, sw = (row >> 1) & 3;
              const u32x4 ap = *reinterpret_cast<const u32x4*>(la + row * 64 + 16 * (lg ^ sw)) & keep;
#pragma unroll
              for (int f = 0; f < 4; ++f) acc[mb][f] = mfma_bf16(ap, bm[f], acc[mb][f]);
            }
          } else {
            // Gate/up (the pre-activations the masks are decided on): the matrix
            // entries m are split by truncation into bf16 mh + ml, and two MFMAs
            // form the same three products as hi*mh + hi*ml + lo*mh: one 16x16x32
            // over [hi | lo] against [mh | mh] (lane group lg: values 8 (lg & 1) .. + 7),
            // and one 16x16x16 of hi against ml, whose lane group lg holds the
            // values 8 (lg & 1) + 4 (lg >> 1) .. + 3 (a subset of the same lane's).
            u32x4 bm[4];
            u32x2 bml[4];
#pragma unroll
            for (int f = F0; f < F1; ++f) {
              const int col = local_col<KIND>(w, f) + lr;
              const int c0 = 2 * (lg & 1);
              const float4 x0 = *reinterpret_cast<const float4*>(lb + col * 64 + 16 * (c0 ^ (col & 3)));
              const float4 x1 = *reinterpret_cast<const float4*>(lb + col * 64 + 16 * ((c0 + 1) ^ (col & 3)));
              u32x2 h0, l0, h1, l1;
              split4_trunc(x0, h0, l0);
              split4_trunc(x1, h1, l1);
              bm[f] = u32x4{h0.x, h0.y, h1.x, h1.y};
              bml[f] = (lg >> 1) ? l1 : l0;
            }
            // plane values at or past R within the half hold no product (they may be stale): mask them
            const int q8 = qh + 8 * (lg & 1);
            const int nval = min(max(R - q8, 0), 8), nval4 = min(max(R - (q8 + 4 * (lg >> 1)), 0), 4);
            u32x4 keep;
            keep.x = (nval > 0 ? 0xffffu : 0u) | (nval > 1 ? 0xffff0000u : 0u);
            keep.y = (nval > 2 ? 0xffffu : 0u) | (nval > 3 ? 0xffff0000u : 0u);
            keep.z = (nval > 4 ? 0xffffu : 0u) | (nval > 5 ? 0xffff0000u : 0u);
            keep.w = (nval > 6 ? 0xffffu : 0u) | (nval > 7 ? 0xffff0000u : 0u);
            const u32x2 keep4 = {(nval4 > 0 ? 0xffffu : 0u) | (nval4 > 1 ? 0xffff0000u : 0u),
                                 (nval4 > 2 ? 0xffffu : 0u) | (nval4 > 3 ? 0xffff0000u : 0u)};
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              const int row = 16 * mb + lr, sw = (row >> 1) & 3;
              const u32x4 ap = *reinterpret_cast<const u32x4*>(la + row * 64 + 16 * (lg ^ sw)) & keep;
              const u32x2 ah =
                  *reinterpret_cast<const u32x2*>(la + row * 64 + 16 * ((lg & 1) ^ sw) + 8 * (lg >> 1)) & keep4;
#pragma unroll
              for (int f = F0; f < F1; ++f) {
                acc[mb][f] = mfma_bf16(ap, bm[f], acc[mb][f]);
                acc[mb][f] = mfma_bf16_k16(ah, bml[f], acc[mb][f]);
              }
            }
          }
        };
        if constexpr (KIND == kGateUp) {
          if (half)
            steps(FTag<2>{});
          else
            steps(FTag<0>{});
        } else {
          steps(FTag<0>{});
        }
      }
    } else {
      uint8_t* la = ring;            // [MT][8 chunks of 16 B], activation swizzle
      uint8_t* lb = ring + kABytes;  // stored: [256 columns][8 chunks]; transposed: hi, lo planes [32][kLBP]
    for (int q0 = 0; q0 < KLP; q0 += kGroup) {
      const int half = q0 >= RP ? 1 : 0;
      const int qh = q0 - half * RP;  // first contraction index of the group within its half
#pragma unroll
      for (int i = 0; i < kAInst; ++i) {
        const int u = w * kAInst + i;
        const int row = kRowsPerInst * u + ((lane >> 3) & (kRowsPerInst - 1));
        const int c = (lane & 7) ^ ((row & 7) ^ ((row >> 3) & 1));
        const size_t m = (size_t)(m0 + min(row, mlen - 1));
        const uint16_t* g = p.lsplit + m * (size_t)(2 * KLP) + (c >> 2) * KLP + q0 + 8 * (c & 3);
        if (MT != 16 || lane < 32) dma16(g, lds_addr(la) + 128 * kRowsPerInst * u);
      }
      if constexpr (!kT) {
        // thread -> output column lc = tid, the group's 32 entries of its row
        const int lc = tid;
        const float* brow;
        bool ok = true;
        if constexpr (KIND == kGateUp) {
          const int n = min(n0 + (lc & (kHChunk - 1)), I - 1);
          brow = (lc < kHChunk ? p.L.bg : p.L.bu) + ((size_t)e * I + n) * R;
          ok = (lc < kHChunk) == (half == 0);
        } else {
          const int n = min(n0 + lc, H - 1);
          brow = p.L.bd + ((size_t)e * H + n) * R;
        }
        const int sw = (lc & 7) ^ ((lc >> 3) & 1);
#pragma unroll 1
        for (int c8 = 0; c8 < 4; ++c8) {
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int q = qh + 8 * c8 + i;
            const float x = brow[min(q, R - 1)];
            v[i] = (ok && q < R) ? x : 0.f;
          }
          u32x4 hi, lo;
          split8(v, hi, lo);
          *reinterpret_cast<u32x4*>(lb + lc * 128 + 16 * (c8 ^ sw)) = hi;
          *reinterpret_cast<u32x4*>(lb + lc * 128 + 16 * ((4 + c8) ^ sw)) = lo;
        }
      } else {
        // thread -> contraction row qi of the group, 32 consecutive output columns
        const int qi = tid >> 3, c32 = 32 * (tid & 7);
        const int q = qh + qi;
        const int c = n0 + c32 < nout ? n0 + c32 : n0;
        const float* src;
        if constexpr (KIND == kDownBwd)
          src = p.L.ad + ((size_t)e * R + min(q, R - 1)) * I + c;
        else
          src = (half ? p.L.au : p.L.ag) + ((size_t)e * R + min(q, R - 1)) * H + c;
#pragma unroll 1
        for (int c8 = 0; c8 < 4; ++c8) {
          const float4 x0 = *reinterpret_cast<const float4*>(src + 8 * c8);
          const float4 x1 = *reinterpret_cast<const float4*>(src + 8 * c8 + 4);
          const bool ok = q < R;
          const float v[8] = {ok ? x0.x : 0.f, ok ? x0.y : 0.f, ok ? x0.z : 0.f, ok ? x0.w : 0.f,
                              ok ? x1.x : 0.f, ok ? x1.y : 0.f, ok ? x1.z : 0.f, ok ? x1.w : 0.f};
          u32x4 hi, lo;
          split8(v, hi, lo);
          *reinterpret_cast<u32x4*>(lb + qi * kLBP + 2 * (c32 + 8 * c8)) = hi;
          *reinterpret_cast<u32x4*>(lb + 32 * kLBP + qi * kLBP + 2 * (c32 + 8 * c8)) = lo;
        }
      }
      compiler_fence();
      wait_vm_lgkm<0>();
      __builtin_amdgcn_s_barrier();
      compiler_fence();

      // plane columns at or past R within the half hold no product: mask them (they may be stale)
      const int nval = min(max(R - (qh + 8 * lg), 0), 8);
      u32x4 keep;
      keep.x = (nval > 0 ? 0xffffu : 0u) | (nval > 1 ? 0xffff0000u : 0u);
      keep.y = (nval > 2 ? 0xffffu : 0u) | (nval > 3 ? 0xffff0000u : 0u);
      keep.z = (nval > 4 ? 0xffffu : 0u) | (nval > 5 ? 0xffff0000u : 0u);
      keep.w = (nval > 6 ? 0xffffu : 0u) | (nval > 7 ? 0xffff0000u : 0u);
      // column blocks f in [F0, F1), as in the DMA-fed steps above
      auto steps = [&](auto f0_tag) {
      constexpr int F0 = decltype(f0_tag)::value, F1 = KIND == kGateUp ? F0 + 2 : 4;
      u32x4 bh[4], bl[4];
#pragma unroll
      for (int f = F0; f < F1; ++f) {
        const int lc = local_col<KIND>(w, f);
        if constexpr (!kT) {
          bh[f] = *reinterpret_cast<const u32x4*>(lb + (lc + lr) * 128 + 16 * (lg ^ aswz));
          bl[f] = *reinterpret_cast<const u32x4*>(lb + (lc + lr) * 128 + 16 * ((4 + lg) ^ aswz));
        } else {
          // lanes 4r..4r+3 address contraction row 8 lg + r (then + 4), columns 4 (lr & 3)..;
          // each lane receives 4 consecutive rows of its column per read
          const uint8_t* base = lb + (8 * lg + (lr >> 2)) * kLBP + 2 * (lc + 4 * (lr & 3));
          const v4s_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base));
          const v4s_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base + 4 * kLBP));
          const v4s_t l0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base + 32 * kLBP));
          const v4s_t l1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base + 36 * kLBP));
          bh[f] = u32x4{pack2(h0.x, h0.y), pack2(h0.z, h0.w), pack2(h1.x, h1.y), pack2(h1.z, h1.w)};
          bl[f] = u32x4{pack2(l0.x, l0.y), pack2(l0.z, l0.w), pack2(l1.x, l1.y), pack2(l1.z, l1.w)};
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4 ah = *reinterpret_cast<const u32x4*>(la + mb * 2048 + lr * 128 + 16 * (lg ^ aswz)) & keep;
        const u32x4 al = *reinterpret_cast<const u32x4*>(la + mb * 2048 + lr * 128 + 16 * ((4 + lg) ^ aswz)) & keep;
#pragma unroll
        for (int f = F0; f < F1; ++f) {
          acc[mb][f] = mfma_bf16(ah, bh[f], acc[mb][f]);
          acc[mb][f] = mfma_bf16(ah, bl[f], acc[mb][f]);
          acc[mb][f] = mfma_bf16(al, bh[f], acc[mb][f]);
        }
      }
      };
      if constexpr (KIND == kGateUp) {
        if (half)
          steps(FTag<2>{});
        else
          steps(FTag<0>{});
      } else {
        steps(FTag<0>{});
      }
      __syncthreads();  // the group is consumed before the next one (or the epilogue) reuses the ring
    }
    }
  }

  // out of the row's power-of-two scaled domain (the LoRA planes carry the same exponent)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ex = s_exp[mb * 16 + lg * 4 + i];
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[mb][f][i] = ldexpf(acc[mb][f][i], -ex);
    }

  // ---------------------------------------------------------------- epilogues
  // acc holds the plain sums.  One pass: every exponent belongs to one wave's
  // columns of one row, so a 16-lane reduction finds it.
  const float limit = p.limit;
  if constexpr (KIND == kGateUp) {
    // g, u saved in fp32 (training), a lane's four rows of a column as one 16-byte store
#pragma unroll
    for (int mb = 0; mb < MB && p.gsave; ++mb) {
      const int r0 = mb * 16 + lg * 4;
      const int64_t qrow = (qb + r0) >> 2;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int col = n0 + w * 32 + f * 16 + lr;
        if (col >= I || r0 >= mlen) continue;
        float* gd = p.gsave + (qrow * I + col) * 4;
        float* ud = p.usave + (qrow * I + col) * 4;
        if (r0 + 3 < mlen) {
          *reinterpret_cast<floatx4*>(gd) = acc[mb][f];
          *reinterpret_cast<floatx4*>(ud) = acc[mb][f + 2];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (r0 + i < mlen) {
              gd[i] = acc[mb][f][i];
              ud[i] = acc[mb][f + 2][i];
            }
        }
      }
    }
    // h in fp16 times 2^p, p per (row, this wave's 32 columns)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mb * 16 + lg * 4 + i;
        const bool vrow = row < mlen;
        const size_t m = (size_t)(m0 + min(row, mlen - 1));
        float h[2];
        float mx = 0.f;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int col = n0 + w * 32 + f * 16 + lr;
          const bool valid = vrow && col < I;
          const float g = acc[mb][f][i];
          const float u = acc[mb][f + 2][i];
          float gp, up, mg, mu;
          clamp_swiglu(g, u, limit, gp, up, mg, mu);
          h[f] = valid ? gp * sigmoid_f(gp) * up : 0.f;
          mx = fmaxf(mx, fabsf(h[f]));
        }
        const int pe = pow2_exponent_for(row16_max(mx));
        if (vrow && lr == 0 && n0 + w * 32 < I) p.hexp[m * p.h_nch + (n0 + w * 32) / kHExp] = pe;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int col = n0 + w * 32 + f * 16 + lr;
          if (vrow && col < I) p.hh[m * I + perm_pos(col)] = float_to_half_bits(ldexpf(h[f], pe));
        }
      }
  } else if constexpr (KIND == kDown || KIND == kGateUpBwd) {
    // per-slot rows (forward y * rw, backward dx) in fp16 times 2^p, p per
    // (row, this wave's 64 columns); the combine sums them per token
    const int chunk = (n0 + w * 64) / kStageExp;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mb * 16 + lg * 4 + i;
        const bool vrow = row < mlen;
        const int slot = vrow ? s_slot[row] : 0;
        const float wgt = (KIND == kDown && vrow) ? s_rw[row] : 1.f;
        float v[4];
        float mx = 0.f;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = n0 + w * 64 + f * 16 + lr;
          v[f] = (vrow && col < H) ? wgt * acc[mb][f][i] : 0.f;
          mx = fmaxf(mx, fabsf(v[f]));
        }
        const int pe = pow2_exponent_for(row16_max(mx));
        if (vrow && lr == 0 && n0 + w * 64 < H) p.stexp[(size_t)slot * p.st_nch + chunk] = pe;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = n0 + w * 64 + f * 16 + lr;
          if (vrow && col < H) p.stage[(size_t)slot * H + col] = float_to_half_bits(ldexpf(v[f], pe));
        }
      }
  } else {  // kDownBwd
    // dRoute partial sums per (row, this wave's 64 columns); dG and dU in fp16
    // times 2^p, p per (row, this wave's 64 columns) for each
    const int half_nch = p.dg_nch / 2;
    const int chunk = (n0 + w * 64) / kDgExp;
    // the saved g, u of this lane's four rows of each column: one 16-byte load
    // each (quads past the tile's rows are not read: they may lie past the
    // buffer).  Row block mb + 1's are requested before row block mb's results
    // are stored, since the compiler cannot move them above those stores itself.
    floatx4 gbuf[2][4], ubuf[2][4];
    auto load_gu = [&](int mb, floatx4 (&gq)[4], floatx4 (&uq)[4]) {
      const int r0 = mb * 16 + lg * 4;
      const int64_t qrow = (qb + r0) >> 2;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int cc = min(n0 + w * 64 + f * 16 + lr, I - 1);
        if (r0 < mlen) {
          gq[f] = *reinterpret_cast<const floatx4*>(p.gsave + (qrow * I + cc) * 4);
          uq[f] = *reinterpret_cast<const floatx4*>(p.usave + (qrow * I + cc) * 4);
        } else {
          gq[f] = floatx4{0.f, 0.f, 0.f, 0.f};
          uq[f] = gq[f];
        }
      }
    };
    load_gu(0, gbuf[0], ubuf[0]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb + 1 < MB) load_gu(mb + 1, gbuf[(mb + 1) & 1], ubuf[(mb + 1) & 1]);
      const floatx4(&gq)[4] = gbuf[mb & 1];
      const floatx4(&uq)[4] = ubuf[mb & 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mb * 16 + lg * 4 + i;
        const bool vrow = row < mlen;
        const size_t m = (size_t)(m0 + min(row, mlen - 1));
        const float wgt = vrow ? s_rw[row] : 0.f;
        float dg[4], du[4];
        float dr = 0.f, mxg = 0.f, mxu = 0.f;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = n0 + w * 64 + f * 16 + lr;
          const bool valid = vrow && col < I;
          const float gh = acc[mb][f][i];
          float gp, up, mg, mu;
          clamp_swiglu(gq[f][i], uq[f][i], limit, gp, up, mg, mu);
          const float sg = sigmoid_f(gp);
          const float si = gp * sg;
          const float dsi = sg * (1.f + gp * (1.f - sg));
          const float dh = wgt * gh;
          dr += valid ? gh * si * up : 0.f;
          dg[f] = valid ? dh * up * dsi * mg : 0.f;
          du[f] = valid ? dh * si * mu : 0.f;
          mxg = fmaxf(mxg, fabsf(dg[f]));
          mxu = fmaxf(mxu, fabsf(du[f]));
        }
        dr = row16_sum(dr);
        const int pg = pow2_exponent_for(row16_max(mxg));
        const int pu = pow2_exponent_for(row16_max(mxu));
        if (vrow && lr == 0 && n0 + w * 64 < I) {
          p.drpart[m * p.dr_nt + chunk] = dr;
          p.dguexp[m * p.dg_nch + chunk] = pg;
          p.dguexp[m * p.dg_nch + half_nch + chunk] = pu;
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = n0 + w * 64 + f * 16 + lr;
          if (!(vrow && col < I)) continue;
          const int pc = perm_pos(col);
          p.dgu[m * (size_t)(2 * I) + pc] = float_to_half_bits(ldexpf(dg[f], pg));
          p.dgu[m * (size_t)(2 * I) + I + pc] = float_to_half_bits(ldexpf(du[f], pu));
        }
      }
    }
  }
}

// Every tile height runs at least two waves per SIMD: a single wave issues VALU
// at half the SIMD's rate, and the weight decode needs the full rate to stay
// under the MFMA time.  One launch covers tiles of every height (each expert's
// rows: full tiles of the largest height, then one tile of the smallest height
// that holds the rest); a tile's height selects its code path.
template <int KIND, bool LDMA, bool MX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm(GemmParams p) {
  __shared__ __align__(16) uint8_t ring[kRingMax];
  __shared__ int32_t s_src[128], s_exp[128], s_slot[128];
  __shared__ float s_rw[128];
  // work item: (list position, column tile).  Position p runs on XCD p % 8
  // (blocks reach the XCDs in turn) and each XCD runs its positions' column
  // tiles in order: a tile's activation rows stay in one XCD's L2, and so do
  // an expert's weights for all its row tiles (the grouping's layout)
  const unsigned nn = (unsigned)p.n_ntiles, ntl = (unsigned)p.counters[kNumGemmTiles];
  const unsigned xcd = blockIdx.x % 8u, local = blockIdx.x / 8u;
  const unsigned tile_u = xcd + 8u * (local / nn);
  if (tile_u >= ntl) return;
  const int tile = (int)tile_u;
  if (p.tile_e[tile] < 0) return;  // an empty position of the list
  const int nt = (int)(local % nn);
  switch (p.tile_mt[tile]) {
    case 16:
      gemm_tile<KIND, 16, LDMA, MX>(p, tile, nt, ring, s_src, s_exp, s_slot, s_rw);
      break;
    case 32:
      gemm_tile<KIND, 32, LDMA, MX>(p, tile, nt, ring, s_src, s_exp, s_slot, s_rw);
      break;
    case 64:
      gemm_tile<KIND, 64, LDMA, MX>(p, tile, nt, ring, s_src, s_exp, s_slot, s_rw);
      break;
    case 96:
      gemm_tile<KIND, 96, LDMA, MX>(p, tile, nt, ring, s_src, s_exp, s_slot, s_rw);
      break;
    default:
      gemm_tile<KIND, 128, LDMA, MX>(p, tile, nt, ring, s_src, s_exp, s_slot, s_rw);
      break;
  }
}

template <int KIND>
static void launch_kind(bool ldma, bool mx, unsigned grid, const GemmParams& p, hipStream_t st) {
  if (mx) {
    if (ldma)
      k_gemm<KIND, true, true><<<grid, 256, 0, st>>>(p);
    else
      k_gemm<KIND, false, true><<<grid, 256, 0, st>>>(p);
  } else {
    if (ldma)
      k_gemm<KIND, true, false><<<grid, 256, 0, st>>>(p);
    else
      k_gemm<KIND, false, false><<<grid, 256, 0, st>>>(p);
  }
  note_launch();
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
  p.tile_e = ws_ptr<int32_t>(ws, w.gtile_e);
  p.tile_m0 = ws_ptr<int32_t>(ws, w.gtile_m0);
  p.tile_mt = ws_ptr<int32_t>(ws, w.gtile_mt);
  p.expert_slot = ws_ptr<int32_t>(ws, w.expert_slot);
  p.sshift = ws_ptr<int32_t>(ws, w.sshift);
  p.counters = ws_ptr<unsigned long long>(ws, w.counters);
  p.L = L;
  p.rw = route_weights;
  p.gsave = w.saves ? ws_ptr<float>(ws, w.g) : nullptr;  // inference: nothing saved
  p.usave = w.saves ? ws_ptr<float>(ws, w.u) : nullptr;
  p.qoffsets = ws_ptr<int32_t>(ws, w.qoffsets);
  p.hh = ws_ptr<uint16_t>(ws, w.hh);
  p.hexp = ws_ptr<int32_t>(ws, w.hexp);
  p.h_nch = (int)w.h_nch;
  p.stage = ws_ptr<uint16_t>(ws, w.stage);
  p.stexp = ws_ptr<int32_t>(ws, w.stexp);
  p.st_nch = (int)w.st_nch;
  p.dgu = ws_ptr<uint16_t>(ws, w.dgu);
  p.dguexp = ws_ptr<int32_t>(ws, w.dguexp);
  p.dg_nch = (int)w.dg_nch;
  p.drpart = ws_ptr<float>(ws, w.drpart);
  p.lsplit = ws_ptr<uint16_t>(ws, w.lsplit);
  p.zero = ws_ptr<unsigned long long>(ws, w.counters) + kZeroWord;
  const bool gu = (kind == kGateUp || kind == kGateUpBwd);
  p.sct0 = ws_ptr<uint16_t>(ws, gu ? w.sct_g : w.sct_d);
  p.sct1 = ws_ptr<uint16_t>(ws, w.sct_u);
  p.dr_nt = (int)w.dr_nt;
  switch (kind) {
    case kGateUp:
      p.n_ntiles = (int)((d.I + kHChunk - 1) / kHChunk);
      p.a_src = ws_ptr<uint16_t>(ws, w.xh);
      p.a_rowexp = ws_ptr<int32_t>(ws, w.xexp);
      p.lda = d.H;
      break;
    case kDown:
      p.n_ntiles = (int)((d.H + kNT - 1) / kNT);
      p.a_src = ws_ptr<uint16_t>(ws, w.hh);
      p.a_chunkexp = ws_ptr<int32_t>(ws, w.hexp);
      p.a_nch = (int)w.h_nch;
      p.lda = d.I;
      break;
    case kDownBwd:
      p.n_ntiles = (int)((d.I + kNT - 1) / kNT);
      p.a_src = ws_ptr<uint16_t>(ws, w.dyh);
      p.a_rowexp = ws_ptr<int32_t>(ws, w.dyexp);
      p.lda = d.H;
      break;
    case kGateUpBwd:
      p.n_ntiles = (int)((d.H + kNT - 1) / kNT);
      p.a_src = ws_ptr<uint16_t>(ws, w.dgu);
      p.a_chunkexp = ws_ptr<int32_t>(ws, w.dguexp);
      p.a_nch = (int)w.dg_nch;
      p.lda = 2 * d.I;
      break;
  }
  const unsigned grid = (unsigned)((w.max_gtiles + 7) / 8 * 8 * p.n_ntiles);  // whole rounds of 8 tiles
  if (grid == 0) return;
  switch (kind) {
    case kGateUp:
      launch_kind<kGateUp>(d.R % 4 == 0, d.fmt == KT_RAWINT4_FORMAT_MXFP4, grid, p, st);
      break;
    case kDown:
      launch_kind<kDown>(d.R % 4 == 0, d.fmt == KT_RAWINT4_FORMAT_MXFP4, grid, p, st);
      break;
    case kDownBwd:
      launch_kind<kDownBwd>(d.R % 4 == 0, d.fmt == KT_RAWINT4_FORMAT_MXFP4, grid, p, st);
      break;
    case kGateUpBwd:
      launch_kind<kGateUpBwd>(d.R % 4 == 0, d.fmt == KT_RAWINT4_FORMAT_MXFP4, grid, p, st);
      break;
  }
}

}  // namespace kt
