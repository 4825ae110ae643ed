// Host-side plan of one layer call: dimensions, tile sizes and the workspace map.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/kt_rawint4.h"

namespace kt {

// Tile geometry shared by the grouping (tile lists) and the matrix kernels.
constexpr int kGroupBlock = 1024;  // slots per block of the grouping histogram
constexpr int kHChunk = 128;       // columns of I per gate/up tile
constexpr int kNT = 256;           // output columns per tile of the other GEMMs
constexpr int kHExp = 32;          // columns of h per exponent (one wave's share of a gate/up tile)
constexpr int kDgExp = 64;         // columns of dG (or dU) per exponent (one wave's share of a down-dX tile)
constexpr int kStageExp = 64;      // columns of a staged per-slot row per exponent (one wave's share of a tile)
constexpr int kHeavyTiles = 8;     // an expert with this many GEMM row tiles or more is spread over the XCDs

// Rows per tile of the LoRA side products for a call: the smallest of
// 16/32/64/128 that covers the mean number of token-slots per expert (heavier
// experts take several tiles).  The expert GEMMs instead take full 128-row
// tiles of each expert and one tile of the smallest of 16/32/64/96/128 rows that
// holds the rest.  KT_RAWINT4_GEMM_ROWS=16|32|64|96|128 makes every GEMM tile
// that tall, and the side-product tiles too except for 96 (tuning and tests).
inline int forced_gemm_rows() {
  if (const char* env = getenv("KT_RAWINT4_GEMM_ROWS")) {
    const int v = atoi(env);
    if (v == 16 || v == 32 || v == 64 || v == 96 || v == 128) return v;
  }
  return 0;
}
inline int choose_gemm_rows(int64_t Ms, int64_t E) {
  // (a forced GEMM height also sets the side products' tiles, which have no 96-row form)
  if (const int v = forced_gemm_rows(); v && v != 96) return v;
  const int64_t active = E < Ms ? E : Ms;
  const int64_t mean = active > 0 ? (Ms + active - 1) / active : 0;
  if (mean <= 16) return 16;
  if (mean <= 32) return 32;
  if (mean <= 64) return 64;
  return 128;
}

// The LoRA side product that an expert GEMM contracts with (the x A^T of
// gate/up, h A_d^T, dY B_d, or dG B_g | dU B_u) is handed over as bf16 hi/lo
// planes with each rank-R half padded to whole 32-value steps: width of one half.
inline int64_t lora_half_width(int64_t R) { return (R + 31) / 32 * 32; }

// Device counters at the head of the workspace (kCounterWords words, all cleared
// by the forward); words kZeroWord.. hold 16 zero bytes that copies of rows past
// the end of an operand read instead.
enum Counter {
  kBadIds = 0,
  kBadScales = 1,
  kNumTiles = 2,      // side-product tiles
  kNumGemmTiles = 3,  // positions of the expert GEMM tile list (empty ones included)
  kNumCounters = 8,
  kZeroWord = 16,
  kCounterWords = 32
};

// LoRA gradient reductions: the rank-wide operand of each of the four families
// (x: [dG B_g | dU B_u], dY: rw ud, h: rw dyB, dG|dU: ua | ub) is laid out as
// 16-bit hi/lo planes [Ms][2][np] with np a whole number of narrow tiles.
inline int64_t grad_rank16(int64_t R) { return (R + 15) / 16 * 16; }
struct GradFam {
  int nut;     // narrow columns per tile: 16, 32, 64 or 128
  int nu;      // narrow tiles
  int64_t np;  // plane width (nu * nut)
};
inline GradFam grad_family(int64_t width) {
  GradFam f;
  f.nut = width <= 16 ? 16 : width <= 32 ? 32 : width <= 64 ? 64 : 128;
  f.nu = (int)((width + f.nut - 1) / f.nut);
  f.np = (int64_t)f.nu * f.nut;
  return f;
}
struct GradGeom {
  int64_t r16;
  GradFam x, dy, h, g;          // g: one half (dG or dU); its planes hold both halves
  int64_t off_x, off_dy, off_h, off_g, row;  // plane offsets within a row (elements) and row width
};
inline GradGeom grad_geom(int64_t R) {
  GradGeom G;
  G.r16 = grad_rank16(R);
  G.x = grad_family(2 * G.r16);
  G.dy = grad_family(G.r16);
  G.h = grad_family(G.r16);
  G.g = grad_family(G.r16);
  // each family's row is [hi np | lo np]; the families sit side by side in one row
  G.off_x = 0;
  G.off_dy = G.off_x + 2 * G.x.np;
  G.off_h = G.off_dy + 2 * G.dy.np;
  G.off_g = G.off_h + 2 * G.h.np;
  G.row = G.off_g + 2 * (2 * G.g.np);
  return G;
}

struct Dims {
  int64_t E, K, H, I, R, qlen, Ms;  // R = 0: no LoRA (inference of the base alone)
  float sc, limit;
  bool train = true;  // false: inference forward (nothing saved for a backward)
  int fmt = 0;        // weight format: 0 RAWINT4, 1 MXFP4 (KT_RAWINT4_FORMAT_*)
};

struct WsMap {
  // fp16 transposed scales of the three projections ([active expert][K/32][rows], experts
  // in use only, at their place in expert_slot), made by the forward
  size_t sct_g, sct_u, sct_d;
  // [E][2]: power-of-two shift s of an expert's gate/up (0) and down (1) scales: the tables
  // hold scale * 2^-s, chosen so that they lie in the exact domain (0 when they already do);
  // the grouping clears it, the scale conversion marks experts that need one
  size_t sshift;
  int64_t nact;  // bound on the experts in use: min(E, token-slots)
  // grouping
  size_t counters, counts, offsets, qoffsets, blockcnt, sorted_slot, row_of_slot, tok_of_row, tile_e, tile_m0;
  size_t expert_slot;  // [E]: place of an expert among those in use (ascending ids), -1 if none of its slots
  size_t gtile_e, gtile_m0, gtile_mt;  // expert GEMM tiles (mixed heights)
  // forward state kept for the backward
  size_t xh, xexp, ua, ub, g, u, hh, hexp, ud;
  // the side product feeding the next expert GEMM, as bf16 hi/lo planes (reused by all four)
  size_t lsplit;
  // transient staging of per-slot rows (forward y * rw, backward dx): fp16 [Ms][H] with one
  // power-of-two exponent per (row, kStageExp columns) [Ms][st_nch]
  size_t stage, stexp;
  // backward
  size_t dyh, dyexp, dyb, dgu, dguexp, dgb, dub, drpart;
  // LoRA gradients: narrow-operand planes ([Ms][GradGeom::row] 16-bit), per-expert exponents [E][2]
  // and the experts in the order their gradient work is dealt out (most rows first) [E];
  // per side-product tile, the largest binary exponents the exponents are made from [max_tiles][2]
  size_t gplanes, gexp, eorder, gtmax;
  size_t group_end;  // bytes needed by the grouping alone
  size_t total;
  bool saves;  // the gate/up pre-activations are kept (g, u allocated)
  int64_t nb, mt, max_tiles, h_nch, dg_nch, dr_nt;
  int64_t gbulk, max_gtiles, st_nch;
  // LoRA side products: contraction ranges per tile and their partial sums [ksplit][Ms][2R]
  int64_t side_ksplit;
  size_t side_part;  // GEMM tiles: full height and bound on their number
  bool gmixed;
};

WsMap plan_workspace(const Dims& d);
WsMap plan_group_workspace(int64_t qlen, int64_t top_k, int64_t E);

template <typename T>
inline T* ws_ptr(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// ---------------------------------------------------------------- launch errors

// Every kernel launch is followed by note_launch(), which keeps the first
// launch error of the current entry-point call (hipGetLastError right after
// the launch, so no later success hides it); begin_launches() clears it and
// any error left by an earlier call before the first launch, and
// first_launch_error() reports it at the end.
void begin_launches();
void note_launch();
hipError_t first_launch_error();

// ---------------------------------------------------------------- entry-point helpers

// Argument checks of a layer call (allow_base: all six LoRA pointers may be
// NULL, the frozen base alone); the error message as kt_rawint4_last_error
// reports it; the inference forward into a given workspace with no profiling
// events (so that nothing is created or allocated on the way).
int check_layer_dims(const kt_rawint4_moe_layer* L, int32_t qlen, Dims* d, bool allow_base);
int set_error(int code, const char* msg);
int run_forward_no_alloc(const kt_rawint4_moe_layer* layer, Dims d, const uint16_t* inputs,
                         const int64_t* expert_ids, const float* route_weights, uint16_t* output, void* workspace,
                         size_t workspace_bytes, void* stream);

// ---------------------------------------------------------------- launchers (enqueue only)

void launch_group(const Dims& d, const WsMap& w, void* ws, const int64_t* ids, hipStream_t st);
void launch_rows_to_half(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* dst, int32_t* exps,
                         hipStream_t st);

struct LayerPtrs {
  const uint8_t *wg, *wu, *wd;
  const uint16_t *sg, *su, *sd;
  const float *ag, *bg, *au, *bu, *ad, *bd;
};

enum GemmKind { kGateUp = 0, kDown = 1, kDownBwd = 2, kGateUpBwd = 3 };

void launch_gemm(GemmKind kind, const Dims& d, const WsMap& w, void* ws, const LayerPtrs& L, const float* route_weights,
                 hipStream_t st);

// LoRA side products and gradient reductions (bf16 hi/lo MFMA)
enum RowSrc { kSrcTokBf16 = 0, kSrcF32 = 1, kSrcHalfChunked = 2 };
struct RowView {
  int kind;
  const void* ptr;
  int64_t ld;       // row stride (elements)
  int64_t col_off;  // added to the column index
  const int32_t* exps;
  int64_t exp_ld, exp_off, chunk_w;
  const float* slot_scale;  // optional per-slot multiplier (route weights)
};

// out[m, q] = sum_k src(m, k) * W(e, q, k), q < R, k < kdim; W is [E, R, kdim]
// (rk = true) or [E, kdim, R] (rk = false).  With W2 set, a second product with
// the same rows goes to out2.  Also writes the product (both halves side by
// side) times the LoRA scale and times 2^(the next expert GEMM's row exponent)
// into the workspace's bf16 hi/lo planes that the GEMM reads: fp16 sources
// carry that exponent themselves, token rows take tok_exp[token].
void launch_lora_rowproj(const Dims& d, const WsMap& w, void* ws, const RowView& src, int64_t kdim, const float* W,
                         const float* W2, bool rk, float* out, float* out2, int64_t split_ld, int64_t split_off,
                         int64_t split_off2, const int32_t* tok_exp, hipStream_t st);
// The six LoRA gradients, G = (accumulate ? G : 0) + scale * dL/dG / sc, from the
// saved side products, h, dG|dU and the caller's inputs and grad_output.
struct LoraGradOut {
  float *ag, *bg, *au, *bu, *ad, *bd;
};
void launch_lora_grads(const Dims& d, const WsMap& w, void* ws, const uint16_t* inputs, const uint16_t* grad_output,
                       const float* route_weights, const LoraGradOut& out, int accumulate, float scale,
                       hipStream_t st);
void launch_fill_zero_f32(float* p, int64_t n, hipStream_t st);
// scales [E][rows][G] bf16 -> [active][G][rows] fp16, rows within-8 permuted, experts in use
// only, each at expert_slot[e] (from the grouping); an expert with a scale outside the
// exact domain is marked in sshift[2 e + grp]
void launch_scales_t(const uint16_t* s, int64_t E, int64_t rows, int64_t G, const int32_t* expert_slot,
                     uint16_t* out, int32_t* sshift, int grp, int fmt, hipStream_t st);
// for every marked expert: the shift that brings its scales into the domain, the tables
// converted again with it, and the scales still outside counted into *bad
void launch_scales_fix(const LayerPtrs& L, const Dims& d, const int32_t* expert_slot, int32_t* sshift,
                       uint16_t* sct_g, uint16_t* sct_u, uint16_t* sct_d, unsigned long long* bad, hipStream_t st);
// one exponent per row for h ([Ms, I], chunks of kHChunk) and dG|dU ([Ms, 2I], chunks of kNT per half)
void launch_normalize_chunks(uint16_t* buf, int32_t* exps, const int32_t* nrows, int64_t max_rows, int64_t cols,
                             int64_t split, int nch, int chunkw, hipStream_t st);

void launch_combine(const Dims& d, const uint16_t* stage, const int32_t* stexp, int64_t st_nch, const int64_t* ids,
                    uint16_t* out, hipStream_t st);
void launch_droute(const Dims& d, const WsMap& w, void* ws, float* grad_route, hipStream_t st);
void launch_saved_preact(const Dims& d, const WsMap& w, const void* ws, float* gate, float* up, hipStream_t st);
void launch_init_counters(void* ws, const WsMap& w, hipStream_t st);

void launch_unpack(const uint8_t* packed, int64_t n, int64_t k, int8_t* codes, hipStream_t st);
void launch_dequant(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, int fmt, float* out,
                    hipStream_t st);

}  // namespace kt
