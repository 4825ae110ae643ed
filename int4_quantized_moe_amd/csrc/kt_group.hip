// Token-slot -> expert grouping: per-block histograms, one scan that also lays
// out the tile lists, and a stable placement of the slots.
//
// The grouping follows the routed loop of the page "rawint4_sft_reference.py"
// (routed_rawint4_lora visits every (token, slot) and indexes its expert); the
// sort-by-expert form follows the token grouping of the page
// "test_gemma4_moe.py" (flatten, sort by expert, expert offsets).  Within one
// expert the slots stay in flat slot order t*k+s, which makes the permutation
// unique.  Ids outside [0, E) are dropped and counted.
#include "kt_common.hpp"
#include "kt_internal.hpp"

namespace kt {

__global__ void k_init_counters(unsigned long long* counters) {
  if (threadIdx.x < kCounterWords) counters[threadIdx.x] = 0ull;
}

// blockcnt[b, e] = number of slots in [b*kGroupBlock, (b+1)*kGroupBlock) routed to e
__global__ __launch_bounds__(256) void k_group_count(const int64_t* __restrict__ ids, int64_t Ms, int E,
                                                     int32_t* __restrict__ blockcnt,
                                                     unsigned long long* __restrict__ counters) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * kGroupBlock;
  int bad = 0;
  for (int j = threadIdx.x; j < kGroupBlock; j += blockDim.x) {
    const int64_t s = s0 + j;
    if (s < Ms) {
      const int64_t e = ids[s];
      if (e >= 0 && e < E)
        atomicAdd(&hist[e], 1);
      else
        ++bad;
    }
  }
  if (bad) atomicAdd(&counters[kBadIds], (unsigned long long)bad);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) blockcnt[(int64_t)blockIdx.x * E + e] = hist[e];
}

// inclusive block-wide scan of one int per thread (blockDim.x <= 1024)
__device__ int block_inclusive_scan(int v, int32_t* buf) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {
    int add = t >= off ? buf[t - off] : 0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  int r = buf[t];
  __syncthreads();
  return r;
}

// Height of the tile that holds the last r rows of an expert (r <= bulk): the
// smallest of 16, 32, 64, 128 that covers them.
__device__ __forceinline__ int rest_tile_rows(int r, int bulk) {
  const int h = r <= 16 ? 16 : r <= 32 ? 32 : r <= 64 ? 64 : r <= 96 ? 96 : 128;
  return h < bulk ? h : bulk;
}

// One block: expert totals, exclusive offsets (and the same with every expert's
// rows rounded up to a multiple of 4, for the quad-row layout of the saved
// pre-activations), each expert's place among the experts in use, per-block
// placement bases
// (blockcnt is rewritten in place), and two lists of (expert, first row) tiles:
// tiles of `mt` rows for the LoRA side products, and tiles for the expert GEMMs
// -- full tiles of `gbulk` rows, then (if `gmixed`) one tile of the smallest
// height that holds the rest of the expert's rows.
//
// The GEMM list is laid out for the eight XCDs: position p runs on XCD p % 8
// (blocks reach the XCDs in turn), after the positions p - 8, p - 16, ... of the
// same XCD.  Tiles of heavy experts (kHeavyTiles or more) come first, dealt to
// the XCDs in turn, so that every XCD starts with its share of the long-running
// work; then each XCD takes a contiguous run of the other experts' tiles (the
// rows of the light part of the list filled XCD by XCD).  An expert's tiles thus
// sit on one XCD, one after another, and run together there, so its weights
// stream through that XCD's L2 once for all its row tiles.  Positions left over
// hold expert -1 (nothing to do).
__global__ __launch_bounds__(1024) void k_group_scan(int E, int64_t nb, int mt, int gbulk, int gmixed,
                                                     int32_t* __restrict__ blockcnt, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ qoffsets,
                                                     int32_t* __restrict__ expert_slot, int32_t* __restrict__ sshift,
                                                     int32_t* __restrict__ tile_e,
                                                     int32_t* __restrict__ tile_m0, int32_t* __restrict__ gtile_e,
                                                     int32_t* __restrict__ gtile_m0, int32_t* __restrict__ gtile_mt,
                                                     unsigned long long* __restrict__ counters) {
  __shared__ int32_t buf[1024];
  const int T = blockDim.x;
  const int per = (E + T - 1) / T;
  const int e0 = min(E, (int)threadIdx.x * per), e1 = min(E, e0 + per);
  __shared__ int32_t totals[2];
  int local = 0, ltiles = 0, lheavy = 0, llight = 0, lq = 0, lact = 0;
  for (int e = e0; e < e1; ++e) {
    int c = 0;
    for (int64_t b = 0; b < nb; ++b) c += blockcnt[b * E + e];
    counts[e] = c;
    local += c;
    lact += c > 0;
    lq += (c + 3) & ~3;
    ltiles += (c + mt - 1) / mt;
    const int ng = (c + gbulk - 1) / gbulk;
    if (ng >= kHeavyTiles)
      lheavy += ng;
    else
      llight += ng;
  }
  const int incl = block_inclusive_scan(local, buf);
  const int qincl = block_inclusive_scan(lq, buf);
  const int tincl = block_inclusive_scan(ltiles, buf);
  const int hincl = block_inclusive_scan(lheavy, buf);
  const int lincl = block_inclusive_scan(llight, buf);
  const int aincl = block_inclusive_scan(lact, buf);
  if ((int)threadIdx.x == T - 1) {
    totals[0] = hincl;
    totals[1] = lincl;
  }
  __syncthreads();
  // GEMM positions: rows of 8 (one per XCD), heavy rows first, then the light rows
  // filled XCD by XCD; clear them all first
  const int kh = (totals[0] + 7) / 8, lc = (totals[1] + 7) / 8, npos = 8 * (kh + lc);
  for (int q = threadIdx.x; q < npos; q += T) gtile_e[q] = -1;
  __syncthreads();
  int run = incl - local, qrun = qincl - lq, trun = tincl - ltiles, arun = aincl - lact;
  int hrun = hincl - lheavy, lrun = lincl - llight;
  for (int e = e0; e < e1; ++e) {
    const int c = counts[e];
    expert_slot[e] = c > 0 ? arun++ : -1;
    if (sshift) sshift[2 * e] = sshift[2 * e + 1] = 0;
    offsets[e] = run;
    qoffsets[e] = qrun;
    qrun += (c + 3) & ~3;
    int base = run;
    for (int64_t b = 0; b < nb; ++b) {
      const int v = blockcnt[b * E + e];
      blockcnt[b * E + e] = base;
      base += v;
    }
    const int nt = (c + mt - 1) / mt;
    for (int j = 0; j < nt; ++j) {
      tile_e[trun + j] = e;
      tile_m0[trun + j] = run + j * mt;
    }
    trun += nt;
    const int ng = (c + gbulk - 1) / gbulk;
    const bool heavy = ng >= kHeavyTiles;
    for (int j = 0; j < ng; ++j) {
      const int rest = c - j * gbulk;
      int q;
      if (heavy) {
        q = hrun + j;  // XCD q % 8, row q / 8
      } else {
        const int l = lrun + j;  // XCD l / lc, row kh + l % lc
        q = 8 * (kh + l % lc) + l / lc;
      }
      gtile_e[q] = e;
      gtile_m0[q] = run + j * gbulk;
      gtile_mt[q] = (gmixed && rest < gbulk) ? rest_tile_rows(rest, gbulk) : gbulk;
    }
    if (heavy)
      hrun += ng;
    else
      lrun += ng;
    run += c;
  }
  if ((int)threadIdx.x == T - 1) {
    offsets[E] = incl;
    qoffsets[E] = qincl;
    counters[kNumTiles] = (unsigned long long)tincl;
    counters[kNumGemmTiles] = (unsigned long long)npos;
  }
}

// Stable placement: a slot's rank among equal experts inside its block comes
// from the slots before it (rounds of blockDim.x slots, earlier rounds counted
// in cnt[]).
__global__ __launch_bounds__(256) void k_group_place(const int64_t* __restrict__ ids, int64_t Ms, int E, int topk,
                                                     const int32_t* __restrict__ blockbase,
                                                     int32_t* __restrict__ sorted_slot,
                                                     int32_t* __restrict__ row_of_slot,
                                                     int32_t* __restrict__ tok_of_row) {
  extern __shared__ int32_t cnt[];
  __shared__ int32_t rid[256];
  const int t = threadIdx.x;
  for (int e = t; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * kGroupBlock;
  for (int r0 = 0; r0 < kGroupBlock; r0 += 256) {
    const int64_t s = s0 + r0 + t;
    int e = -1;
    if (s < Ms) {
      const int64_t v = ids[s];
      if (v >= 0 && v < E) e = (int)v;
    }
    rid[t] = e;
    __syncthreads();
    if (e >= 0) {
      int rank = 0;
      for (int j = 0; j < t; ++j) rank += (rid[j] == e);
      const int pos = blockbase[(int64_t)blockIdx.x * E + e] + cnt[e] + rank;
      sorted_slot[pos] = (int32_t)s;
      tok_of_row[pos] = (int32_t)(s / topk);
      row_of_slot[s] = pos;
    } else if (s < Ms) {
      row_of_slot[s] = -1;
    }
    __syncthreads();
    if (e >= 0) atomicAdd(&cnt[e], 1);
    __syncthreads();
  }
}

void launch_init_counters(void* ws, const WsMap& w, hipStream_t st) {
  k_init_counters<<<1, 64, 0, st>>>(ws_ptr<unsigned long long>(ws, w.counters));
  note_launch();
}

void launch_group(const Dims& d, const WsMap& w, void* ws, const int64_t* ids, hipStream_t st) {
  const int E = (int)d.E;
  int32_t* blockcnt = ws_ptr<int32_t>(ws, w.blockcnt);
  unsigned long long* counters = ws_ptr<unsigned long long>(ws, w.counters);
  const size_t lds = sizeof(int32_t) * (size_t)E;
  if (w.nb > 0) {
    k_group_count<<<(unsigned)w.nb, 256, lds, st>>>(ids, d.Ms, E, blockcnt, counters);
    note_launch();
  }
  k_group_scan<<<1, 1024, 0, st>>>(E, w.nb, (int)w.mt, (int)w.gbulk, w.gmixed ? 1 : 0, blockcnt,
                                   ws_ptr<int32_t>(ws, w.counts), ws_ptr<int32_t>(ws, w.offsets),
                                   ws_ptr<int32_t>(ws, w.qoffsets), ws_ptr<int32_t>(ws, w.expert_slot),
                                   w.sshift ? ws_ptr<int32_t>(ws, w.sshift) : nullptr,
                                   ws_ptr<int32_t>(ws, w.tile_e), ws_ptr<int32_t>(ws, w.tile_m0),
                                   ws_ptr<int32_t>(ws, w.gtile_e), ws_ptr<int32_t>(ws, w.gtile_m0),
                                   ws_ptr<int32_t>(ws, w.gtile_mt), counters);
  note_launch();
  if (w.nb > 0) {
    k_group_place<<<(unsigned)w.nb, 256, lds, st>>>(ids, d.Ms, E, (int)d.K, blockcnt,
                                                   ws_ptr<int32_t>(ws, w.sorted_slot),
                                                   ws_ptr<int32_t>(ws, w.row_of_slot),
                                                   ws_ptr<int32_t>(ws, w.tok_of_row));
    note_launch();
  }
}

}  // namespace kt
