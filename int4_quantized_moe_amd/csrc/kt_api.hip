// C ABI of the RAWINT4 routed-expert LoRA layer: argument checks, workspace map
// and the order of kernel launches for the forward and the backward.
#include <math.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "kt_common.hpp"
#include "kt_internal.hpp"

namespace kt {

static thread_local std::string g_last_error;

static int fail(int code, const char* msg) {
  g_last_error = msg;
  return code;
}

int set_error(int code, const char* msg) { return fail(code, msg); }

static size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct Planner {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  }
};

static void plan_group_part(Planner& pl, WsMap& w, int64_t Ms, int64_t E) {
  w.nb = (Ms + kGroupBlock - 1) / kGroupBlock;
  w.mt = choose_gemm_rows(Ms, E);
  w.max_tiles = Ms / w.mt + (E < Ms ? E : Ms);
  w.counters = pl.take(sizeof(unsigned long long) * kCounterWords);
  w.counts = pl.take(sizeof(int32_t) * (size_t)E);
  w.offsets = pl.take(sizeof(int32_t) * (size_t)(E + 1));
  w.qoffsets = pl.take(sizeof(int32_t) * (size_t)(E + 1));
  w.expert_slot = pl.take(sizeof(int32_t) * (size_t)E);
  w.nact = E < Ms ? E : Ms;
  w.blockcnt = pl.take(sizeof(int32_t) * (size_t)(w.nb * E));
  w.sorted_slot = pl.take(sizeof(int32_t) * (size_t)Ms);
  w.row_of_slot = pl.take(sizeof(int32_t) * (size_t)Ms);
  w.tok_of_row = pl.take(sizeof(int32_t) * (size_t)Ms);
  w.tile_e = pl.take(sizeof(int32_t) * (size_t)w.max_tiles);
  w.tile_m0 = pl.take(sizeof(int32_t) * (size_t)w.max_tiles);
  const int forced = forced_gemm_rows();
  w.gbulk = forced ? forced : 128;
  w.gmixed = forced == 0;
  // tiles, plus the positions the XCD layout of the list may leave empty
  w.max_gtiles = Ms / w.gbulk + (E < Ms ? E : Ms) + 16;
  w.gtile_e = pl.take(sizeof(int32_t) * (size_t)w.max_gtiles);
  w.gtile_m0 = pl.take(sizeof(int32_t) * (size_t)w.max_gtiles);
  w.gtile_mt = pl.take(sizeof(int32_t) * (size_t)w.max_gtiles);
  w.group_end = pl.off;
}

WsMap plan_group_workspace(int64_t qlen, int64_t top_k, int64_t E) {
  WsMap w{};
  Planner pl;
  plan_group_part(pl, w, qlen * top_k, E);
  w.total = pl.off;
  return w;
}

WsMap plan_workspace(const Dims& d) {
  // an inference forward (d.train false) keeps only what the forward itself
  // uses; without LoRA (d.R == 0) no side products either
  WsMap w{};
  Planner pl;
  plan_group_part(pl, w, d.Ms, d.E);
  w.sct_g = pl.take(2 * (size_t)w.nact * (size_t)d.I * (size_t)(d.H / 32));
  w.sct_u = pl.take(2 * (size_t)w.nact * (size_t)d.I * (size_t)(d.H / 32));
  w.sct_d = pl.take(2 * (size_t)w.nact * (size_t)d.H * (size_t)(d.I / 32));
  w.sshift = pl.take(sizeof(int32_t) * 2 * (size_t)d.E);
  w.h_nch = (d.I + kHExp - 1) / kHExp;
  w.dr_nt = (d.I + kDgExp - 1) / kDgExp;
  w.dg_nch = 2 * w.dr_nt;
  const size_t Ms = (size_t)d.Ms, q = (size_t)d.qlen, H = (size_t)d.H, I = (size_t)d.I, R = (size_t)d.R;
  const bool lora = d.R > 0;
  w.saves = d.train;
  w.xh = pl.take(2 * q * H);
  w.xexp = pl.take(4 * q);
  if (lora) {
    w.ua = pl.take(4 * Ms * R);
    w.ub = pl.take(4 * Ms * R);
  }
  if (d.train) {
    // g, u: quad-row layout, each expert's rows from a multiple of 4 (qoffsets)
    w.g = pl.take(4 * (Ms + 3 * d.E) * I);
    w.u = pl.take(4 * (Ms + 3 * d.E) * I);
  }
  w.hh = pl.take(2 * Ms * I);
  w.hexp = pl.take(4 * Ms * (size_t)w.h_nch);
  if (lora) {
    w.ud = pl.take(4 * Ms * R);
    w.lsplit = pl.take(2 * 2 * Ms * 2 * (size_t)lora_half_width((int64_t)R));
  }
  w.st_nch = (d.H + kStageExp - 1) / kStageExp;
  w.stage = pl.take(2 * Ms * H);
  w.stexp = pl.take(4 * Ms * (size_t)w.st_nch);
  if (d.train) {
    w.dyh = pl.take(2 * q * H);
    w.dyexp = pl.take(4 * q);
    w.dyb = pl.take(4 * Ms * R);
    w.dgu = pl.take(2 * Ms * 2 * I);
    w.dguexp = pl.take(4 * Ms * (size_t)w.dg_nch);
    w.dgb = pl.take(4 * Ms * R);
    w.dub = pl.take(4 * Ms * R);
    w.drpart = pl.take(4 * Ms * (size_t)w.dr_nt);
  }
  // ~4096 blocks (the side-product steps are latency-bound, so more blocks in
  // flight pay for the partial sums) when the tiles are fewer
  w.side_ksplit = std::min<int64_t>(16, std::max<int64_t>(1, (4096 + w.max_tiles - 1) / std::max<int64_t>(w.max_tiles, 1)));
  if (lora) w.side_part = pl.take(w.side_ksplit > 1 ? 4 * (size_t)w.side_ksplit * Ms * 2 * R : 0);
  if (d.train) {
    w.gplanes = pl.take(2 * Ms * (size_t)grad_geom(d.R).row);
    w.gexp = pl.take(4 * 2 * (size_t)d.E);
    w.eorder = pl.take(4 * (size_t)d.E);
    w.gtmax = pl.take(4 * 2 * (size_t)std::max<int64_t>(w.max_tiles, 1));
  }
  w.total = pl.off;
  return w;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// allow_base: an inference call may give all six LoRA pointers as NULL (the
// frozen base alone; rank and alpha are then not used)
static int check_layer(const kt_rawint4_moe_layer* L, int32_t qlen, Dims* d, bool allow_base = false) {
  if (!L) return fail(KT_RAWINT4_EINVAL, "layer is NULL");
  if (L->num_experts < 1 || L->num_experts > KT_RAWINT4_MAX_EXPERTS)
    return fail(KT_RAWINT4_EINVAL, "num_experts must be in [1, 8192]");
  if (L->top_k < 1 || L->top_k > L->num_experts) return fail(KT_RAWINT4_EINVAL, "top_k must be in [1, num_experts]");
  if (L->hidden <= 0 || L->hidden % KT_RAWINT4_GROUP_SIZE || L->hidden > 65536)
    return fail(KT_RAWINT4_EINVAL, "hidden must be a positive multiple of 32 (at most 65536)");
  if (L->intermediate <= 0 || L->intermediate % KT_RAWINT4_GROUP_SIZE || L->intermediate > 65536)
    return fail(KT_RAWINT4_EINVAL, "intermediate must be a positive multiple of 32 (at most 65536)");
  const bool base = allow_base && !L->gate_lora_a && !L->gate_lora_b && !L->up_lora_a && !L->up_lora_b &&
                    !L->down_lora_a && !L->down_lora_b;
  if (!base && (L->rank < 1 || L->rank > KT_RAWINT4_MAX_RANK))
    return fail(KT_RAWINT4_EINVAL, "rank must be in [1, 128]");
  if (!base && !isfinite(L->alpha)) return fail(KT_RAWINT4_EINVAL, "alpha must be finite");
  if (!isfinite(L->swiglu_limit) || L->swiglu_limit < 0.f)
    return fail(KT_RAWINT4_EINVAL, "swiglu_limit must be finite and non-negative");
  if (L->weight_format != KT_RAWINT4_FORMAT_RAWINT4 && L->weight_format != KT_RAWINT4_FORMAT_MXFP4)
    return fail(KT_RAWINT4_EINVAL, "weight_format must be KT_RAWINT4_FORMAT_RAWINT4 or KT_RAWINT4_FORMAT_MXFP4");
  if (qlen < 0) return fail(KT_RAWINT4_EINVAL, "qlen must be non-negative");
  if ((int64_t)qlen * L->top_k >= ((int64_t)1 << 31)) return fail(KT_RAWINT4_EINVAL, "qlen * top_k must be below 2^31");
  const void* ptrs[] = {L->gate_packed, L->up_packed,   L->down_packed, L->gate_scale,  L->up_scale,
                        L->down_scale,  L->gate_lora_a, L->gate_lora_b, L->up_lora_a,   L->up_lora_b,
                        L->down_lora_a, L->down_lora_b};
  for (int i = 0; i < (base ? 6 : 12); ++i)
    if (!ptrs[i]) return fail(KT_RAWINT4_EINVAL, "a weight, scale or LoRA pointer is NULL");
  if (!aligned(L->gate_packed, 16) || !aligned(L->up_packed, 16) || !aligned(L->down_packed, 16))
    return fail(KT_RAWINT4_EINVAL, "packed weights must be 16-byte aligned");
  if (!aligned(L->gate_scale, 2) || !aligned(L->up_scale, 2) || !aligned(L->down_scale, 2))
    return fail(KT_RAWINT4_EINVAL, "scales must be 2-byte aligned");
  const float* lora[] = {L->gate_lora_a, L->gate_lora_b, L->up_lora_a, L->up_lora_b, L->down_lora_a, L->down_lora_b};
  if (!base)
    for (const float* p : lora)
      if (!aligned(p, 16)) return fail(KT_RAWINT4_EINVAL, "LoRA tensors must be 16-byte aligned");
  d->E = L->num_experts;
  d->K = L->top_k;
  d->H = L->hidden;
  d->I = L->intermediate;
  d->R = base ? 0 : L->rank;
  d->qlen = qlen;
  d->Ms = (int64_t)qlen * L->top_k;
  d->sc = base ? 0.f : L->alpha / (float)L->rank;
  d->limit = L->swiglu_limit;
  d->fmt = L->weight_format;
  return KT_RAWINT4_OK;
}

int check_layer_dims(const kt_rawint4_moe_layer* L, int32_t qlen, Dims* d, bool allow_base) {
  return check_layer(L, qlen, d, allow_base);
}

static LayerPtrs layer_ptrs(const kt_rawint4_moe_layer* L) {
  LayerPtrs p;
  p.wg = L->gate_packed;
  p.wu = L->up_packed;
  p.wd = L->down_packed;
  p.sg = L->gate_scale;
  p.su = L->up_scale;
  p.sd = L->down_scale;
  p.ag = L->gate_lora_a;
  p.bg = L->gate_lora_b;
  p.au = L->up_lora_a;
  p.bu = L->up_lora_b;
  p.ad = L->down_lora_a;
  p.bd = L->down_lora_b;
  return p;
}

static int check_workspace(void* ws, size_t bytes, size_t need) {
  if (!ws) return fail(KT_RAWINT4_EINVAL, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(KT_RAWINT4_EINVAL, "workspace must be 256-byte aligned");
  if (bytes < need) return fail(KT_RAWINT4_EWORKSPACE, "workspace is smaller than the required size");
  return KT_RAWINT4_OK;
}

static thread_local hipError_t g_first_launch_error = hipSuccess;

void begin_launches() {
  (void)hipGetLastError();
  g_first_launch_error = hipSuccess;
}

void note_launch() {
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess && g_first_launch_error == hipSuccess) g_first_launch_error = err;
}

hipError_t first_launch_error() { return g_first_launch_error; }

// The result of an entry point's launches (and of a HIP call whose error it
// already took, err): the first failure since begin_launches.
static int launched(hipError_t err = hipSuccess) {
  note_launch();
  if (g_first_launch_error == hipSuccess && err != hipSuccess) g_first_launch_error = err;
  if (g_first_launch_error != hipSuccess) {
    g_last_error = std::string("HIP launch failed: ") + hipGetErrorString(g_first_launch_error);
    g_first_launch_error = hipSuccess;
    return KT_RAWINT4_EHIP;
  }
  g_last_error.clear();
  return KT_RAWINT4_OK;
}

static RowView view_tok_bf16(const uint16_t* p, int64_t ld, const float* slot_scale = nullptr) {
  RowView v{};
  v.kind = kSrcTokBf16;
  v.ptr = p;
  v.ld = ld;
  v.slot_scale = slot_scale;
  return v;
}

static RowView view_f32(const float* p, int64_t ld, const float* slot_scale = nullptr) {
  RowView v{};
  v.kind = kSrcF32;
  v.ptr = p;
  v.ld = ld;
  v.slot_scale = slot_scale;
  return v;
}

static RowView view_half(const uint16_t* p, int64_t ld, int64_t col_off, const int32_t* exps, int64_t exp_ld,
                         int64_t exp_off, int64_t chunk_w) {
  RowView v{};
  v.kind = kSrcHalfChunked;
  v.ptr = p;
  v.ld = ld;
  v.col_off = col_off;
  v.exps = exps;
  v.exp_ld = exp_ld;
  v.exp_off = exp_off;
  v.chunk_w = chunk_w;
  return v;
}


// ---------------------------------------------------------------- per-phase event timing

enum Phase {
  kPhGroup = 0,
  kPhScales,
  kPhXHalf,
  kPhLoraXA,
  kPhGemmGateUp,
  kPhHRows,
  kPhLoraHA,
  kPhGemmDown,
  kPhCombineFwd,
  kPhDyHalf,
  kPhLoraDyB,
  kPhGemmDownBwd,
  kPhDguRows,
  kPhLoraDgB,
  kPhGemmGateUpBwd,
  kPhCombineBwd,
  kPhDRoute,
  kPhLoraGrads,
  kNumPhases
};

static const char* const kPhaseNames[kNumPhases] = {
    "group",           "scales_fp16",     "x_to_half",          "lora_a_gate_up",  "gemm_gate_up",
    "h_rows",          "lora_a_down",     "gemm_down",          "combine_fwd",     "dy_to_half",
    "lora_b_down_bwd", "gemm_down_dx",    "dgu_rows",           "lora_b_gate_up_bwd", "gemm_gate_up_dx",
    "combine_bwd",     "droute",          "lora_grads"};

struct ProfRec {
  int phase;
  hipEvent_t a, b;
};

static std::mutex g_prof_mu;
static bool g_prof_on = false;
// set while a call that must create nothing runs on this thread: no profiling events
static thread_local bool g_no_events = false;
static std::vector<hipEvent_t> g_prof_pool;
static std::vector<ProfRec> g_prof_recs;

static hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t ev = g_prof_pool.back();
    g_prof_pool.pop_back();
    return ev;
  }
  hipEvent_t ev = nullptr;
  if (hipEventCreate(&ev) != hipSuccess) return nullptr;
  return ev;
}

// Records a start/stop event pair around the launches of one phase on the
// caller's stream while profiling is enabled.
struct PhaseScope {
  int phase;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  PhaseScope(int ph, hipStream_t s) : phase(ph), st(s) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on || g_no_events) return;
    a = prof_event();
    b = prof_event();
    if (!a || !b || hipEventRecord(a, st) != hipSuccess) release();
  }
  ~PhaseScope() {
    if (!a || !b) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (hipEventRecord(b, st) != hipSuccess) {
      release();
      return;
    }
    g_prof_recs.push_back({phase, a, b});
  }
  // called with g_prof_mu held: give the events back unrecorded
  void release() {
    if (a) g_prof_pool.push_back(a);
    if (b) g_prof_pool.push_back(b);
    a = b = nullptr;
  }
};

}  // namespace kt

using namespace kt;

extern "C" {

size_t kt_rawint4_moe_workspace_bytes(const kt_rawint4_moe_layer* layer, int32_t qlen) {
  Dims d;
  if (check_layer(layer, qlen, &d) != KT_RAWINT4_OK) return 0;
  return plan_workspace(d).total;
}

// The forward's kernels up to what a backward reads: grouping, transposed
// scales, fp16 rows of x, the side products x A_g^T | x A_u^T, the gate/up GEMM
// with SwiGLU (saving the pre-activations when d.train), the rows of h and
// h A_d^T.  Without LoRA (d.R == 0) no side product runs.
static void launch_forward_front(const kt_rawint4_moe_layer* layer, const Dims& d, const WsMap& w, void* ws,
                                 const LayerPtrs& L, const uint16_t* inputs, const int64_t* expert_ids,
                                 const float* route_weights, hipStream_t st) {
  const bool lora = d.R > 0;
  {
    PhaseScope ph(kPhGroup, st);
    launch_init_counters(ws, w, st);
    launch_group(d, w, ws, expert_ids, st);
  }
  {
    PhaseScope ph(kPhScales, st);
    unsigned long long* bad = ws_ptr<unsigned long long>(ws, w.counters) + kBadScales;
    const int32_t* slot = ws_ptr<int32_t>(ws, w.expert_slot);
    int32_t* sshift = ws_ptr<int32_t>(ws, w.sshift);
    launch_scales_t(layer->gate_scale, d.E, d.I, d.H / 32, slot, ws_ptr<uint16_t>(ws, w.sct_g), sshift, 0, d.fmt, st);
    launch_scales_t(layer->up_scale, d.E, d.I, d.H / 32, slot, ws_ptr<uint16_t>(ws, w.sct_u), sshift, 0, d.fmt, st);
    launch_scales_t(layer->down_scale, d.E, d.H, d.I / 32, slot, ws_ptr<uint16_t>(ws, w.sct_d), sshift, 1, d.fmt, st);
    launch_scales_fix(L, d, slot, sshift, ws_ptr<uint16_t>(ws, w.sct_g), ws_ptr<uint16_t>(ws, w.sct_u),
                      ws_ptr<uint16_t>(ws, w.sct_d), bad, st);
  }
  {
    PhaseScope ph(kPhXHalf, st);
    launch_rows_to_half(inputs, d.qlen, d.H, ws_ptr<uint16_t>(ws, w.xh), ws_ptr<int32_t>(ws, w.xexp), st);
  }
  const RowView xv = view_tok_bf16(inputs, d.H);
  if (lora) {
    PhaseScope ph(kPhLoraXA, st);
    launch_lora_rowproj(d, w, ws, xv, d.H, L.ag, L.au, true, ws_ptr<float>(ws, w.ua), ws_ptr<float>(ws, w.ub),
                        2 * lora_half_width(d.R), 0, lora_half_width(d.R), ws_ptr<int32_t>(ws, w.xexp), st);
  }
  {
    PhaseScope ph(kPhGemmGateUp, st);
    launch_gemm(kGateUp, d, w, ws, L, route_weights, st);
  }
  {
    PhaseScope ph(kPhHRows, st);
    launch_normalize_chunks(ws_ptr<uint16_t>(ws, w.hh), ws_ptr<int32_t>(ws, w.hexp),
                            ws_ptr<int32_t>(ws, w.offsets) + d.E, d.Ms, d.I, d.I, (int)w.h_nch, kHExp, st);
  }
  const RowView hv = view_half(ws_ptr<uint16_t>(ws, w.hh), d.I, 0, ws_ptr<int32_t>(ws, w.hexp), w.h_nch, 0, kHExp);
  if (lora) {
    PhaseScope ph(kPhLoraHA, st);
    launch_lora_rowproj(d, w, ws, hv, d.I, L.ad, nullptr, true, ws_ptr<float>(ws, w.ud), nullptr,
                        lora_half_width(d.R), 0, 0, nullptr, st);
  }
}

// The forward of a training call (train: saves what the backward needs) or of
// an inference call (nothing saved; d.R == 0: the base without LoRA).
static int run_forward(const kt_rawint4_moe_layer* layer, Dims d, const uint16_t* inputs, const int64_t* expert_ids,
                       const float* route_weights, uint16_t* output, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (d.qlen == 0) {
    g_last_error.clear();
    return KT_RAWINT4_OK;
  }
  if (!inputs || !expert_ids || !route_weights || !output)
    return fail(KT_RAWINT4_EINVAL, "inputs, expert_ids, route_weights and output must be non-NULL");
  if (!aligned(inputs, 16) || !aligned(output, 8) || !aligned(expert_ids, 8) || !aligned(route_weights, 4))
    return fail(KT_RAWINT4_EINVAL, "inputs must be 16-byte aligned, output and expert_ids 8-byte aligned");
  const WsMap w = plan_workspace(d);
  const int rc = check_workspace(workspace, workspace_bytes, w.total);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const LayerPtrs L = layer_ptrs(layer);
  void* ws = workspace;
  begin_launches();
  launch_forward_front(layer, d, w, ws, L, inputs, expert_ids, route_weights, st);
  {
    PhaseScope ph(kPhGemmDown, st);
    launch_gemm(kDown, d, w, ws, L, route_weights, st);
  }
  {
    PhaseScope ph(kPhCombineFwd, st);
    launch_combine(d, ws_ptr<uint16_t>(ws, w.stage), ws_ptr<int32_t>(ws, w.stexp), w.st_nch, expert_ids, output,
                   st);
  }
  return launched();
}

int kt_rawint4_moe_fwd(const kt_rawint4_moe_layer* layer, int32_t qlen, const uint16_t* inputs,
                       const int64_t* expert_ids, const float* route_weights, uint16_t* output, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Dims d;
  const int rc = check_layer(layer, qlen, &d);
  if (rc) return rc;
  return run_forward(layer, d, inputs, expert_ids, route_weights, output, workspace, workspace_bytes, stream);
}

size_t kt_rawint4_moe_infer_workspace_bytes(const kt_rawint4_moe_layer* layer, int32_t qlen) {
  Dims d;
  if (check_layer(layer, qlen, &d, true) != KT_RAWINT4_OK) return 0;
  d.train = false;
  return plan_workspace(d).total;
}

int kt_rawint4_moe_infer(const kt_rawint4_moe_layer* layer, int32_t qlen, const uint16_t* inputs,
                         const int64_t* expert_ids, const float* route_weights, uint16_t* output, void* workspace,
                         size_t workspace_bytes, void* stream) {
  Dims d;
  const int rc = check_layer(layer, qlen, &d, true);
  if (rc) return rc;
  d.train = false;
  return run_forward(layer, d, inputs, expert_ids, route_weights, output, workspace, workspace_bytes, stream);
}

// The backward; recompute: first rerun the forward's front into the workspace
// (the checkpoint-recompute form, no saved forward needed).
static int run_backward(const kt_rawint4_moe_layer* layer, int32_t qlen, const uint16_t* inputs,
                        const int64_t* expert_ids, const float* route_weights, const uint16_t* grad_output,
                        uint16_t* grad_input, float* grad_route, float* d_gate_a, float* d_gate_b, float* d_up_a,
                        float* d_up_b, float* d_down_a, float* d_down_b, int32_t accumulate, float grad_scale,
                        void* workspace, size_t workspace_bytes, void* stream, bool recompute) {
  Dims d;
  int rc = check_layer(layer, qlen, &d);
  if (rc) return rc;
  float* grads[6] = {d_gate_a, d_gate_b, d_up_a, d_up_b, d_down_a, d_down_b};
  for (float* g : grads) {
    if (!g) return fail(KT_RAWINT4_EINVAL, "the six LoRA gradient buffers must be non-NULL");
    if (!aligned(g, 4)) return fail(KT_RAWINT4_EINVAL, "LoRA gradient buffers must be 4-byte aligned");
  }
  if (!isfinite(grad_scale)) return fail(KT_RAWINT4_EINVAL, "grad_scale must be finite");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t gsz[6] = {d.E * d.R * d.H, d.E * d.I * d.R, d.E * d.R * d.H,
                          d.E * d.I * d.R, d.E * d.R * d.I, d.E * d.H * d.R};
  if (qlen == 0) {
    begin_launches();
    if (!accumulate)
      for (int j = 0; j < 6; ++j) launch_fill_zero_f32(grads[j], gsz[j], st);
    return launched();
  }
  if (!inputs || !expert_ids || !route_weights || !grad_output || !grad_input)
    return fail(KT_RAWINT4_EINVAL, "inputs, expert_ids, route_weights, grad_output and grad_input must be non-NULL");
  if (!aligned(inputs, 16) || !aligned(grad_output, 16) || !aligned(grad_input, 8) || !aligned(expert_ids, 8) ||
      !aligned(route_weights, 4) || (grad_route && !aligned(grad_route, 4)))
    return fail(KT_RAWINT4_EINVAL, "inputs and grad_output must be 16-byte aligned, grad_input 8-byte aligned");
  const WsMap w = plan_workspace(d);
  rc = check_workspace(workspace, workspace_bytes, w.total);
  if (rc) return rc;
  const LayerPtrs L = layer_ptrs(layer);
  void* ws = workspace;
  begin_launches();
  if (recompute) launch_forward_front(layer, d, w, ws, L, inputs, expert_ids, route_weights, st);

  {
    PhaseScope ph(kPhDyHalf, st);
    launch_rows_to_half(grad_output, d.qlen, d.H, ws_ptr<uint16_t>(ws, w.dyh), ws_ptr<int32_t>(ws, w.dyexp), st);
  }
  const RowView dyv = view_tok_bf16(grad_output, d.H);
  {
    PhaseScope ph(kPhLoraDyB, st);
    launch_lora_rowproj(d, w, ws, dyv, d.H, L.bd, nullptr, false, ws_ptr<float>(ws, w.dyb), nullptr,
                        lora_half_width(d.R), 0, 0, ws_ptr<int32_t>(ws, w.dyexp), st);
  }
  {
    PhaseScope ph(kPhGemmDownBwd, st);
    launch_gemm(kDownBwd, d, w, ws, L, route_weights, st);
  }
  {
    PhaseScope ph(kPhDguRows, st);
    launch_normalize_chunks(ws_ptr<uint16_t>(ws, w.dgu), ws_ptr<int32_t>(ws, w.dguexp),
                            ws_ptr<int32_t>(ws, w.offsets) + d.E, d.Ms, 2 * d.I, d.I, (int)w.dg_nch, kDgExp, st);
  }
  const RowView dgv = view_half(ws_ptr<uint16_t>(ws, w.dgu), 2 * d.I, 0, ws_ptr<int32_t>(ws, w.dguexp), w.dg_nch, 0, kDgExp);
  const RowView duv =
      view_half(ws_ptr<uint16_t>(ws, w.dgu), 2 * d.I, d.I, ws_ptr<int32_t>(ws, w.dguexp), w.dg_nch, w.dg_nch / 2, kDgExp);
  {
    PhaseScope ph(kPhLoraDgB, st);
    launch_lora_rowproj(d, w, ws, dgv, d.I, L.bg, nullptr, false, ws_ptr<float>(ws, w.dgb), nullptr,
                        2 * lora_half_width(d.R), 0, 0, nullptr, st);
    launch_lora_rowproj(d, w, ws, duv, d.I, L.bu, nullptr, false, ws_ptr<float>(ws, w.dub), nullptr,
                        2 * lora_half_width(d.R), lora_half_width(d.R), 0, nullptr, st);
  }
  {
    PhaseScope ph(kPhGemmGateUpBwd, st);
    launch_gemm(kGateUpBwd, d, w, ws, L, route_weights, st);
  }
  {
    PhaseScope ph(kPhCombineBwd, st);
    launch_combine(d, ws_ptr<uint16_t>(ws, w.stage), ws_ptr<int32_t>(ws, w.stexp), w.st_nch, expert_ids,
                   grad_input, st);
  }
  if (grad_route) {
    PhaseScope ph(kPhDRoute, st);
    launch_droute(d, w, ws, grad_route, st);
  }
  PhaseScope ph_grads(kPhLoraGrads, st);

  LoraGradOut go{d_gate_a, d_gate_b, d_up_a, d_up_b, d_down_a, d_down_b};
  launch_lora_grads(d, w, ws, inputs, grad_output, route_weights, go, accumulate, grad_scale * d.sc, st);
  return launched();
}

int kt_rawint4_moe_bwd(const kt_rawint4_moe_layer* layer, int32_t qlen, const uint16_t* inputs,
                       const int64_t* expert_ids, const float* route_weights, const uint16_t* grad_output,
                       uint16_t* grad_input, float* grad_route, float* d_gate_a, float* d_gate_b, float* d_up_a,
                       float* d_up_b, float* d_down_a, float* d_down_b, int32_t accumulate, float grad_scale,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return run_backward(layer, qlen, inputs, expert_ids, route_weights, grad_output, grad_input, grad_route, d_gate_a,
                      d_gate_b, d_up_a, d_up_b, d_down_a, d_down_b, accumulate, grad_scale, workspace,
                      workspace_bytes, stream, false);
}

int kt_rawint4_moe_bwd_recompute(const kt_rawint4_moe_layer* layer, int32_t qlen, const uint16_t* inputs,
                                 const int64_t* expert_ids, const float* route_weights, const uint16_t* grad_output,
                                 uint16_t* grad_input, float* grad_route, float* d_gate_a, float* d_gate_b,
                                 float* d_up_a, float* d_up_b, float* d_down_a, float* d_down_b, int32_t accumulate,
                                 float grad_scale, void* workspace, size_t workspace_bytes, void* stream) {
  return run_backward(layer, qlen, inputs, expert_ids, route_weights, grad_output, grad_input, grad_route, d_gate_a,
                      d_gate_b, d_up_a, d_up_b, d_down_a, d_down_b, accumulate, grad_scale, workspace,
                      workspace_bytes, stream, true);
}

int kt_rawint4_unpack(const uint8_t* packed, int64_t n, int64_t k, int8_t* codes, void* stream) {
  if (n < 0 || k < 0 || k % 2) return fail(KT_RAWINT4_EINVAL, "n must be >= 0 and k a non-negative even number");
  if (n * k > 0 && (!packed || !codes)) return fail(KT_RAWINT4_EINVAL, "packed and codes must be non-NULL");
  begin_launches();
  launch_unpack(packed, n, k, codes, static_cast<hipStream_t>(stream));
  return launched();
}

int kt_rawint4_dequant(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, float* weights,
                       void* stream) {
  if (n < 0 || k < 0 || k % KT_RAWINT4_GROUP_SIZE)
    return fail(KT_RAWINT4_EINVAL, "n must be >= 0 and k a multiple of 32");
  if (n * k > 0 && (!packed || !scales || !weights))
    return fail(KT_RAWINT4_EINVAL, "packed, scales and weights must be non-NULL");
  if (!aligned(packed, 4)) return fail(KT_RAWINT4_EINVAL, "packed must be 4-byte aligned");
  begin_launches();
  launch_dequant(packed, scales, n, k, KT_RAWINT4_FORMAT_RAWINT4, weights, static_cast<hipStream_t>(stream));
  return launched();
}

int kt_rawint4_dequant_mxfp4(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, float* weights,
                             void* stream) {
  if (n < 0 || k < 0 || k % KT_RAWINT4_GROUP_SIZE)
    return fail(KT_RAWINT4_EINVAL, "n must be >= 0 and k a multiple of 32");
  if (n * k > 0 && (!packed || !scales || !weights))
    return fail(KT_RAWINT4_EINVAL, "packed, scales and weights must be non-NULL");
  if (!aligned(packed, 4)) return fail(KT_RAWINT4_EINVAL, "packed must be 4-byte aligned");
  begin_launches();
  launch_dequant(packed, scales, n, k, KT_RAWINT4_FORMAT_MXFP4, weights, static_cast<hipStream_t>(stream));
  return launched();
}

size_t kt_rawint4_group_workspace_bytes(int32_t qlen, int32_t top_k, int32_t num_experts) {
  if (qlen < 0 || top_k < 1 || num_experts < 1 || num_experts > KT_RAWINT4_MAX_EXPERTS) {
    fail(KT_RAWINT4_EINVAL, "invalid grouping dimensions");
    return 0;
  }
  return plan_group_workspace(qlen, top_k, num_experts).total;
}

int kt_rawint4_group(const int64_t* expert_ids, int32_t qlen, int32_t top_k, int32_t num_experts, int32_t* offsets,
                     int32_t* sorted_slot, void* workspace, size_t workspace_bytes, void* stream) {
  if (qlen < 0 || top_k < 1 || num_experts < 1 || num_experts > KT_RAWINT4_MAX_EXPERTS)
    return fail(KT_RAWINT4_EINVAL, "invalid grouping dimensions");
  if ((int64_t)qlen * top_k >= ((int64_t)1 << 31)) return fail(KT_RAWINT4_EINVAL, "qlen * top_k must be below 2^31");
  if (!offsets || (qlen > 0 && (!expert_ids || !sorted_slot)))
    return fail(KT_RAWINT4_EINVAL, "expert_ids, offsets and sorted_slot must be non-NULL");
  const WsMap w = plan_group_workspace(qlen, top_k, num_experts);
  int rc = check_workspace(workspace, workspace_bytes, w.total);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Dims d{};
  d.E = num_experts;
  d.K = top_k;
  d.qlen = qlen;
  d.Ms = (int64_t)qlen * top_k;
  begin_launches();
  launch_init_counters(workspace, w, st);
  launch_group(d, w, workspace, expert_ids, st);
  hipError_t err = hipMemcpyAsync(offsets, ws_ptr<int32_t>(workspace, w.offsets),
                                  sizeof(int32_t) * (size_t)(num_experts + 1), hipMemcpyDeviceToDevice, st);
  if (err == hipSuccess && d.Ms > 0)
    err = hipMemcpyAsync(sorted_slot, ws_ptr<int32_t>(workspace, w.sorted_slot), sizeof(int32_t) * (size_t)d.Ms,
                         hipMemcpyDeviceToDevice, st);
  return launched(err);
}

int kt_rawint4_moe_diagnostics(const void* workspace, size_t workspace_bytes, int64_t* bad_ids, int64_t* bad_scales,
                               void* stream) {
  if (!workspace) return fail(KT_RAWINT4_EINVAL, "workspace is NULL");
  if (workspace_bytes < sizeof(unsigned long long) * kNumCounters)
    return fail(KT_RAWINT4_EWORKSPACE, "workspace is smaller than the counter block");
  unsigned long long host[kNumCounters];
  hipStream_t st = static_cast<hipStream_t>(stream);
  begin_launches();
  hipError_t err = hipMemcpyAsync(host, workspace, sizeof(host), hipMemcpyDeviceToHost, st);
  if (err == hipSuccess) err = hipStreamSynchronize(st);
  if (err != hipSuccess) return launched(err);
  if (bad_ids) *bad_ids = (int64_t)host[kBadIds];
  if (bad_scales) *bad_scales = (int64_t)host[kBadScales];
  g_last_error.clear();
  return KT_RAWINT4_OK;
}

int kt_rawint4_moe_saved_preactivations(const kt_rawint4_moe_layer* layer, int32_t qlen, const void* workspace,
                                        size_t workspace_bytes, float* gate, float* up, void* stream) {
  Dims d;
  int rc = check_layer(layer, qlen, &d);
  if (rc) return rc;
  if (qlen == 0) {
    g_last_error.clear();
    return KT_RAWINT4_OK;
  }
  if (!gate || !up) return fail(KT_RAWINT4_EINVAL, "gate and up must be non-NULL");
  const WsMap w = plan_workspace(d);
  rc = check_workspace(const_cast<void*>(workspace), workspace_bytes, w.total);
  if (rc) return rc;
  begin_launches();
  launch_saved_preact(d, w, workspace, gate, up, static_cast<hipStream_t>(stream));
  return launched();
}

int kt_rawint4_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  g_last_error.clear();
  return KT_RAWINT4_OK;
}

int kt_rawint4_profile_read(float* ms, int32_t* launches, int32_t capacity) {
  if (!ms || !launches || capacity < kNumPhases)
    return fail(KT_RAWINT4_EINVAL, "ms and launches need room for every phase");
  for (int i = 0; i < kNumPhases; ++i) {
    ms[i] = 0.f;
    launches[i] = 0;
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int rc = KT_RAWINT4_OK;
  for (const ProfRec& r : g_prof_recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) {
      rc = fail(KT_RAWINT4_EHIP, "event timing failed");
    } else {
      ms[r.phase] += t;
      launches[r.phase] += 1;
    }
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  if (rc == KT_RAWINT4_OK) g_last_error.clear();
  return rc == KT_RAWINT4_OK ? kNumPhases : rc;
}

const char* kt_rawint4_profile_phase_name(int32_t phase) {
  if (phase < 0 || phase >= kNumPhases) return "";
  return kPhaseNames[phase];
}

const char* kt_rawint4_last_error(void) { return g_last_error.c_str(); }

const char* kt_rawint4_weight_layout(void) { return "compressed-tensors-rawint4-g32-v1"; }

}  // extern "C"

int kt::run_forward_no_alloc(const kt_rawint4_moe_layer* layer, Dims d, const uint16_t* inputs,
                             const int64_t* expert_ids, const float* route_weights, uint16_t* output,
                             void* workspace, size_t workspace_bytes, void* stream) {
  g_no_events = true;
  const int rc = run_forward(layer, d, inputs, expert_ids, route_weights, output, workspace, workspace_bytes, stream);
  g_no_events = false;
  return rc;
}
