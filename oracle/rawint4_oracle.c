/*
 * CPU oracle of the RAWINT4 routed-expert LoRA layer (forward and backward).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code with the GPU
 * path: no headers, no tables, no helpers.
 *
 * What it follows (page "rawint4_sft_reference.py", the auditable reference):
 *   - the codec: a byte holds two biased nibbles, low nibble first; nibble c
 *     decodes to (c - 8) times the bf16 scale of its 32-wide group
 *     (module docstring, unpack_rawint4, dequantize_rawint4);
 *   - the MXFP4 weight format of the same layer (page "ext_bindings.cpp"
 *     commit log: MXFP4_SFT_MOE, E2M1 nibbles with a UE8M0 scale per group of
 *     32, the scale handed over as bf16 by a bit-cast; page "backend.py",
 *     layout "mxfp4-e2m1-ue8m0-g32"): nibble c is the E2M1 number of the OCP
 *     microscaling formats -- sign bit 3, exponent bits 2..1 with bias 1,
 *     mantissa bit 0, exponent 0 subnormal -- times the bf16 scale.  Readings:
 *     nibble order as for RAWINT4 (low nibble first), and everything but the
 *     decode (grouping, LoRA, clamp, gradients) as for RAWINT4;
 *   - the layout checks (_validate_rawint4_layout);
 *   - the group-at-a-time transpose-free dX (transpose_free_rawint4_dx);
 *   - the routed LoRA equation (routed_rawint4_lora, _base_linear,
 *     _lora_linear, rawint4_swiglu) and its gradients with respect to the
 *     inputs, the route weights and the six LoRA tensors (run_routed_reference,
 *     which takes them from autograd; here they are written out by hand and
 *     pinned by finite differences and an independent autograd check).
 *
 * Precision: every dot product and every token reduction accumulates in double.
 * With fp32_intermediates = 1 each tensor the reference materialises in fp32
 * (LoRA-A products, gate/up pre-activations, h, y, and their gradients) is
 * rounded to fp32 once, so that the clamp masks are decided on fp32
 * pre-activations as the pages require (commit "fix RAWINT4 SFT wrapper and
 * clamp gradients").  With fp32_intermediates = 0 everything stays in double
 * (used for finite-difference checks).
 *
 * Readings where the pages leave a step open:
 *   - expert ids outside [0, E) are dropped (contribute nothing) and counted;
 *   - the clamp is boundary-inclusive on both sides: the gate passes its
 *     gradient where g <= L, the up projection where -L <= u <= L; L = 0 turns
 *     the clamp off;
 *   - the LoRA scale is alpha / rank;
 *   - a pre-activation on a clamp bound to within the accuracy of the
 *     computation being checked has no unique mask; orc_moe_decided lets the
 *     caller fix the side there (and only there), within a band it gives or
 *     within the a priori error bound of an fp32 computation (preact_bound).
 *
 * Loop order: experts outermost; each active expert is dequantised once and its
 * routed slots are processed together, parallel over output features.  Every
 * output element is one fixed-order sum, so results do not depend on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_GROUP_SIZE 32

#define ORC_FORMAT_RAWINT4 0
#define ORC_FORMAT_MXFP4 1

typedef struct {
  int32_t num_experts, top_k, hidden, intermediate, rank;
  int32_t fp32_intermediates, weight_format; /* ORC_FORMAT_* */
  double alpha, swiglu_limit;
  const uint8_t *gate_packed, *up_packed, *down_packed;    /* [E,I,H/2] [E,I,H/2] [E,H,I/2] */
  const uint16_t *gate_scale, *up_scale, *down_scale;      /* bf16 bits, [E,I,H/32] [E,I,H/32] [E,H,I/32] */
  const double *gate_a, *gate_b, *up_a, *up_b, *down_a, *down_b; /* [E,r,H] [E,I,r] [E,r,H] [E,I,r] [E,r,I] [E,H,r] */
} orc_layer;

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static inline double fp32_round(int enabled, double v) { return enabled ? (double)(float)v : v; }

/* ---------------------------------------------------------------- codec */

/* unpack_rawint4: each byte gives (low nibble - 8, high nibble - 8). */
void orc_unpack(const uint8_t* packed, int64_t nbytes, int8_t* values) {
  for (int64_t i = 0; i < nbytes; ++i) {
    values[2 * i] = (int8_t)((int)(packed[i] & 0x0F) - 8);
    values[2 * i + 1] = (int8_t)((int)(packed[i] >> 4) - 8);
  }
}

/* pack_rawint4_codes: codes in [0, 15], an even count, even index -> low nibble. */
int orc_pack(const int32_t* codes, int64_t count, uint8_t* packed) {
  if (count % 2) return -1;
  for (int64_t i = 0; i < count; ++i)
    if (codes[i] < 0 || codes[i] > 15) return -2;
  for (int64_t i = 0; i < count / 2; ++i)
    packed[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
  return 0;
}

/* _validate_rawint4_layout: group size 32, K = 2 * packed columns divisible by it,
 * scales exactly [N, K/32]. */
int orc_validate_layout(int64_t n, int64_t packed_cols, int64_t scale_rows, int64_t scale_cols,
                        int32_t group_size) {
  if (group_size != ORC_GROUP_SIZE) return -1;
  int64_t k = packed_cols * 2;
  if (k % group_size) return -2;
  if (scale_rows != n || scale_cols != k / group_size) return -3;
  return 0;
}

/* E2M1 (OCP microscaling FP4): (-1)^s * 2^(e - 1) * (1 + m / 2) for e > 0,
 * (-1)^s * m / 2 for e == 0 (subnormal; bias 1). */
static double e2m1_value(int nib) {
  const int sign = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
  const double mag = e ? ldexp(1.0 + 0.5 * m, e - 1) : 0.5 * m;
  return sign ? -mag : mag;
}

/* the unscaled value of one nibble in either weight format */
static double code_value(int fmt, int nib) { return fmt == ORC_FORMAT_MXFP4 ? e2m1_value(nib) : (double)(nib - 8); }

/* E2M1 value of each nibble 0..15 (the table the pins compare). */
void orc_e2m1_table(double* out) {
  for (int c = 0; c < 16; ++c) out[c] = e2m1_value(c);
}

static double weight_at(int fmt, const uint8_t* packed, const uint16_t* scales, int64_t k, int64_t row,
                        int64_t col) {
  uint8_t byte = packed[row * (k / 2) + col / 2];
  int nib = (col & 1) ? (byte >> 4) : (byte & 0x0F);
  return code_value(fmt, nib) * bf16_value(scales[row * (k / ORC_GROUP_SIZE) + col / ORC_GROUP_SIZE]);
}

/* dequantize_rawint4 (and its MXFP4 twin): dense [N, K]; a code value times a
 * bf16 scale has at most 3 + 8 significant bits, exact in fp32 (in range). */
int orc_dequant_format(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, int32_t fmt, float* w) {
  if (k % ORC_GROUP_SIZE) return -2;
  if (fmt != ORC_FORMAT_RAWINT4 && fmt != ORC_FORMAT_MXFP4) return -3;
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < n; ++row)
    for (int64_t col = 0; col < k; ++col) w[row * k + col] = (float)weight_at(fmt, packed, scales, k, row, col);
  return 0;
}

int orc_dequant(const uint8_t* packed, const uint16_t* scales, int64_t n, int64_t k, float* w) {
  return orc_dequant_format(packed, scales, n, k, ORC_FORMAT_RAWINT4, w);
}

/* transpose_free_rawint4_dx: dX[M,K] = dY[M,N] W[N,K] using only original rows,
 * one 32-wide group of one row decoded at a time. */
int orc_transpose_free_dx_format(const double* dy, int64_t m, const uint8_t* packed, const uint16_t* scales,
                                 int64_t n, int64_t k, int32_t fmt, double* dx) {
  if (k % ORC_GROUP_SIZE) return -2;
  if (fmt != ORC_FORMAT_RAWINT4 && fmt != ORC_FORMAT_MXFP4) return -3;
  memset(dx, 0, sizeof(double) * (size_t)(m * k));
  for (int64_t group = 0; group < k / ORC_GROUP_SIZE; ++group) {
    int64_t k0 = group * ORC_GROUP_SIZE;
    for (int64_t row = 0; row < n; ++row) {
      double values[ORC_GROUP_SIZE];
      double scale = bf16_value(scales[row * (k / ORC_GROUP_SIZE) + group]);
      for (int j = 0; j < ORC_GROUP_SIZE / 2; ++j) {
        uint8_t byte = packed[row * (k / 2) + k0 / 2 + j];
        values[2 * j] = code_value(fmt, byte & 0x0F) * scale;
        values[2 * j + 1] = code_value(fmt, byte >> 4) * scale;
      }
      for (int64_t i = 0; i < m; ++i) {
        double g = dy[i * n + row];
        for (int j = 0; j < ORC_GROUP_SIZE; ++j) dx[i * k + k0 + j] += g * values[j];
      }
    }
  }
  return 0;
}

int orc_transpose_free_dx(const double* dy, int64_t m, const uint8_t* packed, const uint16_t* scales, int64_t n,
                          int64_t k, double* dx) {
  return orc_transpose_free_dx_format(dy, m, packed, scales, n, k, ORC_FORMAT_RAWINT4, dx);
}

/* ---------------------------------------------------------------- routing */

/* Token-slot grouping: counts per expert, exclusive offsets, and the flat slot
 * indices t*top_k+s sorted by expert, stable in slot order.  Ids outside
 * [0, E) are dropped and counted in *bad. */
int orc_group(const int64_t* ids, int64_t qlen, int32_t top_k, int32_t num_experts, int32_t* counts,
              int32_t* offsets, int32_t* sorted_slot, int64_t* bad) {
  if (qlen < 0 || top_k < 1 || num_experts < 1) return -1;
  int64_t slots = qlen * top_k;
  int64_t nbad = 0;
  memset(counts, 0, sizeof(int32_t) * (size_t)num_experts);
  for (int64_t s = 0; s < slots; ++s) {
    if (ids[s] < 0 || ids[s] >= num_experts)
      ++nbad;
    else
      ++counts[ids[s]];
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < num_experts; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)num_experts);
  if (!cursor) return -9;
  memcpy(cursor, offsets, sizeof(int32_t) * (size_t)num_experts);
  for (int64_t s = 0; s < slots; ++s)
    if (ids[s] >= 0 && ids[s] < num_experts) sorted_slot[cursor[ids[s]]++] = (int32_t)s;
  free(cursor);
  *bad = nbad;
  return 0;
}

/* ---------------------------------------------------------------- activation */

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }
static double silu(double z) { return z * sigmoid(z); }
/* d/dz z*sigmoid(z) = sigmoid(z) * (1 + z * (1 - sigmoid(z))) */
static double silu_grad(double z) {
  double s = sigmoid(z);
  return s * (1.0 + z * (1.0 - s));
}

/* rawint4_swiglu's clamp: gate clamped from above only, up clamped to [-L, L];
 * the mask is 1 where the un-clamped value passes its gradient (boundaries
 * included); limit 0 means no clamp.  The decision is taken on `side` (the
 * value itself unless a decision is supplied, see orc_moe_decided); the
 * clamped value is the value itself where it passes, the bound it is beyond
 * otherwise. */
static void clamp_gate(double g, double side, double limit, double* clamped, double* mask) {
  if (limit > 0 && !(side <= limit)) {
    *clamped = limit;
    *mask = 0.0;
  } else {
    *clamped = g;
    *mask = 1.0;
  }
}
static void clamp_up(double u, double side, double limit, double* clamped, double* mask) {
  if (limit > 0 && side < -limit) {
    *clamped = -limit;
    *mask = 0.0;
  } else if (limit > 0 && side > limit) {
    *clamped = limit;
    *mask = 0.0;
  } else {
    *clamped = u;
    *mask = 1.0;
  }
}

/* ---------------------------------------------------------------- a priori error bound

 * How far an fp32 computation of a gate/up pre-activation may lie from the
 * exact value, before any knowledge of its result.  The computation is taken
 * to form the base products w x exactly (the decoded weights and the
 * activations are exact in its arithmetic), the LoRA factors with a relative
 * error of at most 2^-13 each, and to add everything in fp32 in any order.
 * The fp32 sums use the probabilistic bound of Higham and Mary ("A new
 * approach to probabilistic rounding error analysis", SIAM J. Sci. Comput.
 * 41(5), 2019, Theorem 2.4): the sum of n terms lies within
 * gamma(n) = exp(lambda sqrt(n) u + n u^2 / (1 - u)) - 1 times the sum of
 * their magnitudes, with probability at least 1 - 2 n exp(-lambda^2 (1 - u)^2 / 2)
 * (u = 2^-24; lambda = 8 makes that 1 - 1.8e-10 at n = 7168).  So, for
 * g = sum_k w_k x_k + sc sum_q B_q a_q with a_q = sum_k A_qk x_k:
 *
 *   bound = u |g|                                   (the oracle's own fp32 rounding)
 *         + gamma(K + R + 1) (sum_k |w_k x_k| + sc sum_q |B_q a_q|)
 *         + 2^-12 sc (sum_q |B_q a_q| + sum_q |B_q| sum_k |A_qk x_k|)
 *
 * the last line covering the relative errors of the LoRA factors (two per
 * product of the B term; the A products' errors carried through B). */
static double gamma_prob(double n) {
  const double u = 0x1p-24, lambda = 8.0;
  return expm1(lambda * sqrt(n) * u + n * u * u / (1.0 - u));
}

static double preact_bound(double g, double sw, double sb, double sab, double sc, int64_t K, int64_t R) {
  return 0x1p-24 * fabs(g) + gamma_prob((double)(K + R + 1)) * (sw + sc * sb) + 0x1p-12 * sc * (sb + sab);
}

/* ---------------------------------------------------------------- dense helpers */

static double dot_dd(const double* a, const double* b, int64_t n) {
  double acc = 0.0;
#pragma omp simd reduction(+ : acc)
  for (int64_t i = 0; i < n; ++i) acc += a[i] * b[i];
  return acc;
}
static double dot_fd(const float* a, const double* b, int64_t n) {
  double acc = 0.0;
#pragma omp simd reduction(+ : acc)
  for (int64_t i = 0; i < n; ++i) acc += (double)a[i] * b[i];
  return acc;
}
/* sums of the magnitudes of the products (for the error bound) */
static double absdot_dd(const double* a, const double* b, int64_t n) {
  double acc = 0.0;
  for (int64_t i = 0; i < n; ++i) acc += fabs(a[i] * b[i]);
  return acc;
}
static double absdot_fd(const float* a, const double* b, int64_t n) {
  double acc = 0.0;
  for (int64_t i = 0; i < n; ++i) acc += fabs((double)a[i] * b[i]);
  return acc;
}

/* out[j][c] = sum_r W[r][c] v[j][r] (+ sum_r W2[r][c] v2[j][r]) for j < m, c < C.
 * W is [Rn][C] row-major; rows are streamed once per block of output columns and
 * every output element sums over r in increasing order (first W, then W2). */
static void transposed_products(const float* W, int64_t Rn, int64_t C, const double* v, int64_t vstride, int64_t m,
                                const float* W2, int64_t Rn2, const double* v2, int64_t v2stride, double* out,
                                int64_t ostride) {
  const int64_t BLK = 64;
#pragma omp parallel for schedule(static)
  for (int64_t c0 = 0; c0 < C; c0 += BLK) {
    int64_t cn = C - c0 < BLK ? C - c0 : BLK;
    double* acc = (double*)calloc((size_t)(m * BLK), sizeof(double));
    for (int pass = 0; pass < (W2 ? 2 : 1); ++pass) {
      const float* w = pass ? W2 : W;
      const double* vv = pass ? v2 : v;
      int64_t rn = pass ? Rn2 : Rn, vs = pass ? v2stride : vstride;
      for (int64_t r = 0; r < rn; ++r) {
        const float* wr = w + r * C + c0;
        for (int64_t j = 0; j < m; ++j) {
          double vj = vv[j * vs + r];
          double* a = acc + j * BLK;
          for (int64_t c = 0; c < cn; ++c) a[c] += (double)wr[c] * vj;
        }
      }
    }
    for (int64_t j = 0; j < m; ++j)
      for (int64_t c = 0; c < cn; ++c) out[j * ostride + c0 + c] = acc[j * BLK + c];
    free(acc);
  }
}

/* ---------------------------------------------------------------- layer */

/*
 * routed_rawint4_lora and its gradients.  For every valid slot (t, s), e = ids[t,s]:
 *   ua = A_g x, ub = A_u x                       (x = inputs[t])
 *   g  = W_g x + sc B_g ua,   u = W_u x + sc B_u ub
 *   h  = silu(clamp_gate(g)) * clamp_up(u)
 *   ud = A_d h,   y = W_d h + sc B_d ud
 *   out[t] += rw[t,s] * y
 * and with dy = grad_output given, the cotangent of y is dyw = rw * dy[t]:
 *   droute[t,s] = <dy[t], y>
 *   dyB = B_d^T dyw;  dh = W_d^T dyw + sc A_d^T dyB
 *   dg = dh * up' * silu'(g') * mask_g;  du = dh * silu(g') * mask_u
 *   dgB = B_g^T dg;  duB = B_u^T du
 *   dx[t] += W_g^T dg + W_u^T du + sc (A_g^T dgB + A_u^T duB)
 *   dB_d += sc dyw (x) ud,  dA_d += sc dyB (x) h
 *   dB_g += sc dg (x) ua,   dA_g += sc dgB (x) x    (likewise for up)
 * The six LoRA gradients returned are these raw sums (no window scaling).
 *
 * The clamp masks are discontinuous at g = L and u = -L, L: a pre-activation
 * that another computation (another summation order, another precision) holds
 * only to within `band` may fall on either side there, and either mask is then
 * a correct result.  With side_g / side_u given ([qlen * top_k][I] in slot
 * order, the pre-activations that computation found), an element whose own
 * value lies within `band` of a bound takes its decision from the supplied
 * value; everywhere else, and with NULL, the oracle decides on its own value.
 * A negative `band` means each element's own a priori bound (preact_bound).
 * pre_g / pre_u, when given ([qlen * top_k][I], slot order), receive the
 * oracle's own pre-activations of every valid slot (other rows untouched), and
 * bnd_g / bnd_u their a priori bounds.
 */
int orc_moe_decided(const orc_layer* L, int64_t qlen, const double* x, const int64_t* ids, const double* rw,
                    const double* dy, double* out, double* dx, double* droute, double* d_gate_a, double* d_gate_b,
                    double* d_up_a, double* d_up_b, double* d_down_a, double* d_down_b, const double* side_g,
                    const double* side_u, double band, double* pre_g, double* pre_u, double* bnd_g,
                    double* bnd_u) {
  if (!L || qlen < 0) return -1;
  const int64_t E = L->num_experts, K = L->top_k, H = L->hidden, I = L->intermediate, R = L->rank;
  if (E < 1 || K < 1 || R < 1 || H % ORC_GROUP_SIZE || I % ORC_GROUP_SIZE || H <= 0 || I <= 0) return -1;
  if (!(L->swiglu_limit >= 0.0) || !isfinite(L->swiglu_limit)) return -1;
  if (L->weight_format != ORC_FORMAT_RAWINT4 && L->weight_format != ORC_FORMAT_MXFP4) return -1;
  const int fr = L->fp32_intermediates;
  const double sc = L->alpha / (double)R, limit = L->swiglu_limit;
  const int64_t slots = qlen * K;
  const int bwd = dy != NULL;

  memset(out, 0, sizeof(double) * (size_t)(qlen * H));
  if (bwd) {
    memset(dx, 0, sizeof(double) * (size_t)(qlen * H));
    memset(droute, 0, sizeof(double) * (size_t)slots);
    memset(d_gate_a, 0, sizeof(double) * (size_t)(E * R * H));
    memset(d_up_a, 0, sizeof(double) * (size_t)(E * R * H));
    memset(d_gate_b, 0, sizeof(double) * (size_t)(E * I * R));
    memset(d_up_b, 0, sizeof(double) * (size_t)(E * I * R));
    memset(d_down_a, 0, sizeof(double) * (size_t)(E * R * I));
    memset(d_down_b, 0, sizeof(double) * (size_t)(E * H * R));
  }
  if (slots == 0) return 0;

  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* sorted = (int32_t*)malloc(sizeof(int32_t) * (size_t)slots);
  double* yslot = (double*)calloc((size_t)(slots * H), sizeof(double));
  double* dxslot = bwd ? (double*)calloc((size_t)(slots * H), sizeof(double)) : NULL;
  float* wg = (float*)malloc(sizeof(float) * (size_t)(I * H));
  float* wu = (float*)malloc(sizeof(float) * (size_t)(I * H));
  float* wd = (float*)malloc(sizeof(float) * (size_t)(H * I));
  int64_t nbad = 0;
  int status = 0;
  if (!counts || !offsets || !sorted || !yslot || (bwd && !dxslot) || !wg || !wu || !wd) {
    status = -9;
    goto done;
  }
  orc_group(ids, qlen, (int32_t)K, (int32_t)E, counts, offsets, sorted, &nbad);

  for (int64_t e = 0; e < E; ++e) {
    const int64_t m = counts[e];
    if (m == 0) continue;
    const int32_t* rows = sorted + offsets[e];
    orc_dequant_format(L->gate_packed + e * I * (H / 2), L->gate_scale + e * I * (H / 32), I, H, L->weight_format, wg);
    orc_dequant_format(L->up_packed + e * I * (H / 2), L->up_scale + e * I * (H / 32), I, H, L->weight_format, wu);
    orc_dequant_format(L->down_packed + e * H * (I / 2), L->down_scale + e * H * (I / 32), H, I, L->weight_format, wd);
    const double* ag = L->gate_a + e * R * H;
    const double* bg = L->gate_b + e * I * R;
    const double* au = L->up_a + e * R * H;
    const double* bu = L->up_b + e * I * R;
    const double* ad = L->down_a + e * R * I;
    const double* bd = L->down_b + e * H * R;

    double* ua = (double*)malloc(sizeof(double) * (size_t)(m * R));
    double* ub = (double*)malloc(sizeof(double) * (size_t)(m * R));
    double* ud = (double*)malloc(sizeof(double) * (size_t)(m * R));
    double* gp = (double*)malloc(sizeof(double) * (size_t)(m * I)); /* clamped gate */
    double* upc = (double*)malloc(sizeof(double) * (size_t)(m * I)); /* clamped up */
    double* mg = (double*)malloc(sizeof(double) * (size_t)(m * I));
    double* mu = (double*)malloc(sizeof(double) * (size_t)(m * I));
    double* hh = (double*)malloc(sizeof(double) * (size_t)(m * I));
    /* a priori bounds: sum_k |A_qk x_k| per slot row and rank index */
    const int need_bound = band < 0 || bnd_g || bnd_u;
    double* sag = need_bound ? (double*)malloc(sizeof(double) * (size_t)(m * R)) : NULL;
    double* sau = need_bound ? (double*)malloc(sizeof(double) * (size_t)(m * R)) : NULL;
    if (!ua || !ub || !ud || !gp || !upc || !mg || !mu || !hh || (need_bound && (!sag || !sau))) {
      status = -9;
      free(ua); free(ub); free(ud); free(gp); free(upc); free(mg); free(mu); free(hh); free(sag); free(sau);
      goto done;
    }

    /* LoRA-A of gate and up: ua = A_g x, ub = A_u x */
#pragma omp parallel for schedule(static)
    for (int64_t jq = 0; jq < m * R; ++jq) {
      int64_t j = jq / R, q = jq % R;
      const double* xt = x + (rows[j] / K) * H;
      ua[jq] = fp32_round(fr, dot_dd(ag + q * H, xt, H));
      ub[jq] = fp32_round(fr, dot_dd(au + q * H, xt, H));
      if (need_bound) {
        sag[jq] = absdot_dd(ag + q * H, xt, H);
        sau[jq] = absdot_dd(au + q * H, xt, H);
      }
    }
    /* gate/up pre-activations, clamp, h */
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < I; ++n) {
      for (int64_t j = 0; j < m; ++j) {
        const double* xt = x + (rows[j] / K) * H;
        double g = dot_fd(wg + n * H, xt, H) + sc * dot_dd(bg + n * R, ua + j * R, R);
        double u = dot_fd(wu + n * H, xt, H) + sc * dot_dd(bu + n * R, ub + j * R, R);
        g = fp32_round(fr, g);
        u = fp32_round(fr, u);
        int64_t idx = j * I + n;
        const int64_t sidx = (int64_t)rows[j] * I + n;
        if (pre_g) pre_g[sidx] = g;
        if (pre_u) pre_u[sidx] = u;
        double band_g = band, band_u = band;
        if (need_bound) {
          double sab_g = 0.0, sab_u = 0.0;
          for (int64_t q = 0; q < R; ++q) {
            sab_g += fabs(bg[n * R + q]) * sag[j * R + q];
            sab_u += fabs(bu[n * R + q]) * sau[j * R + q];
          }
          const double bg_e = preact_bound(g, absdot_fd(wg + n * H, xt, H), absdot_dd(bg + n * R, ua + j * R, R),
                                           sab_g, sc, H, R);
          const double bu_e = preact_bound(u, absdot_fd(wu + n * H, xt, H), absdot_dd(bu + n * R, ub + j * R, R),
                                           sab_u, sc, H, R);
          if (bnd_g) bnd_g[sidx] = bg_e;
          if (bnd_u) bnd_u[sidx] = bu_e;
          if (band < 0) {
            band_g = bg_e;
            band_u = bu_e;
          }
        }
        /* within the band of a bound the mask is not unique: take the supplied side */
        const double sg = (side_g && limit > 0 && fabs(g - limit) <= band_g) ? side_g[sidx] : g;
        const double su =
            (side_u && limit > 0 && (fabs(u - limit) <= band_u || fabs(u + limit) <= band_u)) ? side_u[sidx] : u;
        clamp_gate(g, sg, limit, &gp[idx], &mg[idx]);
        clamp_up(u, su, limit, &upc[idx], &mu[idx]);
        hh[idx] = fp32_round(fr, silu(gp[idx]) * upc[idx]);
      }
    }
    /* down LoRA-A: ud = A_d h */
#pragma omp parallel for schedule(static)
    for (int64_t jq = 0; jq < m * R; ++jq) {
      int64_t j = jq / R, q = jq % R;
      ud[jq] = fp32_round(fr, dot_dd(ad + q * I, hh + j * I, I));
    }
    /* down projection: y = W_d h + sc B_d ud, kept per slot */
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < H; ++n)
      for (int64_t j = 0; j < m; ++j)
        yslot[(int64_t)rows[j] * H + n] =
            fp32_round(fr, dot_fd(wd + n * I, hh + j * I, I) + sc * dot_dd(bd + n * R, ud + j * R, R));

    if (bwd) {
      double* dyw = (double*)malloc(sizeof(double) * (size_t)(m * H));
      double* dyb = (double*)malloc(sizeof(double) * (size_t)(m * R));
      double* dh = (double*)malloc(sizeof(double) * (size_t)(m * I));
      double* dg = (double*)malloc(sizeof(double) * (size_t)(m * I));
      double* du = (double*)malloc(sizeof(double) * (size_t)(m * I));
      double* dgb = (double*)malloc(sizeof(double) * (size_t)(m * R));
      double* dub = (double*)malloc(sizeof(double) * (size_t)(m * R));
      if (!dyw || !dyb || !dh || !dg || !du || !dgb || !dub) {
        status = -9;
        free(dyw); free(dyb); free(dh); free(dg); free(du); free(dgb); free(dub);
        free(ua); free(ub); free(ud); free(gp); free(upc); free(mg); free(mu); free(hh); free(sag); free(sau);
        goto done;
      }
      /* route-weight gradient and the cotangent of y */
      for (int64_t j = 0; j < m; ++j) {
        const int64_t slot = rows[j];
        const double* dyt = dy + (slot / K) * H;
        droute[slot] = fp32_round(fr, dot_dd(dyt, yslot + slot * H, H));
        for (int64_t n = 0; n < H; ++n) dyw[j * H + n] = fp32_round(fr, rw[slot] * dyt[n]);
      }
      /* dyB = B_d^T dyw */
#pragma omp parallel for schedule(static)
      for (int64_t jq = 0; jq < m * R; ++jq) {
        int64_t j = jq / R, q = jq % R;
        double acc = 0.0;
        for (int64_t n = 0; n < H; ++n) acc += bd[n * R + q] * dyw[j * H + n];
        dyb[jq] = fp32_round(fr, acc);
      }
      /* dh = W_d^T dyw + sc A_d^T dyB, then the SwiGLU / clamp gradient */
      transposed_products(wd, H, I, dyw, H, m, NULL, 0, NULL, 0, dh, I);
#pragma omp parallel for schedule(static)
      for (int64_t i = 0; i < I; ++i) {
        for (int64_t j = 0; j < m; ++j) {
          double lora = 0.0;
          for (int64_t q = 0; q < R; ++q) lora += ad[q * I + i] * dyb[j * R + q];
          int64_t idx = j * I + i;
          dh[idx] = fp32_round(fr, dh[idx] + sc * lora);
          dg[idx] = fp32_round(fr, dh[idx] * upc[idx] * silu_grad(gp[idx]) * mg[idx]);
          du[idx] = fp32_round(fr, dh[idx] * silu(gp[idx]) * mu[idx]);
        }
      }
      /* dgB = B_g^T dg, duB = B_u^T du */
#pragma omp parallel for schedule(static)
      for (int64_t jq = 0; jq < m * R; ++jq) {
        int64_t j = jq / R, q = jq % R;
        double a = 0.0, b = 0.0;
        for (int64_t i = 0; i < I; ++i) {
          a += bg[i * R + q] * dg[j * I + i];
          b += bu[i * R + q] * du[j * I + i];
        }
        dgb[jq] = fp32_round(fr, a);
        dub[jq] = fp32_round(fr, b);
      }
      /* per-slot dx = W_g^T dg + W_u^T du + sc (A_g^T dgB + A_u^T duB) */
      double* dxs = (double*)malloc(sizeof(double) * (size_t)(m * H));
      if (!dxs) {
        status = -9;
        free(dyw); free(dyb); free(dh); free(dg); free(du); free(dgb); free(dub);
        free(ua); free(ub); free(ud); free(gp); free(upc); free(mg); free(mu); free(hh); free(sag); free(sau);
        goto done;
      }
      transposed_products(wg, I, H, dg, I, m, wu, I, du, I, dxs, H);
#pragma omp parallel for schedule(static)
      for (int64_t n = 0; n < H; ++n) {
        for (int64_t j = 0; j < m; ++j) {
          double lora = 0.0;
          for (int64_t q = 0; q < R; ++q) lora += ag[q * H + n] * dgb[j * R + q] + au[q * H + n] * dub[j * R + q];
          dxslot[(int64_t)rows[j] * H + n] = fp32_round(fr, dxs[j * H + n] + sc * lora);
        }
      }
      free(dxs);
      /* LoRA gradients of expert e: sums over its slots in slot order */
      double* Gda = d_down_a + e * R * I;
      double* Gdb = d_down_b + e * H * R;
      double* Gga = d_gate_a + e * R * H;
      double* Ggb = d_gate_b + e * I * R;
      double* Gua = d_up_a + e * R * H;
      double* Gub = d_up_b + e * I * R;
#pragma omp parallel for schedule(static)
      for (int64_t nq = 0; nq < H * R; ++nq) {
        int64_t n = nq / R, q = nq % R;
        double acc = 0.0;
        for (int64_t j = 0; j < m; ++j) acc += dyw[j * H + n] * ud[j * R + q];
        Gdb[nq] = fp32_round(fr, sc * acc);
      }
#pragma omp parallel for schedule(static)
      for (int64_t qi = 0; qi < R * I; ++qi) {
        int64_t q = qi / I, i = qi % I;
        double acc = 0.0;
        for (int64_t j = 0; j < m; ++j) acc += dyb[j * R + q] * hh[j * I + i];
        Gda[qi] = fp32_round(fr, sc * acc);
      }
#pragma omp parallel for schedule(static)
      for (int64_t iq = 0; iq < I * R; ++iq) {
        int64_t i = iq / R, q = iq % R;
        double a = 0.0, b = 0.0;
        for (int64_t j = 0; j < m; ++j) {
          a += dg[j * I + i] * ua[j * R + q];
          b += du[j * I + i] * ub[j * R + q];
        }
        Ggb[iq] = fp32_round(fr, sc * a);
        Gub[iq] = fp32_round(fr, sc * b);
      }
#pragma omp parallel for schedule(static)
      for (int64_t qn = 0; qn < R * H; ++qn) {
        int64_t q = qn / H, n = qn % H;
        double a = 0.0, b = 0.0;
        for (int64_t j = 0; j < m; ++j) {
          double xv = x[(rows[j] / K) * H + n];
          a += dgb[j * R + q] * xv;
          b += dub[j * R + q] * xv;
        }
        Gga[qn] = fp32_round(fr, sc * a);
        Gua[qn] = fp32_round(fr, sc * b);
      }
      free(dyw); free(dyb); free(dh); free(dg); free(du); free(dgb); free(dub);
    }
    free(ua); free(ub); free(ud); free(gp); free(upc); free(mg); free(mu); free(hh); free(sag); free(sau);
  }

  /* weighted slot sums per token, slots in order; dropped slots add nothing */
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < qlen; ++t) {
    for (int64_t n = 0; n < H; ++n) {
      double acc = 0.0, accx = 0.0;
      for (int64_t s = 0; s < K; ++s) {
        int64_t slot = t * K + s;
        if (ids[slot] < 0 || ids[slot] >= E) continue;
        acc += rw[slot] * yslot[slot * H + n];
        if (bwd) accx += dxslot[slot * H + n];
      }
      out[t * H + n] = fp32_round(fr, acc);
      if (bwd) dx[t * H + n] = fp32_round(fr, accx);
    }
  }

done:
  free(counts); free(offsets); free(sorted); free(yslot); free(dxslot); free(wg); free(wu); free(wd);
  return status;
}

int orc_moe(const orc_layer* L, int64_t qlen, const double* x, const int64_t* ids, const double* rw,
            const double* dy, double* out, double* dx, double* droute, double* d_gate_a, double* d_gate_b,
            double* d_up_a, double* d_up_b, double* d_down_a, double* d_down_b) {
  return orc_moe_decided(L, qlen, x, ids, rw, dy, out, dx, droute, d_gate_a, d_gate_b, d_up_a, d_up_b, d_down_a,
                         d_down_b, NULL, NULL, 0.0, NULL, NULL, NULL, NULL);
}
