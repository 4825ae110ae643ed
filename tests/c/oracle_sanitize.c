/*
 * Drives the C oracle on one small layer (forward and backward, clamp on,
 * one dropped slot) in a build with -fsanitize=address,undefined: any
 * out-of-bounds access, use of freed memory or undefined arithmetic in the
 * oracle aborts the run.  Inputs are a fixed xorshift stream; only the
 * sanitizers' verdict and finiteness are checked here (the values are pinned by
 * the Python tests).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
  int32_t num_experts, top_k, hidden, intermediate, rank;
  int32_t fp32_intermediates, weight_format;
  double alpha, swiglu_limit;
  const uint8_t *gate_packed, *up_packed, *down_packed;
  const uint16_t *gate_scale, *up_scale, *down_scale;
  const double *gate_a, *gate_b, *up_a, *up_b, *down_a, *down_b;
} orc_layer;

int orc_moe(const orc_layer* L, int64_t qlen, const double* x, const int64_t* ids, const double* rw,
            const double* dy, double* out, double* dx, double* droute, double* d_gate_a, double* d_gate_b,
            double* d_up_a, double* d_up_b, double* d_down_a, double* d_down_b);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}
static double unit(void) { return (double)(next() >> 11) / 9007199254740992.0 - 0.5; }

static void* take(size_t n) {
  void* p = malloc(n);
  if (!p) exit(3);
  return p;
}

int main(void) {
  const int E = 3, K = 2, H = 64, I = 96, R = 4, Q = 7;
  for (int fmt = 0; fmt < 2; ++fmt) {
    uint8_t* wp[3];
    uint16_t* ws[3];
    const int64_t rows[3] = {I, I, H}, cols[3] = {H, H, I};
    for (int j = 0; j < 3; ++j) {
      const int64_t nb = E * rows[j] * cols[j] / 2, ns = E * rows[j] * cols[j] / 32;
      wp[j] = take(nb);
      ws[j] = take(2 * ns);
      for (int64_t i = 0; i < nb; ++i) wp[j][i] = (uint8_t)next();
      for (int64_t i = 0; i < ns; ++i) ws[j][i] = fmt ? (uint16_t)((121 + next() % 4) << 7) : 0x3D00;  // 2^-6.. or 1/32
    }
    const int64_t la[6] = {E * R * H, E * I * R, E * R * H, E * I * R, E * R * I, E * H * R};
    double* lora[6];
    double* grads[6];
    for (int j = 0; j < 6; ++j) {
      lora[j] = take(sizeof(double) * la[j]);
      grads[j] = take(sizeof(double) * la[j]);
      for (int64_t i = 0; i < la[j]; ++i) lora[j][i] = 0.04 * unit();
    }
    double* x = take(sizeof(double) * Q * H);
    double* dy = take(sizeof(double) * Q * H);
    double* out = take(sizeof(double) * Q * H);
    double* dx = take(sizeof(double) * Q * H);
    double* rw = take(sizeof(double) * Q * K);
    double* dr = take(sizeof(double) * Q * K);
    int64_t* ids = take(sizeof(int64_t) * Q * K);
    for (int i = 0; i < Q * H; ++i) x[i] = 4 * unit(), dy[i] = unit();
    for (int i = 0; i < Q * K; ++i) ids[i] = (int64_t)(next() % E), rw[i] = 0.5 + unit();
    ids[3] = -1;  // a dropped slot
    orc_layer L = {E, K, H, I, R, 1, fmt, 8.0, 1.0, wp[0], wp[1], wp[2], ws[0], ws[1], ws[2],
                   lora[0], lora[1], lora[2], lora[3], lora[4], lora[5]};
    const int rc = orc_moe(&L, Q, x, ids, rw, dy, out, dx, dr, grads[0], grads[1], grads[2], grads[3], grads[4],
                           grads[5]);
    int finite = 1;
    for (int i = 0; i < Q * H; ++i) finite &= isfinite(out[i]) && isfinite(dx[i]);
    printf("format %d: rc=%d finite=%d out[0]=%.6f\n", fmt, rc, finite, out[0]);
    if (rc != 0 || !finite) return 1;
    for (int j = 0; j < 3; ++j) free(wp[j]), free(ws[j]);
    for (int j = 0; j < 6; ++j) free(lora[j]), free(grads[j]);
    free(x), free(dy), free(out), free(dx), free(rw), free(dr), free(ids);
  }
  return 0;
}
