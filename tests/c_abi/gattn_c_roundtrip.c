/*
 * A plain C caller of libgattn: device buffers from the HIP runtime, the
 * causal forward and backward through the C ABI (include/gattn.h), and every
 * output compared element by element with the float64 CPU oracle
 * (oracle/libgattn_ref.so) on the same inputs.  No Python, no torch.
 *
 * Inputs are unit-variance normals (splitmix64 and Box-Muller, seeded per
 * case), rounded to the case's storage type (bf16: round to nearest even);
 * the oracle takes the rounded values.  Scale 1/sqrt(hs).  Bars: float32
 * |err| <= 1e-4; bf16 |err| <= 2e-2 + 2^-8 |ref| (the bar plus the rounding
 * of the stored bf16 value).  Also checks that an invalid call is rejected
 * with GATTN_ERR_INVALID_ARG before any launch.
 *
 * Prints one line per case; exit status 0 when every case passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gattn.h"

/* The oracle's backward (it recomputes o and lse as well). */
void gattn_ref_bwd(const double* q, const double* k, const double* v, const double* dO, double* dq,
                   double* dk, double* dv, double* o, double* lse, int B, int H, int T, int hs,
                   double scale, int nthreads);

static uint64_t rng_state;

static uint64_t splitmix64(void) {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Uniform in (0, 1): the top 53 bits, offset by half a step. */
static double uniform01(void) { return ((double)(splitmix64() >> 11) + 0.5) * 0x1.0p-53; }

static double normal(void) {
  const double u1 = uniform01(), u2 = uniform01();
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static uint16_t bf16_bits(float x) { /* round to nearest even; finite inputs only */
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static double bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

#define HIP_OK(call)                                                             \
  do {                                                                           \
    hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #call,              \
              hipGetErrorString(e_));                                            \
      exit(2);                                                                   \
    }                                                                            \
  } while (0)

/* Host values (already rounded to the storage type) -> device buffer. */
static void* upload(const double* x, size_t n, int dtype) {
  const size_t es = dtype == GATTN_F32 ? 4 : 2;
  void* h = malloc(n * es);
  void* d = NULL;
  for (size_t i = 0; i < n; ++i) {
    if (dtype == GATTN_F32)
      ((float*)h)[i] = (float)x[i];
    else
      ((uint16_t*)h)[i] = bf16_bits((float)x[i]);
  }
  HIP_OK(hipMalloc(&d, n * es));
  HIP_OK(hipMemcpy(d, h, n * es, hipMemcpyHostToDevice));
  free(h);
  return d;
}

static void download(double* x, const void* d, size_t n, int dtype) {
  const size_t es = dtype == GATTN_F32 ? 4 : 2;
  void* h = malloc(n * es);
  HIP_OK(hipMemcpy(h, d, n * es, hipMemcpyDeviceToHost));
  for (size_t i = 0; i < n; ++i)
    x[i] = dtype == GATTN_F32 ? (double)((float*)h)[i] : bf16_value(((uint16_t*)h)[i]);
  free(h);
}

/* Largest |got - ref| and whether every element is within tol + rel |ref|. */
static int within(const double* got, const double* ref, size_t n, double tol, double rel,
                  double* worst) {
  int ok = 1;
  *worst = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double e = fabs(got[i] - ref[i]);
    if (!(e <= tol + rel * fabs(ref[i]))) ok = 0;
    if (e > *worst || e != e) *worst = e;
  }
  return ok;
}

static int run_case(int dtype, int B, int H, int T, int hs, uint64_t seed) {
  const size_t n = (size_t)B * H * T * hs, nr = (size_t)B * H * T;
  const double scale = 1.0 / sqrt((double)hs);
  double* in[4];
  rng_state = seed;
  for (int t = 0; t < 4; ++t) { /* q, k, v, dO */
    in[t] = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) {
      const double x = normal();
      in[t][i] = dtype == GATTN_F32 ? (double)(float)x : bf16_value(bf16_bits((float)x));
    }
  }
  void* dq_in = upload(in[0], n, dtype);
  void* dk_in = upload(in[1], n, dtype);
  void* dv_in = upload(in[2], n, dtype);
  void* ddo = upload(in[3], n, dtype);
  const size_t es = dtype == GATTN_F32 ? 4 : 2;
  void *d_o, *d_dq, *d_dk, *d_dv, *d_ws;
  float* d_lse;
  HIP_OK(hipMalloc(&d_o, n * es));
  HIP_OK(hipMalloc(&d_dq, n * es));
  HIP_OK(hipMalloc(&d_dk, n * es));
  HIP_OK(hipMalloc(&d_dv, n * es));
  HIP_OK(hipMalloc((void**)&d_lse, nr * sizeof(float)));
  const size_t wsb = gattn_bwd_workspace_bytes(B, H, T, hs, dtype);
  HIP_OK(hipMalloc(&d_ws, wsb));

  int st = gattn_fwd(dq_in, dk_in, dv_in, d_o, d_lse, B, H, T, hs, (float)scale, dtype, NULL);
  if (st == GATTN_OK)
    st = gattn_bwd(dq_in, dk_in, dv_in, d_o, ddo, d_lse, d_dq, d_dk, d_dv, B, H, T, hs,
                   (float)scale, dtype, d_ws, wsb, NULL);
  HIP_OK(hipDeviceSynchronize());
  if (st != GATTN_OK) {
    printf("dtype %d B=%d H=%d T=%d hs=%d: call failed: %s\n", dtype, B, H, T, hs,
           gattn_status_string(st));
    return 0;
  }

  double* got[5];
  double* ref[5];
  for (int t = 0; t < 5; ++t) {
    const size_t m = t == 4 ? nr : n;
    got[t] = malloc(m * sizeof(double));
    ref[t] = malloc(m * sizeof(double));
  }
  download(got[0], d_dq, n, dtype);
  download(got[1], d_dk, n, dtype);
  download(got[2], d_dv, n, dtype);
  download(got[3], d_o, n, dtype);
  download(got[4], d_lse, nr, GATTN_F32);
  gattn_ref_bwd(in[0], in[1], in[2], in[3], ref[0], ref[1], ref[2], ref[3], ref[4], B, H, T, hs,
                scale, 0);

  static const char* names[5] = {"dq", "dk", "dv", "o", "lse"};
  const double tol = dtype == GATTN_F32 ? 1e-4 : 2e-2;
  const double rel = dtype == GATTN_F32 ? 0.0 : 0x1.0p-8;
  int ok = 1;
  printf("dtype %s B=%d H=%d T=%d hs=%d:", dtype == GATTN_F32 ? "f32" : "bf16", B, H, T, hs);
  for (int t = 0; t < 5; ++t) {
    double worst;
    const int good = within(got[t], ref[t], t == 4 ? nr : n, tol, rel, &worst);
    printf(" %s %.3g%s", names[t], worst, good ? "" : " FAIL");
    ok &= good;
  }
  printf("\n");

  for (int t = 0; t < 5; ++t) {
    free(got[t]);
    free(ref[t]);
  }
  for (int t = 0; t < 4; ++t) free(in[t]);
  void* dev[] = {dq_in, dk_in, dv_in, ddo, d_o, d_dq, d_dk, d_dv, d_lse, d_ws};
  for (size_t i = 0; i < sizeof(dev) / sizeof(dev[0]); ++i) HIP_OK(hipFree(dev[i]));
  return ok;
}

int main(void) {
  int ok = 1;
  /* Rejected before any launch: T = 0 (the pointers are never dereferenced). */
  float* p = NULL;
  HIP_OK(hipMalloc((void**)&p, 256));
  const int bad = gattn_fwd(p, p, p, p, NULL, 1, 1, 0, 64, 0.125f, GATTN_BF16, NULL);
  printf("T=0 rejected: %s\n", gattn_status_string(bad));
  ok &= bad == GATTN_ERR_INVALID_ARG;
  HIP_OK(hipFree(p));

  ok &= run_case(GATTN_F32, 4, 4, 8, 8, 11);    /* the tiny float32 shape */
  ok &= run_case(GATTN_F32, 2, 3, 37, 16, 12);
  ok &= run_case(GATTN_BF16, 2, 3, 300, 64, 13);
  ok &= run_case(GATTN_BF16, 1, 2, 129, 32, 14);
  printf(ok ? "all cases within their bars\n" : "FAILED\n");
  return ok ? 0 : 1;
}
