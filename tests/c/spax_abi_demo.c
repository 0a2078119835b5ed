/*
 * The C ABI of libspax used from plain C, with no Python and no torch: pack a small fp16
 * matrix, build tier masks, run the tiered product, and check the results.
 *
 *   1. An all-FULL TopK mask (n_full = d_in): y must equal the dense product W x.  The
 *      weights and activations are small multiples of 1/64, so every product and partial sum
 *      is exact in fp32 and y is compared with the double-precision sum exactly (up to 1e-6
 *      relative, for the order of the fp32 additions).
 *   2. TopK 100 / 150: the counts are {100, 150, d_in - 250} and both lists are strictly
 *      ascending, disjoint and inside [0, d_in).
 *   3. A NULL activation pointer is rejected with SPAX_ERR_NULL and a message, before
 *      anything is enqueued.
 *
 * Prints one line per check and "spax C ABI demo: ok" at the end; exits 0 only then.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spax.h"

#define D_IN 512
#define D_OUT 256

#define CHECK_HIP(expr)                                                    \
  do {                                                                     \
    hipError_t e_ = (expr);                                                \
    if (e_ != hipSuccess) {                                                \
      printf("HIP error %d at %s\n", (int)e_, #expr);                      \
      return 1;                                                            \
    }                                                                      \
  } while (0)
#define CHECK_SPAX(expr)                                                   \
  do {                                                                     \
    int s_ = (expr);                                                       \
    if (s_ != SPAX_OK) {                                                   \
      printf("spax error %d (%s) at %s\n", s_, spax_last_error(), #expr);  \
      return 1;                                                            \
    }                                                                      \
  } while (0)

/* fp16 bit pattern of k / 64 for |k| < 2048 (exact: such values are fp16 normals or 0). */
static uint16_t half_of_64th(int k) {
  if (k == 0) return 0;
  uint16_t sign = k < 0 ? 0x8000u : 0u;
  double f = fabs((double)k) / 64.0;
  int e;
  double m = frexp(f, &e); /* f = m 2^e, m in [0.5, 1) */
  uint16_t exp16 = (uint16_t)(e - 1 + 15);
  uint16_t mant = (uint16_t)lrint((2.0 * m - 1.0) * 1024.0);
  return (uint16_t)(sign | (uint16_t)(exp16 << 10) | mant);
}

static int w_of(int j, int r) { return (j * 7 + r * 3) % 33 - 16; }
static int x_of(int j) { return (j * 5) % 41 - 20; }

int main(void) {
  printf("%s\n", spax_version());
  static uint16_t hW[D_IN * D_OUT], hx[D_IN];
  for (int j = 0; j < D_IN; ++j) {
    hx[j] = half_of_64th(x_of(j));
    for (int r = 0; r < D_OUT; ++r) hW[j * D_OUT + r] = half_of_64th(w_of(j, r));
  }

  spax_layout L;
  memset(&L, 0, sizeof(L));
  L.n_mats = 1;
  L.d_in = D_IN;
  L.d_out[0] = D_OUT;
  L.base_fmt = SPAX_FMT_FP16;
  L.base_group = 128;
  L.approx_group = 64;
  CHECK_SPAX(spax_layout_init(&L));

  void *W = NULL, *packed = NULL, *x = NULL, *tier = NULL, *f = NULL, *a = NULL, *c = NULL,
       *y = NULL;
  CHECK_HIP(hipMalloc(&W, sizeof(hW)));
  CHECK_HIP(hipMalloc(&packed, (size_t)L.total_bytes));
  CHECK_HIP(hipMalloc(&x, sizeof(hx)));
  CHECK_HIP(hipMalloc(&tier, D_IN));
  CHECK_HIP(hipMalloc(&f, D_IN * sizeof(int32_t)));
  CHECK_HIP(hipMalloc(&a, D_IN * sizeof(int32_t)));
  CHECK_HIP(hipMalloc(&c, 3 * sizeof(int32_t)));
  CHECK_HIP(hipMalloc(&y, D_OUT * sizeof(float)));
  CHECK_HIP(hipMemcpy(W, hW, sizeof(hW), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(x, hx, sizeof(hx), hipMemcpyHostToDevice));

  const uint16_t* Ws[1] = {(const uint16_t*)W};
  CHECK_SPAX(spax_pack_columns(&L, Ws, packed, NULL));

  /* 1. all FULL: the dense product */
  spax_tier_params p;
  memset(&p, 0, sizeof(p));
  p.mode = SPAX_MODE_TOPK;
  p.n_full = D_IN;
  p.n_approx = 0;
  p.approx_den = 1;
  CHECK_SPAX(spax_build_tiers((const uint16_t*)x, D_IN, &p, (uint8_t*)tier, (int32_t*)f,
                              (int32_t*)a, (int32_t*)c, NULL));
  size_t ws_bytes = spax_gemv_workspace_bytes(&L);
  void* ws = NULL;
  if (ws_bytes) CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_SPAX(spax_tiered_gemv(&L, packed, (const uint16_t*)x, (const int32_t*)f,
                              (const int32_t*)a, (const int32_t*)c, (float*)y, ws, ws_bytes,
                              NULL));
  float hy[D_OUT];
  CHECK_HIP(hipMemcpy(hy, y, sizeof(hy), hipMemcpyDeviceToHost));
  double worst = 0.0;
  for (int r = 0; r < D_OUT; ++r) {
    double ref = 0.0;
    for (int j = 0; j < D_IN; ++j) ref += (x_of(j) / 64.0) * (w_of(j, r) / 64.0);
    double err = fabs((double)hy[r] - ref) / (1.0 + fabs(ref));
    if (err > worst) worst = err;
  }
  printf("all-FULL product against the dense sum: worst relative error %.3g\n", worst);
  if (!(worst <= 1e-6)) return 1;

  /* 2. TopK 100 / 150: counts and lists */
  p.n_full = 100;
  p.n_approx = 150;
  CHECK_SPAX(spax_build_tiers((const uint16_t*)x, D_IN, &p, (uint8_t*)tier, (int32_t*)f,
                              (int32_t*)a, (int32_t*)c, NULL));
  int32_t hc[3], hf[D_IN], ha[D_IN];
  CHECK_HIP(hipMemcpy(hc, c, sizeof(hc), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hf, f, sizeof(hf), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(ha, a, sizeof(ha), hipMemcpyDeviceToHost));
  printf("TopK 100/150 counts: %d %d %d\n", hc[0], hc[1], hc[2]);
  if (hc[0] != 100 || hc[1] != 150 || hc[2] != D_IN - 250) return 1;
  static unsigned char seen[D_IN];
  for (int t = 0; t < 2; ++t) {
    const int32_t* l = t ? ha : hf;
    for (int i = 0; i < hc[t]; ++i) {
      if (l[i] < 0 || l[i] >= D_IN || seen[l[i]] || (i > 0 && l[i] <= l[i - 1])) {
        printf("list %d entry %d = %d is out of order, repeated or out of range\n", t, i, l[i]);
        return 1;
      }
      seen[l[i]] = 1;
    }
  }

  /* 3. validation before anything is enqueued */
  int st = spax_build_tiers(NULL, D_IN, &p, (uint8_t*)tier, (int32_t*)f, (int32_t*)a,
                            (int32_t*)c, NULL);
  printf("NULL activations: status %d (%s): %s\n", st, spax_status_string(st), spax_last_error());
  if (st != SPAX_ERR_NULL || spax_last_error()[0] == '\0') return 1;

  CHECK_HIP(hipDeviceSynchronize());
  hipFree(W);
  hipFree(packed);
  hipFree(x);
  hipFree(tier);
  hipFree(f);
  hipFree(a);
  hipFree(c);
  hipFree(y);
  if (ws) hipFree(ws);
  printf("spax C ABI demo: ok\n");
  return 0;
}
