/*
 * One dispatch + combine through the C ABI from plain C, with device memory
 * from hipMalloc (no Python, no torch): compiled and run by
 * tests/test_c_abi.py on a GPU.  Shape N=4 ranks, T=64 tokens, H=256, E=8
 * experts, k=2; token t of rank s picks experts (s+t) mod 8 and (s+t+3) mod 8
 * with weights 1/2 each.  The host checks, from what the calls return:
 *   - every (rank, token, slot) owns exactly one expert-major row (row_src),
 *     whose fp8 bytes times its block scale give the token back to within
 *     the e4m3 rounding bound (relative 2^-4);
 *   - each rank's per-expert offsets count its rows;
 *   - with expert outputs y[i] = (i mod 61) - 30 in every element, the combine
 *     returns bf16((y_a + y_b) / 2) exactly for each token's two rows a, b
 *     (halves of small integers are exact in float32 and bfloat16).
 * Prints one line per failed check; exit status = failures (99: a HIP call
 * or a library call failed).
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_ep.h"

enum { N = 4, T = 64, H = 256, E = 8, K = 2, L = E / N, NB = H / 128 };

#define HIPCHK(x)                                                   \
  do {                                                              \
    if ((x) != hipSuccess) {                                        \
      printf("FAIL HIP call %s at line %d\n", #x, __LINE__);        \
      return 99;                                                    \
    }                                                               \
  } while (0)
#define MOECHK(x)                                                   \
  do {                                                              \
    int rc_ = (x);                                                  \
    if (rc_ != MOE_OK) {                                            \
      printf("FAIL %s returned %d at line %d\n", #x, rc_, __LINE__); \
      return 99;                                                    \
    }                                                               \
  } while (0)

static uint16_t bf16_of(float f) { /* round to nearest even; inputs here are finite */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static float f32_of_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static float e4m3_value(uint8_t q) { /* OCP E4M3: bias 7, subnormals m * 2^-9 */
  const int s = q >> 7, e = (q >> 3) & 15, m = q & 7;
  const float v = e == 0 ? ldexpf((float)m, -9) : ldexpf(1.0f + m / 8.0f, e - 7);
  return s ? -v : v;
}

int main(void) {
  moe_shape sh = {N, T, H, E, K, 0, 0};
  const int64_t rows = moe_recv_rows(&sh), wsb = moe_workspace_bytes(&sh);
  const int slots = N * T * K;
  int fails = 0;
  if (rows != slots || wsb <= 0) {
    printf("FAIL sizes: rows %lld, workspace %lld\n", (long long)rows, (long long)wsb);
    return 99;
  }
  uint16_t *h_x = malloc(sizeof(uint16_t) * N * T * H), *h_y = malloc(sizeof(uint16_t) * rows * H);
  uint16_t *h_out = malloc(sizeof(uint16_t) * N * T * H);
  int32_t *h_idx = malloc(sizeof(int32_t) * slots), *h_pos = malloc(sizeof(int32_t) * slots);
  int32_t *h_src = malloc(sizeof(int32_t) * rows), *h_eoff = malloc(sizeof(int32_t) * N * (L + 1));
  float *h_w = malloc(sizeof(float) * slots), *h_xs = malloc(sizeof(float) * rows * NB);
  uint8_t *h_xq = malloc((size_t)rows * H);
  int *seen = calloc((size_t)slots, sizeof(int));
  if (!h_x || !h_y || !h_out || !h_idx || !h_pos || !h_src || !h_eoff || !h_w || !h_xs || !h_xq || !seen) return 99;

  for (int s = 0; s < N; ++s)
    for (int t = 0; t < T; ++t) {
      for (int h = 0; h < H; ++h) h_x[((size_t)s * T + t) * H + h] = bf16_of((float)((t * 7 + s * 3 + h) % 17 - 8) / 4.0f);
      h_idx[(s * T + t) * K + 0] = (s + t) % E;
      h_idx[(s * T + t) * K + 1] = (s + t + 3) % E;
      h_w[(s * T + t) * K + 0] = 0.5f;
      h_w[(s * T + t) * K + 1] = 0.5f;
    }
  for (int64_t i = 0; i < rows; ++i)
    for (int h = 0; h < H; ++h) h_y[i * H + h] = bf16_of((float)(i % 61 - 30));

  void *ws, *x, *idx, *w, *rq, *rs, *pos, *xq, *xs, *eoff, *src, *y, *comb, *out;
  HIPCHK(hipMalloc(&ws, (size_t)wsb));
  HIPCHK(hipMalloc(&x, sizeof(uint16_t) * N * T * H));
  HIPCHK(hipMalloc(&idx, sizeof(int32_t) * slots));
  HIPCHK(hipMalloc(&w, sizeof(float) * slots));
  HIPCHK(hipMalloc(&rq, (size_t)rows * H));
  HIPCHK(hipMalloc(&rs, sizeof(float) * rows * NB));
  HIPCHK(hipMalloc(&pos, sizeof(int32_t) * slots));
  HIPCHK(hipMalloc(&xq, (size_t)rows * H));
  HIPCHK(hipMalloc(&xs, sizeof(float) * rows * NB));
  HIPCHK(hipMalloc(&eoff, sizeof(int32_t) * N * (L + 1)));
  HIPCHK(hipMalloc(&src, sizeof(int32_t) * rows));
  HIPCHK(hipMalloc(&y, sizeof(uint16_t) * rows * H));
  HIPCHK(hipMalloc(&comb, sizeof(uint16_t) * slots * H));
  HIPCHK(hipMalloc(&out, sizeof(uint16_t) * N * T * H));
  HIPCHK(hipMemcpy(x, h_x, sizeof(uint16_t) * N * T * H, hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(idx, h_idx, sizeof(int32_t) * slots, hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(w, h_w, sizeof(float) * slots, hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(y, h_y, sizeof(uint16_t) * rows * H, hipMemcpyHostToDevice));

  uint32_t flags = 0;
  MOECHK(moe_workspace_init(&sh, ws, NULL));
  MOECHK(moe_dispatch_send(&sh, x, idx, rq, rs, pos, ws, NULL));
  MOECHK(moe_dispatch_recv(&sh, rq, rs, ws, xq, xs, eoff, src, NULL));
  MOECHK(moe_combine_send(&sh, y, src, ws, comb, NULL));
  MOECHK(moe_combine_recv(&sh, comb, pos, w, out, NULL));
  MOECHK(moe_status(ws, NULL, &flags));
  if (flags) {
    printf("FAIL error flags %u\n", flags);
    ++fails;
  }

  HIPCHK(hipMemcpy(h_pos, pos, sizeof(int32_t) * slots, hipMemcpyDeviceToHost));
  HIPCHK(hipMemcpy(h_src, src, sizeof(int32_t) * rows, hipMemcpyDeviceToHost));
  HIPCHK(hipMemcpy(h_xq, xq, (size_t)rows * H, hipMemcpyDeviceToHost));
  HIPCHK(hipMemcpy(h_xs, xs, sizeof(float) * rows * NB, hipMemcpyDeviceToHost));
  HIPCHK(hipMemcpy(h_eoff, eoff, sizeof(int32_t) * N * (L + 1), hipMemcpyDeviceToHost));
  HIPCHK(hipMemcpy(h_out, out, sizeof(uint16_t) * N * T * H, hipMemcpyDeviceToHost));

  /* slot (s, t, j) -> its expert-major row, through row_src = s*T*K + send_pos */
  int *row_of = malloc(sizeof(int) * slots), *slot_of = malloc(sizeof(int) * rows);
  if (!row_of || !slot_of) return 99;
  for (int i = 0; i < slots; ++i) row_of[i] = -1;
  for (int64_t i = 0; i < rows; ++i) slot_of[i] = -1;
  for (int64_t i = 0; i < rows; ++i) {
    const int rsrc = h_src[i];
    if (rsrc < 0 || rsrc >= slots) {
      printf("FAIL row %lld: row_src %d\n", (long long)i, rsrc);
      ++fails;
      continue;
    }
    const int s = rsrc / (T * K), p = rsrc % (T * K);
    int found = -1;
    for (int tj = 0; tj < T * K; ++tj)
      if (h_pos[s * T * K + tj] == p) found = s * T * K + tj;
    if (found < 0 || seen[found]++) {
      printf("FAIL row %lld: no single slot has sender position %d of rank %d\n", (long long)i, p, s);
      ++fails;
      continue;
    }
    row_of[found] = (int)i;
    slot_of[i] = found;
    const int t = (found % (T * K)) / K;
    for (int h = 0; h < H; ++h) {
      const float want = f32_of_bf16(h_x[((size_t)s * T + t) * H + h]);
      const float got = e4m3_value(h_xq[i * H + h]) * h_xs[i * NB + h / 128];
      if (fabsf(got - want) > fabsf(want) / 16.0f + 1e-6f) {
        printf("FAIL row %lld element %d: dequantised %g, token %g\n", (long long)i, h, got, want);
        ++fails;
        break;
      }
    }
  }
  for (int d = 0; d < N; ++d) {   /* rank d's rows: the slots whose expert lives on d */
    int rows_d = 0;
    for (int64_t i = 0; i < rows; ++i)
      if (slot_of[i] >= 0 && h_idx[slot_of[i]] / L == d) ++rows_d;
    if (h_eoff[d * (L + 1)] != 0 || h_eoff[d * (L + 1) + L] != rows_d) {
      printf("FAIL rank %d: expert offsets %d..%d, %d rows\n", d, h_eoff[d * (L + 1)], h_eoff[d * (L + 1) + L], rows_d);
      ++fails;
    }
  }
  for (int st = 0; st < N * T && !fails; ++st) {
    const int a = row_of[st * K], b = row_of[st * K + 1];
    if (a < 0 || b < 0) {
      printf("FAIL token %d has a slot without a row\n", st);
      ++fails;
      break;
    }
    const uint16_t want = bf16_of(0.5f * (float)(a % 61 - 30) + 0.5f * (float)(b % 61 - 30));
    for (int h = 0; h < H; ++h)
      if (h_out[(size_t)st * H + h] != want) {
        printf("FAIL token %d element %d: %04x, want %04x\n", st, h, h_out[(size_t)st * H + h], want);
        ++fails;
        break;
      }
  }
  if (!fails) printf("c abi gpu ok: %lld rows\n", (long long)rows);
  return fails;
}
