/*
 * The C ABI from plain C: compiled by tests/test_c_abi.py with gcc -std=c99
 * against include/moe_ep.h and include/moe_streams.h, linked to the built
 * libmoe_ep.so and libmoe_streams.so.  It
 * calls only the sizing functions and argument checks that return before
 * anything is enqueued, so it needs no GPU.  Prints one line per failed
 * check; the exit status is the number of failures.
 */
#include <stdint.h>
#include <stdio.h>

#include "moe_ep.h"
#include "moe_streams.h"

static int fails = 0;

static void expect(const char *what, int64_t got, int64_t want) {
  if (got != want) {
    printf("FAIL %s: got %lld, want %lld\n", what, (long long)got, (long long)want);
    ++fails;
  }
}

int main(void) {
  moe_shape s = {16, 128, 2048, 128, 8, 0, 0};   /* N, T, H, E, k, early_rows, region_rows */
  void *A = (void *)(uintptr_t)0x10000000u;      /* never dereferenced */
  uint32_t flags = 0;
  int64_t ws;

  expect("packed rows", moe_recv_rows(&s), 16 * 128 * 8);
  s.region_rows = 1000;
  expect("fixed rows", moe_recv_rows(&s), 16 * 1000);
  s.region_rows = 0;
  ws = moe_workspace_bytes(&s);
  expect("workspace is a multiple of 256 bytes", ws > 0 && ws % 256 == 0, 1);

  s.H = 2000;
  expect("H not a multiple of 128", moe_recv_rows(&s), MOE_EINVAL);
  s.H = 2048;
  s.E = 120;
  expect("E not a multiple of N", moe_recv_rows(&s), MOE_EINVAL);
  s.E = 128;
  expect("NULL shape", moe_recv_rows(NULL), MOE_ENULL);

  expect("dispatch send without workspace",
         moe_dispatch_send(&s, A, A, A, A, A, NULL, NULL), MOE_ENULL);
  expect("dispatch send with misaligned tokens",
         moe_dispatch_send(&s, (const uint16_t *)((char *)A + 8), A, A, A, A, A, NULL), MOE_EALIGN);
  expect("combine recv without weights", moe_combine_recv(&s, A, A, NULL, A, NULL), MOE_ENULL);
  expect("status without workspace", moe_status(NULL, NULL, &flags), MOE_ENULL);
  expect("copy of a partial 16-byte unit", moe_copy(A, A, 17, NULL), MOE_EINVAL);
  expect("stream with k = 9", moe_stream(MOE_STREAM_REDUCE, 9, A, A, 16, NULL), MOE_EINVAL);
  expect("stream with another pattern", moe_stream(4, 8, A, A, 16, NULL), MOE_EINVAL);

  if (!fails) printf("c abi ok\n");
  return fails;
}
