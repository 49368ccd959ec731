/*
 * A plain C caller of libpkv.so's host-only entry points (no GPU needed): it includes
 * only include/pkv.h and prints, for the lengths given on the command line, what a
 * step's host side computes. Used by tests/test_c_abi.py, which builds it with gcc
 * and compares the output with the oracle's plan.
 *
 * usage: plan_from_c W Hkv tile L_0 L_1 ...   (bf16, D = 128, P = 16, q_len 1, G = 4)
 * output lines:
 *   abi <version>
 *   status <code> <pkv_status_string>        for codes 0 .. -6
 *   plan <T> <N> <num_partials>
 *   item <b> <g> <i> <slot>                  N lines, grouped by worker
 *   offsets <W + 1 values>
 *   rtb <B + 1 values>
 *   workspace <bytes>
 *   seq_error <status> <pkv_last_error>      a length below q_len is refused
 */
#include <stdio.h>
#include <stdlib.h>

#include "pkv.h"

static int fail(const char* what, int st) {
  fprintf(stderr, "%s: %s (%d): %s\n", what, pkv_status_string(st), st, pkv_last_error());
  return 1;
}

int main(int argc, char** argv) {
  if (argc < 5) {
    fprintf(stderr, "usage: %s W Hkv tile L_0 [L_1 ...]\n", argv[0]);
    return 2;
  }
  const int W = atoi(argv[1]), Hkv = atoi(argv[2]), tile = atoi(argv[3]);
  const int B = argc - 4;
  int32_t* lens = malloc(sizeof(int32_t) * B);
  for (int b = 0; b < B; ++b) lens[b] = atoi(argv[4 + b]);

  printf("abi %d\n", pkv_abi_version());
  for (int s = 0; s >= -6; --s) printf("status %d %s\n", s, pkv_status_string(s));

  int32_t T = 0;
  int64_t N = 0, NP = 0;
  int st = pkv_plan_query(B, lens, 1, 4 * Hkv, Hkv, 128, 16, PKV_KV_BF16, tile, W, &T, &N, &NP);
  if (st != PKV_OK) return fail("pkv_plan_query", st);
  printf("plan %d %lld %lld\n", T, (long long)N, (long long)NP);

  int32_t* items = malloc(sizeof(int32_t) * 4 * (N > 0 ? N : 1));
  int32_t* offs = malloc(sizeof(int32_t) * (W + 1));
  int32_t* rtb = malloc(sizeof(int32_t) * (B + 1));
  st = pkv_plan(B, lens, 1, Hkv, T, W, items, offs, rtb);
  if (st != PKV_OK) return fail("pkv_plan", st);
  for (int64_t k = 0; k < N; ++k)
    printf("item %d %d %d %d\n", items[4 * k], items[4 * k + 1], items[4 * k + 2], items[4 * k + 3]);
  printf("offsets");
  for (int w = 0; w <= W; ++w) printf(" %d", offs[w]);
  printf("\nrtb");
  for (int b = 0; b <= B; ++b) printf(" %d", rtb[b]);
  printf("\n");

  size_t ws = 0;
  st = pkv_workspace_bytes(NP, 4, 128, &ws);
  if (st != PKV_OK) return fail("pkv_workspace_bytes", st);
  printf("workspace %zu\n", ws);

  lens[0] = 0;   /* below max(1, q_len): refused with PKV_ERR_SEQ */
  st = pkv_plan_query(B, lens, 1, 4 * Hkv, Hkv, 128, 16, PKV_KV_BF16, tile, W, &T, &N, &NP);
  printf("seq_error %d %s\n", st, pkv_last_error());

  free(items);
  free(offs);
  free(rtb);
  free(lens);
  return 0;
}
