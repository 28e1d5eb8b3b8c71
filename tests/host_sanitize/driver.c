/* Host-side argument checks of the C ABI under AddressSanitizer and UndefinedBehavior-
 * Sanitizer. Every call below is invalid in some documented way, or runs on a machine
 * without a device; each must return its documented status and leave a message, without
 * any memory error in the host code that checks and formats it. No call reaches a GPU. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/subspec.h"

static int failures = 0;

static void expect(const char* what, ss_status got, ss_status want) {
  const char* msg = ss_last_error();
  if (got != want) {
    printf("FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, msg ? msg : "");
    ++failures;
  } else if (want != SS_OK && (!msg || !msg[0])) {
    printf("FAIL %s: no error message\n", what);
    ++failures;
  } else {
    printf("ok   %s: %s\n", what, msg ? msg : "");
  }
}

static void expect_not_ok(const char* what, ss_status got) {
  const char* msg = ss_last_error();
  if (got == SS_OK || !msg || !msg[0]) {
    printf("FAIL %s: status %d (%s)\n", what, (int)got, msg ? msg : "");
    ++failures;
  } else {
    printf("ok   %s: %d %s\n", what, (int)got, msg);
  }
}

int main(void) {
  /* host buffers stand in for device pointers: every call below fails before using them */
  static _Alignas(256) unsigned char buf[1 << 16];
  void* p = buf;
  int32_t par_ok[5] = {-1, 0, 1, 1, 0}, par_bad[3] = {-1, 0, 2};

  if (ss_abi_version() < 1) { printf("FAIL abi version\n"); ++failures; }
  expect("tree_validate ok", ss_tree_validate(par_ok, 5), SS_OK);
  expect("tree_validate bad", ss_tree_validate(par_bad, 3), SS_ERR_BAD_TREE);
  expect("tree_validate null", ss_tree_validate(NULL, 3), SS_ERR_INVALID_ARG);
  expect("tree_validate T=0", ss_tree_validate(par_ok, 0), SS_ERR_INVALID_ARG);

  expect_not_ok("quantize group 32", ss_quantize_substitute(p, 64, 128, 32, p, p, p, NULL));
  expect_not_ok("quantize k % 64", ss_quantize_substitute(p, 64, 100, 64, p, p, p, NULL));
  expect_not_ok("quantize null", ss_quantize_substitute(NULL, 64, 128, 64, p, p, p, NULL));

  if (ss_w4a16_linear_workspace(0, 64, 128) != 0) { printf("FAIL workspace T=0\n"); ++failures; }
  expect_not_ok("w4a16_linear T=0", ss_w4a16_linear(p, 0, p, p, p, 64, 128, p, NULL, p, 1 << 16, NULL));
  expect_not_ok("w4a16_linear misaligned x",
                ss_w4a16_linear(buf + 2, 16, p, p, p, 64, 128, p, NULL, p, 1 << 16, NULL));
  expect_not_ok("w4a16_linear small ws", ss_w4a16_linear(p, 16, p, p, p, 64, 128, p, NULL, p, 0, NULL));
  expect_not_ok("linear_tiled_noalloc huge",
                ss_w4a16_linear_tiled_noalloc(p, 192, p, 65536, 8192, p, NULL, NULL));

  ss_attn_args a;
  memset(&a, 0, sizeof a);
  a.q = p; a.k_cache = p; a.v_cache = p; a.k_tree = p; a.v_tree = p; a.parents = par_ok;
  a.out = p; a.T = 5; a.C = 100; a.c_stride = 64; a.nq = 4; a.nkv = 2; a.hd = 128;
  expect_not_ok("attention C > c_stride", ss_tree_attention(&a, p, 1 << 16, NULL));
  a.c_stride = 128; a.hd = 96;
  expect_not_ok("attention hd 96", ss_tree_attention(&a, p, 1 << 16, NULL));
  a.hd = 128; a.nq = 5;
  expect_not_ok("attention nq % nkv", ss_tree_attention(&a, p, 1 << 16, NULL));
  expect_not_ok("attention null args", ss_tree_attention(NULL, p, 1 << 16, NULL));

  expect_not_ok("tree_expand_init D >= T",
                ss_tree_expand_init(1, 8, 8, 2, 4, (int32_t*)p, (int32_t*)p, (float*)p, (int32_t*)p, (int32_t*)p, NULL));
  if (ss_tree_expand_workspace(0, 100) != 0) { printf("FAIL expand workspace R=0\n"); ++failures; }
  if (ss_tree_accept_stochastic_workspace(300, 100) != 0) { printf("FAIL stochastic workspace T=300\n"); ++failures; }
  expect_not_ok("row_argmax rows 0", ss_row_argmax((const float*)p, 0, 10, (int32_t*)p, NULL));
  expect_not_ok("draft_select k 0", ss_draft_select((const float*)p, NULL, 2, 100, 1.0f, 0, (int32_t*)p, p, 1 << 16, NULL));

  ss_model m;
  memset(&m, 0, sizeof m);
  ss_step_args s;
  memset(&s, 0, sizeof s);
  expect_not_ok("draft_tree_step null layers", ss_draft_tree_step(&m, &s, p, 1 << 16, NULL));
  expect_not_ok("draft_tree_step null model", ss_draft_tree_step(NULL, &s, p, 1 << 16, NULL));

  /* a long message through the formatter: a tree whose bad parent sits at a large index */
  int32_t* chain = (int32_t*)malloc(256 * sizeof(int32_t));
  chain[0] = -1;
  for (int i = 1; i < 256; ++i) chain[i] = i - 1;
  chain[255] = 300;
  expect("tree_validate bad parent at 255", ss_tree_validate(chain, 256), SS_ERR_BAD_TREE);
  free(chain);

  printf("%s: %d failure(s)\n", failures ? "FAILED" : "PASSED", failures);
  return failures ? 1 : 0;
}
