/* A plain C99 consumer of include/cpattn.h: the header compiles as C and the
 * host-only entry points of libcpattn.so are called through it, checked
 * against the worked values of the G5 context-parallel modelling spec
 * (Definitions table: the head/tail chunk pairs of the balanced split;
 * Formulas section: the pass-KV bytes and the per-step FLOPs of the GQA
 * prefill, S = 32768 at cp = 8, 32/8 heads, head_dim 128, bf16; the pass-Q
 * bytes of the decode workload, b = 8, S = 2^20; no CP traffic at cp = 1).
 * No GPU call is made. Prints one line per failed check, returns the count. */
#include "cpattn.h"

#include <stdio.h>
#include <string.h>

static int bad = 0;

#define CHECK(cond, what)                      \
  do {                                         \
    if (!(cond)) {                             \
      ++bad;                                   \
      printf("failed: %s\n", what);            \
    }                                          \
  } while (0)

static void split_pins(void) {
  /* S = 16, cp = 4: rank r holds chunks r and 7 - r of two tokens each */
  static const int64_t want[4][4] = {{0, 1, 14, 15}, {2, 3, 12, 13}, {4, 5, 10, 11}, {6, 7, 8, 9}};
  const int64_t cu[2] = {0, 16};
  for (int r = 0; r < 4; ++r) {
    int64_t pos[4], cul[2];
    CHECK(cpattn_balanced_split(cu, 1, 4, r, pos, cul) == CPATTN_OK, "split S=16 cp=4 returns OK");
    CHECK(memcmp(pos, want[r], sizeof pos) == 0, "split S=16 cp=4 positions");
    CHECK(cul[0] == 0 && cul[1] == 4, "split S=16 cp=4 cu_local");
  }
  /* S = 8, cp = 2 */
  const int64_t cu8[2] = {0, 8};
  int64_t p0[4], p1[4], c0[2], c1[2];
  CHECK(cpattn_balanced_split(cu8, 1, 2, 0, p0, c0) == CPATTN_OK &&
            cpattn_balanced_split(cu8, 1, 2, 1, p1, c1) == CPATTN_OK,
        "split S=8 cp=2 returns OK");
  CHECK(p0[0] == 0 && p0[1] == 1 && p0[2] == 6 && p0[3] == 7, "split S=8 cp=2 rank 0");
  CHECK(p1[0] == 2 && p1[1] == 3 && p1[2] == 4 && p1[3] == 5, "split S=8 cp=2 rank 1");
}

static void split_errors(void) {
  const int64_t cu[2] = {0, 10};   /* 10 is not a multiple of 2 * 4 */
  int64_t pos[8], cul[2];
  for (int i = 0; i < 8; ++i) pos[i] = -7;
  cul[0] = cul[1] = -7;
  CHECK(cpattn_balanced_split(cu, 1, 4, 0, pos, cul) == CPATTN_E_DIVISIBILITY, "L % 2cp != 0 is rejected");
  CHECK(pos[0] == -7 && cul[0] == -7 && cul[1] == -7, "a rejected split leaves its outputs untouched");
  CHECK(cpattn_balanced_split(cu, 1, 0, 0, pos, cul) == CPATTN_E_ARG, "cp = 0 is rejected");
  CHECK(cpattn_balanced_split(cu, 1, 4, 4, pos, cul) == CPATTN_E_ARG, "rank = cp is rejected");
  int64_t rows = -1;
  CHECK(cpattn_local_rows(cu, 1, 4, 1, &rows) == CPATTN_OK && rows == 4, "padded rows of L = 10 at cp = 4");
  CHECK(cpattn_local_rows(cu, 1, 4, 0, &rows) == CPATTN_E_DIVISIBILITY, "unpadded rows of L = 10 rejected");
}

static void account_pins(void) {
  const int64_t cu[2] = {0, 32768};
  cpattn_account_in in;
  memset(&in, 0, sizeof in);
  in.cp = 8;
  in.n_hq = 32;
  in.n_kv = 8;
  in.head_dim = 128;
  in.dtype_bytes = 2;
  in.layers_local = 1;
  in.cu_seqlens = cu;
  in.num_seqs = 1;
  cpattn_account_out out;
  CHECK(cpattn_account(&in, &out) == CPATTN_OK, "account of the GQA prefill returns OK");
  CHECK(out.tokens_per_rank == 4096, "tokens per rank");
  CHECK(out.ring_steps == 8 && out.p2p_ops == 7, "8 ring steps and 7 transfers");
  CHECK(out.passkv_bytes_per_step == 16777216LL, "pass-KV bytes per step, S/cp * c_kv");
  CHECK(out.passkv_bytes_per_rank == 7LL * 16777216LL, "pass-KV bytes per rank");
  CHECK(out.attn_flops == (1LL << 43), "F_attn = 2^43");
  CHECK(out.step_flops == (1LL << 37), "F_attn / cp^2 = 2^37");
  CHECK(out.step0_flops_exact == 137472507904LL, "inclusive diagonal at step 0");
  CHECK(out.stepN_flops_exact == (1LL << 37), "exact FLOPs of steps >= 1");

  memset(&in, 0, sizeof in);
  in.cp = 8;
  in.n_hq = 32;
  in.n_kv = 8;
  in.head_dim = 128;
  in.dtype_bytes = 2;
  in.layers_local = 1;
  in.batch = 8;
  in.kv_len = 1 << 20;
  CHECK(cpattn_account(&in, &out) == CPATTN_OK, "account of the decode returns OK");
  CHECK(out.decode_kv_bytes_total == (1LL << 35), "decode KV bytes 2^35");
  CHECK(out.passq_dispatch_bytes == 65536, "pass-Q dispatch b d s");
  CHECK(out.passq_reduce_bytes == 66560, "pass-Q reduce b (d + 2 n_h) s");
  CHECK(out.decode_flops == (1LL << 37), "decode FLOPs");

  in.cp = 1;
  CHECK(cpattn_account(&in, &out) == CPATTN_OK, "account at cp = 1 returns OK");
  CHECK(out.passq_dispatch_bytes == 0 && out.passq_reduce_bytes == 0, "no pass-Q traffic at cp = 1");
}

int main(void) {
  const char *v = cpattn_version();
  CHECK(v != NULL && strncmp(v, "cpattn", 6) == 0, "version string");
  split_pins();
  split_errors();
  account_pins();
  printf("%d failed\n", bad);
  return bad;
}
