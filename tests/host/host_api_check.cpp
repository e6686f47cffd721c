// Host-only entry points of libcpattn (csrc/host.cpp) driven over a grid of
// inputs and error cases, for the AddressSanitizer / UndefinedBehaviorSanitizer
// build of tests/test_host_sanitizers.py. Besides running every path, it checks
// the invariants the balanced split and the account must keep (Definitions
// table of the G5 context-parallel modelling spec: 2*cp chunks per sequence, a
// head/tail pair per rank; Formulas: F_attn / cp^2 per ring step):
//   - over all ranks the positions are a permutation of the sequence tokens,
//     each rank holds sum(L_i)/cp rows, and cu_local matches;
//   - the padded split reports exactly the pad slots as -1 and every real token
//     once;
//   - cpattn_local_rows equals the split's row count;
//   - step0_flops_exact = stepN_flops_exact + 4 d n_hq sum(c_i), and
//     rank_flops_exact = step0 + (cp - 1) stepN; step_flops * cp^2 = attn_flops;
//   - invalid inputs return the documented codes and leave outputs untouched.
#include "cpattn.h"

#include <cstdio>
#include <cstdlib>
#include <vector>

static long long bad = 0, checked = 0;

#define CHECK(cond, ...)                   \
  do {                                     \
    ++checked;                             \
    if (!(cond)) {                         \
      if (++bad < 20) printf(__VA_ARGS__); \
    }                                      \
  } while (0)

static std::vector<int64_t> cumulative(const std::vector<int64_t> &lens) {
  std::vector<int64_t> cu(lens.size() + 1, 0);
  for (size_t i = 0; i < lens.size(); ++i) cu[i + 1] = cu[i] + lens[i];
  return cu;
}

static void check_split(const std::vector<int64_t> &lens, int cp, bool padded) {
  const std::vector<int64_t> cu = cumulative(lens);
  const int n = (int)lens.size();
  int64_t rows = -1;
  const int rc_rows = cpattn_local_rows(cu.data(), n, cp, padded ? 1 : 0, &rows);
  bool divisible = true;
  for (int64_t L : lens) divisible = divisible && L % (2 * cp) == 0;
  if (!padded && !divisible) {
    CHECK(rc_rows == CPATTN_E_DIVISIBILITY, "local_rows: expected E_DIVISIBILITY\n");
    std::vector<int64_t> pos(1, 7), cul(n + 1, 7);
    CHECK(cpattn_balanced_split(cu.data(), n, cp, 0, pos.data(), cul.data()) == CPATTN_E_DIVISIBILITY,
          "split: expected E_DIVISIBILITY\n");
    CHECK(pos[0] == 7 && cul[0] == 7, "split wrote outputs on error\n");
    return;
  }
  CHECK(rc_rows == CPATTN_OK, "local_rows failed (%d)\n", rc_rows);
  const int64_t total = cu[n];
  std::vector<int> seen(total, 0);
  int64_t pads = 0;
  for (int r = 0; r < cp; ++r) {
    std::vector<int64_t> pos(rows > 0 ? rows : 1, -7), cul(n + 1, -7);
    const int rc = padded ? cpattn_balanced_split_padded(cu.data(), n, cp, r, pos.data(), cul.data())
                          : cpattn_balanced_split(cu.data(), n, cp, r, pos.data(), cul.data());
    CHECK(rc == CPATTN_OK, "split failed (%d)\n", rc);
    CHECK(cul[0] == 0 && cul[n] == rows, "cu_local end %lld != rows %lld\n", (long long)cul[n], (long long)rows);
    for (int64_t x = 0; x < rows; ++x) {
      const int64_t p = pos[x];
      if (p == -1) {
        ++pads;
        CHECK(padded, "pad slot in an unpadded split\n");
        continue;
      }
      CHECK(p >= 0 && p < total, "position out of range\n");
      if (p >= 0 && p < total) ++seen[p];
    }
  }
  for (int64_t p = 0; p < total; ++p) CHECK(seen[p] == 1, "token %lld seen %d times\n", (long long)p, seen[p]);
  int64_t want_pads = 0;
  for (int64_t L : lens) want_pads += ((L + 2 * cp - 1) / (2 * cp)) * 2 * cp - L;
  CHECK(pads == want_pads, "pad slots %lld != %lld\n", (long long)pads, (long long)want_pads);
}

static void check_account(const std::vector<int64_t> &lens, int cp, int n_hq, int n_kv, int d) {
  const std::vector<int64_t> cu = cumulative(lens);
  cpattn_account_in in{};
  in.cp = cp;
  in.n_hq = n_hq;
  in.n_kv = n_kv;
  in.head_dim = d;
  in.dtype_bytes = 2;
  in.layers_local = 1;
  in.cu_seqlens = cu.data();
  in.num_seqs = (int32_t)lens.size();
  in.batch = 2;
  in.kv_len = 4096LL * cp;
  cpattn_account_out out{};
  const int rc = cpattn_account(&in, &out);
  CHECK(rc == CPATTN_OK, "account failed (%d)\n", rc);
  int64_t sum_c = 0;
  for (int64_t L : lens) sum_c += L / (2 * cp);
  CHECK(out.step0_flops_exact == out.stepN_flops_exact + 4LL * d * n_hq * sum_c, "step0 != stepN + diagonal\n");
  CHECK(out.rank_flops_exact == out.step0_flops_exact + (cp - 1) * out.stepN_flops_exact, "rank flops\n");
  CHECK(out.step_flops * cp * cp == out.attn_flops, "F_step * cp^2 != F_attn\n");
  CHECK(out.ring_steps == cp && out.p2p_ops == cp - 1, "step counts\n");
  CHECK(out.passkv_bytes_per_rank == (cp - 1) * out.passkv_bytes_per_step, "pass-KV bytes\n");
}

static void check_errors() {
  const std::vector<int64_t> cu = {0, 16, 48};
  std::vector<int64_t> pos(64, 3), cul(3, 3);
  CHECK(cpattn_balanced_split(nullptr, 2, 2, 0, pos.data(), cul.data()) == CPATTN_E_ARG, "null cu\n");
  CHECK(cpattn_balanced_split(cu.data(), 2, 0, 0, pos.data(), cul.data()) == CPATTN_E_ARG, "cp 0\n");
  CHECK(cpattn_balanced_split(cu.data(), 2, 2, 2, pos.data(), cul.data()) == CPATTN_E_ARG, "rank 2\n");
  CHECK(cpattn_balanced_split(cu.data(), 2, 2, -1, pos.data(), cul.data()) == CPATTN_E_ARG, "rank -1\n");
  CHECK(cpattn_balanced_split(cu.data(), -1, 2, 0, pos.data(), cul.data()) == CPATTN_E_ARG, "num_seqs -1\n");
  CHECK(cpattn_balanced_split(cu.data(), 2, 2, 0, nullptr, cul.data()) == CPATTN_E_ARG, "null positions\n");
  const std::vector<int64_t> dec = {0, 16, 8};
  CHECK(cpattn_balanced_split_padded(dec.data(), 2, 2, 0, pos.data(), cul.data()) == CPATTN_E_ARG, "decreasing\n");
  int64_t rows = 0;
  CHECK(cpattn_local_rows(cu.data(), 2, 2, 3, &rows) == CPATTN_E_ARG, "padded 3\n");
  CHECK(cpattn_local_rows(cu.data(), 2, 2, 0, nullptr) == CPATTN_E_ARG, "null rows\n");
  CHECK(cpattn_account(nullptr, nullptr) == CPATTN_E_ARG, "null account\n");
  // int64 overflow of the FLOP count is reported, not wrapped
  const std::vector<int64_t> huge = {0, (int64_t)1 << 40};
  cpattn_account_in in{};
  in.cp = 1;
  in.n_hq = 65535;
  in.n_kv = 1;
  in.head_dim = 512;
  in.dtype_bytes = 2;
  in.layers_local = 1;
  in.cu_seqlens = huge.data();
  in.num_seqs = 1;
  cpattn_account_out out{};
  CHECK(cpattn_account(&in, &out) == CPATTN_E_OVERFLOW, "overflow not reported\n");
}

int main() {
  const std::vector<std::vector<int64_t>> grids = {
      {8}, {16, 32}, {256}, {64, 0, 128}, {5, 13, 0, 1, 7}, {3, 10, 6}, {1, 2, 3, 4, 5, 6, 7, 8, 9},
      {12464, 15568, 14688, 9376, 15536, 16048}, {1000003}, {2048, 6144, 4096}};
  for (const auto &lens : grids)
    for (int cp : {1, 2, 3, 4, 8, 16}) {
      check_split(lens, cp, false);
      check_split(lens, cp, true);
      bool div = true;
      for (int64_t L : lens) div = div && L % (2 * cp) == 0;
      if (div) check_account(lens, cp, 32, 8, 128);
    }
  check_errors();
  printf("%lld checks, %lld failures\n", checked, bad);
  return bad != 0;
}
