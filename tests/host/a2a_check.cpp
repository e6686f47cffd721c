// Host model of the Ulysses all-to-all (cpattn_ulysses_all_to_all), built with
// hipcc for the host from the kernel source: the argument checks
// (a2a_prepare), then the kernel's word map (a2a_word) run on host buffers over
// a grid of group sizes, row counts, head counts, head sizes, both directions
// and both word sizes. Checked: every source and destination offset lies inside
// its buffer, every destination word is written exactly once, the result is the
// definition (seq -> head: dst[i][j rows + r][h] = src[j][r][i hn + h]; head ->
// seq the inverse), and a round trip returns the input. Invalid arguments get
// their documented codes.
#include "ulysses.hip"
#include <cstdio>
#include <cstring>
#include <vector>
using namespace cpattn;

static long long bad = 0, checked = 0;

#define CHECK(cond, ...)                   \
  do {                                     \
    ++checked;                             \
    if (!(cond)) {                         \
      if (++bad < 20) printf(__VA_ARGS__); \
    }                                      \
  } while (0)

// runs the kernel's map on host buffers; returns false on an out-of-range or repeated write
static bool emulate(int n, int64_t rows, int n_heads, int64_t hb, const std::vector<std::vector<uint8_t>> &src,
                    std::vector<std::vector<uint8_t>> &dst, int direction) {
  std::vector<const void *> ps(n);
  std::vector<void *> pd(n);
  for (int k = 0; k < n; ++k) {
    ps[k] = src[k].data();
    pd[k] = dst[k].data();
  }
  A2aArgs a;
  int word = 0;
  const int rc = a2a_prepare(n, rows, n_heads, hb, ps.data(), pd.data(), direction, a, word);
  CHECK(rc == CPATTN_OK, "prepare failed %d\n", rc);
  if (rc != CPATTN_OK) return false;
  const int64_t bytes = rows * n_heads * hb, nw = bytes / word;
  std::vector<std::vector<uint8_t>> hit(n, std::vector<uint8_t>((size_t)nw, 0));
  bool ok = true;
  for (int64_t w = 0; w < a.words; ++w) {
    const A2aWord o = a2a_word(a, w);
    const bool in = o.src_rank >= 0 && o.src_rank < n && o.dst_rank >= 0 && o.dst_rank < n && o.src_off >= 0 &&
                    o.src_off < nw && o.dst_off >= 0 && o.dst_off < nw;
    CHECK(in, "word %lld out of range\n", (long long)w);
    if (!in) return false;
    CHECK(hit[o.dst_rank][o.dst_off] == 0, "destination word written twice\n");
    ok = ok && hit[o.dst_rank][o.dst_off] == 0;
    hit[o.dst_rank][o.dst_off] = 1;
    memcpy(&dst[o.dst_rank][o.dst_off * word], &src[o.src_rank][o.src_off * word], word);
  }
  for (int k = 0; k < n; ++k)
    for (int64_t x = 0; x < nw; ++x) CHECK(hit[k][x] == 1, "destination word never written\n");
  return ok;
}

static void check_case(int n, int64_t rows, int n_heads, int64_t hb) {
  const int64_t bytes = rows * n_heads * hb, hn = n_heads / n;
  std::vector<std::vector<uint8_t>> seq(n, std::vector<uint8_t>((size_t)bytes + 16)), head(n), back(n);
  uint32_t x = 12345u + (uint32_t)(n * 7 + rows * 13 + n_heads * 17 + hb);
  for (auto &b : seq)
    for (auto &c : b) c = (uint8_t)((x = x * 1664525u + 1013904223u) >> 24);
  for (int k = 0; k < n; ++k) {
    head[k].assign((size_t)bytes + 16, 0xEE);
    back[k].assign((size_t)bytes + 16, 0xDD);
  }
  if (!emulate(n, rows, n_heads, hb, seq, head, 0)) return;
  // the definition, byte by byte
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j)
      for (int64_t r = 0; r < rows; ++r)
        for (int64_t h = 0; h < hn; ++h) {
          const uint8_t *want = &seq[j][(size_t)((r * n_heads + i * hn + h) * hb)];
          const uint8_t *got = &head[i][(size_t)(((j * rows + r) * hn + h) * hb)];
          CHECK(memcmp(want, got, (size_t)hb) == 0, "seq->head mismatch n=%d rows=%lld heads=%d hb=%lld\n", n,
                (long long)rows, n_heads, (long long)hb);
        }
  for (int k = 0; k < n; ++k)
    for (int64_t b = bytes; b < bytes + 16; ++b) CHECK(head[k][(size_t)b] == 0xEE, "write past the end\n");
  if (!emulate(n, rows, n_heads, hb, head, back, 1)) return;
  for (int k = 0; k < n; ++k)
    CHECK(memcmp(seq[k].data(), back[k].data(), (size_t)bytes) == 0, "round trip differs n=%d rows=%lld\n", n,
          (long long)rows);
}

static void check_errors() {
  std::vector<uint8_t> b0(4096), b1(4096), b2(4096), b3(4096);
  const void *s2[2] = {b0.data(), b1.data()};
  void *d2[2] = {b2.data(), b3.data()};
  A2aArgs a;
  int w = 0;
  CHECK(a2a_prepare(0, 4, 4, 16, s2, d2, 0, a, w) == CPATTN_E_ARG, "n 0\n");
  CHECK(a2a_prepare(65, 4, 65, 16, s2, d2, 0, a, w) == CPATTN_E_UNSUPPORTED, "n 65\n");
  CHECK(a2a_prepare(2, 4, 3, 16, s2, d2, 0, a, w) == CPATTN_E_DIVISIBILITY, "heads 3 over 2 ranks\n");
  CHECK(a2a_prepare(2, 4, 4, 6, s2, d2, 0, a, w) == CPATTN_E_ARG, "head bytes 6\n");
  CHECK(a2a_prepare(2, 4, 4, 16, s2, d2, 2, a, w) == CPATTN_E_ARG, "direction 2\n");
  CHECK(a2a_prepare(2, -1, 4, 16, s2, d2, 0, a, w) == CPATTN_E_ARG, "rows -1\n");
  CHECK(a2a_prepare(2, 4, 4, 16, nullptr, d2, 0, a, w) == CPATTN_E_ARG, "null src\n");
  const void *sn[2] = {b0.data(), nullptr};
  CHECK(a2a_prepare(2, 4, 4, 16, sn, d2, 0, a, w) == CPATTN_E_ARG, "null src entry\n");
  void *dov[2] = {b2.data(), b2.data() + 64};   // the two destinations overlap (256 bytes each)
  CHECK(a2a_prepare(2, 4, 4, 16, s2, dov, 0, a, w) == CPATTN_E_ARG, "overlapping destinations\n");
  void *dsrc[2] = {b2.data(), b1.data() + 128};   // a destination inside a source
  CHECK(a2a_prepare(2, 4, 4, 16, s2, dsrc, 0, a, w) == CPATTN_E_ARG, "destination over a source\n");
  const void *smis[2] = {b0.data() + 2, b1.data()};
  CHECK(a2a_prepare(2, 4, 4, 16, smis, d2, 0, a, w) == CPATTN_E_ARG, "misaligned source\n");
  const void *s4[2] = {b0.data() + 4, b1.data()};
  CHECK(a2a_prepare(2, 4, 4, 16, s4, d2, 0, a, w) == CPATTN_OK && w == 4, "4-byte aligned takes the 4-byte path\n");
  CHECK(a2a_prepare(2, 4, 4, 16, s2, d2, 0, a, w) == CPATTN_OK, "valid call\n");
  CHECK(a2a_prepare(2, 0, 4, 16, s2, d2, 0, a, w) == CPATTN_OK && a.words == 0, "zero rows\n");
  CHECK(a2a_prepare(2, 1LL << 40, 1 << 20, 1LL << 20, s2, d2, 0, a, w) == CPATTN_E_UNSUPPORTED, "int64 overflow\n");
}

int main() {
  check_errors();
  for (int n : {1, 2, 3, 4, 8})
    for (int64_t rows : {0, 1, 5, 32})
      for (int hpr : {1, 2, 3})
        for (int64_t hb : {4, 12, 16, 256, 1028}) check_case(n, rows, n * hpr, hb);
  check_case(16, 7, 32, 64);
  check_case(64, 3, 64, 16);
  printf("%lld checks, %lld failures\n", checked, bad);
  return bad != 0;
}
