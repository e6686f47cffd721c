// Host check of the ring step's copy resources: the running-sum walk (TileWalk)
// gives the directly computed resource (seg_tile_words) bit for bit for every
// tile a workgroup copies, over the launch tables of a set of ring steps (all
// ranks and steps; ragged, padded, empty and single-token sequences; both
// kernels' row blocks) and over random segment geometries whose ranges pass the
// 2^31 clamp. Built with hipcc for the host from the kernel source itself.
#include "prefill.hip"
#include <cstdio>
#include <random>
#include <vector>
using namespace cpattn;

static long long bad = 0, checked = 0;

template <int BN>
static void walk_cmp(const Segs<BN> &sg, int ntiles, const char *blk, uint32_t rb, int t0, int steps) {
  TileWalk<BN> w(sg, ntiles, blk, t0, rb);
  for (int i = 0; i < steps; ++i) {
    const int t = t0 + i;
    const u32x4_t a = w.words(), b = seg_tile_words<BN>(sg, ntiles, blk, t, rb);
    if (t < ntiles) {   // a tile before the end has keys left
      const int s = sg.seg(t), k = sg.k0(t);
      if (sg.end[s] - k <= 0) { ++bad; printf("tile %d before the end has no keys\n", t); }
    }
    ++checked;
    if (a[0] != b[0] || a[1] != b[1] || a[2] != b[2] || a[3] != b[3]) {
      if (++bad < 10)
        printf("MISMATCH t=%d ntiles=%d n0=%d end=%d,%d row=%lld,%lld: walk %08x %08x %08x  direct %08x %08x %08x\n",
               t, ntiles, sg.n0, sg.end[0], sg.end[1], (long long)sg.row[0], (long long)sg.row[1], a[0], a[1], a[2],
               b[0], b[1], b[2]);
    }
    w.next();
  }
}

// The per-row copy resources of the head_dim 512 kernel (RowWalk), for every
// tile from 0 to past the end and every key row q of a 32-key tile and every
// head offset: a row with keys in range reads the 1 KB of one head inside a
// visible key row of the tile's segment (every lane offset is below 1 KB);
// every visible key row of the tile is copied; rows past the visible keys, and
// every row of a tile past the end, have an empty range based at the block
// start.
static long long rows_checked = 0;
static void rows_cmp(const Segs<32> &sg, int ntiles, const char *blk, uint32_t rb, int n_kv) {
  RowWalk<32> w(sg, ntiles, blk, 0, rb);
  const uint64_t b0 = (uint64_t)(uintptr_t)blk;
  for (int t = 0; t <= ntiles + 2; ++t, w.next()) {
    int vis = 0;
    int64_t first = 0;
    if (t < ntiles) {
      const int s = sg.seg(t), k = sg.k0(t);
      vis = std::min(32, sg.end[s] - k);
      first = sg.row[s] + k;
    }
    for (int q = 0; q < 32; ++q)
      for (int g = 0; g < n_kv; g += (n_kv > 4 ? n_kv / 4 : 1)) {
        const uint32_t gbase = (uint32_t)g * 1024u;
        const u32x4_t r = w.row(q, rb, gbase);
        ++rows_checked;
        const uint64_t base = (uint64_t)(r[1] & 0xFFFFu) << 32 | r[0];
        const bool want = q < vis;
        const bool ok = want ? (r[2] == 1024u && base == b0 + (uint64_t)(first + q) * rb + gbase &&
                                gbase + 1024u <= rb)
                             : (r[2] == 0u && base == b0);
        if (!ok && ++bad < 10)
          printf("ROW MISMATCH t=%d q=%d g=%d vis=%d nrec=%u base=%llx\n", t, q, g, vis, r[2],
                 (unsigned long long)base);
      }
  }
}

// every workgroup of one ring step, geometry as in the kernels
template <int BN>
static void launch_cmp(const std::vector<long long> &lens, int cp, int rank, int step, int bm, int n_kv, int d) {
  const int src = ((rank - step) % cp + cp) % cp;
  StepArgs a{};
  a.a_head = rank; a.a_tail = 2 * cp - 1 - rank; a.b_head = src; a.b_tail = 2 * cp - 1 - src;
  SeqTable t{};
  t.start[0] = 0;
  long long units = 0, row_off = 0;
  for (long long L : lens) {
    const long long c = (L + 2 * cp - 1) / (2 * cp);
    t.c[t.n] = (int)c; t.len[t.n] = (int)L; t.row_off[t.n] = row_off;
    units += 2 * ((c + bm - 1) / bm);
    t.start[t.n + 1] = (int)units;
    row_off += 2 * c;
    ++t.n;
  }
  const uint32_t rb = (uint32_t)(n_kv * d * 2);
  const char *blk = reinterpret_cast<const char *>((uintptr_t)0x7f1234560000ull);
  for (int unit = 0; unit < units; ++unit) {
    const int si = find_seq(t, unit);
    const int c = t.c[si];
    const int nt = (c + bm - 1) / bm;
    const int lt = unit - t.start[si];
    const bool tail = lt < nt;
    const int tile = tail ? (nt - 1 - lt) : (nt - 1 - (lt - nt));
    const int qa = tail ? a.a_tail : a.a_head;
    const int wg_row_end = std::min(c, tile * bm + bm);
    const int len = t.len[si];
    const int q_valid = chunk_valid(len, qa, c);
    const Segs<BN> sg = make_segs<BN>(a, qa, c, len, t.row_off[si], std::min(wg_row_end, q_valid));
    if (sg.nseg == 0) continue;
    const int ntiles = sg.tiles();
    walk_cmp<BN>(sg, ntiles, blk, rb, 2, ntiles + 3);   // K: tiles 2 .. past the end
    walk_cmp<BN>(sg, ntiles, blk, rb, 1, ntiles + 3);   // V: tiles 1 ..
    if constexpr (BN == 32) rows_cmp(sg, ntiles, blk, rb, n_kv);
  }
}

template <int BN>
static void configs(int bm, int d) {
  struct C { std::vector<long long> lens; int cp, n_kv; };
  std::vector<C> cs = {
      {{2 * 2 * 96, 2 * 2 * 40}, 2, 2}, {{600, 198}, 3, 2}, {{800}, 4, 2}, {{280, 520, 36}, 2, 8},
      {{1 << 15}, 8, 8}, {{1 << 17}, 8, 8}, {{17, 1, 0, 5000, 333}, 4, 1}, {{64 * 16, 64 * 16 + 7}, 8, 4},
      {{3, 64, 65, 127, 128, 129}, 1, 1}, {{100000, 40000, 1}, 4, 64}, {{83680}, 4, 64}};
  for (auto &c : cs)
    for (int r = 0; r < c.cp; ++r)
      for (int s = 0; s < c.cp; ++s) launch_cmp<BN>(c.lens, c.cp, r, s, bm, c.n_kv, d);
}

template <int BN>
static void random_segs(int n) {
  std::mt19937_64 g(12345);
  for (int i = 0; i < n; ++i) {
    Segs<BN> sg{};
    sg.nseg = 1 + (int)(g() % 2);
    const int big = (int)(g() % 3);
    auto len = [&]() { return 1 + (int)(g() % (big == 2 ? (1u << 22) : big == 1 ? 4096u : 200u)); };
    sg.end[0] = len();
    sg.end[1] = sg.nseg > 1 ? len() : 0;
    sg.row[0] = (int64_t)(g() % (1u << 22));
    sg.row[1] = (int64_t)(g() % (1u << 22));
    sg.n0 = (sg.end[0] + BN - 1) / BN;
    const int ntiles = sg.tiles();
    const uint32_t rb = (uint32_t)((1 + g() % 128) * 1024);   // up to 128 KB per key row
    const char *blk = reinterpret_cast<const char *>((uintptr_t)(0x100000000ull + (g() % (1ull << 40))));
    const int t0 = (int)(g() % 3);
    const int steps = ntiles > 4000 ? 4000 : ntiles + 3;
    walk_cmp<BN>(sg, ntiles, blk, rb, t0, steps);
  }
}

int main() {
  configs<64>(32 * 8 / 4, 128);   // d64/128 kernel, 4 heads per workgroup
  configs<64>(32 * 8 / 2, 128);
  configs<64>(32 * 8 / 1, 64);
  configs<32>(kRowsWide<1>, 512);   // d512 kernel: K and V walks both from tile 1
  configs<32>(kRowsWide<2>, 512);
  configs<32>(kRowsWide<4>, 512);
  random_segs<64>(20000);
  random_segs<32>(20000);
  printf("checked %lld resources and %lld row resources, %lld mismatches\n", checked, rows_checked, bad);
  return bad != 0;
}
