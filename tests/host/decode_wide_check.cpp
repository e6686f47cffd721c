// Host model of decode_wide's indexing (the head_dim 512 decode for more than
// 112 query heads per kv head), over a grid of descriptions that the planner
// routes to it. Built with hipcc for the host from the kernel source, so the
// planner, the argument block, the workgroup decode (wide_block), the key split
// as a segment (split_segs) and the copy walk (RowWalk) are the kernel's own.
// Checked for every workgroup:
//   - the workgroups map one to one onto (shard, batch entry, split, kv head,
//     head block);
//   - every Q load and every split-triple write of a head lane lies inside its
//     tensor (heads past the kv group are neither loaded nor stored);
//   - every copy resource of every tile (and of the tile past the last, which
//     the loop also issues) either covers exactly the 1 KB of the kv head in a
//     key row of the split, inside the shard's rows of the batch entry, or is
//     empty; each key row of the split is copied once;
//   - every LDS read (K fragments, transposed V reads) and every copy
//     destination stays inside its double-buffered tile.
#include "decode.hip"
#include <cstdio>
#include <vector>
using namespace cpattn;

static long long bad = 0, checked = 0, rows_checked = 0;

#define CHECK(cond, ...)                   \
  do {                                     \
    ++checked;                             \
    if (!(cond)) {                         \
      if (++bad < 20) printf(__VA_ARGS__); \
    }                                      \
  } while (0)

constexpr int D = 512, BN = 32, TSZ = BN * D;

// LDS element offsets of the kernel's reads (cur: buffer 0 or 1)
static void check_lds() {
  for (int lane = 0; lane < 64; ++lane) {
    const int col = lane & 15, grp = lane >> 4;
    for (int cur = 0; cur < 2; ++cur) {
      for (int ks = 0; ks < D / 32; ++ks)
        for (int blk = 0; blk < 2; ++blk) {
          const int j = ks & 3;
          const long off = col * D + 8 * (4 * (j ^ (col >> 2)) + (grp ^ (col & 3))) + cur * TSZ + 128 * (ks >> 2) +
                           blk * 16 * D;
          CHECK(off >= 0 && off + 8 <= 2L * TSZ, "K read out of the tiles: lane %d ks %d\n", lane, ks);
        }
      const int vrow = 4 * grp + (col >> 2);
      for (int db = 0; db < D / 16; ++db) {
        const int j = db & 7;
        const long p0 = vrow * D + 16 * (j ^ (vrow & 7)) + 8 * ((col >> 1) & 1) + 4 * (col & 1) + cur * TSZ +
                        128 * (db >> 3);
        CHECK(p0 >= cur * (long)TSZ && p0 + 16L * D + 4 <= (cur + 1L) * TSZ, "V read out of its tile: lane %d db %d\n",
              lane, db);
      }
    }
  }
  for (int q = 0; q < BN; ++q) CHECK(q * 512 + 512 <= TSZ, "copy destination of row %d\n", q);
}

static void check_desc(int cp, int batch, int64_t per_shard, int n_hq, int n_kv, bool full_walk) {
  cpattn_decode_desc d{};
  d.batch = batch;
  d.cp = cp;
  d.kv_len = per_shard * cp;
  d.n_hq = n_hq;
  d.n_kv = n_kv;
  d.head_dim = D;
  d.dtype = CPATTN_DT_BF16;
  d.scale = 0.05f;
  const DecodePlan p = plan_decode(d);
  const int G = n_hq / n_kv;
  CHECK(p.wide == ((G + 15) / 16 >= kWideWaves), "%d/%d: routed to decode_wide %d\n", n_hq, n_kv, p.wide);
  if (!p.wide) return;
  CHECK(p.ncb == (G + kWideHeads - 1) / kWideHeads, "%d/%d: %d head blocks\n", n_hq, n_kv, p.ncb);
  // fake device addresses, far apart
  const uint64_t QB = 0x100000000000ull, KB = 0x200000000000ull, VB = 0x300000000000ull;
  const void *ks[kMaxShards], *vs[kMaxShards];
  for (int s = 0; s < cp; ++s) {
    ks[s] = (const void *)(uintptr_t)(KB + (uint64_t)s * (1ull << 40));
    vs[s] = (const void *)(uintptr_t)(VB + (uint64_t)s * (1ull << 40));
  }
  const MfmaArgs a = mfma_args(d, p, (const void *)(uintptr_t)QB, ks, vs, nullptr, nullptr, nullptr);
  const int64_t shard_len = per_shard;
  const int64_t units = (int64_t)cp * batch * p.nsplit;
  const int64_t blocks = units * n_kv * p.ncb;
  const int64_t triples = (int64_t)cp * batch * n_hq * p.nsplit;
  const uint32_t rb = (uint32_t)(n_kv * D * 2);
  std::vector<int> seen((size_t)blocks, 0);
  for (int64_t b = 0; b < blocks; ++b) {
    const WideBlock wb = wide_block(a, b);
    const bool in = wb.s >= 0 && wb.s < cp && wb.bi >= 0 && wb.bi < batch && wb.sp >= 0 && wb.sp < p.nsplit &&
                    wb.g >= 0 && wb.g < n_kv && wb.hs >= 0 && wb.hs < p.ncb;
    CHECK(in, "block %lld decodes out of range\n", (long long)b);
    if (!in) continue;
    const int64_t id = ((((int64_t)wb.s * batch + wb.bi) * p.nsplit + wb.sp) * n_kv + wb.g) * p.ncb + wb.hs;
    ++seen[(size_t)id];
    CHECK(wb.k_begin >= 0 && wb.k_end <= shard_len, "split [%lld, %lld) outside the shard\n", (long long)wb.k_begin,
          (long long)wb.k_end);
    const int nkeys = wb.k_end > wb.k_begin ? (int)(wb.k_end - wb.k_begin) : 0;
    const int ntiles = (nkeys + BN - 1) / BN;
    // head lanes: Q loads and triple writes
    for (int wave = 0; wave < kWideWaves; ++wave)
      for (int lane = 0; lane < 64; ++lane) {
        const int col = lane & 15, grp = lane >> 4;
        const int hc = wb.hs * kWideHeads + wave * 16 + col;
        const bool head_ok = hc < a.rep;
        const int h = wb.g * a.rep + (head_ok ? hc : 0);
        CHECK(h >= 0 && h < n_hq, "head %d\n", h);
        if (!head_ok || ntiles == 0) continue;
        const int64_t q_last = ((int64_t)wb.bi * n_hq + h) * D + 8 * grp + 32 * 15 + 8;
        CHECK(q_last <= (int64_t)batch * n_hq * D, "Q load past the end\n");
        const int64_t wi = ((((int64_t)wb.s * batch + wb.bi) * n_hq + (int64_t)wb.g * a.rep) + hc) * p.nsplit + wb.sp;
        CHECK(wi >= 0 && wi < triples, "triple %lld of %lld\n", (long long)wi, (long long)triples);
        CHECK(wi * D + 4 * grp + 16 * 31 + 4 <= triples * D, "numerator write past the end\n");
      }
    if (!full_walk && b > 3 && b < blocks - 4) continue;
    // copy resources: tiles 0 .. ntiles (the loop issues the copies of tile it+1 during tile it)
    const Segs<BN> sg = split_segs<BN>(wb.bi, shard_len, wb.k_begin, nkeys);
    const char *kblk = (const char *)a.k[wb.s];
    const uint32_t gbase = (uint32_t)(wb.g * D * 2);
    CHECK(gbase + 1024u <= rb, "kv head past the key row\n");
    RowWalk<BN> kw(sg, ntiles, kblk, 0, rb);
    std::vector<int> copied((size_t)nkeys + 1, 0);
    for (int t = 0; t <= ntiles; ++t, kw.next()) {
      for (int q = 0; q < BN; ++q) {   // row q is copied by wave q % 8, copy q / 8
        const u32x4_t r = kw.row(q, rb, gbase);
        ++rows_checked;
        const uint64_t base = (uint64_t)(r[1] & 0xFFFFu) << 32 | r[0];
        const int64_t k = (int64_t)t * BN + q;
        if (t < ntiles && k < nkeys) {
          const int64_t rowi = (int64_t)wb.bi * shard_len + wb.k_begin + k;
          CHECK(r[2] == 1024u && base == (uint64_t)(uintptr_t)kblk + (uint64_t)rowi * rb + gbase,
                "visible row t %d q %d: nrec %u base %llx\n", t, q, r[2], (unsigned long long)base);
          CHECK(rowi >= (int64_t)wb.bi * shard_len && rowi < ((int64_t)wb.bi + 1) * shard_len &&
                    rowi < (int64_t)batch * shard_len,
                "row %lld outside the batch entry's rows\n", (long long)rowi);
          ++copied[(size_t)k];
        } else {
          CHECK(r[2] == 0u && base == (uint64_t)(uintptr_t)kblk, "row past the split: t %d q %d nrec %u\n", t, q, r[2]);
        }
      }
    }
    for (int k = 0; k < nkeys; ++k) CHECK(copied[(size_t)k] == 1, "key %d copied %d times\n", k, copied[(size_t)k]);
  }
  for (int64_t i = 0; i < blocks; ++i) CHECK(seen[(size_t)i] == 1, "unit %lld seen %d times\n", (long long)i, seen[(size_t)i]);
}

int main() {
  check_lds();
  const int layouts[][2] = {{128, 1}, {120, 1}, {136, 1}, {192, 1}, {256, 1}, {256, 2}, {384, 3}, {128, 4}, {112, 1},
                            {64, 1}};
  const int cps[] = {1, 2, 3, 8};
  const int batches[] = {1, 3, 8};
  const int64_t lens[] = {0, 1, 31, 32, 33, 95, 1000, 4096, 16411};
  for (auto &hl : layouts)
    for (int cp : cps)
      for (int b : batches)
        for (int64_t L : lens) check_desc(cp, b, L, hl[0], hl[1], true);
  // the MLA-like decode workload and larger shards, first and last workgroups walked in full
  check_desc(8, 8, 131072, 128, 1, false);
  check_desc(8, 2, 1 << 20, 256, 2, false);
  check_desc(4, 16, 65536 + 7, 128, 1, false);
  printf("%lld checks (%lld copy resources), %lld failures\n", checked, rows_checked, bad);
  return bad != 0;
}
