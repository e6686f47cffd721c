// Host check of the pass-Q decode planner: for every description in a grid of
// batch sizes, shard counts, key lengths, head layouts and head dims, the key
// splits of a shard must tile [0, shard_len) exactly once (every split but the
// last full, none empty unless the shard is), be whole rounds of the kernel's
// key step, and bring the grid close to the planner's workgroup target without
// going over it by more than one split per group. Built with hipcc for the host
// from the kernel source itself.
#include "decode.hip"
#include <cstdio>
#include <vector>
using namespace cpattn;

static long long bad = 0, checked = 0;

#define CHECK(cond, ...)                       \
  do {                                         \
    if (!(cond)) {                             \
      if (++bad < 20) printf(__VA_ARGS__);     \
    }                                          \
  } while (0)

int main() {
  const int dims[] = {64, 128, 512};
  const int cps[] = {1, 2, 3, 4, 8, 16};
  const int batches[] = {1, 2, 3, 8, 32};
  const int64_t lens[] = {0, 1, 7, 32, 63, 64, 65, 1000, 4096, 65536, 131072, 1 << 20};
  const int layouts[][2] = {{1, 1}, {2, 2}, {4, 1}, {8, 2}, {16, 1}, {32, 1}, {32, 4}, {32, 8},
                            {48, 1}, {64, 1}, {96, 2}, {128, 1}, {256, 1}, {64, 2}};
  for (int D : dims)
    for (int cp : cps)
      for (int b : batches)
        for (int64_t per_shard : lens)
          for (auto &hl : layouts)
            for (int dt = 0; dt < 2; ++dt) {
              cpattn_decode_desc d{};
              d.batch = b;
              d.cp = cp;
              d.kv_len = per_shard * cp;
              d.n_hq = hl[0];
              d.n_kv = hl[1];
              d.head_dim = D;
              d.dtype = dt ? CPATTN_DT_BF16 : CPATTN_DT_F32;
              d.scale = 0.1f;
              const DecodePlan p = plan_decode(d);
              const int64_t shard_len = d.kv_len / d.cp;
              ++checked;
              // the kernel's key step: one round of its waves
              int64_t step;
              int64_t groups;
              int64_t target;
              if (p.mfma16) {
                step = 32;
                groups = (int64_t)cp * b * d.n_kv * p.ncb;
                target = 512;
              } else if (p.mfma) {
                step = 32LL * kg_of(D);
                groups = (int64_t)cp * b * d.n_kv * p.ncb;
                target = 512;
              } else {
                step = (int64_t)(64 / (D / 8)) * kDecWaves * kUnroll;
                groups = (int64_t)cp * b * (d.n_hq / p.gv);
                target = 8192;
              }
              CHECK(p.nsplit >= 1, "D%d cp%d b%d len%lld %d/%d: nsplit %d\n", D, cp, b, (long long)per_shard, hl[0],
                    hl[1], p.nsplit);
              CHECK(p.split_len >= step && p.split_len % step == 0,
                    "D%d cp%d b%d len%lld %d/%d: split_len %lld, step %lld\n", D, cp, b, (long long)per_shard, hl[0],
                    hl[1], (long long)p.split_len, (long long)step);
              // exact cover: nsplit - 1 full splits, the last one non-empty (or a single empty split)
              CHECK((int64_t)p.nsplit * p.split_len >= shard_len, "D%d cp%d b%d len%lld: splits do not cover\n", D, cp,
                    b, (long long)per_shard);
              if (shard_len > 0)
                CHECK((int64_t)(p.nsplit - 1) * p.split_len < shard_len, "D%d cp%d b%d len%lld: an empty split\n", D,
                      cp, b, (long long)per_shard);
              else
                CHECK(p.nsplit == 1, "empty shard, %d splits\n", p.nsplit);
              // the grid: at most the target rounded up to whole groups. The split count is capped at
              // ceil(shard_len / 4 rounds), so a split holds more than 2 rounds of keys, at least 3
              // once rounded up to whole rounds, whenever the shard is split at all
              CHECK(groups * p.nsplit <= ((target + groups - 1) / groups) * groups,
                    "D%d cp%d b%d len%lld %d/%d: %lld workgroups for target %lld\n", D, cp, b, (long long)per_shard,
                    hl[0], hl[1], (long long)(groups * p.nsplit), (long long)target);
              if (p.nsplit > 1)
                CHECK(p.split_len >= 3 * step, "D%d cp%d b%d len%lld: split of %lld keys under 3 rounds\n", D, cp, b,
                      (long long)per_shard, (long long)p.split_len);
              // kernel choice: matrix cores for bf16 with 8 or more heads per kv head
              const int G = d.n_hq / d.n_kv;
              CHECK(p.mfma == (dt == 1 && G >= 8) && p.mfma16 == (dt == 1 && G > 32),
                    "D%d %d/%d dt%d: kernel choice mfma %d mfma16 %d\n", D, hl[0], hl[1], dt, p.mfma, p.mfma16);
            }
  printf("checked %lld plans, %lld failures\n", checked, bad);
  return bad != 0;
}
