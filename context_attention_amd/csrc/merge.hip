// Merge of online-softmax triples and finalisation (G5 context-parallel
// modelling spec, Definitions table, "Partial attention": partials carry the
// max, the numerator and the denominator, and their merge is associative and
// independent of order).
//
// One wavefront per (row, head): every lane reads the n_parts + 1 maxima and
// denominators (the same addresses, served as broadcasts), computes the merge
// weights, rescales and sums its share of the numerator, and lane 0 writes
// back the merged max and denominator after all lanes have read them. The
// tree-order reduction at the end of this file chains the same kernel.
#include "kernels.h"

namespace cpattn {
namespace {

constexpr int kMaxParts = 16;   // parts per launch; the host chains launches beyond that

struct MergeArgs {
  const float *pm[kMaxParts];
  const float *pd[kMaxParts];
  const float *pn[kMaxParts];
  int32_t n_parts;
  float *am;
  float *ad;
  float *an;
  float *out;
  float *lse;
  int64_t items;   // rows * n_hq
};

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int PER = D / 64;   // numerator elements per lane (1, 2 or 8)
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.items) return;
  const int lane = threadIdx.x & 63;

  float m = a.am[item];
  float den = a.ad[item];
  float acc[PER];
  float *anp = a.an + item * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = anp[e];

  for (int p = 0; p < a.n_parts; ++p) {
    const float mp = a.pm[p][item];
    const float dp = a.pd[p][item];
    float mn, w0, w1;
    merge_weights(m, mp, mn, w0, w1);
    const float *pnp = a.pn[p] + item * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = w0 * acc[e] + w1 * pnp[e];
    den = w0 * den + w1 * dp;
    m = mn;
  }
  if (a.n_parts > 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) anp[e] = acc[e];
    if (lane == 0) {
      a.am[item] = m;
      a.ad[item] = den;
    }
  }
  if (a.out != nullptr) {
    const float inv = den > 0.f ? 1.f / den : 0.f;
    float *op = a.out + item * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) op[e] = acc[e] * inv;
  }
  if (a.lse != nullptr && lane == 0) a.lse[item] = den > 0.f ? m + logf(den) : kNegInf;
}

template <int D>
hipError_t launch_merge(const MergeArgs &a, hipStream_t s) {
  const int64_t blocks = (a.items + 3) / 4;
  hipLaunchKernelGGL(merge_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace cpattn

extern "C" int cpattn_merge(int64_t rows, int32_t n_hq, int32_t head_dim, const cpattn_partial *parts,
                            int32_t n_parts, const cpattn_partial *acc, float *out, float *lse,
                            hipStream_t stream) {
  using namespace cpattn;
  if (rows < 0 || n_hq < 1 || n_parts < 0 || acc == nullptr) return CPATTN_E_ARG;
  if (n_parts > 0 && parts == nullptr) return CPATTN_E_ARG;
  if (head_dim != 64 && head_dim != 128 && head_dim != 512) return CPATTN_E_UNSUPPORTED;
  if (rows == 0) return CPATTN_OK;
  if (acc->m == nullptr || acc->den == nullptr || acc->num == nullptr) return CPATTN_E_ARG;
  for (int p = 0; p < n_parts; ++p)
    if (parts[p].m == nullptr || parts[p].den == nullptr || parts[p].num == nullptr) return CPATTN_E_ARG;
  const int64_t items = rows * (int64_t)n_hq;
  if ((items + 3) / 4 > 0x7FFFFFFFLL) return CPATTN_E_UNSUPPORTED;

  int done = 0;
  do {
    MergeArgs a;
    const int n = n_parts - done < kMaxParts ? n_parts - done : kMaxParts;
    for (int p = 0; p < n; ++p) {
      a.pm[p] = parts[done + p].m;
      a.pd[p] = parts[done + p].den;
      a.pn[p] = parts[done + p].num;
    }
    a.n_parts = n;
    a.am = acc->m;
    a.ad = acc->den;
    a.an = acc->num;
    const bool last = done + n >= n_parts;
    a.out = last ? out : nullptr;
    a.lse = last ? lse : nullptr;
    a.items = items;
    hipError_t e;
    if (head_dim == 64) e = launch_merge<64>(a, stream);
    else if (head_dim == 128) e = launch_merge<128>(a, stream);
    else e = launch_merge<512>(a, stream);
    if (e != hipSuccess) return CPATTN_E_DEVICE;
    done += n;
  } while (done < n_parts);
  return CPATTN_OK;
}

// Tree-order reduction of n_parts triples (the Tree Attention reduction the
// G5 spec lists as follow-up work for pass-Q: Limitations table, "pass-Q
// reduction topology fixed"): round k merges part s + 2^k into part s for every
// s that is a multiple of 2^(k+1), the exchange pattern of a tree over n_parts
// ranks; ceil(log2 n_parts) rounds, n_parts - 1 merges in all. Each merge is one
// merge_kernel launch with the receiving part as the accumulator.
extern "C" int cpattn_tree_reduce(int64_t rows, int32_t n_hq, int32_t head_dim, const cpattn_partial *parts,
                                  int32_t n_parts, float *out, float *lse, hipStream_t stream) {
  using namespace cpattn;
  if (rows < 0 || n_hq < 1 || n_parts < 1 || parts == nullptr) return CPATTN_E_ARG;
  if (head_dim != 64 && head_dim != 128 && head_dim != 512) return CPATTN_E_UNSUPPORTED;
  for (int p = 0; p < n_parts; ++p) {
    if (parts[p].m == nullptr || parts[p].den == nullptr || parts[p].num == nullptr) return CPATTN_E_ARG;
    for (int q = 0; q < p; ++q)   // a part merged into itself would be counted twice
      if (parts[p].m == parts[q].m || parts[p].den == parts[q].den || parts[p].num == parts[q].num)
        return CPATTN_E_ARG;
  }
  if (rows == 0) return CPATTN_OK;
  const int64_t items = rows * (int64_t)n_hq;
  if ((items + 3) / 4 > 0x7FFFFFFFLL) return CPATTN_E_UNSUPPORTED;
  auto launch = [&](const cpattn_partial *from, const cpattn_partial &into, float *o, float *l) {
    MergeArgs a;
    a.n_parts = from ? 1 : 0;
    if (from) {
      a.pm[0] = from->m;
      a.pd[0] = from->den;
      a.pn[0] = from->num;
    }
    a.am = into.m;
    a.ad = into.den;
    a.an = into.num;
    a.out = o;
    a.lse = l;
    a.items = items;
    if (head_dim == 64) return launch_merge<64>(a, stream);
    if (head_dim == 128) return launch_merge<128>(a, stream);
    return launch_merge<512>(a, stream);
  };
  for (int span = 1; span < n_parts; span *= 2)
    for (int s = 0; s + span < n_parts; s += 2 * span)
      if (launch(&parts[s + span], parts[s], nullptr, nullptr) != hipSuccess) return CPATTN_E_DEVICE;
  if ((out != nullptr || lse != nullptr) && launch(nullptr, parts[0], out, lse) != hipSuccess) return CPATTN_E_DEVICE;
  return CPATTN_OK;
}
