// Pass-Q decode (G5 context-parallel modelling spec, Definitions table,
// "Pass-Q"; Use case, decode): the query of every batch entry goes to all cp
// shards, each shard computes the partial attention triple over its own keys
// (no mask), and the cp triples are reduced (max, denominator, numerator).
//
// decode_partial<T, D, G>: streams K and V from HBM. A workgroup owns one
//   (shard, batch entry, kv head, key split); D/8 lanes share one key row
//   (16 bytes of bf16 each, so a wavefront load covers whole contiguous rows),
//   the G query heads of the kv group are scored together and reduced with a
//   butterfly over those lanes, and every group of lanes keeps its own online
//   softmax state, merged across lanes and waves once at the end.
// decode_reduce<D>: one wavefront per (batch entry, query head): folds the
//   key splits into the per-shard triples (the partial that rank s would send),
//   then reduces the cp shard triples into out and lse.
#include "kernels.h"

namespace cpattn {
namespace {

constexpr int kMaxShards = 64;
constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kUnroll = 4;      // keys per lane group per iteration

struct DecodeArgs {
  const void *q;
  const void *k[kMaxShards];
  const void *v[kMaxShards];
  float *ws_m;
  float *ws_den;
  float *ws_num;
  int32_t batch;
  int32_t n_hq;
  int32_t n_kv;
  int32_t nsplit;
  int64_t shard_len;
  int64_t split_len;
  float scale;
};

template <typename T>
struct Raw16;   // 8 elements as raw words
template <>
struct Raw16<__bf16> {
  u32x4_t w;
  // K and V are streamed once: non-temporal loads keep them from displacing
  // other cached data
  __device__ __forceinline__ void load(const __bf16 *p) {
    w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  }
  __device__ __forceinline__ void zero() { w = u32x4_t{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t x = w[e >> 1];
    return (e & 1) ? __uint_as_float(x & 0xFFFF0000u) : __uint_as_float(x << 16);
  }
};
template <>
struct Raw16<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
    b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p + 4));
  }
  __device__ __forceinline__ void zero() { a = f32x4_t{0.f, 0.f, 0.f, 0.f}; b = a; }
  __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

template <typename T, int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_partial(DecodeArgs a) {
  constexpr int LPK = D / 8;            // lanes per key row
  constexpr int KPW = 64 / LPK;         // keys per wave per step
  constexpr int KPI = KPW * kDecWaves;  // keys per workgroup per step
  __shared__ float red_m[kDecWaves][G];
  __shared__ float red_l[kDecWaves][G];
  __shared__ float red_n[kDecWaves][G][D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int slot = lane / LPK;
  const int part = lane - slot * LPK;

  // block -> (shard, batch, split, kv head) with the kv head fastest
  int64_t bid = blockIdx.x;
  const int g = (int)(bid % a.n_kv);
  bid /= a.n_kv;
  const int sp = (int)(bid % a.nsplit);
  bid /= a.nsplit;
  const int bi = (int)(bid % a.batch);
  const int s = (int)(bid / a.batch);

  const int64_t k_begin = (int64_t)sp * a.split_len;
  const int64_t k_end = min(a.shard_len, k_begin + a.split_len);
  const float sl2 = a.scale * kLog2e;

  // query slice of the G heads, prescaled into the exp2 domain
  float qr[G][8];
  {
    const T *qp = reinterpret_cast<const T *>(a.q) + ((int64_t)bi * a.n_hq + g * G) * D + part * 8;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      Elem<T>::load8(qp + gg * D, qr[gg]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[gg][e] *= sl2;
    }
  }

  const T *kb = reinterpret_cast<const T *>(a.k[s]);
  const T *vb = reinterpret_cast<const T *>(a.v[s]);
  const int64_t row_stride = (int64_t)a.n_kv * D;
  const int64_t base = ((int64_t)bi * a.shard_len) * row_stride + (int64_t)g * D + part * 8;

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    m[gg] = kNegInf;
    l[gg] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[gg][e] = 0.f;
  }

  for (int64_t k0 = k_begin; k0 < k_end; k0 += (int64_t)KPI * kUnroll) {
    Raw16<T> kr[kUnroll], vr[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t key = k0 + u * KPI + wave * KPW + slot;
      ok[u] = key < k_end;
      if (ok[u]) {
        kr[u].load(kb + base + key * row_stride);
        vr[u].load(vb + base + key * row_stride);
      } else {
        kr[u].zero();
        vr[u].zero();
      }
    }
    float sc[kUnroll][G];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qr[gg][e], kr[u].get(e), d);
        sc[u][gg] = d;
      }
#pragma unroll
    for (int off = 1; off < LPK; off <<= 1)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int gg = 0; gg < G; ++gg) sc[u][gg] += __shfl_xor(sc[u][gg], off);
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      float mx = m[gg];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (!ok[u]) sc[u][gg] = kNegInf;
        mx = fmaxf(mx, sc[u][gg]);
      }
      const float mref = (mx == kNegInf) ? 0.f : mx;
      const float alpha = exp2_fast(m[gg] - mref);
      m[gg] = mx;
      float psum = 0.f;
      float p[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        p[u] = exp2_fast(sc[u][gg] - mref);
        psum += p[u];
      }
      l[gg] = l[gg] * alpha + psum;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[gg][e] * alpha;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x = fmaf(p[u], vr[u].get(e), x);
        acc[gg][e] = x;
      }
    }
  }

  // merge the KPW lane groups of this wave (same part, different slot)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const float mo = __shfl_xor(m[gg], off);
      const float lo = __shfl_xor(l[gg], off);
      const float mn = fmaxf(m[gg], mo);
      const float mref = (mn == kNegInf) ? 0.f : mn;
      const float w0 = exp2_fast(m[gg] - mref);
      const float w1 = exp2_fast(mo - mref);
      l[gg] = w0 * l[gg] + w1 * lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = __shfl_xor(acc[gg][e], off);
        acc[gg][e] = w0 * acc[gg][e] + w1 * ao;
      }
      m[gg] = mn;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      if (part == 0) {
        red_m[wave][gg] = m[gg];
        red_l[wave][gg] = l[gg];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) red_n[wave][gg][part * 8 + e] = acc[gg][e];
    }
  }
  __syncthreads();
  // wave 0 merges the waves and writes the split's triple (natural-log max)
  if (wave == 0) {
    for (int gg = 0; gg < G; ++gg) {
      float mt = kNegInf;
      for (int w = 0; w < kDecWaves; ++w) mt = fmaxf(mt, red_m[w][gg]);
      const float mref = (mt == kNegInf) ? 0.f : mt;
      float wt[kDecWaves];
      float lt = 0.f;
      for (int w = 0; w < kDecWaves; ++w) {
        wt[w] = exp2_fast(red_m[w][gg] - mref);
        lt += wt[w] * red_l[w][gg];
      }
      const int h = g * G + gg;
      const int64_t wi = (((int64_t)s * a.batch + bi) * a.n_hq + h) * a.nsplit + sp;
      for (int d = lane; d < D; d += 64) {
        float x = 0.f;
        for (int w = 0; w < kDecWaves; ++w) x += wt[w] * red_n[w][gg][d];
        a.ws_num[wi * D + d] = x;
      }
      if (lane == 0) {
        a.ws_m[wi] = (mt == kNegInf) ? kNegInf : mt * kLn2;
        a.ws_den[wi] = lt;
      }
    }
  }
}

struct ReduceArgs {
  const float *ws_m;
  const float *ws_den;
  const float *ws_num;
  float *sp_m;
  float *sp_den;
  float *sp_num;
  float *out;
  float *lse;
  int32_t cp;
  int32_t batch;
  int32_t n_hq;
  int32_t nsplit;
};

template <int D>
__global__ __launch_bounds__(64) void decode_reduce(ReduceArgs a) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const int64_t item = blockIdx.x;   // bi * n_hq + h
  float tm = kNegInf, tl = 0.f, tacc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) tacc[e] = 0.f;
  for (int s = 0; s < a.cp; ++s) {
    const int64_t srow = (int64_t)s * a.batch * a.n_hq + item;   // shard-major row
    float sm = kNegInf, sl = 0.f, sacc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) sacc[e] = 0.f;
    for (int sp = 0; sp < a.nsplit; ++sp) {
      const int64_t wi = srow * a.nsplit + sp;
      float mn, w0, w1;
      merge_weights(sm, a.ws_m[wi], mn, w0, w1);
      sl = w0 * sl + w1 * a.ws_den[wi];
#pragma unroll
      for (int e = 0; e < PER; ++e) sacc[e] = w0 * sacc[e] + w1 * a.ws_num[wi * D + lane * PER + e];
      sm = mn;
    }
    // the shard's partial (what rank s contributes to the reduction)
#pragma unroll
    for (int e = 0; e < PER; ++e) a.sp_num[srow * D + lane * PER + e] = sacc[e];
    if (lane == 0) {
      a.sp_m[srow] = sm;
      a.sp_den[srow] = sl;
    }
    float mn, w0, w1;
    merge_weights(tm, sm, mn, w0, w1);
    tl = w0 * tl + w1 * sl;
#pragma unroll
    for (int e = 0; e < PER; ++e) tacc[e] = w0 * tacc[e] + w1 * sacc[e];
    tm = mn;
  }
  const float inv = tl > 0.f ? 1.f / tl : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) a.out[item * D + lane * PER + e] = tacc[e] * inv;
  if (lane == 0) a.lse[item] = tl > 0.f ? tm + logf(tl) : kNegInf;
}

// Split geometry: enough workgroups to fill the chip several times over, and
// split lengths that are whole numbers of workgroup steps.
void plan_splits(const cpattn_decode_desc &d, int32_t &nsplit, int64_t &split_len) {
  const int64_t shard_len = d.kv_len / d.cp;
  const int64_t step = (int64_t)(64 / (d.head_dim / 8)) * kDecWaves * kUnroll;
  const int64_t groups = (int64_t)d.cp * d.batch * d.n_kv;
  int64_t want = (4096 + groups - 1) / groups;
  int64_t max_by_len = (shard_len + 4 * step - 1) / (4 * step);   // at least 4 steps per split
  if (max_by_len < 1) max_by_len = 1;
  if (want > max_by_len) want = max_by_len;
  if (want < 1) want = 1;
  int64_t len = (shard_len + want - 1) / want;
  len = ((len + step - 1) / step) * step;
  if (len < step) len = step;
  nsplit = (int32_t)((shard_len + len - 1) / len);
  if (nsplit < 1) nsplit = 1;
  split_len = len;
}

template <typename T, int D>
hipError_t launch_partial_g(const DecodeArgs &a, int G, int64_t blocks, hipStream_t s) {
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_partial<T, D, 1>), dim3((unsigned)blocks), dim3(kDecThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_partial<T, D, 2>), dim3((unsigned)blocks), dim3(kDecThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_partial<T, D, 4>), dim3((unsigned)blocks), dim3(kDecThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_partial<T, D, 8>), dim3((unsigned)blocks), dim3(kDecThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_partial(const DecodeArgs &a, int D, int G, int64_t blocks, hipStream_t s) {
  if (D == 64) return launch_partial_g<T, 64>(a, G, blocks, s);
  if (D == 128) return launch_partial_g<T, 128>(a, G, blocks, s);
  return launch_partial_g<T, 512>(a, G, blocks, s);
}

}  // namespace
}  // namespace cpattn

extern "C" int cpattn_passq_decode(const cpattn_decode_desc *desc, const void *q, const void *const *k_shards,
                                   const void *const *v_shards, const cpattn_partial *shard_partials, float *out,
                                   float *lse, void *ws, size_t *ws_bytes, hipStream_t stream) {
  using namespace cpattn;
  if (desc == nullptr || ws_bytes == nullptr) return CPATTN_E_ARG;
  const cpattn_decode_desc d = *desc;
  if (d.cp < 1 || d.batch < 0 || d.kv_len < 0 || d.n_hq < 1 || d.n_kv < 1) return CPATTN_E_ARG;
  if (d.dtype != CPATTN_DT_F32 && d.dtype != CPATTN_DT_BF16) return CPATTN_E_ARG;
  if (!(d.scale > 0.f) || !(d.scale < __builtin_huge_valf())) return CPATTN_E_ARG;
  if (d.n_hq % d.n_kv != 0) return CPATTN_E_DIVISIBILITY;
  if (d.kv_len % d.cp != 0) return CPATTN_E_DIVISIBILITY;
  if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 512) return CPATTN_E_UNSUPPORTED;
  const int G = d.n_hq / d.n_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return CPATTN_E_UNSUPPORTED;
  if (d.cp > kMaxShards) return CPATTN_E_UNSUPPORTED;

  int32_t nsplit;
  int64_t split_len;
  plan_splits(d, nsplit, split_len);
  const int64_t triples = (int64_t)d.cp * d.batch * d.n_hq * nsplit;
  const size_t need = (size_t)triples * (size_t)(2 + d.head_dim) * sizeof(float);
  if (ws == nullptr) {
    *ws_bytes = need;
    return CPATTN_OK;
  }
  if (*ws_bytes < need) return CPATTN_E_WORKSPACE;
  if (d.batch == 0) return CPATTN_OK;
  if (q == nullptr || k_shards == nullptr || v_shards == nullptr || shard_partials == nullptr || out == nullptr ||
      lse == nullptr)
    return CPATTN_E_ARG;
  if (shard_partials->m == nullptr || shard_partials->den == nullptr || shard_partials->num == nullptr)
    return CPATTN_E_ARG;
  for (int s = 0; s < d.cp; ++s)
    if (d.kv_len > 0 && (k_shards[s] == nullptr || v_shards[s] == nullptr)) return CPATTN_E_ARG;
  const int64_t blocks = (int64_t)d.cp * d.batch * nsplit * d.n_kv;
  if (blocks > 0x7FFFFFFFLL || (int64_t)d.batch * d.n_hq > 0x7FFFFFFFLL) return CPATTN_E_UNSUPPORTED;

  DecodeArgs a;
  a.q = q;
  for (int s = 0; s < d.cp; ++s) {
    a.k[s] = k_shards[s];
    a.v[s] = v_shards[s];
  }
  float *wsf = reinterpret_cast<float *>(ws);
  a.ws_m = wsf;
  a.ws_den = wsf + triples;
  a.ws_num = wsf + 2 * triples;
  a.batch = d.batch;
  a.n_hq = d.n_hq;
  a.n_kv = d.n_kv;
  a.nsplit = nsplit;
  a.shard_len = d.kv_len / d.cp;
  a.split_len = split_len;
  a.scale = d.scale;
  hipError_t e = d.dtype == CPATTN_DT_BF16 ? launch_partial<__bf16>(a, d.head_dim, G, blocks, stream)
                                           : launch_partial<float>(a, d.head_dim, G, blocks, stream);
  if (e != hipSuccess) return CPATTN_E_DEVICE;

  ReduceArgs r;
  r.ws_m = a.ws_m;
  r.ws_den = a.ws_den;
  r.ws_num = a.ws_num;
  r.sp_m = shard_partials->m;
  r.sp_den = shard_partials->den;
  r.sp_num = shard_partials->num;
  r.out = out;
  r.lse = lse;
  r.cp = d.cp;
  r.batch = d.batch;
  r.n_hq = d.n_hq;
  r.nsplit = nsplit;
  const unsigned rb = (unsigned)((int64_t)d.batch * d.n_hq);
  if (d.head_dim == 64) hipLaunchKernelGGL(decode_reduce<64>, dim3(rb), dim3(64), 0, stream, r);
  else if (d.head_dim == 128) hipLaunchKernelGGL(decode_reduce<128>, dim3(rb), dim3(64), 0, stream, r);
  else hipLaunchKernelGGL(decode_reduce<512>, dim3(rb), dim3(64), 0, stream, r);
  if (hipGetLastError() != hipSuccess) return CPATTN_E_DEVICE;
  return CPATTN_OK;
}
