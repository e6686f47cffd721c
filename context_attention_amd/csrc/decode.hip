// Pass-Q decode (G5 context-parallel modelling spec, Definitions table,
// "Pass-Q"; Use case, decode): the query of every batch entry goes to all cp
// shards, each shard computes the partial attention triple over its own keys
// (no mask), and the cp triples are reduced (max, denominator, numerator).
//
// decode_partial<T, D, G>: streams K and V from HBM. A workgroup owns one
//   (shard, batch entry, key split, block of G query heads of one kv head);
//   D/8 lanes share one key row (16 bytes of bf16 each, so a wavefront load
//   covers whole contiguous rows), the G query heads are scored together and
//   reduced with a butterfly over those lanes, and every group of lanes keeps its
//   own online softmax state, merged across lanes and waves once at the end.
//   Groups of up to 8 query heads per kv head run as one block; larger groups
//   (multiples of 8) as several blocks of 8 over the same keys.
// decode_mfma<D>: bf16, groups of 8 or more query heads per kv head (MQA-like
//   layouts among them): the heads of a kv group are the 32 columns of
//   S^T = K Q^T and O^T = V^T P^T on the matrix cores (below).
// decode_reduce<D>: one workgroup per (batch entry, query head): folds the
//   key splits into the per-shard triples (the partial that rank s would send),
//   then reduces the cp shard triples into out and lse.
#include <mutex>

#include "kernels.h"
#include "lds_tiles.h"

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
  int32_t rep;     // query heads per kv head
  int32_t n_blk;   // blocks of G query heads: n_hq / G
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

  // block -> (shard, batch, split, head block) with the head block fastest
  int64_t bid = blockIdx.x;
  const int hb = (int)(bid % a.n_blk) * G;   // first query head of the block
  const int g = hb / a.rep;                  // its kv head
  bid /= a.n_blk;
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
    const T *qp = reinterpret_cast<const T *>(a.q) + ((int64_t)bi * a.n_hq + hb) * D + part * 8;
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
      const int h = hb + gg;
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

// ----------------------------------------------------------------------------
// MFMA kernel (bf16, groups of 8 or more query heads per kv head)
// ----------------------------------------------------------------------------
// A workgroup owns one (shard, batch entry, key split, kv head) and a block of
// 32 of the kv head's query heads, which are the 32 columns of S^T = K Q^T and
// O^T = V^T P^T (v_mfma_f32_32x32x16_bf16); each lane owns one head, so the
// softmax needs one cross-lane exchange per 32-key tile. Heads past the group
// are zero columns that are not stored.
//   head_dim 64 / 128: KG = 8 / 4 waves; wave w streams the split's 32-key tiles
//     w, w + KG, ... through its own ring of NST = 2 LDS buffers (buffer-to-LDS
//     copies of whole rows, one tile in flight while one computes: the HBM
//     latency is covered by bytes in flight, which the LDS bounds, and the KG
//     waves share them out), so the key loop has no barrier; the KG partial
//     triples are merged through LDS at the end.
//   head_dim 512: a quad of waves, each owning a quarter of d and copying only
//     that quarter of every tile (32 + 64 registers of Q and accumulator); the
//     four partial score tiles are exchanged through LDS and summed in one fixed
//     order, so every wave runs the same softmax on identical scores.
// The column blocks of one key range read the same K and V: with the blocks
// walked XCD-major they run side by side on one XCD and share its L2.
template <int D>
struct DecCfg;
template <>
struct DecCfg<64> {
  static constexpr int DS = 1, KG = 8, NST = 2;
};
template <>
struct DecCfg<128> {
  static constexpr int DS = 1, KG = 4, NST = 2;
};
template <>
struct DecCfg<512> {
  static constexpr int DS = 4, KG = 1, NST = 2;
};

// LDS of decode_mfma<D>: per wave NST buffers of a K and a V tile (32 keys x
// D/DS columns), the score exchange of a quad (two buffers), and the merge of
// the KG key groups (aliasing the tiles once the key loop is over).
template <int D>
struct DecLds {
  static constexpr int DS = DecCfg<D>::DS, KG = DecCfg<D>::KG, NST = DecCfg<D>::NST, NW = DS * KG;
  static constexpr int DQ = D / DS;                        // columns of d per wave
  static constexpr int TSZ = 32 * DQ;                      // bf16 elements of one K (or V) tile of a wave
  static constexpr int TILE_BYTES = NW * NST * 2 * TSZ * 2;
  static constexpr int SX_BYTES = DS > 1 ? 2 * DS * 4 * 64 * 16 : 0;
  static constexpr int OXS = D + 4;                        // row stride of the merged numerators (floats)
  static constexpr int MERGE_BYTES = KG > 1 ? KG * 32 * (OXS + 2) * 4 : 0;
  static constexpr int REGION = TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES;
  static constexpr int BYTES = REGION + SX_BYTES;
  static_assert(BYTES <= 160 * 1024, "LDS of one workgroup");
};

struct MfmaArgs {
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
  int32_t rep;        // query heads per kv head
  int32_t ncb;        // head blocks per kv head (32 heads: decode_mfma; 16 NW: decode_mfma16; 128: decode_wide)
  int32_t xcd_major;  // 1: the ncb workgroups of one key range sit 8 apart (one XCD)
  int64_t shard_len;
  int64_t split_len;
  float scale;
};

template <int D>
__global__ __launch_bounds__(64 * DecCfg<D>::DS * DecCfg<D>::KG) void decode_mfma(MfmaArgs a) {
  using L = DecLds<D>;
  constexpr int DS = L::DS, KG = L::KG, NST = L::NST, NW = L::NW, DQ = L::DQ, TSZ = L::TSZ;
  constexpr int KSQ = DQ / 16;   // QK^T k-steps over a wave's columns
  constexpr int DBQ = DQ / 32;   // 32-wide blocks of a wave's output columns
  constexpr int NCH = DQ / 16;   // 1 KB copies per K (or V) tile of a wave
  constexpr int RPK = 512 / DQ;  // key rows per 1 KB copy
  constexpr int KCH = DQ / 8;    // 16-byte chunks per row of a wave's columns
  static_assert((NST - 1) * 2 * NCH <= 63, "copies in flight must fit the vmcnt counter");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int qi = lane & 31;
  const int hf = lane >> 5;
  const int kg = wave / DS, dq = wave % DS;

  // workgroup -> (key range, column block); key range -> (shard, batch, split, kv head)
  int64_t unit;
  int cb;
  {
    const int64_t b = blockIdx.x;
    if (a.xcd_major) {
      const int64_t j = b >> 3;
      unit = (j / a.ncb) * 8 + (b & 7);
      cb = (int)(j % a.ncb);
    } else {
      unit = b / a.ncb;
      cb = (int)(b % a.ncb);
    }
  }
  const int g = (int)(unit % a.n_kv);
  unit /= a.n_kv;
  const int sp = (int)(unit % a.nsplit);
  unit /= a.nsplit;
  const int bi = (int)(unit % a.batch);
  const int s = (int)(unit / a.batch);

  const int64_t k_begin = (int64_t)sp * a.split_len;
  const int64_t k_end = min(a.shard_len, k_begin + a.split_len);
  const int ntile = k_end > k_begin ? (int)((k_end - k_begin + 31) / 32) : 0;
  const int n_my = ntile > kg ? (ntile - kg + KG - 1) / KG : 0;   // tiles of this key group

  const int hc = cb * 32 + qi;      // this lane's head within the kv group
  const bool head_ok = hc < a.rep;
  const int h = g * a.rep + (head_ok ? hc : 0);

  // byte offsets of this lane's 16-byte pieces of a tile (rows of this wave's
  // columns, chunks placed by the swizzles)
  const uint32_t row_bytes = (uint32_t)(a.n_kv * D * 2);
  uint32_t koff[NCH], voff[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int key = i * RPK + lane / KCH;
    const int pc = lane % KCH;
    const uint32_t base = key * row_bytes + (uint32_t)((g * D + dq * DQ) * 2);
    koff[i] = base + (uint32_t)((pc ^ k_swizzle<DQ>(key)) * 16);
    voff[i] = base + (uint32_t)((pc ^ v_swizzle<DQ>(key)) * 16);
  }
  __bf16 *const tiles = reinterpret_cast<__bf16 *>(smem) + wave * NST * 2 * TSZ;   // [buffer][K, V][TSZ]
  const char *kblk = reinterpret_cast<const char *>(a.k[s]);
  const char *vblk = reinterpret_cast<const char *>(a.v[s]);
  const int64_t row0 = (int64_t)bi * a.shard_len;
  // copies of this wave's tile j into buffer `buf`; past the last tile an empty
  // range (zeros, no memory touched), so every iteration issues the same count
  auto issue = [&](int j, int buf) {
    const bool ok = j < n_my;
    const int64_t k0 = k_begin + (int64_t)(kg + j * KG) * 32;
    const int64_t r = ok ? row0 + k0 : 0;
    const int left = ok ? (int)(k_end - k0) : 0;
    const u32x4_t rk = uniform_words(tile_words(kblk, r, left, row_bytes));
    const u32x4_t rv = uniform_words(tile_words(vblk, r, left, row_bytes));
#pragma unroll
    for (int i = 0; i < NCH; ++i) dma_1k(koff[i], rk, tiles + (buf * 2) * TSZ + i * 512);
#pragma unroll
    for (int i = 0; i < NCH; ++i) dma_1k(voff[i], rv, tiles + (buf * 2 + 1) * TSZ + i * 512);
  };

  const float sl2 = a.scale * kLog2e;
  const float thr = kRescaleLog2 / sl2;   // rescale threshold in raw-score units
  float m_ref = kNegInf;                  // reference max of raw scores (this lane's head)
  float l_run = 0.f;                      // this lane's share of the denominator
  f32x16_t oacc[DBQ];
#pragma unroll
  for (int db = 0; db < DBQ; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  f32x4_t(*Sx)[DS][4][64] = reinterpret_cast<f32x4_t(*)[DS][4][64]>(smem + L::REGION);

  // Q fragments (B operand of S^T = K Q^T): lane holds q[h][dq DQ + 16 ks + 8 hf .. +8]
  bf16x8_t qf[KSQ];
  if (n_my > 0) {
#pragma unroll
    for (int t = 0; t < NST - 1; ++t) issue(t, t);
    const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) + ((int64_t)bi * a.n_hq + h) * D + dq * DQ + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks)
      qf[ks] = head_ok ? *reinterpret_cast<const bf16x8_t *>(qp + 16 * ks)
                       : __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
    // Q and the first NST-1 tiles have landed; waiting here also tells the
    // compiler that no load of its own is outstanding inside the loop (it
    // cannot see the copies)
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (int j = 0; j < n_my; ++j) {
      const int cur = j % NST;
      // this wave's reads of tile j-1 have completed before the copies of tile
      // j+NST-1 overwrite its buffer
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      asm volatile("" ::: "memory");
      issue(j + NST - 1, (j + NST - 1) % NST);
      // all but the copies of the NST-1 newer tiles: tile j has landed
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((NST - 1) * 2 * NCH));
      asm volatile("" ::: "memory");
      const __bf16 *Kc = tiles + (cur * 2) * TSZ;
      const __bf16 *Vc = tiles + (cur * 2 + 1) * TSZ;

      f32x16_t sacc;
#pragma unroll
      for (int ks = 0; ks < KSQ; ++ks) {
        const bf16x8_t kf =
            *reinterpret_cast<const bf16x8_t *>(&Kc[qi * DQ + (((2 * ks + hf) ^ k_swizzle<DQ>(qi)) * 8)]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], ks == 0 ? f32x16_t{} : sacc, 0, 0, 0);
      }
      if constexpr (DS > 1) {
        // full scores: the quad's partials summed in one fixed order
        put_scores(Sx[j & 1][dq], sacc);
        __syncthreads();
        sacc = get_scores(Sx[j & 1][0]);
#pragma unroll
        for (int w = 1; w < DS; ++w) sacc += get_scores(Sx[j & 1][w]);
      }
      const int64_t k0 = k_begin + (int64_t)(kg + j * KG) * 32;
      if (k0 + 32 > k_end) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 8 * (r >> 2) + 4 * hf + (r & 3);
          if (k0 + kk >= k_end) sacc[r] = kNegInf;
        }
      }

      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
      mx = max_across_halves(mx);
      if (__any(mx > m_ref + thr)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = (m_new == kNegInf) ? 1.f : exp2_fast((m_ref - m_new) * sl2);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DBQ; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m_ref = m_new;
      }
      const float mref = (m_ref == kNegInf) ? 0.f : m_ref * sl2;
      uint32_t pk[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = exp2_fast(fmaf(sacc[r], sl2, -mref));
        const float p1 = exp2_fast(fmaf(sacc[r + 1], sl2, -mref));
        pk[r >> 1] = pack_bf16x2(p0, p1);
        // denominator from the same rounded values the PV product uses
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[r >> 1]), ones, l_run, false);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4_t pw = {pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
        const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
        for (int db = 0; db < DBQ; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_fragment<DQ>(Vc, ks, db * 32), pf, oacc[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // the trailing empty copies have landed too
  }

  // ---- epilogue: the split's triple of each head (natural-log max)
  const float l_sum = l_run + __shfl_xor(l_run, 32);
  const int64_t hrow = ((int64_t)s * a.batch + bi) * a.n_hq + (int64_t)g * a.rep;   // head 0 of the kv group
  if constexpr (KG == 1) {
    // the DS waves hold identical statistics; each stores its columns
    if (head_ok) {
      const int64_t wi = (hrow + hc) * a.nsplit + sp;
      if (dq == 0 && hf == 0) {
        a.ws_m[wi] = (m_ref == kNegInf) ? kNegInf : m_ref * a.scale;
        a.ws_den[wi] = l_sum;
      }
      float *np = a.ws_num + wi * D + dq * DQ;
#pragma unroll
      for (int db = 0; db < DBQ; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<f32x4_t *>(np + db * 32 + 8 * g4 + 4 * hf) =
              f32x4_t{oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2], oacc[db][4 * g4 + 3]};
    }
  } else {
    // merge the KG key groups through LDS (the tile buffers are free now)
    __syncthreads();
    float *Ox = reinterpret_cast<float *>(smem);   // [KG][32 heads][OXS]
    float *Mx = Ox + KG * 32 * L::OXS;              // [KG][32]
    float *Lx = Mx + KG * 32;                       // [KG][32]
    float *orow = Ox + (kg * 32 + qi) * L::OXS;
#pragma unroll
    for (int db = 0; db < DBQ; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4_t *>(orow + db * 32 + 8 * g4 + 4 * hf) =
            f32x4_t{oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2], oacc[db][4 * g4 + 3]};
    if (hf == 0) {
      Mx[kg * 32 + qi] = m_ref;
      Lx[kg * 32 + qi] = l_sum;
    }
    __syncthreads();
    for (int e = tid; e < 32 * D; e += 64 * NW) {
      const int n = e / D, d = e - n * D;
      if (cb * 32 + n >= a.rep) break;   // e only grows: later elements are past the group too
      float mt = kNegInf;
#pragma unroll
      for (int k = 0; k < KG; ++k) mt = fmaxf(mt, Mx[k * 32 + n]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int k = 0; k < KG; ++k) {
        const float mk = Mx[k * 32 + n];
        const float w = (mk == kNegInf) ? 0.f : exp2_fast((mk - mt) * sl2);
        num += w * Ox[(k * 32 + n) * L::OXS + d];
        den += w * Lx[k * 32 + n];
      }
      const int64_t wi = (hrow + cb * 32 + n) * a.nsplit + sp;
      a.ws_num[wi * D + d] = num;
      if (d == 0) {
        a.ws_m[wi] = (mt == kNegInf) ? kNegInf : mt * a.scale;
        a.ws_den[wi] = den;
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

// ----------------------------------------------------------------------------
// MFMA kernel for many query heads per kv head (bf16, more than 32)
// ----------------------------------------------------------------------------
// A workgroup owns one (shard, batch entry, key split, kv head) and up to 16 NW
// of the kv head's query heads (NW = 8, or 4 at head_dim 512): wave w takes 16 of them, which are the 16
// columns of S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16, each
// over the full head_dim (head_dim 512: 64 registers of Q and 128 of
// accumulator, no exchange between waves). The NW waves share every 32-key K
// and V tile in LDS, copied once per workgroup by all of them together, so each
// key is read from HBM once for all the heads of the workgroup. Lane l holds
// head l % 16; its 16-lane group g = l / 16 holds keys 4 g + {0..3} and
// 16 + 4 g + {0..3} of a tile, in the (group, element) order that the P and V
// operands of the PV product share.
// Keys per LDS stage (TK) and stages (NST). At head_dim 512 a stage takes
// 64 KB, so two fit. Measured on MI355X at 128/1 heads, head_dim 512: 16-key
// stages (five fit; PV on v_mfma_f32_16x16x16_bf16) were 47% slower, and the
// kernel is limited by the matrix work of its single wave per SIMD rather than
// by bytes in flight.
template <int D>
struct Dec16Cfg;
template <>
struct Dec16Cfg<64> {
  static constexpr int TK = 32, NST = 4;
};
template <>
struct Dec16Cfg<128> {
  static constexpr int TK = 32, NST = 4;
};
template <>
struct Dec16Cfg<512> {
  static constexpr int TK = 32, NST = 2;
};


typedef float f32x4v_t __attribute__((ext_vector_type(4)));

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void decode_mfma16(MfmaArgs a) {
  constexpr int NST = Dec16Cfg<D>::NST;
  constexpr int TK = Dec16Cfg<D>::TK;          // keys per tile
  constexpr int TSZ = TK * D;                  // bf16 elements of a K (or V) tile
  constexpr int CH = TSZ * 2 / 1024;           // 1 KB copies per K (or V) tile
  constexpr int CPW = CH >= NW ? CH / NW : 1;  // copies per wave (waves past CH repeat a chunk)
  constexpr int RPK = 512 / D;                 // key rows per 1 KB copy
  constexpr int KCH = D / 8;                   // 16-byte chunks per row
  constexpr int KS = D / 32;                   // QK^T k-steps
  constexpr int DB = D / 16;                   // 16-row blocks of O^T
  static_assert(CH % NW == 0 || NW % CH == 0, "copies split evenly over the waves");
  static_assert((NST - 1) * 2 * CPW <= 63, "copies in flight must fit the vmcnt counter");
  __shared__ __attribute__((aligned(16))) __bf16 Kt[NST][TSZ];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[NST][TSZ];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;     // head of this lane within the wave's 16
  const int grp = lane >> 4;     // 16-lane group

  int64_t unit;
  int hs;
  {
    const int64_t b = blockIdx.x;
    if (a.xcd_major) {
      const int64_t j = b >> 3;
      unit = (j / a.ncb) * 8 + (b & 7);
      hs = (int)(j % a.ncb);
    } else {
      unit = b / a.ncb;
      hs = (int)(b % a.ncb);
    }
  }
  const int g = (int)(unit % a.n_kv);
  unit /= a.n_kv;
  const int sp = (int)(unit % a.nsplit);
  unit /= a.nsplit;
  const int bi = (int)(unit % a.batch);
  const int s = (int)(unit / a.batch);

  const int64_t k_begin = (int64_t)sp * a.split_len;
  const int64_t k_end = min(a.shard_len, k_begin + a.split_len);
  const int ntile = k_end > k_begin ? (int)((k_end - k_begin + TK - 1) / TK) : 0;

  const int hb0 = (hs * NW + wave) * 16;     // first head of this wave within the kv group
  const bool wave_on = hb0 < a.rep;           // the wave has heads (uniform)
  const int hc = hb0 + col;
  const bool head_ok = hc < a.rep;
  const int h = g * a.rep + (head_ok ? hc : 0);

  // copy offsets: chunk q of a tile holds key rows q RPK .. q RPK + RPK - 1
  const uint32_t row_bytes = (uint32_t)(a.n_kv * D * 2);
  uint32_t koff[CPW], voff[CPW];
  int kq[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int q = (wave * CPW + i) % CH;
    kq[i] = q;
    const int key = q * RPK + lane / KCH;
    const int pc = lane % KCH;
    const uint32_t base = key * row_bytes + (uint32_t)(g * D * 2);
    koff[i] = base + (uint32_t)((pc ^ k_swizzle<D>(key)) * 16);
    voff[i] = base + (uint32_t)((pc ^ v16_swizzle<D>(key)) * 16);
  }
  static_assert(CH * RPK == TK, "the copies of a tile cover its key rows");
  const char *kblk = reinterpret_cast<const char *>(a.k[s]);
  const char *vblk = reinterpret_cast<const char *>(a.v[s]);
  const int64_t row0 = (int64_t)bi * a.shard_len;
  auto issue = [&](int j, int buf) {
    const bool ok = j < ntile;
    const int64_t k0 = k_begin + (int64_t)j * TK;
    const int64_t r = ok ? row0 + k0 : 0;
    const int left = ok ? (int)(k_end - k0) : 0;
    const u32x4_t rk = uniform_words(tile_words(kblk, r, left, row_bytes));
    const u32x4_t rv = uniform_words(tile_words(vblk, r, left, row_bytes));
#pragma unroll
    for (int i = 0; i < CPW; ++i) dma_1k(koff[i], rk, &Kt[buf][kq[i] * 512]);
#pragma unroll
    for (int i = 0; i < CPW; ++i) dma_1k(voff[i], rv, &Vt[buf][kq[i] * 512]);
  };

  const float sl2 = a.scale * kLog2e;
  const float thr = kRescaleLog2 / sl2;
  float m_ref = kNegInf, l_run = 0.f;
  f32x4v_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4v_t{0.f, 0.f, 0.f, 0.f};
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Q fragments (B operand of S^T = K Q^T): lane holds q[h][32 ks + 8 grp .. +8]
  bf16x8_t qf[KS];
  if (ntile > 0) {
#pragma unroll
    for (int t = 0; t < NST - 1; ++t) issue(t, t);
    const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) + ((int64_t)bi * a.n_hq + h) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = head_ok ? *reinterpret_cast<const bf16x8_t *>(qp + 32 * ks)
                       : __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (int j = 0; j < ntile; ++j) {
      const int cur = j % NST;
      // this wave's copies of tile j have landed (those of the NST-2 newer tiles
      // may still fly); after the barrier every wave's have, and every wave is
      // done with the buffer that tile j+NST-1 goes into (tile j-1's)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((NST - 2) * 2 * CPW));
      __syncthreads();
      issue(j + NST - 1, (j + NST - 1) % NST);
      if (!wave_on) continue;
      const __bf16 *Kc = Kt[cur];
      f32x4v_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = 4 * ks + grp;
        const int r0 = col, r1 = 16 + col;
        const bf16x8_t k0f = *reinterpret_cast<const bf16x8_t *>(&Kc[r0 * D + ((ch ^ k_swizzle<D>(r0)) * 8)]);
        const bf16x8_t k1f = *reinterpret_cast<const bf16x8_t *>(&Kc[r1 * D + ((ch ^ k_swizzle<D>(r1)) * 8)]);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0f, qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1f, qf[ks], s1, 0, 0, 0);
      }
      const int64_t k0 = k_begin + (int64_t)j * TK;
      if (k0 + 32 > k_end) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (k0 + 4 * grp + t >= k_end) s0[t] = kNegInf;
          if (k0 + 16 + 4 * grp + t >= k_end) s1[t] = kNegInf;
        }
      }
      float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])), fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = max_across_halves(mx);
      if (__any(mx > m_ref + thr)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = (m_new == kNegInf) ? 1.f : exp2_fast((m_ref - m_new) * sl2);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        m_ref = m_new;
      }
      const float mref = (m_ref == kNegInf) ? 0.f : m_ref * sl2;
      uint32_t pk[4];
      pk[0] = pack_bf16x2(exp2_fast(fmaf(s0[0], sl2, -mref)), exp2_fast(fmaf(s0[1], sl2, -mref)));
      pk[1] = pack_bf16x2(exp2_fast(fmaf(s0[2], sl2, -mref)), exp2_fast(fmaf(s0[3], sl2, -mref)));
      pk[2] = pack_bf16x2(exp2_fast(fmaf(s1[0], sl2, -mref)), exp2_fast(fmaf(s1[1], sl2, -mref)));
      pk[3] = pack_bf16x2(exp2_fast(fmaf(s1[2], sl2, -mref)), exp2_fast(fmaf(s1[3], sl2, -mref)));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[i]), ones, l_run, false);
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
      // V^T operand: lane (d row = col, group) needs V[4 grp + 0..3][16 db + col]
      // and V[16 + 4 grp + 0..3][16 db + col]: two transposed reads
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#if defined(__HIP_DEVICE_COMPILE__)
        const int row = 4 * grp + (col >> 2);
        const int cc = 16 * db + 4 * (col & 3);
        const int off = row * D + 8 * ((cc >> 3) ^ v16_swizzle<D>(row)) + (cc & 7);   // rows +16 share the swizzle
        typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
        const lds_i16x4 *vp = (const lds_i16x4 *)(Vt[cur] + off);
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)vp);
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vp + 4 * D));
        const i16x4_t both[2] = {lo, hi};
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, both);
#else
        const bf16x8_t vf = {};
#endif
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[db], 0, 0, 0);
      }
        }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // the trailing empty copies have landed
  }

  // ---- epilogue: the split's triple of each head (natural-log max)
  float l_sum = l_run + __shfl_xor(l_run, 16);
  l_sum += __shfl_xor(l_sum, 32);
  if (head_ok) {
    const int64_t wi = ((((int64_t)s * a.batch + bi) * a.n_hq + (int64_t)g * a.rep) + hc) * a.nsplit + sp;
    if (grp == 0) {
      a.ws_m[wi] = (m_ref == kNegInf) ? kNegInf : m_ref * a.scale;
      a.ws_den[wi] = l_sum;
    }
    float *np = a.ws_num + wi * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4v_t *>(np + 16 * db) = oacc[db];
  }
}

// ----------------------------------------------------------------------------
// head_dim 512 with more than 112 query heads per kv head (MLA-like layouts)
// ----------------------------------------------------------------------------
// The ring step's head_dim 512 loop over a key split: a workgroup of 8 waves
// (two per SIMD) owns one (shard, batch entry, key split, kv head) and a block
// of 128 of the kv head's query heads; wave w takes 16 of them as the columns
// of v_mfma_f32_16x16x32_bf16 in S^T = K Q^T and O^T = V^T P^T over the whole
// head_dim (64 registers of Q, 128 of accumulator). The 32-key K and V tiles
// (32 KB each) are copied once per workgroup into double-buffered LDS, each
// 1 KB key row through a copy resource of its own (RowWalk over the split as a
// single key segment), and the copies of tile t+1 are spread over the QK^T
// k-steps of tile t. Heads past the kv group are zero columns, not stored.
constexpr int kWideWaves = 8;
constexpr int kWideHeads = 16 * kWideWaves;   // query heads of one workgroup

// What workgroup b of decode_wide owns: shard s, batch entry bi, key split sp
// ([k_begin, k_end) of the shard's keys), kv head g and head block hs.
struct WideBlock {
  int s, bi, sp, g, hs;
  int64_t k_begin, k_end;
};

__host__ __device__ __forceinline__ WideBlock wide_block(const MfmaArgs &a, int64_t b) {
  WideBlock w;
  int64_t unit;
  if (a.xcd_major) {
    const int64_t j = b >> 3;
    unit = (j / a.ncb) * 8 + (b & 7);
    w.hs = (int)(j % a.ncb);
  } else {
    unit = b / a.ncb;
    w.hs = (int)(b % a.ncb);
  }
  w.g = (int)(unit % a.n_kv);
  unit /= a.n_kv;
  w.sp = (int)(unit % a.nsplit);
  unit /= a.nsplit;
  w.bi = (int)(unit % a.batch);
  w.s = (int)(unit / a.batch);
  w.k_begin = (int64_t)w.sp * a.split_len;
  w.k_end = a.shard_len < w.k_begin + a.split_len ? a.shard_len : w.k_begin + a.split_len;
  return w;
}

// The key split as one key segment of the shard's rows of batch entry bi (the
// shard holds batch entries one after the other, shard_len rows each).
template <int BN>
__host__ __device__ __forceinline__ Segs<BN> split_segs(int bi, int64_t shard_len, int64_t k_begin, int nkeys) {
  Segs<BN> sg;
  sg.nseg = nkeys > 0 ? 1 : 0;
  sg.n0 = (nkeys + BN - 1) / BN;
  sg.row[0] = (int64_t)bi * shard_len + k_begin;
  sg.row[1] = 0;
  sg.end[0] = nkeys;
  sg.end[1] = 0;
  sg.diag[0] = false;
  sg.diag[1] = false;
  return sg;
}

__global__ __launch_bounds__(64 * kWideWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_wide(MfmaArgs a) {
  constexpr int D = 512;
  constexpr int BN = 32;                        // keys per tile
  constexpr int NW = kWideWaves;
  constexpr int KS = D / 32;                    // QK^T k-steps
  constexpr int DB = D / 16;                    // 16-column blocks of O^T
  constexpr int TSZ = BN * D;                   // bf16 elements of a K (or V) tile
  constexpr int CPW = BN / NW;                  // key rows each wave copies per tile
  static_assert(NW == 8 && CPW % 2 == 0, "the copy offsets assume 8 waves");

  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][TSZ];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[2][TSZ];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;     // head of this lane within the wave's 16
  const int grp = lane >> 4;     // 16-lane group

  const WideBlock wb = wide_block(a, blockIdx.x);
  const int s = wb.s, bi = wb.bi, sp = wb.sp, g = wb.g;
  const int nkeys = wb.k_end > wb.k_begin ? (int)(wb.k_end - wb.k_begin) : 0;
  const int ntiles = (nkeys + BN - 1) / BN;

  const int hc = wb.hs * kWideHeads + wave * 16 + col;   // head of this lane within the kv group
  const bool head_ok = hc < a.rep;
  const int h = g * a.rep + (head_ok ? hc : 0);
  const Segs<BN> sg = split_segs<BN>(bi, a.shard_len, wb.k_begin, nkeys);

  const char *kblock = reinterpret_cast<const char *>(a.k[s]);
  const char *vblock = reinterpret_cast<const char *>(a.v[s]);
  const uint32_t row_bytes = (uint32_t)(a.n_kv * D * 2);
  // copy offsets: key row q = w + 8 i of a tile, swizzled chunk L ^ swizzle(q)
  // (the ring step's head_dim 512 copies)
  const int wv = wave;
  const uint32_t koff0 = (uint32_t)((lane ^ k_swizzle<D>(wv)) * 16);
  const uint32_t koff1 = (uint32_t)((lane ^ k_swizzle<D>(wv + 8)) * 16);
  const uint32_t voff = (uint32_t)((lane ^ v16_swizzle<D>(wv)) * 16);
  const uint32_t gbase = (uint32_t)(g * D * 2);
  // LDS read addresses: base registers plus immediates (the ring step's layout)
  const __bf16 *kp[4];
  const __bf16 *vp[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) kp[j] = &Ks[0][col * D + 8 * (4 * (j ^ (col >> 2)) + (grp ^ (col & 3)))];
  {
    const int vrow = 4 * grp + (col >> 2);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      vp[j] = &Vt[0][vrow * D + 16 * (j ^ (vrow & 7)) + 8 * ((col >> 1) & 1) + 4 * (col & 1)];
  }

  const float sl2 = a.scale * kLog2e;
  const float thr = kRescaleLog2 / sl2;
  float m_ref = kNegInf, l_run = 0.f;
  f32x4_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (ntiles > 0) {
    RowWalk<BN> kw(sg, ntiles, kblock, 0, row_bytes), vw(sg, ntiles, vblock, 0, row_bytes);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int q = wv + NW * i;
      dma_1k((i & 1) ? koff1 : koff0, uniform_words(kw.row(q, row_bytes, gbase)), Ks[0] + q * 512);
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int q = wv + NW * i;
      dma_1k(voff, uniform_words(vw.row(q, row_bytes, gbase)), Vt[0] + q * 512);
    }
    kw.next();
    vw.next();

    // Q fragments (B operand of S^T = K Q^T): lane holds q[h][32 ks + 8 grp .. +8]
    bf16x8_t qf[KS];
    {
      const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) + ((int64_t)bi * a.n_hq + h) * D + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[ks] = head_ok ? *reinterpret_cast<const bf16x8_t *>(qp + 32 * ks)
                         : __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
    }
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

    auto tile_step = [&](int it, const int cur) {
      // this wave's copies of tile it have landed; after the barrier every
      // wave's have, and every wave is done with tile it-1, whose buffer the
      // copies of tile it+1 overwrite
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      const int k0 = it * BN;

      f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      auto kread = [&](int ks, int blk) {
        return *reinterpret_cast<const bf16x8_t *>(kp[ks & 3] + cur * TSZ + 128 * (ks >> 2) + blk * 16 * D);
      };
      bf16x8_t ka = kread(0, 0), kb = kread(0, 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8_t na = ka, nb = kb;
        if (ks + 1 < KS) {
          na = kread(ks + 1, 0);
          nb = kread(ks + 1, 1);
        }
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qf[ks], s1, 0, 0, 0);
        if ((ks & 1) == 0) {
          const int i = ks >> 1;   // copy i of tile it+1: K rows for i < CPW, then V rows
          const int q = wv + NW * (i % CPW);
          if (i < CPW)
            dma_1k((i & 1) ? koff1 : koff0, uniform_words(kw.row(q, row_bytes, gbase)), Ks[cur ^ 1] + q * 512);
          else
            dma_1k(voff, uniform_words(vw.row(q, row_bytes, gbase)), Vt[cur ^ 1] + q * 512);
        }
        ka = na;
        kb = nb;
      }
      kw.next();
      vw.next();
      if (k0 + BN > nkeys) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (k0 + 4 * grp + t >= nkeys) s0[t] = kNegInf;
          if (k0 + 16 + 4 * grp + t >= nkeys) s1[t] = kNegInf;
        }
      }

      // online softmax: the head's 32 keys lie in the 4 lanes col, col + 16, ...
      float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])), fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
      mx = max_across_rows16(mx);
      mx = max_across_halves(mx);
      if (__any(mx > m_ref + thr)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = (m_new == kNegInf) ? 1.f : exp2_fast((m_ref - m_new) * sl2);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        m_ref = m_new;
      }
      const float mref = (m_ref == kNegInf) ? 0.f : m_ref * sl2;
      uint32_t pk[4];
      pk[0] = pack_bf16x2(exp2_fast(fmaf(s0[0], sl2, -mref)), exp2_fast(fmaf(s0[1], sl2, -mref)));
      pk[1] = pack_bf16x2(exp2_fast(fmaf(s0[2], sl2, -mref)), exp2_fast(fmaf(s0[3], sl2, -mref)));
      pk[2] = pack_bf16x2(exp2_fast(fmaf(s1[0], sl2, -mref)), exp2_fast(fmaf(s1[1], sl2, -mref)));
      pk[3] = pack_bf16x2(exp2_fast(fmaf(s1[2], sl2, -mref)), exp2_fast(fmaf(s1[3], sl2, -mref)));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[i]), ones, l_run, false);
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});

      // O^T += V^T P^T, the next block's transposed reads ahead of this block's product
      auto vread = [&](int db) { return v16_read<D>(vp[db & 7] + cur * TSZ + 128 * (db >> 3)); };
      bf16x8_t vf = vread(0);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8_t nv = db + 1 < DB ? vread(db + 1) : vf;
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[db], 0, 0, 0);
        vf = nv;
      }
    };
    for (int it = 0; it < ntiles; it += 2) {
      tile_step(it, 0);
      if (it + 1 < ntiles) tile_step(it + 1, 1);
    }
    // the copies issued past the last tile (empty ranges: zeros, no memory
    // read) land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }

  // ---- epilogue: the split's triple of each head (natural-log max); the 4
  // groups hold disjoint keys, so their denominators add up
  float l_sum = l_run + __shfl_xor(l_run, 16);
  l_sum += __shfl_xor(l_sum, 32);
  if (head_ok) {
    const int64_t wi = ((((int64_t)s * a.batch + bi) * a.n_hq + (int64_t)g * a.rep) + hc) * a.nsplit + sp;
    if (grp == 0) {
      a.ws_m[wi] = (m_ref == kNegInf) ? kNegInf : m_ref * a.scale;
      a.ws_den[wi] = l_sum;
    }
    float *np = a.ws_num + wi * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4_t *>(np + 16 * db) = oacc[db];
  }
}

// Wave-wide max and sum (butterfly over the 64 lanes).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

constexpr int kRedWaves = 8;   // waves of a reduce workgroup (shards handled side by side)

// One workgroup per (batch entry, query head). Wave w folds the key splits of
// shards w, w + 8, ... into the shard triples (written out: the partial rank s
// would send) and merges them; the waves' results are then merged through LDS.
// A shard's splits are folded at once: the lanes take the splits' maxima and
// denominators, the shard max and the split weights follow from two wave
// reductions, and the numerator is the weighted sum over splits, whose loads
// are independent of each other.
template <int D>
__global__ __launch_bounds__(64 * kRedWaves) void decode_reduce(ReduceArgs a) {
  constexpr int PER = D / 64;
  __shared__ float r_m[kRedWaves], r_l[kRedWaves];
  __shared__ float r_n[kRedWaves][D];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int64_t item = blockIdx.x;   // bi * n_hq + h
  float tm = kNegInf, tl = 0.f, tacc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) tacc[e] = 0.f;
  for (int s = wave; s < a.cp; s += nw) {
    const int64_t srow = (int64_t)s * a.batch * a.n_hq + item;   // shard-major row
    const int64_t w0 = srow * a.nsplit;
    float sm = kNegInf;
    for (int c = lane; c < a.nsplit; c += 64) sm = fmaxf(sm, a.ws_m[w0 + c]);
    sm = wave_max(sm);
    float sl = 0.f, sacc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) sacc[e] = 0.f;
    for (int c0 = 0; c0 < a.nsplit; c0 += 64) {
      const int c = c0 + lane;
      float wgt = 0.f, dl = 0.f;
      if (c < a.nsplit) {
        const float mc = a.ws_m[w0 + c];
        wgt = (mc == kNegInf) ? 0.f : expf(mc - sm);
        dl = wgt * a.ws_den[w0 + c];
      }
      sl += wave_sum(dl);
      const int nc = min(64, a.nsplit - c0);
      const float *np = a.ws_num + (w0 + c0) * D + lane * PER;
      // eight splits per round: their loads are issued before any is used
      int i = 0;
      for (; i + 8 <= nc; i += 8) {
        float x[8][PER];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int e = 0; e < PER; ++e) x[u][e] = np[(int64_t)(i + u) * D + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wi = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wgt), i + u));
#pragma unroll
          for (int e = 0; e < PER; ++e) sacc[e] = fmaf(wi, x[u][e], sacc[e]);
        }
      }
      for (; i < nc; ++i) {
        const float wi = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wgt), i));
#pragma unroll
        for (int e = 0; e < PER; ++e) sacc[e] = fmaf(wi, np[(int64_t)i * D + e], sacc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) a.sp_num[srow * D + lane * PER + e] = sacc[e];
    if (lane == 0) {
      a.sp_m[srow] = sm;
      a.sp_den[srow] = sl;
    }
    float mn, w0t, w1t;
    merge_weights(tm, sm, mn, w0t, w1t);
    tl = w0t * tl + w1t * sl;
#pragma unroll
    for (int e = 0; e < PER; ++e) tacc[e] = w0t * tacc[e] + w1t * sacc[e];
    tm = mn;
  }
  if (lane == 0) {
    r_m[wave] = tm;
    r_l[wave] = tl;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) r_n[wave][lane * PER + e] = tacc[e];
  __syncthreads();
  if (wave != 0) return;
  float fm = kNegInf;
  for (int w = 0; w < nw; ++w) fm = fmaxf(fm, r_m[w]);
  float fl = 0.f, facc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) facc[e] = 0.f;
  for (int w = 0; w < nw; ++w) {
    const float wt = (r_m[w] == kNegInf) ? 0.f : expf(r_m[w] - fm);
    fl += wt * r_l[w];
#pragma unroll
    for (int e = 0; e < PER; ++e) facc[e] += wt * r_n[w][lane * PER + e];
  }
  const float inv = fl > 0.f ? 1.f / fl : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) a.out[item * D + lane * PER + e] = facc[e] * inv;
  if (lane == 0) a.lse[item] = fl > 0.f ? fm + logf(fl) : kNegInf;
}

// Split geometry: about `target` workgroups over the `groups` (shard, batch
// entry, head block) triples, split lengths that are whole rounds of `step`
// keys, and no more splits than a quarter of the shard's rounds (so a shard
// that is split at all gets at least 3 rounds per split).
void plan_splits(int64_t shard_len, int64_t step, int64_t groups, int64_t target, int32_t &nsplit,
                 int64_t &split_len) {
  int64_t want = (target + groups - 1) / groups;
  int64_t max_by_len = (shard_len + 4 * step - 1) / (4 * step);
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

// The partial kernel a description runs on and its split geometry.
struct DecodePlan {
  bool mfma;       // decode_mfma (else decode_partial)
  bool mfma16;     // decode_mfma16 (takes precedence over decode_mfma)
  bool wide;       // decode_wide (takes precedence over both)
  int G;           // query heads per kv head
  int gv;          // decode_partial: query heads per block
  int ncb;         // decode_mfma: 32-head column blocks per kv head; decode_mfma16: head blocks of 16 NW
  int nw;          // decode_mfma16: waves per workgroup
  int32_t nsplit;
  int64_t split_len;
};

int kg_of(int d) { return d == 64 ? DecCfg<64>::KG : d == 128 ? DecCfg<128>::KG : DecCfg<512>::KG; }

DecodePlan plan_decode(const cpattn_decode_desc &d) {
  DecodePlan p;
  p.G = d.n_hq / d.n_kv;
  // measured on MI355X: at 8 heads per kv head the vector kernel is ALU-bound
  // (3.6 TB/s on 32/4 heads against 5.7 for decode_mfma); at 4 it streams faster
  p.mfma = d.dtype == CPATTN_DT_BF16 && p.G >= 8;
  // more than 32 heads per kv head: one workgroup serves up to 128 of them from
  // one copy of each K and V tile
  p.mfma16 = d.dtype == CPATTN_DT_BF16 && p.G > 32;
  // head_dim 512 with at least 8 blocks of 16 heads: 8 waves of the ring step's
  // head_dim 512 loop, 128 heads per workgroup
  p.wide = p.mfma16 && d.head_dim == 512 && (p.G + 15) / 16 >= kWideWaves;
  p.gv = p.G <= 8 ? p.G : 8;
  p.ncb = (p.G + 31) / 32;
  p.nw = 0;
  const int64_t shard_len = d.kv_len / d.cp;
  // about 512 workgroups for the two matrix-core kernels: measured on MI355X,
  // 2-4% faster than 2048 on the single-kv-head layouts (a workgroup's prologue
  // and final merge are paid once per split) and level on GQA 32/4
  if (p.wide) {
    p.nw = kWideWaves;
    p.ncb = (p.G + kWideHeads - 1) / kWideHeads;
    const int64_t groups = (int64_t)d.cp * d.batch * d.n_kv * p.ncb;
    plan_splits(shard_len, 32, groups, 512, p.nsplit, p.split_len);
  } else if (p.mfma16) {
    const int blk16 = (p.G + 15) / 16;
    // head_dim 512 keeps 4 waves (one per SIMD): 8 would not fit their Q and
    // accumulators in the registers of two waves per SIMD
    p.nw = (blk16 >= 8 && d.head_dim != 512) ? 8 : 4;
    p.ncb = (blk16 + p.nw - 1) / p.nw;
    const int64_t groups = (int64_t)d.cp * d.batch * d.n_kv * p.ncb;
    plan_splits(shard_len, 32, groups, 512, p.nsplit, p.split_len);
  } else if (p.mfma) {
    const int64_t groups = (int64_t)d.cp * d.batch * d.n_kv * p.ncb;
    plan_splits(shard_len, 32LL * kg_of(d.head_dim), groups, 512, p.nsplit, p.split_len);
  } else {
    const int64_t step = (int64_t)(64 / (d.head_dim / 8)) * kDecWaves * kUnroll;
    const int64_t groups = (int64_t)d.cp * d.batch * (d.n_hq / p.gv);
    // about 8192 workgroups for the vector kernel (measured on MI355X: +2% on
    // GQA 32/8 d128 over 4096, level at batch 2, slower at 16384 and beyond)
    plan_splits(shard_len, step, groups, 8192, p.nsplit, p.split_len);
  }
  return p;
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

hipError_t launch_mfma16(const MfmaArgs &a, int D, int nw, int64_t blocks, hipStream_t s) {
  const dim3 grid((unsigned)blocks), block(64 * nw);
  if (D == 64) {
    if (nw == 8) hipLaunchKernelGGL((decode_mfma16<64, 8>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_mfma16<64, 4>), grid, block, 0, s, a);
  } else if (D == 128) {
    if (nw == 8) hipLaunchKernelGGL((decode_mfma16<128, 8>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_mfma16<128, 4>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((decode_mfma16<512, 4>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_mfma(const MfmaArgs &a, int D, int64_t blocks, hipStream_t s) {
  if (D == 64)
    hipLaunchKernelGGL(decode_mfma<64>, dim3((unsigned)blocks), dim3(64 * DecCfg<64>::DS * DecCfg<64>::KG), 0, s, a);
  else if (D == 128)
    hipLaunchKernelGGL(decode_mfma<128>, dim3((unsigned)blocks), dim3(64 * DecCfg<128>::DS * DecCfg<128>::KG), 0, s,
                       a);
  else
    hipLaunchKernelGGL(decode_mfma<512>, dim3((unsigned)blocks), dim3(64 * DecCfg<512>::DS * DecCfg<512>::KG), 0, s,
                       a);
  return hipGetLastError();
}

// Arguments of the matrix-core partial kernels for a description and its plan.
MfmaArgs mfma_args(const cpattn_decode_desc &d, const DecodePlan &p, const void *q, const void *const *k_shards,
                   const void *const *v_shards, float *ws_m, float *ws_den, float *ws_num) {
  MfmaArgs a;
  a.q = q;
  for (int s = 0; s < d.cp; ++s) {
    a.k[s] = k_shards[s];
    a.v[s] = v_shards[s];
  }
  a.ws_m = ws_m;
  a.ws_den = ws_den;
  a.ws_num = ws_num;
  a.batch = d.batch;
  a.n_hq = d.n_hq;
  a.n_kv = d.n_kv;
  a.nsplit = p.nsplit;
  a.rep = d.n_hq / d.n_kv;
  a.ncb = p.ncb;
  const int64_t units = (int64_t)d.cp * d.batch * p.nsplit;
  a.xcd_major = (p.ncb > 1 && (units * d.n_kv) % 8 == 0) ? 1 : 0;
  a.shard_len = d.kv_len / d.cp;
  a.split_len = p.split_len;
  a.scale = d.scale;
  return a;
}

// The pass-Q decode of cpattn_passq_decode with the workspace given (ws ==
// nullptr: only the size is stored).
int passq_decode(const cpattn_decode_desc *desc, const void *q, const void *const *k_shards,
                 const void *const *v_shards, const cpattn_partial *shard_partials, float *out, float *lse, void *ws,
                 size_t *ws_bytes, hipStream_t stream) {
  if (desc == nullptr || ws_bytes == nullptr) return CPATTN_E_ARG;
  const cpattn_decode_desc d = *desc;
  if (d.cp < 1 || d.batch < 0 || d.kv_len < 0 || d.n_hq < 1 || d.n_kv < 1) return CPATTN_E_ARG;
  if (d.dtype != CPATTN_DT_F32 && d.dtype != CPATTN_DT_BF16) return CPATTN_E_ARG;
  if (!(d.scale > 0.f) || !(d.scale < __builtin_huge_valf())) return CPATTN_E_ARG;
  if (d.n_hq % d.n_kv != 0) return CPATTN_E_DIVISIBILITY;
  if (d.kv_len % d.cp != 0) return CPATTN_E_DIVISIBILITY;
  if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 512) return CPATTN_E_UNSUPPORTED;
  const int G = d.n_hq / d.n_kv;
  if (!(G == 1 || G == 2 || G == 4 || G % 8 == 0)) return CPATTN_E_UNSUPPORTED;
  if (d.cp > kMaxShards) return CPATTN_E_UNSUPPORTED;
  // a tile's key rows lie within the 2^31-byte range of one copy resource
  if ((int64_t)d.n_kv * d.head_dim * 2 * 64 > 0x7FFFFFFFLL) return CPATTN_E_UNSUPPORTED;

  const DecodePlan p = plan_decode(d);
  const int32_t nsplit = p.nsplit;
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
  const int64_t units = (int64_t)d.cp * d.batch * nsplit;
  const int64_t blocks = (p.mfma || p.mfma16) ? units * d.n_kv * p.ncb : units * (d.n_hq / p.gv);
  if (blocks > 0x7FFFFFFFLL || (int64_t)d.batch * d.n_hq > 0x7FFFFFFFLL) return CPATTN_E_UNSUPPORTED;
  if (p.split_len > 0x7FFFFFFFLL) return CPATTN_E_UNSUPPORTED;

  float *wsf = reinterpret_cast<float *>(ws);
  float *ws_m = wsf, *ws_den = wsf + triples, *ws_num = wsf + 2 * triples;
  hipError_t e;
  if (p.mfma || p.mfma16) {
    const MfmaArgs a = mfma_args(d, p, q, k_shards, v_shards, ws_m, ws_den, ws_num);
    if (p.wide) {
      hipLaunchKernelGGL(decode_wide, dim3((unsigned)blocks), dim3(64 * kWideWaves), 0, stream, a);
      e = hipGetLastError();
    } else {
      e = p.mfma16 ? launch_mfma16(a, d.head_dim, p.nw, blocks, stream) : launch_mfma(a, d.head_dim, blocks, stream);
    }
  } else {
    DecodeArgs a;
    a.q = q;
    for (int s = 0; s < d.cp; ++s) {
      a.k[s] = k_shards[s];
      a.v[s] = v_shards[s];
    }
    a.ws_m = ws_m;
    a.ws_den = ws_den;
    a.ws_num = ws_num;
    a.batch = d.batch;
    a.n_hq = d.n_hq;
    a.n_kv = d.n_kv;
    a.nsplit = nsplit;
    a.rep = G;
    a.n_blk = d.n_hq / p.gv;
    a.shard_len = d.kv_len / d.cp;
    a.split_len = p.split_len;
    a.scale = d.scale;
    e = d.dtype == CPATTN_DT_BF16 ? launch_partial<__bf16>(a, d.head_dim, p.gv, blocks, stream)
                                  : launch_partial<float>(a, d.head_dim, p.gv, blocks, stream);
  }
  if (e != hipSuccess) return CPATTN_E_DEVICE;

  ReduceArgs r;
  r.ws_m = ws_m;
  r.ws_den = ws_den;
  r.ws_num = ws_num;
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
  const dim3 rt(64 * (d.cp < kRedWaves ? d.cp : kRedWaves));
  if (d.head_dim == 64) hipLaunchKernelGGL(decode_reduce<64>, dim3(rb), rt, 0, stream, r);
  else if (d.head_dim == 128) hipLaunchKernelGGL(decode_reduce<128>, dim3(rb), rt, 0, stream, r);
  else hipLaunchKernelGGL(decode_reduce<512>, dim3(rb), rt, 0, stream, r);
  if (hipGetLastError() != hipSuccess) return CPATTN_E_DEVICE;
  return CPATTN_OK;
}

}  // namespace
}  // namespace cpattn

extern "C" int cpattn_passq_decode(const cpattn_decode_desc *desc, const void *q, const void *const *k_shards,
                                   const void *const *v_shards, const cpattn_partial *shard_partials, float *out,
                                   float *lse, void *ws, size_t *ws_bytes, hipStream_t stream) {
  return cpattn::passq_decode(desc, q, k_shards, v_shards, shard_partials, out, lse, ws, ws_bytes, stream);
}

// ----------------------------------------------------------------------------
// Pass-Q decode without allocation: the split triples live in a file-scope
// device array instead of a caller's workspace. Each GPU holds its own copy of
// the array from the module's load until the process ends; host code reaches it
// only through the address hipGetSymbolAddress returns for the current device
// (the array's name is a host-side stand-in, not a device address).
// ----------------------------------------------------------------------------

static __device__ __align__(256) unsigned char scratch[CPATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device; nullptr when the runtime cannot give it.
void *scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int cpattn_passq_decode_noalloc(const cpattn_decode_desc *desc, const void *q,
                                           const void *const *k_shards, const void *const *v_shards,
                                           const cpattn_partial *shard_partials, float *out, float *lse,
                                           hipStream_t stream) {
  // the split triples need no clearing: every (shard, batch entry, head, split)
  // triple is written by the partial kernel before the reduction reads it
  size_t need = 0;
  const int rc = cpattn::passq_decode(desc, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, &need,
                                      stream);
  if (rc != CPATTN_OK) return rc;
  if (need > (size_t)CPATTN_NOALLOC_SCRATCH_BYTES) return CPATTN_E_WORKSPACE;
  void *ws = scratch_address();
  if (ws == nullptr) return CPATTN_E_DEVICE;
  size_t have = (size_t)CPATTN_NOALLOC_SCRATCH_BYTES;
  return cpattn::passq_decode(desc, q, k_shards, v_shards, shard_partials, out, lse, ws, &have, stream);
}
