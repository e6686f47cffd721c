// Pass-KV ring step: causal partial attention of one rank's rows over the KV
// block of the rank (rank - step) mod cp, carrying the online-softmax triple
// (G5 context-parallel modelling spec, Definitions table: "Pass-KV", "Ring
// step", "Partial attention", "Balanced chunk split").
//
// Work geometry. Under the balanced split rank r holds chunk a_h = r (head) and
// a_t = 2cp-1-r (tail) of every sequence; the block of rank j holds key chunks
// b_h = j and b_t = 2cp-1-j. A (query chunk a, key chunk b) pair of the same
// sequence is fully visible when b < a, a causal triangle when b == a (only at
// step 0) and empty when b > a. The kernels below walk, for their query rows,
// only the key chunks that are not empty, and mask only the triangle and the
// ragged end of a chunk. In the padded layout (lengths rounded up to a multiple
// of 2cp) a chunk's real tokens are its first min(c, L - chunk c) slots: key
// segments stop there and rows past it get the merge identity.
//
// Kernels
//   ring_step_mfma<D, HG>  bf16, head_dim 64/128: a workgroup of 8 waves (two per
//       SIMD) owns 32*8/HG query rows x HG query heads of one kv group; K and V
//       tiles of 64 keys are copied straight from HBM into double-buffered LDS
//       (the next tiles' copies are in flight while the current one computes,
//       issued between the k-steps of a QK^T, their buffer resources walked by
//       running sums) and shared by the 8 waves. S^T = K Q^T and O^T = V^T P^T run on
//       v_mfma_f32_32x32x16_bf16, so every lane owns one query column of both
//       products and the softmax needs a single cross-lane exchange per tile.
//   ring_step_wide<HG>  bf16, head_dim 512: 16 query rows per wave over the
//       whole of d on v_mfma_f32_16x16x32_bf16 (below).
//   ring_step_generic<T, D>  fp32: one workgroup per (query row, query head),
//       fp32 arithmetic throughout.
#include "kernels.h"
#include "lds_tiles.h"

namespace cpattn {
namespace {

constexpr int kMaxSeq = 64;  // sequences per launch (the host splits larger batches)

struct SeqTable {
  int32_t n;                      // sequences in this launch
  int32_t c[kMaxSeq];             // chunk length c_i = Lp_i / (2 cp), Lp_i = L_i rounded up to a multiple of 2 cp
  int32_t len[kMaxSeq];           // true length L_i: slots at or past it are pad tokens
  int64_t row_off[kMaxSeq];       // first local row of sequence i (same in q and kv blocks)
  int32_t start[kMaxSeq + 1];     // prefix of work units (tiles or rows) per sequence
};

struct StepArgs {
  const void *q;
  const void *k;
  const void *v;
  float *m;
  float *den;
  float *num;
  int32_t n_hq;
  int32_t n_kv;
  int32_t a_head, a_tail;  // query chunk ids: rank, 2cp-1-rank
  int32_t b_head, b_tail;  // key chunk ids: src, 2cp-1-src
  float scale;             // softmax scale (natural units)
  int32_t accumulate;
};

// Real (non-pad) tokens of chunk `chunk` of a sequence of true length len
// split into chunks of c slots.
__host__ __device__ __forceinline__ int chunk_valid(int len, int chunk, int c) {
  const int v = len - chunk * c;
  return v < 0 ? 0 : (v < c ? v : c);
}

__host__ __device__ __forceinline__ int find_seq(const SeqTable &t, int32_t unit) {
  int i = 0;
  while (i + 1 < t.n && t.start[i + 1] <= unit) ++i;
  return i;
}

// Stores the max and the denominator of one (row, head) triple (the caller
// stores the numerator and has already merged with the old triple if asked).
__device__ __forceinline__ void store_stats(float *mp, float *dp, float m_new, float d_new) {
  *mp = m_new;
  *dp = d_new;
}

// ----------------------------------------------------------------------------
// MFMA kernel (bf16)
// ----------------------------------------------------------------------------

// Per head_dim configuration: keys per tile (BN), waves per workgroup (NW),
// 32-row blocks per wave (NB) and waves per SIMD (WPE). head_dim 64/128: 8
// waves, two per SIMD, so one wave's MFMAs overlap the other's softmax and
// latencies (a wave per SIMD with two row blocks halves LDS reads per MFMA but
// measured half the speed). head_dim 512 runs ring_step_wide (wave quads split d).
template <int D>
struct Cfg;
template <>
struct Cfg<64> {
  static constexpr int BN = 64, NW = 8, NB = 1, WPE = 2;
};
template <>
struct Cfg<128> {
  static constexpr int BN = 64, NW = 8, NB = 1, WPE = 2;
};
template <>
struct Cfg<512> {
  static constexpr int BN = 32, NW = 8, WPE = 2;
  static constexpr int RW = 16;  // query rows of a wave (the columns of v_mfma_f32_16x16x32_bf16)
};
template <int D>
constexpr int kThreadsOf = 64 * Cfg<D>::NW;
// Query rows of one workgroup: the kernels use these, and the host tiles every
// chunk by the same numbers.
template <int D, int HG>
constexpr int kRowsMfma = 32 * Cfg<D>::NB * Cfg<D>::NW / HG;
template <int HG>
constexpr int kRowsWide = Cfg<512>::RW * Cfg<512>::NW / HG;

// Per-thread byte offsets (relative to the first key row of a tile) of the
// buffer-to-LDS copies of a K and a V tile. Lane L of a wave writes bytes
// [16L, 16L+16) of the 1 KB LDS chunk the wave names, so it loads the global
// chunk that belongs at that position of the swizzled tile; every copy
// instruction moves whole rows, which keeps the loads at full line width.
template <int D>
struct StageMap {
  static constexpr int BN = Cfg<D>::BN, KCH = D / 8;
  static constexpr int KN = (BN * D * 2 / 1024) / Cfg<D>::NW;   // 1 KB chunks per wave and tile
  static_assert(KN * 1024 * Cfg<D>::NW == BN * D * 2, "a tile must split into whole 1 KB chunks per wave");
  uint32_t k[KN];
  uint32_t v[KN];
};

template <int D>
__device__ __forceinline__ StageMap<D> stage_map(uint32_t row_bytes, int g) {
  using M = StageMap<D>;
  StageMap<D> o;
  constexpr int ROWS_PER_KB = 1024 / (D * 2);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < M::KN; ++i) {
    const int q = wave * M::KN + i;                    // 1 KB chunk of the tile
    const int key = q * ROWS_PER_KB + lane / M::KCH;
    const int pc = lane % M::KCH;                      // physical chunk in the LDS row
    const uint32_t base = key * row_bytes + (uint32_t)(g * D * 2);
    o.k[i] = base + (uint32_t)((pc ^ k_swizzle<D>(key)) * 16);   // logical chunk held there
    o.v[i] = base + (uint32_t)((pc ^ v_swizzle<D>(key)) * 16);
  }
  return o;
}

// Starts the copies of a tile straight into its LDS buffer: the wave's KN
// chunks of 1 KB.
template <int D>
__device__ __forceinline__ void load_tile(const uint32_t (&off)[StageMap<D>::KN], u32x4_t rsrc, __bf16 *dst) {
  const int wave = threadIdx.x >> 6;
  const u32x4_t rs = uniform_words(rsrc);
#pragma unroll
  for (int i = 0; i < StageMap<D>::KN; ++i) dma_1k(off[i], rs, dst + (wave * StageMap<D>::KN + i) * 512);
}

// Work unit and head group of a workgroup. When the head groups come in
// multiples of 8, the grid walks them XCD-major: workgroup b runs on XCD b % 8
// and takes head group (b % 8) + 8 * ((b / 8) / units), so the workgroups
// resident on one XCD at a time share a head group, and with it the K and V
// tiles in that XCD's L2. Otherwise unit-major, head group fastest.
__device__ __forceinline__ void unit_and_group(int n_hg, int &unit, int &hg) {
  const int b = blockIdx.x;
  if ((n_hg & 7) == 0) {
    const int units = gridDim.x / n_hg;
    const int j = b >> 3;
    unit = j % units;
    hg = (b & 7) + 8 * (j / units);
  } else {
    unit = b / n_hg;
    hg = b - unit * n_hg;
  }
}

// S^T = K Q^T for the keys of a staged tile, in 32-key blocks, for the NB
// 32-row blocks of the wave: every K fragment read from LDS feeds NB MFMAs.
template <int D, int NB>
__device__ __forceinline__ void qk_tile(const __bf16 *Kc, const bf16x8_t (&qf)[NB][D / 16],
                                        f32x16_t (&sacc)[NB][Cfg<D>::BN / 32]) {
  const int lane = threadIdx.x & 63;
  const int qi = lane & 31, hf = lane >> 5;
  // k-step major: consecutive products go to different accumulators
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int ch = ks * 2 + hf;
#pragma unroll
    for (int mb = 0; mb < Cfg<D>::BN / 32; ++mb) {
      const int key = mb * 32 + qi;
      const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(&Kc[key * D + ((ch ^ k_swizzle<D>(key)) * 8)]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        sacc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[nb][ks], ks == 0 ? f32x16_t{} : sacc[nb][mb],
                                                              0, 0, 0);
    }
  }
}


// The key segments of a workgroup whose query rows lie in chunk qa: the tail
// key chunk, then the head key chunk, each kept when it is causally visible
// and holds a real key. A diagonal segment (same chunk) ends at the
// workgroup's last real row; others at the chunk's real keys.
template <int BN>
__host__ __device__ __forceinline__ Segs<BN> make_segs(const StepArgs &a, int qa, int c, int len, int64_t row_off,
                                              int row_end) {
  const bool diag_t = a.b_tail == qa, diag_h = a.b_head == qa;
  const int lim_t = diag_t ? row_end : c, lim_h = diag_h ? row_end : c;
  const int val_t = chunk_valid(len, a.b_tail, c), val_h = chunk_valid(len, a.b_head, c);
  const int end_t = lim_t < val_t ? lim_t : val_t;
  const int end_h = lim_h < val_h ? lim_h : val_h;
  const bool ok_t = a.b_tail <= qa && end_t > 0;
  const bool ok_h = a.b_head <= qa && end_h > 0;
  Segs<BN> sg;
  sg.nseg = (int)ok_t + (int)ok_h;
  sg.row[0] = ok_t ? row_off + c : row_off;
  sg.diag[0] = ok_t ? diag_t : diag_h;
  sg.end[0] = ok_t ? end_t : (ok_h ? end_h : 0);
  sg.row[1] = row_off;   // a second segment is always the head key chunk
  sg.diag[1] = diag_h;
  sg.end[1] = (ok_t && ok_h) ? end_h : 0;
  sg.n0 = (sg.end[0] + BN - 1) / BN;
  return sg;
}

// Buffer resource of tile t of the key segments: based at the tile's first key
// row, with the visible keys of its segment from there on as the range; past
// the last tile an empty range at the block start (the copy then writes zeros
// and touches no memory, so the tile loops need no branch).
template <int BN>
__host__ __device__ __forceinline__ u32x4_t seg_tile_words(const Segs<BN> &sg, int ntiles, const char *blk, int t,
                                                           uint32_t rb) {
  const bool ok = t < ntiles;
  const int s = sg.seg(t), k = sg.k0(t);
  return tile_words(blk, ok ? sg.row[s] + k : 0, ok ? sg.end[s] - k : 0, rb);
}

// seg_tile_words for the tiles t0, t0 + 1, ... as running sums: each step moves
// the tile's address forward and its range down by one tile, and the second
// segment's first tile restarts both from that segment, so a step costs a few
// scalar additions instead of the products and selects. The resources are the
// same words bit for bit (the range clamp is done on the two 32-bit halves).
template <int BN>
struct TileWalk {
  int t, n0, ntiles;
  uint64_t blk;
  uint64_t addr;          // address of tile t's first key row
  int64_t lim;            // bytes of visible keys from there to its segment's end
  uint64_t addr1;         // the same for the first tile of the second segment
  int64_t lim1;
  int64_t step;           // bytes of one tile
  __host__ __device__ __forceinline__ TileWalk(const Segs<BN> &sg, int ntiles_, const char *blk_, int t0,
                                               uint32_t rb)
      : t(t0), n0(sg.n0), ntiles(ntiles_), blk((uint64_t)(uintptr_t)blk_) {
    const int s = sg.seg(t0), k = sg.k0(t0);
    addr = blk + (uint64_t)((sg.row[s] + k) * (int64_t)rb);
    lim = (int64_t)(sg.end[s] - k) * rb;
    addr1 = blk + (uint64_t)(sg.row[1] * (int64_t)rb);
    lim1 = (int64_t)sg.end[1] * rb;
    step = (int64_t)BN * rb;
  }
  __host__ __device__ __forceinline__ void next() {
    ++t;
    if (t == n0) {
      addr = addr1;
      lim = lim1;
    } else {
      addr += (uint64_t)step;
      lim -= step;
    }
  }
  // a tile before the end has lim > 0, so the clamp of tile_words to 0x7FFFFFFF
  // reads as: high half zero and low half below the cap, else the cap
  __host__ __device__ __forceinline__ u32x4_t words() const {
    const bool ok = t < ntiles;
    const uint64_t base = ok ? addr : blk;
    const uint32_t lo = (uint32_t)(uint64_t)lim, hi = (uint32_t)((uint64_t)lim >> 32);
    const uint32_t nrec = ok ? ((hi == 0u && lo < 0x7FFFFFFFu) ? lo : 0x7FFFFFFFu) : 0u;
    return u32x4_t{(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, nrec, kBufferWord3};
  }
};

template <int D, int HG>
__global__ __launch_bounds__(kThreadsOf<D>) __attribute__((amdgpu_waves_per_eu(Cfg<D>::WPE, Cfg<D>::WPE)))
void ring_step_mfma(SeqTable tab, StepArgs a) {
  constexpr int BN = Cfg<D>::BN;
  constexpr int NW = Cfg<D>::NW;
  constexpr int NB = Cfg<D>::NB;                // 32-row blocks per wave
  constexpr int MB = BN / 32;                   // 32-key blocks per tile
  constexpr int PKS = BN / 16;                  // 16-key MFMA k-steps of the PV product
  constexpr int BM = kRowsMfma<D, HG>;          // query rows per workgroup
  constexpr int KS = D / 16;                    // MFMA k-steps for QK^T
  constexpr int DB = D / 32;                    // 32-wide d blocks of the output
  constexpr int KSZ = BN * D;                   // K tile (bf16 elements)
  constexpr int VSZ = BN * D;                   // V tile

  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][KSZ];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[2][VSZ];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int qi = lane & 31;
  const int hf = lane >> 5;

  const int n_hg = a.n_hq / HG;
  int unit, hg;
  unit_and_group(n_hg, unit, hg);
  const int si = find_seq(tab, unit);
  const int c = tab.c[si];
  const int nt = (c + BM - 1) / BM;
  const int lt = unit - tab.start[si];
  // tail-chunk tiles first (they see at least as many keys), each chunk in
  // descending row order
  const bool tail = lt < nt;
  const int tile = tail ? (nt - 1 - lt) : (nt - 1 - (lt - nt));
  const int qa = tail ? a.a_tail : a.a_head;
  const int64_t qrow0 = tab.row_off[si] + (tail ? c : 0);   // first local row of this chunk

  const int h = hg * HG + (wave % HG);
  const int rep = a.n_hq / a.n_kv;
  const int g = h / rep;
  const int wrow0 = tile * BM + (wave / HG) * 32 * NB;      // wave's first row inside the chunk
  const int wg_row_end = min(c, tile * BM + BM);            // rows of the workgroup: [tile*BM, wg_row_end)

  // key segments that are not empty, the tail key chunk first
  const int len = tab.len[si];
  const int q_valid = chunk_valid(len, qa, c);              // real rows of this query chunk
  const Segs<BN> sg = make_segs<BN>(a, qa, c, len, tab.row_off[si], min(wg_row_end, q_valid));
  const int nseg = sg.nseg;

  int row[NB];
  bool row_ok[NB], row_in[NB];
  int64_t grow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    row[nb] = wrow0 + nb * 32 + qi;
    row_in[nb] = row[nb] < c;        // a row of the local buffer
    row_ok[nb] = row[nb] < q_valid;  // a real (non-pad) row
    grow[nb] = qrow0 + row[nb];      // local row index in the rank's buffer
  }

  if (nseg == 0) {
    // every row of this tile sees no key: the identity (unchanged when accumulating)
    if (!a.accumulate) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (!row_in[nb]) continue;
        if (hf == 0) store_stats(a.m + grow[nb] * a.n_hq + h, a.den + grow[nb] * a.n_hq + h, kNegInf, 0.f);
        float *nptr = a.num + (grow[nb] * a.n_hq + h) * (int64_t)D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<f32x4_t *>(nptr + db * 32 + 8 * g4 + 4 * hf) = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }
  const int ntiles = sg.tiles();

  // Q fragments: B operands of S^T = K Q^T, lane holds q[row][ks*16 + 8*hf .. +8]
  const __bf16 *qbase = reinterpret_cast<const __bf16 *>(a.q);
  bf16x8_t qf[NB][KS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const __bf16 *qp = qbase + (grow[nb] * a.n_hq + h) * (int64_t)D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[nb][ks] = row_ok[nb] ? *reinterpret_cast<const bf16x8_t *>(qp + ks * 16)
                              : __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
  }

  const float sl2 = a.scale * kLog2e;
  const float thr = kRescaleLog2 / sl2;   // rescale threshold in raw-score units
  float m_ref[NB], l_run[NB];             // reference max of raw scores; this lane's share of the denominator
  f32x16_t oacc[NB][DB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_ref[nb] = kNegInf;
    l_run[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[nb][db][r] = 0.f;
  }

  const char *kblock = reinterpret_cast<const char *>(a.k);
  const char *vblock = reinterpret_cast<const char *>(a.v);
  const uint32_t row_bytes = (uint32_t)(a.n_kv * D * 2);   // bytes between consecutive keys
  const StageMap<D> smap = stage_map<D>(row_bytes, g);
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Prologue: K and V of tile 0 and K of tile 1 into LDS. Through the loop the K
  // pipeline runs one tile ahead of V: iteration `it` multiplies K of tile it+1
  // (QK^T of the next tile, on the matrix cores) while the exponentials of tile
  // it run on the vector ALUs, then V of tile it. A tile that lies entirely in
  // the future of a wave's rows is masked to -inf and contributes zeros.
  {
    load_tile<D>(smap.k, tile_words(kblock, sg.row[0], sg.end[0], row_bytes), Ks[0]);
    load_tile<D>(smap.v, tile_words(vblock, sg.row[0], sg.end[0], row_bytes), Vt[0]);
    if (ntiles > 1) {
      const int s1 = sg.seg(1), k1 = sg.k0(1);
      load_tile<D>(smap.k, tile_words(kblock, sg.row[s1] + k1, sg.end[s1] - k1, row_bytes), Ks[1]);
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();

  f32x16_t snext[NB][MB];
  qk_tile<D, NB>(Ks[0], qf, snext);
  // every wave has read K of tile 0 before the first iteration's copy replaces it
  __syncthreads();
  // copy resources of K from tile 2 on and of V from tile 1 on; each iteration
  // uses the pair computed at the end of the one before
  TileWalk<BN> kw(sg, ntiles, kblock, 2, row_bytes), vw(sg, ntiles, vblock, 1, row_bytes);
  u32x4_t kd = kw.words(), vd = vw.words();

  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int sc = sg.seg(it);
    const int k0 = sg.k0(it);
    const int kend = sg.end[sc];
    const bool diag = sg.diag[sc];

    // prefetch: K of tile it+2 into the LDS buffer of K of tile it (read in the
    // previous iteration) and V of tile it+1 into that of V of tile it-1. The
    // copies are spread over the MFMAs of the next tile's QK^T (copy_after(i)
    // follows product i) rather than issued together: eight waves issuing them
    // at once queue on the CU's load path (about 62 bytes per clock) with
    // nothing else to run.
    constexpr int KN = StageMap<D>::KN;
    const u32x4_t rk = uniform_words(kd), rv = uniform_words(vd);
    auto copy_after = [&](int i) {
#pragma unroll
      for (int j = 0; j < 2 * KN; ++j)
        if (j * KS * MB / (2 * KN) == i) {
          if (j < KN) dma_1k(smap.k[j], rk, Ks[cur] + (wave * KN + j) * 512);
          else dma_1k(smap.v[j - KN], rv, Vt[cur ^ 1] + (wave * KN + j - KN) * 512);
        }
    };

    // this tile's scores are used in place: a block's next-tile QK^T starts
    // only after the block's exponentials have read it
    f32x16_t (&sacc)[NB][MB] = snext;
    if ((k0 + BN > kend) || (diag && k0 + BN - 1 > wrow0)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = k0 + mb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool vis = (kk < kend) && (!diag || kk <= row[nb]);
            if (!vis) sacc[nb][mb][r] = kNegInf;
          }
    }

    // ---- online softmax (lane = query column; keys split over the two halves)
    float mx[NB];
    bool grows = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // four independent partial maxima, then combined
      float x4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) x4[r & 3] = fmaxf(x4[r & 3], sacc[nb][mb][r]);
      mx[nb] = max_across_halves(fmaxf(fmaxf(x4[0], x4[1]), fmaxf(x4[2], x4[3])));
      grows |= mx[nb] > m_ref[nb] + thr;
    }
    if (__any(grows)) {
      // the max grew past the threshold for some query of this wave: move every
      // lane's reference to its current max (exact rescale)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float m_new = fmaxf(m_ref[nb], mx[nb]);
        const float alpha = (m_new == kNegInf) ? 1.f : exp2_fast((m_ref[nb] - m_new) * sl2);
        l_run[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[nb][db][r] *= alpha;
        m_ref[nb] = m_new;
      }
    }
    float mref[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) mref[nb] = (m_ref[nb] == kNegInf) ? 0.f : m_ref[nb] * sl2;

    // ---- one scheduling region: QK^T of the next tile (matrix cores) with this
    // tile's exponentials (vector ALUs), then this tile's PV product. The
    // scores stay in the registers the next QK^T writes, so each 32-key block
    // is exponentiated before its next-tile product starts (no copy of the
    // scores, which would sit in the phase where both waves of a SIMD run
    // vector work only)
    uint32_t pk[NB][MB][8];
    auto exps_block = [&](int mb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = exp2_fast(fmaf(sacc[nb][mb][r], sl2, -mref[nb]));
          const float p1 = exp2_fast(fmaf(sacc[nb][mb][r + 1], sl2, -mref[nb]));
          pk[nb][mb][r >> 1] = pack_bf16x2(p0, p1);
          // denominator from the same rounded values the PV product uses
          l_run[nb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[nb][mb][r >> 1]), ones,
                                                      l_run[nb], false);
        }
    };
    // exponentials of block 0; then, per 32-key block, the next tile's QK^T
    // (matrix cores) beside the exponentials of the following block
    const __bf16 *Kn = Ks[cur ^ 1];
    exps_block(0);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int key = mb * 32 + qi;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = ks * 2 + hf;
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(&Kn[key * D + ((ch ^ k_swizzle<D>(key)) * 8)]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          snext[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[nb][ks], ks == 0 ? f32x16_t{} : snext[nb][mb],
                                                                 0, 0, 0);
        copy_after(mb * KS + ks);
      }
      if (mb + 1 < MB) exps_block(mb + 1);
    }
    const __bf16 *Vc = Vt[cur];
#pragma unroll
    for (int ks = 0; ks < PKS; ++ks) {
      const int mb = ks >> 1;
      const int base = (ks & 1) * 4;
      bf16x8_t pf[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        u32x4_t pw = {pk[nb][mb][base], pk[nb][mb][base + 1], pk[nb][mb][base + 2], pk[nb][mb][base + 3]};
        pf[nb] = __builtin_bit_cast(bf16x8_t, pw);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8_t vf = v_fragment<D>(Vc, ks, db * 32);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          oacc[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[nb], oacc[nb][db], 0, 0, 0);
      }
    }

    kw.next();
    vw.next();
    kd = kw.words();
    vd = vw.words();
    // K of tile it+2 replaces K of tile it; V of tile it+1 replaces V of tile it-1
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }

  // ---- epilogue: natural-log max, full denominator, optional merge, store
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // a pad row is stored as a row that saw no key (the merge identity)
    const float l_sum = l_run[nb] + __shfl_xor(l_run[nb], 32);
    const float l_tot = row_ok[nb] ? l_sum : 0.f;
    if (!row_in[nb]) continue;
    float *mptr = a.m + (grow[nb] * a.n_hq + h);
    float *dptr = a.den + (grow[nb] * a.n_hq + h);
    float *nptr = a.num + (grow[nb] * a.n_hq + h) * (int64_t)D;
    const float m_nat = (m_ref[nb] == kNegInf || !row_ok[nb]) ? kNegInf : m_ref[nb] * a.scale;
    auto out_at = [&](int db, int g4) {
      const f32x4_t o = {oacc[nb][db][4 * g4], oacc[nb][db][4 * g4 + 1], oacc[nb][db][4 * g4 + 2],
                         oacc[nb][db][4 * g4 + 3]};
      return row_ok[nb] ? o : f32x4_t{0.f, 0.f, 0.f, 0.f};
    };
    if (a.accumulate) {
      // every load of the previous triple is issued before the first use, so
      // the row's accumulator read costs one memory latency, not one per load
      const float m_old = *mptr;
      const float d_old = *dptr;
      f32x4_t old[DB][4];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          old[db][g4] = *reinterpret_cast<const f32x4_t *>(nptr + db * 32 + 8 * g4 + 4 * hf);
      float w_old, w_new, m_out;
      merge_weights(m_old, m_nat, m_out, w_old, w_new);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<f32x4_t *>(nptr + db * 32 + 8 * g4 + 4 * hf) = old[db][g4] * w_old + out_at(db, g4) * w_new;
      if (hf == 0) store_stats(mptr, dptr, m_out, w_old * d_old + w_new * l_tot);
    } else {
      if (hf == 0) store_stats(mptr, dptr, m_nat, l_tot);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<f32x4_t *>(nptr + db * 32 + 8 * g4 + 4 * hf) = out_at(db, g4);
    }
  }
}

// ----------------------------------------------------------------------------
// head_dim 512 (bf16): 16 query rows per wave over the whole of d.
// ----------------------------------------------------------------------------
// A workgroup of 8 waves (two per SIMD) holds HG query heads of one kv group x
// 128 / HG query rows; wave w owns 16 rows of head w % HG. The rows are the 16
// columns of v_mfma_f32_16x16x32_bf16 in both products, S^T = K Q^T (16-key
// blocks x 16 rows, k-steps of 32 columns of d) and O^T = V^T P^T (16-column
// blocks of d x 16 rows, the 32 keys of a tile as one k-step), so a wave keeps
// its Q fragments (64 registers) and its whole output (128 registers) and no
// score leaves the wave: the softmax needs two cross-lane exchanges per tile
// and nothing goes through LDS but the K and V tiles. Lane l holds row l % 16;
// its 16-lane group g holds keys 4g + {0..3} and 16 + 4g + {0..3} of a tile,
// the order the P operand and the transposed reads of V^T share. 32-key K and V
// tiles (32 KB each) are copied straight into double-buffered LDS (128 KB),
// every 1 KB copy a whole key row; the copies of tile t+1 fly while tile t
// computes, with one barrier per tile.
template <int HG>
__global__ __launch_bounds__(kThreadsOf<512>) __attribute__((amdgpu_waves_per_eu(Cfg<512>::WPE, Cfg<512>::WPE)))
void ring_step_wide(SeqTable tab, StepArgs a) {
  constexpr int D = 512;
  constexpr int BN = Cfg<D>::BN;                // 32 keys per tile
  constexpr int NW = Cfg<D>::NW;
  constexpr int RW = Cfg<D>::RW;                // 16 rows per wave
  constexpr int BM = kRowsWide<HG>;             // query rows per workgroup
  constexpr int KS = D / 32;                    // QK^T k-steps
  constexpr int DB = D / 16;                    // 16-column blocks of O^T
  constexpr int TSZ = BN * D;                   // bf16 elements of a K (or V) tile
  constexpr int CPW = BN / NW;                  // 1 KB key rows each wave copies per tile
  static_assert(CPW * NW == BN, "a tile's key rows split evenly over the waves");

  __shared__ __attribute__((aligned(16))) __bf16 Ks[2][TSZ];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[2][TSZ];

  const int tid = threadIdx.x;
  // the wave index as a scalar: head, rows and copy addresses derived from it
  // stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;     // the lane's query row within the wave's 16
  const int grp = lane >> 4;     // 16-lane group

  const int n_hg = a.n_hq / HG;
  int unit, hg;
  unit_and_group(n_hg, unit, hg);
  const int si = find_seq(tab, unit);
  const int c = tab.c[si];
  const int nt = (c + BM - 1) / BM;
  const int lt = unit - tab.start[si];
  const bool tail = lt < nt;
  const int tile = tail ? (nt - 1 - lt) : (nt - 1 - (lt - nt));
  const int qa = tail ? a.a_tail : a.a_head;
  const int64_t qrow0 = tab.row_off[si] + (tail ? c : 0);

  const int h = hg * HG + (wave % HG);
  const int rep = a.n_hq / a.n_kv;
  const int g = h / rep;
  const int wrow0 = tile * BM + (wave / HG) * RW;           // wave's first row inside the chunk
  const int wg_row_end = min(c, tile * BM + BM);

  const int len = tab.len[si];
  const int q_valid = chunk_valid(len, qa, c);
  const Segs<BN> sg = make_segs<BN>(a, qa, c, len, tab.row_off[si], min(wg_row_end, q_valid));
  const int nseg = sg.nseg;

  const int row = wrow0 + col;
  const bool row_in = row < c;          // a row of the local buffer
  const bool row_ok = row < q_valid;    // a real (non-pad) row
  const int64_t grow = qrow0 + row;
  const bool wave_idle = wrow0 >= q_valid;   // every row of the wave is a pad row (or past the chunk)

  if (nseg == 0) {
    float *mptr = a.m + (grow * a.n_hq + h);
    float *dptr = a.den + (grow * a.n_hq + h);
    float *nptr = a.num + (grow * a.n_hq + h) * (int64_t)D;
    // every row of this workgroup sees no key: the identity (unchanged when accumulating)
    if (!a.accumulate && row_in) {
      if (grp == 0) store_stats(mptr, dptr, kNegInf, 0.f);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4_t *>(nptr + 16 * db + 4 * grp) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int ntiles = sg.tiles();

  const char *kblock = reinterpret_cast<const char *>(a.k);
  const char *vblock = reinterpret_cast<const char *>(a.v);
  const uint32_t row_bytes = (uint32_t)(a.n_kv * D * 2);
  // Copies: wave w copies key rows q = w + NW i (i < CPW) of a tile, each
  // through a buffer resource of its own (RowWalk: based at the row's head, 1 KB
  // in range when the row holds a visible key, else empty), so every lane
  // offset stays below 1 KB. Lane L loads the 16 bytes that belong at position
  // L of the swizzled LDS row, the logical chunk L ^ swizzle(q); with
  // q = w + 8 i that is L ^ (w + 8 (i & 1)) for K and L ^ 2 w for V, so three
  // lane offsets serve every copy.
  const int wv = wave;
  static_assert(NW == 8 && CPW % 2 == 0, "the copy offsets assume 8 waves");
  const uint32_t koff0 = (uint32_t)((lane ^ k_swizzle<D>(wv)) * 16);
  const uint32_t koff1 = (uint32_t)((lane ^ k_swizzle<D>(wv + 8)) * 16);
  const uint32_t voff = (uint32_t)((lane ^ v16_swizzle<D>(wv)) * 16);
  const uint32_t gbase = (uint32_t)(g * D * 2);
  auto issue = [&](const RowWalk<BN> &kw, const RowWalk<BN> &vw, int buf) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int q = wv + NW * i;
      dma_1k((i & 1) ? koff1 : koff0, uniform_words(kw.row(q, row_bytes, gbase)), Ks[buf] + q * 512);
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int q = wv + NW * i;
      dma_1k(voff, uniform_words(vw.row(q, row_bytes, gbase)), Vt[buf] + q * 512);
    }
  };
  // LDS read addresses. K (A operand of S^T = K Q^T, k-step ks = 4 m + j):
  // row col, logical chunk 4 ks + grp, swizzled by col: chunk
  // 4 (ks ^ (col >> 2)) + (grp ^ (col & 3)) = 16 m + 4 (j ^ (col >> 2)) + ...,
  // so kp[j] + 128 m, and 16 rows further for the second key block. V^T
  // (16-column block db = 8 m + j, v16_fragment's addresses): vp[j] + 128 m.
  // With the buffer index a constant (the loop below handles two tiles per
  // iteration) every read is one of these 12 registers plus an immediate.
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

  // tile 0 into buffer 0, then the walks move on to tile 1
  RowWalk<BN> kw(sg, ntiles, kblock, 0, row_bytes), vw(sg, ntiles, vblock, 0, row_bytes);
  issue(kw, vw, 0);
  kw.next();
  vw.next();

  // Q fragments (B operand of S^T = K Q^T): lane holds q[row][32 ks + 8 grp .. +8]
  bf16x8_t qf[KS];
  {
    const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) + (grow * a.n_hq + h) * (int64_t)D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = row_ok ? *reinterpret_cast<const bf16x8_t *>(qp + 32 * ks)
                      : __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
  }

  const float sl2 = a.scale * kLog2e;
  const float thr = kRescaleLog2 / sl2;   // rescale threshold in raw-score units
  float m_ref = kNegInf, l_run = 0.f;
  f32x4_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // one tile in buffer `cur` (a constant in each of the two calls below)
  auto tile_step = [&](int it, const int cur) {
    // this wave's copies of tile it have landed; after the barrier every
    // wave's have, and every wave is done with tile it-1, whose buffer the
    // copies of tile it+1 overwrite
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    const int sc = sg.seg(it);
    const int k0 = sg.k0(it);
    const int kend = sg.end[sc];
    const bool diag = sg.diag[sc];

    // ---- S^T = K Q^T: key blocks 0..15 (s0) and 16..31 (s1) of the tile; the
    // K fragments of the next k-step are read before this one's products
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    auto kread = [&](int ks, int blk) {
      return *reinterpret_cast<const bf16x8_t *>(kp[ks & 3] + cur * TSZ + 128 * (ks >> 2) + blk * 16 * D);
    };
    bf16x8_t ka = kread(0, 0), kb = kread(0, 1);
    // the copies of tile it+1 are spread over the k-steps (one per two): issued
    // together, the 64 copies of the workgroup queue on the CU's load path and
    // hold up the waves that issue them
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
        const int i = ks >> 1;   // copy i: K rows for i < CPW, then V rows
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
    if ((k0 + BN > kend) || (diag && k0 + BN - 1 > wrow0)) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kk0 = k0 + 4 * grp + t, kk1 = kk0 + 16;
        if (!(kk0 < kend && (!diag || kk0 <= row))) s0[t] = kNegInf;
        if (!(kk1 < kend && (!diag || kk1 <= row))) s1[t] = kNegInf;
      }
    }

    // ---- online softmax: the row's 32 keys lie in the 4 lanes col, col + 16, ...
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
    // denominator from the same rounded values the PV product uses
#pragma unroll
    for (int i = 0; i < 4; ++i)
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[i]), ones, l_run, false);
    const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});

    // ---- O^T += V^T P^T: lane (d column col of block db, group grp) takes
    // V[4 grp + 0..3][16 db + col] and V[16 + 4 grp + 0..3][16 db + col], two
    // transposed reads; the next block's are issued before this block's product
    auto vread = [&](int db) { return v16_read<D>(vp[db & 7] + cur * TSZ + 128 * (db >> 3)); };
    bf16x8_t vf = vread(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8_t nv = db + 1 < DB ? vread(db + 1) : vf;
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[db], 0, 0, 0);
      vf = nv;
    }
  };
  if (wave_idle) {
    // no row of this wave is real: its outputs are the identity whatever the
    // keys, so it only keeps the workgroup's copy and barrier schedule, one
    // tile at a time (the same waits, barriers and copies as tile_step)
    for (int it = 0; it < ntiles; ++it) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      const int nxt = (it & 1) ^ 1;
#pragma unroll
      for (int i = 0; i < KS / 2; ++i) {
        const int q = wv + NW * (i % CPW);
        if (i < CPW)
          dma_1k((i & 1) ? koff1 : koff0, uniform_words(kw.row(q, row_bytes, gbase)), Ks[nxt] + q * 512);
        else
          dma_1k(voff, uniform_words(vw.row(q, row_bytes, gbase)), Vt[nxt] + q * 512);
      }
      kw.next();
      vw.next();
    }
  } else {
    for (int it = 0; it < ntiles; it += 2) {
      tile_step(it, 0);
      if (it + 1 < ntiles) tile_step(it + 1, 1);
    }
  }
  // the copies issued past the last tile (empty ranges: zeros, no memory read)
  // land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // ---- epilogue: natural-log max, full denominator, optional merge, store
  // (the 4 groups hold disjoint keys of the row: their sums add up)
  float l_sum = l_run + __shfl_xor(l_run, 16);
  l_sum += __shfl_xor(l_sum, 32);
  const float l_tot = row_ok ? l_sum : 0.f;   // a pad row is stored as a row that saw no key
  if (!row_in) return;
  // (the row's pointers are formed here, not kept through the loop)
  const int64_t ri = (qrow0 + (tile * BM + (wave / HG) * RW) + (threadIdx.x & 15)) * a.n_hq + h;
  float *mptr = a.m + ri;
  float *dptr = a.den + ri;
  float *nptr = a.num + ri * (int64_t)D;
  const float m_nat = (m_ref == kNegInf || !row_ok) ? kNegInf : m_ref * a.scale;
  if (a.accumulate) {
    // the previous triple is read in groups of kEpiBlocks 16-column blocks,
    // every load of a group issued before the group's first use; the stats go
    // last so that no load waits behind a store the compiler cannot tell apart
    const float m_old = *mptr;
    const float d_old = *dptr;
    constexpr int kEpiBlocks = 8;
    static_assert(DB % kEpiBlocks == 0, "whole groups of output blocks");
    f32x4_t old[kEpiBlocks];
#pragma unroll
    for (int i = 0; i < kEpiBlocks; ++i) old[i] = *reinterpret_cast<const f32x4_t *>(nptr + 16 * i + 4 * grp);
    float w_old, w_new, m_out;
    merge_weights(m_old, m_nat, m_out, w_old, w_new);
#pragma unroll
    for (int g0 = 0; g0 < DB; g0 += kEpiBlocks) {
      if (g0 > 0) {
#pragma unroll
        for (int i = 0; i < kEpiBlocks; ++i)
          old[i] = *reinterpret_cast<const f32x4_t *>(nptr + 16 * (g0 + i) + 4 * grp);
      }
#pragma unroll
      for (int i = 0; i < kEpiBlocks; ++i) {
        const f32x4_t o = row_ok ? oacc[g0 + i] : f32x4_t{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4_t *>(nptr + 16 * (g0 + i) + 4 * grp) = old[i] * w_old + o * w_new;
      }
    }
    if (grp == 0) store_stats(mptr, dptr, m_out, w_old * d_old + w_new * l_tot);
  } else {
    if (grp == 0) store_stats(mptr, dptr, m_nat, l_tot);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<f32x4_t *>(nptr + 16 * db + 4 * grp) = row_ok ? oacc[db] : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// ----------------------------------------------------------------------------
// Generic kernel: one workgroup per (local row, query head), fp32 arithmetic.
// ----------------------------------------------------------------------------

constexpr int kGenThreads = 256;

__device__ __forceinline__ float block_reduce_max(float v, float *scratch) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  float r = scratch[0];
  for (int i = 1; i < kGenThreads / 64; ++i) r = fmaxf(r, scratch[i]);
  return r;
}

__device__ __forceinline__ float block_reduce_sum(float v, float *scratch) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < kGenThreads / 64; ++i) r += scratch[i];
  return r;
}

template <typename T, int D>
__global__ __launch_bounds__(kGenThreads) void ring_step_generic(SeqTable tab, StepArgs a) {
  constexpr int PER = (D + kGenThreads - 1) / kGenThreads;   // output elements per thread
  __shared__ float qs[D];
  __shared__ float pbuf[kGenThreads];
  __shared__ float red[kGenThreads / 64];

  const int tid = threadIdx.x;
  const int unit = blockIdx.x;         // local row within this launch
  const int h = blockIdx.y;
  const int si = find_seq(tab, unit);
  const int c = tab.c[si];
  const int lr = unit - tab.start[si];         // 0 .. 2c-1
  const bool tail = lr >= c;
  const int qrow = tail ? lr - c : lr;         // row inside its chunk
  const int qa = tail ? a.a_tail : a.a_head;
  const int64_t grow = tab.row_off[si] + lr;
  const int rep = a.n_hq / a.n_kv;
  const int g = h / rep;
  const int len = tab.len[si];
  const bool real = qrow < chunk_valid(len, qa, c);   // pad rows see no key

  const T *qp = reinterpret_cast<const T *>(a.q) + (grow * a.n_hq + h) * (int64_t)D;
  for (int d = tid; d < D; d += kGenThreads) qs[d] = real ? Elem<T>::load1(qp + d) : 0.f;
  __syncthreads();

  const T *kb = reinterpret_cast<const T *>(a.k);
  const T *vb = reinterpret_cast<const T *>(a.v);
  const int64_t kv_stride = (int64_t)a.n_kv * D;

  float m_run = kNegInf, l_run = 0.f;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;

  for (int sg = 0; sg < 2; ++sg) {
    const int b = sg == 0 ? a.b_head : a.b_tail;
    if (b > qa || !real) continue;
    const int kend = min((b == qa) ? qrow + 1 : c, chunk_valid(len, b, c));
    const int64_t krow0 = tab.row_off[si] + (sg == 0 ? 0 : c);
    for (int k0 = 0; k0 < kend; k0 += kGenThreads) {
      const int key = k0 + tid;
      float s = kNegInf;
      if (key < kend) {
        const T *kp = kb + (krow0 + key) * kv_stride + g * D;
        float dot = 0.f;
        for (int d = 0; d < D; d += 8) {
          float kv8[8];
          Elem<T>::load8(kp + d, kv8);
#pragma unroll
          for (int e = 0; e < 8; ++e) dot = fmaf(qs[d + e], kv8[e], dot);
        }
        s = dot * a.scale;
      }
      const float cmax = block_reduce_max(s, red);
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = (m_run == kNegInf) ? 0.f : expf(m_run - m_new);
      const float p = (key < kend) ? expf(s - m_new) : 0.f;
      pbuf[tid] = p;
      const float psum = block_reduce_sum(p, red);   // its barriers also publish pbuf
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const int nk = min(kGenThreads, kend - k0);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int d = tid + i * kGenThreads;
        if (d < D) {
          float sum = 0.f;
          const T *vp = vb + (krow0 + k0) * kv_stride + g * D + d;
          for (int x = 0; x < nk; ++x) sum = fmaf(pbuf[x], Elem<T>::load1(vp + x * kv_stride), sum);
          acc[i] = acc[i] * alpha + sum;
        }
      }
      __syncthreads();   // pbuf is rewritten by the next chunk
    }
  }

  float *mp = a.m + (grow * a.n_hq + h);
  float *dp = a.den + (grow * a.n_hq + h);
  float *np_ = a.num + (grow * a.n_hq + h) * (int64_t)D;
  float w_old = 0.f, w_new = 1.f;
  if (a.accumulate) {
    float m_out;
    merge_weights(*mp, m_run, m_out, w_old, w_new);
    const float d_out = w_old * (*dp) + w_new * l_run;
    __syncthreads();   // every thread has read m and den
    if (tid == 0) store_stats(mp, dp, m_out, d_out);
  } else if (tid == 0) {
    store_stats(mp, dp, m_run, l_run);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = tid + i * kGenThreads;
    if (d < D) np_[d] = a.accumulate ? (w_old * np_[d] + w_new * acc[i]) : acc[i];
  }
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------

int pick_hg(int rep) { return (rep % 4 == 0) ? 4 : (rep % 2 == 0) ? 2 : 1; }

template <int D, int HG>
hipError_t launch_mfma(const SeqTable &t, const StepArgs &a, int units, hipStream_t s) {
  const int n_hg = a.n_hq / HG;
  const int64_t blocks = (int64_t)units * n_hg;
  hipLaunchKernelGGL((ring_step_mfma<D, HG>), dim3((unsigned)blocks), dim3(kThreadsOf<D>), 0, s, t, a);
  return hipGetLastError();
}

template <int HG>
hipError_t launch_wide(const SeqTable &t, const StepArgs &a, int units, hipStream_t s) {
  const int n_hg = a.n_hq / HG;
  const int64_t blocks = (int64_t)units * n_hg;
  hipLaunchKernelGGL((ring_step_wide<HG>), dim3((unsigned)blocks), dim3(kThreadsOf<512>), 0, s, t, a);
  return hipGetLastError();
}

// heads per workgroup: up to 4 query heads of one kv group
int pick_hg_d(int d, int rep) {
  (void)d;
  return pick_hg(rep);
}

template <int D>
hipError_t launch_mfma_d(const SeqTable &t, const StepArgs &a, int units, hipStream_t s) {
  if constexpr (D == 512) {
    const int hg = pick_hg_d(512, a.n_hq / a.n_kv);
    if (hg == 4) return launch_wide<4>(t, a, units, s);
    if (hg == 2) return launch_wide<2>(t, a, units, s);
    return launch_wide<1>(t, a, units, s);
  } else {
    const int hg = pick_hg(a.n_hq / a.n_kv);
    if (hg == 4) return launch_mfma<D, 4>(t, a, units, s);
    if (hg == 2) return launch_mfma<D, 2>(t, a, units, s);
    return launch_mfma<D, 1>(t, a, units, s);
  }
}

template <typename T, int D>
hipError_t launch_generic(const SeqTable &t, const StepArgs &a, int units, hipStream_t s) {
  hipLaunchKernelGGL((ring_step_generic<T, D>), dim3((unsigned)units, (unsigned)a.n_hq), dim3(kGenThreads), 0, s,
                     t, a);
  return hipGetLastError();
}

// The MFMA kernel covers bf16 (head_dim 64, 128, 512); fp32 runs the generic kernel.
bool use_mfma(int dtype, int d) { return dtype == CPATTN_DT_BF16 && (d == 64 || d == 128 || d == 512); }

template <int D>
int rows_mfma(int hg) {
  return hg == 4 ? kRowsMfma<D, 4> : hg == 2 ? kRowsMfma<D, 2> : kRowsMfma<D, 1>;
}

// rows per work unit of the kernel that launch() runs for (dtype, d, rep), with
// the head grouping launch_mfma_d picks
int rows_per_unit(int dtype, int d, int rep) {
  if (!use_mfma(dtype, d)) return 1;
  if (d == 512) {
    const int hg = pick_hg_d(512, rep);
    return hg == 4 ? kRowsWide<4> : hg == 2 ? kRowsWide<2> : kRowsWide<1>;
  }
  const int hg = pick_hg(rep);
  return d == 64 ? rows_mfma<64>(hg) : rows_mfma<128>(hg);
}

hipError_t launch(int dtype, int d, const SeqTable &t, const StepArgs &a, int units, hipStream_t s) {
  if (dtype == CPATTN_DT_BF16) {
    if (d == 64) return launch_mfma_d<64>(t, a, units, s);
    if (d == 128) return launch_mfma_d<128>(t, a, units, s);
    return launch_mfma_d<512>(t, a, units, s);
  }
  if (d == 64) return launch_generic<float, 64>(t, a, units, s);
  if (d == 128) return launch_generic<float, 128>(t, a, units, s);
  return launch_generic<float, 512>(t, a, units, s);
}

// Sequences go into launches of at most kMaxSeq sequences and 2^31 - 1
// workgroups. With a == nullptr the partition is only checked:
// hipErrorInvalidValue when a single sequence needs more workgroups than one
// launch holds. cpattn_ring_step_partial checks before it launches, so that an
// error leaves no work enqueued.
hipError_t run_launches(const cpattn_prefill_desc *desc, const StepArgs *a, hipStream_t stream) {
  const int cp = desc->cp;
  const int d = desc->head_dim;
  const int64_t *cu = desc->cu_seqlens;
  const int rep = desc->n_hq / desc->n_kv;
  const int rpu = rows_per_unit(desc->dtype, d, rep);
  const bool mfma = use_mfma(desc->dtype, d);
  const int64_t groups = mfma ? desc->n_hq / pick_hg_d(d, rep) : 1;
  int i = 0;
  int64_t row_off = 0;
  while (i < desc->num_seqs) {
    SeqTable t;
    t.n = 0;
    t.start[0] = 0;
    int64_t units = 0;
    while (i < desc->num_seqs && t.n < kMaxSeq) {
      const int64_t L = cu[i + 1] - cu[i];
      const int64_t c = (L + 2 * cp - 1) / (2 * cp);   // = L / (2 cp) unless padded
      const int64_t u = mfma ? 2 * ((c + rpu - 1) / rpu) : 2 * c;
      const int64_t blocks_after = (units + u) * groups;
      if (t.n > 0 && blocks_after > 0x7FFFFFFFLL) break;
      if (blocks_after > 0x7FFFFFFFLL) return hipErrorInvalidValue;
      t.c[t.n] = (int32_t)c;
      t.len[t.n] = (int32_t)L;
      t.row_off[t.n] = row_off;
      units += u;
      t.start[t.n + 1] = (int32_t)units;
      row_off += 2 * c;
      ++t.n;
      ++i;
    }
    if (a == nullptr || units == 0) continue;
    const hipError_t e = launch(desc->dtype, d, t, *a, (int)units, stream);
    if (e != hipSuccess) return e == hipErrorInvalidValue ? hipErrorLaunchFailure : e;
  }
  return hipSuccess;
}

}  // namespace
}  // namespace cpattn

int cpattn::check_launches(const cpattn_prefill_desc *desc) {
  return run_launches(desc, nullptr, nullptr) == hipSuccess ? CPATTN_OK : CPATTN_E_UNSUPPORTED;
}

int cpattn::check_prefill(const cpattn_prefill_desc *desc, int32_t rank, int32_t step) {
  if (desc == nullptr) return CPATTN_E_ARG;
  const int cp = desc->cp;
  if (cp < 1 || rank < 0 || rank >= cp || step < 0 || step >= cp) return CPATTN_E_ARG;
  if (desc->num_seqs < 0 || (desc->num_seqs > 0 && desc->cu_seqlens == nullptr)) return CPATTN_E_ARG;
  if (desc->n_hq < 1 || desc->n_kv < 1) return CPATTN_E_ARG;
  if (desc->dtype != CPATTN_DT_F32 && desc->dtype != CPATTN_DT_BF16) return CPATTN_E_ARG;
  if (!(desc->scale > 0.f) || !(desc->scale < __builtin_huge_valf())) return CPATTN_E_ARG;
  if (desc->n_hq % desc->n_kv != 0) return CPATTN_E_DIVISIBILITY;
  const int d = desc->head_dim;
  if (d != 64 && d != 128 && d != 512) return CPATTN_E_UNSUPPORTED;
  if (desc->n_hq > 65535) return CPATTN_E_UNSUPPORTED;
  // the 64 key rows of a tile lie within the 2^31-byte range of one copy resource
  if ((int64_t)desc->n_kv * d * 2 * 64 > 0x7FFFFFFFLL) return CPATTN_E_UNSUPPORTED;
  if (desc->padded != 0 && desc->padded != 1) return CPATTN_E_ARG;
  const int64_t *cu = desc->cu_seqlens;
  if (desc->num_seqs > 0 && cu[0] != 0) return CPATTN_E_ARG;
  for (int i = 0; i < desc->num_seqs; ++i) {
    const int64_t L = cu[i + 1] - cu[i];
    if (L < 0) return CPATTN_E_ARG;
    if (!desc->padded && L % (2 * (int64_t)cp) != 0) return CPATTN_E_DIVISIBILITY;
    if (L > (int64_t)1 << 30) return CPATTN_E_UNSUPPORTED;
  }
  return CPATTN_OK;
}

int64_t cpattn::local_rows(const cpattn_prefill_desc *desc) {
  const int64_t two_cp = 2 * (int64_t)desc->cp;
  int64_t rows = 0;
  for (int i = 0; i < desc->num_seqs; ++i)
    rows += 2 * ((desc->cu_seqlens[i + 1] - desc->cu_seqlens[i] + two_cp - 1) / two_cp);
  return rows;
}

extern "C" int cpattn_ring_step_partial(const cpattn_prefill_desc *desc, int32_t rank, int32_t step,
                                        const void *q_local, const void *k_blk, const void *v_blk,
                                        const cpattn_partial *dst, int32_t accumulate, hipStream_t stream) {
  using namespace cpattn;
  if (desc == nullptr || dst == nullptr) return CPATTN_E_ARG;
  const int chk = check_prefill(desc, rank, step);
  if (chk != CPATTN_OK) return chk;
  if (accumulate != 0 && accumulate != 1) return CPATTN_E_ARG;
  const int cp = desc->cp;
  const int64_t *cu = desc->cu_seqlens;
  const int64_t total = desc->num_seqs > 0 ? cu[desc->num_seqs] : 0;
  if (total == 0) return CPATTN_OK;
  if (q_local == nullptr || k_blk == nullptr || v_blk == nullptr || dst->m == nullptr || dst->den == nullptr ||
      dst->num == nullptr)
    return CPATTN_E_ARG;

  const int src = ((rank - step) % cp + cp) % cp;
  StepArgs a;
  a.q = q_local;
  a.k = k_blk;
  a.v = v_blk;
  a.m = dst->m;
  a.den = dst->den;
  a.num = dst->num;
  a.n_hq = desc->n_hq;
  a.n_kv = desc->n_kv;
  a.a_head = rank;
  a.a_tail = 2 * cp - 1 - rank;
  a.b_head = src;
  a.b_tail = 2 * cp - 1 - src;
  a.scale = desc->scale;
  a.accumulate = accumulate;

  if (run_launches(desc, nullptr, nullptr) != hipSuccess) return CPATTN_E_UNSUPPORTED;
  const hipError_t e = run_launches(desc, &a, stream);
  return e == hipSuccess ? CPATTN_OK : CPATTN_E_DEVICE;
}
