// K and V tiles staged in LDS for the MFMA kernels (gfx950): the swizzled
// [key][d] layout, the buffer-to-LDS copies that fill it, the transposed reads
// of V, and the LDS exchange of 32 x 32 score tiles. Shared by the ring-step and
// the decode kernels.
#pragma once

#include "kernels.h"

namespace cpattn {

// Rescale threshold of a running max in the exp2 domain: the numerator and
// denominator are only rescaled when the max grows by more than 2^8, so
// exp2(s - m_ref) stays below 256.
constexpr float kRescaleLog2 = 8.0f;

// A tile sits in LDS as it is in HBM, [key][W] bf16 with W columns of d per
// row, with the 16-byte chunks of each row permuted (chunk c of row r at
// position c ^ swizzle(r)).
//   K: read as the A operand of S^T = K Q^T, 16 bytes of one row per lane, 32
//     consecutive rows per wave; k_swizzle spreads 16 consecutive rows of one
//     chunk over 16 distinct bank groups.
//   V: read transposed by ds_read_b64_tr_b16 (v_fragment); a 16-lane group reads
//     8 bytes from each of 4 consecutive rows, and v_swizzle puts those 4 rows on
//     disjoint banks whether the LDS serves 32 or 64 banks per cycle.
template <int W>
__device__ __forceinline__ int k_swizzle(int row) {
  return (W == 64) ? ((row >> 1) & 7) : (row & 15);
}
template <int W>
__device__ __forceinline__ int v_swizzle(int row) {
  return (W == 64) ? 2 * (row & 3) : 4 * (row & 1) + 10 * ((row >> 1) & 1);
}

constexpr uint32_t kBufferWord3 = 0x00020000u;   // raw buffer resource word 3 on gfx9
constexpr int kWaitVmcnt0 = 0x0F70;              // s_waitcnt vmcnt(0), other counters unconstrained
// s_waitcnt immediate that waits until at most n vector memory operations of the
// wave are outstanding (gfx9 encoding: vmcnt bits 3:0 and 15:14)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitLgkm0 = 0xC07F;               // s_waitcnt lgkmcnt(0)

// Buffer resource of a tile: base at key row `row`, loads at or past
// rows_left * row_bytes return zeros.
__host__ __device__ __forceinline__ u32x4_t tile_words(const char *block, int64_t row, int rows_left, uint32_t row_bytes) {
  const int64_t lim = (int64_t)rows_left * row_bytes;
  const uint32_t nrec = (uint32_t)(lim < 0x7FFFFFFF ? lim : 0x7FFFFFFF);
  const uint64_t base = (uint64_t)(block + row * (int64_t)row_bytes);
  return u32x4_t{(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, nrec, kBufferWord3};
}

// The resource is uniform over the wave; readfirstlane keeps it in scalar
// registers, where the copy instruction needs it.
__device__ __forceinline__ u32x4_t uniform_words(u32x4_t r) {
  return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane(r[0]), (uint32_t)__builtin_amdgcn_readfirstlane(r[1]),
                 (uint32_t)__builtin_amdgcn_readfirstlane(r[2]), (uint32_t)__builtin_amdgcn_readfirstlane(r[3])};
}

// One buffer-to-LDS copy (buffer_load ... lds): lane L loads 16 bytes at byte
// offset `off` of the resource and the wave writes them to bytes [16L, 16L+16)
// of the 1 KB at `chunk` (M0). Written as inline assembly on purpose: the
// compiler tracks its own buffer-to-LDS copies and, unable to tell LDS ranges
// apart, makes the first LDS read after one wait for every outstanding vector
// load, which would expose the whole load latency at the top of each tile. The
// kernels wait for these copies themselves (s_waitcnt vmcnt). gfx9 asks for one
// wait state between a scalar write of M0 and an LDS DMA that reads it; the
// compiler inserts it for its own copies but cannot see that this one reads M0
// that way, so the s_nop is part of the copy.
__device__ __forceinline__ void dma_1k(uint32_t off, u32x4_t rs, __bf16 *chunk) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) __bf16 *)chunk);
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(rs), "{m0}"(lds));
#else
  (void)off; (void)rs; (void)chunk;
#endif
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// A operand of O^T = V^T P^T for k-step ks (16 keys) and the 32 columns
// [d0, d0 + 32) of a V tile with W columns per row: lane (m = lane % 32, h =
// lane / 32) needs V[key][d0 + m] for the keys 16 ks + 4 h + {0..3} (elements
// 0..3) and 16 ks + 8 + 4 h + {0..3} (elements 4..7), the order in which the
// S^T accumulator lays out the keys of the P fragment. ds_read_b64_tr_b16 gives
// lane i of a 16-lane group element e of the 8 bytes addressed by lane 4e + i/4,
// so when lane j of the group addresses row k0 + j/4 at column c0 + 4 (j % 4),
// lane i receives V[k0 .. k0 + 3][c0 + i]: one read per 4 keys, the second 8
// rows further on. d0 must be a multiple of 32.
template <int W>
__device__ __forceinline__ bf16x8_t v_fragment(const __bf16 *Vc, int ks, int d0) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const int row = 16 * ks + 4 * (lane >> 5) + (j >> 2);
  const int col = d0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const int off = row * W + 8 * ((col >> 3) ^ v_swizzle<W>(row)) + (col & 7);   // rows +8 share the swizzle
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const lds_i16x4 *p = (const lds_i16x4 *)(Vc + off);
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 2 * W));
  const i16x4_t both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8_t, both);
#else
  (void)Vc; (void)ks; (void)d0;
  return bf16x8_t{};
#endif
}

// Chunk permutation of a V tile read by v16_fragment: the 16 rows one
// transposed read of a wave touches land on distinct banks (checked for 32- and
// 64-bank LDS).
template <int W>
__device__ __forceinline__ int v16_swizzle(int row) {
  return (W == 64) ? 2 * ((row ^ (row >> 2)) & 1) + 4 * ((row >> 1) & 1) : 2 * (row & 7);
}

// The two transposed reads of v16_fragment at an address already computed
// (element offset of the lane's first read; the second is 16 rows further on).
template <int W>
__device__ __forceinline__ bf16x8_t v16_read(const __bf16 *p0) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const lds_i16x4 *p = (const lds_i16x4 *)p0;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * W));
  const i16x4_t both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8_t, both);
#else
  (void)p0;
  return bf16x8_t{};
#endif
}

// A operand of O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 for the 16 columns
// [16 db, 16 db + 16) of a 32-key V tile with W columns per row (chunks placed
// by v16_swizzle): lane (i = lane % 16, group gr = lane / 16) needs
// V[4 gr + 0..3][16 db + i] (elements 0..3) and V[16 + 4 gr + 0..3][16 db + i]
// (elements 4..7), the key order in which the S^T accumulators of two 16-key
// blocks lay out the P fragment. Two ds_read_b64_tr_b16, lane j of a group
// addressing row 4 gr + j / 4 at column 16 db + 4 (j % 4).
template <int W>
__device__ __forceinline__ bf16x8_t v16_fragment(const __bf16 *Vc, int db) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, gr = lane >> 4;
  const int row = 4 * gr + (i >> 2);
  const int cc = 16 * db + 4 * (i & 3);
  const int off = row * W + 8 * ((cc >> 3) ^ v16_swizzle<W>(row)) + (cc & 7);   // rows +16 share the swizzle
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const lds_i16x4 *p = (const lds_i16x4 *)(Vc + off);
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 4 * W));
  const i16x4_t both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8_t, both);
#else
  (void)Vc; (void)db;
  return bf16x8_t{};
#endif
}

// A 32 x 32 fp32 score tile of one wave in LDS, stored [quarter][lane] as
// float4 so that every 16-byte access of a wave covers 1 KB of consecutive
// banks.
__device__ __forceinline__ void put_scores(f32x4_t (*x)[64], const f32x16_t &s) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int g = 0; g < 4; ++g) x[g][lane] = f32x4_t{s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3]};
}

__device__ __forceinline__ f32x16_t get_scores(const f32x4_t (*x)[64]) {
  const int lane = threadIdx.x & 63;
  f32x16_t s;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4_t t = x[g][lane];
    s[4 * g] = t[0];
    s[4 * g + 1] = t[1];
    s[4 * g + 2] = t[2];
    s[4 * g + 3] = t[3];
  }
  return s;
}

// Tile geometry of flattened tile index t over the (up to two) key segments.
template <int BN>
struct Segs {
  int nseg;               // non-empty segments (0, 1 or 2)
  int n0;                 // tiles of segment 0
  int64_t row[2];         // first key row of each segment in the block
  int end[2];             // visible keys of each segment
  bool diag[2];
  __host__ __device__ __forceinline__ int seg(int t) const { return t < n0 ? 0 : 1; }
  __host__ __device__ __forceinline__ int k0(int t) const { return (t < n0 ? t : t - n0) * BN; }
  __host__ __device__ __forceinline__ int tiles() const {
    return n0 + (nseg > 1 ? (end[1] + BN - 1) / BN : 0);
  }
};

// The copy resources of the head_dim 512 kernels (ring step and decode), one per key row of a tile,
// walked tile by tile in scalar registers: for tile t (t0, t0 + 1, ...) and key
// row q, the 1 KB of one head at byte gbase of the row, based there with 1 KB
// in range when the row holds a visible key, and otherwise (rows past the
// segment's visible keys, tiles past the last) an empty range at the block
// start (the copy then writes zeros and touches no memory).
template <int BN>
struct RowWalk {
  int t, n0, ntiles;
  uint64_t blk;
  uint64_t addr, addr1;    // first key row of tile t; of the second segment's first tile
  int left, left1;         // visible keys from there to the segment's end
  uint32_t step;           // bytes of one tile
  __host__ __device__ __forceinline__ RowWalk(const Segs<BN> &sg, int ntiles_, const char *blk_, int t0, uint32_t rb)
      : t(t0), n0(sg.n0), ntiles(ntiles_), blk((uint64_t)(uintptr_t)blk_) {
    const int s = sg.seg(t0), k = sg.k0(t0);
    addr = blk + (uint64_t)((sg.row[s] + k) * (int64_t)rb);
    left = sg.end[s] - k;
    addr1 = blk + (uint64_t)(sg.row[1] * (int64_t)rb);
    left1 = sg.end[1];
    step = (uint32_t)BN * rb;
  }
  __host__ __device__ __forceinline__ void next() {
    ++t;
    if (t == n0) {
      addr = addr1;
      left = left1;
    } else {
      addr += step;
      left -= BN;
    }
  }
  // q * rb + gbase fits 32 bits: both callers reject key rows of 2^25 bytes or more
  __host__ __device__ __forceinline__ u32x4_t row(int q, uint32_t rb, uint32_t gbase) const {
    const bool ok = t < ntiles && q < left;
    const uint64_t base = ok ? addr + (uint32_t)((uint32_t)q * rb + gbase) : blk;
    return u32x4_t{(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, ok ? 1024u : 0u, kBufferWord3};
  }
};

}  // namespace cpattn
