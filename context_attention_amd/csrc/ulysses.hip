// All-to-all of a Ulysses group, emulated on one GPU (G5 context-parallel
// modelling spec, "Limitations and follow-up work": Ulysses and hybrid CP are
// the follow-up after the pass-KV ring; "Goals and non-goals": the spec itself
// leaves the All-to-All scheme out).
//
// A Ulysses group of n ranks holds a sequence either sharded by tokens (rank j:
// `rows` token rows of every one of the n_heads heads) or sharded by heads
// (rank i: all n * rows token rows of heads [i hn, (i + 1) hn), hn = n_heads / n).
// The all-to-all moves between the two: in the head-sharded layout the rows of
// rank j come j-th, in their own order, so
//   seq -> head:  dst[i][j rows + r][h] = src[j][r][i hn + h]
//   head -> seq:  dst[j][r][i hn + h]   = src[i][j rows + r][h]
// for every rank pair (i, j), row r < rows and head h < hn, a head being
// head_bytes bytes. Either way every destination row segment (the hn heads of
// one token row) is one contiguous run of hn * head_bytes bytes in the source:
// the exchange is n * n * rows copies of that length, which one grid-stride
// kernel does word by word (16-byte words when every length and pointer allows,
// else 4-byte words).
#include "kernels.h"

namespace cpattn {
namespace {

constexpr int kA2aThreads = 256;
constexpr int kMaxA2aRanks = 64;

struct A2aArgs {
  const char *src[kMaxA2aRanks];
  char *dst[kMaxA2aRanks];
  int32_t n;            // ranks
  int32_t direction;    // 0: seq -> head, 1: head -> seq
  int64_t rows;         // token rows per rank in the sequence-sharded layout
  int64_t seg_words;    // words of one row segment (hn * head_bytes / word)
  int64_t row_words;    // words of one full token row (n_heads * head_bytes / word)
  int64_t words;        // total words moved: n * n * rows * seg_words
};

// Source and destination word offsets (and ranks) of word w of the exchange.
// Word w belongs to segment s = w / seg_words, which is (destination rank i of
// the head layout, source rank j of the sequence layout, row r); the segment
// is row j rows + r of head-rank i and the heads [i hn, (i + 1) hn) of row r
// of sequence-rank j.
struct A2aWord {
  int32_t src_rank, dst_rank;
  int64_t src_off, dst_off;   // in words
};

__host__ __device__ __forceinline__ A2aWord a2a_word(const A2aArgs &a, int64_t w) {
  const int64_t seg = w / a.seg_words, e = w - seg * a.seg_words;
  const int64_t r = seg % a.rows;
  const int64_t ij = seg / a.rows;
  const int32_t j = (int32_t)(ij % a.n), i = (int32_t)(ij / a.n);
  const int64_t head_off = (j * a.rows + r) * a.seg_words + e;    // in head-rank i's buffer
  const int64_t seq_off = r * a.row_words + i * a.seg_words + e;  // in sequence-rank j's buffer
  A2aWord o;
  if (a.direction == 0) {
    o.src_rank = j; o.src_off = seq_off;
    o.dst_rank = i; o.dst_off = head_off;
  } else {
    o.src_rank = i; o.src_off = head_off;
    o.dst_rank = j; o.dst_off = seq_off;
  }
  return o;
}

template <typename W>
__global__ __launch_bounds__(kA2aThreads) void a2a_copy(A2aArgs a) {
  const int64_t stride = (int64_t)gridDim.x * kA2aThreads;
  for (int64_t w = (int64_t)blockIdx.x * kA2aThreads + threadIdx.x; w < a.words; w += stride) {
    const A2aWord o = a2a_word(a, w);
    const W v = reinterpret_cast<const W *>(a.src[o.src_rank])[o.src_off];
    reinterpret_cast<W *>(a.dst[o.dst_rank])[o.dst_off] = v;
  }
}

// Checks of cpattn_ulysses_all_to_all in the order of its contract; fills the
// kernel arguments and the word size (4 or 16) on success.
int a2a_prepare(int32_t n, int64_t rows, int32_t n_heads, int64_t head_bytes, const void *const *src,
                void *const *dst, int32_t direction, A2aArgs &a, int &word) {
  if (n < 1 || rows < 0 || n_heads < 1 || head_bytes <= 0 || (direction != 0 && direction != 1)) return CPATTN_E_ARG;
  if (n > kMaxA2aRanks) return CPATTN_E_UNSUPPORTED;
  if (n_heads % n != 0) return CPATTN_E_DIVISIBILITY;
  if (head_bytes % 4 != 0) return CPATTN_E_ARG;
  if (src == nullptr || dst == nullptr) return CPATTN_E_ARG;
  const int64_t hn = n_heads / n;
  if (rows > 0 && (int64_t)n_heads > INT64_MAX / head_bytes / rows) return CPATTN_E_UNSUPPORTED;
  const int64_t bytes = rows * n_heads * head_bytes;   // every buffer, either layout
  if (bytes > INT64_MAX / n) return CPATTN_E_UNSUPPORTED;
  bool a16 = (hn * head_bytes) % 16 == 0;
  for (int k = 0; k < n; ++k) {
    if (bytes > 0 && (src[k] == nullptr || dst[k] == nullptr)) return CPATTN_E_ARG;
    if (((uintptr_t)src[k] & 3) != 0 || ((uintptr_t)dst[k] & 3) != 0) return CPATTN_E_ARG;
    a16 = a16 && ((uintptr_t)src[k] & 15) == 0 && ((uintptr_t)dst[k] & 15) == 0;
  }
  if (bytes > 0) {
    // no destination range overlaps another destination or any source
    for (int x = 0; x < n; ++x) {
      const uintptr_t d0 = (uintptr_t)dst[x], d1 = d0 + (uintptr_t)bytes;
      for (int y = 0; y < n; ++y) {
        const uintptr_t s0 = (uintptr_t)src[y], s1 = s0 + (uintptr_t)bytes;
        if (d0 < s1 && s0 < d1) return CPATTN_E_ARG;
        if (y != x) {
          const uintptr_t e0 = (uintptr_t)dst[y], e1 = e0 + (uintptr_t)bytes;
          if (d0 < e1 && e0 < d1) return CPATTN_E_ARG;
        }
      }
    }
  }
  word = a16 ? 16 : 4;
  for (int k = 0; k < n; ++k) {
    a.src[k] = reinterpret_cast<const char *>(src[k]);
    a.dst[k] = reinterpret_cast<char *>(dst[k]);
  }
  a.n = n;
  a.direction = direction;
  a.rows = rows;
  a.seg_words = hn * head_bytes / word;
  a.row_words = (int64_t)n_heads * head_bytes / word;
  a.words = (int64_t)n * n * rows * a.seg_words;
  return CPATTN_OK;
}

}  // namespace
}  // namespace cpattn

extern "C" int cpattn_ulysses_all_to_all(int32_t n, int64_t rows, int32_t n_heads, int64_t head_bytes,
                                         const void *const *src, void *const *dst, int32_t direction,
                                         hipStream_t stream) {
  using namespace cpattn;
  A2aArgs a;
  int word = 0;
  const int rc = a2a_prepare(n, rows, n_heads, head_bytes, src, dst, direction, a, word);
  if (rc != CPATTN_OK) return rc;
  if (a.words == 0) return CPATTN_OK;
  // about 8 grid-stride rounds per thread once the exchange is large
  const int64_t want = (a.words + kA2aThreads * 8 - 1) / (kA2aThreads * 8);
  const unsigned blocks = (unsigned)(want < 1 ? 1 : want > 65536 ? 65536 : want);
  if (word == 16)
    hipLaunchKernelGGL(a2a_copy<u32x4_t>, dim3(blocks), dim3(kA2aThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(a2a_copy<uint32_t>, dim3(blocks), dim3(kA2aThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? CPATTN_OK : CPATTN_E_DEVICE;
}
