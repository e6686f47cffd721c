// Host-only entry points of cpattn: the balanced chunk split (and its padded
// form for lengths not divisible by 2*cp) and the byte / FLOP / memory account. Plain C++ with no GPU code, so it builds with
// g++ as well as with hipcc.
#include "cpattn.h"

#include <cstring>

namespace {

// Validates cu_seqlens and the divisibility of every length by `div`.
int check_seqlens(const int64_t *cu, int32_t n, int64_t div) {
  if (n < 0) return CPATTN_E_ARG;
  if (cu == nullptr) return CPATTN_E_ARG;
  if (cu[0] != 0) return CPATTN_E_ARG;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t L = cu[i + 1] - cu[i];
    if (L < 0) return CPATTN_E_ARG;
    if (L % div != 0) return CPATTN_E_DIVISIBILITY;
  }
  return CPATTN_OK;
}

// Checked int64 arithmetic: each helper sets *ok = false on overflow.
struct Checked {
  bool ok = true;
  int64_t mul(int64_t a, int64_t b) {
    int64_t r = 0;
    if (__builtin_mul_overflow(a, b, &r)) ok = false;
    return r;
  }
  int64_t add(int64_t a, int64_t b) {
    int64_t r = 0;
    if (__builtin_add_overflow(a, b, &r)) ok = false;
    return r;
  }
  int64_t mul(std::initializer_list<int64_t> xs) {
    int64_t r = 1;
    for (int64_t x : xs) r = mul(r, x);
    return r;
  }
};

}  // namespace

extern "C" int cpattn_balanced_split(const int64_t *cu_seqlens, int32_t num_seqs, int32_t cp,
                                     int32_t rank, int64_t *positions, int64_t *cu_local) {
  // Definitions table, "Balanced chunk split": 2*cp chunks per sequence, rank r
  // holds the head/tail pair (chunk r, chunk 2cp-1-r).
  if (cp < 1 || rank < 0 || rank >= cp) return CPATTN_E_ARG;
  if (positions == nullptr || cu_local == nullptr) return CPATTN_E_ARG;
  const int rc = check_seqlens(cu_seqlens, num_seqs, 2 * (int64_t)cp);
  if (rc != CPATTN_OK) return rc;
  int64_t w = 0;
  cu_local[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t start = cu_seqlens[i];
    const int64_t c = (cu_seqlens[i + 1] - start) / (2 * (int64_t)cp);
    const int64_t head = start + (int64_t)rank * c;
    const int64_t tail = start + (int64_t)(2 * cp - 1 - rank) * c;
    for (int64_t x = 0; x < c; ++x) positions[w++] = head + x;
    for (int64_t x = 0; x < c; ++x) positions[w++] = tail + x;
    cu_local[i + 1] = cu_local[i] + 2 * c;
  }
  return CPATTN_OK;
}

extern "C" int cpattn_balanced_split_padded(const int64_t *cu_seqlens, int32_t num_seqs, int32_t cp,
                                            int32_t rank, int64_t *positions, int64_t *cu_local) {
  // the split of cpattn_balanced_split over sequences padded to a multiple of
  // 2*cp; slots past the true length are pad rows (-1)
  if (cp < 1 || rank < 0 || rank >= cp) return CPATTN_E_ARG;
  if (positions == nullptr || cu_local == nullptr) return CPATTN_E_ARG;
  const int rc = check_seqlens(cu_seqlens, num_seqs, 1);
  if (rc != CPATTN_OK) return rc;
  const int64_t two_cp = 2 * (int64_t)cp;
  int64_t w = 0;
  cu_local[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t start = cu_seqlens[i];
    const int64_t L = cu_seqlens[i + 1] - start;
    const int64_t c = (L + two_cp - 1) / two_cp;
    const int64_t chunks[2] = {(int64_t)rank * c, (two_cp - 1 - rank) * c};
    for (const int64_t first : chunks)
      for (int64_t x = 0; x < c; ++x) positions[w++] = (first + x < L) ? start + first + x : -1;
    cu_local[i + 1] = cu_local[i] + 2 * c;
  }
  return CPATTN_OK;
}

extern "C" int cpattn_local_rows(const int64_t *cu_seqlens, int32_t num_seqs, int32_t cp, int32_t padded,
                                 int64_t *rows) {
  // rows of one rank's local buffers: sum over sequences of 2 c_i, with
  // c_i = L_i / (2 cp), or ceil(L_i / (2 cp)) in the padded layout
  if (cp < 1 || rows == nullptr || (padded != 0 && padded != 1)) return CPATTN_E_ARG;
  const int64_t two_cp = 2 * (int64_t)cp;
  const int rc = check_seqlens(cu_seqlens, num_seqs, padded ? 1 : two_cp);
  if (rc != CPATTN_OK) return rc;
  int64_t r = 0;
  for (int32_t i = 0; i < num_seqs; ++i) r += 2 * ((cu_seqlens[i + 1] - cu_seqlens[i] + two_cp - 1) / two_cp);
  *rows = r;
  return CPATTN_OK;
}

extern "C" int cpattn_account(const cpattn_account_in *in, cpattn_account_out *out) {
  if (in == nullptr || out == nullptr) return CPATTN_E_ARG;
  const int64_t cp = in->cp;
  if (cp < 1 || in->n_hq < 1 || in->n_kv < 1 || in->head_dim < 1 || in->dtype_bytes < 1 ||
      in->c_kv < 0 || in->d_model < 0 || in->layers_local < 1 || in->batch < 0 || in->kv_len < 0)
    return CPATTN_E_ARG;
  if (in->n_hq % in->n_kv != 0) return CPATTN_E_DIVISIBILITY;
  if (in->cu_seqlens != nullptr) {
    const int rc = check_seqlens(in->cu_seqlens, in->num_seqs, 2 * cp);
    if (rc != CPATTN_OK) return rc;
  }
  if (in->kv_len > 0 && in->kv_len % cp != 0) return CPATTN_E_DIVISIBILITY;

  Checked ck;
  cpattn_account_out r;
  std::memset(&r, 0, sizeof(r));
  const int64_t dh = in->head_dim, hq = in->n_hq, s = in->dtype_bytes;
  // Definitions table: c_kv already counts K and V; d is the model hidden size.
  const int64_t c_kv = in->c_kv ? in->c_kv : ck.mul({2, (int64_t)in->n_kv, dh, s});
  const int64_t d = in->d_model ? in->d_model : ck.mul(hq, dh);
  r.ring_steps = cp;
  r.p2p_ops = cp - 1;

  if (in->cu_seqlens != nullptr) {
    const int64_t S = in->cu_seqlens[in->num_seqs];
    int64_t f_attn = 0, pairs0 = 0, pairsN = 0;
    for (int32_t i = 0; i < in->num_seqs; ++i) {
      const int64_t L = in->cu_seqlens[i + 1] - in->cu_seqlens[i];
      const int64_t c = L / (2 * cp);
      f_attn = ck.add(f_attn, ck.mul({2, hq, dh, L, L}));
      const int64_t cc2 = ck.mul({2, c, c});
      pairsN = ck.add(pairsN, cc2);
      pairs0 = ck.add(pairs0, ck.add(cc2, c));
    }
    r.tokens_per_rank = S / cp;
    // eq. g5cp-passkv-bytes: (cp-1) * S/cp * c_kv, one S/cp * c_kv block per step.
    r.passkv_bytes_per_step = cp > 1 ? ck.mul(S / cp, c_kv) : 0;
    r.passkv_bytes_per_rank = ck.mul({cp - 1, S / cp, c_kv});
    r.attn_flops = f_attn;
    // eq. g5cp-step-flops: F_step = F_attn / cp^2 (exact: each L_i is a multiple of 2cp).
    r.step_flops = f_attn / (cp * cp);
    r.rank_flops = f_attn / cp;
    r.step0_flops_exact = ck.mul({4, dh, hq, pairs0});
    r.stepN_flops_exact = ck.mul({4, dh, hq, pairsN});
    r.rank_flops_exact = ck.add(r.step0_flops_exact, ck.mul(cp - 1, r.stepN_flops_exact));
    // Formulas: per-rank KV memory b * S * c_kv * L_local / cp (b folded into S).
    r.kv_bytes_per_rank = ck.mul({S, c_kv, in->layers_local}) / cp;
  }
  if (in->kv_len > 0) {
    const int64_t b = in->batch, S = in->kv_len;
    // Formulas: pass-Q dispatch b*d*s and reduce b*(d + 2 n_h)*s; Constraints: no
    // transfer at cp = 1.
    r.passq_dispatch_bytes = cp > 1 ? ck.mul({b, d, s}) : 0;
    r.passq_reduce_bytes = cp > 1 ? ck.mul({b, ck.add(d, 2 * hq), s}) : 0;
    r.decode_kv_bytes_total = ck.mul({b, S, c_kv, in->layers_local});
    r.decode_kv_bytes_per_rank = r.decode_kv_bytes_total / cp;
    r.decode_flops = ck.mul({4, b, hq, dh, S});
  }
  if (!ck.ok) return CPATTN_E_OVERFLOW;
  *out = r;
  return CPATTN_OK;
}

extern "C" const char *cpattn_version(void) { return "cpattn 0.2.0 gfx950"; }
