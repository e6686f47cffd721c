// The path driven from C++ through include/cpattn.h alone: no Python, no torch.
// Device memory, copies and the stream come from the HIP runtime; every step of
// the method runs in libcpattn.
//
//   cp_attention_c prefill <in> <out>
//     in : int64 num_seqs, cp, n_hq, n_kv, head_dim; int64 cu_seqlens[num_seqs+1];
//          float32 scale (padded to 8 bytes); then bf16 q [T, n_hq, d], k and v
//          [T, n_kv, d] in global packed token order (T = cu_seqlens[num_seqs]).
//     Every rank's rows are gathered with cpattn_balanced_split, its pass-KV ring
//     runs as cp fused cpattn_ring_step_partial calls (the block of rank
//     (r - t) mod cp at step t), cpattn_merge finalizes it, and the rows are
//     scattered back to global order.
//     out: float32 out [T, n_hq, d], then float32 lse [T, n_hq].
//   cp_attention_c decode <in> <out>
//     in : int64 batch, kv_len, cp, n_hq, n_kv, head_dim; float32 scale (padded
//          to 8 bytes); bf16 q [b, n_hq, d], k and v [b, kv_len, n_kv, d].
//     The keys are cut into cp contiguous shards; cpattn_passq_decode runs with
//     a workspace of the size it asks for.
//     out: float32 out [b, n_hq, d], then float32 lse [b, n_hq].
//
// Before the real calls each mode makes one call the library must reject
// (rank = cp; a too small workspace) and checks the status. Exit status 0 on
// success; otherwise a message on stderr.
#include "cpattn.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#define HIP_OK(x)                                                                  \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(2);                                                                     \
    }                                                                              \
  } while (0)
#define CP_OK(x)                                                                   \
  do {                                                                             \
    int s_ = (x);                                                                  \
    if (s_ != CPATTN_OK) {                                                         \
      fprintf(stderr, "%s:%d: %s returned %d\n", __FILE__, __LINE__, #x, s_);      \
      exit(3);                                                                     \
    }                                                                              \
  } while (0)

static std::vector<char> read_file(const char *path) {
  FILE *f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    exit(2);
  }
  std::vector<char> buf;
  char tmp[1 << 16];
  size_t n;
  while ((n = fread(tmp, 1, sizeof tmp, f)) > 0) buf.insert(buf.end(), tmp, tmp + n);
  fclose(f);
  return buf;
}

struct Reader {
  const std::vector<char> &b;
  size_t at = 0;
  void take(void *dst, size_t n) {
    if (at + n > b.size()) {
      fprintf(stderr, "input file too short\n");
      exit(2);
    }
    memcpy(dst, b.data() + at, n);
    at += n;
  }
  int64_t i64() {
    int64_t v;
    take(&v, 8);
    return v;
  }
};

static void write_file(const char *path, const std::vector<float> &a, const std::vector<float> &b) {
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(a.data(), 4, a.size(), f) != a.size() || fwrite(b.data(), 4, b.size(), f) != b.size()) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(2);
  }
  fclose(f);
}

template <typename T>
static T *device_copy(const T *src, size_t n) {
  T *d = nullptr;
  HIP_OK(hipMalloc(reinterpret_cast<void **>(&d), n * sizeof(T) + 16));
  if (n) HIP_OK(hipMemcpy(d, src, n * sizeof(T), hipMemcpyHostToDevice));
  return d;
}

static float *device_floats(size_t n) {
  float *d = nullptr;
  HIP_OK(hipMalloc(reinterpret_cast<void **>(&d), n * sizeof(float) + 16));
  return d;
}

static int prefill(const char *in, const char *outp) {
  const std::vector<char> buf = read_file(in);
  Reader r{buf};
  const int64_t num_seqs = r.i64(), cp = r.i64(), n_hq = r.i64(), n_kv = r.i64(), d = r.i64();
  std::vector<int64_t> cu((size_t)num_seqs + 1);
  r.take(cu.data(), cu.size() * 8);
  float scale;
  r.take(&scale, 4);
  r.at += 4;
  const int64_t T = cu[(size_t)num_seqs];
  std::vector<uint16_t> q((size_t)(T * n_hq * d)), k((size_t)(T * n_kv * d)), v((size_t)(T * n_kv * d));
  r.take(q.data(), q.size() * 2);
  r.take(k.data(), k.size() * 2);
  r.take(v.data(), v.size() * 2);

  int64_t rows = 0;
  CP_OK(cpattn_local_rows(cu.data(), (int32_t)num_seqs, (int32_t)cp, 0, &rows));
  cpattn_prefill_desc desc;
  memset(&desc, 0, sizeof desc);
  desc.cp = (int32_t)cp;
  desc.num_seqs = (int32_t)num_seqs;
  desc.cu_seqlens = cu.data();
  desc.n_hq = (int32_t)n_hq;
  desc.n_kv = (int32_t)n_kv;
  desc.head_dim = (int32_t)d;
  desc.dtype = CPATTN_DT_BF16;
  desc.scale = scale;
  desc.padded = 0;

  // every rank's local rows, gathered on the host from the split
  std::vector<std::vector<int64_t>> pos((size_t)cp, std::vector<int64_t>((size_t)rows));
  std::vector<uint16_t *> qd((size_t)cp), kd((size_t)cp), vd((size_t)cp);
  std::vector<int64_t> cul((size_t)num_seqs + 1);
  for (int64_t rk = 0; rk < cp; ++rk) {
    CP_OK(cpattn_balanced_split(cu.data(), (int32_t)num_seqs, (int32_t)cp, (int32_t)rk, pos[(size_t)rk].data(),
                                cul.data()));
    std::vector<uint16_t> ql((size_t)(rows * n_hq * d)), kl((size_t)(rows * n_kv * d)), vl((size_t)(rows * n_kv * d));
    for (int64_t i = 0; i < rows; ++i) {
      const int64_t p = pos[(size_t)rk][(size_t)i];
      memcpy(&ql[(size_t)(i * n_hq * d)], &q[(size_t)(p * n_hq * d)], (size_t)(n_hq * d) * 2);
      memcpy(&kl[(size_t)(i * n_kv * d)], &k[(size_t)(p * n_kv * d)], (size_t)(n_kv * d) * 2);
      memcpy(&vl[(size_t)(i * n_kv * d)], &v[(size_t)(p * n_kv * d)], (size_t)(n_kv * d) * 2);
    }
    qd[(size_t)rk] = device_copy(ql.data(), ql.size());
    kd[(size_t)rk] = device_copy(kl.data(), kl.size());
    vd[(size_t)rk] = device_copy(vl.data(), vl.size());
  }

  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  cpattn_partial acc = {device_floats((size_t)(rows * n_hq)), device_floats((size_t)(rows * n_hq)),
                        device_floats((size_t)(rows * n_hq * d))};
  float *out = device_floats((size_t)(rows * n_hq * d));
  float *lse = device_floats((size_t)(rows * n_hq));

  // a call the library must reject: rank outside [0, cp)
  if (cpattn_ring_step_partial(&desc, (int32_t)cp, 0, qd[0], kd[0], vd[0], &acc, 0, s) != CPATTN_E_ARG) {
    fprintf(stderr, "rank = cp was not rejected with CPATTN_E_ARG\n");
    return 4;
  }

  std::vector<float> out_g((size_t)(T * n_hq * d)), lse_g((size_t)(T * n_hq));
  std::vector<float> ol((size_t)(rows * n_hq * d)), ll((size_t)(rows * n_hq));
  for (int64_t rk = 0; rk < cp; ++rk) {
    for (int64_t t = 0; t < cp; ++t) {
      const int64_t j = ((rk - t) % cp + cp) % cp;   // the block in hand at step t
      CP_OK(cpattn_ring_step_partial(&desc, (int32_t)rk, (int32_t)t, qd[(size_t)rk], kd[(size_t)j], vd[(size_t)j],
                                     &acc, t > 0 ? 1 : 0, s));
    }
    CP_OK(cpattn_merge(rows, (int32_t)n_hq, (int32_t)d, nullptr, 0, &acc, out, lse, s));
    HIP_OK(hipMemcpyAsync(ol.data(), out, ol.size() * 4, hipMemcpyDeviceToHost, s));
    HIP_OK(hipMemcpyAsync(ll.data(), lse, ll.size() * 4, hipMemcpyDeviceToHost, s));
    HIP_OK(hipStreamSynchronize(s));
    for (int64_t i = 0; i < rows; ++i) {
      const int64_t p = pos[(size_t)rk][(size_t)i];
      memcpy(&out_g[(size_t)(p * n_hq * d)], &ol[(size_t)(i * n_hq * d)], (size_t)(n_hq * d) * 4);
      memcpy(&lse_g[(size_t)(p * n_hq)], &ll[(size_t)(i * n_hq)], (size_t)n_hq * 4);
    }
  }
  write_file(outp, out_g, lse_g);
  for (int64_t rk = 0; rk < cp; ++rk) {
    HIP_OK(hipFree(qd[(size_t)rk]));
    HIP_OK(hipFree(kd[(size_t)rk]));
    HIP_OK(hipFree(vd[(size_t)rk]));
  }
  HIP_OK(hipFree(acc.m));
  HIP_OK(hipFree(acc.den));
  HIP_OK(hipFree(acc.num));
  HIP_OK(hipFree(out));
  HIP_OK(hipFree(lse));
  HIP_OK(hipStreamDestroy(s));
  return 0;
}

static int decode(const char *in, const char *outp) {
  const std::vector<char> buf = read_file(in);
  Reader r{buf};
  const int64_t b = r.i64(), S = r.i64(), cp = r.i64(), n_hq = r.i64(), n_kv = r.i64(), d = r.i64();
  float scale;
  r.take(&scale, 4);
  r.at += 4;
  std::vector<uint16_t> q((size_t)(b * n_hq * d)), k((size_t)(b * S * n_kv * d)), v((size_t)(b * S * n_kv * d));
  r.take(q.data(), q.size() * 2);
  r.take(k.data(), k.size() * 2);
  r.take(v.data(), v.size() * 2);
  const int64_t n = S / cp;
  const int64_t row = n_kv * d;   // elements of one key row

  // shard s: keys [s n, (s + 1) n) of every batch entry, [b, n, n_kv, d]
  std::vector<const void *> ks((size_t)cp), vs((size_t)cp);
  std::vector<uint16_t *> kd((size_t)cp), vd((size_t)cp);
  for (int64_t sh = 0; sh < cp; ++sh) {
    std::vector<uint16_t> kl((size_t)(b * n * row)), vl((size_t)(b * n * row));
    for (int64_t bi = 0; bi < b; ++bi) {
      memcpy(&kl[(size_t)(bi * n * row)], &k[(size_t)((bi * S + sh * n) * row)], (size_t)(n * row) * 2);
      memcpy(&vl[(size_t)(bi * n * row)], &v[(size_t)((bi * S + sh * n) * row)], (size_t)(n * row) * 2);
    }
    kd[(size_t)sh] = device_copy(kl.data(), kl.size());
    vd[(size_t)sh] = device_copy(vl.data(), vl.size());
    ks[(size_t)sh] = kd[(size_t)sh];
    vs[(size_t)sh] = vd[(size_t)sh];
  }
  uint16_t *qd = device_copy(q.data(), q.size());
  cpattn_decode_desc desc;
  memset(&desc, 0, sizeof desc);
  desc.batch = (int32_t)b;
  desc.cp = (int32_t)cp;
  desc.kv_len = S;
  desc.n_hq = (int32_t)n_hq;
  desc.n_kv = (int32_t)n_kv;
  desc.head_dim = (int32_t)d;
  desc.dtype = CPATTN_DT_BF16;
  desc.scale = scale;

  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  cpattn_partial sp = {device_floats((size_t)(cp * b * n_hq)), device_floats((size_t)(cp * b * n_hq)),
                       device_floats((size_t)(cp * b * n_hq * d))};
  float *out = device_floats((size_t)(b * n_hq * d));
  float *lse = device_floats((size_t)(b * n_hq));
  size_t need = 0;
  CP_OK(cpattn_passq_decode(&desc, qd, ks.data(), vs.data(), &sp, out, lse, nullptr, &need, s));
  void *ws = nullptr;
  HIP_OK(hipMalloc(&ws, need + 16));
  if (need > 0) {
    // a call the library must reject: a workspace one byte short
    size_t small = need - 1;
    if (cpattn_passq_decode(&desc, qd, ks.data(), vs.data(), &sp, out, lse, ws, &small, s) != CPATTN_E_WORKSPACE) {
      fprintf(stderr, "a short workspace was not rejected with CPATTN_E_WORKSPACE\n");
      return 4;
    }
  }
  size_t have = need;
  CP_OK(cpattn_passq_decode(&desc, qd, ks.data(), vs.data(), &sp, out, lse, ws, &have, s));
  std::vector<float> o((size_t)(b * n_hq * d)), l((size_t)(b * n_hq));
  HIP_OK(hipMemcpyAsync(o.data(), out, o.size() * 4, hipMemcpyDeviceToHost, s));
  HIP_OK(hipMemcpyAsync(l.data(), lse, l.size() * 4, hipMemcpyDeviceToHost, s));
  HIP_OK(hipStreamSynchronize(s));
  write_file(outp, o, l);
  for (int64_t sh = 0; sh < cp; ++sh) {
    HIP_OK(hipFree(kd[(size_t)sh]));
    HIP_OK(hipFree(vd[(size_t)sh]));
  }
  HIP_OK(hipFree(qd));
  HIP_OK(hipFree(ws));
  HIP_OK(hipFree(sp.m));
  HIP_OK(hipFree(sp.den));
  HIP_OK(hipFree(sp.num));
  HIP_OK(hipFree(out));
  HIP_OK(hipFree(lse));
  HIP_OK(hipStreamDestroy(s));
  return 0;
}

int main(int argc, char **argv) {
  if (argc != 4) {
    fprintf(stderr, "usage: %s prefill|decode <in> <out>\n", argv[0]);
    return 1;
  }
  if (strcmp(argv[1], "prefill") == 0) return prefill(argv[2], argv[3]);
  if (strcmp(argv[1], "decode") == 0) return decode(argv[2], argv[3]);
  fprintf(stderr, "unknown mode %s\n", argv[1]);
  return 1;
}
