// Pass-KV ring of one rank on one GPU with the transfer made explicit
// (G5 context-parallel modelling spec: Definitions table, "Pass-KV" and "Ring
// step"; Rationale, the dependency contract of the ring; Acceptance,
// "overlap effective").
//
// cpattn_ring_pass stands in for the point-to-point transfer of a KV block
// between neighbouring ranks: either a copy on one of the GPU's DMA (SDMA)
// engines, which uses no compute unit (as a transfer over xGMI does), or a
// copy kernel restricted to a caller-chosen number of workgroups, so that it
// takes roughly one link's worth of bandwidth. The engine copy is the one that
// truly runs beside a ring step: a copy kernel on another stream only gets
// compute units once the ring step's grid has been fully dispatched.
//
// cpattn_ring_prefill_overlapped enqueues the whole ring of one rank on two
// streams, with HIP events carrying exactly the edges of the contract:
//   compute(i)  waits for transfer(i-1)   (the block it reads has arrived),
//   transfer(i) follows transfer(i-1)     (it forwards what that one delivered),
//   transfer(i) waits for compute(i+1-n)  (with n receive buffers, it
//                                          overwrites the buffer that compute
//                                          read; i+1-n >= 1),
// and no edge from compute(i) to transfer(i), so a step's transfer runs
// concurrently with that step's compute.
#include "kernels.h"

namespace cpattn {
namespace {

constexpr int kLinkThreads = 256;
constexpr int kLinkUnroll = 4;
constexpr int kMaxLinkGroups = 65535;
constexpr int kMaxRecv = 16;   // receive buffers per rank

// Grid-stride copy of n16 16-byte words; kLinkUnroll loads are in flight per
// thread before the stores, and the data bypasses the caches on both sides.
__global__ __launch_bounds__(kLinkThreads) void link_copy(const u32x4_t *__restrict__ src,
                                                          u32x4_t *__restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kLinkThreads;
  int64_t i = (int64_t)blockIdx.x * kLinkThreads + threadIdx.x;
  for (; i + (kLinkUnroll - 1) * stride < n16; i += kLinkUnroll * stride) {
    u32x4_t v[kLinkUnroll];
#pragma unroll
    for (int u = 0; u < kLinkUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kLinkUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

int validate_pass(const void *src, void *dst, int64_t bytes, int32_t workgroups) {
  if (bytes < 0 || workgroups < 0 || workgroups > kMaxLinkGroups) return CPATTN_E_ARG;
  if (bytes == 0) return CPATTN_OK;
  if (src == nullptr || dst == nullptr) return CPATTN_E_ARG;
  if ((bytes & 15) != 0 || ((uintptr_t)src & 15) != 0 || ((uintptr_t)dst & 15) != 0) return CPATTN_E_ARG;
  const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
  if (s < d + (uintptr_t)bytes && d < s + (uintptr_t)bytes) return CPATTN_E_ARG;   // ranges overlap
  return CPATTN_OK;
}

hipError_t launch_pass(const void *src, void *dst, int64_t bytes, int32_t workgroups, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (workgroups == 0) return hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyDeviceToDeviceNoCU, stream);
  const int64_t n16 = bytes / 16;
  const int64_t need = (n16 + kLinkThreads - 1) / kLinkThreads;
  const unsigned grid = (unsigned)(need < workgroups ? need : workgroups);
  hipLaunchKernelGGL(link_copy, dim3(grid), dim3(kLinkThreads), 0, stream, (const u32x4_t *)src, (u32x4_t *)dst,
                     n16);
  return hipGetLastError();
}

struct Events {
  hipEvent_t *e = nullptr;
  int n = 0;
  explicit Events(int count) : e(new hipEvent_t[count]()), n(0) {
    for (; n < count; ++n)
      if (hipEventCreateWithFlags(&e[n], hipEventDisableTiming) != hipSuccess) break;
  }
  bool ok(int count) const { return n == count; }
  ~Events() {
    // an event still pending on a stream is released once it completes
    for (int i = 0; i < n; ++i) (void)hipEventDestroy(e[i]);
    delete[] e;
  }
};

}  // namespace
}  // namespace cpattn

extern "C" int cpattn_ring_pass(const void *src, void *dst, int64_t bytes, int32_t workgroups, hipStream_t stream) {
  using namespace cpattn;
  const int rc = validate_pass(src, dst, bytes, workgroups);
  if (rc != CPATTN_OK) return rc;
  return launch_pass(src, dst, bytes, workgroups, stream) == hipSuccess ? CPATTN_OK : CPATTN_E_DEVICE;
}

extern "C" int cpattn_ring_prefill_overlapped(const cpattn_prefill_desc *desc, int32_t rank, const void *q_local,
                                              const void *const *k_blocks, const void *const *v_blocks,
                                              void *const *k_recv, void *const *v_recv, int32_t n_recv,
                                              const cpattn_partial *acc, int32_t link_workgroups, hipStream_t compute,
                                              hipStream_t transfer) {
  using namespace cpattn;
  if (desc == nullptr || acc == nullptr || k_blocks == nullptr || v_blocks == nullptr) return CPATTN_E_ARG;
  const int chk = check_prefill(desc, rank, 0);
  if (chk != CPATTN_OK) return chk;
  const int cp = desc->cp;
  if (link_workgroups < 0 || link_workgroups > kMaxLinkGroups) return CPATTN_E_ARG;
  if (cp > 1 && (k_recv == nullptr || v_recv == nullptr || n_recv < 2 || n_recv > kMaxRecv)) return CPATTN_E_ARG;
  const int64_t total = desc->num_seqs > 0 ? desc->cu_seqlens[desc->num_seqs] : 0;
  if (total == 0) return CPATTN_OK;
  if (q_local == nullptr || acc->m == nullptr || acc->den == nullptr || acc->num == nullptr) return CPATTN_E_ARG;
  if (k_blocks[rank] == nullptr || v_blocks[rank] == nullptr) return CPATTN_E_ARG;
  const int64_t elem = desc->dtype == CPATTN_DT_BF16 ? 2 : 4;
  const int64_t block_bytes = local_rows(desc) * desc->n_kv * desc->head_dim * elem;
  if (cp > 1) {
    // every receive buffer is aligned, disjoint from every source block and from
    // every other receive buffer
    for (int j = 0; j < cp; ++j)
      for (int b = 0; b < n_recv; ++b)
        if (validate_pass(k_blocks[j], k_recv[b], block_bytes, 1) != CPATTN_OK ||
            validate_pass(k_blocks[j], v_recv[b], block_bytes, 1) != CPATTN_OK ||
            validate_pass(v_blocks[j], k_recv[b], block_bytes, 1) != CPATTN_OK ||
            validate_pass(v_blocks[j], v_recv[b], block_bytes, 1) != CPATTN_OK)
          return CPATTN_E_ARG;
    for (int x = 0; x < 2 * n_recv; ++x)
      for (int y = x + 1; y < 2 * n_recv; ++y) {
        void *const bx = x < n_recv ? k_recv[x] : v_recv[x - n_recv];
        void *const by = y < n_recv ? k_recv[y] : v_recv[y - n_recv];
        if (validate_pass(bx, by, block_bytes, 1) != CPATTN_OK) return CPATTN_E_ARG;
      }
  }

  Events comp(cp), comm(cp);
  if (!comp.ok(cp) || !comm.ok(cp)) return CPATTN_E_DEVICE;
  for (int i = 0; i < cp; ++i) {
    // compute(i) on the block in hand: the rank's own at step 0, then the one
    // transfer(i-1) delivered into receive buffer (i-1) % n_recv
    if (i > 0 && hipStreamWaitEvent(compute, comm.e[i - 1], 0) != hipSuccess) return CPATTN_E_DEVICE;
    const void *k = i == 0 ? k_blocks[rank] : k_recv[(i - 1) % n_recv];
    const void *v = i == 0 ? v_blocks[rank] : v_recv[(i - 1) % n_recv];
    const int rc = cpattn_ring_step_partial(desc, rank, i, q_local, k, v, acc, i > 0 ? 1 : 0, compute);
    if (rc != CPATTN_OK) return rc;
    if (hipEventRecord(comp.e[i], compute) != hipSuccess) return CPATTN_E_DEVICE;
    if (i == cp - 1) break;
    // transfer(i): the block of rank (rank - i - 1) mod cp into receive buffer
    // i % n_recv, last read by compute(i + 1 - n_recv)
    const int war = i + 1 - n_recv;
    if (war >= 1 && hipStreamWaitEvent(transfer, comp.e[war], 0) != hipSuccess) return CPATTN_E_DEVICE;
    const int src = ((rank - i - 1) % cp + cp) % cp;
    if (launch_pass(k_blocks[src], k_recv[i % n_recv], block_bytes, link_workgroups, transfer) != hipSuccess ||
        launch_pass(v_blocks[src], v_recv[i % n_recv], block_bytes, link_workgroups, transfer) != hipSuccess)
      return CPATTN_E_DEVICE;
    if (hipEventRecord(comm.e[i], transfer) != hipSuccess) return CPATTN_E_DEVICE;
  }
  return CPATTN_OK;
}
