// Pass-KV ring of a CP group on one GPU with the transfers made explicit
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
// cpattn_ring_prefill_overlapped enqueues the whole ring of the CP group (every
// rank emulated on the one GPU) on two streams. At step i every rank r computes
// its partial on the block in hand and forwards that same block to rank r+1,
// which computes on it at step i+1. HIP events carry exactly the edges of the
// contract, step by step over the group:
//   compute(i)  waits for transfer(i-1)   (the blocks it reads have arrived),
//   transfer(i) follows transfer(i-1)     (it forwards what that one delivered),
//   transfer(i) waits for compute(i+1-n)  (with n receive buffers, it
//                                          overwrites the buffers that compute
//                                          read; i+1-n >= 1),
// and no edge from compute(i) to transfer(i), so a step's transfers run
// concurrently with that step's compute. The transfers of the first step wait
// for the work the caller enqueued on the compute stream before the call.
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

}  // namespace
}  // namespace cpattn

extern "C" int cpattn_ring_pass(const void *src, void *dst, int64_t bytes, int32_t workgroups, hipStream_t stream) {
  using namespace cpattn;
  const int rc = validate_pass(src, dst, bytes, workgroups);
  if (rc != CPATTN_OK) return rc;
  return launch_pass(src, dst, bytes, workgroups, stream) == hipSuccess ? CPATTN_OK : CPATTN_E_DEVICE;
}

extern "C" int cpattn_ring_prefill_overlapped(const cpattn_prefill_desc *desc, const void *const *q_local,
                                              const void *const *k_blocks, const void *const *v_blocks,
                                              void *const *k_recv, void *const *v_recv, int32_t n_recv,
                                              const cpattn_partial *acc, int32_t link_workgroups, hipStream_t compute,
                                              hipStream_t transfer, hipEvent_t *events, int32_t n_events) {
  using namespace cpattn;
  if (desc == nullptr || acc == nullptr || q_local == nullptr || k_blocks == nullptr || v_blocks == nullptr)
    return CPATTN_E_ARG;
  const int chk = check_prefill(desc, 0, 0);
  if (chk != CPATTN_OK) return chk;
  const int cp = desc->cp;
  if (link_workgroups < 0 || link_workgroups > kMaxLinkGroups) return CPATTN_E_ARG;
  if (cp > 1 && (k_recv == nullptr || v_recv == nullptr || n_recv < 2 || n_recv > kMaxRecv)) return CPATTN_E_ARG;
  if (events == nullptr || n_events < 2 * cp) return CPATTN_E_ARG;
  for (int e = 0; e < 2 * cp; ++e)
    if (events[e] == nullptr) return CPATTN_E_ARG;
  const int64_t total = desc->num_seqs > 0 ? desc->cu_seqlens[desc->num_seqs] : 0;
  if (total == 0) return CPATTN_OK;
  const int fit = check_launches(desc);   // the ring-step launches below cannot fail validation
  if (fit != CPATTN_OK) return fit;
  for (int r = 0; r < cp; ++r) {
    if (q_local[r] == nullptr || k_blocks[r] == nullptr || v_blocks[r] == nullptr) return CPATTN_E_ARG;
    if (acc[r].m == nullptr || acc[r].den == nullptr || acc[r].num == nullptr) return CPATTN_E_ARG;
  }
  const int64_t elem = desc->dtype == CPATTN_DT_BF16 ? 2 : 4;
  const int64_t block_bytes = local_rows(desc) * desc->n_kv * desc->head_dim * elem;
  const int n_buf = cp > 1 ? cp * n_recv : 0;
  // every receive buffer is aligned and disjoint from every block and from
  // every other receive buffer
  for (int x = 0; x < 2 * n_buf; ++x) {
    void *const bx = x < n_buf ? k_recv[x] : v_recv[x - n_buf];
    for (int j = 0; j < cp; ++j)
      if (validate_pass(k_blocks[j], bx, block_bytes, 1) != CPATTN_OK ||
          validate_pass(v_blocks[j], bx, block_bytes, 1) != CPATTN_OK)
        return CPATTN_E_ARG;
    for (int y = x + 1; y < 2 * n_buf; ++y) {
      void *const by = y < n_buf ? k_recv[y] : v_recv[y - n_buf];
      if (validate_pass(bx, by, block_bytes, 1) != CPATTN_OK) return CPATTN_E_ARG;
    }
  }
  // events[0]: entry (compute stream); events[1 + i]: transfers of step i done;
  // events[cp + i]: compute of step i done
  hipEvent_t *const entry = events, *const comm = events + 1, *const comp = events + cp;
  if (cp > 1) {
    if (hipEventRecord(*entry, compute) != hipSuccess || hipStreamWaitEvent(transfer, *entry, 0) != hipSuccess)
      return CPATTN_E_DEVICE;
  }
  for (int i = 0; i < cp; ++i) {
    // compute(i): every rank on the block in hand, its own at step 0, then the
    // one that transfer(i-1) delivered into its receive buffer (i-1) % n_recv
    if (i > 0 && hipStreamWaitEvent(compute, comm[i - 1], 0) != hipSuccess) return CPATTN_E_DEVICE;
    for (int r = 0; r < cp; ++r) {
      const void *k = i == 0 ? k_blocks[r] : k_recv[r * n_recv + (i - 1) % n_recv];
      const void *v = i == 0 ? v_blocks[r] : v_recv[r * n_recv + (i - 1) % n_recv];
      const int rc = cpattn_ring_step_partial(desc, r, i, q_local[r], k, v, &acc[r], i > 0 ? 1 : 0, compute);
      if (rc != CPATTN_OK) return rc;
    }
    if (i == cp - 1) break;
    if (hipEventRecord(comp[i], compute) != hipSuccess) return CPATTN_E_DEVICE;
    // transfer(i): rank r forwards the block in hand to rank r+1's receive
    // buffer i % n_recv, which compute(i + 1 - n_recv) read last
    const int war = i + 1 - n_recv;
    if (war >= 1 && hipStreamWaitEvent(transfer, comp[war], 0) != hipSuccess) return CPATTN_E_DEVICE;
    for (int r = 0; r < cp; ++r) {
      const int to = (r + 1) % cp;
      const void *k = i == 0 ? k_blocks[r] : k_recv[r * n_recv + (i - 1) % n_recv];
      const void *v = i == 0 ? v_blocks[r] : v_recv[r * n_recv + (i - 1) % n_recv];
      if (launch_pass(k, k_recv[to * n_recv + i % n_recv], block_bytes, link_workgroups, transfer) != hipSuccess ||
          launch_pass(v, v_recv[to * n_recv + i % n_recv], block_bytes, link_workgroups, transfer) != hipSuccess)
        return CPATTN_E_DEVICE;
    }
    if (hipEventRecord(comm[i], transfer) != hipSuccess) return CPATTN_E_DEVICE;
  }
  return CPATTN_OK;
}
