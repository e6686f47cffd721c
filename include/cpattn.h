/*
 * cpattn — context-parallel attention for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the G5 context-parallel modelling spec ("G5
 * 上下文并行建模设计规格"): the balanced chunk split, the pass-KV ring step
 * computing a causal partial attention that carries the online-softmax
 * triple (max, numerator, denominator), the associative merge of triples,
 * pass-Q decode (per-shard partials plus the reduction of the three
 * quantities), and the byte / FLOP / memory formulas of its Formulas section.
 * Around them: the one-GPU emulation of the ring's block transfers overlapped
 * with its compute (the spec's dependency contract), a padded layout for
 * sequence lengths not divisible by 2*cp (after the padding rule of the TP/EP
 * design page), a tree-order reduction of triples and the all-to-all of
 * Ulysses and hybrid CP (the spec's follow-up work). Sections cited below are sections of the G5 spec unless another page
 * is named.
 *
 * Conventions shared by every entry point
 *   - Return value: CPATTN_OK (0) or one of the CPATTN_E_* codes. Nothing is
 *     thrown across this interface and nothing is printed. When a call
 *     returns an error it has not written any output and has not enqueued
 *     any GPU work (except CPATTN_E_DEVICE, raised when the runtime refuses
 *     a launch that was already validated).
 *   - The caller owns all memory. Host pointers are read during the call
 *     only. Device pointers must stay valid until the work enqueued on the
 *     given stream has finished; the library keeps no pointer after it
 *     returns, allocates no memory (device or host) and creates no HIP
 *     object (streams and events are the caller's), and has no global state
 *     (one exception: the per-GPU scratch buffer of
 *     cpattn_passq_decode_noalloc, below). Calls are reentrant. Faults of enqueued kernels surface at the caller's next
 *     synchronisation.
 *   - There are no defaults: cp, scale and the shapes are explicit (the
 *     spec's interface appendix: cp is an explicit positive integer, a
 *     missing value is an error, never a silent default).
 *   - Layouts are token-major and contiguous with head_dim innermost.
 *     Device tensors must be 16-byte aligned.
 *   - Supported head_dim: 64, 128, 512. Supported element types of Q, K, V:
 *     fp32 and bf16. Partials, outputs and log-sum-exp are fp32.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CPATTN_OK 0
#define CPATTN_E_ARG 1          /* null pointer, negative size, rank/step out of range, bad enum */
#define CPATTN_E_DIVISIBILITY 2 /* a length not divisible by 2*cp (prefill) or cp (decode),
                                   or n_hq not a multiple of n_kv */
#define CPATTN_E_UNSUPPORTED 3  /* head_dim or dtype without a kernel, shape past a kernel limit */
#define CPATTN_E_OVERFLOW 4     /* an int64 result of cpattn_account would overflow */
#define CPATTN_E_WORKSPACE 5    /* workspace smaller than the size cpattn_passq_decode asked for */
#define CPATTN_E_DEVICE 6       /* the HIP runtime rejected a launch */

typedef enum { CPATTN_DT_F32 = 0, CPATTN_DT_BF16 = 1 } cpattn_dtype;

/* An online-softmax triple for `rows` x n_hq (row, head) pairs, all device fp32
 * (Definitions table, "Partial attention"):
 *   m   [rows, n_hq]        running max of the scaled scores, natural-log units
 *   den [rows, n_hq]        sum of exp(s - m) over the keys seen
 *   num [rows, n_hq, d_h]   sum of exp(s - m) * v over the keys seen (not normalised)
 * A (row, head) that has seen no key is the merge identity: m = -inf, den = 0,
 * num = 0. A triple is defined up to (m + x, e^-x den, e^-x num). */
typedef struct {
  float *m;
  float *den;
  float *num;
} cpattn_partial;

/* Prefill problem description.
 *   cp          CP degree, >= 1.
 *   num_seqs    number of packed sequences, >= 0.
 *   cu_seqlens  HOST array [num_seqs + 1]: cu_seqlens[0] = 0, non-decreasing;
 *               sequence i holds global packed tokens [cu[i], cu[i+1]). With
 *               padded = 0 every length must be divisible by 2*cp (Definitions
 *               table, "Balanced chunk split": 2*cp chunks per sequence).
 *   n_hq, n_kv  query heads and key/value heads; q head h reads kv head
 *               h / (n_hq / n_kv).
 *   head_dim    64, 128 or 512.
 *   dtype       element type of Q, K, V.
 *   scale       softmax scale applied to q.k (e.g. 1/sqrt(head_dim)), > 0, finite.
 *   padded      0: lengths divisible by 2*cp. 1: sequence i of length L_i is
 *               padded at its end to Lp_i, the next multiple of 2*cp, and split
 *               as a sequence of Lp_i tokens (cpattn_balanced_split_padded); the
 *               pad tokens take no part: no query sees them as keys and their
 *               own rows get the identity triple. Local buffers then hold
 *               sum(Lp_i)/cp rows, pad rows included (their contents are not
 *               read). */
typedef struct {
  int32_t cp;
  int32_t num_seqs;
  const int64_t *cu_seqlens;
  int32_t n_hq;
  int32_t n_kv;
  int32_t head_dim;
  int32_t dtype;
  float scale;
  int32_t padded;
} cpattn_prefill_desc;

/* Decode problem description: `batch` queries of one token each, each against
 * its own kv_len keys, split into cp contiguous shards of kv_len/cp keys. */
typedef struct {
  int32_t batch;
  int32_t cp;
  int64_t kv_len;
  int32_t n_hq;
  int32_t n_kv;
  int32_t head_dim;
  int32_t dtype;
  float scale;
} cpattn_decode_desc;

/* Balanced chunk split (Definitions table, "Balanced chunk split"; Rationale).
 * Host only. Each sequence i of length L_i is cut into 2*cp chunks of
 * c_i = L_i / (2*cp) tokens; rank `rank` keeps chunk `rank` (head) and chunk
 * 2*cp-1-rank (tail). Local order: sequence by sequence, head chunk then tail.
 *   positions  out, HOST int64 [sum(L_i)/cp]: global packed token index of
 *              every local row.
 *   cu_local   out, HOST int64 [num_seqs + 1]: local cumulative lengths 2*c_i.
 * Errors: E_ARG (null pointer, num_seqs < 0, rank outside [0, cp), cp < 1,
 * decreasing cu_seqlens), E_DIVISIBILITY (L_i % (2*cp) != 0). */
int cpattn_balanced_split(const int64_t *cu_seqlens, int32_t num_seqs, int32_t cp, int32_t rank,
                          int64_t *positions, int64_t *cu_local);

/* Balanced chunk split of sequences of any length (the padded layout of
 * cpattn_prefill_desc). Host only. Sequence i of length L_i is padded at its
 * end to Lp_i = ceil(L_i / (2*cp)) * 2*cp and cut into 2*cp chunks of
 * c_i = Lp_i / (2*cp) slots; rank `rank` keeps slot chunks `rank` and
 * 2*cp-1-rank as in cpattn_balanced_split. A slot past L_i is a pad row.
 *   positions  out, HOST int64 [sum(Lp_i)/cp]: the global packed token index
 *              cu_seqlens[i] + slot of every local row, or -1 for a pad row.
 *   cu_local   out, HOST int64 [num_seqs + 1]: local cumulative lengths 2*c_i.
 * With every L_i divisible by 2*cp the result equals cpattn_balanced_split's.
 * Padding follows the precedent of the TP/EP design page (tokens that do not
 * divide evenly are padded; padding takes no part in the outputs).
 * Errors: E_ARG (null pointer, num_seqs < 0, rank outside [0, cp), cp < 1,
 * decreasing cu_seqlens). */
int cpattn_balanced_split_padded(const int64_t *cu_seqlens, int32_t num_seqs, int32_t cp, int32_t rank,
                                 int64_t *positions, int64_t *cu_local);

/* Rows of one rank's local buffers (Q, K, V blocks and triples of a prefill
 * description): sum over sequences of 2 * c_i, with c_i = L_i / (2*cp)
 * (padded = 0; every L_i divisible by 2*cp) or ceil(L_i / (2*cp)) (padded = 1,
 * pad rows included). Host only.
 *   rows  out, HOST int64.
 * Errors: E_ARG (null pointer, cp < 1, num_seqs < 0, padded not 0/1,
 * cu_seqlens[0] != 0 or decreasing), E_DIVISIBILITY (padded = 0 and a length
 * not divisible by 2*cp). */
int cpattn_local_rows(const int64_t *cu_seqlens, int32_t num_seqs, int32_t cp, int32_t padded, int64_t *rows);

/* One pass-KV ring step of one rank (Definitions table, "Pass-KV", "Ring step",
 * "Partial attention"). Computes, for every local query row of rank `rank`
 * and every query head, the causal partial attention over the KV block that
 * rank (rank - step) mod cp holds:
 *   visible keys: same sequence, global key position <= global query position;
 *   triple over them as in cpattn_partial (rows that see no key: identity).
 *   q_local  device [R, n_hq, head_dim] rows of `rank`, in the local order of
 *            cpattn_balanced_split (or cpattn_balanced_split_padded when
 *            desc->padded). R = S/cp with S = cu_seqlens[num_seqs]; padded:
 *            R = sum over sequences of 2 * ceil(L_i / (2 cp)).
 *   k_blk, v_blk  device [R, n_kv, head_dim], the rows of rank (rank-step) mod cp
 *            in that rank's local order.
 *   dst      device triple for R rows.
 *   accumulate  0: dst = partial; 1: dst = merge(dst, partial) (dst must then hold
 *            a valid triple, e.g. the previous step's result).
 * bf16 inputs use MFMA with fp32 accumulation; fp32 inputs compute in fp32.
 * Errors: E_ARG, E_DIVISIBILITY, E_UNSUPPORTED (head_dim not 64/128/512,
 * n_hq > 65535, a length > 2^30, or n_kv * head_dim >= 2^24, where 64 key rows
 * pass 2^31 bytes), E_DEVICE. */
int cpattn_ring_step_partial(const cpattn_prefill_desc *desc, int32_t rank, int32_t step,
                             const void *q_local, const void *k_blk, const void *v_blk,
                             const cpattn_partial *dst, int32_t accumulate, hipStream_t stream);

/* Emulated pass-KV transfer (Definitions table, "Pass-KV": each ring step a
 * rank forwards the KV block in hand to its successor). On one GPU the
 * point-to-point transfer is a device copy of `bytes` from src to dst:
 *   workgroups = 0      on a DMA (SDMA) copy engine, using no compute unit, as
 *                       a transfer over xGMI does; runs beside any kernel.
 *   workgroups 1..65535 by a copy kernel of at most that many 256-thread
 *                       workgroups (about one link's worth of bandwidth for a
 *                       few workgroups); it only runs beside another stream's
 *                       kernel while that kernel leaves compute units free.
 *   src, dst    device, 16-byte aligned, non-overlapping; bytes % 16 == 0, >= 0.
 * Errors: E_ARG, E_DEVICE. */
int cpattn_ring_pass(const void *src, void *dst, int64_t bytes, int32_t workgroups, hipStream_t stream);

/* The whole pass-KV ring of the CP group, every rank emulated on this GPU, with
 * the block transfers overlapping the compute (Definitions table, "Pass-KV" and
 * "Ring step": each step a rank computes on the block in hand while forwarding
 * it to its successor; Rationale: the ring's dependency contract; Acceptance,
 * "overlap effective"). For step i = 0 .. cp-1 it enqueues on `compute` the ring
 * steps of every rank r (cpattn_ring_step_partial on the block in hand: its own
 * block at step 0, later the one received at step i-1; step 0 writes acc[r],
 * later steps merge into it), and for i < cp-1 on `transfer` the copies
 * (cpattn_ring_pass, K and V) by which every rank r forwards the block in hand
 * to rank (r+1) mod cp's receive buffer i % n_recv. Rank r's block in hand at
 * step i is therefore the block of rank (r - i) mod cp, as in
 * cpattn_ring_step_partial. Events carry exactly these edges:
 *   compute(i)  waits for transfer(i-1);
 *   transfer(i) follows transfer(i-1) and, when i+1-n_recv >= 1, waits for
 *               compute(i+1-n_recv), which read the buffers it overwrites;
 *   transfer(0) waits for the work enqueued on `compute` before the call.
 * No edge runs from compute(i) to transfer(i): the two run concurrently. When
 * the call returns, all enqueued work is ordered before later work on `compute`
 * (compute(cp-1) waits for the last transfer), so calls may follow one another
 * on the same streams without a host synchronisation.
 *   desc                  as for cpattn_ring_step_partial (rank and step are
 *                         implied).
 *   q_local               HOST array of cp device pointers: rank r's rows
 *                         [R, n_hq, head_dim], R as for cpattn_ring_step_partial.
 *   k_blocks, v_blocks    HOST arrays of cp device pointers: the block rank r
 *                         holds, [R, n_kv, head_dim] in its local order; read only.
 *   k_recv, v_recv        HOST arrays of cp * n_recv device pointers, rank-major
 *                         (buffer b of rank r at r * n_recv + b), one block each,
 *                         pairwise disjoint and disjoint from the blocks (unused
 *                         when cp = 1).
 *   n_recv                2 .. 16 when cp > 1.
 *   acc                   HOST array of cp device triples for R rows each.
 *   link_workgroups       `workgroups` of each transfer (0: copy engine), as for
 *                         cpattn_ring_pass.
 *   compute, transfer     streams; passing the same stream serialises the ring.
 *   events, n_events      HOST array of n_events >= 2 * cp events created by the
 *                         caller (hipEventCreateWithFlags; hipEventDisableTiming
 *                         is enough), used to carry the edges above. The library
 *                         records them and makes the streams wait on them; it
 *                         creates and destroys none. They may be reused by the
 *                         next call once this one has returned.
 * Errors: those of cpattn_ring_step_partial and cpattn_ring_pass, E_ARG for a
 * null event or n_events < 2 * cp, all returned before any work is enqueued;
 * E_DEVICE if the runtime refuses an event or a launch part-way. */
int cpattn_ring_prefill_overlapped(const cpattn_prefill_desc *desc, const void *const *q_local,
                                   const void *const *k_blocks, const void *const *v_blocks,
                                   void *const *k_recv, void *const *v_recv, int32_t n_recv,
                                   const cpattn_partial *acc, int32_t link_workgroups, hipStream_t compute,
                                   hipStream_t transfer, hipEvent_t *events, int32_t n_events);

/* Merge and finalize (Definitions table, "Partial attention": the merge is
 * associative and order-independent).
 *   acc   in/out device triple [rows, n_hq(, head_dim)]: acc = merge(acc, parts[0], ...,
 *         parts[n_parts-1]) with m = max m_i, alpha_i = exp(m_i - m) (0 for m_i = -inf),
 *         den = sum alpha_i den_i, num = sum alpha_i num_i.
 *   parts HOST array of n_parts device triples of the same shape (n_parts >= 0;
 *         parts may be NULL when n_parts == 0).
 *   out   device fp32 [rows, n_hq, head_dim] or NULL: num / den (0 for identity rows).
 *   lse   device fp32 [rows, n_hq] or NULL: m + ln(den) (-inf for identity rows).
 * Errors: E_ARG, E_UNSUPPORTED, E_DEVICE. */
int cpattn_merge(int64_t rows, int32_t n_hq, int32_t head_dim,
                 const cpattn_partial *parts, int32_t n_parts, const cpattn_partial *acc,
                 float *out, float *lse, hipStream_t stream);

/* Tree-order reduction of partial triples: the Tree Attention reduction that
 * the spec lists as follow-up work for pass-Q (Limitations table, "pass-Q
 * reduction topology fixed": its O(log) steps are not visible with a fixed
 * topology). With one triple per rank, round k (k = 0, 1, ...) merges part
 * s + 2^k into part s for every s that is a multiple of 2^(k+1): the exchanges
 * of a tree over n_parts ranks, ceil(log2 n_parts) rounds and n_parts - 1
 * merges. The merge is the associative one of cpattn_merge, so the result
 * equals the linear reduction up to the order of fp32 rounding.
 *   parts  HOST array of n_parts >= 1 device triples [rows, n_hq(, head_dim)],
 *          pairwise distinct. Overwritten: after the call parts[0] holds the
 *          merged triple, the others the partial results of the rounds.
 *   out    device fp32 [rows, n_hq, head_dim] or NULL: num / den of the result.
 *   lse    device fp32 [rows, n_hq] or NULL: m + ln(den).
 * Errors: E_ARG (bad counts, null or repeated parts), E_UNSUPPORTED, E_DEVICE. */
int cpattn_tree_reduce(int64_t rows, int32_t n_hq, int32_t head_dim, const cpattn_partial *parts,
                       int32_t n_parts, float *out, float *lse, hipStream_t stream);

/* All-to-all of a Ulysses group of n ranks, every rank emulated on this GPU:
 * the exchange of Ulysses sequence parallelism, which the spec names as the
 * follow-up to its pass-KV ring together with hybrid CP (Limitations and
 * follow-up work) and leaves out of its own scope (Goals and non-goals). A
 * sequence is held sharded by tokens (rank j: `rows` token rows x n_heads
 * heads) or sharded by heads (rank i: all n*rows token rows x the hn =
 * n_heads/n heads [i*hn, (i+1)*hn), the rows of rank j at rows j*rows ..
 * (j+1)*rows-1 in their own order); a head is head_bytes bytes (head_dim
 * elements of Q, K, V or an output, or one log-sum-exp):
 *   direction 0, seq -> head:  dst[i][j*rows + r][h] = src[j][r][i*hn + h]
 *   direction 1, head -> seq:  dst[j][r][i*hn + h]   = src[i][j*rows + r][h]
 *   src, dst  HOST arrays of n device pointers, each buffer rows*n_heads*
 *             head_bytes bytes (the same in both layouts), 4-byte aligned
 *             (16-byte alignment and 16-byte multiples of hn*head_bytes take
 *             the faster path). No destination overlaps a source or another
 *             destination.
 *   head_bytes > 0, a multiple of 4; 1 <= n <= 64.
 * Byte-exact: a permutation of the source bytes. The attention of a Ulysses
 * rank over its heads is then a ring step over the whole sequence (cp = 1), and
 * of a hybrid group (u Ulysses ranks inside each of c ring ranks) the pass-KV
 * ring over c ranks on its heads.
 * Errors: E_ARG, E_DIVISIBILITY (n_heads % n), E_UNSUPPORTED (n > 64, sizes past
 * int64), E_DEVICE. */
int cpattn_ulysses_all_to_all(int32_t n, int64_t rows, int32_t n_heads, int64_t head_bytes,
                              const void *const *src, void *const *dst, int32_t direction, hipStream_t stream);

/* Pass-Q decode (Definitions table, "Pass-Q"; Use case, decode): the query is
 * sent to every shard, shard s computes the partial triple over its kv_len/cp
 * keys (no mask), and the cp shard triples are reduced into the result.
 *   q         device [batch, n_hq, head_dim].
 *   k_shards, v_shards  HOST arrays of cp device pointers, each [batch, kv_len/cp, n_kv, head_dim].
 *             Query heads per kv head, n_hq / n_kv: 1, 2, 4 or any multiple of 8
 *             (n_kv = 1 with many query heads is the MQA layout that compressed-KV
 *             schemes such as MLA decode with); E_UNSUPPORTED otherwise.
 *   shard_partials  device triple with rows = cp*batch (shard-major: row s*batch + b):
 *             the per-shard triples, written by this call.
 *   out       device fp32 [batch, n_hq, head_dim];  lse device fp32 [batch, n_hq].
 *   ws, ws_bytes  device workspace. With ws == NULL the call only stores the
 *             required size in *ws_bytes and returns CPATTN_OK. Otherwise *ws_bytes
 *             is the size available (E_WORKSPACE if too small).
 * Errors: E_ARG, E_DIVISIBILITY, E_UNSUPPORTED (also cp > 64 shards, or
 * n_kv * head_dim >= 2^24), E_WORKSPACE, E_DEVICE. */
int cpattn_passq_decode(const cpattn_decode_desc *desc, const void *q,
                        const void *const *k_shards, const void *const *v_shards,
                        const cpattn_partial *shard_partials, float *out, float *lse,
                        void *ws, size_t *ws_bytes, hipStream_t stream);

/* Size of the scratch buffer of cpattn_passq_decode_noalloc, in bytes (32 MiB). */
#define CPATTN_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Pass-Q decode that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. The same computation, kernels and results as
 * cpattn_passq_decode (bit for bit), with its workspace taken from a scratch
 * buffer of CPATTN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on, from the module's load until the process ends; its address on the
 * current device is looked up once, on the first call there. The call makes no
 * allocation of its own (no hipMalloc, hipFree or allocating library routine).
 *   arguments  as for cpattn_passq_decode, without ws / ws_bytes.
 * Every call on a GPU uses that GPU's one scratch buffer: calls that may run at
 * the same time on one GPU (from several streams or threads) race and must be
 * ordered by the caller. Nothing in the buffer needs clearing between calls.
 * Errors: those of cpattn_passq_decode; E_WORKSPACE when the description needs
 * more than CPATTN_NOALLOC_SCRATCH_BYTES of workspace (the size
 * cpattn_passq_decode reports with ws == NULL), returned before any device
 * call; E_DEVICE when the runtime cannot give the buffer's address. This entry
 * point keeps per-device state (the buffer and its looked-up address), unlike
 * the others. */
int cpattn_passq_decode_noalloc(const cpattn_decode_desc *desc, const void *q,
                                const void *const *k_shards, const void *const *v_shards,
                                const cpattn_partial *shard_partials, float *out, float *lse,
                                hipStream_t stream);

/* Inputs of cpattn_account. Prefill fields are used when cu_seqlens != NULL,
 * decode fields when kv_len > 0.
 *   cp, n_hq, n_kv, head_dim  as above; dtype_bytes = s, the model element size.
 *   c_kv           K+V bytes per token per layer (Definitions table); 0 means
 *                  2 * n_kv * head_dim * dtype_bytes.
 *   d_model        d, the model hidden size (Definitions table); 0 means n_hq * head_dim.
 *   layers_local   L_local of the memory formula, >= 1.
 *   cu_seqlens, num_seqs  HOST, packed prefill lengths (b folded in), each % (2*cp) == 0.
 *   batch, kv_len  decode batch b and KV length S (kv_len % cp == 0). */
typedef struct {
  int32_t cp;
  int32_t n_hq;
  int32_t n_kv;
  int32_t head_dim;
  int32_t dtype_bytes;
  int64_t c_kv;
  int64_t d_model;
  int64_t layers_local;
  const int64_t *cu_seqlens;
  int32_t num_seqs;
  int32_t batch;
  int64_t kv_len;
} cpattn_account_in;

/* Formulas section; every field exact in int64. Fields of a part that was not
 * requested are 0.
 *   tokens_per_rank         S/cp
 *   ring_steps, p2p_ops     cp compute steps and cp-1 transfers per rank and layer
 *   passkv_bytes_per_step   S/cp * c_kv (0 at cp = 1)
 *   passkv_bytes_per_rank   (cp-1) * S/cp * c_kv            (eq. g5cp-passkv-bytes)
 *   attn_flops              F_attn = sum_i 2 * n_hq * head_dim * L_i^2
 *   step_flops              F_attn / cp^2                   (eq. g5cp-step-flops)
 *   rank_flops              F_attn / cp
 *   step0_flops_exact       4 * head_dim * n_hq * sum_i (2 c_i^2 + c_i)   (inclusive diagonal)
 *   stepN_flops_exact       4 * head_dim * n_hq * sum_i 2 c_i^2           (steps >= 1)
 *   rank_flops_exact        step0 + (cp-1) * stepN
 *   kv_bytes_per_rank       S * c_kv * L_local / cp          (prefill KV memory)
 *   passq_dispatch_bytes    b * d * s   (0 at cp = 1)
 *   passq_reduce_bytes      b * (d + 2 n_h) * s   (0 at cp = 1; n_h = n_hq)
 *   decode_kv_bytes_per_rank  b * S * c_kv * L_local / cp
 *   decode_kv_bytes_total   b * S * c_kv * L_local
 *   decode_flops            4 * b * n_hq * head_dim * S */
typedef struct {
  int64_t tokens_per_rank;
  int64_t ring_steps;
  int64_t p2p_ops;
  int64_t passkv_bytes_per_step;
  int64_t passkv_bytes_per_rank;
  int64_t attn_flops;
  int64_t step_flops;
  int64_t rank_flops;
  int64_t step0_flops_exact;
  int64_t stepN_flops_exact;
  int64_t rank_flops_exact;
  int64_t kv_bytes_per_rank;
  int64_t passq_dispatch_bytes;
  int64_t passq_reduce_bytes;
  int64_t decode_kv_bytes_per_rank;
  int64_t decode_kv_bytes_total;
  int64_t decode_flops;
} cpattn_account_out;

/* Host only. Errors: E_ARG, E_DIVISIBILITY, E_OVERFLOW. */
int cpattn_account(const cpattn_account_in *in, cpattn_account_out *out);

/* Library version string (static storage). */
const char *cpattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
