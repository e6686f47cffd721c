"""GPU parity of the pass-KV ring step (cpattn_ring_step_partial) and the
merge (cpattn_merge) against the fp64 oracle, through the C-ABI binding.

Small cases compare every (rank, step) partial in canonical form
(num/den, m + ln den) and the merged result, element by element, with the
-inf (identity) rows required to coincide exactly. Full-size cases (the GQA
workload, S = 32768 over cp = 8, and rank 0's share of the 1M-token workload)
run in the launch configuration the benchmark times and compare sampled rows
against the oracle computed row by row."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import (TOL_BF16, TOL_F32, canonical_np, compare, global_inputs_np, local_buffers, log,
                         need_gpu, np_to_device, run_ring)

pytestmark = pytest.mark.gpu

# name, lengths, cp, n_hq, n_kv, head_dim, dtype, input scale
CASES = [
    ("tiny-f32-S256-cp2", [256], 2, 2, 2, 64, "f32", 1.0),
    ("gqa4-bf16-d128-c200", [2 * 4 * 200], 4, 8, 2, 128, "bf16", 0.5),
    ("mha-bf16-d64-varlen", [2 * 2 * 70, 2 * 2 * 130, 2 * 2 * 9], 2, 4, 4, 64, "bf16", 0.5),
    ("gqa2-bf16-d128-cp3", [2 * 3 * 100, 2 * 3 * 33], 3, 4, 2, 128, "bf16", 0.5),
    ("mha-bf16-d512-varlen", [2 * 2 * 37, 2 * 2 * 20], 2, 2, 2, 512, "bf16", 0.5),
    ("gqa2-bf16-d512-cp4", [2 * 4 * 70, 2 * 4 * 33], 4, 4, 2, 512, "bf16", 0.5),
    ("mha-bf16-d512-cp3-long-chunks", [2 * 3 * 150], 3, 2, 2, 512, "bf16", 0.5),
    ("gqa2-f32-d128", [2 * 2 * 50], 2, 4, 2, 128, "f32", 1.0),
    ("gqa2-f32-d512", [2 * 2 * 12], 2, 2, 1, 512, "f32", 1.0),
    ("cp1-bf16-d128", [300, 64], 1, 8, 2, 128, "bf16", 0.5),
    ("cp8-bf16-d128-mqa", [2 * 8 * 40], 8, 4, 1, 128, "bf16", 0.5),
    # one kv head shared by many query heads (MQA; MLA-like at head_dim 512)
    ("mqa32-bf16-d128-cp4", [2 * 4 * 96, 2 * 4 * 17], 4, 32, 1, 128, "bf16", 0.5),
    ("mqa64-bf16-d512-cp2", [2 * 2 * 40], 2, 64, 1, 512, "bf16", 0.5),
    ("mqa16-bf16-d64-cp2", [2 * 2 * 75], 2, 16, 1, 64, "bf16", 0.5),
    ("empty-seqs-bf16", [0, 2 * 2 * 33, 0], 2, 4, 2, 64, "bf16", 0.5),
]


def _setup(lens, cp, n_hq, n_kv, d, dtype, sc, seed=5):
    import context_attention_amd as ca
    q, k, v, cu = global_inputs_np(lens, n_hq, n_kv, d, seed, dtype, sc)
    dev = [np_to_device(x, dtype) for x in (q, k, v)]
    local = local_buffers(ca, cu, cp, dev)
    desc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=n_hq, n_kv=n_kv, head_dim=d, dtype=dtype,
                          scale=1.0 / np.sqrt(d))
    return ca, q, k, v, cu, local, desc


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ring_step_partials_and_merge(case):
    need_gpu()
    import torch
    name, lens, cp, n_hq, n_kv, d, dtype, sc = case
    log(f"[prefill parity] {name} lens={lens} cp={cp} heads={n_hq}/{n_kv} d={d} {dtype}")
    ca, q, k, v, cu, local, desc = _setup(lens, cp, n_hq, n_kv, d, dtype, sc)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    ref = oracle.ring_prefill(q, k, v, cu, cp, 1.0 / np.sqrt(d))
    T = int(cu[-1])
    unfused = run_ring(ca, desc, local, fused=False)
    fused = run_ring(ca, desc, local, fused=True)
    for r in range(cp):
        pos = local[r][0]
        np.testing.assert_array_equal(pos, ref["positions"][r])
        for t in range(cp):
            p = unfused[r]["parts"][t]
            go, gl = canonical_np(p.m.cpu().numpy(), p.den.cpu().numpy(), p.num.cpu().numpy())
            wo, wl = oracle.finalize(ref["partials"][r][t])
            compare(f"r{r} t{t} partial", go, gl, wo, wl, tol)
        for tag, res in (("unfused", unfused[r]), ("fused", fused[r])):
            compare(f"r{r} merged {tag}", res["out"].cpu().numpy(), res["lse"].cpu().numpy(),
                    ref["out"][pos], ref["lse"][pos], tol)
        # fused accumulation and separate merge differ only in fp32 rounding
        a = fused[r]["out"].cpu().numpy()
        b = unfused[r]["out"].cpu().numpy()
        assert np.abs(a - b).max(initial=0) <= 1e-5 * max(1.0, np.abs(b).max(initial=0))
    # global result against the unsplit definition too
    if T:
        out_g = np.zeros((T, n_hq, d))
        lse_g = np.zeros((T, n_hq))
        for r in range(cp):
            out_g[local[r][0]] = fused[r]["out"].cpu().numpy()
            lse_g[local[r][0]] = fused[r]["lse"].cpu().numpy()
        uo, ul = oracle.attention_reference(q, k, v, cu, 1.0 / np.sqrt(d))
        compare("global vs unsplit", out_g, lse_g, uo, ul, tol)


def test_identity_rows_and_poison():
    """Every row of the destination is written (NaN poison disappears), and the
    rows that see no key are exactly the oracle's identity rows."""
    need_gpu()
    import torch
    ca, q, k, v, cu, local, desc = _setup([2 * 4 * 48, 2 * 4 * 17], 4, 4, 2, 128, "bf16", 0.5)
    ref = oracle.ring_prefill(q, k, v, cu, 4, 1.0 / np.sqrt(128))
    rows = int(cu[-1]) // 4
    for r in range(4):
        for t in range(4):
            p = ca.new_partial(rows, 4, 128)
            for x in (p.m, p.den, p.num):
                x.fill_(float("nan"))
            j = (r - t) % 4
            ca.ring_step_partial(desc, r, t, local[r][1][0], local[j][1][1], local[j][1][2], p)
            m = p.m.cpu().numpy()
            assert not np.isnan(m).any() and not np.isnan(p.num.cpu().numpy()).any()
            want_empty = ~np.isfinite(ref["partials"][r][t][0])
            np.testing.assert_array_equal(np.isneginf(m), want_empty)
            assert np.all(p.den.cpu().numpy()[want_empty] == 0)


def test_merge_order_independent_gpu():
    """cpattn_merge in ring order, reversed and shuffled gives the same result
    up to fp32 rounding (the merge is associative and order-independent)."""
    need_gpu()
    import torch
    cp = 4
    ca, q, k, v, cu, local, desc = _setup([2 * cp * 64], cp, 8, 2, 128, "bf16", 0.5)
    res = run_ring(ca, desc, local, fused=False)
    rows = int(cu[-1]) // cp
    rng = np.random.default_rng(0)
    for r in range(cp):
        parts = res[r]["parts"]
        outs = []
        for order in (list(range(cp)), list(range(cp))[::-1], list(rng.permutation(cp))):
            acc = ca.Partial(parts[order[0]].m.clone(), parts[order[0]].den.clone(), parts[order[0]].num.clone())
            out = torch.empty(rows, 8, 128, device="cuda")
            lse = torch.empty(rows, 8, device="cuda")
            ca.merge(acc, [parts[i] for i in order[1:]], out=out, lse=lse)
            outs.append((out.cpu().numpy(), lse.cpu().numpy()))
        for o, l in outs[1:]:
            assert np.abs(o - outs[0][0]).max() <= 1e-5
            assert np.abs(l - outs[0][1]).max() <= 1e-5


def test_cp1_is_the_unsplit_path():
    """CP=1 degeneration: one ring step over the whole sequence gives plain
    causal attention; the cp=1 call on the global tensors is the unsplit call."""
    need_gpu()
    import torch
    ca, q, k, v, cu, local, desc = _setup([512, 128], 1, 8, 2, 128, "bf16", 0.5)
    res = run_ring(ca, desc, local)
    np.testing.assert_array_equal(local[0][0], np.arange(640))
    uo, ul = oracle.attention_reference(q, k, v, cu, 1.0 / np.sqrt(128))
    compare("cp1 vs unsplit", res[0]["out"].cpu().numpy(), res[0]["lse"].cpu().numpy(), uo, ul, TOL_BF16)


def _sampled_rows(c, rng, n_rand):
    base = [0, 1, c - 1, c, c + 1, 2 * c - 1]
    extra = list(rng.integers(0, 2 * c, n_rand))
    return np.unique(np.array(base + extra, dtype=np.int64))


def test_gqa_workload_full_size_sampled():
    """The GQA workload (S = 32768, cp = 8, 32/8 heads, d = 128, bf16): all 64
    ring-step calls fused per rank, then sampled rows of ranks 0, 3 and 7
    against the unsplit oracle over every head."""
    need_gpu()
    import torch
    import context_attention_amd as ca
    w = synth.WORKLOADS["gqa"]
    S, cp, d = w.total_tokens, w.cp, w.head_dim
    log(f"[prefill full] {w.name}")
    q = synth.tensor_torch(w.seed, synth.TENSOR_Q, (S, w.n_hq, d), w.scale_in, w.dtype, "cuda")
    k = synth.tensor_torch(w.seed, synth.TENSOR_K, (S, w.n_kv, d), w.scale_in, w.dtype, "cuda")
    v = synth.tensor_torch(w.seed, synth.TENSOR_V, (S, w.n_kv, d), w.scale_in, w.dtype, "cuda")
    cu = w.cu_seqlens
    local = local_buffers(ca, cu, cp, [q, k, v])
    del q, k, v
    desc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=w.n_hq, n_kv=w.n_kv, head_dim=d, dtype=w.dtype,
                          scale=w.softmax_scale)
    res = run_ring(ca, desc, local, fused=True)
    qn = synth.tensor_np(w.seed, synth.TENSOR_Q, (S, w.n_hq, d), w.scale_in, w.dtype)
    kn = synth.tensor_np(w.seed, synth.TENSOR_K, (S, w.n_kv, d), w.scale_in, w.dtype)
    vn = synth.tensor_np(w.seed, synth.TENSOR_V, (S, w.n_kv, d), w.scale_in, w.dtype)
    rng = np.random.default_rng(1)
    c = S // (2 * cp)
    for r in (0, 3, 7):
        rows = _sampled_rows(c, rng, 10)
        gpos = local[r][0][rows]
        wo, wl = oracle.attention_reference_rows(qn[gpos], gpos, kn, vn, w.softmax_scale)
        compare(f"gqa rank {r} sampled", res[r]["out"].cpu().numpy()[rows], res[r]["lse"].cpu().numpy()[rows],
                wo, wl, TOL_BF16)


def test_long_context_rank0_share_sampled():
    """Rank 0's share of the 1M-token workload (cp = 8: chunks 0 and 15, 2 x 65536
    query rows) over all 8 ring-step KV blocks, fused, as the benchmark runs it.
    Sampled rows of the head and tail chunk are compared with the oracle on the
    4 query heads of kv head 3 (the oracle reads that kv head's 1M keys)."""
    need_gpu()
    import torch
    import context_attention_amd as ca
    w = synth.WORKLOADS["long"]
    S, cp, d, H, G = w.total_tokens, w.cp, w.head_dim, w.n_hq, w.n_kv
    log(f"[prefill full] {w.name}")
    cu = w.cu_seqlens
    pos0, _ = ca.balanced_split(cu, cp, 0)
    c = S // (2 * cp)
    q0 = torch.cat([synth.tensor_torch(w.seed, synth.TENSOR_Q, (S, H, d), w.scale_in, w.dtype, "cuda",
                                       row_start=int(pos0[0]), rows=c),
                    synth.tensor_torch(w.seed, synth.TENSOR_Q, (S, H, d), w.scale_in, w.dtype, "cuda",
                                       row_start=int(pos0[c]), rows=c)])
    k = synth.tensor_torch(w.seed, synth.TENSOR_K, (S, G, d), w.scale_in, w.dtype, "cuda")
    v = synth.tensor_torch(w.seed, synth.TENSOR_V, (S, G, d), w.scale_in, w.dtype, "cuda")
    blocks = []
    for j in range(cp):
        pj, _ = ca.balanced_split(cu, cp, j)
        idx = torch.from_numpy(pj).cuda()
        blocks.append((k.index_select(0, idx).contiguous(), v.index_select(0, idx).contiguous()))
    del k, v
    torch.cuda.synchronize()
    desc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=H, n_kv=G, head_dim=d, dtype=w.dtype, scale=w.softmax_scale)
    rows = S // cp
    acc = ca.new_partial(rows, H, d)
    for t in range(cp):
        j = (0 - t) % cp
        ca.ring_step_partial(desc, 0, t, q0, blocks[j][0], blocks[j][1], acc, accumulate=(t > 0))
    out = torch.empty(rows, H, d, device="cuda")
    lse = torch.empty(rows, H, device="cuda")
    ca.merge(acc, [], out=out, lse=lse)
    torch.cuda.synchronize()
    g = 3
    heads = list(range(g * (H // G), (g + 1) * (H // G)))
    rng = np.random.default_rng(2)
    sample = _sampled_rows(c, rng, 6)
    gpos = pos0[sample]
    log(f"  oracle: {len(sample)} rows x heads {heads}; generating kv head {g} (1M keys)")
    kg = synth.head_slice_np(w.seed, synth.TENSOR_K, (S, G, d), g, w.scale_in, w.dtype)
    vg = synth.head_slice_np(w.seed, synth.TENSOR_V, (S, G, d), g, w.scale_in, w.dtype)
    qn = np.concatenate([synth.values_at_np(w.seed, synth.TENSOR_Q,
                                            ((p * H + np.array(heads))[:, None] * d + np.arange(d)[None, :])[None],
                                            w.scale_in, w.dtype) for p in gpos])
    wo, wl = oracle.attention_reference_rows(qn, gpos, kg, vg, w.softmax_scale, key_block=1 << 16)
    go = out[torch.from_numpy(sample).cuda()][:, heads].cpu().numpy()
    gl = lse[torch.from_numpy(sample).cuda()][:, heads].cpu().numpy()
    compare("long rank 0 sampled", go, gl, wo, wl, TOL_BF16)


def test_wide_head_varlen_workload_sampled():
    """The wide-head varlen workload (6 packed sequences of 9376..16048 tokens,
    cp = 4, 64 heads, head_dim 512, bf16): every rank's full ring, fused, then
    sampled rows of ranks 0 and 3 against the oracle on heads 5 and 42."""
    need_gpu()
    import torch
    import context_attention_amd as ca
    w = synth.WORKLOADS["varlen"]
    T, cp, d, H = w.total_tokens, w.cp, w.head_dim, w.n_hq
    log(f"[prefill full] {w.name}")
    cu = w.cu_seqlens
    q = synth.tensor_torch(w.seed, synth.TENSOR_Q, (T, H, d), w.scale_in, w.dtype, "cuda")
    k = synth.tensor_torch(w.seed, synth.TENSOR_K, (T, w.n_kv, d), w.scale_in, w.dtype, "cuda")
    v = synth.tensor_torch(w.seed, synth.TENSOR_V, (T, w.n_kv, d), w.scale_in, w.dtype, "cuda")
    local = local_buffers(ca, cu, cp, [q, k, v])
    del q, k, v
    desc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=H, n_kv=w.n_kv, head_dim=d, dtype=w.dtype,
                          scale=w.softmax_scale)
    res = run_ring(ca, desc, local, fused=True)
    heads = [5, 42]
    rng = np.random.default_rng(5)
    for r in (0, 3):
        pos = local[r][0]
        rows = np.unique(np.concatenate([[0, len(pos) - 1], rng.integers(0, len(pos), 10)]))
        for h in heads:
            kh = synth.head_slice_np(w.seed, synth.TENSOR_K, (T, w.n_kv, d), h, w.scale_in, w.dtype)
            vh = synth.head_slice_np(w.seed, synth.TENSOR_V, (T, w.n_kv, d), h, w.scale_in, w.dtype)
            for row in rows:
                g = int(pos[row])
                si = int(np.searchsorted(cu, g, side="right") - 1)
                a0, a1 = int(cu[si]), int(cu[si + 1])
                qh = synth.values_at_np(w.seed, synth.TENSOR_Q, (g * H + h) * d + np.arange(d), w.scale_in, w.dtype)
                wo, wl = oracle.attention_reference_rows(qh[None, None, :], np.array([g - a0]), kh[a0:a1], vh[a0:a1],
                                                         w.softmax_scale)
                compare(f"varlen r{r} row {row} head {h}", res[r]["out"][row, h].cpu().numpy()[None, None],
                        res[r]["lse"][row, h].cpu().numpy()[None, None], wo, wl, TOL_BF16)
