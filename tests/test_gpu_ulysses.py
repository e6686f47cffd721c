"""GPU tests of the Ulysses all-to-all (cpattn_ulysses_all_to_all) and of
Ulysses and hybrid CP built from it and the ring step (G5 context-parallel
modelling spec, "Limitations and follow-up work": Ulysses and hybrid CP).

The all-to-all is a byte permutation: compared bit for bit with the same
permutation written with torch indexing, in both directions, with the bytes
past every destination left alone. Ulysses: the sequence is sharded by tokens
over u ranks; the all-to-all gives each rank all tokens of n_hq/u query heads
and n_kv/u kv heads, the rank runs causal attention over the whole sequence
for its heads (one ring step with cp = 1), and the inverse all-to-all brings
the outputs back to the token shards. Hybrid: u Ulysses ranks inside each of c
ring ranks (cp = u c): ring rank j holds the balanced split's rows of j over c
ranks, its u Ulysses ranks hold consecutive slices of those rows; the
all-to-all inside each ring group, then the pass-KV ring over the c ring ranks
on each head group, then the inverse all-to-all. Outputs and log-sum-exps are
compared with the oracle's unsplit attention at the global positions of each
rank's rows."""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL_BF16, TOL_F32, compare, global_inputs_np, log, need_gpu, np_to_device

pytestmark = pytest.mark.gpu


def _torch_seq_to_head(src, n):
    """The seq -> head layout by indexing: dst[i] = rows of every rank, heads of group i."""
    import torch
    hn = src[0].shape[1] // n
    return [torch.cat([s[:, i * hn:(i + 1) * hn] for s in src], dim=0).contiguous() for i in range(n)]


@pytest.mark.parametrize("n,rows,heads,inner,dtype", [
    (1, 7, 4, (64,), "bf16"), (2, 5, 4, (128,), "bf16"), (4, 33, 8, (128,), "bf16"), (8, 16, 32, (128,), "bf16"),
    (3, 9, 6, (512,), "bf16"), (4, 12, 8, (), "f32"), (2, 3, 6, (3,), "f32"), (4, 0, 8, (128,), "bf16"),
    (8, 20, 64, (128,), "f32")])
def test_all_to_all_is_the_permutation(n, rows, heads, inner, dtype):
    need_gpu()
    import torch
    import context_attention_amd as ca
    log(f"ulysses all-to-all n={n} rows={rows} heads={heads} head={inner} {dtype}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(n * 1000 + rows)
    src = [torch.randn((rows, heads) + inner, generator=g, device="cuda").to(tdt) for _ in range(n)]
    want = _torch_seq_to_head(src, n)
    # destinations as views at the front of larger buffers, the tails poisoned
    numel = rows * heads * int(np.prod(inner))
    big = [torch.full((numel + 64,), 7, dtype=tdt, device="cuda") for _ in range(n)]
    dst = [b[:numel].view((n * rows, heads // n) + inner) for b in big]
    ca.ulysses_all_to_all(src, dst, heads, "seq_to_head")
    back_big = [torch.full((numel + 64,), 5, dtype=tdt, device="cuda") for _ in range(n)]
    back = [b[:numel].view((rows, heads) + inner) for b in back_big]
    ca.ulysses_all_to_all(dst, back, heads, "head_to_seq")
    torch.cuda.synchronize()
    for i in range(n):
        assert torch.equal(dst[i].view(torch.int16 if dtype == "bf16" else torch.int32),
                           want[i].view(torch.int16 if dtype == "bf16" else torch.int32)), f"rank {i} differs"
        assert torch.all(big[i][numel:] == 7), "write past the end of a destination"
        assert torch.equal(back[i], src[i]), f"round trip differs on rank {i}"
        assert torch.all(back_big[i][numel:] == 5), "write past the end of a destination"


def _check_rank(name, out_seq, lse_seq, pos, ref_out, ref_lse, tol):
    compare(name, out_seq.cpu().numpy(), lse_seq.cpu().numpy(), ref_out[pos], ref_lse[pos], tol)


CASES = [
    # lens, u (Ulysses ranks), c (ring ranks), n_hq, n_kv, d, dtype
    ([1024], 4, 1, 16, 4, 128, "bf16"),
    ([768, 256], 2, 1, 8, 2, 64, "bf16"),
    ([1024], 2, 4, 16, 4, 128, "bf16"),
    ([512, 1024], 4, 2, 16, 8, 128, "bf16"),
    ([640], 2, 2, 8, 2, 64, "f32"),
    ([512], 2, 2, 8, 4, 512, "bf16"),
]


def _random_cases(n, seed=77):
    """Seeded random Ulysses (c = 1) and hybrid shapes: u in {1, 2, 4, 8}, c in
    {1, 2, 3, 4}, GQA ratios 1-8 with u dividing the kv heads, d 64/128/512, bf16
    and fp32, one to three packed sequences whose lengths are multiples of 2c,
    and a ring rank's rows a multiple of u."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        u = int(g.choice([1, 2, 4, 8]))
        c = int(g.choice([1, 2, 3, 4]))
        n_kv = u * int(g.choice([1, 2]))
        n_hq = n_kv * int(g.choice([1, 2, 4, 8]))
        d = int(g.choice([64, 128, 512]))
        dtype = "f32" if g.random() < 0.25 else "bf16"
        nseq = int(g.integers(1, 4))
        lens = [2 * c * int(g.integers(1, 1200 // (2 * c * nseq) + 2)) for _ in range(nseq)]
        if (sum(lens) // c) % u or n_hq * d * sum(lens) > 6_000_000:
            continue
        out.append((lens, u, c, n_hq, n_kv, d, dtype))
    return out


CASES = CASES + _random_cases(10)


@pytest.mark.parametrize("lens,u,c,n_hq,n_kv,d,dtype", CASES,
                         ids=[f"u{x[1]}-c{x[2]}-{x[6]}-d{x[5]}-h{x[3]}x{x[4]}-S{sum(x[0])}-{len(x[0])}seq" for x in CASES])
def test_ulysses_and_hybrid_match_the_oracle(lens, u, c, n_hq, n_kv, d, dtype):
    need_gpu()
    import torch
    import context_attention_amd as ca
    log(f"ulysses/hybrid lens={lens} u={u} c={c} heads={n_hq}/{n_kv} d={d} {dtype}")
    scale = 1.0 / np.sqrt(d)
    qn, kn, vn, cu = global_inputs_np(lens, n_hq, n_kv, d, seed=41, dtype=dtype, scale=0.5)
    q, k, v = (np_to_device(a, dtype) for a in (qn, kn, vn))
    ref_out, ref_lse = oracle.attention_reference(qn, kn, vn, cu, scale)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    # ring rank j: the balanced split's rows over c ranks; Ulysses rank i of it: slice i of those rows
    pos = [ca.balanced_split(cu, c, j)[0] for j in range(c)]
    L = len(pos[0])
    assert L % u == 0
    R = L // u
    idx = [torch.from_numpy(p).to("cuda") for p in pos]
    seq = {name: [[t.index_select(0, idx[j][i * R:(i + 1) * R]).contiguous() for i in range(u)] for j in range(c)]
           for name, t in (("q", q), ("k", k), ("v", v))}
    # all-to-all inside each ring group: head-sharded [L, heads/u, d] per (i, j)
    head = {}
    for name, nh in (("q", n_hq), ("k", n_kv), ("v", n_kv)):
        head[name] = []
        for j in range(c):
            dst = [torch.empty((L, nh // u, d), dtype=seq[name][j][0].dtype, device="cuda") for _ in range(u)]
            ca.ulysses_all_to_all(seq[name][j], dst, nh, "seq_to_head")
            head[name].append(dst)
    # the pass-KV ring over the c ring ranks on each head group
    desc = ca.PrefillDesc(cp=c, cu_seqlens=cu, n_hq=n_hq // u, n_kv=n_kv // u, head_dim=d, dtype=dtype, scale=scale)
    out_h = [[None] * u for _ in range(c)]
    lse_h = [[None] * u for _ in range(c)]
    for i in range(u):
        for r in range(c):
            acc = ca.new_partial(L, n_hq // u, d)
            for t in range(c):
                j = (r - t) % c
                ca.ring_step_partial(desc, r, t, head["q"][r][i], head["k"][j][i], head["v"][j][i], acc,
                                     accumulate=t > 0)
            out_h[r][i] = torch.empty(L, n_hq // u, d, device="cuda")
            lse_h[r][i] = torch.empty(L, n_hq // u, device="cuda")
            ca.merge(acc, [], out=out_h[r][i], lse=lse_h[r][i])
    # back to the token shards and against the oracle
    for r in range(c):
        out_s = [torch.empty(R, n_hq, d, device="cuda") for _ in range(u)]
        lse_s = [torch.empty(R, n_hq, device="cuda") for _ in range(u)]
        ca.ulysses_all_to_all(out_h[r], out_s, n_hq, "head_to_seq")
        ca.ulysses_all_to_all(lse_h[r], lse_s, n_hq, "head_to_seq")
        torch.cuda.synchronize()
        for i in range(u):
            _check_rank(f"ring rank {r}, Ulysses rank {i}", out_s[i], lse_s[i], pos[r][i * R:(i + 1) * R],
                        ref_out, ref_lse, tol)


def test_ulysses_gqa_workload_full_size_sampled():
    """Ulysses over u = 8 ranks at the size the bench times: the GQA prefill
    (S = 32768, 32q/8kv, d128, bf16), all-to-all, per-rank attention over 4q/1kv
    heads, inverse all-to-all. Sampled check: 6 rows of every Ulysses rank (its
    first, last and four between) x all 32 heads against the oracle's unsplit
    attention over the whole sequence."""
    need_gpu()
    import torch
    import context_attention_amd as ca
    import synth
    w = synth.WORKLOADS["gqa"]
    S, H, G, d, u = w.total_tokens, w.n_hq, w.n_kv, w.head_dim, 8
    R = S // u
    log(f"ulysses full size S={S} heads={H}/{G} d={d} u={u}")
    q = synth.tensor_torch(w.seed, synth.TENSOR_Q, (S, H, d), w.scale_in, w.dtype, "cuda")
    k = synth.tensor_torch(w.seed, synth.TENSOR_K, (S, G, d), w.scale_in, w.dtype, "cuda")
    v = synth.tensor_torch(w.seed, synth.TENSOR_V, (S, G, d), w.scale_in, w.dtype, "cuda")
    seq = {n: [t[i * R:(i + 1) * R].contiguous() for i in range(u)] for n, t in (("q", q), ("k", k), ("v", v))}
    head = {}
    for n, nh in (("q", H), ("k", G), ("v", G)):
        head[n] = [torch.empty(S, nh // u, d, dtype=q.dtype, device="cuda") for _ in range(u)]
        ca.ulysses_all_to_all(seq[n], head[n], nh, "seq_to_head")
    desc = ca.PrefillDesc(cp=1, cu_seqlens=w.cu_seqlens, n_hq=H // u, n_kv=G // u, head_dim=d, dtype=w.dtype,
                          scale=w.softmax_scale)
    out_h, lse_h = [], []
    for i in range(u):
        acc = ca.new_partial(S, H // u, d)
        ca.ring_step_partial(desc, 0, 0, head["q"][i], head["k"][i], head["v"][i], acc, accumulate=False)
        out_h.append(torch.empty(S, H // u, d, device="cuda"))
        lse_h.append(torch.empty(S, H // u, device="cuda"))
        ca.merge(acc, [], out=out_h[i], lse=lse_h[i])
    out_s = [torch.empty(R, H, d, device="cuda") for _ in range(u)]
    lse_s = [torch.empty(R, H, device="cuda") for _ in range(u)]
    ca.ulysses_all_to_all(out_h, out_s, H, "head_to_seq")
    ca.ulysses_all_to_all(lse_h, lse_s, H, "head_to_seq")
    torch.cuda.synchronize()
    kn = k.view(torch.int16).cpu().numpy().view(np.uint16)
    vn = v.view(torch.int16).cpu().numpy().view(np.uint16)
    for i in range(u):
        local = np.unique(np.linspace(0, R - 1, 6).astype(np.int64))
        pos = i * R + local
        qr = q[torch.from_numpy(pos).to("cuda")].view(torch.int16).cpu().numpy().view(np.uint16)
        ro, rl = oracle.attention_reference_rows(qr, pos, kn, vn, w.softmax_scale)
        compare(f"Ulysses rank {i}", out_s[i][torch.from_numpy(local).to("cuda")].cpu().numpy(),
                lse_s[i][torch.from_numpy(local).to("cuda")].cpu().numpy(), ro, rl, TOL_BF16)


def test_hybrid_gqa_workload_full_size_sampled():
    """Hybrid CP at the size the bench times: the GQA prefill (S = 32768,
    32q/8kv, d128, bf16), u = 2 Ulysses ranks inside each of c = 4 ring ranks:
    all-to-all inside each ring group, the pass-KV ring over the 4 ring ranks on
    each 16q/4kv head group, inverse all-to-all. Sampled check: 6 rows of every
    (ring rank, Ulysses rank) (its first, last and four between) x all 32 heads
    against the oracle's unsplit attention over the whole sequence."""
    need_gpu()
    import torch
    import context_attention_amd as ca
    import synth
    w = synth.WORKLOADS["gqa"]
    S, H, G, d, u, c = w.total_tokens, w.n_hq, w.n_kv, w.head_dim, 2, 4
    log(f"hybrid full size S={S} heads={H}/{G} d={d} u={u} c={c}")
    pos = [ca.balanced_split(w.cu_seqlens, c, j)[0] for j in range(c)]
    L = len(pos[0])
    R = L // u
    q = synth.tensor_torch(w.seed, synth.TENSOR_Q, (S, H, d), w.scale_in, w.dtype, "cuda")
    k = synth.tensor_torch(w.seed, synth.TENSOR_K, (S, G, d), w.scale_in, w.dtype, "cuda")
    v = synth.tensor_torch(w.seed, synth.TENSOR_V, (S, G, d), w.scale_in, w.dtype, "cuda")
    idx = [torch.from_numpy(p).to("cuda") for p in pos]
    seq = {n: [[t.index_select(0, idx[j][i * R:(i + 1) * R]).contiguous() for i in range(u)] for j in range(c)]
           for n, t in (("q", q), ("k", k), ("v", v))}
    head = {}
    for n, nh in (("q", H), ("k", G), ("v", G)):
        head[n] = []
        for j in range(c):
            dst = [torch.empty(L, nh // u, d, dtype=q.dtype, device="cuda") for _ in range(u)]
            ca.ulysses_all_to_all(seq[n][j], dst, nh, "seq_to_head")
            head[n].append(dst)
    desc = ca.PrefillDesc(cp=c, cu_seqlens=w.cu_seqlens, n_hq=H // u, n_kv=G // u, head_dim=d, dtype=w.dtype,
                          scale=w.softmax_scale)
    kn = k.view(torch.int16).cpu().numpy().view(np.uint16)
    vn = v.view(torch.int16).cpu().numpy().view(np.uint16)
    for r in range(c):
        out_h, lse_h = [], []
        for i in range(u):
            acc = ca.new_partial(L, H // u, d)
            for t in range(c):
                j = (r - t) % c
                ca.ring_step_partial(desc, r, t, head["q"][r][i], head["k"][j][i], head["v"][j][i], acc,
                                     accumulate=t > 0)
            out_h.append(torch.empty(L, H // u, d, device="cuda"))
            lse_h.append(torch.empty(L, H // u, device="cuda"))
            ca.merge(acc, [], out=out_h[i], lse=lse_h[i])
        out_s = [torch.empty(R, H, d, device="cuda") for _ in range(u)]
        lse_s = [torch.empty(R, H, device="cuda") for _ in range(u)]
        ca.ulysses_all_to_all(out_h, out_s, H, "head_to_seq")
        ca.ulysses_all_to_all(lse_h, lse_s, H, "head_to_seq")
        torch.cuda.synchronize()
        for i in range(u):
            local = np.unique(np.linspace(0, R - 1, 6).astype(np.int64))
            gpos = pos[r][i * R + local]
            qr = q[torch.from_numpy(gpos).to("cuda")].view(torch.int16).cpu().numpy().view(np.uint16)
            ro, rl = oracle.attention_reference_rows(qr, gpos, kn, vn, w.softmax_scale)
            sel = torch.from_numpy(local).to("cuda")
            compare(f"ring rank {r}, Ulysses rank {i}", out_s[i][sel].cpu().numpy(), lse_s[i][sel].cpu().numpy(),
                    ro, rl, TOL_BF16)
