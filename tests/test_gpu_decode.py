"""GPU parity of pass-Q decode (cpattn_passq_decode) against the fp64 oracle
through the C-ABI binding: the per-shard partials (canonical form) and the
reduced result, element by element; at the full decode workload (b = 8,
kv_len = 1M, cp = 8) on a sampled (batch entry, kv group)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import TOL_BF16, TOL_F32, canonical_np, compare, log, need_gpu, np_to_device

pytestmark = pytest.mark.gpu

# name, batch, kv_len, cp, n_hq, n_kv, head_dim, dtype
CASES = [
    ("gqa4-bf16-d128-cp8", 3, 8 * 640, 8, 8, 2, 128, "bf16"),
    ("gqa4-bf16-d128-ragged-shards", 2, 4 * 1000, 4, 8, 2, 128, "bf16"),
    ("mha-bf16-d64-cp2", 2, 2 * 777, 2, 4, 4, 64, "bf16"),
    ("gqa8-bf16-d128-cp1", 2, 3000, 1, 8, 1, 128, "bf16"),
    ("gqa2-bf16-d512-cp4", 2, 4 * 300, 4, 4, 2, 512, "bf16"),
    ("gqa4-f32-d64-cp2", 2, 2 * 500, 2, 4, 1, 64, "f32"),
    ("tiny-keys-bf16-cp8", 1, 8, 8, 4, 2, 128, "bf16"),
    # groups of 16 or more query heads per kv head (MQA-like; bf16 runs decode_mfma)
    ("mqa32-bf16-d128-ragged-tiles", 2, 4 * 1000, 4, 32, 1, 128, "bf16"),
    ("mqa16-bf16-d64-half-block", 2, 2 * 777, 2, 16, 1, 64, "bf16"),
    ("mqa48-bf16-d64-two-blocks", 2, 2 * 5000, 2, 48, 1, 64, "bf16"),
    ("mla-like-128-bf16-d512-cp4", 2, 4 * 300, 4, 128, 1, 512, "bf16"),
    ("mqa40-bf16-d512-cp1", 1, 3000, 1, 40, 1, 512, "bf16"),
    ("gqa32-bf16-d128-two-kv-heads", 3, 8 * 640, 8, 64, 2, 128, "bf16"),
    ("mqa32-bf16-one-key-shards", 1, 8, 8, 32, 1, 128, "bf16"),
    # more than 32 query heads per kv head (bf16 runs decode_mfma16)
    ("gqa128-bf16-d128-8-waves", 2, 4 * 100, 4, 256, 2, 128, "bf16"),
    ("mqa96-bf16-d64-partial-head-blocks", 2, 2 * 777, 2, 96, 1, 64, "bf16"),
    ("mqa64-bf16-one-key-shards", 1, 8, 8, 64, 1, 128, "bf16"),
    # head_dim 512 with more than 112 query heads per kv head (decode_wide: 128 heads per workgroup)
    ("mla-like-128-bf16-d512-ragged-shards", 3, 3 * 1001, 3, 128, 1, 512, "bf16"),
    ("gqa128-bf16-d512-two-kv-heads", 2, 2 * 500, 2, 256, 2, 512, "bf16"),
    ("mqa192-bf16-d512-partial-head-block", 1, 4 * 200, 4, 192, 1, 512, "bf16"),
    ("mqa136-bf16-d512-one-key-shards", 2, 8, 8, 136, 1, 512, "bf16"),
    ("mqa16-f32-d128-head-blocks", 2, 2 * 500, 2, 16, 1, 128, "f32"),
    ("gqa16-f32-d64-two-kv-heads", 2, 2 * 300, 2, 32, 2, 64, "f32"),
]


def _run(ca, desc, q, ks, vs):
    import torch
    b, H, D, cp = desc.batch, desc.n_hq, desc.head_dim, desc.cp
    sp = ca.new_partial(cp * b, H, D)
    for x in (sp.m, sp.den, sp.num):
        x.fill_(float("nan"))
    out = torch.full((b, H, D), float("nan"), device="cuda")
    lse = torch.full((b, H), float("nan"), device="cuda")
    ca.passq_decode(desc, q, ks, vs, sp, out, lse)
    torch.cuda.synchronize()
    return sp, out, lse


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(case):
    need_gpu()
    import context_attention_amd as ca
    name, b, S, cp, H, G, D, dtype = case
    log(f"[decode parity] {name} b={b} kv_len={S} cp={cp} heads={H}/{G} d={D} {dtype}")
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    q = synth.tensor_np(9, synth.TENSOR_Q, (b, H, D), 1.0, dtype)
    k = synth.tensor_np(9, synth.TENSOR_K, (b, S, G, D), 1.0, dtype)
    v = synth.tensor_np(9, synth.TENSOR_V, (b, S, G, D), 1.0, dtype)
    n = S // cp
    ks = [np_to_device(np.ascontiguousarray(k[:, s * n:(s + 1) * n]), dtype) for s in range(cp)]
    vs = [np_to_device(np.ascontiguousarray(v[:, s * n:(s + 1) * n]), dtype) for s in range(cp)]
    desc = ca.DecodeDesc(batch=b, cp=cp, kv_len=S, n_hq=H, n_kv=G, head_dim=D, dtype=dtype, scale=1 / np.sqrt(D))
    sp, out, lse = _run(ca, desc, np_to_device(q, dtype), ks, vs)
    shards, wo, wl = oracle.passq_decode(q, k, v, cp, 1 / np.sqrt(D))
    m = sp.m.cpu().numpy().reshape(cp, b, H)
    den = sp.den.cpu().numpy().reshape(cp, b, H)
    num = sp.num.cpu().numpy().reshape(cp, b, H, D)
    for s in range(cp):
        go, gl = canonical_np(m[s], den[s], num[s])
        so, sl = oracle.finalize(shards[s])
        compare(f"shard {s}", go, gl, so, sl, tol)
    compare("reduced", out.cpu().numpy(), lse.cpu().numpy(), wo, wl, tol)


def test_decode_empty_kv():
    """kv_len = 0: every shard is the identity and the result is out = 0,
    lse = -inf."""
    need_gpu()
    import torch
    import context_attention_amd as ca
    b, H, G, D, cp = 2, 4, 2, 128, 2
    q = torch.zeros(b, H, D, dtype=torch.bfloat16, device="cuda")
    ks = [torch.zeros(b, 0, G, D, dtype=torch.bfloat16, device="cuda") for _ in range(cp)]
    desc = ca.DecodeDesc(batch=b, cp=cp, kv_len=0, n_hq=H, n_kv=G, head_dim=D, dtype="bf16", scale=0.1)
    sp, out, lse = _run(ca, desc, q, ks, ks)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(torch.isneginf(sp.m)) and torch.all(sp.den == 0)


def test_decode_workload_full_size_sampled():
    """The decode workload: b = 8, kv_len = 1048576 in cp = 8 shards of 131072,
    32/8 heads, d = 128, bf16. Sampled check: batch entry 5, kv head 6 (q
    heads 24..27): the 8 shard partials and the reduced output against the
    oracle over that kv head's 1M keys."""
    need_gpu()
    import torch
    import context_attention_amd as ca
    w = synth.WORKLOADS["decode"]
    b, S, cp, H, G, D = w.batch, w.kv_len, w.cp, w.n_hq, w.n_kv, w.head_dim
    log(f"[decode full] {w.name}")
    n = S // cp
    q = synth.tensor_torch(w.seed, synth.TENSOR_Q, (b, H, D), w.scale_in, w.dtype, "cuda")
    ks, vs = [], []
    for tid, lst in ((synth.TENSOR_K, ks), (synth.TENSOR_V, vs)):
        full = synth.tensor_torch(w.seed, tid, (b * S, G, D), w.scale_in, w.dtype, "cuda").view(b, S, G, D)
        for s in range(cp):
            lst.append(full[:, s * n:(s + 1) * n].contiguous())
        del full
    torch.cuda.synchronize()
    desc = ca.DecodeDesc(batch=b, cp=cp, kv_len=S, n_hq=H, n_kv=G, head_dim=D, dtype=w.dtype, scale=w.softmax_scale)
    sp, out, lse = _run(ca, desc, q, ks, vs)
    bi, g = 5, 6
    heads = np.arange(g * (H // G), (g + 1) * (H // G))
    log("  oracle: generating one (batch, kv head) slice of 1M keys")
    # K[bi, :, g, :] of the [b, S, G, D] tensor, as [1, S, 1, D]
    kg = synth.head_slice_np(w.seed, synth.TENSOR_K, (b * S, G, D), g, w.scale_in, w.dtype,
                             row_start=bi * S, rows=S)[None]
    vg = synth.head_slice_np(w.seed, synth.TENSOR_V, (b * S, G, D), g, w.scale_in, w.dtype,
                             row_start=bi * S, rows=S)[None]
    qg = synth.tensor_np(w.seed, synth.TENSOR_Q, (b, H, D), w.scale_in, w.dtype)[bi:bi + 1, heads]
    shards, wo, wl = oracle.passq_decode(qg, kg, vg, cp, w.softmax_scale)
    m = sp.m.cpu().numpy().reshape(cp, b, H)
    den = sp.den.cpu().numpy().reshape(cp, b, H)
    num = sp.num.cpu().numpy().reshape(cp, b, H, D)
    for s in range(cp):
        go, gl = canonical_np(m[s, bi, heads], den[s, bi, heads], num[s, bi, heads])
        so, sl = oracle.finalize(shards[s])
        compare(f"shard {s}", go, gl, so[0], sl[0], TOL_BF16)
    compare("reduced", out[bi, heads].cpu().numpy(), lse[bi, heads].cpu().numpy(), wo[0], wl[0], TOL_BF16)
    # every output is finite and every lse is a real number (all rows saw keys)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()


def test_mla_like_decode_full_size_sampled():
    """The MLA-like decode at the size the bench times: b = 8, kv_len = 1048576 in
    cp = 8 shards, 128 query heads on one kv head, head_dim 512, bf16 (it runs
    decode_wide). Sampled check: batch entry 3, query heads 5, 21, ..., 117 (one
    in every 16-head block, so every wave of the workload's workgroups): the 8
    shard partials and the reduced output against the oracle over the 1M keys.
    The K/V slice of that batch entry is the shared input generator's output
    (generated on the device, copied to the host)."""
    need_gpu()
    import torch
    import context_attention_amd as ca
    b, S, cp, H, G, D = 8, 1 << 20, 8, 128, 1, 512
    seed, scale_in = 23, 1.0
    scale = D ** -0.5
    log(f"[decode full] MLA-like b={b} kv_len={S} cp={cp} heads={H}/{G} d={D}")
    n = S // cp
    q = synth.tensor_torch(seed, synth.TENSOR_Q, (b, H, D), scale_in, "bf16", "cuda")
    ks, vs, host = [], [], {}
    bi = 3
    for tid, lst in ((synth.TENSOR_K, ks), (synth.TENSOR_V, vs)):
        full = synth.tensor_torch(seed, tid, (b * S, G, D), scale_in, "bf16", "cuda").view(b, S, G, D)
        host[tid] = full[bi].view(torch.int16).cpu().numpy().view(np.uint16)[None]   # [1, S, 1, D] bf16 bits
        for s in range(cp):
            lst.append(full[:, s * n:(s + 1) * n].contiguous())
        del full
    torch.cuda.synchronize()
    desc = ca.DecodeDesc(batch=b, cp=cp, kv_len=S, n_hq=H, n_kv=G, head_dim=D, dtype="bf16", scale=scale)
    sp, out, lse = _run(ca, desc, q, ks, vs)
    del ks, vs
    heads = np.arange(5, H, 16)
    qg = synth.tensor_np(seed, synth.TENSOR_Q, (b, H, D), scale_in, "bf16")[bi:bi + 1, heads]
    log("  oracle: 8 query heads over the batch entry's 1M keys")
    shards, wo, wl = oracle.passq_decode(qg, host[synth.TENSOR_K], host[synth.TENSOR_V], cp, scale)
    m = sp.m.cpu().numpy().reshape(cp, b, H)
    den = sp.den.cpu().numpy().reshape(cp, b, H)
    num = sp.num.cpu().numpy().reshape(cp, b, H, D)
    for s in range(cp):
        go, gl = canonical_np(m[s, bi, heads], den[s, bi, heads], num[s, bi, heads])
        so, sl = oracle.finalize(shards[s])
        compare(f"shard {s}", go, gl, so[0], sl[0], TOL_BF16)
    compare("reduced", out[bi, heads].cpu().numpy(), lse[bi, heads].cpu().numpy(), wo[0], wl[0], TOL_BF16)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
