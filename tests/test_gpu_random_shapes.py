"""GPU parity over shapes drawn at random from a fixed seed, beside the
hand-picked cases: head_dim 64/128/512, 1 to 4 kv heads with 1 to 32 query
heads each, cp from 1 to 8, 1 to 4 packed sequences of any admissible length
(with empty ones), the plain and the padded layout, bf16 and fp32, plus query
heads per kv head that are not powers of two (3, 5, 6, 12); and pass-Q
decode over batch, shard count, group size and head_dim (plus a set at head_dim
512 with 120 to 256 query heads per kv head). Every configuration
runs the whole fused ring of every rank (or the decode) through the C-ABI and
is compared with the fp64 oracle on every real row. The draw is deterministic,
so a failure names a reproducible case."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_helpers import (TOL_BF16, TOL_F32, canonical_np, compare, global_inputs_np, local_buffers, log, need_gpu,
                         np_to_device)
import synth

pytestmark = pytest.mark.gpu


def _prefill_cases(n, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(g.choice([64, 128, 512], p=[0.4, 0.4, 0.2]))
        n_kv = int(g.choice([1, 2, 4]))
        rep = int(g.choice([1, 2, 4, 8, 16, 32]))
        if d == 512 and n_kv * rep > 16:
            continue
        cp = int(g.choice([1, 2, 3, 4, 5, 8]))
        dtype = "f32" if g.random() < 0.15 else "bf16"
        padded = bool(g.random() < 0.4)
        ns = int(g.integers(1, 5))
        cap = 900 if d < 512 else 400
        if padded:
            lens = [int(x) for x in g.integers(0, cap // ns + 1, ns)]
        else:
            lens = [2 * cp * int(x) for x in g.integers(0, cap // (2 * cp * ns) + 1, ns)]
        if sum(lens) == 0:
            continue
        name = f"p{len(out):02d}-d{d}-h{n_kv * rep}x{n_kv}-cp{cp}-{dtype}-{'pad' if padded else 'exact'}-{ns}seq"
        out.append((name, lens, cp, n_kv * rep, n_kv, d, dtype, padded))
    return out


def _decode_cases(n, seed=2025):
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        D = int(g.choice([64, 128, 512], p=[0.4, 0.4, 0.2]))
        n_kv = int(g.choice([1, 2, 4]))
        rep = int(g.choice([1, 2, 4, 8, 16, 24, 32, 48, 64]))
        if D == 512 and n_kv * rep > 64:
            continue
        cp = int(g.choice([1, 2, 3, 4, 8]))
        b = int(g.integers(1, 4))
        S = cp * int(g.integers(1, 900 // cp + 1))
        dtype = "f32" if g.random() < 0.15 else "bf16"
        out.append((f"d{len(out):02d}-D{D}-h{n_kv * rep}x{n_kv}-cp{cp}-b{b}-S{S}-{dtype}", b, S, cp, n_kv * rep, n_kv,
                    D, dtype))
    return out


def _wide_decode_cases(n, seed=2026):
    """head_dim 512 with more than 112 query heads per kv head (the 128-head
    workgroups of the MLA-like layouts), bf16: full and partly filled head
    blocks, several kv heads, shards shorter than a 32-key tile."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        n_kv = int(g.choice([1, 2, 3]))
        rep = int(g.choice([120, 128, 136, 160, 192, 256]))
        cp = int(g.choice([1, 2, 3, 4, 8]))
        b = int(g.integers(1, 4))
        S = cp * int(g.integers(1, 400 // cp + 1))
        out.append((f"w{len(out):02d}-D512-h{n_kv * rep}x{n_kv}-cp{cp}-b{b}-S{S}-bf16", b, S, cp, n_kv * rep, n_kv,
                    512, "bf16"))
    return out


def _odd_group_cases(n, seed=2027):
    """Prefill with query heads per kv head that are not powers of two (3, 5,
    6, 12: head groups of 1, 2 and 4 heads per workgroup, head-group counts
    that are not multiples of 8, so the unit-major workgroup order) and 1 to 3
    kv heads."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(g.choice([64, 128, 512], p=[0.4, 0.4, 0.2]))
        n_kv = int(g.choice([1, 2, 3]))
        rep = int(g.choice([3, 5, 6, 12]))
        if d == 512 and n_kv * rep > 16:
            continue
        cp = int(g.choice([1, 2, 3, 4, 8]))
        dtype = "f32" if g.random() < 0.15 else "bf16"
        padded = bool(g.random() < 0.3)
        ns = int(g.integers(1, 4))
        cap = 900 if d < 512 else 400
        if padded:
            lens = [int(x) for x in g.integers(1, cap // ns + 1, ns)]
        else:
            lens = [2 * cp * int(x) for x in g.integers(1, cap // (2 * cp * ns) + 2, ns)]
        name = f"o{len(out):02d}-d{d}-h{n_kv * rep}x{n_kv}-cp{cp}-{dtype}-{'pad' if padded else 'exact'}-{ns}seq"
        out.append((name, lens, cp, n_kv * rep, n_kv, d, dtype, padded))
    return out


PREFILL = _prefill_cases(48) + _odd_group_cases(10)
DECODE = _decode_cases(32) + _wide_decode_cases(12)


def _padded_locals(ca, cu, cp, tensors):
    import torch
    out = []
    for r in range(cp):
        pos, _ = ca.balanced_split_padded(cu, cp, r)
        idx = torch.from_numpy(np.maximum(pos, 0)).to("cuda")
        pad = torch.from_numpy(pos < 0).to("cuda")
        locs = []
        for t in tensors:
            x = t.index_select(0, idx).contiguous()
            x[pad] = float("nan")
            locs.append(x)
        out.append((pos, locs))
    return out


@pytest.mark.parametrize("case", PREFILL, ids=[c[0] for c in PREFILL])
def test_random_prefill_shape(case):
    need_gpu()
    import torch
    import context_attention_amd as ca
    name, lens, cp, H, G, d, dtype, padded = case
    log(f"[random prefill] {name} lens={lens}")
    q, k, v, cu = global_inputs_np(lens, H, G, d, seed=31, dtype=dtype, scale=0.5 if dtype == "bf16" else 1.0)
    scale = 1.0 / np.sqrt(d)
    dev = [np_to_device(x, dtype) for x in (q, k, v)]
    desc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=H, n_kv=G, head_dim=d, dtype=dtype, scale=scale,
                          padded=padded)
    local = _padded_locals(ca, cu, cp, dev) if padded else local_buffers(ca, cu, cp, dev)
    want_out, want_lse = oracle.attention_reference(q, k, v, cu, scale)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    rows = desc.rows
    for r in range(cp):
        pos, (q_r, _, _) = local[r]
        acc = ca.new_partial(rows, H, d)
        for t in range(cp):
            j = (r - t) % cp
            ca.ring_step_partial(desc, r, t, q_r, local[j][1][1], local[j][1][2], acc, accumulate=t > 0)
        out = torch.empty(rows, H, d, device="cuda")
        lse = torch.empty(rows, H, device="cuda")
        ca.merge(acc, [], out=out, lse=lse)
        torch.cuda.synchronize()
        real = pos >= 0
        if real.any():
            compare(f"rank {r}", out.cpu().numpy()[real], lse.cpu().numpy()[real], want_out[pos[real]],
                    want_lse[pos[real]], tol)
        if padded and (~real).any():
            m, den = acc.m.cpu().numpy(), acc.den.cpu().numpy()
            assert np.all(np.isneginf(m[~real])) and np.all(den[~real] == 0), f"rank {r}: pad rows not the identity"


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_random_decode_shape(case):
    need_gpu()
    import torch
    import context_attention_amd as ca
    name, b, S, cp, H, G, D, dtype = case
    log(f"[random decode] {name}")
    sc = 1.0
    q = synth.tensor_np(33, synth.TENSOR_Q, (b, H, D), sc, dtype)
    k = synth.tensor_np(33, synth.TENSOR_K, (b, S, G, D), sc, dtype)
    v = synth.tensor_np(33, synth.TENSOR_V, (b, S, G, D), sc, dtype)
    n = S // cp
    ks = [np_to_device(np.ascontiguousarray(k[:, s * n:(s + 1) * n]), dtype) for s in range(cp)]
    vs = [np_to_device(np.ascontiguousarray(v[:, s * n:(s + 1) * n]), dtype) for s in range(cp)]
    desc = ca.DecodeDesc(batch=b, cp=cp, kv_len=S, n_hq=H, n_kv=G, head_dim=D, dtype=dtype, scale=1 / np.sqrt(D))
    sp = ca.new_partial(cp * b, H, D)
    out = torch.full((b, H, D), float("nan"), device="cuda")
    lse = torch.full((b, H), float("nan"), device="cuda")
    ca.passq_decode(desc, np_to_device(q, dtype), ks, vs, sp, out, lse)
    torch.cuda.synchronize()
    shards, wo, wl = oracle.passq_decode(q, k, v, cp, 1 / np.sqrt(D))
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    m = sp.m.cpu().numpy().reshape(cp, b, H)
    den = sp.den.cpu().numpy().reshape(cp, b, H)
    num = sp.num.cpu().numpy().reshape(cp, b, H, D)
    for s in range(cp):
        go, gl = canonical_np(m[s], den[s], num[s])
        so, sl = oracle.finalize(shards[s])
        compare(f"shard {s}", go, gl, so, sl, tol)
    compare("reduced", out.cpu().numpy(), lse.cpu().numpy(), wo, wl, tol)
