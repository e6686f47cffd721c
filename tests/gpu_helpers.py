"""Shared pieces of the GPU parity tests: building inputs on the device with
the seeded generator, laying them out per rank with the library's split,
running the ring through the C-ABI binding, and comparing canonical forms."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

import synth

TOL_BF16 = 2e-2
TOL_F32 = 1e-5


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_attention_amd as ca
    ca.load()          # a missing library on a GPU machine is a failure, not a skip


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def np_to_device(a: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def global_inputs_np(lens, n_hq, n_kv, d, seed, dtype, scale):
    T = int(sum(lens))
    q = synth.tensor_np(seed, synth.TENSOR_Q, (T, n_hq, d), scale, dtype)
    k = synth.tensor_np(seed, synth.TENSOR_K, (T, n_kv, d), scale, dtype)
    v = synth.tensor_np(seed, synth.TENSOR_V, (T, n_kv, d), scale, dtype)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, cu


def local_buffers(ca, cu, cp, tensors_dev):
    """Per rank: (positions, [tensor[positions] for each device tensor])."""
    import torch
    out = []
    for r in range(cp):
        pos, _ = ca.balanced_split(cu, cp, r)
        idx = torch.from_numpy(pos).to(tensors_dev[0].device)
        out.append((pos, [t.index_select(0, idx).contiguous() for t in tensors_dev]))
    return out


def run_ring(ca, desc, local, fused=True, keep_partials=False):
    """Runs every (rank, step) ring partial through the C-ABI. Returns per rank
    the accumulator (fused) or the list of step partials, plus out / lse."""
    import torch
    cp = desc.cp
    rows = int(desc.cu_seqlens[-1]) // cp
    res = []
    for r in range(cp):
        q_r = local[r][1][0]
        acc = ca.new_partial(rows, desc.n_hq, desc.head_dim)
        parts = []
        for t in range(cp):
            j = (r - t) % cp
            k_j, v_j = local[j][1][1], local[j][1][2]
            if fused:
                ca.ring_step_partial(desc, r, t, q_r, k_j, v_j, acc, accumulate=(t > 0))
            else:
                p = ca.new_partial(rows, desc.n_hq, desc.head_dim)
                ca.ring_step_partial(desc, r, t, q_r, k_j, v_j, p, accumulate=False)
                parts.append(p)
        if not fused:
            acc = ca.Partial(parts[0].m.clone(), parts[0].den.clone(), parts[0].num.clone())
        out = torch.empty(rows, desc.n_hq, desc.head_dim, dtype=torch.float32, device="cuda")
        lse = torch.empty(rows, desc.n_hq, dtype=torch.float32, device="cuda")
        ca.merge(acc, parts[1:] if not fused else [], out=out, lse=lse)
        res.append(dict(acc=acc, parts=parts, out=out, lse=lse))
    torch.cuda.synchronize()
    return res


def canonical_np(m, den, num):
    """(num / den, m + ln den) with identity rows mapped to (0, -inf)."""
    m = np.asarray(m, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    num = np.asarray(num, dtype=np.float64)
    ok = den > 0
    out = np.zeros_like(num)
    out[ok] = num[ok] / den[ok][..., None]
    lse = np.full_like(m, -np.inf)
    lse[ok] = m[ok] + np.log(den[ok])
    return out, lse


def compare(name, got_out, got_lse, want_out, want_lse, tol):
    """Element-wise |diff| <= tol on out and lse; -inf entries must coincide."""
    got_out = np.asarray(got_out, dtype=np.float64)
    got_lse = np.asarray(got_lse, dtype=np.float64)
    ninf_g = np.isneginf(got_lse)
    ninf_w = np.isneginf(want_lse)
    assert np.array_equal(ninf_g, ninf_w), f"{name}: identity rows differ ({ninf_g.sum()} vs {ninf_w.sum()})"
    assert np.all(np.isfinite(got_out)), f"{name}: non-finite out"
    fin = ~ninf_w
    d_out = np.abs(got_out - want_out)
    d_lse = np.abs(got_lse[fin] - want_lse[fin]) if fin.any() else np.zeros(1)
    mo, ml = float(d_out.max(initial=0)), float(d_lse.max(initial=0))
    p_out = float(np.quantile(d_out, 0.999)) if d_out.size else 0.0
    log(f"  {name}: max|d out| {mo:.3e} (p99.9 {p_out:.3e})  max|d lse| {ml:.3e}  tol {tol:g}")
    assert mo <= tol and ml <= tol, f"{name}: out {mo:.3e} lse {ml:.3e} > {tol}"
    return mo, ml
