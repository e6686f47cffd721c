"""GPU parity of the padded layout: sequence lengths not divisible by 2*cp,
each sequence padded at its end to the next multiple of 2*cp (reading listed
with the oracle's balanced_split_padded). Every rank runs the fused ring
through the C-ABI on local buffers whose pad rows hold NaN (they must never be
read); real rows must match the oracle's padded ring, pad rows must hold the
identity triple."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL_BF16, TOL_F32, canonical_np, compare, global_inputs_np, log, need_gpu, np_to_device

pytestmark = pytest.mark.gpu

CASES = [
    # lens, cp, n_hq, n_kv, d, dtype
    ([5, 1000, 77, 0, 3], 4, 8, 2, 128, "bf16"),
    ([1, 2, 3, 4, 5, 6, 7, 300], 8, 4, 4, 64, "bf16"),
    ([513, 1031], 2, 4, 2, 512, "bf16"),
    ([10, 33, 2], 3, 4, 2, 128, "f32"),
    ([4097, 129], 4, 32, 8, 128, "bf16"),
]


def _padded_locals(ca, cu, cp, tensors):
    """Per rank: positions (-1 = pad) and the local copies of each tensor with
    NaN in the pad rows."""
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


@pytest.mark.parametrize("lens,cp,n_hq,n_kv,d,dtype", CASES,
                         ids=[f"cp{c[1]}-{c[5]}-d{c[4]}-{len(c[0])}seqs" for c in CASES])
def test_padded_ring_matches_oracle(lens, cp, n_hq, n_kv, d, dtype):
    need_gpu()
    import torch
    import context_attention_amd as ca
    log(f"padded ring lens={lens} cp={cp} heads={n_hq}/{n_kv} d={d} {dtype}")
    qn, kn, vn, cu = global_inputs_np(lens, n_hq, n_kv, d, seed=23, dtype=dtype, scale=0.5)
    q, k, v = (np_to_device(a, dtype) for a in (qn, kn, vn))
    scale = 1.0 / np.sqrt(d)
    desc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=n_hq, n_kv=n_kv, head_dim=d, dtype=dtype, scale=scale,
                          padded=True)
    local = _padded_locals(ca, cu, cp, [q, k, v])
    ref = oracle.ring_prefill_padded(qn, kn, vn, cu, cp, scale)
    rows = desc.rows
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for r in range(cp):
        pos, (q_r, _, _) = local[r]
        acc = ca.new_partial(rows, n_hq, d)
        for t in range(cp):
            j = (r - t) % cp
            ca.ring_step_partial(desc, r, t, q_r, local[j][1][1], local[j][1][2], acc, accumulate=t > 0)
        torch.cuda.synchronize()
        m, den, num = (x.cpu().numpy() for x in (acc.m, acc.den, acc.num))
        pad = pos < 0
        assert np.all(np.isneginf(m[pad])) and np.all(den[pad] == 0) and np.all(num[pad] == 0), \
            f"rank {r}: pad rows are not the identity"
        go, gl = canonical_np(m[~pad], den[~pad], num[~pad])
        compare(f"rank {r} real rows", go, gl, ref["out"][pos[~pad]], ref["lse"][pos[~pad]], tol)


def test_padded_ring_overlapped_equals_sequential():
    """The overlapped ring sizes its transfers from the padded local rows."""
    need_gpu()
    import torch
    import context_attention_amd as ca
    lens, cp, n_hq, n_kv, d = [1000, 37, 2049], 4, 8, 2, 128
    qn, kn, vn, cu = global_inputs_np(lens, n_hq, n_kv, d, seed=29, dtype="bf16", scale=0.5)
    q, k, v = (np_to_device(a, "bf16") for a in (qn, kn, vn))
    desc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=n_hq, n_kv=n_kv, head_dim=d, dtype="bf16",
                          scale=1.0 / np.sqrt(d), padded=True)
    local = _padded_locals(ca, cu, cp, [q, k, v])
    comp, xfer = torch.cuda.Stream(), torch.cuda.Stream()
    seqs = []
    for r in range(cp):
        q_r = local[r][1][0]
        seq = ca.new_partial(desc.rows, n_hq, d)
        for t in range(cp):
            j = (r - t) % cp
            ca.ring_step_partial(desc, r, t, q_r, local[j][1][1], local[j][1][2], seq, accumulate=t > 0)
        seqs.append(seq)
    x = ca.overlap.make_inputs(desc, [l[1][0] for l in local], [l[1][1] for l in local],
                               [l[1][2] for l in local])
    torch.cuda.synchronize()
    ca.ring_prefill_overlapped(desc, x.q, x.k_blocks, x.v_blocks, x.k_recv, x.v_recv, x.acc, 0, comp, xfer,
                               events=x.events)
    torch.cuda.synchronize()
    for r in range(cp):
        for a, b in ((x.acc[r].m, seqs[r].m), (x.acc[r].den, seqs[r].den), (x.acc[r].num, seqs[r].num)):
            assert torch.equal(a, b), f"rank {r}"
