"""GPU parity of the tree-order reduction (cpattn_tree_reduce): the pass-Q
shard triples and a rank's ring-step partials merged in tree order, against
the oracle's tree merge and against the library's own linear reduction."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import (TOL_BF16, canonical_np, compare, global_inputs_np, local_buffers, log, need_gpu,
                         np_to_device, run_ring)

pytestmark = pytest.mark.gpu


def _views(part, n, rows):
    import context_attention_amd as ca
    return [ca.Partial(part.m[i * rows:(i + 1) * rows], part.den[i * rows:(i + 1) * rows],
                       part.num[i * rows:(i + 1) * rows]) for i in range(n)]


@pytest.mark.parametrize("cp,G", [(1, 2), (3, 2), (5, 1), (8, 2)])
def test_tree_reduce_of_decode_shards(cp, G):
    need_gpu()
    import torch
    import context_attention_amd as ca
    b, H, D, n = 2, 8, 128, 96
    S = cp * n
    log(f"[tree reduce] decode cp={cp} heads={H}/{G}")
    q = synth.tensor_np(13, synth.TENSOR_Q, (b, H, D), 1.0, "bf16")
    k = synth.tensor_np(13, synth.TENSOR_K, (b, S, G, D), 1.0, "bf16")
    v = synth.tensor_np(13, synth.TENSOR_V, (b, S, G, D), 1.0, "bf16")
    ks = [np_to_device(np.ascontiguousarray(k[:, s * n:(s + 1) * n]), "bf16") for s in range(cp)]
    vs = [np_to_device(np.ascontiguousarray(v[:, s * n:(s + 1) * n]), "bf16") for s in range(cp)]
    desc = ca.DecodeDesc(batch=b, cp=cp, kv_len=S, n_hq=H, n_kv=G, head_dim=D, dtype="bf16", scale=D ** -0.5)
    sp = ca.new_partial(cp * b, H, D)
    out = torch.empty(b, H, D, device="cuda")
    lse = torch.empty(b, H, device="cuda")
    ca.passq_decode(desc, np_to_device(q, "bf16"), ks, vs, sp, out, lse)
    out_t = torch.full((b, H, D), float("nan"), device="cuda")
    lse_t = torch.full((b, H), float("nan"), device="cuda")
    ca.tree_reduce(_views(sp, cp, b), out_t, lse_t)
    torch.cuda.synchronize()
    # the same triples merged in another order: equal up to fp32 rounding
    ot, lt, ol, ll = (x.cpu().numpy() for x in (out_t, lse_t, out, lse))
    assert np.abs(ot - ol).max() <= 1e-5 * max(1.0, np.abs(ol).max())
    assert np.abs(lt - ll).max() <= 1e-5 * max(1.0, np.abs(ll).max())
    shards, _, _ = oracle.passq_decode(q, k, v, cp, D ** -0.5)
    wo, wl = oracle.finalize(oracle.merge_tree(shards))
    compare("tree vs oracle", ot, lt, wo, wl, TOL_BF16)


def test_tree_reduce_of_ring_partials():
    """A rank's cp ring-step partials (unfused) merged in tree order equal the
    oracle's merged result for that rank."""
    need_gpu()
    import torch
    import context_attention_amd as ca
    lens, cp, H, G, d = [2 * 6 * 70, 2 * 6 * 33], 6, 4, 2, 128
    q, k, v, cu = global_inputs_np(lens, H, G, d, 5, "bf16", 0.5)
    dev = [np_to_device(x, "bf16") for x in (q, k, v)]
    local = local_buffers(ca, cu, cp, dev)
    desc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=H, n_kv=G, head_dim=d, dtype="bf16", scale=1.0 / np.sqrt(d))
    res = run_ring(ca, desc, local, fused=False)
    ref = oracle.ring_prefill(q, k, v, cu, cp, 1.0 / np.sqrt(d))
    for r in (0, cp - 1):
        parts = res[r]["parts"]
        rows = parts[0].m.shape[0]
        out_t = torch.empty(rows, H, d, device="cuda")
        lse_t = torch.empty(rows, H, device="cuda")
        ca.tree_reduce(parts, out_t, lse_t)
        torch.cuda.synchronize()
        pos = local[r][0]
        compare(f"rank {r} tree", out_t.cpu().numpy(), lse_t.cpu().numpy(), ref["out"][pos], ref["lse"][pos],
                TOL_BF16)
