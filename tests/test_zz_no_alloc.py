"""cpattn_passq_decode_noalloc, the pass-Q decode that allocates nothing (its
split triples live in the library's per-GPU scratch buffer), against
cpattn_passq_decode with a caller workspace: the same kernels and split plan,
so the per-shard triples, out and lse must be equal bit for bit. Two calls in
a row through the C ABI, the second on a smaller input, so the second reads a
scratch buffer that still holds the first call's contents. A description that
needs more workspace than the buffer holds is rejected before any device call.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import log, need_gpu, np_to_device

pytestmark = pytest.mark.gpu

# name, batch, kv_len, cp, n_hq, n_kv, head_dim (bf16): the vector kernel
# (4 query heads per kv head), then the matrix-core kernel on a smaller input
CALLS = [
    ("gqa4-d128-b4-cp4", 4, 4 * 16384, 4, 32, 8, 128),
    ("mqa16-d64-b2-cp2", 2, 2 * 3000, 2, 16, 1, 64),
]


def _inputs(ca, b, S, cp, H, G, D, seed):
    q = np_to_device(synth.tensor_np(seed, synth.TENSOR_Q, (b, H, D), 1.0, "bf16"), "bf16")
    k = synth.tensor_np(seed, synth.TENSOR_K, (b, S, G, D), 1.0, "bf16")
    v = synth.tensor_np(seed, synth.TENSOR_V, (b, S, G, D), 1.0, "bf16")
    n = S // cp
    ks = [np_to_device(np.ascontiguousarray(k[:, s * n:(s + 1) * n]), "bf16") for s in range(cp)]
    vs = [np_to_device(np.ascontiguousarray(v[:, s * n:(s + 1) * n]), "bf16") for s in range(cp)]
    desc = ca.DecodeDesc(batch=b, cp=cp, kv_len=S, n_hq=H, n_kv=G, head_dim=D, dtype="bf16", scale=D ** -0.5)
    return desc, q, ks, vs


def _outputs(ca, desc):
    import torch
    b, H, D = desc.batch, desc.n_hq, desc.head_dim
    sp = ca.new_partial(desc.cp * b, H, D)
    for x in (sp.m, sp.den, sp.num):
        x.fill_(float("nan"))
    return sp, torch.full((b, H, D), float("nan"), device="cuda"), torch.full((b, H), float("nan"), device="cuda")


def test_noalloc_decode_equals_decode_with_workspace_twice():
    need_gpu()
    import torch
    import context_attention_amd as ca
    for i, (name, b, S, cp, H, G, D) in enumerate(CALLS):
        log(f"[noalloc decode] call {i + 1}: {name}")
        desc, q, ks, vs = _inputs(ca, b, S, cp, H, G, D, seed=31 + i)
        assert ca.passq_workspace_bytes(desc) <= ca.NOALLOC_SCRATCH_BYTES
        ref_sp, ref_out, ref_lse = _outputs(ca, desc)
        ca.passq_decode(desc, q, ks, vs, ref_sp, ref_out, ref_lse)
        sp, out, lse = _outputs(ca, desc)
        ca.passq_decode_noalloc(desc, q, ks, vs, sp, out, lse)
        torch.cuda.synchronize()
        for what, got, want in (("out", out, ref_out), ("lse", lse, ref_lse), ("m", sp.m, ref_sp.m),
                                ("den", sp.den, ref_sp.den), ("num", sp.num, ref_sp.num)):
            assert torch.equal(got, want), f"{name}: {what} differs from cpattn_passq_decode"
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()


def test_noalloc_decode_rejects_a_workspace_past_the_buffer():
    """MLA-like 128/1 heads at head_dim 512, b = 8, kv_len = 1M, cp = 8 needs more
    split triples than the scratch buffer holds: E_WORKSPACE, nothing written."""
    need_gpu()
    import torch
    import context_attention_amd as ca
    desc = ca.DecodeDesc(batch=8, cp=8, kv_len=1 << 20, n_hq=128, n_kv=1, head_dim=512, dtype="bf16",
                         scale=512 ** -0.5)
    assert ca.passq_workspace_bytes(desc) > ca.NOALLOC_SCRATCH_BYTES
    n = desc.kv_len // desc.cp
    q = torch.zeros(8, 128, 512, dtype=torch.bfloat16, device="cuda")
    ks = [torch.zeros(8, n, 1, 512, dtype=torch.bfloat16, device="cuda") for _ in range(1)] * desc.cp
    sp, out, lse = _outputs(ca, desc)
    with pytest.raises(ca.CpattnError) as e:
        ca.passq_decode_noalloc(desc, q, ks, ks, sp, out, lse)
    assert e.value.code == ca.E_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(lse).all()
