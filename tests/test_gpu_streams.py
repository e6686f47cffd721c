"""Reentrancy on the GPU: the library keeps no state between calls (every
call reads its description and enqueues on the caller's stream), so
independent calls issued on three streams at once, with no synchronisation
between them, give bit for bit what the same calls give one after another on
one stream. Three problems: a fused d128 bf16 GQA ring over two packed
sequences, a d64 fp32 ring with ragged chunks, and a pass-Q decode
(MQA 32/1 d128); each writes its own outputs."""
import numpy as np
import pytest

from gpu_helpers import global_inputs_np, local_buffers, log, need_gpu, np_to_device

pytestmark = pytest.mark.gpu


def _ring_problem(ca, lens, cp, n_hq, n_kv, d, dtype, seed):
    qn, kn, vn, cu = global_inputs_np(lens, n_hq, n_kv, d, seed=seed, dtype=dtype, scale=0.5)
    q, k, v = (np_to_device(a, dtype) for a in (qn, kn, vn))
    desc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=n_hq, n_kv=n_kv, head_dim=d, dtype=dtype,
                          scale=1.0 / np.sqrt(d))
    return desc, local_buffers(ca, cu, cp, [q, k, v])


def _enqueue_ring(ca, desc, local, stream):
    """Every rank's fused ring on `stream`; returns the accumulators."""
    import torch
    cp = desc.cp
    rows = int(desc.cu_seqlens[-1]) // cp
    accs = []
    with torch.cuda.stream(stream):
        for r in range(cp):
            acc = ca.new_partial(rows, desc.n_hq, desc.head_dim)
            for t in range(cp):
                j = (r - t) % cp
                ca.ring_step_partial(desc, r, t, local[r][1][0], local[j][1][1], local[j][1][2], acc,
                                     accumulate=t > 0, stream=stream)
            accs.append(acc)
    return accs


def _decode_problem(ca, seed):
    import torch
    b, S, cp, H, G, D = 2, 4 * 2000, 4, 32, 1, 128
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn(b, H, D, device="cuda", generator=g).to(torch.bfloat16)
    n = S // cp
    ks = [torch.randn(b, n, G, D, device="cuda", generator=g).to(torch.bfloat16) for _ in range(cp)]
    vs = [torch.randn(b, n, G, D, device="cuda", generator=g).to(torch.bfloat16) for _ in range(cp)]
    desc = ca.DecodeDesc(batch=b, cp=cp, kv_len=S, n_hq=H, n_kv=G, head_dim=D, dtype="bf16", scale=D ** -0.5)
    return desc, q, ks, vs


def _enqueue_decode(ca, desc, q, ks, vs, stream):
    import torch
    b, H, D, cp = desc.batch, desc.n_hq, desc.head_dim, desc.cp
    with torch.cuda.stream(stream):
        sp = ca.new_partial(cp * b, H, D)
        out = torch.empty(b, H, D, device="cuda")
        lse = torch.empty(b, H, device="cuda")
        ws = torch.empty(max(ca.passq_workspace_bytes(desc), 16), dtype=torch.uint8, device="cuda")
        ca.passq_decode(desc, q, ks, vs, sp, out, lse, ws=ws, stream=stream)
    return sp, out, lse, ws


def test_calls_on_three_streams_equal_the_calls_in_sequence():
    need_gpu()
    import torch
    import context_attention_amd as ca
    log("three problems on three streams against the same on one stream")
    pa = _ring_problem(ca, [1536, 512], 4, 8, 2, 128, "bf16", seed=31)
    pb = _ring_problem(ca, [6 * 37, 6 * 20], 3, 4, 4, 64, "f32", seed=32)
    pc = _decode_problem(ca, seed=33)
    torch.cuda.synchronize()
    s0 = torch.cuda.current_stream()
    ref_a = _enqueue_ring(ca, *pa, s0)
    ref_b = _enqueue_ring(ca, *pb, s0)
    ref_c = _enqueue_decode(ca, *pc, s0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    for rep in range(2):
        got_a = _enqueue_ring(ca, *pa, streams[0])
        got_c = _enqueue_decode(ca, *pc, streams[2])
        got_b = _enqueue_ring(ca, *pb, streams[1])
        torch.cuda.synchronize()
        for name, got, ref in (("ring A", got_a, ref_a), ("ring B", got_b, ref_b)):
            for r, (x, y) in enumerate(zip(got, ref)):
                for a, b in ((x.m, y.m), (x.den, y.den), (x.num, y.num)):
                    assert torch.equal(a, b), f"{name}, rank {r}, repetition {rep}: differs from the sequential run"
        for a, b in ((got_c[0].m, ref_c[0].m), (got_c[0].den, ref_c[0].den), (got_c[0].num, ref_c[0].num),
                     (got_c[1], ref_c[1]), (got_c[2], ref_c[2])):
            assert torch.equal(a, b), f"decode, repetition {rep}: differs from the sequential run"
