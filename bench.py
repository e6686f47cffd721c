"""Benchmark of the context-parallel attention hot path on one MI355X.

One step = one pass of the whole path on synthetic inputs already resident in
HBM:
  * prefill (pass-KV) on rank 0's share of the 1M-token workload (S = 1048576,
    cp = 8, 32 q / 8 kv heads, head_dim 128, bf16): the balanced split, the
    8 ring steps (each a pointer select of the block of rank (0 - t) mod 8 and
    one fused cpattn_ring_step_partial launch), and the merge / finalize;
  * pass-Q decode (b = 8, kv_len = 1048576 in cp = 8 shards, same heads): the
    per-shard partials and the three-quantity reduction;
  * the byte / FLOP account of both.

Printed: one JSON line. `value` is the prefill ring-step throughput in TFLOP/s
(exact causal FLOPs of rank 0's 8 steps / time of those launches); the decode
HBM throughput rides along under "decode". `roofline` covers the dominant
kernel (the ring-step partial), timed with HIP events on the launch stream;
`cpu_baseline` times the fp64 oracle on a bounded sample on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill ring-step TFLOP/s (% MFMA peak); pass-Q decode HBM GB/s (% peak)"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline_prefill(w, rows=64, target_s=15.0):
    """The oracle (fp64 numpy) on a bounded sample of the prefill metric's unit
    of work: tail-chunk query rows of rank 0 x all 32 heads against the full KV
    block of rank 7 (ring step 1, every key visible). A first pass on `rows`
    rows sizes the reported pass to about `target_s` seconds."""
    import oracle
    import synth
    S, cp, H, G, d = w.total_tokens, w.cp, w.n_hq, w.n_kv, w.head_dim
    c = S // (2 * cp)
    tail0 = (2 * cp - 1) * c
    qs = synth.tensor_np(w.seed, synth.TENSOR_Q, (S, H, d), w.scale_in, w.dtype, row_start=tail0, rows=rows)
    # rank 7 holds chunks 7 and 8
    kb = np.concatenate([synth.tensor_np(w.seed, synth.TENSOR_K, (S, G, d), w.scale_in, w.dtype,
                                         row_start=ch * c, rows=c) for ch in (7, 8)])
    vb = np.concatenate([synth.tensor_np(w.seed, synth.TENSOR_V, (S, G, d), w.scale_in, w.dtype,
                                         row_start=ch * c, rows=c) for ch in (7, 8)])
    n = kb.shape[0]
    t0 = time.perf_counter()
    oracle.partial_attention(qs, kb, vb, np.arange(rows), np.arange(n), None, w.softmax_scale, causal=False)
    dt = time.perf_counter() - t0
    more = int(min(2048, max(rows, rows * target_s / max(dt, 1e-3))) // 64 * 64)
    if more > rows:
        rows = more
        qs = synth.tensor_np(w.seed, synth.TENSOR_Q, (S, H, d), w.scale_in, w.dtype, row_start=tail0, rows=rows)
        t0 = time.perf_counter()
        oracle.partial_attention(qs, kb, vb, np.arange(rows), np.arange(n), None, w.softmax_scale, causal=False)
        dt = time.perf_counter() - t0
    flops = 4 * d * H * rows * n
    cores = len(os.sched_getaffinity(0))
    step_flops = 4 * d * H * c * n   # one ring step of rank 0 at t >= 1: its c tail-chunk rows see every key of the block
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} tail-chunk query rows of rank 0 x {H} heads against rank 7's full KV block "
                      f"({n} keys, ring step 1, no mask): {flops:.3e} flop in {dt:.2f} s (fp64 numpy)",
            "extrapolated_step_s": round(step_flops / (flops / dt), 1),
            "seconds": dt}


def cpu_baseline_configs():
    """The oracle (fp64 numpy, the same code the parity tests use) timed beside
    the other workloads, each on the unit of work the GPU figure is quoted on
    or a bounded sample of it:
      tiny     the full problem: every rank's ring (partials and merges), the
               unsplit two-pass reference and the pure-Python brute force;
      gqa      one ring-step partial in full: rank 0 at step 1 (its 2048
               tail-chunk rows x 32 heads against rank 7's block of 4096 keys,
               all visible; the head-chunk rows see no key);
      decode   one (batch entry, kv head, shard): 4 query heads against 131072
               keys; the full decode (8 x 8 x 8 such units) is extrapolated;
      varlen   rank 0 at step 1 of the wide-head workload on a sample: the
               tail-chunk rows of every sequence that fall on every 16th row,
               8 of the 64 heads, against the block of rank 3; the full call is
               extrapolated by exact FLOPs.
    Extrapolated times are labelled as such."""
    import oracle
    import synth
    out = {}
    perf = time.perf_counter
    # ---- tiny: everything
    w = synth.WORKLOADS["tiny"]
    S = w.total_tokens
    q, k, v = (synth.tensor_np(w.seed, t, (S, w.n_hq, w.head_dim), w.scale_in, w.dtype)
               for t in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V))
    t0 = perf()
    oracle.ring_prefill(q, k, v, w.cu_seqlens, w.cp, w.softmax_scale)
    t1 = perf()
    oracle.attention_reference(q, k, v, w.cu_seqlens, w.softmax_scale)
    t2 = perf()
    oracle.brute_force_attention(q, k, v, w.cu_seqlens, w.softmax_scale)
    t3 = perf()
    out["tiny_prefill"] = {"sample": "the full problem", "ring_s": round(t1 - t0, 4),
                           "reference_s": round(t2 - t1, 4), "brute_force_s": round(t3 - t2, 3)}
    # ---- gqa: rank 0, step 1, in full
    w = synth.WORKLOADS["gqa"]
    S, cp, H, G, d = w.total_tokens, w.cp, w.n_hq, w.n_kv, w.head_dim
    c = S // (2 * cp)
    qs = synth.tensor_np(w.seed, synth.TENSOR_Q, (S, H, d), w.scale_in, w.dtype, row_start=(2 * cp - 1) * c, rows=c)
    kb = synth.tensor_np(w.seed, synth.TENSOR_K, (S, G, d), w.scale_in, w.dtype, row_start=(cp - 1) * c, rows=2 * c)
    vb = synth.tensor_np(w.seed, synth.TENSOR_V, (S, G, d), w.scale_in, w.dtype, row_start=(cp - 1) * c, rows=2 * c)
    t0 = perf()
    oracle.partial_attention(qs, kb, vb, np.arange(c), np.arange(2 * c), None, w.softmax_scale, causal=False)
    dt = perf() - t0
    flops = 4 * d * H * c * 2 * c
    out["gqa_prefill"] = {"sample": f"one ring-step partial in full (rank 0, step 1: {c} rows x {H} heads x {2 * c} keys)",
                          "seconds": round(dt, 3), "flops": flops, "gflop_per_s": round(flops / dt / 1e9, 2)}
    # ---- decode: one (batch entry, kv head, shard), extrapolated
    w = synth.WORKLOADS["decode"]
    b, Sd, dcp, H, G, d = w.batch, w.kv_len, w.cp, w.n_hq, w.n_kv, w.head_dim
    n = Sd // dcp
    rep = H // G
    qd = synth.tensor_np(w.seed, synth.TENSOR_Q, (b, H, d), w.scale_in, w.dtype)[:1, :rep]
    kd = synth.head_slice_np(w.seed, synth.TENSOR_K, (b * Sd, G, d), 0, w.scale_in, w.dtype, row_start=0, rows=n)
    vd = synth.head_slice_np(w.seed, synth.TENSOR_V, (b * Sd, G, d), 0, w.scale_in, w.dtype, row_start=0, rows=n)
    t0 = perf()
    oracle.passq_decode(qd, kd[None], vd[None], 1, w.softmax_scale)
    dt = perf() - t0
    units = b * G * dcp
    kv_bytes = 2 * n * d * 2
    out["pass_q_decode"] = {"sample": f"one (batch entry, kv head, shard): {rep} query heads x {n} keys; "
                                      f"the full decode is {units} such units",
                            "seconds": round(dt, 3), "kv_gb_per_s": round(kv_bytes / dt / 1e9, 3),
                            "extrapolated_full_s": round(dt * units, 1)}
    # ---- varlen: rank 0, step 1, sampled rows and heads, extrapolated
    w = synth.WORKLOADS["varlen"]
    cp, H, d = w.cp, w.n_hq, w.head_dim
    heads = list(range(0, H, 8))
    cu = w.cu_seqlens
    t_sum, f_sum, f_full = 0.0, 0, 0
    for i, L in enumerate(w.seqlens):
        c = L // (2 * cp)
        start = int(cu[i])
        rows = np.arange((2 * cp - 1) * c, 2 * cp * c, 16)
        f_full += 4 * d * H * c * 2 * c
        for hh in heads:
            qh = synth.values_at_np(w.seed, synth.TENSOR_Q, ((start + rows)[:, None] * H + hh) * d
                                    + np.arange(d)[None, :], w.scale_in, w.dtype)[:, None, :]
            kh = synth.head_slice_np(w.seed, synth.TENSOR_K, (w.total_tokens, H, d), hh, w.scale_in, w.dtype,
                                     row_start=start + (cp - 1) * c, rows=2 * c)
            vh = synth.head_slice_np(w.seed, synth.TENSOR_V, (w.total_tokens, H, d), hh, w.scale_in, w.dtype,
                                     row_start=start + (cp - 1) * c, rows=2 * c)
            t0 = perf()
            oracle.partial_attention(qh, kh, vh, np.arange(rows.size), np.arange(2 * c), None, w.softmax_scale,
                                     causal=False)
            t_sum += perf() - t0
            f_sum += 4 * d * rows.size * 2 * c
    out["wide_varlen_prefill"] = {"sample": f"rank 0, step 1: every 16th tail-chunk row of each sequence, heads "
                                            f"{heads[0]}, {heads[1]}, ... ({len(heads)} of {H}) against rank 3's block",
                                  "seconds": round(t_sum, 3), "flops": f_sum,
                                  "gflop_per_s": round(f_sum / t_sum / 1e9, 2),
                                  "extrapolated_call_s": round(t_sum * f_full / f_sum, 1)}
    return out


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when the kernel sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, "context_attention_amd", "csrc", f), "rb").read())
    return rec["traffic_bytes"] if h.hexdigest() == rec["sha256"] else None


def overlap_report(ca, synth, torch):
    """The pass-KV ring of the whole CP group with its block transfers beside
    the ring steps (cpattn_ring_prefill_overlapped, three receive buffers per
    rank), after the timed steps. The link is the copy kernel on a few compute
    units set apart by CU masks (overlap.link_streams), about one xGMI link's
    rate. Reported: the spec's middle-band check on the GQA prefill workload
    (S=32768, cp=8; transfer/compute ratio in [0.5, 2]) and its large-S/cp
    metamorphic check on S=262144, cp=8 with the same heads (< 10% from pure
    compute)."""
    ov = ca.overlap
    comp, xfer = ov.link_streams(ov.LINK_CUS)
    rnd = lambda d: {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}
    res = {"transfer": f"copy kernel, {ov.LINK_WORKGROUPS} workgroups on {ov.LINK_CUS} CUs set apart by CU masks",
           "receive_buffers": 3}
    for key, w, fn in (("middle_band", synth.WORKLOADS["gqa"], ov.overlap_effective),
                       ("large_block", synth.PrefillWorkload(name="gqa 256k", seqlens=[262144], cp=8, n_hq=32,
                                                             n_kv=8, head_dim=128, dtype="bf16", scale_in=0.5,
                                                             seed=1), ov.overlap_metamorphic)):
        log(f"bench: overlap, {key}")
        S = w.total_tokens
        full = [synth.tensor_torch(w.seed, t, (S, h, w.head_dim), w.scale_in, w.dtype, "cuda")
                for t, h in ((synth.TENSOR_Q, w.n_hq), (synth.TENSOR_K, w.n_kv), (synth.TENSOR_V, w.n_kv))]
        qs, ks, vs = [], [], []
        for j in range(w.cp):
            idx = torch.from_numpy(ca.balanced_split(w.cu_seqlens, w.cp, j)[0]).to("cuda")
            for lst, t in zip((qs, ks, vs), full):
                lst.append(t.index_select(0, idx).contiguous())
        del full
        desc = ca.PrefillDesc(cp=w.cp, cu_seqlens=w.cu_seqlens, n_hq=w.n_hq, n_kv=w.n_kv, head_dim=w.head_dim,
                              dtype=w.dtype, scale=w.softmax_scale)
        x = ov.make_inputs(desc, qs, ks, vs, n_recv=3)
        r = fn(x, ov.LINK_WORKGROUPS, comp, xfer, reps=5 if key == "middle_band" else 2)
        r.pop("workgroups")
        res[key] = dict(workload=f"S={S}, cp={w.cp}, {w.n_hq}q/{w.n_kv}kv, d{w.head_dim}, all ranks", **rnd(r))
        del x, qs, ks, vs
        torch.cuda.empty_cache()
    return res


def _full_ring_tflops(ca, synth, torch, w, reps=3):
    """Every rank's full ring (cp fused ring steps per rank, then finalize) of a
    prefill workload: exact causal FLOPs of all cp^2 ring-step launches / their
    HIP-event time on the launch stream, one event pair around each rank's cp
    back-to-back launches (the finalize between ranks is outside), summed over
    the ranks (median over reps). One more pass with an event pair around every
    launch gives the per-call figures."""
    S, cp, H, G, d = w.total_tokens, w.cp, w.n_hq, w.n_kv, w.head_dim
    cu = w.cu_seqlens
    q = synth.tensor_torch(w.seed, synth.TENSOR_Q, (S, H, d), w.scale_in, w.dtype, "cuda")
    k = synth.tensor_torch(w.seed, synth.TENSOR_K, (S, G, d), w.scale_in, w.dtype, "cuda")
    v = synth.tensor_torch(w.seed, synth.TENSOR_V, (S, G, d), w.scale_in, w.dtype, "cuda")
    loc = []
    for r in range(cp):
        idx = torch.from_numpy(ca.balanced_split(cu, cp, r)[0]).to("cuda")
        loc.append(tuple(t.index_select(0, idx).contiguous() for t in (q, k, v)))
    del q, k, v
    desc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=H, n_kv=G, head_dim=d, dtype=w.dtype, scale=w.softmax_scale)
    rows = S // cp
    acc = ca.new_partial(rows, H, d)
    out = torch.empty(rows, H, d, device="cuda")
    lse = torch.empty(rows, H, device="cuda")
    stream = torch.cuda.current_stream()
    exact = ca.account(cp=cp, n_hq=H, n_kv=G, head_dim=d, dtype_bytes=2, cu_seqlens=cu)
    flops = exact["rank_flops_exact"] * cp

    def ring(per_call):
        evs = []
        for r in range(cp):
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for t in range(cp):
                j = (r - t) % cp
                ca.ring_step_partial(desc, r, t, loc[r][0], loc[j][1], loc[j][2], acc, accumulate=t > 0)
                if per_call or t == cp - 1:
                    e1 = torch.cuda.Event(enable_timing=True)
                    e1.record(stream)
                    evs.append((e0, e1))
                    e0 = e1
            ca.merge(acc, [], out=out, lse=lse)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    ring(False)                     # warm-up
    totals = [sum(ring(False)) for _ in range(reps)]
    times = ring(True)              # per (rank, step); step 0 holds the diagonal triangles
    calls = np.array([(exact["step0_flops_exact"] if i % cp == 0 else exact["stepN_flops_exact"]) / (x * 1e-3) / 1e12
                      for i, x in enumerate(times)])
    ms = float(np.median(totals))
    del loc
    return {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "ring_ms": round(ms, 3), "launches": cp * cp, "flops": flops,
            "per_launch_events_ms": round(float(sum(times)), 3),
            "per_call_tflops": {"min": round(float(calls.min()), 1), "median": round(float(np.median(calls)), 1),
                                "max": round(float(calls.max()), 1)}}


def _decode_gbs(ca, torch, b, S, cp, H, G, d, reps=5):
    n = S // cp
    gen = torch.Generator(device="cuda").manual_seed(11)
    q = torch.randn(b, H, d, device="cuda", generator=gen).to(torch.bfloat16)
    ks = [torch.randn(b, n, G, d, device="cuda", generator=gen).to(torch.bfloat16) for _ in range(cp)]
    vs = [torch.randn(b, n, G, d, device="cuda", generator=gen).to(torch.bfloat16) for _ in range(cp)]
    desc = ca.DecodeDesc(batch=b, cp=cp, kv_len=S, n_hq=H, n_kv=G, head_dim=d, dtype="bf16", scale=d ** -0.5)
    sp = ca.new_partial(cp * b, H, d)
    out = torch.empty(b, H, d, device="cuda")
    lse = torch.empty(b, H, device="cuda")
    ws = torch.empty(max(ca.passq_workspace_bytes(desc), 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    ca.passq_decode(desc, q, ks, vs, sp, out, lse, ws=ws)   # untimed
    torch.cuda.synchronize()
    # calls back to back between two events: the host enqueues ahead of the GPU,
    # so the binding's per-call host work is not in the interval (median of 3)
    ts = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            ca.passq_decode(desc, q, ks, vs, sp, out, lse, ws=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / reps)
    ms = float(np.median(ts))
    kv = 2 * b * S * G * d * 2
    byts = kv + q.numel() * 2 + cp * b * H * (d + 2) * 4 + b * H * (d + 1) * 4
    del ks, vs
    return {"ms": round(ms, 3), "gb_per_s": round(byts / (ms * 1e-3) / 1e9, 1),
            "frac": round(byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "bytes": byts}


def _ulysses_gqa(ca, synth, torch, w, u=8, reps=3):
    """Ulysses attention of a prefill workload over u ranks emulated on the GPU:
    the token shards (u consecutive row slices) of Q, K, V go through the
    all-to-all to head shards (n_hq/u query, n_kv/u kv heads over all tokens),
    each rank runs the unsplit causal attention over its heads (a ring step with
    cp = 1, then finalize), and out and lse go back through the inverse
    all-to-all. Reported: the all-to-all's HBM throughput (every byte read once
    and written once) and the attention's TFLOP/s (exact causal FLOPs over the
    summed kernel time), each from HIP events; median over reps."""
    S, H, G, d = w.total_tokens, w.n_hq, w.n_kv, w.head_dim
    R = S // u
    q = synth.tensor_torch(w.seed, synth.TENSOR_Q, (S, H, d), w.scale_in, w.dtype, "cuda")
    k = synth.tensor_torch(w.seed, synth.TENSOR_K, (S, G, d), w.scale_in, w.dtype, "cuda")
    v = synth.tensor_torch(w.seed, synth.TENSOR_V, (S, G, d), w.scale_in, w.dtype, "cuda")
    seq = {n: [t[i * R:(i + 1) * R].contiguous() for i in range(u)] for n, t in (("q", q), ("k", k), ("v", v))}
    del q, k, v
    head = {n: [torch.empty(S, nh // u, d, dtype=seq[n][0].dtype, device="cuda") for _ in range(u)]
            for n, nh in (("q", H), ("k", G), ("v", G))}
    desc = ca.PrefillDesc(cp=1, cu_seqlens=w.cu_seqlens, n_hq=H // u, n_kv=G // u, head_dim=d, dtype=w.dtype,
                          scale=w.softmax_scale)
    acc = [ca.new_partial(S, H // u, d) for _ in range(u)]
    out_h = [torch.empty(S, H // u, d, device="cuda") for _ in range(u)]
    lse_h = [torch.empty(S, H // u, device="cuda") for _ in range(u)]
    out_s = [torch.empty(R, H, d, device="cuda") for _ in range(u)]
    lse_s = [torch.empty(R, H, device="cuda") for _ in range(u)]
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    a2a_ms, att_ms, tot_ms = [], [], []
    for rep_i in range(reps + 1):
        e = [ev() for _ in range(5)]
        e[0].record(stream)
        for n, nh in (("q", H), ("k", G), ("v", G)):
            ca.ulysses_all_to_all(seq[n], head[n], nh, "seq_to_head")
        e[1].record(stream)
        for i in range(u):
            ca.ring_step_partial(desc, 0, 0, head["q"][i], head["k"][i], head["v"][i], acc[i], accumulate=False)
        e[2].record(stream)
        for i in range(u):
            ca.merge(acc[i], [], out=out_h[i], lse=lse_h[i])
        e[3].record(stream)
        ca.ulysses_all_to_all(out_h, out_s, H, "head_to_seq")
        ca.ulysses_all_to_all(lse_h, lse_s, H, "head_to_seq")
        e[4].record(stream)
        torch.cuda.synchronize()
        if rep_i:
            a2a_ms.append(e[0].elapsed_time(e[1]) + e[3].elapsed_time(e[4]))
            att_ms.append(e[1].elapsed_time(e[2]))
            tot_ms.append(e[0].elapsed_time(e[4]))
    a2a_bytes = 2 * (S * (H + 2 * G) * d * 2 + S * H * (d + 1) * 4)
    flops = ca.account(cp=1, n_hq=H, n_kv=G, head_dim=d, dtype_bytes=2, cu_seqlens=w.cu_seqlens)["rank_flops_exact"]
    a, t, tot = float(np.median(a2a_ms)), float(np.median(att_ms)), float(np.median(tot_ms))
    return {"u": u, "all_to_all_ms": round(a, 3), "all_to_all_gb_per_s": round(a2a_bytes / (a * 1e-3) / 1e9, 1),
            "all_to_all_frac": round(a2a_bytes / (a * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "all_to_all_bytes": a2a_bytes,
            "attention_ms": round(t, 3), "attention_tflops": round(flops / (t * 1e-3) / 1e12, 1),
            "attention_frac": round(flops / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "total_ms": round(tot, 3),
            "flops": flops}


def _hybrid_gqa(ca, synth, torch, w, u=2, c=4, reps=3):
    """Hybrid CP of a prefill workload, u Ulysses ranks inside each of c ring
    ranks (cp = u c), emulated on the GPU: ring rank j holds the balanced
    split's rows of rank j over c ranks and its u Ulysses ranks consecutive
    slices of them; the all-to-all inside each ring group gives every Ulysses
    rank all L = S/c rows of its ring rank for n_hq/u query and n_kv/u kv heads;
    the pass-KV ring runs over the c ring ranks on each head group (c fused ring
    steps per (ring rank, head group), then finalize); the inverse all-to-all
    returns out and lse to the token slices. Reported: the all-to-alls' HBM
    throughput (every byte read once and written once) and the rings' TFLOP/s
    (exact causal FLOPs over the HIP-event time of each (ring rank, head group)'s
    c back-to-back launches, summed); median over reps."""
    S, H, G, d = w.total_tokens, w.n_hq, w.n_kv, w.head_dim
    cu = w.cu_seqlens
    pos = [ca.balanced_split(cu, c, j)[0] for j in range(c)]
    L = len(pos[0])
    R = L // u
    q = synth.tensor_torch(w.seed, synth.TENSOR_Q, (S, H, d), w.scale_in, w.dtype, "cuda")
    k = synth.tensor_torch(w.seed, synth.TENSOR_K, (S, G, d), w.scale_in, w.dtype, "cuda")
    v = synth.tensor_torch(w.seed, synth.TENSOR_V, (S, G, d), w.scale_in, w.dtype, "cuda")
    idx = [torch.from_numpy(p).to("cuda") for p in pos]
    seq = {n: [[t.index_select(0, idx[j][i * R:(i + 1) * R]).contiguous() for i in range(u)] for j in range(c)]
           for n, t in (("q", q), ("k", k), ("v", v))}
    del q, k, v, idx
    head = {n: [[torch.empty(L, nh // u, d, dtype=seq[n][0][0].dtype, device="cuda") for _ in range(u)]
                for _ in range(c)] for n, nh in (("q", H), ("k", G), ("v", G))}
    desc = ca.PrefillDesc(cp=c, cu_seqlens=cu, n_hq=H // u, n_kv=G // u, head_dim=d, dtype=w.dtype,
                          scale=w.softmax_scale)
    acc = [[ca.new_partial(L, H // u, d) for _ in range(u)] for _ in range(c)]
    out_h = [[torch.empty(L, H // u, d, device="cuda") for _ in range(u)] for _ in range(c)]
    lse_h = [[torch.empty(L, H // u, device="cuda") for _ in range(u)] for _ in range(c)]
    out_s = [[torch.empty(R, H, d, device="cuda") for _ in range(u)] for _ in range(c)]
    lse_s = [[torch.empty(R, H, device="cuda") for _ in range(u)] for _ in range(c)]
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    a2a_ms, ring_ms, tot_ms = [], [], []
    for rep_i in range(reps + 1):
        e0, e1, e2, e3 = ev(), ev(), ev(), ev()
        e0.record(stream)
        for j in range(c):
            for n, nh in (("q", H), ("k", G), ("v", G)):
                ca.ulysses_all_to_all(seq[n][j], head[n][j], nh, "seq_to_head")
        e1.record(stream)
        rings = []
        for r in range(c):
            for i in range(u):
                a, b = ev(), ev()
                a.record(stream)
                for t in range(c):
                    j = (r - t) % c
                    ca.ring_step_partial(desc, r, t, head["q"][r][i], head["k"][j][i], head["v"][j][i], acc[r][i],
                                         accumulate=t > 0)
                b.record(stream)
                rings.append((a, b))
                ca.merge(acc[r][i], [], out=out_h[r][i], lse=lse_h[r][i])
        e2.record(stream)
        for j in range(c):
            ca.ulysses_all_to_all(out_h[j], out_s[j], H, "head_to_seq")
            ca.ulysses_all_to_all(lse_h[j], lse_s[j], H, "head_to_seq")
        e3.record(stream)
        torch.cuda.synchronize()
        if rep_i:
            a2a_ms.append(e0.elapsed_time(e1) + e2.elapsed_time(e3))
            ring_ms.append(sum(x.elapsed_time(y) for x, y in rings))
            tot_ms.append(e0.elapsed_time(e3))
    a2a_bytes = 2 * (S * (H + 2 * G) * d * 2 + S * H * (d + 1) * 4)
    flops = ca.account(cp=c, n_hq=H, n_kv=G, head_dim=d, dtype_bytes=2, cu_seqlens=cu)["rank_flops_exact"] * c
    a, t, tot = float(np.median(a2a_ms)), float(np.median(ring_ms)), float(np.median(tot_ms))
    return {"u": u, "c": c, "all_to_all_ms": round(a, 3), "all_to_all_gb_per_s": round(a2a_bytes / (a * 1e-3) / 1e9, 1),
            "all_to_all_frac": round(a2a_bytes / (a * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "all_to_all_bytes": a2a_bytes,
            "ring_ms": round(t, 3), "ring_tflops": round(flops / (t * 1e-3) / 1e12, 1),
            "ring_frac": round(flops / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "launches": u * c * c,
            "total_ms": round(tot, 3), "flops": flops}


def configs_report(ca, synth, torch):
    """The other workloads, after the timed steps: the GQA prefill and the
    wide-head varlen prefill as full rings over every rank, the pass-Q decode
    with one kv head (MQA 32/1 at head_dim 128; MLA-like 128/1 at head_dim 512;
    b = 8, kv_len = 1048576, cp = 8, K/V ~ N(0,1)), and the GQA prefill under
    Ulysses (u = 8) and hybrid CP (u = 2 inside c = 4 ring ranks)."""
    log("bench: GQA prefill, full ring")
    gqa = _full_ring_tflops(ca, synth, torch, synth.WORKLOADS["gqa"])
    torch.cuda.empty_cache()
    log("bench: wide-head varlen prefill, full ring")
    wide = _full_ring_tflops(ca, synth, torch, synth.WORKLOADS["varlen"], reps=2)
    torch.cuda.empty_cache()
    log("bench: single-kv-head decode")
    mqa = _decode_gbs(ca, torch, 8, 1 << 20, 8, 32, 1, 128)
    torch.cuda.empty_cache()
    mla = _decode_gbs(ca, torch, 8, 1 << 20, 8, 128, 1, 512)
    torch.cuda.empty_cache()
    log("bench: Ulysses attention of the GQA prefill")
    uly = _ulysses_gqa(ca, synth, torch, synth.WORKLOADS["gqa"])
    torch.cuda.empty_cache()
    log("bench: hybrid CP of the GQA prefill")
    hyb = _hybrid_gqa(ca, synth, torch, synth.WORKLOADS["gqa"])
    torch.cuda.empty_cache()
    return {
        "gqa_prefill": dict(workload="S=32768, cp=8, 32q/8kv, d128, bf16; all 8 ranks x 8 steps", **gqa),
        "wide_varlen_prefill": dict(workload=f"6 packed sequences ({synth.WORKLOADS['varlen'].total_tokens} tokens), "
                                             "cp=4, 64 heads, d512, bf16; all 4 ranks x 4 steps", **wide),
        "mqa_decode": dict(workload="b=8, kv_len=1048576, cp=8, 32q/1kv, d128, bf16", **mqa),
        "mla_like_decode": dict(workload="b=8, kv_len=1048576, cp=8, 128q/1kv, d512, bf16", **mla),
        "ulysses_gqa_prefill": dict(workload="S=32768, 32q/8kv, d128, bf16; Ulysses over u=8 ranks: all-to-all of "
                                             "Q, K, V, per-rank attention over 4q/1kv heads, inverse all-to-all "
                                             "of out and lse", **uly),
        "hybrid_gqa_prefill": dict(workload="S=32768, 32q/8kv, d128, bf16; hybrid CP, u=2 Ulysses ranks inside each "
                                            "of c=4 ring ranks: all-to-all inside ring groups, pass-KV ring over "
                                            "the ring ranks per head group (16q/4kv), inverse all-to-all", **hyb),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the measurements of the other workloads that follow the timed steps")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the transfer/compute overlap measurements that follow the timed steps")
    ap.add_argument("--config-only", choices=["gqa", "varlen", "mqa", "mla", "ulysses", "hybrid"], default=None,
                    help="measure only this workload of the configs report (for profiling its kernels) and "
                         "print its JSON; no headline step")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB "
                         "(reference for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (the cp ranks are emulated on it); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import context_attention_amd as ca
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ca.load()
    if args.config_only:
        if args.config_only in ("gqa", "varlen"):
            r = _full_ring_tflops(ca, synth, torch, synth.WORKLOADS[args.config_only], reps=args.steps)
        elif args.config_only == "ulysses":
            r = _ulysses_gqa(ca, synth, torch, synth.WORKLOADS["gqa"], reps=args.steps)
        elif args.config_only == "hybrid":
            r = _hybrid_gqa(ca, synth, torch, synth.WORKLOADS["gqa"], reps=args.steps)
        else:
            heads = {"mqa": (32, 128), "mla": (128, 512)}[args.config_only]
            r = _decode_gbs(ca, torch, 8, 1 << 20, 8, heads[0], 1, heads[1], reps=args.steps)
        print(json.dumps({"config": args.config_only, **r}), flush=True)
        return
    dev = "cuda"
    wp = synth.WORKLOADS["long"]
    wd = synth.WORKLOADS["decode"]
    S, cp, H, G, d = wp.total_tokens, wp.cp, wp.n_hq, wp.n_kv, wp.head_dim
    cu = wp.cu_seqlens
    rank = 0
    c = S // (2 * cp)
    rows = S // cp

    # ---------------- inputs, generated on the device (not timed)
    log("bench: generating prefill inputs")
    pos0, _ = ca.balanced_split(cu, cp, rank)
    q0 = torch.cat([synth.tensor_torch(wp.seed, synth.TENSOR_Q, (S, H, d), wp.scale_in, wp.dtype, dev,
                                       row_start=int(pos0[0]), rows=c),
                    synth.tensor_torch(wp.seed, synth.TENSOR_Q, (S, H, d), wp.scale_in, wp.dtype, dev,
                                       row_start=int(pos0[c]), rows=c)])
    kfull = synth.tensor_torch(wp.seed, synth.TENSOR_K, (S, G, d), wp.scale_in, wp.dtype, dev)
    vfull = synth.tensor_torch(wp.seed, synth.TENSOR_V, (S, G, d), wp.scale_in, wp.dtype, dev)
    blocks = []
    for j in range(cp):
        pj, _ = ca.balanced_split(cu, cp, j)
        idx = torch.from_numpy(pj).to(dev)
        blocks.append((kfull.index_select(0, idx).contiguous(), vfull.index_select(0, idx).contiguous()))
    del kfull, vfull
    acc = ca.new_partial(rows, H, d, dev)
    out = torch.empty(rows, H, d, device=dev)
    lse = torch.empty(rows, H, device=dev)
    pdesc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=H, n_kv=G, head_dim=d, dtype=wp.dtype, scale=wp.softmax_scale)

    log("bench: generating decode inputs")
    b, Sd, dcp = wd.batch, wd.kv_len, wd.cp
    n = Sd // dcp
    qd = synth.tensor_torch(wd.seed, synth.TENSOR_Q, (b, H, d), wd.scale_in, wd.dtype, dev)
    kshards, vshards = [], []
    for tid, lst in ((synth.TENSOR_K, kshards), (synth.TENSOR_V, vshards)):
        full = synth.tensor_torch(wd.seed, tid, (b * Sd, G, d), wd.scale_in, wd.dtype, dev).view(b, Sd, G, d)
        for s in range(dcp):
            lst.append(full[:, s * n:(s + 1) * n].contiguous())
        del full
    ddesc = ca.DecodeDesc(batch=b, cp=dcp, kv_len=Sd, n_hq=H, n_kv=G, head_dim=d, dtype=wd.dtype,
                          scale=wd.softmax_scale)
    sp = ca.new_partial(dcp * b, H, d, dev)
    dout = torch.empty(b, H, d, device=dev)
    dlse = torch.empty(b, H, device=dev)
    ws = torch.empty(max(ca.passq_workspace_bytes(ddesc), 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    acc_p = ca.account(cp=cp, n_hq=H, n_kv=G, head_dim=d, dtype_bytes=2, cu_seqlens=cu)
    acc_d = ca.account(cp=dcp, n_hq=H, n_kv=G, head_dim=d, dtype_bytes=2, batch=b, kv_len=Sd)
    stream = torch.cuda.current_stream()

    def step(rec):
        # A1 split (host) and A8 account are part of the step
        ca.balanced_split(cu, cp, rank)
        ca.account(cp=cp, n_hq=H, n_kv=G, head_dim=d, dtype_bytes=2, cu_seqlens=cu)
        for t in range(cp):
            j = (rank - t) % cp                 # A2: the block in hand at step t
            if rec is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            ca.ring_step_partial(pdesc, rank, t, q0, blocks[j][0], blocks[j][1], acc, accumulate=t > 0)
            if rec is not None:
                e1 = torch.cuda.Event(enable_timing=True)
                e1.record(stream)
                rec["ring"].append((e0, e1, t))
        ca.merge(acc, [], out=out, lse=lse)      # A4 finalize
        if rec is not None:
            e2 = torch.cuda.Event(enable_timing=True)
            e2.record(stream)
        ca.passq_decode(ddesc, qd, kshards, vshards, sp, dout, dlse, ws=ws)   # A5-A7
        if rec is not None:
            e3 = torch.cuda.Event(enable_timing=True)
            e3.record(stream)
            rec["decode"].append((e2, e3))

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    rec = {"ring": [], "decode": []}
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ring_ms = [a.elapsed_time(b_) for (a, b_, _) in rec["ring"]]
    dec_ms = [a.elapsed_time(b_) for (a, b_) in rec["decode"]]
    ring_flops = acc_p["rank_flops_exact"] * args.steps          # exact causal FLOPs of all timed ring launches
    tflops = ring_flops / (sum(ring_ms) * 1e-3) / 1e12
    per_launch_flops = acc_p["rank_flops_exact"] / cp
    avg_launch_s = float(np.mean(ring_ms)) * 1e-3
    achieved = per_launch_flops / avg_launch_s / 1e12
    # decode algorithmic bytes: KV + q + shard triples + out/lse
    dec_bytes = (acc_d["decode_kv_bytes_total"] + qd.numel() * 2 + dcp * b * H * (d + 2) * 4 + b * H * (d + 1) * 4)
    dec_gbs = dec_bytes / (float(np.mean(dec_ms)) * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "prefill: rank 0 share of S=1048576, cp=8 (2x65536 query rows x 8 ring-step KV blocks), "
                        "32q/8kv heads, head_dim 128, bf16 inputs ~N(0,1)*0.5, fp32 accumulate; "
                        "decode: b=8, kv_len=1048576 in cp=8 shards, 32q/8kv, head_dim 128, bf16",
            "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "ring_launch_ms": [round(x, 3) for x in ring_ms[:cp]],
        },
        "roofline": {
            "bound": "mfma", "kernel": "ring_step_mfma<128,4>",
            "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic("ring_step"),
            "flops_per_launch": per_launch_flops, "avg_launch_ms": round(avg_launch_s * 1e3, 3),
        },
        "decode": {
            "value": round(dec_gbs, 1), "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
            "ms": round(float(np.mean(dec_ms)), 3), "bytes": dec_bytes,
            "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("decode_partial")},
        },
    }
    del kshards, vshards
    if not args.no_overlap:
        res["overlap"] = overlap_report(ca, synth, torch)
    del blocks
    torch.cuda.empty_cache()
    if not args.no_configs:
        res["configs"] = configs_report(ca, synth, torch)
    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = src.numel() * 4
        del src, dst
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the CPU")
        cb = cpu_baseline_prefill(wp)
        cb.pop("seconds")
        log("bench: timing the oracle beside the other workloads")
        cb["configs"] = cpu_baseline_configs()
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
