"""GPU parity where the lazy rescale of the running max actually runs.

The kernels keep a reference max per row and rescale the numerator and the
denominator only when a tile's max exceeds it by more than 2^8 in the exp2
domain (8 ln 2 in natural units); with the standard inputs (scores of a few
units) that happens only at a row's first tile. Here the keys grow in
magnitude along the sequence (a geometric ramp per key row), so a row's
running max keeps rising from tile to tile (the rows whose query points
against the keys' direction keep their max at the start, so about half the
rows is the natural share): a CPU check on the inputs pins that at least 30%
of the rows rescale after their first tile, and the
GPU results (every ring-step partial, the merged ring, the decode shards and
the reduced decode) must still match the fp64 oracle within the bf16
tolerance. Covers the head_dim 64/128 and 512 ring-step kernels and the three
decode kernels (vector, 32x32 and 16x16 MFMA)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import TOL_BF16, canonical_np, compare, local_buffers, log, need_gpu, np_to_device, run_ring

pytestmark = pytest.mark.gpu

THRESH = 8.0 * np.log(2.0)   # natural-log growth of a row max that forces a rescale
TILE = 64


def _ramped_keys(seed, shape, lo, hi):
    """bf16 keys of N(0,1) values times lo * (hi/lo)^(row / rows), rounded to
    bf16: the magnitude grows geometrically along the first (token) axis."""
    base = synth.bf16_bits_to_f32(synth.tensor_np(seed, synth.TENSOR_K, shape, 1.0, "bf16"))
    axis = 1 if len(shape) == 4 else 0       # decode keys are [b, S, G, D]
    n = shape[axis]
    ramp = lo * (hi / lo) ** (np.arange(n, dtype=np.float64) / max(n - 1, 1))
    bshape = [1] * len(shape)
    bshape[axis] = n
    return synth.f32_to_bf16_bits((base * ramp.reshape(bshape)).astype(np.float32))


def _rescale_fraction(scores):
    """Fraction of rows (scores [rows, keys], -inf for masked keys) that rescale
    at least once after their first tile when walked in ascending 64-key tiles:
    the reference is the first visible tile's max and moves only when a tile's
    max exceeds it by more than the threshold, as in the kernels."""
    hits = 0
    for s in scores:
        ref, grew = -np.inf, False
        for i in range(0, s.size, TILE):
            t = s[i:i + TILE]
            t = t[np.isfinite(t)]
            if t.size == 0:
                continue
            mx = t.max()
            if not np.isfinite(ref):
                ref = mx
            elif mx > ref + THRESH:
                grew, ref = True, mx
        hits += grew
    return hits / len(scores)


# name, lengths, cp, n_hq, n_kv, head_dim, key ramp (lo, hi)
PREFILL = [
    ("gqa2-d128-cp2", [2 * 2 * 256], 2, 4, 2, 128, (0.25, 32.0)),
    ("mha-d64-cp2", [2 * 2 * 300, 2 * 2 * 70], 2, 2, 2, 64, (0.25, 32.0)),
    ("mqa32-d128-cp2", [2 * 2 * 160], 2, 32, 1, 128, (0.25, 32.0)),
    ("mha-d512-cp2", [2 * 2 * 128], 2, 2, 2, 512, (0.25, 32.0)),
]


@pytest.mark.parametrize("case", PREFILL, ids=[c[0] for c in PREFILL])
def test_prefill_with_rescales(case):
    need_gpu()
    import context_attention_amd as ca
    name, lens, cp, H, G, d, (lo, hi) = case
    log(f"[rescale prefill] {name} lens={lens} cp={cp} heads={H}/{G} d={d} keys x {lo}..{hi}")
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = synth.tensor_np(11, synth.TENSOR_Q, (T, H, d), 1.0, "bf16")
    k = _ramped_keys(11, (T, G, d), lo, hi)
    v = synth.tensor_np(11, synth.TENSOR_V, (T, G, d), 0.5, "bf16")
    scale = 1.0 / np.sqrt(d)

    # the inputs do drive the running max past the threshold after the first tile
    qf, kf = synth.bf16_bits_to_f32(q).astype(np.float64), synth.bf16_bits_to_f32(k).astype(np.float64)
    L0 = int(lens[0])
    s = np.einsum("pd,kd->pk", qf[:L0, 0], kf[:L0, 0]) * scale
    s[np.triu_indices(L0, 1)] = -np.inf
    frac = _rescale_fraction(s[TILE:])
    log(f"  rows whose max grows by more than 8 ln 2 after their first tile: {frac:.2f}")
    assert frac >= 0.3, frac

    dev = [np_to_device(x, "bf16") for x in (q, k, v)]
    local = local_buffers(ca, cu, cp, dev)
    desc = ca.PrefillDesc(cp=cp, cu_seqlens=cu, n_hq=H, n_kv=G, head_dim=d, dtype="bf16", scale=scale)
    ref = oracle.ring_prefill(q, k, v, cu, cp, scale)
    unfused = run_ring(ca, desc, local, fused=False)
    fused = run_ring(ca, desc, local, fused=True)
    for r in range(cp):
        pos = local[r][0]
        for t in range(cp):
            p = unfused[r]["parts"][t]
            go, gl = canonical_np(p.m.cpu().numpy(), p.den.cpu().numpy(), p.num.cpu().numpy())
            wo, wl = oracle.finalize(ref["partials"][r][t])
            compare(f"r{r} t{t} partial", go, gl, wo, wl, TOL_BF16)
        compare(f"r{r} merged", fused[r]["out"].cpu().numpy(), fused[r]["lse"].cpu().numpy(),
                ref["out"][pos], ref["lse"][pos], TOL_BF16)


# name, batch, kv_len, cp, n_hq, n_kv, head_dim, key ramp (lo, hi)
DECODE = [
    ("gqa4-d128-vector", 2, 4 * 2000, 4, 8, 2, 128, (0.25, 32.0)),
    ("mqa32-d128-mfma", 2, 4 * 2000, 4, 32, 1, 128, (0.25, 32.0)),
    ("mqa64-d128-mfma16", 2, 2 * 2000, 2, 64, 1, 128, (0.25, 32.0)),
    ("mla16-d512-mfma", 2, 2 * 1000, 2, 16, 1, 512, (0.25, 32.0)),
]


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_decode_with_rescales(case):
    need_gpu()
    import context_attention_amd as ca
    name, b, S, cp, H, G, D, (lo, hi) = case
    log(f"[rescale decode] {name} b={b} kv_len={S} cp={cp} heads={H}/{G} d={D} keys x {lo}..{hi}")
    q = synth.tensor_np(12, synth.TENSOR_Q, (b, H, D), 1.0, "bf16")
    k = _ramped_keys(12, (b, S, G, D), lo, hi)
    v = synth.tensor_np(12, synth.TENSOR_V, (b, S, G, D), 0.5, "bf16")
    scale = 1.0 / np.sqrt(D)

    qf, kf = synth.bf16_bits_to_f32(q).astype(np.float64), synth.bf16_bits_to_f32(k).astype(np.float64)
    n = S // cp
    rows = [np.einsum("d,kd->k", qf[bi, h], kf[bi, s * n:(s + 1) * n, h // (H // G)]) * scale
            for bi in range(b) for h in range(H) for s in range(cp)]
    frac = _rescale_fraction(np.stack(rows))
    log(f"  (row, shard) pairs whose max grows by more than 8 ln 2 after their first tile: {frac:.2f}")
    assert frac >= 0.3, frac

    ks = [np_to_device(np.ascontiguousarray(k[:, s * n:(s + 1) * n]), "bf16") for s in range(cp)]
    vs = [np_to_device(np.ascontiguousarray(v[:, s * n:(s + 1) * n]), "bf16") for s in range(cp)]
    desc = ca.DecodeDesc(batch=b, cp=cp, kv_len=S, n_hq=H, n_kv=G, head_dim=D, dtype="bf16", scale=scale)
    import torch
    sp = ca.new_partial(cp * b, H, D)
    out = torch.full((b, H, D), float("nan"), device="cuda")
    lse = torch.full((b, H), float("nan"), device="cuda")
    ca.passq_decode(desc, np_to_device(q, "bf16"), ks, vs, sp, out, lse)
    torch.cuda.synchronize()
    shards, wo, wl = oracle.passq_decode(q, k, v, cp, scale)
    m = sp.m.cpu().numpy().reshape(cp, b, H)
    den = sp.den.cpu().numpy().reshape(cp, b, H)
    num = sp.num.cpu().numpy().reshape(cp, b, H, D)
    for s in range(cp):
        go, gl = canonical_np(m[s], den[s], num[s])
        so, sl = oracle.finalize(shards[s])
        compare(f"shard {s}", go, gl, so, sl, TOL_BF16)
    compare("reduced", out.cpu().numpy(), lse.cpu().numpy(), wo, wl, TOL_BF16)
