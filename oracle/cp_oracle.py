"""Plain fp64 reference for context-parallel attention (test infrastructure only).

Source of every definition: the G5 context-parallel modelling spec ("G5
上下文并行建模设计规格"), cited below by section:
  * Definitions table (名词定义): pass-KV, pass-Q, ring step, partial attention
    (incomplete attention over a KV subset carrying max / numerator /
    denominator, merged associatively and order-independently), balanced chunk
    split (2*cp chunks, each rank holds a head/tail pair), c_kv, d / n_h,
    CP=1 degeneration.
  * Rationale (设计原理): balanced split gives each rank 1/cp^2 of the work per
    ring step.
  * Formulas (算法 / 公式): eq. g5cp-passkv-bytes, eq. g5cp-step-flops, pass-Q
    dispatch / reduce bytes, per-rank KV memory.
  * Constraints (约束与规则): cp=1 produces no CP sub-operations or transfers.
  * Acceptance (验收标准): transfer conservation, DAG structure, CP=1
    degeneration, memory split.

Readings of points the page leaves open (each also listed in the design notes):
  * rank r holds chunks r and 2*cp-1-r, head chunk first;
  * at ring step t rank r holds the KV block of rank (r - t) mod cp;
  * the causal mask is inclusive (key position <= query position) on global
    positions inside one sequence; no attention across packed sequences;
  * the numerator is unnormalised, the max is in natural-log units;
  * a row that sees no key is the merge identity (m = -inf, den = 0, num = 0);
  * F_attn counts 4*d_h flops per (query head, key) pair over L^2/2 pairs, i.e.
    F_attn = sum_i 2*b*n_hq*d_h*L_i^2;
  * q head h reads kv head floor(h / (n_hq / n_kv)).

Tensor layouts (token-major, head_dim innermost, global packed order):
  prefill  q [T, n_hq, d], k / v [T, n_kv, d], cu_seqlens [n+1]
  decode   q [b, n_hq, d], k / v [b, S, n_kv, d]
bf16 inputs arrive as uint16 bit patterns and are widened exactly to fp64.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

IDENTITY_M = -np.inf

Triple = Tuple[np.ndarray, np.ndarray, np.ndarray]   # (m [..], den [..], num [.., d])


# ----------------------------------------------------------------------------- inputs

def upcast(x) -> np.ndarray:
    """Exact widening to fp64. uint16 arrays are bf16 bit patterns."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _cu(cu_seqlens) -> np.ndarray:
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0 and be non-decreasing")
    return cu


def _check_cp(cp: int) -> None:
    if int(cp) != cp or cp < 1:
        # Interface appendix: cp is an explicit positive integer, no default.
        raise ValueError("cp must be a positive integer")


# ----------------------------------------------------------------------------- split (O1)

def balanced_split(cu_seqlens, cp: int, rank: int) -> Tuple[np.ndarray, np.ndarray]:
    """Balanced chunk split (Definitions table, 'Balanced chunk split'; Rationale).

    Each sequence of length L is cut into 2*cp chunks of c = L / (2*cp) tokens;
    rank r keeps chunk r (head) and chunk 2*cp-1-r (tail), head first. Returns
    the packed global token index of every local row (sequence-major) and the
    local cumulative lengths cu_local [n+1].
    """
    _check_cp(cp)
    cu = _cu(cu_seqlens)
    if not 0 <= rank < cp:
        raise ValueError("rank out of range")
    pos: List[int] = []
    cu_local = [0]
    for i in range(cu.size - 1):
        start, L = int(cu[i]), int(cu[i + 1] - cu[i])
        if L % (2 * cp):
            raise ValueError(f"sequence {i}: length {L} not divisible by 2*cp={2 * cp}")
        c = L // (2 * cp)
        head = range(start + rank * c, start + (rank + 1) * c)
        tail = range(start + (2 * cp - 1 - rank) * c, start + (2 * cp - rank) * c)
        pos.extend(head)
        pos.extend(tail)
        cu_local.append(cu_local[-1] + 2 * c)
    return np.asarray(pos, dtype=np.int64), np.asarray(cu_local, dtype=np.int64)


def balanced_split_padded(cu_seqlens, cp: int, rank: int) -> Tuple[np.ndarray, np.ndarray]:
    """Balanced chunk split of sequences of any length. Reading taken (the pages
    fix the split only for lengths divisible by 2*cp; the TP/EP design page pads
    a token count that does not divide evenly and lets padding take no part in
    the outputs): a sequence of length L is padded at its end to
    Lp = ceil(L / (2*cp)) * 2*cp slots and split as one of Lp tokens. Returns the
    packed global token index of every local slot, -1 for a pad slot, and the
    local cumulative slot counts."""
    _check_cp(cp)
    cu = _cu(cu_seqlens)
    if not 0 <= rank < cp:
        raise ValueError("rank out of range")
    pos: List[int] = []
    cu_local = [0]
    for i in range(cu.size - 1):
        start, L = int(cu[i]), int(cu[i + 1] - cu[i])
        c = -(-L // (2 * cp))                                     # ceil
        for first in (rank * c, (2 * cp - 1 - rank) * c):
            pos.extend(start + x if x < L else -1 for x in range(first, first + c))
        cu_local.append(cu_local[-1] + 2 * c)
    return np.asarray(pos, dtype=np.int64), np.asarray(cu_local, dtype=np.int64)


def sequential_split(cu_seqlens, cp: int, rank: int) -> np.ndarray:
    """The contrast layout of the Definitions table: rank r holds the r-th
    contiguous 1/cp of every sequence."""
    _check_cp(cp)
    cu = _cu(cu_seqlens)
    pos: List[int] = []
    for i in range(cu.size - 1):
        start, L = int(cu[i]), int(cu[i + 1] - cu[i])
        if L % cp:
            raise ValueError("length not divisible by cp")
        n = L // cp
        pos.extend(range(start + rank * n, start + (rank + 1) * n))
    return np.asarray(pos, dtype=np.int64)


def ring_schedule(cp: int) -> List[Tuple[int, int, int]]:
    """Pass-KV ring (Definitions: pass-KV, ring step). Returns (step t, rank r,
    source rank j) for every compute operation; rank r computes on the block of
    rank (r - t) mod cp at step t. Blocks move cp-1 times per rank."""
    _check_cp(cp)
    return [(t, r, (r - t) % cp) for t in range(cp) for r in range(cp)]


def _seq_of(cu: np.ndarray) -> np.ndarray:
    T = int(cu[-1])
    return np.repeat(np.arange(cu.size - 1, dtype=np.int64), np.diff(cu)) if T else np.zeros(0, np.int64)


def step_pair_counts(cu_seqlens, cp: int, rank: int, step: int, split: str = "balanced") -> int:
    """Number of visible (query, key) pairs rank `rank` handles at ring step
    `step`, per head: same sequence and key index <= query index. Computed by
    counting over the actual index sets (no closed form)."""
    cu = _cu(cu_seqlens)
    seq = _seq_of(cu)
    if split == "balanced":
        q_idx, _ = balanced_split(cu, cp, rank)
        k_idx, _ = balanced_split(cu, cp, (rank - step) % cp)
    else:
        q_idx = sequential_split(cu, cp, rank)
        k_idx = sequential_split(cu, cp, (rank - step) % cp)
    total = 0
    for s in range(cu.size - 1):
        qs = np.sort(q_idx[seq[q_idx] == s]) if q_idx.size else q_idx
        ks = np.sort(k_idx[seq[k_idx] == s]) if k_idx.size else k_idx
        # for every query, the keys of the same sequence at or before it
        total += int(np.searchsorted(ks, qs, side="right").sum())
    return total


# ----------------------------------------------------------------------------- account (O1)

def account(*, cp: int, n_hq: int, n_kv: int, head_dim: int, dtype_bytes: int,
            cu_seqlens=None, batch: int = 1, kv_len: Optional[int] = None,
            c_kv: Optional[int] = None, d_model: Optional[int] = None,
            layers_local: int = 1) -> Dict[str, int]:
    """Byte / FLOP / memory bookkeeping of the Formulas section, in Python
    integers (exact).

    c_kv (Definitions): K+V bytes per token per layer, both already counted;
    default 2 * n_kv * head_dim * dtype_bytes. d (Definitions): model hidden
    size, default n_hq * head_dim. n_h: attention (query) heads.
    Prefill quantities use the packed lengths (b = 1 per packed sequence);
    decode quantities use batch and kv_len.
    """
    _check_cp(cp)
    if n_kv < 1 or n_hq % n_kv:
        raise ValueError("n_hq must be a multiple of n_kv")
    if c_kv is None:
        c_kv = 2 * n_kv * head_dim * dtype_bytes
    if d_model is None:
        d_model = n_hq * head_dim
    out: Dict[str, int] = {
        "ring_steps": cp,
        "p2p_ops": cp - 1,
    }
    if cu_seqlens is not None:
        cu = _cu(cu_seqlens)
        L = np.diff(cu).astype(object)
        if any(int(x) % (2 * cp) for x in L):
            raise ValueError("every length must be divisible by 2*cp")
        S = int(sum(L))
        c = [int(x) // (2 * cp) for x in L]
        # Definitions / Formulas: per rank S/cp tokens.
        out["tokens_per_rank"] = S // cp
        # eq. g5cp-passkv-bytes: per step S/cp * c_kv, cp-1 steps.
        out["passkv_bytes_per_step"] = (S // cp) * c_kv if cp > 1 else 0
        out["passkv_bytes_per_rank"] = (cp - 1) * (S // cp) * c_kv
        # F_attn = sum 2 * n_hq * d_h * L^2 (4 d_h flops per pair, L^2/2 pairs).
        f_attn = sum(2 * n_hq * head_dim * int(x) * int(x) for x in L)
        out["attn_flops"] = f_attn
        # eq. g5cp-step-flops
        out["step_flops"] = f_attn // (cp * cp)
        out["rank_flops"] = f_attn // cp
        # exact inclusive-causal pair counts: every (rank, step) has 2 c^2 pairs
        # per sequence, step 0 adds the c diagonal entries.
        out["step0_flops_exact"] = 4 * head_dim * n_hq * sum(2 * x * x + x for x in c)
        out["stepN_flops_exact"] = 4 * head_dim * n_hq * sum(2 * x * x for x in c)
        out["rank_flops_exact"] = out["step0_flops_exact"] + (cp - 1) * out["stepN_flops_exact"]
        # Formulas: per-rank KV memory b * S * c_kv * L_local / cp (b folded into S).
        out["kv_bytes_per_rank"] = S * c_kv * layers_local // cp
    if kv_len is not None:
        if kv_len % cp:
            raise ValueError("kv_len must be divisible by cp")
        # Formulas: pass-Q dispatch b*d*s, reduce b*(d + 2 n_h)*s; none at cp = 1.
        out["passq_dispatch_bytes"] = batch * d_model * dtype_bytes if cp > 1 else 0
        out["passq_reduce_bytes"] = batch * (d_model + 2 * n_hq) * dtype_bytes if cp > 1 else 0
        out["decode_kv_bytes_per_rank"] = batch * kv_len * c_kv * layers_local // cp
        out["decode_kv_bytes_total"] = batch * kv_len * c_kv * layers_local
        out["decode_flops"] = 4 * batch * n_hq * head_dim * kv_len
    return out


# ----------------------------------------------------------------------------- attention (O2, O3)

def _gqa(n_hq: int, n_kv: int) -> int:
    if n_kv < 1 or n_hq % n_kv:
        raise ValueError("n_hq must be a multiple of n_kv")
    return n_hq // n_kv


def partial_attention(q, k, v, q_idx, k_idx, seq_of, scale: float, causal: bool = True) -> Triple:
    """Partial attention with its online-softmax triple (Definitions table,
    'Partial attention'): for every query row p and query head h, over the keys
    j of the given KV subset that it may see,
        s_j = scale * <q_p,h , k_j,g(h)>,  m = max_j s_j,
        den = sum_j exp(s_j - m),          num = sum_j exp(s_j - m) * v_j,g(h).
    A row that sees no key gets the identity (-inf, 0, 0).
    q, k, v are global packed arrays; q_idx / k_idx select rows; seq_of maps a
    packed index to its sequence. Returns m, den [P, Hq] and num [P, Hq, D]."""
    Q = upcast(q[np.asarray(q_idx, dtype=np.int64)])
    K = upcast(k[np.asarray(k_idx, dtype=np.int64)])
    V = upcast(v[np.asarray(k_idx, dtype=np.int64)])
    P, Hq, D = Q.shape
    rep = _gqa(Hq, K.shape[1])
    q_idx = np.asarray(q_idx, dtype=np.int64)
    k_idx = np.asarray(k_idx, dtype=np.int64)
    if causal:
        seq_of = np.asarray(seq_of, dtype=np.int64)
        vis = (seq_of[q_idx][:, None] == seq_of[k_idx][None, :]) & (k_idx[None, :] <= q_idx[:, None])
    else:
        vis = np.ones((P, k_idx.size), dtype=bool)
    any_vis = vis.any(axis=1)
    m = np.full((P, Hq), IDENTITY_M)
    den = np.zeros((P, Hq))
    num = np.zeros((P, Hq, D))
    if k_idx.size == 0 or not any_vis.any():
        return m, den, num
    for h in range(Hq):
        g = h // rep
        s = scale * (Q[:, h, :] @ K[:, g, :].T)                       # [P, J]
        s = np.where(vis, s, -np.inf)
        mh = s.max(axis=1)                                            # pass 1: row max
        e = np.zeros_like(s)
        rows = any_vis
        e[rows] = np.exp(s[rows] - mh[rows, None])                    # pass 2: sums
        m[rows, h] = mh[rows]
        den[:, h] = e.sum(axis=1)
        num[:, h, :] = e @ V[:, g, :]
    return m, den, num


def merge_two(a: Triple, b: Triple) -> Triple:
    """Merge two triples (Definitions table: partial attention merges are
    associative and order-independent):
        m = max(m1, m2), alpha_i = exp(m_i - m) (0 when m_i = -inf),
        den = sum alpha_i den_i, num = sum alpha_i num_i."""
    m1, d1, n1 = a
    m2, d2, n2 = b
    m = np.maximum(m1, m2)
    fin = np.isfinite(m)
    a1 = np.zeros_like(m)
    a2 = np.zeros_like(m)
    ok1 = fin & np.isfinite(m1)
    ok2 = fin & np.isfinite(m2)
    a1[ok1] = np.exp(m1[ok1] - m[ok1])
    a2[ok2] = np.exp(m2[ok2] - m[ok2])
    den = a1 * d1 + a2 * d2
    num = a1[..., None] * n1 + a2[..., None] * n2
    return m, den, num


def merge(parts: Sequence[Triple]) -> Triple:
    """Left fold of merge_two in the given order."""
    acc = parts[0]
    for p in parts[1:]:
        acc = merge_two(acc, p)
    return acc


def tree_rounds(n: int) -> List[List[Tuple[int, int]]]:
    """The exchanges of a tree reduction over n ranks, the Tree Attention
    reduction that the G5 spec lists as follow-up work for pass-Q (Limitations
    table): round k holds the pairs (receiver s, sender s + 2^k) for every s that
    is a multiple of 2^(k+1) with s + 2^k < n."""
    if n < 1:
        raise ValueError("at least one rank")
    rounds = []
    span = 1
    while span < n:
        rounds.append([(s, s + span) for s in range(0, n - span, 2 * span)])
        span *= 2
    return rounds


def merge_tree(parts: Sequence[Triple]) -> Triple:
    """Merges one triple per rank along tree_rounds: after the last round rank 0
    holds the result. `parts` is left untouched."""
    held = list(parts)
    for rnd in tree_rounds(len(held)):
        for recv, send in rnd:
            held[recv] = merge_two(held[recv], held[send])
    return held[0]


def finalize(t: Triple) -> Tuple[np.ndarray, np.ndarray]:
    """out = num / den, lse = m + ln(den); identity rows give out 0, lse -inf."""
    m, den, num = t
    ok = den > 0
    out = np.zeros_like(num)
    out[ok] = num[ok] / den[ok][..., None]
    lse = np.full_like(m, -np.inf)
    lse[ok] = m[ok] + np.log(den[ok])
    return out, lse


canonical = finalize


def attention_reference(q, k, v, cu_seqlens, scale: float, causal: bool = True):
    """Unsplit causal softmax attention per packed sequence (the non-CP result
    that CP must reproduce: Definitions, 'CP=1 degeneration'). Two passes: the
    full row max, then the sums. Returns out [T, Hq, D], lse [T, Hq]."""
    Q, K, V = upcast(q), upcast(k), upcast(v)
    T, Hq, D = Q.shape
    rep = _gqa(Hq, K.shape[1])
    cu = _cu(cu_seqlens)
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    for i in range(cu.size - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        if b == a:
            continue
        L = b - a
        mask = np.tril(np.ones((L, L), dtype=bool)) if causal else np.ones((L, L), dtype=bool)
        for h in range(Hq):
            g = h // rep
            s = scale * (Q[a:b, h, :] @ K[a:b, g, :].T)
            s = np.where(mask, s, -np.inf)
            mx = s.max(axis=1)
            e = np.exp(s - mx[:, None])
            den = e.sum(axis=1)
            out[a:b, h, :] = (e @ V[a:b, g, :]) / den[:, None]
            lse[a:b, h] = mx + np.log(den)
    return out, lse


def attention_reference_rows(q_rows, q_pos, k_seq, v_seq, scale: float, causal: bool = True,
                             key_block: int = 8192):
    """Unsplit attention for selected query rows of ONE sequence, streaming the
    keys of that sequence in blocks (two passes over the blocks: row max, then
    sums). q_rows [P, Hq, D]; q_pos [P] positions inside the sequence; k_seq /
    v_seq [L, Hkv, D] the whole sequence. Returns out [P, Hq, D], lse [P, Hq]."""
    Q = upcast(q_rows)
    P, Hq, D = Q.shape
    L, Hkv, _ = k_seq.shape
    rep = _gqa(Hq, Hkv)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    limit = int(q_pos.max()) + 1 if causal else L
    mx = np.full((P, Hq), -np.inf)
    for kb in range(0, limit, key_block):
        ke = min(limit, kb + key_block)
        Kb = upcast(k_seq[kb:ke])
        kp = np.arange(kb, ke)
        vis = (kp[None, :] <= q_pos[:, None]) if causal else np.ones((P, ke - kb), bool)
        for h in range(Hq):
            s = scale * (Q[:, h, :] @ Kb[:, h // rep, :].T)
            s = np.where(vis, s, -np.inf)
            mx[:, h] = np.maximum(mx[:, h], s.max(axis=1))
    den = np.zeros((P, Hq))
    num = np.zeros((P, Hq, D))
    for kb in range(0, limit, key_block):
        ke = min(limit, kb + key_block)
        Kb = upcast(k_seq[kb:ke])
        Vb = upcast(v_seq[kb:ke])
        kp = np.arange(kb, ke)
        vis = (kp[None, :] <= q_pos[:, None]) if causal else np.ones((P, ke - kb), bool)
        for h in range(Hq):
            s = scale * (Q[:, h, :] @ Kb[:, h // rep, :].T)
            e = np.where(vis, np.exp(s - mx[:, h, None]), 0.0)
            den[:, h] += e.sum(axis=1)
            num[:, h, :] += e @ Vb[:, h // rep, :]
    return num / den[..., None], mx + np.log(den)


def brute_force_attention(q, k, v, cu_seqlens, scale: float, causal: bool = True):
    """Pure-Python loops with math.fsum; tiny inputs only."""
    Q, K, V = upcast(q), upcast(k), upcast(v)
    T, Hq, D = Q.shape
    rep = Hq // K.shape[1]
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    out = np.zeros((T, Hq, D))
    lse = np.zeros((T, Hq))
    for i in range(len(cu) - 1):
        for p in range(cu[i], cu[i + 1]):
            for h in range(Hq):
                g = h // rep
                keys = range(cu[i], p + 1) if causal else range(cu[i], cu[i + 1])
                s = [scale * math.fsum(Q[p, h, x] * K[j, g, x] for x in range(D)) for j in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                den = math.fsum(w)
                for x in range(D):
                    out[p, h, x] = math.fsum(wj * V[j, g, x] for wj, j in zip(w, keys)) / den
                lse[p, h] = mx + math.log(den)
    return out, lse


def ring_prefill(q, k, v, cu_seqlens, cp: int, scale: float, order: Optional[Sequence[int]] = None):
    """The method's own prefill steps (Definitions: pass-KV, ring step, partial
    attention, balanced split): for every rank r and ring step t, the partial
    triple of r's rows over the block of rank (r - t) mod cp, then the merge
    of a rank's cp partials (in ring order, or in `order` of steps).

    Returns dict with
      'partials'[r][t] : triple over rank-local rows,
      'positions'[r]   : packed global index of each local row,
      'out', 'lse'     : merged results scattered back to global order."""
    cu = _cu(cu_seqlens)
    seq = _seq_of(cu)
    T = int(cu[-1])
    Qf = np.asarray(q)
    Hq, D = Qf.shape[1], Qf.shape[2]
    split = [balanced_split(cu, cp, r)[0] for r in range(cp)]
    partials: List[List[Triple]] = []
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    for r in range(cp):
        row = []
        for t in range(cp):
            j = (r - t) % cp
            row.append(partial_attention(q, k, v, split[r], split[j], seq, scale, causal=True))
        partials.append(row)
        steps = list(range(cp)) if order is None else list(order)
        o, l = finalize(merge([row[t] for t in steps]))
        out[split[r]] = o
        lse[split[r]] = l
    return {"partials": partials, "positions": split, "out": out, "lse": lse}


def ring_prefill_padded(q, k, v, cu_seqlens, cp: int, scale: float):
    """ring_prefill over the padded split: pad slots take no part -- a pad slot is
    no key for anyone, and a pad query slot keeps the identity triple. Returns
    'partials'[r][t] over every local slot (pad slots included), 'positions'[r]
    (-1 for pad slots), and 'out' / 'lse' for the real tokens in global order."""
    cu = _cu(cu_seqlens)
    seq = _seq_of(cu)
    T = int(cu[-1])
    Hq, D = np.asarray(q).shape[1], np.asarray(q).shape[2]
    split = [balanced_split_padded(cu, cp, r)[0] for r in range(cp)]
    partials: List[List[Triple]] = []
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    for r in range(cp):
        rows = split[r]
        real = rows >= 0
        row = []
        for t in range(cp):
            keys = split[(r - t) % cp]
            m = np.full((rows.size, Hq), IDENTITY_M)
            den = np.zeros((rows.size, Hq))
            num = np.zeros((rows.size, Hq, D))
            pm, pd, pn = partial_attention(q, k, v, rows[real], keys[keys >= 0], seq, scale, causal=True)
            m[real], den[real], num[real] = pm, pd, pn
            row.append((m, den, num))
        partials.append(row)
        o, l = finalize(merge(row))
        out[rows[real]] = o[real]
        lse[rows[real]] = l[real]
    return {"partials": partials, "positions": split, "out": out, "lse": lse}


def decode_reference(q, k, v, scale: float, key_block: int = 1 << 16):
    """Plain decode attention: one query per batch entry against all kv_len keys,
    no mask; two passes over key blocks. q [b, Hq, D], k / v [b, S, Hkv, D]."""
    Q = upcast(q)
    b, Hq, D = Q.shape
    S, Hkv = k.shape[1], k.shape[2]
    rep = _gqa(Hq, Hkv)
    out = np.zeros((b, Hq, D))
    lse = np.zeros((b, Hq))
    for bi in range(b):
        for g in range(Hkv):
            Qg = Q[bi, g * rep:(g + 1) * rep, :]                      # [rep, D]
            mx = np.full(rep, -np.inf)
            for kb in range(0, S, key_block):
                Kb = upcast(k[bi, kb:kb + key_block, g, :])
                mx = np.maximum(mx, (scale * (Qg @ Kb.T)).max(axis=1))
            den = np.zeros(rep)
            num = np.zeros((rep, D))
            for kb in range(0, S, key_block):
                Kb = upcast(k[bi, kb:kb + key_block, g, :])
                Vb = upcast(v[bi, kb:kb + key_block, g, :])
                e = np.exp(scale * (Qg @ Kb.T) - mx[:, None])
                den += e.sum(axis=1)
                num += e @ Vb
            out[bi, g * rep:(g + 1) * rep] = num / den[:, None]
            lse[bi, g * rep:(g + 1) * rep] = mx + np.log(den)
    return out, lse


def passq_decode(q, k, v, cp: int, scale: float, order: Optional[Sequence[int]] = None):
    """The method's decode steps (Definitions: pass-Q): the query goes to every
    shard, shard s holds keys [s*S/cp, (s+1)*S/cp), each shard computes its
    partial triple over all its keys (no mask), and the cp triples are reduced
    with the same merge (the 'three-quantity' reduction of max, denominator and
    numerator). Returns (shard triples [cp] each (m [b,Hq], den, num [b,Hq,D]),
    out, lse)."""
    _check_cp(cp)
    Q = upcast(q)
    b, Hq, D = Q.shape
    S, Hkv = k.shape[1], k.shape[2]
    if S % cp:
        raise ValueError("kv_len must be divisible by cp")
    rep = _gqa(Hq, Hkv)
    n = S // cp
    shards: List[Triple] = []
    for s in range(cp):
        m = np.full((b, Hq), IDENTITY_M)
        den = np.zeros((b, Hq))
        num = np.zeros((b, Hq, D))
        for bi in range(b):
            Kb = upcast(k[bi, s * n:(s + 1) * n])                      # [n, Hkv, D]
            Vb = upcast(v[bi, s * n:(s + 1) * n])
            for h in range(Hq):
                sc = scale * (Kb[:, h // rep, :] @ Q[bi, h, :])
                if sc.size == 0:
                    continue
                mx = sc.max()
                e = np.exp(sc - mx)
                m[bi, h] = mx
                den[bi, h] = e.sum()
                num[bi, h, :] = e @ Vb[:, h // rep, :]
        shards.append((m, den, num))
    steps = list(range(cp)) if order is None else list(order)
    out, lse = finalize(merge([shards[s] for s in steps]))
    return shards, out, lse
