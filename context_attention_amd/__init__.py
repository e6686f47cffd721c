"""Python binding of libcpattn (context-parallel attention for MI355X).

Argument marshalling only: every computation runs in the C library (host
split / account) or its HIP kernels. torch tensors provide device memory and
streams. The binding fails loudly when the library has not been built; there
is no fallback path.

Entry points mirror the C names of include/cpattn.h:
    balanced_split, balanced_split_padded, local_rows, ring_step_partial, ring_pass,
    ring_prefill_overlapped, merge, tree_reduce, passq_decode, account
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "CpattnError", "Partial", "PrefillDesc", "DecodeDesc", "lib_path", "load",
    "balanced_split", "balanced_split_padded", "local_rows", "padded_rows", "ring_step_partial", "ring_pass",
    "ring_prefill_overlapped", "merge", "tree_reduce", "passq_decode", "passq_decode_noalloc",
    "passq_workspace_bytes", "NOALLOC_SCRATCH_BYTES",
    "account", "new_partial", "RingEvents",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libcpattn.so")

OK, E_ARG, E_DIVISIBILITY, E_UNSUPPORTED, E_OVERFLOW, E_WORKSPACE, E_DEVICE = range(7)
_ERR_NAMES = {1: "CPATTN_E_ARG", 2: "CPATTN_E_DIVISIBILITY", 3: "CPATTN_E_UNSUPPORTED",
              4: "CPATTN_E_OVERFLOW", 5: "CPATTN_E_WORKSPACE", 6: "CPATTN_E_DEVICE"}
DT_F32, DT_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 32 << 20    # CPATTN_NOALLOC_SCRATCH_BYTES

EXPORTS = ["cpattn_balanced_split", "cpattn_balanced_split_padded", "cpattn_local_rows", "cpattn_ring_step_partial",
           "cpattn_ring_pass",
           "cpattn_ring_prefill_overlapped", "cpattn_merge", "cpattn_tree_reduce", "cpattn_passq_decode",
           "cpattn_passq_decode_noalloc", "cpattn_ulysses_all_to_all",
           "cpattn_account", "cpattn_version"]


class CpattnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {_ERR_NAMES.get(code, code)}")


# ------------------------------------------------------------------ C structs

class _Partial(ctypes.Structure):
    _fields_ = [("m", ctypes.c_void_p), ("den", ctypes.c_void_p), ("num", ctypes.c_void_p)]


class _PrefillDesc(ctypes.Structure):
    _fields_ = [("cp", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("cu_seqlens", ctypes.POINTER(ctypes.c_int64)),
                ("n_hq", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("padded", ctypes.c_int32)]


class _DecodeDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("cp", ctypes.c_int32), ("kv_len", ctypes.c_int64),
                ("n_hq", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class _AccountIn(ctypes.Structure):
    _fields_ = [("cp", ctypes.c_int32), ("n_hq", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype_bytes", ctypes.c_int32),
                ("c_kv", ctypes.c_int64), ("d_model", ctypes.c_int64), ("layers_local", ctypes.c_int64),
                ("cu_seqlens", ctypes.POINTER(ctypes.c_int64)), ("num_seqs", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("kv_len", ctypes.c_int64)]


ACCOUNT_FIELDS = ["tokens_per_rank", "ring_steps", "p2p_ops", "passkv_bytes_per_step",
                  "passkv_bytes_per_rank", "attn_flops", "step_flops", "rank_flops",
                  "step0_flops_exact", "stepN_flops_exact", "rank_flops_exact", "kv_bytes_per_rank",
                  "passq_dispatch_bytes", "passq_reduce_bytes", "decode_kv_bytes_per_rank",
                  "decode_kv_bytes_total", "decode_flops"]


class _AccountOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ACCOUNT_FIELDS]


_lib = None


def load():
    """Loads libcpattn.so (built by context_attention_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(f"libcpattn.so is not built ({lib_path}); run "
                           "`python -m context_attention_amd.build`")
    lib = ctypes.CDLL(lib_path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.cpattn_balanced_split.argtypes = [ctypes.POINTER(ctypes.c_int64), i32, i32, i32,
                                          ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.cpattn_balanced_split_padded.argtypes = lib.cpattn_balanced_split.argtypes
    lib.cpattn_local_rows.argtypes = [ctypes.POINTER(ctypes.c_int64), i32, i32, i32, ctypes.POINTER(ctypes.c_int64)]
    lib.cpattn_ring_step_partial.argtypes = [ctypes.POINTER(_PrefillDesc), i32, i32, vp, vp, vp,
                                             ctypes.POINTER(_Partial), i32, vp]
    lib.cpattn_ring_pass.argtypes = [vp, vp, i64, i32, vp]
    lib.cpattn_ring_prefill_overlapped.argtypes = [ctypes.POINTER(_PrefillDesc), ctypes.POINTER(vp),
                                                   ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                                   ctypes.POINTER(vp), i32, ctypes.POINTER(_Partial), i32, vp, vp,
                                                   ctypes.POINTER(vp), i32]
    lib.cpattn_merge.argtypes = [i64, i32, i32, ctypes.POINTER(_Partial), i32, ctypes.POINTER(_Partial),
                                 vp, vp, vp]
    lib.cpattn_tree_reduce.argtypes = [i64, i32, i32, ctypes.POINTER(_Partial), i32, vp, vp, vp]
    lib.cpattn_passq_decode.argtypes = [ctypes.POINTER(_DecodeDesc), vp, ctypes.POINTER(vp),
                                        ctypes.POINTER(vp), ctypes.POINTER(_Partial), vp, vp, vp,
                                        ctypes.POINTER(ctypes.c_size_t), vp]
    lib.cpattn_ulysses_all_to_all.argtypes = [i32, i64, i32, i64, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp]
    lib.cpattn_passq_decode_noalloc.argtypes = [ctypes.POINTER(_DecodeDesc), vp, ctypes.POINTER(vp),
                                                ctypes.POINTER(vp), ctypes.POINTER(_Partial), vp, vp, vp]
    lib.cpattn_account.argtypes = [ctypes.POINTER(_AccountIn), ctypes.POINTER(_AccountOut)]
    lib.cpattn_version.restype = ctypes.c_char_p
    for name in EXPORTS:
        getattr(lib, name).restype = ctypes.c_char_p if name == "cpattn_version" else ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int, where: str) -> None:
    if rc != OK:
        raise CpattnError(rc, where)


def _i64_array(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _i64_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


# ------------------------------------------------------------------ host entry points

def balanced_split(cu_seqlens, cp: int, rank: int):
    """cpattn_balanced_split: returns (positions int64 [S/cp], cu_local int64 [n+1])."""
    lib = load()
    cu = _i64_array(cu_seqlens)
    n = cu.size - 1
    total = int(cu[-1]) if cu.size else 0
    pos = np.zeros(max(total // max(cp, 1), 1), dtype=np.int64)
    cul = np.zeros(n + 1, dtype=np.int64)
    _check(lib.cpattn_balanced_split(_i64_ptr(cu), n, cp, rank, _i64_ptr(pos), _i64_ptr(cul)),
           "cpattn_balanced_split")
    return pos[: total // cp], cul


def balanced_split_padded(cu_seqlens, cp: int, rank: int):
    """cpattn_balanced_split_padded: returns (positions int64 [sum(Lp)/cp] with -1
    for pad rows, cu_local int64 [n+1])."""
    lib = load()
    cu = _i64_array(cu_seqlens)
    n = cu.size - 1
    rows = padded_rows(cu, cp)
    pos = np.zeros(max(rows, 1), dtype=np.int64)
    cul = np.zeros(n + 1, dtype=np.int64)
    _check(lib.cpattn_balanced_split_padded(_i64_ptr(cu), n, cp, rank, _i64_ptr(pos), _i64_ptr(cul)),
           "cpattn_balanced_split_padded")
    return pos[:rows], cul


def local_rows(cu_seqlens, cp: int, padded: bool = False) -> int:
    """cpattn_local_rows: rows of one rank's local buffers (pad rows included
    when `padded`)."""
    lib = load()
    cu = _i64_array(cu_seqlens)
    out = ctypes.c_int64(0)
    _check(lib.cpattn_local_rows(_i64_ptr(cu), cu.size - 1, cp, int(bool(padded)), ctypes.byref(out)),
           "cpattn_local_rows")
    return int(out.value)


def padded_rows(cu_seqlens, cp: int) -> int:
    """Local rows of one rank when every sequence is padded to a multiple of 2*cp."""
    return local_rows(cu_seqlens, cp, padded=True)


def account(*, cp: int, n_hq: int, n_kv: int, head_dim: int, dtype_bytes: int, cu_seqlens=None,
            batch: int = 0, kv_len: int = 0, c_kv: int = 0, d_model: int = 0, layers_local: int = 1) -> dict:
    """cpattn_account: the byte / FLOP / memory formulas as a dict of ints."""
    lib = load()
    a = _AccountIn(cp=cp, n_hq=n_hq, n_kv=n_kv, head_dim=head_dim, dtype_bytes=dtype_bytes,
                   c_kv=c_kv, d_model=d_model, layers_local=layers_local, batch=batch, kv_len=kv_len)
    keep = None
    if cu_seqlens is not None:
        keep = _i64_array(cu_seqlens)
        a.cu_seqlens = _i64_ptr(keep)
        a.num_seqs = keep.size - 1
    out = _AccountOut()
    _check(lib.cpattn_account(ctypes.byref(a), ctypes.byref(out)), "cpattn_account")
    return {n: int(getattr(out, n)) for n in ACCOUNT_FIELDS}


# ------------------------------------------------------------------ device entry points

@dataclass
class Partial:
    """A device triple: m, den [rows, n_hq] and num [rows, n_hq, head_dim], fp32."""
    m: "torch.Tensor"
    den: "torch.Tensor"
    num: "torch.Tensor"

    def _c(self) -> _Partial:
        for t in (self.m, self.den, self.num):
            _dev_check(t, "float32")
        return _Partial(self.m.data_ptr(), self.den.data_ptr(), self.num.data_ptr())


def new_partial(rows: int, n_hq: int, head_dim: int, device="cuda") -> Partial:
    import torch
    return Partial(torch.empty(rows, n_hq, dtype=torch.float32, device=device),
                   torch.empty(rows, n_hq, dtype=torch.float32, device=device),
                   torch.empty(rows, n_hq, head_dim, dtype=torch.float32, device=device))


@dataclass
class PrefillDesc:
    cp: int
    cu_seqlens: Sequence[int]
    n_hq: int
    n_kv: int
    head_dim: int
    dtype: str       # 'bf16' or 'f32'
    scale: float
    padded: bool = False   # sequences padded to a multiple of 2*cp (see include/cpattn.h)

    @property
    def rows(self) -> int:
        """Rows of one rank's local buffers (pad rows included)."""
        return local_rows(self.cu_seqlens, self.cp, self.padded)

    def _c(self):
        cu = _i64_array(self.cu_seqlens)
        d = _PrefillDesc(cp=self.cp, num_seqs=cu.size - 1, cu_seqlens=_i64_ptr(cu), n_hq=self.n_hq,
                         n_kv=self.n_kv, head_dim=self.head_dim, dtype=_dtype_code(self.dtype),
                         scale=self.scale, padded=int(bool(self.padded)))
        return d, cu


@dataclass
class DecodeDesc:
    batch: int
    cp: int
    kv_len: int
    n_hq: int
    n_kv: int
    head_dim: int
    dtype: str
    scale: float

    def _c(self):
        return _DecodeDesc(batch=self.batch, cp=self.cp, kv_len=self.kv_len, n_hq=self.n_hq, n_kv=self.n_kv,
                           head_dim=self.head_dim, dtype=_dtype_code(self.dtype), scale=self.scale)


def _dtype_code(name: str) -> int:
    if name == "bf16":
        return DT_BF16
    if name == "f32":
        return DT_F32
    raise ValueError(f"dtype must be 'bf16' or 'f32', not {name!r}")


_TORCH_DT = {"bf16": "bfloat16", "f32": "float32", "float32": "float32"}


def _dev_check(t, dtype: str) -> None:
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    if str(t.dtype) != "torch." + _TORCH_DT[dtype]:
        raise ValueError(f"tensor dtype {t.dtype}, expected {_TORCH_DT[dtype]}")
    if t.data_ptr() % 16:
        raise ValueError("device tensor must be 16-byte aligned")


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check_partial(p: Partial, rows: int, n_hq: int, head_dim: int, what: str) -> None:
    """Shapes of a triple for rows x n_hq (row, head) pairs."""
    if tuple(p.m.shape) != (rows, n_hq) or tuple(p.den.shape) != (rows, n_hq) \
            or tuple(p.num.shape) != (rows, n_hq, head_dim):
        raise ValueError(f"{what} shape mismatch: m {tuple(p.m.shape)}, den {tuple(p.den.shape)}, "
                         f"num {tuple(p.num.shape)}; expected ({rows}, {n_hq}) and ({rows}, {n_hq}, {head_dim})")


def ring_step_partial(desc: PrefillDesc, rank: int, step: int, q_local, k_blk, v_blk, dst: Partial,
                      accumulate: bool = False, stream=None) -> None:
    """cpattn_ring_step_partial (see include/cpattn.h)."""
    lib = load()
    rows = desc.rows
    for t, h in ((q_local, desc.n_hq), (k_blk, desc.n_kv), (v_blk, desc.n_kv)):
        if tuple(t.shape) != (rows, h, desc.head_dim):
            raise ValueError(f"shape {tuple(t.shape)} != {(rows, h, desc.head_dim)}")
    _check_partial(dst, rows, desc.n_hq, desc.head_dim, "dst")
    for t in (q_local, k_blk, v_blk):
        _dev_check(t, desc.dtype)
    d, keep = desc._c()
    p = dst._c()
    _check(lib.cpattn_ring_step_partial(ctypes.byref(d), rank, step, q_local.data_ptr(), k_blk.data_ptr(),
                                        v_blk.data_ptr(), ctypes.byref(p), int(bool(accumulate)),
                                        _stream(stream)), "cpattn_ring_step_partial")


def ring_pass(src, dst, workgroups: int, stream=None) -> None:
    """cpattn_ring_pass: device copy of src into dst (same byte size) on at most
    `workgroups` workgroups, the emulated transfer of a KV block."""
    lib = load()
    for t in (src, dst):
        if not t.is_cuda or not t.is_contiguous() or t.data_ptr() % 16:
            raise ValueError("contiguous, 16-byte aligned device tensors expected")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst sizes differ")
    _check(lib.cpattn_ring_pass(src.data_ptr(), dst.data_ptr(), nbytes, workgroups, _stream(stream)),
           "cpattn_ring_pass")


def ulysses_all_to_all(src, dst, n_heads: int, direction: str, stream=None) -> None:
    """cpattn_ulysses_all_to_all over n = len(src) ranks. direction "seq_to_head":
    src[j] [rows, n_heads, *head] -> dst[i] [n*rows, n_heads/n, *head];
    "head_to_seq": the inverse (src[i] [n*rows, n_heads/n, *head] ->
    dst[j] [rows, n_heads, *head]). Every tensor contiguous, on the device, of
    one dtype."""
    lib = load()
    n = len(src)
    if n < 1 or len(dst) != n:
        raise ValueError("src and dst must hold the same number (>= 1) of ranks")
    if direction not in ("seq_to_head", "head_to_seq"):
        raise ValueError("direction must be 'seq_to_head' or 'head_to_seq'")
    if n_heads % n:
        raise ValueError(f"n_heads {n_heads} is not a multiple of the {n} ranks")
    seq, head = (src, dst) if direction == "seq_to_head" else (dst, src)
    rows = seq[0].shape[0]
    inner = tuple(seq[0].shape[2:])
    want_seq, want_head = (rows, n_heads) + inner, (n * rows, n_heads // n) + inner
    for t in seq:
        if tuple(t.shape) != want_seq:
            raise ValueError(f"sequence-sharded shape {tuple(t.shape)}, expected {want_seq}")
    for t in head:
        if tuple(t.shape) != want_head:
            raise ValueError(f"head-sharded shape {tuple(t.shape)}, expected {want_head}")
    for t in list(src) + list(dst):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != seq[0].dtype:
            raise ValueError("contiguous device tensors of one dtype expected")
    head_bytes = seq[0].element_size()
    for x in inner:
        head_bytes *= x
    ps = (ctypes.c_void_p * n)(*[t.data_ptr() for t in src])
    pd = (ctypes.c_void_p * n)(*[t.data_ptr() for t in dst])
    _check(lib.cpattn_ulysses_all_to_all(n, rows, n_heads, head_bytes, ps, pd,
                                         0 if direction == "seq_to_head" else 1, _stream(stream)),
           "cpattn_ulysses_all_to_all")


class RingEvents:
    """HIP events owned by the caller of cpattn_ring_prefill_overlapped (2*cp of
    them, created with hipEventDisableTiming on the current device, destroyed
    with this object)."""

    def __init__(self, count: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._vp = ctypes.c_void_p      # kept for __del__, which can run at interpreter exit
        self.handles = (ctypes.c_void_p * count)()
        self.count = 0
        for i in range(count):
            rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self.handles, i * ctypes.sizeof(ctypes.c_void_p)),
                                                   ctypes.c_uint(2))
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed with HIP error {rc}")
            self.count += 1

    def __del__(self):
        hip, vp = getattr(self, "_hip", None), getattr(self, "_vp", None)
        if hip is None or vp is None:
            return
        for i in range(getattr(self, "count", 0)):
            hip.hipEventDestroy(vp(self.handles[i]))


def ring_prefill_overlapped(desc: PrefillDesc, q_local: Sequence, k_blocks: Sequence, v_blocks: Sequence,
                            k_recv: Sequence, v_recv: Sequence, acc: Sequence[Partial], link_workgroups: int,
                            compute_stream=None, transfer_stream=None, events: Optional[RingEvents] = None) -> None:
    """cpattn_ring_prefill_overlapped (see include/cpattn.h): the whole ring of the
    CP group, rank r's steps on compute_stream on the block in hand, every block
    forwarded to the next rank's receive buffers on transfer_stream. q_local,
    k_blocks, v_blocks and acc hold one entry per rank; k_recv and v_recv hold
    cp * n_recv buffers, rank-major. `events` (2*cp of them) are created for
    the call when not given."""
    lib = load()
    cp = desc.cp
    rows = desc.rows
    if len(q_local) != cp or len(k_blocks) != cp or len(v_blocks) != cp or len(acc) != cp:
        raise ValueError("need cp queries, K and V blocks and accumulators")
    if len(k_recv) != len(v_recv) or len(k_recv) % cp or (cp > 1 and len(k_recv) // cp < 2):
        raise ValueError("need cp * n_recv K and V receive buffers, n_recv >= 2")
    n_recv = len(k_recv) // cp
    for t in q_local:
        if tuple(t.shape) != (rows, desc.n_hq, desc.head_dim):
            raise ValueError(f"q_local shape {tuple(t.shape)} != {(rows, desc.n_hq, desc.head_dim)}")
    for t in list(k_blocks) + list(v_blocks) + list(k_recv) + list(v_recv):
        if tuple(t.shape) != (rows, desc.n_kv, desc.head_dim):
            raise ValueError(f"block shape {tuple(t.shape)} != {(rows, desc.n_kv, desc.head_dim)}")
    for p in acc:
        _check_partial(p, rows, desc.n_hq, desc.head_dim, "acc")
    for t in list(q_local) + list(k_blocks) + list(v_blocks) + list(k_recv) + list(v_recv):
        _dev_check(t, desc.dtype)
    if events is None:
        events = RingEvents(2 * cp)
    if events.count < 2 * cp:
        raise ValueError(f"need {2 * cp} events")
    d, keep = desc._c()
    parts = (_Partial * cp)(*[p._c() for p in acc])
    arr = lambda ts: (ctypes.c_void_p * max(len(ts), 1))(*[t.data_ptr() for t in ts])
    _check(lib.cpattn_ring_prefill_overlapped(ctypes.byref(d), arr(q_local), arr(k_blocks), arr(v_blocks),
                                              arr(k_recv), arr(v_recv), n_recv, parts, link_workgroups,
                                              _stream(compute_stream), _stream(transfer_stream), events.handles,
                                              events.count), "cpattn_ring_prefill_overlapped")


def merge(acc: Partial, parts: Sequence[Partial] = (), out=None, lse=None, stream=None) -> None:
    """cpattn_merge: acc = merge(acc, *parts); optionally out = num/den, lse = m + ln den."""
    lib = load()
    if acc.num.dim() != 3:
        raise ValueError("acc.num must be [rows, n_hq, head_dim]")
    rows, n_hq, hd = acc.num.shape
    _check_partial(acc, rows, n_hq, hd, "acc")
    for p in parts:
        _check_partial(p, rows, n_hq, hd, "part")
    if out is not None and tuple(out.shape) != (rows, n_hq, hd):
        raise ValueError("out shape mismatch")
    if lse is not None and tuple(lse.shape) != (rows, n_hq):
        raise ValueError("lse shape mismatch")
    for t in (out, lse):
        if t is not None:
            _dev_check(t, "f32")
    arr = (_Partial * max(len(parts), 1))(*[p._c() for p in parts])
    a = acc._c()
    _check(lib.cpattn_merge(rows, n_hq, hd, arr if parts else None, len(parts), ctypes.byref(a),
                            out.data_ptr() if out is not None else None,
                            lse.data_ptr() if lse is not None else None, _stream(stream)), "cpattn_merge")


def tree_reduce(parts: Sequence[Partial], out=None, lse=None, stream=None) -> None:
    """cpattn_tree_reduce: merges `parts` in tree order (round k merges part
    s + 2^k into part s, s a multiple of 2^(k+1)); parts[0] then holds the
    result, the other parts are overwritten; optionally out = num/den, lse."""
    lib = load()
    if not parts:
        raise ValueError("at least one part")
    if parts[0].num.dim() != 3:
        raise ValueError("num must be [rows, n_hq, head_dim]")
    rows, n_hq, hd = parts[0].num.shape
    for p in parts:
        _check_partial(p, rows, n_hq, hd, "part")
    if out is not None and tuple(out.shape) != (rows, n_hq, hd):
        raise ValueError("out shape mismatch")
    if lse is not None and tuple(lse.shape) != (rows, n_hq):
        raise ValueError("lse shape mismatch")
    for t in (out, lse):
        if t is not None:
            _dev_check(t, "f32")
    arr = (_Partial * len(parts))(*[p._c() for p in parts])
    _check(lib.cpattn_tree_reduce(rows, n_hq, hd, arr, len(parts),
                                  out.data_ptr() if out is not None else None,
                                  lse.data_ptr() if lse is not None else None, _stream(stream)),
           "cpattn_tree_reduce")


def passq_workspace_bytes(desc: DecodeDesc) -> int:
    lib = load()
    d = desc._c()
    n = ctypes.c_size_t(0)
    _check(lib.cpattn_passq_decode(ctypes.byref(d), None, None, None, None, None, None, None,
                                   ctypes.byref(n), None), "cpattn_passq_decode")
    return int(n.value)


def _check_decode(desc: DecodeDesc, q, k_shards: Sequence, v_shards: Sequence, shard_partials: Partial,
                  out, lse) -> None:
    b, hq, hd = desc.batch, desc.n_hq, desc.head_dim
    if tuple(q.shape) != (b, hq, hd):
        raise ValueError("q shape mismatch")
    if len(k_shards) != desc.cp or len(v_shards) != desc.cp:
        raise ValueError("need cp K and V shards")
    shard_len = desc.kv_len // desc.cp
    for t in list(k_shards) + list(v_shards):
        if tuple(t.shape) != (b, shard_len, desc.n_kv, hd):
            raise ValueError(f"shard shape {tuple(t.shape)} != {(b, shard_len, desc.n_kv, hd)}")
    _check_partial(shard_partials, desc.cp * b, hq, hd, "shard_partials")
    if tuple(out.shape) != (b, hq, hd):
        raise ValueError(f"out shape {tuple(out.shape)} != {(b, hq, hd)}")
    if tuple(lse.shape) != (b, hq):
        raise ValueError(f"lse shape {tuple(lse.shape)} != {(b, hq)}")
    _dev_check(q, desc.dtype)
    for t in list(k_shards) + list(v_shards):
        _dev_check(t, desc.dtype)
    _dev_check(out, "f32")
    _dev_check(lse, "f32")


def passq_decode(desc: DecodeDesc, q, k_shards: Sequence, v_shards: Sequence, shard_partials: Partial,
                 out, lse, ws=None, stream=None) -> None:
    """cpattn_passq_decode (see include/cpattn.h). Allocates the workspace with
    torch when `ws` is None."""
    import torch
    lib = load()
    _check_decode(desc, q, k_shards, v_shards, shard_partials, out, lse)
    need = passq_workspace_bytes(desc)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if not ws.is_cuda or ws.data_ptr() % 16:
        raise ValueError("workspace must be an aligned device tensor")
    d = desc._c()
    ks = (ctypes.c_void_p * desc.cp)(*[t.data_ptr() for t in k_shards])
    vs = (ctypes.c_void_p * desc.cp)(*[t.data_ptr() for t in v_shards])
    sp = shard_partials._c()
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check(lib.cpattn_passq_decode(ctypes.byref(d), q.data_ptr(), ks, vs, ctypes.byref(sp), out.data_ptr(),
                                   lse.data_ptr(), ws.data_ptr(), ctypes.byref(n), _stream(stream)),
           "cpattn_passq_decode")


def passq_decode_noalloc(desc: DecodeDesc, q, k_shards: Sequence, v_shards: Sequence, shard_partials: Partial,
                         out, lse, stream=None) -> None:
    """cpattn_passq_decode_noalloc (see include/cpattn.h): pass-Q decode with
    the workspace in the library's per-GPU scratch buffer; nothing is
    allocated."""
    lib = load()
    _check_decode(desc, q, k_shards, v_shards, shard_partials, out, lse)
    d = desc._c()
    ks = (ctypes.c_void_p * desc.cp)(*[t.data_ptr() for t in k_shards])
    vs = (ctypes.c_void_p * desc.cp)(*[t.data_ptr() for t in v_shards])
    sp = shard_partials._c()
    _check(lib.cpattn_passq_decode_noalloc(ctypes.byref(d), q.data_ptr(), ks, vs, ctypes.byref(sp),
                                           out.data_ptr(), lse.data_ptr(), _stream(stream)),
           "cpattn_passq_decode_noalloc")


def version() -> str:
    return load().cpattn_version().decode()


from . import overlap  # noqa: E402  (transfer/compute overlap harness built on the entry points above)
