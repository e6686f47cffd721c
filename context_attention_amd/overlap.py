"""One-GPU emulation of the pass-KV ring's transfer/compute overlap.

The G5 context-parallel modelling spec fixes the ring's dependency contract
(Rationale: step i's transfer runs concurrently with step i's compute; step
i+1's compute waits for step i's transfer) and two acceptance checks
(Acceptance table): "overlap effective" -- with a compute/transfer time ratio
in [0.5, 2], the ring takes at most 1.1 x max(compute, transfer) and at most
0.7 x (compute + transfer), which a serial ring (ratio 1.0 to the sum) fails
-- and "overlap metamorphic" -- with a large S/cp, the ring deviates from the
pure compute time by less than 10%.

Here the whole CP group runs on the one GPU: compute = the cp ring steps of
every rank, step by step (cp^2 launches on one stream); transfer = the
forwarding copies of every rank (cp - 1 steps of cp K and cp V copies,
cpattn_ring_pass, on one stream); ring = cpattn_ring_prefill_overlapped on two
streams; serial = the same call with one stream for both. Times are medians of
HIP-event intervals on the stream the work ends on. Only the library's entry
points run on the GPU; torch supplies memory, streams and events.

The link. A point-to-point transfer over xGMI moves a block at about one
link's rate (about 150 GB/s) and uses none of the compute GPU's compute units
or memory bandwidth beyond the block's own bytes. Two emulations:
  * `link_cus` > 0: the copy kernel of cpattn_ring_pass with `workgroups`
    workgroups (about 30 GB/s each) on a stream whose CU mask holds only
    `link_cus` compute units, while the compute stream's mask holds every other
    compute unit. The two streams have hardware queues of their own and share
    no compute unit, so the copy neither waits for compute units nor takes any
    from the ring steps, and its traffic is a link's worth of bytes.
  * `link_cus` = 0, `workgroups` = 0: a DMA (SDMA) copy engine. It uses no
    compute unit, but it copies at several hundred GB/s, far above a link, and
    that read + write traffic slows the ring steps beside it.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

from . import (Partial, PrefillDesc, RingEvents, new_partial, ring_pass, ring_prefill_overlapped,
               ring_step_partial)

LOW, HIGH = 0.5, 2.0          # the middle band of compute/transfer ratios
MAX_FACTOR, SUM_FACTOR = 1.1, 0.7
METAMORPHIC_LIMIT = 0.10
# the emulated link: the copy kernel on LINK_WORKGROUPS workgroups, on a
# stream whose CU mask holds LINK_CUS compute units
LINK_CUS = 8
LINK_WORKGROUPS = 3


@dataclass
class RingInputs:
    desc: PrefillDesc
    q: List["torch.Tensor"]            # rank r's query rows, [S/cp, n_hq, d]
    k_blocks: List["torch.Tensor"]     # block held by each rank, [S/cp, n_kv, d]
    v_blocks: List["torch.Tensor"]
    k_recv: List["torch.Tensor"]       # cp * n_recv receive buffers, rank-major
    v_recv: List["torch.Tensor"]
    acc: List[Partial]                 # one accumulator per rank
    events: RingEvents

    @property
    def n_recv(self) -> int:
        return len(self.k_recv) // self.desc.cp

    @property
    def block_bytes(self) -> int:
        t = self.k_blocks[0]
        return t.numel() * t.element_size()

    def in_hand(self, r: int, i: int):
        """K and V blocks rank r holds at step i (its own, then received)."""
        if i == 0:
            return self.k_blocks[r], self.v_blocks[r]
        b = r * self.n_recv + (i - 1) % self.n_recv
        return self.k_recv[b], self.v_recv[b]


def make_inputs(desc: PrefillDesc, q: Sequence, k_blocks: Sequence, v_blocks: Sequence,
                n_recv: int = 3) -> RingInputs:
    import torch
    cp = desc.cp
    rows = desc.rows
    recv = lambda: [torch.empty_like(k_blocks[0]) for _ in range(cp * n_recv)] if cp > 1 else []
    return RingInputs(desc, list(q), list(k_blocks), list(v_blocks), recv(), recv(),
                      [new_partial(rows, desc.n_hq, desc.head_dim, device=q[0].device) for _ in range(cp)],
                      RingEvents(2 * cp))


def _median_ms(fn, stream, reps: int, warmup: int) -> float:
    import torch
    times = []
    for i in range(warmup + reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= warmup:
            times.append(e0.elapsed_time(e1))
    return float(np.median(times))


def compute_ms(x: RingInputs, stream, reps: int = 5, warmup: int = 1) -> float:
    """The ring steps of every rank alone, in the order the overlapped ring
    issues them (each rank on the block of rank (r - i) mod cp)."""
    cp = x.desc.cp

    def run():
        for i in range(cp):
            for r in range(cp):
                j = (r - i) % cp
                ring_step_partial(x.desc, r, i, x.q[r], x.k_blocks[j], x.v_blocks[j], x.acc[r],
                                  accumulate=i > 0, stream=stream)
    return _median_ms(run, stream, reps, warmup)


def transfer_ms(x: RingInputs, workgroups: int, stream, reps: int = 5, warmup: int = 1) -> float:
    """The forwarding copies of every rank alone: the transfers of the
    overlapped ring, step by step."""
    cp = x.desc.cp

    def run():
        for i in range(cp - 1):
            for r in range(cp):
                k, v = x.in_hand(r, i)
                b = ((r + 1) % cp) * x.n_recv + i % x.n_recv
                ring_pass(k, x.k_recv[b], workgroups, stream)
                ring_pass(v, x.v_recv[b], workgroups, stream)
    return _median_ms(run, stream, reps, warmup)


def ring_ms(x: RingInputs, workgroups: int, compute_stream, transfer_stream, reps: int = 5,
            warmup: int = 1) -> float:
    def run():
        ring_prefill_overlapped(x.desc, x.q, x.k_blocks, x.v_blocks, x.k_recv, x.v_recv, x.acc, workgroups,
                                compute_stream, transfer_stream, x.events)
    return _median_ms(run, compute_stream, reps, warmup)


def overlap_effective(x: RingInputs, workgroups: int, compute_stream, transfer_stream, reps: int = 5) -> dict:
    """The spec's "overlap effective" measurement at one transfer width."""
    t_c = compute_ms(x, compute_stream, reps)
    t_t = transfer_ms(x, workgroups, transfer_stream, reps)
    t_r = ring_ms(x, workgroups, compute_stream, transfer_stream, reps)
    t_s = ring_ms(x, workgroups, compute_stream, compute_stream, reps)
    big, total = max(t_c, t_t), t_c + t_t
    return {
        "workgroups": workgroups, "compute_ms": t_c, "transfer_ms": t_t, "ring_ms": t_r, "serial_ms": t_s,
        "ratio": t_t / t_c, "in_band": LOW <= t_t / t_c <= HIGH,
        "ring_over_max": t_r / big, "ring_over_sum": t_r / total, "serial_over_sum": t_s / total,
        "overlap_effective": t_r <= MAX_FACTOR * big and t_r <= SUM_FACTOR * total,
        "serial_rejected": not (t_s <= MAX_FACTOR * big and t_s <= SUM_FACTOR * total),
        "transfer_gb_per_s": 2 * x.desc.cp * (x.desc.cp - 1) * x.block_bytes / (t_t * 1e6),
    }


def overlap_metamorphic(x: RingInputs, workgroups: int, compute_stream, transfer_stream, reps: int = 3) -> dict:
    """The spec's "overlap metamorphic" check: at large S/cp the overlapped ring
    stays within 10% of the pure compute time."""
    t_c = compute_ms(x, compute_stream, reps)
    t_t = transfer_ms(x, workgroups, transfer_stream, reps)
    t_r = ring_ms(x, workgroups, compute_stream, transfer_stream, reps)
    dev = abs(t_r - t_c) / t_c
    return {"workgroups": workgroups, "compute_ms": t_c, "transfer_ms": t_t, "ring_ms": t_r,
            "deviation": dev, "within_limit": dev < METAMORPHIC_LIMIT}


_STREAMS: dict = {}


def _masked_stream(bits: Sequence[int], n_cu: int, dev: int):
    import torch
    hip = ctypes.CDLL("libamdhip64.so")
    words = (n_cu + 31) // 32
    mask = [0] * words
    for b in bits:
        mask[b // 32] |= 1 << (b % 32)
    arr = (ctypes.c_uint32 * words)(*mask)
    handle = ctypes.c_void_p()
    rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), ctypes.c_uint32(words), arr)
    if rc != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask failed with HIP error {rc}")
    return torch.cuda.ExternalStream(handle.value, device=dev)


def link_streams(link_cus: int) -> Tuple[object, object]:
    """(compute stream, transfer stream) of the current device, each on a
    hardware queue of its own: the transfer stream's CU mask holds the first
    `link_cus` mask bits, the compute stream's every other bit (link_cus = 0:
    both hold every compute unit). Created once per process and kept until it
    ends (default priority)."""
    import torch
    dev = torch.cuda.current_device()
    key = (dev, link_cus)
    if key not in _STREAMS:
        n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
        if not 0 <= link_cus < n_cu:
            raise ValueError(f"link_cus must lie in [0, {n_cu})")
        comp = _masked_stream(range(link_cus, n_cu) if link_cus else range(n_cu), n_cu, dev)
        xfer = _masked_stream(range(link_cus) if link_cus else range(n_cu), n_cu, dev)
        _STREAMS[key] = (comp, xfer)
    return _STREAMS[key]
