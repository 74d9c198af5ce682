"""Seeded synthetic workloads for SQuad-Attention.

This module holds the workload shapes and the seeded input generators, and
nothing of the attention arithmetic itself.  Both the fp64 oracle (through the
tests) and the HIP path draw their inputs from here, so it must stay free of any
softmax, matmul or re-indexing logic.

Shapes follow the pages' workloads:
  * Wan 2.2 5B at 81x704x1280: latent grid 21x22x40 (n = 18,480), window
    21x2x4 = 168 tokens, 110 windows, 24 heads of dim 128 (agihunt.info
    summary, results table; paperpeel full text, sec. 4.2 and the appendix
    paragraph on the FLOP sweep).
  * Wan 2.1 1.3B at 480x832x81: n = 32,760, 12 heads of dim 128, window
    21x2x4 (paperpeel full text, sec. 4.2).
  * 4x the 5B tokens (n = 73,920, window 21x4x4) and a 14B-shaped block
    (40 heads) at the same grid, batched over a CFG pair.

Value recipe (in the pages' video models a handful of keys take most of a
query's softmax weight -- agihunt.info summary, the paragraph on the
observation the method starts from):
  Q, K, V ~ N(0, 1) drawn in float32; for the bf16 workloads, round(0.02 n)
  distinct token positions per batch element have their K rows multiplied by 4
  for every head; then every tensor is rounded to bf16 (round to nearest even).

Each (tensor, batch, head) slice comes from its own PCG64 stream seeded with
SeedSequence([seed, tensor_id, b, h]), so any single head can be regenerated
alone (the oracle checks sampled heads of the large workloads) and the full
tensor is the concatenation of those slices in [B, n, heads, d] layout.
"""

from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_BOOST = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    d: int
    T: int
    Hs: int
    Ws: int
    wt: int
    wh: int
    ww: int
    dtype: str          # "bf16" or "f32"
    boost_frac: float   # fraction of K token rows boosted x4 (0 = none)
    prescale: bool = False  # multiply Q, K, V by d**-0.5 after drawing

    @property
    def n(self) -> int:
        return self.T * self.Hs * self.Ws

    @property
    def m(self) -> int:
        return self.wt * self.wh * self.ww

    @property
    def n_windows(self) -> int:
        return self.n // self.m

    def geometry(self) -> tuple:
        return (self.B, self.heads, self.T, self.Hs, self.Ws, self.wt, self.wh, self.ww, self.d)

    def n_boost(self) -> int:
        return int(round(self.boost_frac * self.n))


WORKLOADS = {
    # tiny fp32 case: 3x4x4 grid, 3x2x2 windows (12 tokens, 4 windows)
    "tiny_f32": Workload("tiny_f32", 1, 2, 64, 3, 4, 4, 3, 2, 2, "f32", 0.0),
    "tiny_f32_prescaled": Workload("tiny_f32_prescaled", 1, 2, 64, 3, 4, 4, 3, 2, 2, "f32", 0.0, prescale=True),
    # Wan 2.2 5B block at 704x1280x81: the headline shape
    "wan5b_704p": Workload("wan5b_704p", 1, 24, 128, 21, 22, 40, 21, 2, 4, "bf16", 0.02),
    # Wan 2.1 1.3B block at 480x832x81
    "wan1p3b_480p": Workload("wan1p3b_480p", 1, 12, 128, 21, 30, 52, 21, 2, 4, "bf16", 0.02),
    # 5B-shaped block at 4x the tokens
    "wan5b_4x": Workload("wan5b_4x", 1, 24, 128, 21, 44, 80, 21, 4, 4, "bf16", 0.02),
    # 14B-shaped block, CFG pair
    "wan14b_4x_cfg": Workload("wan14b_4x_cfg", 2, 40, 128, 21, 44, 80, 21, 4, 4, "bf16", 0.02),
}

HEADLINE = "wan5b_704p"


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the raw uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))
    return ((bits + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def boost_tokens(w: Workload, b: int, seed: int = 0) -> np.ndarray:
    """Sorted token indices whose K rows are boosted x4 in batch element b."""
    nb = w.n_boost()
    if nb == 0:
        return np.zeros(0, dtype=np.int64)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TENSOR_BOOST, b])))
    return np.sort(g.choice(w.n, size=nb, replace=False)).astype(np.int64)


def head_slice_f32(w: Workload, tensor: int, b: int, h: int, seed: int = 0) -> np.ndarray:
    """One [n, d] float32 slice of Q (tensor 0), K (1) or V (2) for batch b, head h.

    The value returned is exactly what the device sees: for bf16 workloads it is
    already rounded to bf16 and widened back to float32.
    """
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, b, h])))
    x = g.standard_normal((w.n, w.d), dtype=np.float32)
    if tensor == TENSOR_K and w.boost_frac > 0:
        x[boost_tokens(w, b, seed)] *= np.float32(4.0)
    if w.prescale:
        x *= np.float32(1.0 / np.sqrt(w.d))
    if w.dtype == "bf16":
        x = bf16_bits_to_f32(bf16_round_bits(x))
    return x


def head_slices_f64(w: Workload, b: int, h: int, seed: int = 0):
    """(q, k, v) for one (b, h) as float64 [n, d] arrays (the oracle's input)."""
    return tuple(head_slice_f32(w, t, b, h, seed).astype(np.float64) for t in (TENSOR_Q, TENSOR_K, TENSOR_V))


def full_inputs_f32(w: Workload, seed: int = 0, heads=None):
    """(q, k, v) as float32 [B, n, heads, d] host arrays (values exactly representable in w.dtype)."""
    hs = range(w.heads) if heads is None else heads
    out = []
    for t in (TENSOR_Q, TENSOR_K, TENSOR_V):
        a = np.zeros((w.B, w.n, w.heads, w.d), dtype=np.float32)
        for b in range(w.B):
            for h in hs:
                a[b, :, h, :] = head_slice_f32(w, t, b, h, seed)
        out.append(a)
    return tuple(out)


def random_geometry_inputs(B, heads, n, d, dtype, seed=0, scale=1.0):
    """Plain N(0, scale^2) [B, n, heads, d] float32 inputs for ad-hoc shapes (edge-case tests)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99, B, heads, n, d])))
    out = []
    for _ in range(3):
        x = (g.standard_normal((B, n, heads, d), dtype=np.float32) * np.float32(scale))
        if dtype == "bf16":
            x = bf16_bits_to_f32(bf16_round_bits(x))
        out.append(x)
    return tuple(out)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 4
    return max(1, min(16, n))


def device_inputs(w: Workload, seed: int = 0, device: str = "cuda"):
    """(q, k, v) as torch tensors [B, n, heads, d] on `device`, in w.dtype.

    Exactly the values head_slice_f32 gives, slice by slice (generated on the
    host in parallel threads, then copied once).
    """
    import torch
    out = []
    for tid in (TENSOR_Q, TENSOR_K, TENSOR_V):
        if w.dtype == "bf16":
            host = np.empty((w.B, w.n, w.heads, w.d), dtype=np.uint16)

            def fill(bh, host=host, tid=tid):
                b, h = bh
                host[b, :, h, :] = bf16_round_bits(head_slice_f32(w, tid, b, h, seed))

            with cf.ThreadPoolExecutor(_workers()) as ex:
                list(ex.map(fill, [(b, h) for b in range(w.B) for h in range(w.heads)]))
            out.append(torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).to(device))
        else:
            host = np.empty((w.B, w.n, w.heads, w.d), dtype=np.float32)
            for b in range(w.B):
                for h in range(w.heads):
                    host[b, :, h, :] = head_slice_f32(w, tid, b, h, seed)
            out.append(torch.from_numpy(host).to(device))
    return tuple(out)
