"""Seeded synthetic inputs for the row-reduce operations.

This module only draws random numbers and lays them out; it holds none of the
operations' arithmetic.  Both the GPU parity tests and the CPU oracle take
their inputs from here (and nowhere else), so the two sides see exactly the
same numbers.

Conventions
-----------
* Generator: ``numpy.random.default_rng(seed)`` (PCG64), one generator per
  workload, draws taken in the order listed for each workload, in float32.
* bf16 tensors are made from the float32 draws with torch's
  ``.to(torch.bfloat16)`` (round to nearest, ties to even).
* "N(0, s)" means a normal draw with standard deviation s.
* All arrays are row-major and contiguous: element (i, j) of an [M, N] array
  sits at offset i * N + j.

The five named workloads mirror the pages' own shapes (Qwen2.5-7B hidden size
3584 and vocabulary 152064, 28 heads x 4096 x 4096 attention scores, an
8192 x 4096 bf16 RMSNorm):

========  ==========================================================  =========
name      what                                                        sizes
========  ==========================================================  =========
rms_f32   RMSNorm fp32, x~N(0,1), gamma~U(0.5,1.5), eps 1e-6          64 x 3584
fused     fused residual add + RMSNorm, bf16 I/O; x, residual~N(0,1);  8192 x 4096
          gamma~U(0.5,1.5); eps 1e-6
sm_wave   softmax fp32 -> fp32, x~N(0,8), rows i%7==6 get +1000       16384 x 1024
sm_vocab  softmax bf16 -> fp32, x~N(0,3), 16 distinct columns per     256 x 152064
          row overwritten by U(20,30) spikes before the bf16 cast
sm_causal softmax fp32 -> fp32 attention scores, x~N(0,1); row r is   114688 x 4096
          query i = r mod 4096 and keys j > i hold -inf (diagonal
          kept)
layernorm LayerNorm fp32, x~U(100,102) (mean far above the spread),    256 x 5120
          gamma~U(0.5,1.5), beta~U(-1,1), eps 1e-5
========  ==========================================================  =========
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

NAMES = ("rms_f32", "fused", "sm_wave", "sm_vocab", "sm_causal", "layernorm")


@dataclass
class Workload:
    name: str
    op: str                 # "rmsnorm" | "fused_add_rmsnorm" | "softmax"
    M: int
    N: int
    in_dtype: str           # "f32" | "bf16"
    out_dtype: str
    eps: float = 0.0
    seed: int = 0
    arrays: dict = field(default_factory=dict)   # name -> torch CPU tensor

    @property
    def description(self) -> str:
        return f"{self.name}: {self.op} {self.M}x{self.N} {self.in_dtype}->{self.out_dtype}"


SHAPES = {
    "rms_f32": ("rmsnorm", 64, 3584, "f32", "f32", 1e-6),
    "fused": ("fused_add_rmsnorm", 8192, 4096, "bf16", "bf16", 1e-6),
    "sm_wave": ("softmax", 16384, 1024, "f32", "f32", 0.0),
    "sm_vocab": ("softmax", 256, 152064, "bf16", "f32", 0.0),
    "sm_causal": ("softmax", 28 * 4096, 4096, "f32", "f32", 0.0),
    "layernorm": ("layernorm", 256, 5120, "f32", "f32", 1e-5),
}


def _torch():
    import torch
    return torch


def to_dtype(a_f32: np.ndarray, dtype: str):
    """float32 numpy array -> torch CPU tensor of the I/O dtype (RNE for bf16)."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


def causal_mask_inplace(x: np.ndarray, period: int, row0: int = 0) -> None:
    """Set x[r, j] = -inf for j > (row0 + r) mod period (keys after the query)."""
    M, N = x.shape
    for r in range(M):
        i = (row0 + r) % period
        if i + 1 < N:
            x[r, i + 1:] = -np.inf


def make(name: str, rows: Optional[int] = None, seed: int = 0) -> Workload:
    """Build one named workload.  ``rows`` keeps only the first rows: their
    values are exactly the first rows of the full-size workload (numpy fills
    a float32 normal draw in row-major order, so a shorter draw is a prefix
    of the longer one; per-row draws that follow the bulk draw are taken for
    every row of the full size before slicing)."""
    op, M_full, N, idt, odt, eps = SHAPES[name]
    M = M_full if rows is None else min(M_full, int(rows))
    w = Workload(name, op, M, N, idt, odt, eps, seed)
    rng = np.random.default_rng(seed)
    if name == "rms_f32":
        x = rng.standard_normal((M_full, N), dtype=np.float32)[:M]
        g = rng.uniform(0.5, 1.5, N).astype(np.float32)
        w.arrays = {"x": to_dtype(x, idt), "gamma": to_dtype(g, idt)}
    elif name == "fused":
        x = rng.standard_normal((M_full, N), dtype=np.float32)[:M]
        r = rng.standard_normal((M_full, N), dtype=np.float32)[:M]
        g = rng.uniform(0.5, 1.5, N).astype(np.float32)
        w.arrays = {"x": to_dtype(x, idt), "residual": to_dtype(r, idt),
                    "gamma": to_dtype(g, idt)}
    elif name == "sm_wave":
        x = rng.standard_normal((M, N), dtype=np.float32) * np.float32(8.0)
        x[np.arange(M) % 7 == 6] += np.float32(1000.0)
        w.arrays = {"x": to_dtype(x, idt)}
    elif name == "sm_vocab":
        x = rng.standard_normal((M_full, N), dtype=np.float32) * np.float32(3.0)
        for r in range(M_full):
            cols = rng.choice(N, 16, replace=False)
            x[r, cols] = rng.uniform(20.0, 30.0, 16).astype(np.float32)
        w.arrays = {"x": to_dtype(x[:M], idt)}
    elif name == "sm_causal":
        x = rng.standard_normal((M, N), dtype=np.float32)
        causal_mask_inplace(x, 4096)
        w.arrays = {"x": to_dtype(x, idt)}
    elif name == "layernorm":
        x = rng.uniform(100.0, 102.0, (M_full, N)).astype(np.float32)[:M]
        g = rng.uniform(0.5, 1.5, N).astype(np.float32)
        b = rng.uniform(-1.0, 1.0, N).astype(np.float32)
        w.arrays = {"x": to_dtype(x, idt), "gamma": to_dtype(g, idt), "beta": to_dtype(b, idt)}
    else:
        raise KeyError(name)
    return w


def causal_rows(row_ids, N: int = 4096, period: int = 4096, seed: int = 0,
                M_full: int = 28 * 4096) -> np.ndarray:
    """Rows ``row_ids`` of the full ``sm_causal`` input, drawn without
    materialising the whole tensor: the full draw is row-major, so row r's
    values are standard normals number r*N .. r*N+N-1 of the stream.  The
    generator is advanced in row-sized steps (identical values to ``make``)."""
    row_ids = sorted(int(r) for r in row_ids)
    rng = np.random.default_rng(seed)
    out = np.empty((len(row_ids), N), dtype=np.float32)
    cur = 0
    k = 0
    chunk = 256
    while k < len(row_ids):
        target = row_ids[k]
        # skip whole blocks of rows before the next wanted row
        while cur + chunk <= target:
            rng.standard_normal((chunk, N), dtype=np.float32)
            cur += chunk
        n = min(chunk, M_full - cur)
        block = rng.standard_normal((n, N), dtype=np.float32)
        while k < len(row_ids) and row_ids[k] < cur + n:
            out[k] = block[row_ids[k] - cur]
            k += 1
        cur += n
    for i, r in enumerate(row_ids):
        q = r % period
        out[i, q + 1:] = -np.inf
    return out


def random_rows(M: int, N: int, seed: int, kind: str = "normal", scale: float = 1.0,
                offset_every: int = 0, offset: float = 0.0, masked_frac: float = 0.0,
                full_mask_rows=()) -> np.ndarray:
    """General float32 test rows: N(0, scale) draws, an optional offset on
    rows i % offset_every == offset_every - 1, an optional fraction of -inf
    entries (never the row's first column, so each row keeps a finite entry)
    and optional fully -inf rows."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        x = (scale * rng.standard_normal((M, N), dtype=np.float32)).astype(np.float32)
    elif kind == "uniform":
        x = rng.uniform(-scale, scale, (M, N)).astype(np.float32)
    else:
        raise ValueError(kind)
    if offset_every:
        x[np.arange(M) % offset_every == offset_every - 1] += np.float32(offset)
    if masked_frac > 0.0 and N > 1:
        mask = rng.random((M, N)) < masked_frac
        mask[:, 0] = False
        x[mask] = -np.inf
    for r in full_mask_rows:
        if 0 <= r < M:
            x[r, :] = -np.inf
    return x


def gamma_vector(N: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.uniform(0.5, 1.5, N).astype(np.float32)
