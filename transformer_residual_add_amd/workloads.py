"""Seeded synthetic inputs for the row kernels (SkipLayerNormalization,
its root-mean-square form, BiasAdd and BiasSoftmax).

This module only draws random numbers and rounds them to the I/O element
type; it holds none of the operator's arithmetic.  Both the HIP path (via the
tests and the benchmark) and the CPU oracle consume the arrays it returns, so
the two sides always see the same bytes.

Tensor roles follow the com.microsoft SkipLayerNormalization WebGPU manifest
(`inputs`: input, skip, gamma, beta, bias; `outputs`: output and the optional
input_skip_bias_sum).  Rank-3 input ``(N, S, H)`` is addressed as
``rows = N * S`` rows of ``H`` contiguous elements; a broadcast skip has
``S`` rows (the manifest's `Params.skipRows` = numel(skip) / H).  For
BiasSoftmax (com.microsoft BiasSoftmax manifest) ``input`` is the data,
``rows`` its batchCount, ``H`` its blockSize, and ``skip`` the bias rows
(biasBlockCount of them), reused cyclically or, with ``inner``, by
consecutive groups of rows.

Recipe (one per tensor, fixed draw order input, skip, bias, gamma, beta):

* Large tensors are drawn in blocks of ``BLOCK_ROWS`` rows.  Block ``b`` of
  tensor ``t`` uses ``numpy.random.default_rng([seed, t, b])``, so any row
  block can be regenerated on its own (the oracle checks sampled rows of the
  largest workloads without materialising the whole tensor).
* Per-column vectors (bias, gamma, beta) use ``default_rng([seed, t])``.
* Values are drawn in float64 (``mu + sigma * standard_normal`` or
  ``uniform(lo, hi)``) and rounded once, round-to-nearest-even, to the I/O
  type (numpy converts float64 to float16 directly, without passing through
  float32).
* An additive key-padding mask (``padmask(min_keep, fill)``): each row keeps
  its first ``ceil(H * u)`` columns at 0, ``u ~ uniform(min_keep, 1)`` drawn
  per row, and sets the rest to ``fill`` (e.g. -10000 or -inf) -- the
  length mix of padded attention batches.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import numpy as np

BLOCK_ROWS = 256

# Tensor ids used as the second element of every seed sequence.
T_INPUT, T_SKIP, T_BIAS, T_GAMMA, T_BETA = 0, 1, 2, 3, 4

DTYPES = {"f32": np.float32, "f16": np.float16}


@dataclass(frozen=True)
class Dist:
    """A scalar distribution: ``normal`` (mu, sigma) or ``uniform`` (lo, hi)."""

    kind: str
    a: float
    b: float

    def draw(self, rng: np.random.Generator, shape) -> np.ndarray:
        if self.kind == "normal":
            return self.a + self.b * rng.standard_normal(shape)
        if self.kind == "uniform":
            return rng.uniform(self.a, self.b, shape)
        if self.kind == "padmask":
            n_rows, h = shape
            keep = np.maximum(1, np.ceil(h * rng.uniform(self.a, 1.0, n_rows))).astype(np.int64)
            out = np.zeros(shape)
            out[np.arange(h)[None, :] >= keep[:, None]] = self.b
            return out
        raise ValueError(f"unknown distribution {self.kind!r}")


def normal(mu: float, sigma: float) -> Dist:
    return Dist("normal", float(mu), float(sigma))


def uniform(lo: float, hi: float) -> Dist:
    return Dist("uniform", float(lo), float(hi))


def padmask(min_keep: float, fill: float) -> Dist:
    return Dist("padmask", float(min_keep), float(fill))


@dataclass(frozen=True)
class Workload:
    """One synthetic SkipLayerNormalization problem.

    ``shape`` is the logical input shape (rank 2 ``(rows, H)`` or rank 3
    ``(N, S, H)``).  ``skip_shape`` is the skip tensor's shape: equal to
    ``shape`` for an exact skip, ``(S, H)`` or ``(1, S, H)`` for a skip
    broadcast across the batch.
    """

    name: str
    shape: Tuple[int, ...]
    dtype: str
    skip_shape: Tuple[int, ...]
    input_dist: Dist
    skip_dist: Dist
    gamma_dist: Optional[Dist] = field(default_factory=lambda: uniform(0.5, 1.5))
    beta_dist: Optional[Dist] = field(default_factory=lambda: normal(0.0, 0.1))
    bias_dist: Optional[Dist] = None
    residual: bool = False
    eps: float = 1e-12
    seed: int = 0
    # "layer_norm", "simplified" (root-mean-square form), "bias_add" or
    # "bias_softmax"
    op: str = "layer_norm"
    # BiasSoftmax: bias rows reused by consecutive groups of rows (inner
    # broadcast) instead of cyclically
    inner: bool = False

    @property
    def hidden(self) -> int:
        return int(self.shape[-1])

    @property
    def rows(self) -> int:
        return int(np.prod(self.shape[:-1], dtype=np.int64))

    @property
    def skip_rows(self) -> int:
        return int(np.prod(self.skip_shape[:-1], dtype=np.int64))

    @property
    def broadcast(self) -> bool:
        return tuple(self.skip_shape) != tuple(self.shape)

    @property
    def np_dtype(self):
        return DTYPES[self.dtype]

    @property
    def itemsize(self) -> int:
        return np.dtype(self.np_dtype).itemsize

    def algorithmic_bytes(self) -> int:
        """Bytes the operator must move once: input, skip (the broadcast skip
        counted once), gamma/beta/bias once, output and the optional residual."""
        h, r, b = self.hidden, self.rows, self.itemsize
        n = r * h * b  # input
        n += self.skip_rows * h * b  # skip
        n += h * b if self.gamma_dist is not None else 0
        n += h * b if self.beta_dist is not None else 0
        n += h * b if self.bias_dist is not None else 0
        n += r * h * b  # output
        n += r * h * b if self.residual else 0
        return int(n)

    @property
    def skip_group(self) -> int:
        """Rows sharing one skip row under inner (grouped) reuse, else 0."""
        return self.rows // self.skip_rows if self.inner and self.broadcast and self.skip_rows else 0

    def skip_row_of(self, rows: np.ndarray) -> np.ndarray:
        """Index of the skip row that each of ``rows`` reads."""
        rows = np.asarray(rows, dtype=np.int64)
        if not self.broadcast:
            return rows
        return rows // self.skip_group if self.inner else rows % self.skip_rows

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five synthetic workloads: a tiny rank-3 fp32 case, a BERT-base-shaped
# fp32 case that emits the residual, a rank-2 fp16 case, a rank-3 fp32 case with
# a skip broadcast across the batch, and a large rank-2 fp16 case whose rows
# have mean ~100 (variance cancellation).  Where a distribution is not stated
# for bias/beta the 0-mean, 0.1-sigma law of the other workloads is used, and a
# skip with no stated law is standard normal.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(
            name="tiny_2x8x64_f32",
            shape=(2, 8, 64),
            dtype="f32",
            skip_shape=(2, 8, 64),
            input_dist=normal(0, 1),
            skip_dist=normal(0, 1),
            eps=1e-12,
            seed=1001,
        ),
        Workload(
            name="bert_base_8x128x768_f32",
            shape=(8, 128, 768),
            dtype="f32",
            skip_shape=(8, 128, 768),
            input_dist=normal(0, 1),
            skip_dist=normal(0, 0.5),
            bias_dist=normal(0, 0.1),
            residual=True,
            eps=1e-12,
            seed=1002,
        ),
        Workload(
            name="rows16384_h1024_f16",
            shape=(16384, 1024),
            dtype="f16",
            skip_shape=(16384, 1024),
            input_dist=normal(0, 1),
            skip_dist=normal(0, 1),
            bias_dist=normal(0, 0.1),
            residual=True,
            eps=1e-5,
            seed=1003,
        ),
        Workload(
            name="bcast_64x512x4096_f32",
            shape=(64, 512, 4096),
            dtype="f32",
            skip_shape=(512, 4096),
            input_dist=normal(0, 1),
            skip_dist=normal(0, 1),
            eps=1e-12,
            seed=1004,
        ),
        Workload(
            name="rows65536_h8192_f16_mean100",
            shape=(65536, 8192),
            dtype="f16",
            skip_shape=(65536, 8192),
            input_dist=normal(100, 1),
            skip_dist=normal(0, 1),
            bias_dist=normal(0, 0.1),
            residual=True,
            eps=1e-5,
            seed=1005,
        ),
    ]
}

# Workloads in the order they are listed above.
ORDER = list(WORKLOADS)

# The same data flows through the two other operations of the row kernels:
# BiasAdd (com.microsoft BiasAdd manifest; (N, S, C) input, skip of the same
# shape, length-C bias) and the root-mean-square ("simplified") form.
EXTRA: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(
            name="biasadd_8x128x768_f32",
            shape=(8, 128, 768),
            dtype="f32",
            skip_shape=(8, 128, 768),
            input_dist=normal(0, 1),
            skip_dist=normal(0, 0.5),
            gamma_dist=None,
            beta_dist=None,
            bias_dist=normal(0, 0.1),
            seed=1011,
            op="bias_add",
        ),
        Workload(
            name="biasadd_64x512x4096_f16",
            shape=(64, 512, 4096),
            dtype="f16",
            skip_shape=(64, 512, 4096),
            input_dist=normal(0, 1),
            skip_dist=normal(0, 1),
            gamma_dist=None,
            beta_dist=None,
            bias_dist=normal(0, 0.1),
            seed=1012,
            op="bias_add",
        ),
        Workload(
            name="rms_rows65536_h8192_f16",
            shape=(65536, 8192),
            dtype="f16",
            skip_shape=(65536, 8192),
            input_dist=normal(0, 1),
            skip_dist=normal(0, 1),
            bias_dist=normal(0, 0.1),
            residual=True,
            eps=1e-5,
            seed=1013,
            op="simplified",
        ),
        # 2 GiB layer norms of common hidden sizes (one block per row tile, the
        # single-tile kernel form).
        *[Workload(name=f"rows{rows}_h{h}_f16", shape=(rows, h), dtype="f16", skip_shape=(rows, h),
                   input_dist=normal(0, 1), skip_dist=normal(0, 1), bias_dist=normal(0, 0.1), residual=True,
                   eps=1e-5, seed=1040 + i)
          for i, (rows, h) in enumerate(((65536, 4096), (131072, 2048), (16384, 16384)))],
        # A large launch of float32 rows past the LDS-staged kernel's switch
        # point (3072 chunks per row: 1024-lane single-tile row tiles).
        Workload(name="rows16384_h12288_f32", shape=(16384, 12288), dtype="f32", skip_shape=(16384, 12288),
                 input_dist=normal(0, 1), skip_dist=normal(0, 1), bias_dist=normal(0, 0.1), residual=True, eps=1e-5,
                 seed=1044),
        # ... and of 3584 chunks (1024 x 4 tiles, one block per CU).
        Workload(name="rows16384_h14336_f32", shape=(16384, 14336), dtype="f32", skip_shape=(16384, 14336),
                 input_dist=normal(0, 1), skip_dist=normal(0, 1), bias_dist=normal(0, 0.1), residual=True, eps=1e-5,
                 seed=1045),
        # Rows beyond one workgroup's LDS (65536 values): the register-resident
        # rows against the generic kernel's chunk form (part of each row
        # parked in LDS) and the split-row kernels; 512 rows, so that every CU
        # holds a row or two, and 4096 rows, sixteen per CU.
        Workload(
            name="longrow_512x65536_f32",
            shape=(512, 65536),
            dtype="f32",
            skip_shape=(512, 65536),
            input_dist=normal(0, 1),
            skip_dist=normal(0, 1),
            bias_dist=normal(0, 0.1),
            residual=True,
            eps=1e-5,
            seed=1031,
        ),
        Workload(
            name="longrow_4096x65536_f32",
            shape=(4096, 65536),
            dtype="f32",
            skip_shape=(4096, 65536),
            input_dist=normal(0, 1),
            skip_dist=normal(0, 1),
            bias_dist=normal(0, 0.1),
            residual=True,
            eps=1e-5,
            seed=1033,
        ),
        Workload(
            name="rms_longrow_512x65536_f16",
            shape=(512, 65536),
            dtype="f16",
            skip_shape=(512, 65536),
            input_dist=normal(0, 1),
            skip_dist=normal(0, 1),
            bias_dist=normal(0, 0.1),
            residual=True,
            eps=1e-5,
            seed=1032,
            op="simplified",
        ),
        # BiasSoftmax on attention scores: (batch, heads, queries, keys) data,
        # softmax over the keys.  A per-sequence key-padding mask (B, 1, 1, K)
        # is shared by the heads x queries rows of each sequence (inner
        # broadcast); a per-head position bias (1, heads, Q, K) is shared by
        # every sequence of the batch (outer broadcast).
        Workload(
            name="softmax_attn_16x16x512x512_f16_padmask",
            shape=(16 * 16 * 512, 512),
            dtype="f16",
            skip_shape=(16, 512),
            input_dist=normal(0, 2),
            skip_dist=padmask(0.25, -float("inf")),
            gamma_dist=None,
            beta_dist=None,
            seed=1021,
            op="bias_softmax",
            inner=True,
        ),
        Workload(
            name="softmax_relpos_64x12x128x128_f32",
            shape=(64 * 12 * 128, 128),
            dtype="f32",
            skip_shape=(12 * 128, 128),
            input_dist=normal(0, 2),
            skip_dist=normal(0, 1),
            gamma_dist=None,
            beta_dist=None,
            seed=1022,
            op="bias_softmax",
        ),
        # A per-head position bias over a long sequence (16 heads x 2048
        # queries x 2048 keys, 128 MiB) shared by the 8 sequences of the batch
        # (outer broadcast): larger than the caches, so each block keeps its
        # bias rows across batches.
        Workload(
            name="softmax_headbias_8x16x2048x2048_f16",
            shape=(8 * 16 * 2048, 2048),
            dtype="f16",
            skip_shape=(16 * 2048, 2048),
            input_dist=normal(0, 2),
            skip_dist=normal(0, 1),
            gamma_dist=None,
            beta_dist=None,
            seed=1025,
            op="bias_softmax",
        ),
        # Attention over 1500 keys (an audio encoder's frames), with an
        # additive bias as large as the scores (one bias row per data row):
        # rows of 3000 bytes, not whole 16-byte chunks, so each row starts at
        # its own offset within a chunk.
        Workload(
            name="softmax_frames_8x8x1500x1500_f16_fullbias",
            shape=(8 * 8 * 1500, 1500),
            dtype="f16",
            skip_shape=(8 * 8 * 1500, 1500),
            input_dist=normal(0, 2),
            skip_dist=normal(0, 1),
            gamma_dist=None,
            beta_dist=None,
            seed=1024,
            op="bias_softmax",
        ),
        # Softmax over a vocabulary (sampling from language-model logits): rows
        # of 128256 values, beyond one workgroup's LDS, so they split across
        # workgroups; one bias row (a logit bias) shared by every row.
        Workload(
            name="softmax_vocab_4096x128256_f16",
            shape=(4096, 128256),
            dtype="f16",
            skip_shape=(1, 128256),
            input_dist=normal(0, 3),
            skip_dist=normal(0, 0.5),
            gamma_dist=None,
            beta_dist=None,
            seed=1023,
            op="bias_softmax",
        ),
        Workload(
            name="rms_bert_base_8x128x768_f32",
            shape=(8, 128, 768),
            dtype="f32",
            skip_shape=(8, 128, 768),
            input_dist=normal(0, 1),
            skip_dist=normal(0, 0.5),
            bias_dist=normal(0, 0.1),
            residual=True,
            eps=1e-6,
            seed=1014,
            op="simplified",
        ),
    ]
}


def get(name: str) -> Workload:
    """A workload of WORKLOADS or EXTRA by name."""
    return WORKLOADS[name] if name in WORKLOADS else EXTRA[name]


def _round(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a.astype(dtype))


def vector(w: Workload, tensor: int) -> Optional[np.ndarray]:
    """gamma / beta / bias of length H, or None when the workload has none."""
    dist = {T_GAMMA: w.gamma_dist, T_BETA: w.beta_dist, T_BIAS: w.bias_dist}[tensor]
    if dist is None:
        return None
    rng = np.random.default_rng([w.seed, tensor])
    return _round(dist.draw(rng, (w.hidden,)), w.np_dtype)


def row_block(w: Workload, tensor: int, block: int, n_rows_total: int) -> np.ndarray:
    """Rows ``[block*BLOCK_ROWS, ...)`` of the input (tensor 0) or skip (1)."""
    dist = {T_INPUT: w.input_dist, T_SKIP: w.skip_dist}[tensor]
    r0 = block * BLOCK_ROWS
    r1 = min(n_rows_total, r0 + BLOCK_ROWS)
    rng = np.random.default_rng([w.seed, tensor, block])
    return _round(dist.draw(rng, (r1 - r0, w.hidden)), w.np_dtype)


def _fill(w: Workload, tensor: int, n_rows: int, threads: int) -> np.ndarray:
    out = np.empty((n_rows, w.hidden), dtype=w.np_dtype)
    n_blocks = (n_rows + BLOCK_ROWS - 1) // BLOCK_ROWS

    def one(b):
        r0 = b * BLOCK_ROWS
        blk = row_block(w, tensor, b, n_rows)
        out[r0 : r0 + blk.shape[0]] = blk

    if threads <= 1 or n_blocks <= 1:
        for b in range(n_blocks):
            one(b)
    else:
        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(n_blocks)))
    return out


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_inputs(w: Workload, threads: Optional[int] = None) -> Dict[str, Optional[np.ndarray]]:
    """All inputs of ``w`` as host arrays of the I/O type.

    ``input`` is ``(rows, H)``, ``skip`` is ``(skip_rows, H)``; reshape to the
    logical shapes with ``w.shape`` / ``w.skip_shape``.
    """
    t = default_threads() if threads is None else threads
    return {
        "input": _fill(w, T_INPUT, w.rows, t),
        "skip": _fill(w, T_SKIP, w.skip_rows, t),
        "bias": vector(w, T_BIAS),
        "gamma": vector(w, T_GAMMA),
        "beta": vector(w, T_BETA),
    }


def make_rows(w: Workload, r0: int, r1: int) -> Dict[str, Optional[np.ndarray]]:
    """Rows ``[r0, r1)`` of the input, with the skip rows those rows read.

    Returns the same dict as :func:`make_inputs`, where ``input`` holds only
    rows ``[r0, r1)`` (bit-identical to the same rows of ``make_inputs``) and
    ``skip`` is the matching exact-skip slice, or the whole broadcast skip.
    """
    assert 0 <= r0 <= r1 <= w.rows
    b0, b1 = r0 // BLOCK_ROWS, (r1 + BLOCK_ROWS - 1) // BLOCK_ROWS

    def rows_of(tensor, n_total):
        parts = [row_block(w, tensor, b, n_total) for b in range(b0, b1)]
        if not parts:
            return np.empty((0, w.hidden), dtype=w.np_dtype)
        blk = np.concatenate(parts)
        off = r0 - b0 * BLOCK_ROWS
        return np.ascontiguousarray(blk[off : off + (r1 - r0)])

    x = rows_of(T_INPUT, w.rows)
    if w.broadcast:
        skip = _fill(w, T_SKIP, w.skip_rows, default_threads())
    else:
        skip = rows_of(T_SKIP, w.skip_rows)
    return {
        "input": x,
        "skip": skip,
        "bias": vector(w, T_BIAS),
        "gamma": vector(w, T_GAMMA),
        "beta": vector(w, T_BETA),
    }


def small_case(
    rows: int,
    hidden: int,
    dtype: str = "f32",
    *,
    skip_rows: Optional[int] = None,
    beta: bool = True,
    bias: bool = False,
    residual: bool = False,
    eps: float = 1e-5,
    seed: int = 7,
    input_dist: Dist = normal(0, 1),
    skip_dist: Dist = normal(0, 1),
    op: str = "layer_norm",
    inner: bool = False,
) -> Workload:
    """A workload for the flag/shape matrix of the parity tests.

    Rank 2 ``(rows, H)`` with an exact skip, or, when ``skip_rows`` is given
    and differs from ``rows``, rank 3 ``(rows // skip_rows, skip_rows, H)``
    with an ``(S, H)`` skip broadcast across the batch.  BiasSoftmax keeps
    rank 2: ``(rows, H)`` data and ``(skip_rows, H)`` bias rows, reused by
    groups (``inner``) or cyclically.
    """
    softmax = op == "bias_softmax"
    if skip_rows is None or skip_rows == rows:
        shape, skip_shape = (rows, hidden), (rows, hidden)
    elif softmax:
        assert skip_rows > 0 and rows % skip_rows == 0
        shape, skip_shape = (rows, hidden), (skip_rows, hidden)
    else:
        assert skip_rows > 0 and rows % skip_rows == 0
        shape, skip_shape = (rows // skip_rows, skip_rows, hidden), (skip_rows, hidden)
    if softmax:
        return Workload(
            name=f"case_{op}_{rows}x{hidden}_{dtype}",
            shape=shape,
            dtype=dtype,
            skip_shape=skip_shape,
            input_dist=input_dist,
            skip_dist=skip_dist,
            gamma_dist=None,
            beta_dist=None,
            bias_dist=None,
            residual=False,
            eps=0.0,
            seed=seed,
            op=op,
            inner=inner,
        )
    bias_add = op == "bias_add"
    return Workload(
        name=f"case_{op}_{rows}x{hidden}_{dtype}",
        shape=shape,
        dtype=dtype,
        skip_shape=skip_shape,
        input_dist=input_dist,
        skip_dist=skip_dist,
        gamma_dist=None if bias_add else uniform(0.5, 1.5),
        beta_dist=normal(0, 0.1) if beta and not bias_add else None,
        bias_dist=normal(0, 0.1) if bias or bias_add else None,
        residual=residual and not bias_add,
        eps=eps,
        seed=seed,
        op=op,
    )
