"""Seeded synthetic inputs for the MoBA forward pass.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the GPU path's tests/benchmark and the CPU oracle's
tests take their inputs from here.

Recipe (per workload and seed):
  * q[T][Hq][d], k[T][Hkv][d], v[T][Hkv][d] are iid N(0, 1) float32;
  * every (sequence, local block of B rows, kv head) gets an offset vector
    0.5 * N(0, 1) of length d that is added to that block's key rows, so block
    means differ and the gate has structure to find;
  * bf16 workloads round the float32 values to bf16 (round to nearest even)
    after the offset is added.
Random streams: tensor X in {q: 0, k: 1, v: 2} is drawn in chunks of whole
rows; chunk i uses PCG64 seeded with SeedSequence([seed, X, i]). The offsets
use SeedSequence([seed, 3]) and are drawn as one [blocks][Hkv][d] array in
global block order. Chunks are independent, so they are drawn in parallel and
the bytes do not depend on the thread count.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROWS_ELEMS_PER_CHUNK = 1 << 22  # about 4M elements per random chunk


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    lengths: tuple
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "fp32" or "bf16"
    block_size: int
    topk: int
    seed: int

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)


def _w(name, lengths, hq, hkv, dtype, B, k, seed, d=128):
    return Workload(name, tuple(lengths), hq, hkv, d, dtype, B, k, seed)


# The shapes of the pages' workloads: an MQAR-shaped multi-head layer (16 heads,
# chunk 256, top-4, length 2048) and Llama-3.1-8B-shaped GQA layers (32 query
# heads, 8 kv heads, d = 128) at 32K / 128K / 1M tokens plus a packed batch.
WORKLOADS = {w.name: w for w in [
    _w("mha16_t2k_b256_k4_fp32", [2048], 16, 16, "fp32", 256, 4, 0),
    _w("gqa32x8_t32k_b512_k3_bf16", [32768], 32, 8, "bf16", 512, 3, 1),
    _w("gqa32x8_t128k_b4096_k12_bf16", [131072], 32, 8, "bf16", 4096, 12, 2),
    _w("gqa32x8_t1m_b4096_k12_bf16", [1048576], 32, 8, "bf16", 4096, 12, 3),
    _w("gqa32x8_varlen4_t256k_b4096_k12_bf16", [8192, 32768, 65536, 155648], 32, 8, "bf16",
       4096, 12, 4),
    # extra packed batch whose sequences end inside a block (short last blocks)
    _w("gqa32x8_varlen4ragged_t256k_b4096_k12_bf16", [5000, 30000, 70000, 157144], 32, 8,
       "bf16", 4096, 12, 4),
]}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _block_index_of_rows(lengths, block_size):
    """Global block index of every row (blocks restart at each sequence)."""
    parts, first = [], 0
    for L in lengths:
        parts.append(first + np.arange(L, dtype=np.int64) // block_size)
        first += -(-L // block_size)
    return (np.concatenate(parts) if parts else np.zeros(0, np.int64)), first


@dataclasses.dataclass
class Inputs:
    workload: Workload
    q: np.ndarray  # float32 or uint16 (bf16 bits)
    k: np.ndarray
    v: np.ndarray
    cu_seqlens: np.ndarray


def generate(w: Workload, seed: int | None = None, threads: int | None = None) -> Inputs:
    seed = w.seed if seed is None else int(seed)
    T, d = w.total_tokens, w.head_dim
    blk_of_row, nblocks = _block_index_of_rows(w.lengths, w.block_size)
    offsets = (np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 3])))
               .standard_normal((max(nblocks, 1), w.num_kv_heads, d), dtype=np.float32)
               * np.float32(0.5))
    out_dtype = np.uint16 if w.dtype == "bf16" else np.float32
    threads = threads or min(16, os.cpu_count() or 1)

    def make(tensor_id, heads, add_offsets):
        arr = np.empty((T, heads, d), dtype=out_dtype)
        rows_per_chunk = max(1, ROWS_ELEMS_PER_CHUNK // (heads * d))
        nchunks = -(-T // rows_per_chunk)

        def fill(i):
            r0, r1 = i * rows_per_chunk, min(T, (i + 1) * rows_per_chunk)
            g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, i])))
            x = g.standard_normal((r1 - r0, heads, d), dtype=np.float32)
            if add_offsets:
                x += offsets[blk_of_row[r0:r1]]
            arr[r0:r1] = f32_to_bf16_bits(x) if out_dtype == np.uint16 else x

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
        return arr

    q = make(0, w.num_q_heads, False)
    k = make(1, w.num_kv_heads, True)
    v = make(2, w.num_kv_heads, False)
    return Inputs(w, q, k, v, w.cu_seqlens())


def custom(lengths, hq, hkv, d, dtype, block_size, topk, seed, name="custom") -> Inputs:
    """Inputs for an ad-hoc shape with the same recipe (used by tests)."""
    return generate(Workload(name, tuple(int(x) for x in lengths), hq, hkv, d, dtype, block_size,
                             topk, seed))


def ramped(inp: Inputs, q_scale: float, k_lo: float, k_hi: float) -> Inputs:
    """A copy of `inp` with the queries multiplied by q_scale and each key row
    by a factor that grows linearly from k_lo to k_hi across its block (local
    position / block size). Later keys of a block then score ever higher, so
    the running maximum of an online softmax keeps moving inside a block.
    Values are rounded back to the workload's dtype."""
    w = inp.workload
    bf16 = w.dtype == "bf16"

    def f32(x):
        return bf16_bits_to_f32(x) if bf16 else np.asarray(x, dtype=np.float32)

    def back(x):
        return f32_to_bf16_bits(x) if bf16 else x.astype(np.float32)

    pos = np.concatenate([np.arange(n) % w.block_size for n in w.lengths]).astype(np.float32)
    fac = np.float32(k_lo) + np.float32(k_hi - k_lo) * pos / np.float32(w.block_size)
    q = back(f32(inp.q) * np.float32(q_scale))
    k = back(f32(inp.k) * fac[:, None, None])
    return Inputs(w, q, k, inp.v.copy(), inp.cu_seqlens)
