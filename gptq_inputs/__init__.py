"""Seeded synthetic inputs for quantizing one linear layer.

This module is shared by the HIP path (tests, benchmark) and by the CPU oracle.
It only draws random numbers and casts them to the storage dtype; it contains
no step of the quantization method itself.

Workloads follow the pages' calibration shape (128 sequences x 2048 tokens,
the GPTQ practice page at m.lqnn.cn/news/117696, section 3.2) and Llama-shaped
linear layers.  Real calibration text (C4 / wikitext2) and trained weights are
replaced by the distributions below:

* W: i.i.d. normal with the stated standard deviation, cast to fp16 (fp32 for
  the small case).
* X: token-major [tokens, d_in]; normal or Student-t (location 0, scale 1),
  a fixed set of "outlier" channels multiplied by a factor, cast to bf16
  (fp32 for the small case) with round-to-nearest-even.
* Seeds: ``1000*config + 1`` (W), ``+2`` (up_proj), ``+3`` (down_proj),
  ``+99`` (outlier channel choice), ``+100+c`` (X chunk c).  X is produced in
  chunks of 16 sequences (32768 tokens); each chunk is split into fixed
  4096-token sub-streams (``SeedSequence.spawn``) drawn in parallel threads, so
  the bytes do not depend on the thread count.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field, replace
from typing import Dict, Iterator, List, Optional, Sequence, Tuple

import numpy as np

CHUNK_TOKENS = 32768          # 16 sequences of 2048 tokens
SUBSTREAM_TOKENS = 4096       # fixed split of a chunk into independent streams

# ----------------------------------------------------------------------------
# dtype helpers (storage encodings only)
# ----------------------------------------------------------------------------

DTYPES = ("f32", "f16", "bf16")


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the
    16-bit patterns as uint16.  Inputs are finite."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_float64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values (f32 / f16 / bf16 bit patterns) to float64."""
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    if dtype in ("f32", "f16"):
        return np.asarray(a).astype(np.float64)
    raise ValueError(dtype)


def cast_storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float32 draws to the storage dtype (round to nearest even)."""
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "f16":
        return a32.astype(np.float16)
    if dtype == "bf16":
        return bf16_from_f32(a32)
    raise ValueError(dtype)


def itemsize(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


# ----------------------------------------------------------------------------
# workload descriptions
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class CalibSpec:
    """Calibration activations X [seqs*seq_len, d_in], token-major."""
    seqs: int
    seq_len: int
    d_in: int
    dtype: str = "bf16"
    dist: str = "normal"            # "normal" | "t"
    nu: float = 4.0                 # Student-t degrees of freedom
    outlier_frac: float = 0.0
    outlier_factor: float = 1.0

    @property
    def n_tokens(self) -> int:
        return self.seqs * self.seq_len


@dataclass(frozen=True)
class LayerSpec:
    name: str
    d_out: int
    d_in: int
    dtype: str = "f16"
    std: float = 0.02
    seed_offset: int = 1            # 1: W, 2: up_proj, 3: down_proj


@dataclass(frozen=True)
class QuantSpec:
    bits: int = 4
    group_size: int = 128
    block_size: int = 128
    damp_percent: float = 0.01
    desc_act: int = 0
    sym: int = 0


@dataclass(frozen=True)
class Workload:
    key: str
    config: int
    description: str
    layers: Tuple[LayerSpec, ...]
    calib: Tuple[CalibSpec, ...]          # one per distinct d_in
    quant: Tuple[QuantSpec, ...]

    def calib_for(self, d_in: int) -> CalibSpec:
        for c in self.calib:
            if c.d_in == d_in:
                return c
        raise KeyError(d_in)


def _q(**kw) -> QuantSpec:
    return QuantSpec(**kw)


WORKLOADS: Dict[str, Workload] = {
    "c1_tiny_256": Workload(
        "c1_tiny_256", 0,
        "W[256x256] fp32 N(0,0.02); X 16x128 tokens fp32 N(0,1), 1% channels x20; "
        "4-bit asym g128 b128 damp 0.01",
        (LayerSpec("linear", 256, 256, "f32", 0.02, 1),),
        (CalibSpec(16, 128, 256, "f32", "normal", 0.0, 0.01, 20.0),),
        (_q(bits=4, group_size=128),),
    ),
    "c2_llama7b_q_proj": Workload(
        "c2_llama7b_q_proj", 1,
        "Llama-7B q_proj W[4096x4096] fp16 N(0,0.02); X 128x2048 tokens x 4096 bf16 "
        "Student-t(4), 0.5% channels x30; 4-bit asym g128 b128 damp 0.01",
        (LayerSpec("q_proj", 4096, 4096, "f16", 0.02, 1),),
        (CalibSpec(128, 2048, 4096, "bf16", "t", 4.0, 0.005, 30.0),),
        (_q(bits=4, group_size=128),),
    ),
    "c3_llama7b_mlp": Workload(
        "c3_llama7b_mlp", 2,
        "Llama-7B MLP: gate/up W[11008x4096] sharing one H, down W[4096x11008]; fp16 "
        "N(0,0.02); X 128x2048 tokens bf16 Student-t(4); 4-bit asym g128",
        (LayerSpec("gate_proj", 11008, 4096, "f16", 0.02, 1),
         LayerSpec("up_proj", 11008, 4096, "f16", 0.02, 2),
         LayerSpec("down_proj", 4096, 11008, "f16", 0.02, 3)),
        (CalibSpec(128, 2048, 4096, "bf16", "t", 4.0),
         CalibSpec(128, 2048, 11008, "bf16", "t", 4.0)),
        (_q(bits=4, group_size=128),),
    ),
    "c4_13b_desc_act": Workload(
        "c4_13b_desc_act", 3,
        "13B-shaped W[5120x5120] and down W[5120x13824] fp16 N(0,0.02); X 128x2048 "
        "tokens bf16 N(0,1), 1% channels x20; desc_act; {3,4}-bit x g{64,128}",
        (LayerSpec("o_proj", 5120, 5120, "f16", 0.02, 1),
         LayerSpec("down_proj", 5120, 13824, "f16", 0.02, 3)),
        (CalibSpec(128, 2048, 5120, "bf16", "normal", 0.0, 0.01, 20.0),
         CalibSpec(128, 2048, 13824, "bf16", "normal", 0.0, 0.01, 20.0)),
        (_q(bits=3, group_size=64, desc_act=1), _q(bits=3, group_size=128, desc_act=1),
         _q(bits=4, group_size=64, desc_act=1), _q(bits=4, group_size=128, desc_act=1)),
    ),
    "c5_70b_down_proj": Workload(
        "c5_70b_down_proj", 4,
        "70B down_proj W[8192x28672] fp16 N(0,0.015); X 128x2048 tokens x 28672 bf16 "
        "Student-t(3); 4-bit asym g128 b128 damp 0.01 desc_act",
        (LayerSpec("down_proj", 8192, 28672, "f16", 0.015, 3),),
        (CalibSpec(128, 2048, 28672, "bf16", "t", 3.0),),
        (_q(bits=4, group_size=128, desc_act=1),),
    ),
}


def workload(key: str) -> Workload:
    return WORKLOADS[key]


# ----------------------------------------------------------------------------
# drawing
# ----------------------------------------------------------------------------

def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw(gen: np.random.Generator, shape, dist: str, nu: float) -> np.ndarray:
    """float32 draws: standard normal, or Student-t(nu) built as Z / sqrt(2G/nu)
    with G ~ Gamma(nu/2, 1) (so 2G is chi-square with nu degrees of freedom)."""
    z = gen.standard_normal(shape, dtype=np.float32)
    if dist == "normal":
        return z
    if dist == "t":
        g = gen.standard_gamma(np.float32(nu / 2.0), shape, dtype=np.float32)
        g *= np.float32(2.0 / nu)
        np.sqrt(g, out=g)
        z /= g
        return z
    raise ValueError(dist)


def weight(layer: LayerSpec, config: int) -> np.ndarray:
    """W [d_out, d_in] in its storage dtype (float32 or float16)."""
    gen = np.random.Generator(np.random.PCG64(1000 * config + layer.seed_offset))
    w = gen.standard_normal((layer.d_out, layer.d_in), dtype=np.float32)
    w *= np.float32(layer.std)
    return cast_storage(w, layer.dtype)


def outlier_channels(calib: CalibSpec, config: int) -> np.ndarray:
    if calib.outlier_frac <= 0.0:
        return np.zeros(0, dtype=np.int64)
    k = max(1, int(round(calib.outlier_frac * calib.d_in)))
    gen = np.random.Generator(np.random.PCG64(1000 * config + 99))
    return np.sort(gen.choice(calib.d_in, size=k, replace=False))


def n_chunks(calib: CalibSpec) -> int:
    return (calib.n_tokens + CHUNK_TOKENS - 1) // CHUNK_TOKENS


def chunk_rows(calib: CalibSpec, c: int) -> int:
    return min(CHUNK_TOKENS, calib.n_tokens - c * CHUNK_TOKENS)


def x_chunk(calib: CalibSpec, config: int, c: int,
            out: Optional[np.ndarray] = None) -> np.ndarray:
    """Chunk c of X: [rows, d_in] in storage dtype (uint16 bit patterns for bf16)."""
    rows = chunk_rows(calib, c)
    cols = outlier_channels(calib, config)
    ss = np.random.SeedSequence(1000 * config + 100 + c)
    nsub = (rows + SUBSTREAM_TOKENS - 1) // SUBSTREAM_TOKENS
    subs = ss.spawn(nsub)
    np_dtype = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[calib.dtype]
    if out is None:
        out = np.empty((rows, calib.d_in), dtype=np_dtype)
    assert out.shape == (rows, calib.d_in) and out.dtype == np_dtype

    def one(k: int) -> None:
        r0 = k * SUBSTREAM_TOKENS
        r1 = min(rows, r0 + SUBSTREAM_TOKENS)
        gen = np.random.Generator(np.random.PCG64(subs[k]))
        a = _draw(gen, (r1 - r0, calib.d_in), calib.dist, calib.nu)
        if cols.size:
            a[:, cols] *= np.float32(calib.outlier_factor)
        out[r0:r1] = cast_storage(a, calib.dtype)

    if nsub == 1:
        one(0)
    else:
        with _cf.ThreadPoolExecutor(max_workers=min(_threads(), nsub)) as ex:
            list(ex.map(one, range(nsub)))
    return out


def x_chunks(calib: CalibSpec, config: int) -> Iterator[np.ndarray]:
    for c in range(n_chunks(calib)):
        yield x_chunk(calib, config, c)


def x_full(calib: CalibSpec, config: int) -> np.ndarray:
    """All of X [n_tokens, d_in] in storage dtype (only for small workloads)."""
    np_dtype = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[calib.dtype]
    out = np.empty((calib.n_tokens, calib.d_in), dtype=np_dtype)
    for c in range(n_chunks(calib)):
        r0 = c * CHUNK_TOKENS
        x_chunk(calib, config, c, out=out[r0:r0 + chunk_rows(calib, c)])
    return out


# ----------------------------------------------------------------------------
# small random cases for tests
# ----------------------------------------------------------------------------

@dataclass
class Case:
    """A small self-contained layer: W [d_out, d_in] and X [n_tokens, d_in]."""
    W: np.ndarray
    X: np.ndarray
    w_dtype: str
    x_dtype: str
    seed: int
    meta: dict = field(default_factory=dict)


def random_case(d_out: int, d_in: int, n_tokens: int, seed: int, *,
                w_dtype: str = "f32", x_dtype: str = "f32", dist: str = "normal",
                nu: float = 4.0, w_std: float = 0.02, outlier_frac: float = 0.0,
                outlier_factor: float = 1.0, correlated_rank: int = 0,
                noise: float = 0.1) -> Case:
    """A seeded small layer.  With correlated_rank r > 0, X = Z A + noise*E with
    Z [n, r], A [r, d_in] (strongly correlated input channels)."""
    gen = np.random.Generator(np.random.PCG64(seed))
    w = gen.standard_normal((d_out, d_in), dtype=np.float32) * np.float32(w_std)
    if correlated_rank > 0:
        z = _draw(gen, (n_tokens, correlated_rank), dist, nu)
        a = gen.standard_normal((correlated_rank, d_in), dtype=np.float32)
        e = gen.standard_normal((n_tokens, d_in), dtype=np.float32)
        x = (z @ a).astype(np.float32) + np.float32(noise) * e
    else:
        x = _draw(gen, (n_tokens, d_in), dist, nu)
    if outlier_frac > 0.0:
        k = max(1, int(round(outlier_frac * d_in)))
        cols = gen.choice(d_in, size=k, replace=False)
        x[:, cols] *= np.float32(outlier_factor)
    return Case(cast_storage(w, w_dtype), cast_storage(x, x_dtype), w_dtype, x_dtype, seed,
                dict(d_out=d_out, d_in=d_in, n_tokens=n_tokens, dist=dist))


__all__ = [
    "CHUNK_TOKENS", "SUBSTREAM_TOKENS", "DTYPES", "bf16_from_f32", "bf16_to_f32", "to_float64",
    "cast_storage", "itemsize", "CalibSpec", "LayerSpec", "QuantSpec", "Workload", "WORKLOADS",
    "workload", "weight", "outlier_channels", "n_chunks", "chunk_rows", "x_chunk", "x_chunks",
    "x_full", "Case", "random_case", "replace",
]
