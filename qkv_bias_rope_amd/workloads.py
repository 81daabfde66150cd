"""Seeded synthetic workloads for the attention-input epilogue.

This module only draws random inputs and names workload shapes; it holds none
of the epilogue's arithmetic.  The tests feed the same arrays to the CPU oracle
and to the HIP library, and the benchmark draws its inputs here too.

Shapes are the attention geometry of the Qwen2.5-class models the page
"73 · D3-8 — G4 FusedQKV ported to CUDA" measures on (§1-§2: 14B has 40 query
heads and 8 kv heads of 128, so q is 5120 wide and k/v 1024; 7B has 3584 and
512), plus the 0.5B geometry of "07 · The allocator" §2.5 (2 kv heads of 64).
Values: q/k/v standard normal, biases normal with standard deviation 0.1,
drawn as float32 from numpy's PCG64 (``default_rng``).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

CACHE_F32 = 0
CACHE_F16 = 1
THETA = 1.0e6


@dataclass(frozen=True)
class Workload:
    name: str
    n_head: int
    n_kv_head: int
    head_dim: int
    nt: int                 # tokens per launch
    n_ctx: int              # positions per cache slot
    n_slots: int            # cache slots (sequences)
    layers: int             # launches per step (one per layer)
    seed: int
    cache_dtypes: tuple = (CACHE_F16,)
    theta: float = THETA
    notes: str = ""
    pos_mode: str = "uniform"   # "fixed", "uniform", "arange"
    fixed_pos: int = 0
    concat_even_layers: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def nqt(self) -> int:
        return self.n_head * self.head_dim

    @property
    def nkt(self) -> int:
        return self.n_kv_head * self.head_dim


TINY_DECODE = Workload(
    "tiny_decode_0.5b", 14, 2, 64, nt=1, n_ctx=32, n_slots=1, layers=1, seed=0,
    cache_dtypes=(CACHE_F32,), pos_mode="fixed", fixed_pos=5,
    notes="one token at position 5, f32 cache of 32 positions")
DECODE_7B = Workload(
    "decode_7b", 28, 4, 128, nt=1, n_ctx=4096, n_slots=1, layers=28, seed=1,
    notes="one token per step, 28 layers, f16 cache of 4096 positions per layer")
DECODE_14B = Workload(
    "decode_14b", 40, 8, 128, nt=1, n_ctx=4096, n_slots=1, layers=48, seed=2,
    concat_even_layers=True,
    notes="one token per step, 48 layers; even layers read one concat q|k|v row, "
          "odd layers three separate buffers")
PREFILL_14B = Workload(
    "prefill_14b_4096", 40, 8, 128, nt=4096, n_ctx=4096, n_slots=1, layers=1, seed=3,
    pos_mode="arange", notes="4096 tokens at positions 0..4095 of one sequence")
BATCHED_DECODE_14B = Workload(
    "batched_decode_14b_256seq", 40, 8, 128, nt=256, n_ctx=32768, n_slots=256, layers=1,
    seed=4, cache_dtypes=(CACHE_F16, CACHE_F32),
    notes="256 sequences, one token each, slot s for sequence s, "
          "position uniform in [0, 32767]")

ALL = (TINY_DECODE, DECODE_7B, DECODE_14B, PREFILL_14B, BATCHED_DECODE_14B)
BY_NAME = {w.name: w for w in ALL}


def layer_stream(w: Workload, layer: int = 0) -> np.random.Generator:
    """The random stream of one layer: seed*1000 + layer."""
    return np.random.default_rng(w.seed * 1000 + layer)


def draw_layer(w: Workload, layer: int = 0, nt: int | None = None) -> dict:
    """Inputs of one launch: q [nt][nqt], k/v [nt][nkt], biases, pos, slot.

    Returns float32/int32 numpy arrays; ``slot`` is None for a one-sequence
    workload.  ``nt`` overrides the token count (for scaled-down cases).
    """
    nt = w.nt if nt is None else nt
    rng = layer_stream(w, layer)
    q = rng.standard_normal((nt, w.nqt), dtype=np.float32)
    k = rng.standard_normal((nt, w.nkt), dtype=np.float32)
    v = rng.standard_normal((nt, w.nkt), dtype=np.float32)
    bq = rng.standard_normal(w.nqt, dtype=np.float32) * np.float32(0.1)
    bk = rng.standard_normal(w.nkt, dtype=np.float32) * np.float32(0.1)
    bv = rng.standard_normal(w.nkt, dtype=np.float32) * np.float32(0.1)
    if w.pos_mode == "fixed":
        pos = np.full(nt, w.fixed_pos, dtype=np.int32)
    elif w.pos_mode == "arange":
        pos = np.arange(nt, dtype=np.int32) % np.int32(w.n_ctx)
    else:
        pos = rng.integers(0, w.n_ctx, size=nt, dtype=np.int32)
    slot = None
    if w.n_slots > 1:
        slot = (np.arange(nt, dtype=np.int32) % np.int32(w.n_slots)).astype(np.int32)
    return dict(q=q, k=k, v=v, bq=bq, bk=bk, bv=bv, pos=pos, slot=slot)


def draw_norm_weights(w: Workload, layer: int = 0) -> dict:
    """Per-head q/k norm weights of one layer ([head_dim] each), drawn as
    1 + 0.1*N(0,1) in float32 from the stream seed*1000 + 500 + layer."""
    rng = np.random.default_rng(w.seed * 1000 + 500 + layer)
    wq = (np.float32(1.0) + rng.standard_normal(w.head_dim, dtype=np.float32) * np.float32(0.1))
    wk = (np.float32(1.0) + rng.standard_normal(w.head_dim, dtype=np.float32) * np.float32(0.1))
    return dict(wq=wq.astype(np.float32), wk=wk.astype(np.float32))


QK_NORM_EPS = 1.0e-6


def step_positions(w: Workload, steps: int) -> np.ndarray:
    """Decode positions for `steps` steps (one position per step, shared by all
    layers of that step), uniform in [0, n_ctx)."""
    rng = np.random.default_rng(w.seed * 1000 + 999)
    return rng.integers(0, w.n_ctx, size=steps, dtype=np.int32)


def concat_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Pack per-token rows into one [nt][nqt + 2*nkt] q|k|v buffer."""
    return np.ascontiguousarray(np.concatenate([q, k, v], axis=1))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) and return the
    uint16 bit patterns (input generation only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def draw_projection(w: Workload, hidden: int, layer: int = 0, nt: int | None = None) -> dict:
    """Inputs of the projection-fed epilogue: bfloat16 activations x [nt][hidden]
    ~ N(0,1) and concat weight rows w [nqt+2*nkt][hidden] ~ N(0, 1/hidden) (so
    the projected q/k/v are about N(0,1)), plus the epilogue's biases/positions
    from draw_layer.  Stream seed*1000 + 700 + layer."""
    nt = w.nt if nt is None else nt
    rng = np.random.default_rng(w.seed * 1000 + 700 + layer)
    x = bf16_bits(rng.standard_normal((nt, hidden), dtype=np.float32))
    wt = bf16_bits(rng.standard_normal((w.nqt + 2 * w.nkt, hidden), dtype=np.float32)
                   * np.float32(1.0 / np.sqrt(hidden)))
    d = draw_layer(w, layer, nt=nt)
    return dict(x=x, w=wt, bq=d["bq"], bk=d["bk"], bv=d["bv"], pos=d["pos"], slot=d["slot"])


def draw_e4m3_weights(n_out: int, hidden: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Synthetic 8-bit float weights for the projection: OCP E4M3 codes
    (uint8 [n_out][hidden]) and f32 row scales [n_out].  Codes are drawn
    directly, never rounded from real values: both signs, the exponent field
    uniform over 1..11 (magnitudes 2^-6 .. 30) with the mantissa uniform, and
    one code in 32 from the zero/subnormal patterns; scales log-uniform in
    [2^-9, 2^-6].  Stream seed*1000 + 800."""
    rng = np.random.default_rng(seed * 1000 + 800)
    shape = (n_out, hidden)
    code = rng.integers(8, 96, shape)                       # exponent field 1..11
    sub = rng.integers(0, 32, shape) == 0
    code = np.where(sub, rng.integers(0, 8, shape), code)   # exponent field 0
    code = code | (rng.integers(0, 2, shape) << 7)
    scale = np.exp2(rng.uniform(-9.0, -6.0, n_out)).astype(np.float32)
    return code.astype(np.uint8), scale


HIDDEN = {"decode_7b": 3584, "decode_14b": 5120, "prefill_14b_4096": 5120,
          "batched_decode_14b_256seq": 5120, "tiny_decode_0.5b": 896}
