"""Seeded synthetic inputs and token packings for the PACK3D operator.

This module is shared by the fp64 oracle (``oracle/``), the tests and the
bench.  It holds none of the operator's arithmetic: only random draws, the
rounding of those draws to bf16 values, the bijections between lattice cells
and packed sequence positions, and the generation of normalised summary
weights, which are an *input* of the operator ("Geometry Matters in Packed 3D
Attention", papernotes.org notes, key design 2: the weights are a normalised
weighted average whose production the pages do not describe).

Recipe (stated once, used everywhere):

* Values are drawn per lattice cell in raster order with
  ``numpy.random.default_rng(seed)`` (PCG64), in the order
  Q, K_loc, V_loc, K_cmp, V_cmp, summary scores, gate logits; all N(0, 1)
  float32.  For bf16 workloads Q/K/V are rounded to bf16 (round to nearest
  even) and kept as float32 arrays holding bf16-representable values.
* Summary weights ``a`` are either uniform ``1/v`` or the softmax, inside each
  block and per KV group, of the drawn scores (computed in float64, stored
  float32).
* Gate logits stay float32 ``[N, 2]``.
* The arrays are then permuted from raster order into the requested packing;
  ``coords[i]`` is the lattice cell of packed position ``i`` and
  ``cell_to_pos[raster cell] = i`` its inverse.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

PACKINGS = ("raster", "morton", "block", "block_morton", "random")


# ----------------------------------------------------------------------------
# lattice and packings ("Geometry Matters in Packed 3D Attention", ai.info
# summary, Methodology in Plain English: a packing is a bijection from sequence
# positions to lattice cells; the named layouts are raster, Morton,
# block-contiguous (raster_block) and random)
# ----------------------------------------------------------------------------

def lattice_cells(grid: Sequence[int]) -> np.ndarray:
    """All cells of a Z x Y x X lattice as int64 ``[N, 3]`` (z, y, x), raster order."""
    z, y, x = np.meshgrid(np.arange(grid[0]), np.arange(grid[1]), np.arange(grid[2]),
                          indexing="ij")
    return np.stack([z.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.int64)


def _morton_key(cells: np.ndarray) -> np.ndarray:
    """Bit interleave: x bit b -> 3b, y bit b -> 3b+1, z bit b -> 3b+2."""
    key = np.zeros(len(cells), dtype=np.uint64)
    for b in range(21):
        for axis, off in ((2, 0), (1, 1), (0, 2)):
            bit = (cells[:, axis].astype(np.uint64) >> np.uint64(b)) & np.uint64(1)
            key |= bit << np.uint64(3 * b + off)
    return key


def packing_order(grid: Sequence[int], kind: str, seed: int = 0,
                  block: Sequence[int] = (1, 4, 4)) -> np.ndarray:
    """Raster cell index stored at each packed position (int64 ``[N]``).

    * ``raster``: identity.
    * ``morton``: stable sort of the cells by their Morton key.
    * ``block``: block-contiguous (raster_block): blocks of shape ``block`` in
      raster order, raster order inside each block.
    * ``block_morton``: the two-level layout: blocks of shape ``block`` in
      Morton order of their block indices, raster order inside each block.
    * ``random``: ``default_rng(seed + 100).permutation(N)``.
    """
    n = int(np.prod(grid))
    cells = lattice_cells(grid)
    if kind == "raster":
        return np.arange(n, dtype=np.int64)
    if kind == "morton":
        return np.argsort(_morton_key(cells), kind="stable").astype(np.int64)
    if kind == "block":
        bz, by, bx = block
        nby, nbx = -(-grid[1] // by), -(-grid[2] // bx)
        bid = ((cells[:, 0] // bz) * nby + cells[:, 1] // by) * nbx + cells[:, 2] // bx
        inner = ((cells[:, 0] % bz) * by + cells[:, 1] % by) * bx + cells[:, 2] % bx
        return np.lexsort((inner, bid)).astype(np.int64)
    if kind == "block_morton":
        bz, by, bx = block
        bidx = np.stack([cells[:, 0] // bz, cells[:, 1] // by, cells[:, 2] // bx], axis=1)
        inner = ((cells[:, 0] % bz) * by + cells[:, 1] % by) * bx + cells[:, 2] % bx
        return np.lexsort((inner, _morton_key(bidx))).astype(np.int64)
    if kind == "random":
        return np.random.default_rng(seed + 100).permutation(n).astype(np.int64)
    raise ValueError(f"unknown packing {kind!r}")


def packing(grid: Sequence[int], kind: str, seed: int = 0,
            block: Sequence[int] = (1, 4, 4)):
    """Return ``(order, coords int32 [N,3], cell_to_pos int32 [N])`` for a packing."""
    order = packing_order(grid, kind, seed, block)
    cells = lattice_cells(grid)
    coords = cells[order].astype(np.int32)
    cell_to_pos = np.empty(len(order), dtype=np.int32)
    cell_to_pos[order] = np.arange(len(order), dtype=np.int32)
    return order, coords, cell_to_pos


# ----------------------------------------------------------------------------
# value draws
# ----------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    Works in chunks of 2^24 values, so multi-gigabyte tensors need no more
    than one extra chunk of scratch memory.  Finite inputs: the 32-bit
    carry of the rounding increment can only wrap for NaN bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    src, dst = x.reshape(-1).view(np.uint32), out.reshape(-1).view(np.uint32)
    step = 1 << 24
    for i in range(0, src.size, step):
        u = src[i:i + step]
        r = dst[i:i + step]
        np.right_shift(u, np.uint32(16), out=r)
        np.bitwise_and(r, np.uint32(1), out=r)
        r += u
        r += np.uint32(0x7FFF)
        r &= np.uint32(0xFFFF0000)
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and recipe of one synthetic workload."""
    name: str
    grid: tuple
    packing: str
    n_q_heads: int
    n_kv_heads: int
    window: tuple
    block: tuple
    dtype: str            # "f32" or "bf16"
    weights: str          # "uniform" or "softmax"
    seed: int
    head_dim: int = 64
    rope_pairs: tuple = (11, 11, 10)
    rope_base: float = 10000.0
    summary_mode: str = "token"   # "token", "centre" or "blind" (compressed-branch variant)

    @property
    def n_tokens(self) -> int:
        return int(np.prod(self.grid))

    @property
    def n_blocks(self) -> int:
        return self.n_tokens // int(np.prod(self.block))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads of the PACK3D forward, with the pages' shapes: d_h = 64 with an
# 11/11/10 rotary split and base 10 000, 1x4x4 blocks, two KV groups at 262 144
# tokens (papernotes.org notes, key designs 1-3; onedev.kr summary on the two KV
# groups).
WORKLOADS = {
    "tiny_f32_4x16x16": Workload("tiny_f32_4x16x16", (4, 16, 16), "raster", 2, 1,
                                 (3, 5, 5), (1, 4, 4), "f32", "uniform", 1),
    "morton_bf16_16x64x64": Workload("morton_bf16_16x64x64", (16, 64, 64), "morton", 8, 2,
                                     (3, 7, 7), (1, 4, 4), "bf16", "softmax", 2),
    "block_bf16_64x64x64": Workload("block_bf16_64x64x64", (64, 64, 64), "block", 8, 2,
                                    (3, 7, 7), (1, 4, 4), "bf16", "softmax", 3),
    # reach: 4M and 8M tokens (the pages' query-tiled systems-reach sizes)
    "reach_bf16_64x256x256": Workload("reach_bf16_64x256x256", (64, 256, 256), "block", 8, 2,
                                      (3, 7, 7), (1, 4, 4), "bf16", "softmax", 6),
    "reach_bf16_128x256x256": Workload("reach_bf16_128x256x256", (128, 256, 256), "block", 8,
                                       2, (3, 7, 7), (1, 4, 4), "bf16", "softmax", 7),
    "random_bf16_64x128x128": Workload("random_bf16_64x128x128", (64, 128, 128), "random", 8, 2,
                                       (3, 7, 7), (1, 4, 4), "bf16", "softmax", 4),
}


def block_softmax_weights(scores: np.ndarray, grid: Sequence[int],
                          block: Sequence[int]) -> np.ndarray:
    """Normalised summary weights from raster-order scores ``[N, Hkv]``.

    Softmax over the cells of each block, separately for every KV group, in
    float64; returned as float32.
    """
    z, y, x = grid
    bz, by, bx = block
    s = scores.astype(np.float64).reshape(z // bz, bz, y // by, by, x // bx, bx, -1)
    s = s - s.max(axis=(1, 3, 5), keepdims=True)
    e = np.exp(s)
    w = e / e.sum(axis=(1, 3, 5), keepdims=True)
    return w.reshape(z * y * x, -1).astype(np.float32)


@dataclasses.dataclass
class Inputs:
    """One workload's inputs, already in packed order (float32 host arrays)."""
    workload: Workload
    order: np.ndarray        # int64 [N]: raster cell at each packed position
    coords: np.ndarray       # int32 [N, 3]
    cell_to_pos: np.ndarray  # int32 [N]
    q: np.ndarray            # [N, Hq, D]
    k_loc: np.ndarray        # [N, Hkv, D]
    v_loc: np.ndarray
    k_cmp: np.ndarray
    v_cmp: np.ndarray
    a: Optional[np.ndarray]  # [N, Hkv] or None for uniform 1/v
    gate: np.ndarray         # [N, 2]

    def repacked(self, kind: str, seed: Optional[int] = None) -> "Inputs":
        """The same per-cell values under another packing."""
        w = self.workload
        order, coords, c2p = packing(w.grid, kind, w.seed if seed is None else seed, w.block)
        # position of each cell in self -> value of cell at new position
        src = self.cell_to_pos[order]
        take = lambda t: None if t is None else np.ascontiguousarray(t[src])
        return Inputs(w.with_(packing=kind), order, coords, c2p, take(self.q),
                      take(self.k_loc), take(self.v_loc), take(self.k_cmp),
                      take(self.v_cmp), take(self.a), take(self.gate))


def make_inputs(w: Workload, explicit_uniform: bool = False, progress=None) -> Inputs:
    """Draw a workload's inputs (see the module docstring for the recipe).

    With ``weights == "uniform"`` the weights are ``None`` (the operator's
    uniform ``1/v`` default) unless ``explicit_uniform`` asks for the array.
    ``progress`` (optional callable) is told after each tensor is drawn.
    """
    n, hq, hkv, d = w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim
    rng = np.random.default_rng(w.seed)
    say = progress or (lambda *a: None)

    def draw(*shape):
        t = rng.standard_normal(shape, dtype=np.float32)
        t = round_to_bf16(t) if w.dtype == "bf16" else t
        say(f"  drew {shape}")
        return t

    q = draw(n, hq, d)
    k_loc = draw(n, hkv, d)
    v_loc = draw(n, hkv, d)
    k_cmp = draw(n, hkv, d)
    v_cmp = draw(n, hkv, d)
    scores = rng.standard_normal((n, hkv), dtype=np.float32)
    gate = rng.standard_normal((n, 2), dtype=np.float32)
    if w.weights == "softmax":
        a = block_softmax_weights(scores, w.grid, w.block)
    elif explicit_uniform:
        a = np.full((n, hkv), 1.0 / np.prod(w.block), dtype=np.float32)
    else:
        a = None
    order, coords, c2p = packing(w.grid, w.packing, w.seed, w.block)
    take = lambda t: None if t is None else np.ascontiguousarray(t[order])
    q = take(q)
    say("  packed q")
    return Inputs(w, order, coords, c2p, q, take(k_loc), take(v_loc), take(k_cmp),
                  take(v_cmp), take(a), take(gate))


def make_upstream_grad(inp: Inputs, seed_offset: int = 200) -> np.ndarray:
    """Upstream gradient of the output, ``[N, Hq, D]`` ~ N(0, 1), drawn per
    lattice cell in raster order from ``default_rng(seed + seed_offset)`` and
    then placed in the inputs' packing (bf16-rounded for bf16 workloads), so
    every packing of a workload carries the same per-cell gradient."""
    w = inp.workload
    rng = np.random.default_rng(w.seed + seed_offset)
    g = rng.standard_normal((w.n_tokens, w.n_q_heads, w.head_dim), dtype=np.float32)
    if w.dtype == "bf16":
        g = round_to_bf16(g)
    # inp.order[i] is the raster cell at packed position i
    return np.ascontiguousarray(g[inp.order])


@dataclasses.dataclass
class LayerInputs:
    """The layer around the operator: hidden states and weights (float32 host
    arrays; bf16-rounded for bf16 workloads except the LayerNorm affine)."""
    h: np.ndarray            # [N, C] in the operator inputs' packing
    gamma: np.ndarray        # [C] fp32
    beta: np.ndarray         # [C] fp32
    w_qkv: np.ndarray        # [Hq*D + 4*Hkv*D, C]
    w_o: np.ndarray          # [C, Hq*D]


def make_layer_inputs(inp: Inputs, width: Optional[int] = None,
                      seed_offset: int = 300) -> LayerInputs:
    """Hidden states h ~ N(0, 1) drawn per lattice cell in raster order and
    placed in ``inp``'s packing; gamma = 1 + 0.1 N(0, 1), beta = 0.1 N(0, 1);
    W_qkv ~ N(0, 1/C) (so the projections are ~N(0, 1) like the operator's
    own inputs) and W_O ~ N(0, 1/(Hq*D)), all from ``default_rng(seed +
    seed_offset)``.  The model width C defaults to Hq * D."""
    w = inp.workload
    c = width or w.n_q_heads * w.head_dim
    rng = np.random.default_rng(w.seed + seed_offset)
    rnd = (lambda t: round_to_bf16(t)) if w.dtype == "bf16" else (lambda t: t)
    h = rnd(rng.standard_normal((w.n_tokens, c), dtype=np.float32))
    gamma = (1.0 + 0.1 * rng.standard_normal(c)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(c)).astype(np.float32)
    cout = (w.n_q_heads + 4 * w.n_kv_heads) * w.head_dim
    w_qkv = rnd((rng.standard_normal((cout, c)) / np.sqrt(c)).astype(np.float32))
    w_o = rnd((rng.standard_normal((c, w.n_q_heads * w.head_dim))
               / np.sqrt(w.n_q_heads * w.head_dim)).astype(np.float32))
    return LayerInputs(np.ascontiguousarray(h[inp.order]), gamma, beta, w_qkv, w_o)
