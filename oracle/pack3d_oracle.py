"""fp64 CPU oracle of the PACK3D local-global attention forward and backward.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously correct
statement of what the operator computes.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or call it.  The product path (``libpack3d`` and its Python binding) never
does, and the two share no code: the only common module is ``synthgen``,
which draws seeded inputs and holds none of the operator's arithmetic.

Source: "Geometry Matters in Packed 3D Attention" (arXiv 2610.38694), as
described on the papernotes.org notes page (method section, key designs 1-3
and the flowchart) and restated on the ai.info summary page ("Methodology in
Plain English").  Every function below cites the passage it follows.

Everything is evaluated in float64 with numpy; inputs that were bf16 values
are taken exactly (their float32 carriers upcast).

Readings taken where the pages leave a step open (each is a parameter or a
single constant; the full list with reasons is kept with the design notes):

* frequencies: omega_{a,r} = base ** (-r / m_a) for r = 0..m_a-1 on each axis
  a in (z, y, x); the pages fix only base 10 000 and m = (11, 11, 10).
  PARITY UNPINNED for this choice: every identity the pages state holds for
  any frequencies, so no pin below can tell two frequency rules apart.
* pairs: rotation pair p acts on dims (2p, 2p+1), z pairs first, then y,
  then x, as the block-diagonal direct sum is printed; dims past 2*sum(m)
  are left alone (the identity block).
* sign: each 2x2 block is [[cos, -sin], [sin, cos]] applied as R(c) x.
* coordinates: integer lattice indices (z, y, x), origin 0.
* softmax scale tau = 1/sqrt(d_h) in both branches unless given.
* window: per-axis box |dz|<=wz//2, |dy|<=wy//2, |dx|<=wx//2, clipped at the
  lattice faces, the query itself included.
* summaries: aligned blocks, block index in block-raster order; every query
  attends to all M summaries (its own block included); weights a are given
  per token and KV group, uniform 1/v when absent.
* KV groups: query head h reads KV group h // (Hq / Hkv).
* gate: one 2-way softmax per token (index 0 = local, 1 = compressed), or
  one per token and head when logits are [N, Hq, 2].
* summary variants (the notes' key design 2 and the summary's contributions:
  a cheaper summary-centre placement of the rotation, and a coordinate-blind
  compressed branch named as the missing control):
  "token"  (default) every cell's key is rotated by R(c_u) before the
           weighted sum - the exact form;
  "centre" the weighted sum of the UNROTATED keys is rotated once by
           R(c^_j), c^_j the geometric centre of the aligned block
           (origin + (b - 1) / 2 per axis, a half-integer for even extents);
  "blind"  no rotation on either side of the compressed branch: unrotated
           keys are pooled and the branch's logits use the unrotated query.
  Values are pooled the same way in all three; the local branch is
  unchanged.
* the layer around the operator (notes, flowchart nodes B and G, and key
  design 1's q = R(c) W_Q LN(h), k^b = R(c) W_K^b LN(h), v^b = W_V^b LN(h)):
  pre-norm LayerNorm over the model width with learned scale and shift and
  eps = 1e-5 (biased variance); the five projections are bias-free and
  stacked in one weight [Hq*D + 4*Hkv*D, C] in the order Q, K_loc, V_loc,
  K_cmp, V_cmp; the block returns h + O W_O^T with a bias-free W_O
  [C, Hq*D] applied to the heads' gated outputs concatenated (the
  feed-forward network after it is not part of the operator).
* backward: the pages print no backward; the gradients below are the exact
  derivatives of the forward above (chain rule through the gate, the two
  softmax attentions, the block sums and the rotations) for an upstream
  gradient of the output.  The weights ``a`` are treated as given (no
  gradient is returned for them).
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "axial_frequencies", "rotation_matrix", "rotate", "block_index",
    "block_summaries", "local_attention", "global_attention", "gate_weights",
    "gate_mix", "forward", "local_window_sizes",
    "rotate_transpose", "local_attention_backward", "global_attention_backward",
    "block_summaries_backward", "gate_backward", "backward",
    "SUMMARY_MODES", "block_centres",
    "layer_norm", "qkv_projection", "layer_forward",
]

SUMMARY_MODES = ("token", "centre", "blind")


# ----------------------------------------------------------------------------
# Axial grid RoPE  (papernotes.org notes, key design 1, the equation for R(c))
# ----------------------------------------------------------------------------

def axial_frequencies(rope_pairs: Sequence[int] = (11, 11, 10),
                      base: float = 10000.0) -> list:
    """Per-axis rotary frequencies omega_{a,r} = base^(-r/m_a), r < m_a."""
    return [base ** (-np.arange(m, dtype=np.float64) / m) for m in rope_pairs]


def rotation_matrix(c: Sequence[int], head_dim: int = 64,
                    rope_pairs: Sequence[int] = (11, 11, 10),
                    base: float = 10000.0) -> np.ndarray:
    """The d_h x d_h matrix R(c): a direct sum over axes z, y, x and r < m_a of
    2x2 rotations by omega_{a,r} * c_a, followed by an identity block."""
    if 2 * sum(rope_pairs) > head_dim:
        raise ValueError("rotary pairs exceed the head dimension")
    omega = axial_frequencies(rope_pairs, base)
    R = np.eye(head_dim)
    p = 0
    for a, m in enumerate(rope_pairs):
        for r in range(m):
            th = omega[a][r] * float(c[a])
            R[2 * p:2 * p + 2, 2 * p:2 * p + 2] = [[math.cos(th), -math.sin(th)],
                                                   [math.sin(th), math.cos(th)]]
            p += 1
    return R


def rotate(x: np.ndarray, coords: np.ndarray,
           rope_pairs: Sequence[int] = (11, 11, 10),
           base: float = 10000.0) -> np.ndarray:
    """R(c_i) x_{i,h} for every token i and head h.

    ``x`` is ``[N, H, D]``; ``coords`` is integer ``[N, 3]`` (z, y, x).  The
    same 2x2 blocks as :func:`rotation_matrix`, applied pair by pair.
    """
    x = np.asarray(x, dtype=np.float64)
    y = x.copy()
    omega = axial_frequencies(rope_pairs, base)
    p = 0
    for a, m in enumerate(rope_pairs):
        ca = np.asarray(coords[:, a], dtype=np.float64)
        for r in range(m):
            th = omega[a][r] * ca
            cs, sn = np.cos(th)[:, None], np.sin(th)[:, None]
            x0, x1 = x[:, :, 2 * p], x[:, :, 2 * p + 1]
            y[:, :, 2 * p] = cs * x0 - sn * x1
            y[:, :, 2 * p + 1] = sn * x0 + cs * x1
            p += 1
    return y


# ----------------------------------------------------------------------------
# Rotate-before-compression block summaries (papernotes.org notes, key
# design 2, the equations for k~_j and v~_j; blocks are contiguous 3D boxes of
# volume v, M = N / v)
# ----------------------------------------------------------------------------

def block_index(coords: np.ndarray, grid: Sequence[int], block: Sequence[int]) -> np.ndarray:
    """Index j of the aligned block holding each cell, blocks in raster order."""
    nby, nbx = grid[1] // block[1], grid[2] // block[2]
    c = np.asarray(coords, dtype=np.int64)
    return ((c[:, 0] // block[0]) * nby + c[:, 1] // block[1]) * nbx + c[:, 2] // block[2]


def block_centres(grid: Sequence[int], block: Sequence[int]) -> np.ndarray:
    """Geometric centre (z, y, x) of every aligned block, block-raster order:
    the block's origin plus (b - 1) / 2 on each axis (the summary-centre
    variant rotates the pooled key there)."""
    nb = [g // b for g, b in zip(grid, block)]
    jz, jy, jx = np.meshgrid(*[np.arange(k) for k in nb], indexing="ij")
    idx = np.stack([jz.ravel(), jy.ravel(), jx.ravel()], axis=1).astype(np.float64)
    return idx * np.asarray(block, np.float64) + (np.asarray(block, np.float64) - 1.0) / 2.0


def block_summaries(k_cmp: np.ndarray, v_cmp: np.ndarray, a: Optional[np.ndarray],
                    coords: np.ndarray, grid: Sequence[int], block: Sequence[int],
                    rope_pairs: Sequence[int] = (11, 11, 10), base: float = 10000.0,
                    rope_coords: Optional[np.ndarray] = None, mode: str = "token"):
    """k~_j = sum_{u in B_j} a_u R(c_u) k_u and v~_j = sum_{u in B_j} a_u v_u.

    ``k_cmp``/``v_cmp`` are ``[N, Hkv, D]`` (K unrotated: the rotation happens
    here, before the weighted sum); ``a`` is ``[N, Hkv]`` or ``None`` for
    uniform ``1/v``.  ``rope_coords`` replaces the coordinates used by the
    rotation only (block membership still follows ``coords``).
    ``mode`` "centre" instead rotates sum_u a_u k_u once by R(c^_j) (the
    block's centre, :func:`block_centres`); "blind" leaves it unrotated.
    Returns ``(k_sum, v_sum)``, each ``[Hkv, M, D]`` float64.
    """
    if mode not in SUMMARY_MODES:
        raise ValueError(f"summary mode {mode!r}")
    grid, block = tuple(grid), tuple(block)
    if any(g % b for g, b in zip(grid, block)):
        raise ValueError("block must divide the grid")
    n, hkv, d = k_cmp.shape
    vol = int(np.prod(block))
    m = n // vol
    if mode == "token":
        kr = rotate(k_cmp, coords if rope_coords is None else rope_coords, rope_pairs, base)
    else:
        kr = np.asarray(k_cmp, np.float64)
    w = (np.full((n, hkv), 1.0 / vol) if a is None else np.asarray(a, dtype=np.float64))
    j = block_index(coords, grid, block)
    cell = (np.asarray(coords[:, 0], np.int64) * grid[1] + coords[:, 1]) * grid[2] + coords[:, 2]
    # group the members of each block together, raster order inside the block
    srt = np.lexsort((cell, j))
    wk = (w[:, :, None] * kr)[srt].reshape(m, vol, hkv, d).sum(axis=1)
    wv = (w[:, :, None] * np.asarray(v_cmp, np.float64))[srt].reshape(m, vol, hkv, d).sum(axis=1)
    if mode == "centre":
        wk = rotate(wk, block_centres(grid, block), rope_pairs, base)
    return np.ascontiguousarray(wk.transpose(1, 0, 2)), np.ascontiguousarray(wv.transpose(1, 0, 2))


# ----------------------------------------------------------------------------
# Exact local-neighbourhood attention (papernotes.org notes, key design 3: the
# neighbourhood N(i) is defined by lattice coordinates; ai.info summary,
# Methodology in Plain English, the first of the three contracts)
# ----------------------------------------------------------------------------

def _window_offsets(window: Sequence[int]):
    rz, ry, rx = (w // 2 for w in window)
    return [(dz, dy, dx) for dz in range(-rz, rz + 1) for dy in range(-ry, ry + 1)
            for dx in range(-rx, rx + 1)]


def local_window_sizes(coords: np.ndarray, grid: Sequence[int], window: Sequence[int]) -> np.ndarray:
    """|N(i)| for each token: the clipped box size."""
    c = np.asarray(coords, np.int64)
    size = np.ones(len(c), dtype=np.int64)
    for a in range(3):
        r = window[a] // 2
        lo = np.maximum(c[:, a] - r, 0)
        hi = np.minimum(c[:, a] + r, grid[a] - 1)
        size *= hi - lo + 1
    return size


def local_attention(q_rot: np.ndarray, k_rot: np.ndarray, v: np.ndarray,
                    coords: np.ndarray, grid: Sequence[int], window: Sequence[int],
                    scale: float, rows: Optional[np.ndarray] = None, chunk: int = 8192,
                    q_is_rows: bool = False):
    """o_loc[i,h] = sum_{u in N(i)} softmax_u(scale * <q_i,h, k_u,g>) v_u,g.

    Inputs are already rotated.  ``rows`` selects the query tokens computed
    (default: all); with ``q_is_rows`` the queries are given for those rows
    only.  Returns ``(o_loc [R, Hq, D], lse [R, Hq])`` where ``lse`` is the
    natural-log log-sum-exp of the scaled logits.
    """
    grid = tuple(int(g) for g in grid)
    if any(w % 2 == 0 for w in window):
        raise ValueError("window extents must be odd")
    n = k_rot.shape[0]
    hq, d = q_rot.shape[1:]
    hkv = k_rot.shape[1]
    grp = hq // hkv
    coords = np.asarray(coords, np.int64)
    lattice = np.full(grid, -1, dtype=np.int64)
    lattice[coords[:, 0], coords[:, 1], coords[:, 2]] = np.arange(n)
    offs = np.array(_window_offsets(window), dtype=np.int64)
    rows = np.arange(n) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((len(rows), hq, d))
    lse = np.zeros((len(rows), hq))
    gmax = np.array(grid, dtype=np.int64) - 1
    for s in range(0, len(rows), chunk):
        r = rows[s:s + chunk]
        nr = len(r)
        qsel = np.arange(s, s + nr) if q_is_rows else r
        qc = np.asarray(q_rot[qsel], np.float64).reshape(nr, hkv, grp, d)
        ci = coords[r]
        logit = np.full((nr, len(offs), hkv, grp), -np.inf)
        pos = np.zeros((nr, len(offs)), dtype=np.int64)
        valid = np.zeros((nr, len(offs)), dtype=bool)
        for t, off in enumerate(offs):
            cu = ci + off
            ok = np.all((cu >= 0) & (cu <= gmax), axis=1)
            cc = np.clip(cu, 0, gmax)
            pu = lattice[cc[:, 0], cc[:, 1], cc[:, 2]]
            ku = np.asarray(k_rot[pu], np.float64)               # [nr, hkv, d]
            lg = scale * np.einsum("nkgd,nkd->nkg", qc, ku)
            logit[:, t] = np.where(ok[:, None, None], lg, -np.inf)
            pos[:, t], valid[:, t] = pu, ok
        mx = logit.max(axis=1, keepdims=True)
        p = np.exp(logit - mx)
        l = p.sum(axis=1)                                         # [nr, hkv, grp]
        acc = np.zeros((nr, hkv, grp, d))
        for t in range(len(offs)):
            vu = np.asarray(v[pos[:, t]], np.float64) * valid[:, t, None, None]
            acc += p[:, t, :, :, None] * vu[:, :, None, :]
        out[s:s + nr] = (acc / l[..., None]).reshape(nr, hq, d)
        lse[s:s + nr] = (mx[:, 0] + np.log(l)).reshape(nr, hq)
    return out, lse


# ----------------------------------------------------------------------------
# Query -> all-summaries attention (papernotes.org notes, key design 3: each
# query attends to the M summaries with a softmax; ai.info summary,
# Methodology in Plain English, the second contract: all M summaries)
# ----------------------------------------------------------------------------

def global_attention(q_rot: np.ndarray, k_sum: np.ndarray, v_sum: np.ndarray,
                     scale: float, rows: Optional[np.ndarray] = None, q_is_rows: bool = False):
    """o_cmp[i,h] = sum_{j<M} softmax_j(scale * <q_i,h, k~_j,g>) v~_j,g.

    ``q_rot`` is ``[N, Hq, D]`` (or ``[R, Hq, D]`` with ``q_is_rows``);
    ``k_sum``/``v_sum`` are ``[Hkv, M, D]``.  Returns
    ``(o_cmp [R, Hq, D], lse [R, Hq])`` (natural-log log-sum-exp).
    """
    n, hq, d = q_rot.shape
    hkv, m, _ = k_sum.shape
    grp = hq // hkv
    if q_is_rows:
        q_rot, rows = q_rot, np.arange(n)
    rows = np.arange(n) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((len(rows), hq, d))
    lse = np.zeros((len(rows), hq))
    chunk = max(1, (1 << 24) // (grp * m))
    for s in range(0, len(rows), chunk):
        r = rows[s:s + chunk]
        for g in range(hkv):
            qg = np.asarray(q_rot[r, g * grp:(g + 1) * grp], np.float64).reshape(-1, d)
            t = scale * (qg @ np.asarray(k_sum[g], np.float64).T)     # [R*grp, M]
            mx = t.max(axis=1, keepdims=True)
            e = np.exp(t - mx)
            l = e.sum(axis=1, keepdims=True)
            o = (e @ np.asarray(v_sum[g], np.float64)) / l
            out[s:s + len(r), g * grp:(g + 1) * grp] = o.reshape(len(r), grp, d)
            lse[s:s + len(r), g * grp:(g + 1) * grp] = (mx + np.log(l)).reshape(len(r), grp)
    return out, lse


# ----------------------------------------------------------------------------
# Tokenwise softmax gate (papernotes.org notes, flowchart node F and the
# overall framework; ai.info summary: a learned tokenwise softmax mixer)
# ----------------------------------------------------------------------------

def gate_weights(gate_logits: np.ndarray) -> np.ndarray:
    """(g_loc, g_cmp) = softmax over the last axis of size 2."""
    lg = np.asarray(gate_logits, np.float64)
    e = np.exp(lg - lg.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def gate_mix(o_loc: np.ndarray, o_cmp: np.ndarray, gate_logits: np.ndarray) -> np.ndarray:
    """O = g_loc * o_loc + g_cmp * o_cmp with logits ``[N, 2]`` or ``[N, Hq, 2]``."""
    g = gate_weights(gate_logits)
    if g.ndim == 2:
        g = g[:, None, :]
    return g[..., 0:1] * o_loc + g[..., 1:2] * o_cmp


# ----------------------------------------------------------------------------
# The whole forward, in the flowchart's order (papernotes.org notes, overall
# framework flowchart: RoPE, then the two branches, then the gate)
# ----------------------------------------------------------------------------

def forward(p, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, gate_logits,
            rows: Optional[np.ndarray] = None, scale: Optional[float] = None) -> dict:
    """Run the five steps and return the output and every intermediate.

    ``p`` carries ``grid``, ``window``, ``block``, ``rope_pairs``,
    ``rope_base`` and ``head_dim``.  Arrays are in packed order.  With
    ``rows`` only those query tokens are computed (summaries are always
    built in full) and ``q_rot`` covers those rows only.
    """
    tau = 1.0 / math.sqrt(p.head_dim) if scale is None else scale
    coords = np.asarray(coords)
    if rows is None:
        q_rot = rotate(q, coords, p.rope_pairs, p.rope_base)
    else:
        rows = np.asarray(rows, np.int64)
        q_rot = rotate(np.asarray(q)[rows], coords[rows], p.rope_pairs, p.rope_base)
    k_rot = rotate(k_loc, coords, p.rope_pairs, p.rope_base)
    mode = getattr(p, "summary_mode", "token")
    k_sum, v_sum = block_summaries(k_cmp, v_cmp, a, coords, p.grid, p.block,
                                   p.rope_pairs, p.rope_base, mode=mode)
    # the compressed branch's query: rotated, except in the coordinate-blind
    # variant
    if mode != "blind":
        q_cmp = q_rot
    else:
        q_cmp = np.asarray(q, np.float64) if rows is None else np.asarray(q, np.float64)[rows]
    o_loc, lse_loc = local_attention(q_rot, k_rot, v_loc, coords, p.grid, p.window, tau, rows,
                                     q_is_rows=rows is not None)
    o_cmp, lse_cmp = global_attention(q_cmp, k_sum, v_sum, tau, q_is_rows=rows is not None)
    g = gate_logits if rows is None else np.asarray(gate_logits)[rows]
    out = gate_mix(o_loc, o_cmp, g)
    return dict(out=out, o_loc=o_loc, o_cmp=o_cmp, lse_loc=lse_loc, lse_cmp=lse_cmp,
                k_sum=k_sum, v_sum=v_sum, q_rot=q_rot, k_rot=k_rot, q_cmp=q_cmp)


# ----------------------------------------------------------------------------
# Backward.  The operator is a block of a trained network (papernotes.org
# notes, the loss / training paragraph); its gradients are the derivatives of
# the forward above.  For one softmax attention o = sum_u p_u v_u with
# p = softmax(scale * <q, k_u>) and upstream gradient g:
#   dp_u = <g, v_u>,  D = sum_u p_u dp_u (= <g, o>),  ds_u = p_u (dp_u - D),
#   dq = scale * sum_u ds_u k_u,  dk_u = scale * ds_u q,  dv_u = p_u g.
# ----------------------------------------------------------------------------

def rotate_transpose(x: np.ndarray, coords: np.ndarray,
                     rope_pairs: Sequence[int] = (11, 11, 10),
                     base: float = 10000.0) -> np.ndarray:
    """R(c_i)^T x_{i,h}: each 2x2 block of R(c) transposed (the inverse)."""
    x = np.asarray(x, dtype=np.float64)
    y = x.copy()
    omega = axial_frequencies(rope_pairs, base)
    p = 0
    for a, m in enumerate(rope_pairs):
        ca = np.asarray(coords[:, a], dtype=np.float64)
        for r in range(m):
            th = omega[a][r] * ca
            cs, sn = np.cos(th)[:, None], np.sin(th)[:, None]
            x0, x1 = x[:, :, 2 * p], x[:, :, 2 * p + 1]
            y[:, :, 2 * p] = cs * x0 + sn * x1
            y[:, :, 2 * p + 1] = -sn * x0 + cs * x1
            p += 1
    return y


def local_attention_backward(q_rot: np.ndarray, k_rot: np.ndarray, v: np.ndarray,
                             coords: np.ndarray, grid: Sequence[int], window: Sequence[int],
                             scale: float, d_out: np.ndarray,
                             rows: Optional[np.ndarray] = None, chunk: int = 4096,
                             q_is_rows: bool = False):
    """Gradients of the local branch for upstream ``d_out`` [N, Hq, D].

    Returns ``(dq [R, Hq, D], dk [N, Hkv, D], dv [N, Hkv, D])``: ``dq`` for the
    query rows ``rows`` (default all) and the contributions of those rows to
    every key.  The window is symmetric (u in N(i) iff i in N(u)), so ``dk``
    and ``dv`` are exact at every key whose own window lies inside ``rows``.
    With ``q_is_rows`` the queries and ``d_out`` are given for those rows only.
    """
    grid = tuple(int(g) for g in grid)
    n = k_rot.shape[0]
    hq, d = q_rot.shape[1:]
    hkv = k_rot.shape[1]
    grp = hq // hkv
    coords = np.asarray(coords, np.int64)
    lattice = np.full(grid, -1, dtype=np.int64)
    lattice[coords[:, 0], coords[:, 1], coords[:, 2]] = np.arange(n)
    offs = np.array(_window_offsets(window), dtype=np.int64)
    rows = np.arange(n) if rows is None else np.asarray(rows, np.int64)
    gmax = np.array(grid, dtype=np.int64) - 1
    dq = np.zeros((len(rows), hq, d))
    dk = np.zeros((n, hkv, d))
    dv = np.zeros((n, hkv, d))
    for s in range(0, len(rows), chunk):
        r = rows[s:s + chunk]
        nr = len(r)
        qsel = np.arange(s, s + nr) if q_is_rows else r
        qc = np.asarray(q_rot[qsel], np.float64).reshape(nr, hkv, grp, d)
        gc = np.asarray(d_out[qsel], np.float64).reshape(nr, hkv, grp, d)
        ci = coords[r]
        pos = np.zeros((nr, len(offs)), dtype=np.int64)
        valid = np.zeros((nr, len(offs)), dtype=bool)
        logit = np.full((nr, len(offs), hkv, grp), -np.inf)
        dp = np.zeros((nr, len(offs), hkv, grp))
        for t, off in enumerate(offs):
            cu = ci + off
            ok = np.all((cu >= 0) & (cu <= gmax), axis=1)
            cc = np.clip(cu, 0, gmax)
            pu = lattice[cc[:, 0], cc[:, 1], cc[:, 2]]
            ku = np.asarray(k_rot[pu], np.float64)
            vu = np.asarray(v[pu], np.float64)
            logit[:, t] = np.where(ok[:, None, None], scale * np.einsum("nkgd,nkd->nkg", qc, ku),
                                   -np.inf)
            dp[:, t] = np.einsum("nkgd,nkd->nkg", gc, vu)
            pos[:, t], valid[:, t] = pu, ok
        mx = logit.max(axis=1, keepdims=True)
        e = np.exp(logit - mx)
        p = e / e.sum(axis=1, keepdims=True)                      # [nr, T, hkv, grp]
        big_d = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - big_d)
        dqc = np.zeros((nr, hkv, grp, d))
        for t in range(len(offs)):
            ok = valid[:, t]
            pu = pos[ok, t]
            ku = np.asarray(k_rot[pu], np.float64)
            dqc[ok] += scale * ds[ok, t][..., None] * ku[:, :, None, :]
            np.add.at(dk, pu, scale * np.einsum("nkg,nkgd->nkd", ds[ok, t], qc[ok]))
            np.add.at(dv, pu, np.einsum("nkg,nkgd->nkd", p[ok, t], gc[ok]))
        dq[s:s + nr] = dqc.reshape(nr, hq, d)
    return dq, dk, dv


def global_attention_backward(q_rot: np.ndarray, k_sum: np.ndarray, v_sum: np.ndarray,
                              scale: float, d_out: np.ndarray,
                              rows: Optional[np.ndarray] = None):
    """Gradients of the query->summary branch for upstream ``d_out``.

    Returns ``(dq [R, Hq, D], dk_sum [Hkv, M, D], dv_sum [Hkv, M, D])`` for the
    query rows ``rows`` (default all); the summary gradients hold the
    contributions of those rows.
    """
    n, hq, d = q_rot.shape
    hkv, m, _ = k_sum.shape
    grp = hq // hkv
    rows = np.arange(n) if rows is None else np.asarray(rows, np.int64)
    dq = np.zeros((len(rows), hq, d))
    dk = np.zeros((hkv, m, d))
    dv = np.zeros((hkv, m, d))
    chunk = max(1, (1 << 23) // (grp * m))
    for s in range(0, len(rows), chunk):
        r = rows[s:s + chunk]
        for g in range(hkv):
            kg = np.asarray(k_sum[g], np.float64)
            vg = np.asarray(v_sum[g], np.float64)
            qg = np.asarray(q_rot[r, g * grp:(g + 1) * grp], np.float64).reshape(-1, d)
            gg = np.asarray(d_out[r, g * grp:(g + 1) * grp], np.float64).reshape(-1, d)
            t = scale * (qg @ kg.T)
            e = np.exp(t - t.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)                  # [R*grp, M]
            dp = gg @ vg.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[s:s + len(r), g * grp:(g + 1) * grp] = (scale * (ds @ kg)).reshape(len(r), grp, d)
            dk[g] += scale * (ds.T @ qg)
            dv[g] += p.T @ gg
    return dq, dk, dv


def block_summaries_backward(dk_sum: np.ndarray, dv_sum: np.ndarray, a: Optional[np.ndarray],
                             coords: np.ndarray, grid: Sequence[int], block: Sequence[int],
                             rope_pairs: Sequence[int] = (11, 11, 10), base: float = 10000.0,
                             mode: str = "token"):
    """Gradients of (k~, v~) with respect to (k_cmp, v_cmp): since
    k~_j = sum_{u in B_j} a_u R(c_u) k_u and v~_j = sum a_u v_u,
    dk_u = a_u R(c_u)^T dk~_j(u) and dv_u = a_u dv~_j(u).  For the
    summary-centre variant R(c_u) is R(c^_j(u)); coordinate-blind: no R."""
    hkv, m, d = dk_sum.shape
    n = len(coords)
    vol = int(np.prod(block))
    w = (np.full((n, hkv), 1.0 / vol) if a is None else np.asarray(a, dtype=np.float64))
    j = block_index(coords, grid, block)
    gk = np.asarray(dk_sum, np.float64)[:, j].transpose(1, 0, 2)      # [N, Hkv, D]
    gv = np.asarray(dv_sum, np.float64)[:, j].transpose(1, 0, 2)
    if mode == "token":
        dk = rotate_transpose(w[:, :, None] * gk, coords, rope_pairs, base)
    elif mode == "centre":
        dk = rotate_transpose(w[:, :, None] * gk, block_centres(grid, block)[j], rope_pairs,
                              base)
    elif mode == "blind":
        dk = w[:, :, None] * gk
    else:
        raise ValueError(f"summary mode {mode!r}")
    dv = w[:, :, None] * gv
    return dk, dv


def gate_backward(gate_logits: np.ndarray, d_out: np.ndarray, o_loc: np.ndarray,
                  o_cmp: np.ndarray):
    """Gradients through O = g_loc o_loc + g_cmp o_cmp, g = softmax(logits).

    Returns ``(dgate, d_loc, d_cmp)``: the logits' gradient (same shape as
    the logits) and the upstream gradients of the two branches, g_b * d_out.
    With one gate per token the gate's gradient sums over heads.
    """
    g = gate_weights(gate_logits)
    gh = g[:, None, :] if g.ndim == 2 else g
    d_out = np.asarray(d_out, np.float64)
    dg_loc = (d_out * o_loc).sum(axis=-1)                              # [N, Hq]
    dg_cmp = (d_out * o_cmp).sum(axis=-1)
    if g.ndim == 2:
        dg_loc, dg_cmp = dg_loc.sum(axis=1), dg_cmp.sum(axis=1)
    # softmax Jacobian of two logits: dl0 = g0 g1 (dg0 - dg1) = -dl1
    t = g[..., 0] * g[..., 1] * (dg_loc - dg_cmp)
    dgate = np.stack([t, -t], axis=-1)
    return dgate, gh[..., 0:1] * d_out, gh[..., 1:2] * d_out


def backward(p, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, gate_logits, d_out,
             scale: Optional[float] = None) -> dict:
    """All input gradients of the forward for the upstream gradient ``d_out``
    of its output: dq, dk_loc, dv_loc, dk_cmp, dv_cmp and dgate (plus the
    branch intermediates).  ``p`` as in :func:`forward`."""
    tau = 1.0 / math.sqrt(p.head_dim) if scale is None else scale
    coords = np.asarray(coords)
    f = forward(p, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, gate_logits, scale=tau)
    dgate, d_loc, d_cmp = gate_backward(gate_logits, d_out, f["o_loc"], f["o_cmp"])
    dq_l, dk_r, dv_loc = local_attention_backward(f["q_rot"], f["k_rot"], v_loc, coords, p.grid,
                                                  p.window, tau, d_loc)
    dq_c, dk_sum, dv_sum = global_attention_backward(f["q_cmp"], f["k_sum"], f["v_sum"], tau,
                                                     d_cmp)
    mode = getattr(p, "summary_mode", "token")
    if mode != "blind":
        dq = rotate_transpose(dq_l + dq_c, coords, p.rope_pairs, p.rope_base)
    else:       # the compressed branch saw the unrotated query
        dq = rotate_transpose(dq_l, coords, p.rope_pairs, p.rope_base) + dq_c
    dk_loc = rotate_transpose(dk_r, coords, p.rope_pairs, p.rope_base)
    dk_cmp, dv_cmp = block_summaries_backward(dk_sum, dv_sum, a, coords, p.grid, p.block,
                                              p.rope_pairs, p.rope_base, mode=mode)
    return dict(dq=dq, dk_loc=dk_loc, dv_loc=dv_loc, dk_cmp=dk_cmp, dv_cmp=dv_cmp,
                dgate=dgate, dk_sum=dk_sum, dv_sum=dv_sum, d_loc=d_loc, d_cmp=d_cmp,
                fwd=f)


# ----------------------------------------------------------------------------
# The layer around the operator (papernotes.org notes, flowchart node B
# "linear projection and layer normalisation produce Q, K_loc, V_loc, K_cmp,
# V_cmp" and node G "residual output"; key design 1 writes the projections as
# W LN(h))
# ----------------------------------------------------------------------------

def layer_norm(h: np.ndarray, gamma: Optional[np.ndarray], beta: Optional[np.ndarray],
               eps: float = 1e-5) -> np.ndarray:
    """(h - mean) / sqrt(var + eps) * gamma + beta over the last axis, with the
    biased variance; gamma / beta None mean 1 / 0."""
    h = np.asarray(h, np.float64)
    mu = h.mean(axis=-1, keepdims=True)
    var = ((h - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (h - mu) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, np.float64)
    if beta is not None:
        y = y + np.asarray(beta, np.float64)
    return y


def qkv_projection(x: np.ndarray, w_qkv: np.ndarray, n_q_heads: int, n_kv_heads: int,
                   head_dim: int = 64):
    """The five bias-free projections x W^T, split in the order Q, K_loc,
    V_loc, K_cmp, V_cmp and shaped per head: ``(q [N, Hq, D], k_loc, v_loc,
    k_cmp, v_cmp [N, Hkv, D])``."""
    y = np.asarray(x, np.float64) @ np.asarray(w_qkv, np.float64).T
    n = y.shape[0]
    sizes = [n_q_heads * head_dim] + [n_kv_heads * head_dim] * 4
    if y.shape[1] != sum(sizes):
        raise ValueError("w_qkv rows must be Hq*D + 4*Hkv*D")
    out, off = [], 0
    for sz in sizes:
        out.append(y[:, off:off + sz].reshape(n, sz // head_dim, head_dim))
        off += sz
    return tuple(out)


def layer_forward(p, h, gamma, beta, w_qkv, w_o, a, coords, gate_logits, eps: float = 1e-5,
                  rows: Optional[np.ndarray] = None, scale: Optional[float] = None) -> dict:
    """h' = h + O W_O^T with O the operator's gated output on the projections
    of LN(h) (concatenated over heads).  ``h`` is ``[N, C]`` in packed order;
    with ``rows`` only those tokens' outputs are computed (every key and
    summary is still built)."""
    x = layer_norm(h, gamma, beta, eps)
    q, k_loc, v_loc, k_cmp, v_cmp = qkv_projection(x, w_qkv, p.n_q_heads, p.n_kv_heads,
                                                   p.head_dim)
    f = forward(p, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, gate_logits, rows=rows,
                scale=scale)
    o = f["out"].reshape(f["out"].shape[0], -1)
    hr = np.asarray(h, np.float64) if rows is None else np.asarray(h, np.float64)[rows]
    out = hr + o @ np.asarray(w_o, np.float64).T
    return dict(out=out, x=x, q=q, k_loc=k_loc, v_loc=v_loc, k_cmp=k_cmp, v_cmp=v_cmp,
                o=o, fwd=f)
