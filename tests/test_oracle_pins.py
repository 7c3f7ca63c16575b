"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test states the fact it checks and where it comes from ("Geometry Matters
in Packed 3D Attention": papernotes.org notes = key designs and tables;
ai.info summary; onedev.kr summary).  None of them re-types an oracle formula:
they check identities, special cases that reduce to a library routine
(torch's scaled_dot_product_attention in float64 on the CPU), closed forms,
brute force on tiny lattices, and the sizes the pages print.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synthgen as sg
from oracle import pack3d_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAIRS, BASE, D = (11, 11, 10), 10000.0, 64


def _small(grid=(4, 8, 8), hq=4, hkv=2, window=(3, 5, 5), block=(1, 4, 4), packing="raster",
           dtype="f32", weights="softmax", seed=11):
    return sg.Workload("t", grid, packing, hq, hkv, window, block, dtype, weights, seed)


def _fwd(inp, **kw):
    w = inp.workload
    return orc.forward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a,
                       inp.coords, inp.gate, **kw)


def _sdpa(q, k, v, mask=None, scale=0.125):
    """Library attention in float64: q [N,Hq,D], k/v [N,Hkv,D] -> [N,Hq,D]."""
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale, enable_gqa=True)
    return o[0].numpy().transpose(1, 0, 2)


# --------------------------------------------------------------------------
# rotation (key design 1: R(c) is an orthogonal direct sum of 2x2 rotations)
# --------------------------------------------------------------------------

def test_rotation_orthogonal_and_identity_at_origin():
    rng = np.random.default_rng(0)
    assert np.array_equal(orc.rotation_matrix((0, 0, 0)), np.eye(D))
    for _ in range(50):
        c = rng.integers(-200, 200, size=3)
        R = orc.rotation_matrix(c)
        assert np.abs(R.T @ R - np.eye(D)).max() <= 1e-13


def test_relative_displacement_identity():
    """R(c_i)^T R(c_j) = R(c_j - c_i): logits depend only on displacement
    (key design 1; onedev.kr summary, how it works)."""
    rng = np.random.default_rng(1)
    worst = 0.0
    for _ in range(2000):
        ci, cj = rng.integers(0, 128, size=3), rng.integers(0, 128, size=3)
        lhs = orc.rotation_matrix(ci).T @ orc.rotation_matrix(cj)
        worst = max(worst, np.abs(lhs - orc.rotation_matrix(cj - ci)).max())
    assert worst <= 1e-12


def test_rotation_sign_axis_split_and_pairs():
    """The printed 2x2 block [[cos,-sin],[sin,cos]]: a quarter turn sends
    e_{2p} to +e_{2p+1}.  The 11/11/10 split: a z-only coordinate moves only
    dims 0..21, y-only 22..43, x-only 44..63; nothing else couples."""
    R = orc.rotation_matrix((math.pi / 2, 0, 0))  # r = 0 has omega = 1
    e0 = np.zeros(D)
    e0[0] = 1.0
    got = R @ e0
    want = np.zeros(D)
    want[1] = 1.0
    assert np.abs(got - want).max() <= 1e-15
    spans = {0: range(0, 22), 1: range(22, 44), 2: range(44, 64)}
    for axis, span in spans.items():
        c = [0, 0, 0]
        c[axis] = 37
        R = orc.rotation_matrix(c)
        moved = {i for i in range(D) if abs(R[i, i] - 1.0) > 1e-15 or
                 np.abs(np.delete(R[i], i)).max() > 0}
        assert moved == set(span)
    # 2x2 coupling only: off the pair blocks everything is zero
    R = orc.rotation_matrix((5, 9, 13))
    blk = np.kron(np.eye(32), np.ones((2, 2)))
    assert np.abs(R * (1 - blk)).max() == 0.0


def test_rotate_agrees_with_rotation_matrix():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((40, 3, D))
    c = rng.integers(0, 64, size=(40, 3))
    got = orc.rotate(x, c)
    want = np.stack([orc.rotation_matrix(c[i]) @ x[i].T for i in range(40)]).transpose(0, 2, 1)
    assert np.abs(got - want).max() <= 1e-13


def test_translation_invariance():
    """Rotating Q and K with c + t for an integer t changes no logit (a
    corollary of the displacement identity), so both branches are unchanged."""
    w = _small()
    inp = sg.make_inputs(w)
    t = np.array([7, -3, 11])
    tau = 0.125
    q0, k0 = orc.rotate(inp.q, inp.coords), orc.rotate(inp.k_loc, inp.coords)
    q1, k1 = orc.rotate(inp.q, inp.coords + t), orc.rotate(inp.k_loc, inp.coords + t)
    o0, _ = orc.local_attention(q0, k0, inp.v_loc, inp.coords, w.grid, w.window, tau)
    o1, _ = orc.local_attention(q1, k1, inp.v_loc, inp.coords, w.grid, w.window, tau)
    assert np.abs(o0 - o1).max() <= 1e-11
    ks0, vs0 = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block)
    ks1, vs1 = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block,
                                   rope_coords=inp.coords + t)
    g0, _ = orc.global_attention(q0, ks0, vs0, tau)
    g1, _ = orc.global_attention(q1, ks1, vs1, tau)
    assert np.abs(g0 - g1).max() <= 1e-11


# --------------------------------------------------------------------------
# summaries (key design 2, Proposition 2 / Theorem 7)
# --------------------------------------------------------------------------

def _members_brute_force(grid, block):
    """Cells of each aligned block, found by scanning the whole lattice;
    blocks enumerated in raster order of their corner cell."""
    cells = sg.lattice_cells(grid)
    corners = [tuple(c) for c in cells if all(c[a] % block[a] == 0 for a in range(3))]
    return [np.array([i for i, c in enumerate(cells)
                      if all(corner[a] <= c[a] < corner[a] + block[a] for a in range(3))])
            for corner in corners]


def test_proposition2_query_summary_logit():
    """<R(c_i) q_i, k~_j> = sum_{u in B_j} a_u q_i^T R(c_u - c_i) k_u."""
    w = _small(grid=(2, 8, 8), hq=2, hkv=1, block=(2, 4, 4), packing="random")
    inp = sg.make_inputs(w)
    ks, _ = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block)
    members = _members_brute_force(w.grid, w.block)     # raster cell indices
    pos_of_cell = inp.cell_to_pos
    qr = orc.rotate(inp.q, inp.coords)
    rng = np.random.default_rng(3)
    worst = 0.0
    for i in rng.choice(w.n_tokens, 12, replace=False):
        for j, cells in enumerate(members):
            for h in range(w.n_q_heads):
                lhs = qr[i, h] @ ks[0, j]
                rhs = 0.0
                for cell in cells:
                    u = pos_of_cell[cell]
                    Rd = orc.rotation_matrix(inp.coords[u] - inp.coords[i])
                    rhs += inp.a[u, 0] * (inp.q[i, h] @ Rd @ inp.k_cmp[u, 0])
                worst = max(worst, abs(lhs - rhs))
    assert worst <= 1e-11


def test_value_summaries_closed_form_with_zero_keys():
    """K_cmp = 0 makes every summary logit 0, so o_cmp is the plain mean of the
    M value summaries; with uniform weights that is the mean of V_cmp over the
    whole lattice, per KV group."""
    w = _small(weights="uniform", packing="morton")
    inp = sg.make_inputs(w)
    ks, vs = orc.block_summaries(np.zeros_like(inp.k_cmp), inp.v_cmp, None, inp.coords,
                                 w.grid, w.block)
    q = orc.rotate(inp.q, inp.coords)
    o, lse = orc.global_attention(q, ks, vs, 0.125)
    grp = w.n_q_heads // w.n_kv_heads
    for h in range(w.n_q_heads):
        want = inp.v_cmp[:, h // grp].astype(np.float64).mean(axis=0)
        assert np.abs(o[:, h] - want).max() <= 1e-12
    assert np.abs(lse - math.log(w.n_blocks)).max() <= 1e-12


def test_value_summaries_with_softmax_weights():
    """v~_j is the a-weighted sum of the values of block j's cells, with each
    KV group's own weights (notes, key design 2, the equation for v~_j: a
    normalised weighted average).  Pinned two ways on a randomly packed
    lattice with two KV groups and per-group softmax weights:
    * brute force: block members found by scanning the lattice, summed with
      their weights one by one;
    * a closed form at any size: K_cmp = 0 makes every query->summary logit 0,
      so o_cmp is the mean over j of v~_j, i.e. (1/M) sum_u a_u v_u over all
      tokens of the group (no block membership involved).
    Plausible mistakes (pooling V uniformly, or with the other group's
    weights) fail both."""
    w = _small(grid=(2, 8, 8), hq=4, hkv=2, block=(2, 4, 4), packing="random")
    inp = sg.make_inputs(w)
    a = inp.a
    assert np.abs(a[:, 0] - a[:, 1]).max() > 0.1          # the groups' weights differ
    assert np.abs(a - 1.0 / 32).max() > 0.1                # and are far from uniform
    _, vs = orc.block_summaries(inp.k_cmp, inp.v_cmp, a, inp.coords, w.grid, w.block)
    members = _members_brute_force(w.grid, w.block)
    want = np.zeros_like(vs)
    for j, cells in enumerate(members):
        for cell in cells:
            u = inp.cell_to_pos[cell]
            for g in range(w.n_kv_heads):
                want[g, j] += a[u, g] * inp.v_cmp[u, g].astype(np.float64)
    assert np.abs(vs - want).max() <= 1e-13
    # the closed form through the compressed branch with zero keys
    ks0, vs0 = orc.block_summaries(np.zeros_like(inp.k_cmp), inp.v_cmp, a, inp.coords, w.grid,
                                   w.block)
    o, _ = orc.global_attention(orc.rotate(inp.q, inp.coords), ks0, vs0, 0.125)
    grp = w.n_q_heads // w.n_kv_heads
    pooled = [(a[:, g, None] * inp.v_cmp[:, g].astype(np.float64)).sum(0) / w.n_blocks
              for g in range(w.n_kv_heads)]
    for h in range(w.n_q_heads):
        assert np.abs(o[:, h] - pooled[h // grp]).max() <= 1e-13
    # test power: the plausible mistakes are far outside both bounds
    for bad_a in (None, np.ascontiguousarray(a[:, ::-1])):
        _, bad = orc.block_summaries(inp.k_cmp, inp.v_cmp, bad_a, inp.coords, w.grid, w.block)
        assert np.abs(bad - want).max() > 1e-2
        _, bad0 = orc.block_summaries(np.zeros_like(inp.k_cmp), inp.v_cmp, bad_a, inp.coords,
                                      w.grid, w.block)
        ob, _ = orc.global_attention(orc.rotate(inp.q, inp.coords), ks0, bad0, 0.125)
        assert max(np.abs(ob[:, h] - pooled[h // grp]).max() for h in range(w.n_q_heads)) > 1e-3


def test_summaries_with_unit_blocks_are_rotated_keys():
    """With 1x1x1 blocks and a = 1 each summary is one rotated key, in raster
    cell order."""
    w = _small(block=(1, 1, 1), packing="random")
    inp = sg.make_inputs(w)
    ks, vs = orc.block_summaries(inp.k_cmp, inp.v_cmp, np.ones((w.n_tokens, w.n_kv_heads)),
                                 inp.coords, w.grid, w.block)
    kr = orc.rotate(inp.k_cmp, inp.coords)
    # raster cell index -> packed position
    assert np.abs(ks.transpose(1, 0, 2) - kr[inp.cell_to_pos]).max() <= 1e-15
    assert np.abs(vs.transpose(1, 0, 2) - inp.v_cmp[inp.cell_to_pos]).max() == 0.0


# --------------------------------------------------------------------------
# branches against library attention
# --------------------------------------------------------------------------

def _box_mask(coords, window):
    r = np.array([x // 2 for x in window])
    d = np.abs(coords[:, None, :].astype(np.int64) - coords[None, :, :].astype(np.int64))
    return np.all(d <= r, axis=2)


@pytest.mark.parametrize("packing", ["raster", "random"])
def test_local_branch_is_masked_dense_attention(packing):
    """Local attention = attention over all tokens with a boolean box mask
    built by brute force from the coordinates (key design 3)."""
    w = sg.WORKLOADS["tiny_f32_4x16x16"].with_(packing=packing)
    inp = sg.make_inputs(w)
    q, k = orc.rotate(inp.q, inp.coords), orc.rotate(inp.k_loc, inp.coords)
    o, _ = orc.local_attention(q, k, inp.v_loc, inp.coords, w.grid, w.window, 0.125)
    want = _sdpa(q, k, inp.v_loc.astype(np.float64), _box_mask(inp.coords, w.window))
    assert np.abs(o - want).max() <= 1e-12


def test_local_branch_window_covering_lattice_is_dense():
    w = _small(window=(7, 15, 15))
    inp = sg.make_inputs(w)
    q, k = orc.rotate(inp.q, inp.coords), orc.rotate(inp.k_loc, inp.coords)
    o, _ = orc.local_attention(q, k, inp.v_loc, inp.coords, w.grid, w.window, 0.125)
    assert np.abs(o - _sdpa(q, k, inp.v_loc.astype(np.float64))).max() <= 1e-12


def test_local_branch_zero_keys_is_box_mean():
    """K_loc = 0: uniform weights over the clipped box, i.e. the box mean of
    V_loc, computed here with 3-D prefix sums on the lattice."""
    w = _small(grid=(5, 9, 11), window=(3, 5, 7), packing="morton", weights="uniform")
    inp = sg.make_inputs(w)
    q = orc.rotate(inp.q, inp.coords)
    o, lse = orc.local_attention(q, np.zeros_like(inp.k_loc), inp.v_loc, inp.coords, w.grid,
                                 w.window, 0.125)
    Z, Y, X = w.grid
    lat = np.zeros((Z, Y, X, w.n_kv_heads, D))
    lat[inp.coords[:, 0], inp.coords[:, 1], inp.coords[:, 2]] = inp.v_loc
    P = np.zeros((Z + 1, Y + 1, X + 1, w.n_kv_heads, D))
    P[1:, 1:, 1:] = lat.cumsum(0).cumsum(1).cumsum(2)
    grp = w.n_q_heads // w.n_kv_heads
    worst = 0.0
    for i, (z, y, x) in enumerate(inp.coords):
        lo = [max(c - r // 2, 0) for c, r in zip((z, y, x), w.window)]
        hi = [min(c + r // 2, g - 1) + 1 for c, r, g in zip((z, y, x), w.window, w.grid)]
        s = (P[hi[0], hi[1], hi[2]] - P[lo[0], hi[1], hi[2]] - P[hi[0], lo[1], hi[2]]
             - P[hi[0], hi[1], lo[2]] + P[lo[0], lo[1], hi[2]] + P[lo[0], hi[1], lo[2]]
             + P[hi[0], lo[1], lo[2]] - P[lo[0], lo[1], lo[2]])
        cnt = np.prod([b - a for a, b in zip(lo, hi)])
        for h in range(w.n_q_heads):
            worst = max(worst, np.abs(o[i, h] - s[h // grp] / cnt).max())
        assert abs(lse[i, 0] - math.log(cnt)) <= 1e-12
    assert worst <= 1e-12


def test_unit_blocks_make_the_compressed_branch_dense_attention():
    """v = 1 (1x1x1 blocks, a = 1) with the gate forced to the compressed
    branch: the operator is dense axial-RoPE attention over
    (R(c)Q, R(c)K_cmp, V_cmp) (key design 2 with |B_j| = 1)."""
    w = _small(block=(1, 1, 1), packing="random")
    inp = sg.make_inputs(w)
    gate = np.tile(np.array([[-1e3, 1e3]]), (w.n_tokens, 1))
    r = orc.forward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp,
                    np.ones((w.n_tokens, w.n_kv_heads)), inp.coords, gate)
    want = _sdpa(orc.rotate(inp.q, inp.coords), orc.rotate(inp.k_cmp, inp.coords),
                 inp.v_cmp.astype(np.float64))
    assert np.abs(r["out"] - want).max() <= 1e-12


def test_gate_extremes_and_midpoint():
    """Forcing g_loc -> 1 returns the local branch, g_cmp -> 1 the compressed
    branch (the clamps of Table 3), and equal logits their mean."""
    w = _small()
    inp = sg.make_inputs(w)
    n = w.n_tokens
    outs = {}
    for name, lg in (("loc", [40.0, -40.0]), ("cmp", [-40.0, 40.0]), ("mid", [0.3, 0.3])):
        r = _fwd(inp.__class__(**{**inp.__dict__, "gate": np.tile(np.array([lg]), (n, 1))}))
        outs[name] = r
    e80 = math.exp(-80) * 4
    assert np.abs(outs["loc"]["out"] - outs["loc"]["o_loc"]).max() <= e80
    assert np.abs(outs["cmp"]["out"] - outs["cmp"]["o_cmp"]).max() <= e80
    mid = outs["mid"]
    assert np.abs(mid["out"] - 0.5 * (mid["o_loc"] + mid["o_cmp"])).max() <= 1e-15
    # per-head logits broadcast the same way
    gh = np.tile(np.array([[[40.0, -40.0]]]), (n, w.n_q_heads, 1))
    assert np.abs(orc.gate_mix(mid["o_loc"], mid["o_cmp"], gh) - mid["o_loc"]).max() <= e80


# --------------------------------------------------------------------------
# packing equivariance (Proposition 1)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("wname", ["tiny_f32_4x16x16", "small_gqa"])
def test_packing_equivariance(wname):
    w = sg.WORKLOADS.get(wname) or _small(grid=(4, 8, 12), window=(3, 7, 7))
    base = sg.make_inputs(w.with_(packing="raster"))
    ref = _fwd(base)
    for kind in ("morton", "block", "block_morton", "random"):
        inp = base.repacked(kind)
        r = _fwd(inp)
        back = inp.cell_to_pos[base.order]   # packed position of each raster cell
        for key in ("out", "o_loc", "o_cmp", "lse_loc", "lse_cmp"):
            assert np.abs(r[key][back] - ref[key]).max() <= 1e-12, (kind, key)
        assert np.abs(r["k_sum"] - ref["k_sum"]).max() <= 1e-12


def test_negative_control_sequence_rope_breaks_equivariance():
    """Rotating by the packed index instead of the cell (the packed-sequence
    RoPE baseline) is not packing-equivariant; the equivariance check must
    see it."""
    w = _small()
    base = sg.make_inputs(w.with_(packing="raster"))
    seqc = lambda n: np.stack([np.zeros(n), np.zeros(n), np.arange(n)], 1).astype(np.int64)

    def out(inp):
        c = seqc(w.n_tokens)
        q, k = orc.rotate(inp.q, c), orc.rotate(inp.k_loc, c)
        o, _ = orc.local_attention(q, k, inp.v_loc, inp.coords, w.grid, w.window, 0.125)
        return o

    ref = out(base)
    inp = base.repacked("random")
    back = inp.cell_to_pos[base.order]
    assert np.abs(out(inp)[back] - ref).max() > 1e-3


def test_negative_control_unrotated_keys_break_proposition2():
    """Pooling unrotated keys and rotating the pooled vector at the block
    corner does not give the displacement-weighted logit of Proposition 2."""
    w = _small(grid=(1, 4, 4), hq=1, hkv=1, block=(1, 4, 4))
    inp = sg.make_inputs(w)
    kz = (inp.a[:, :, None] * inp.k_cmp).sum(axis=0)            # [1, D], pooled raw
    wrong = orc.rotate(kz[None], np.zeros((1, 3), np.int64))[0, 0]
    right, _ = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block)
    assert np.abs(wrong - right[0, 0]).max() > 1e-2


# --------------------------------------------------------------------------
# sizes printed on the pages, and the window count
# --------------------------------------------------------------------------

def test_golden_sizes_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "pages_shapes.json")))
    tg = g["allen_token_grid"]
    assert [v // p for v, p in zip(tg["voxels"], tg["patch"])] == tg["token_grid"]
    grid = tuple(tg["token_grid"])
    cells = sg.lattice_cells(grid)
    assert len(cells) == tg["n_tokens"]
    j = orc.block_index(cells, grid, tuple(g["block"]["shape"]))
    m = int(j.max()) + 1
    assert m == g["summaries_at_262144"]["n_summaries"]
    assert np.bincount(j).tolist() == [g["block"]["volume"]] * m
    assert len(cells) // m == g["summaries_at_262144"]["comparison_reduction_vs_dense"]
    qs = g["query_summary_tensor"]
    assert round(len(cells) * m / 1e9, 2) == qs["entries_per_head_group_billions"]
    assert 2 * len(cells) * m / 1e9 > qs["two_kv_groups_exceed_billions"]
    r = g["rope"]
    R = orc.rotation_matrix((3, 5, 7), r["head_dim"], tuple(r["pairs_zyx"]), r["base"])
    assert np.all(np.abs(np.diag(R) - 1.0) > 0)   # no identity remainder at d_h = 64


def test_window_size_sum_matches_separable_count():
    """sum_i |N(i)| of a clipped box factorises over axes: per axis the sum of
    clipped extents.  3x7x7 on 64^3 gives 190 * 436 * 436."""
    def axis_sum(E, r):
        return sum(min(c + r, E - 1) - max(c - r, 0) + 1 for c in range(E))
    grid, window = (64, 64, 64), (3, 7, 7)
    coords = sg.lattice_cells(grid)
    got = int(orc.local_window_sizes(coords, grid, window).sum())
    assert got == axis_sum(64, 1) * axis_sum(64, 3) * axis_sum(64, 3) == 36118240


# --------------------------------------------------------------------------
# the input generator's packings
# --------------------------------------------------------------------------

def test_packings_are_bijections_and_morton_is_z_order():
    grid = (2, 4, 4)
    for kind in sg.PACKINGS:
        order, coords, c2p = sg.packing(grid, kind, 5)
        assert sorted(order.tolist()) == list(range(32))
        assert np.array_equal(c2p[order], np.arange(32))
    _, coords, _ = sg.packing((1, 4, 4), "morton")
    want = [(0, 0), (0, 1), (1, 0), (1, 1), (0, 2), (0, 3), (1, 2), (1, 3),
            (2, 0), (2, 1), (3, 0), (3, 1), (2, 2), (2, 3), (3, 2), (3, 3)]
    assert [tuple(c[1:]) for c in coords] == want
    _, coords, _ = sg.packing((1, 4, 8), "block")
    assert [tuple(c[1:]) for c in coords[:5]] == [(0, 0), (0, 1), (0, 2), (0, 3), (1, 0)]
    assert tuple(coords[16][1:]) == (0, 4)
    # two-level block-Morton: 1x2x2 blocks of a 1x4x4 lattice visited in z
    # order of their block indices (0,0), (0,1), (1,0), (1,1), raster inside
    _, coords, _ = sg.packing((1, 4, 4), "block_morton", block=(1, 2, 2))
    want = [(0, 0), (0, 1), (1, 0), (1, 1), (0, 2), (0, 3), (1, 2), (1, 3),
            (2, 0), (2, 1), (3, 0), (3, 1), (2, 2), (2, 3), (3, 2), (3, 3)]
    assert [tuple(c[1:]) for c in coords] == want
    _, coords, _ = sg.packing((1, 8, 8), "block_morton", block=(1, 4, 4))
    assert [tuple(c[1:]) for c in coords[:5]] == [(0, 0), (0, 1), (0, 2), (0, 3), (1, 0)]
    assert [tuple(c[1:]) for c in coords[16:32:15]] == [(0, 4), (3, 7)]
    assert tuple(coords[32][1:]) == (4, 0)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-40], dtype=np.float32)
    got = sg.round_to_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got, want)
    # across chunk boundaries and with a multi-dimensional shape
    y = np.random.default_rng(0).standard_normal((3, (1 << 23) + 5), dtype=np.float32)
    assert np.array_equal(sg.round_to_bf16(y),
                          torch.from_numpy(y).to(torch.bfloat16).to(torch.float32).numpy())


def test_sampled_rows_equal_full_rows():
    """Computing a subset of query rows gives those rows of the full result."""
    w = _small(packing="random")
    inp = sg.make_inputs(w)
    full = _fwd(inp)
    rows = np.array([0, 5, 17, 100, w.n_tokens - 1])
    part = _fwd(inp, rows=rows)
    for key in ("out", "o_loc", "o_cmp", "lse_loc", "lse_cmp"):
        assert np.abs(part[key] - full[key][rows]).max() <= 1e-13, key
