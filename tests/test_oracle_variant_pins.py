"""Pins of the oracle's compressed-branch variants ("Geometry Matters in Packed
3D Attention": papernotes.org notes, key design 2 - rotation before the
block sum is exact; the summary's contributions and findings - a cheaper
summary-centre placement of the rotation, and a coordinate-blind compressed
branch as the missing control).

"centre" rotates the pooled unrotated keys once at the block's centre,
"blind" uses no rotation on either side of the compressed branch.  Pinned by
special cases that reduce to the exact form or to a library routine, by a
trigonometric closed form for blocks of equal keys, by packing equivariance,
and by finite differences for the backward.  None re-types an oracle
formula.
"""

import math

import numpy as np
import pytest

import synthgen as sg
from oracle import pack3d_oracle as orc
from tests.test_oracle_bwd_pins import _bwd, _fd_check, _inputs
from tests.test_oracle_pins import _fwd, _sdpa, _small


def test_centre_equals_token_for_unit_blocks():
    """A 1x1x1 block's centre is its cell: both placements coincide."""
    w = _small(block=(1, 1, 1), packing="random")
    inp = sg.make_inputs(w)
    tok = _fwd(inp)
    cen = orc.forward(w.with_(summary_mode="centre"), inp.q, inp.k_loc, inp.v_loc, inp.k_cmp,
                      inp.v_cmp, inp.a, inp.coords, inp.gate)
    for key in ("out", "o_cmp", "lse_cmp", "k_sum", "v_sum"):
        assert np.abs(tok[key] - cen[key]).max() <= 1e-12, key


def _constant_block_keys(w, rng):
    """K_cmp equal on every cell of a block (per KV group), uniform weights."""
    inp = sg.make_inputs(w)
    j = orc.block_index(inp.coords, w.grid, w.block)
    kb = rng.standard_normal((w.n_blocks, w.n_kv_heads, 64))
    return inp, kb, kb[j]


@pytest.mark.parametrize("block", [(2, 3, 4), (1, 4, 4), (3, 1, 2)])
def test_token_summary_of_equal_keys_is_damped_centre_summary(block):
    """For equal keys k in a block and uniform weights, the exact summary is
    (1/v) sum_u R(c_u) k.  Per rotary pair (axis a, frequency w) the offsets
    of the cells from the block centre are symmetric, so the sines cancel:
    sum_u R(c_u) = R(c^) * v * mean_u cos(w (c_u,a - c^_a)).  Hence every
    pair of the exact summary equals s_p times the same pair of the
    centre-placed summary, s_p = mean over the block's offsets on axis a of
    cos(w * offset).  Only the geometric centre makes the sines cancel."""
    grid = tuple(2 * b for b in block)
    w = _small(grid=grid, hq=2, hkv=2, block=block, packing="random")
    rng = np.random.default_rng(4)
    inp, kb, k_cmp = _constant_block_keys(w, rng)
    args = (k_cmp, inp.v_cmp, None, inp.coords, w.grid, w.block)
    tok, _ = orc.block_summaries(*args, mode="token")
    cen, _ = orc.block_summaries(*args, mode="centre")
    blind, vs = orc.block_summaries(*args, mode="blind")
    # blind: the mean of equal keys is the key itself
    assert np.abs(blind - kb.transpose(1, 0, 2)).max() <= 1e-13
    # rotation keeps the norm of every pair
    pn = lambda x: np.hypot(x[..., 0::2], x[..., 1::2])
    assert np.abs(pn(cen) - pn(blind)).max() <= 1e-12
    omega = orc.axial_frequencies(w.rope_pairs, w.rope_base)
    p = 0
    for ax, m in enumerate(w.rope_pairs):
        off = np.arange(block[ax]) - (block[ax] - 1) / 2.0
        for r in range(m):
            s_p = np.cos(omega[ax][r] * off).mean()
            for comp in (0, 1):
                got = tok[..., 2 * p + comp]
                want = s_p * cen[..., 2 * p + comp]
                assert np.abs(got - want).max() <= 1e-12, (ax, r, comp)
            p += 1


def test_damped_centre_relation_detects_a_wrong_centre(monkeypatch):
    """Negative control: placing the rotation at the block origin instead of
    its centre breaks the relation above."""
    block = (2, 3, 4)
    w = _small(grid=(4, 6, 8), hq=2, hkv=2, block=block, packing="raster")
    inp, kb, k_cmp = _constant_block_keys(w, np.random.default_rng(4))
    args = (k_cmp, inp.v_cmp, None, inp.coords, w.grid, w.block)
    tok, _ = orc.block_summaries(*args, mode="token")
    real = orc.block_centres
    monkeypatch.setattr(orc, "block_centres",
                        lambda g, b: real(g, b) - (np.asarray(b, float) - 1.0) / 2.0)
    cen, _ = orc.block_summaries(*args, mode="centre")
    omega = orc.axial_frequencies(w.rope_pairs, w.rope_base)
    off = np.arange(block[2]) - (block[2] - 1) / 2.0
    p = w.rope_pairs[0] + w.rope_pairs[1] + 1          # an x-axis pair, r = 1
    s_p = np.cos(omega[2][1] * off).mean()
    assert np.abs(tok[..., 2 * p] - s_p * cen[..., 2 * p]).max() > 1e-3


def test_block_centres_are_cell_means():
    """The centre of each aligned block is the mean of its cells'
    coordinates (brute force over the lattice)."""
    grid, block = (4, 6, 8), (2, 3, 4)
    cells = sg.lattice_cells(grid)
    j = orc.block_index(cells, grid, block)
    want = np.zeros((int(np.prod(grid)) // int(np.prod(block)), 3))
    np.add.at(want, j, cells.astype(np.float64))
    want /= np.prod(block)
    assert np.array_equal(orc.block_centres(grid, block), want)


def test_blind_unit_blocks_is_plain_attention():
    """Coordinate-blind with 1x1x1 blocks, a = 1 and the gate forced to the
    compressed branch: the operator is plain attention over (Q, K_cmp,
    V_cmp) with no rotation anywhere (library routine)."""
    w = _small(block=(1, 1, 1), packing="random").with_(summary_mode="blind")
    inp = sg.make_inputs(w)
    gate = np.tile(np.array([[-1e3, 1e3]]), (w.n_tokens, 1))
    r = orc.forward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp,
                    np.ones((w.n_tokens, w.n_kv_heads)), inp.coords, gate)
    want = _sdpa(inp.q.astype(np.float64), inp.k_cmp.astype(np.float64),
                 inp.v_cmp.astype(np.float64))
    assert np.abs(r["out"] - want).max() <= 1e-12
    # and the local branch still sees the rotated query: it differs from the
    # token form's only through the compressed branch
    tok = orc.forward(w.with_(summary_mode="token"), inp.q, inp.k_loc, inp.v_loc, inp.k_cmp,
                      inp.v_cmp, np.ones((w.n_tokens, w.n_kv_heads)), inp.coords, gate)
    assert np.abs(r["o_loc"] - tok["o_loc"]).max() == 0.0


@pytest.mark.parametrize("mode", ["centre", "blind"])
def test_variants_are_packing_equivariant(mode):
    """Proposition 1 holds for both variants: repacking permutes the output."""
    w = _small(grid=(4, 8, 8), window=(3, 5, 5)).with_(summary_mode=mode)
    base = sg.make_inputs(w.with_(packing="raster"))
    ref = _fwd(base)
    for kind in ("morton", "random"):
        inp = base.repacked(kind)
        r = _fwd(inp)
        back = inp.cell_to_pos[base.order]
        for key in ("out", "o_cmp", "lse_cmp"):
            assert np.abs(r[key][back] - ref[key]).max() <= 1e-12, (kind, key)


@pytest.mark.parametrize("mode", ["centre", "blind"])
def test_variant_backward_matches_finite_differences(mode):
    """Every gradient of each variant equals the central difference quotient
    of <dO, O> (the definition of the derivative)."""
    w = sg.Workload("b", (2, 4, 4), "raster", 2, 1, (3, 3, 3), (1, 2, 2), "f32", "softmax",
                    21).with_(summary_mode=mode)
    inp, x = _inputs(w)
    dout = np.random.default_rng(5).standard_normal((w.n_tokens, w.n_q_heads, 64))
    g = _bwd(w, x, dout)
    assert _fd_check(w, x, dout, g) <= 1e-7


def test_variant_fd_check_detects_token_gradients():
    """Negative control: the exact form's gradients (rotation by R(c_u)) do
    not pass the centre variant's finite-difference pin, nor does the
    rotated-query dq pass the blind variant's."""
    w = sg.Workload("b", (2, 4, 4), "raster", 2, 1, (3, 3, 3), (1, 2, 2), "f32", "softmax", 21)
    inp, x = _inputs(w)
    dout = np.random.default_rng(5).standard_normal((w.n_tokens, w.n_q_heads, 64))
    tok = _bwd(w, x, dout)
    assert _fd_check(w.with_(summary_mode="centre"), x, dout, tok, probes=6) > 1e-3
    assert _fd_check(w.with_(summary_mode="blind"), x, dout, tok, probes=6) > 1e-3


def test_unknown_mode_is_rejected():
    w = _small()
    inp = sg.make_inputs(w)
    with pytest.raises(ValueError):
        orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block,
                            mode="center-of-mass")
    assert math.isclose(orc.block_centres((1, 4, 4), (1, 4, 4))[0, 1], 1.5)
