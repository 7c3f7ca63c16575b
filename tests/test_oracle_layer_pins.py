"""Pins of the oracle's layer around the operator ("Geometry Matters in Packed
3D Attention": papernotes.org notes, flowchart node B - linear projection
and layer normalisation produce Q, K_loc, V_loc, K_cmp, V_cmp - node G -
residual output - and key design 1, which writes every projection as
W LN(h)).

LayerNorm and the linear maps are checked against library routines
(torch.nn.functional.layer_norm / linear in float64 on the CPU), the split
order of the stacked projection weight by a closed form, the residual by a
zero output projection, and the whole block by packing equivariance.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synthgen as sg
from oracle import pack3d_oracle as orc


def _w(grid=(2, 8, 8), hq=4, hkv=2, packing="random", dtype="f32", seed=41):
    return sg.Workload("layer", grid, packing, hq, hkv, (3, 5, 5), (1, 4, 4), dtype, "softmax",
                       seed)


def _t(x):
    return torch.from_numpy(np.asarray(x, np.float64))


def test_layer_norm_is_the_library_layer_norm():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((37, 96)) * 3 + 1.5
    g, b = 1 + 0.2 * rng.standard_normal(96), 0.3 * rng.standard_normal(96)
    want = F.layer_norm(_t(h), (96,), _t(g), _t(b), eps=1e-5).numpy()
    assert np.abs(orc.layer_norm(h, g, b) - want).max() <= 1e-12
    plain = F.layer_norm(_t(h), (96,), eps=1e-5).numpy()
    assert np.abs(orc.layer_norm(h, None, None) - plain).max() <= 1e-12


def test_projection_split_order():
    """Rows of the stacked weight map to Q, K_loc, V_loc, K_cmp, V_cmp in that
    order: with W = the identity on a width that equals the stacked output,
    each output is its own slice of the input."""
    hq, hkv, d = 4, 2, 64
    cout = (hq + 4 * hkv) * d
    x = np.random.default_rng(2).standard_normal((5, cout))
    q, kl, vl, kc, vc = orc.qkv_projection(x, np.eye(cout), hq, hkv)
    off = [0, hq * d, (hq + hkv) * d, (hq + 2 * hkv) * d, (hq + 3 * hkv) * d, cout]
    for i, t in enumerate((q, kl, vl, kc, vc)):
        assert np.array_equal(t.reshape(5, -1), x[:, off[i]:off[i + 1]])
    assert q.shape == (5, hq, d) and vc.shape == (5, hkv, d)
    # and a general weight is the library's linear map
    w = np.random.default_rng(3).standard_normal((cout, 96))
    x2 = np.random.default_rng(4).standard_normal((7, 96))
    got = np.concatenate([t.reshape(7, -1) for t in orc.qkv_projection(x2, w, hq, hkv)], 1)
    assert np.abs(got - F.linear(_t(x2), _t(w)).numpy()).max() <= 1e-12
    with pytest.raises(ValueError):
        orc.qkv_projection(x2, w[:-64], hq, hkv)


def test_layer_is_the_library_composition():
    """h + linear(operator(linear(layer_norm(h))), W_O) with torch's
    layer_norm and linear (the operator itself is pinned elsewhere)."""
    w = _w()
    inp = sg.make_inputs(w)
    L = sg.make_layer_inputs(inp)
    r = orc.layer_forward(w, L.h, L.gamma, L.beta, L.w_qkv, L.w_o, inp.a, inp.coords, inp.gate)
    x = F.layer_norm(_t(L.h), (L.h.shape[1],), _t(L.gamma), _t(L.beta), eps=1e-5)
    y = F.linear(x, _t(L.w_qkv)).numpy()
    n, d = w.n_tokens, 64
    hq, hkv = w.n_q_heads, w.n_kv_heads
    parts = np.split(y, np.cumsum([hq * d] + [hkv * d] * 3), axis=1)
    q, kl, vl, kc, vc = [p.reshape(n, -1, d) for p in parts]
    f = orc.forward(w, q, kl, vl, kc, vc, inp.a, inp.coords, inp.gate)
    want = (_t(L.h) + F.linear(_t(f["out"].reshape(n, -1)), _t(L.w_o))).numpy()
    assert np.abs(r["out"] - want).max() <= 1e-11


def test_zero_output_projection_returns_the_residual():
    w = _w()
    inp = sg.make_inputs(w)
    L = sg.make_layer_inputs(inp)
    r = orc.layer_forward(w, L.h, L.gamma, L.beta, L.w_qkv, np.zeros_like(L.w_o), inp.a,
                          inp.coords, inp.gate)
    assert np.array_equal(r["out"], L.h.astype(np.float64))


def test_layer_is_packing_equivariant_and_rows_agree():
    """Proposition 1 for the whole block (LayerNorm and the projections act
    per token), and sampled rows equal the full result's rows."""
    w = _w(packing="raster")
    base = sg.make_inputs(w)
    L = sg.make_layer_inputs(base)
    ref = orc.layer_forward(w, L.h, L.gamma, L.beta, L.w_qkv, L.w_o, base.a, base.coords,
                            base.gate)["out"]
    for kind in ("morton", "random"):
        inp = base.repacked(kind)
        h = L.h[base.cell_to_pos[inp.order]]
        got = orc.layer_forward(w, h, L.gamma, L.beta, L.w_qkv, L.w_o, inp.a, inp.coords,
                                inp.gate)["out"]
        back = inp.cell_to_pos[base.order]
        assert np.abs(got[back] - ref).max() <= 1e-12, kind
    rows = np.array([0, 5, 17, 100])
    sub = orc.layer_forward(w, L.h, L.gamma, L.beta, L.w_qkv, L.w_o, base.a, base.coords,
                            base.gate, rows=rows)["out"]
    assert np.abs(sub - ref[rows]).max() <= 1e-12


def test_layer_inputs_recipe():
    """Seeded, per-cell hidden states (repacking permutes them), bf16-exact
    values for bf16 workloads, and projections of unit scale."""
    w = _w(dtype="bf16", packing="raster")
    base = sg.make_inputs(w)
    L = sg.make_layer_inputs(base)
    inp = base.repacked("morton")
    L2 = sg.make_layer_inputs(inp)
    assert np.array_equal(L2.h, L.h[base.cell_to_pos[inp.order]])
    for t in (L.h, L.w_qkv, L.w_o):
        assert np.array_equal(sg.round_to_bf16(t), t)
    x = orc.layer_norm(L.h, L.gamma, L.beta)
    q = orc.qkv_projection(x, L.w_qkv, w.n_q_heads, w.n_kv_heads)[0]
    assert 0.7 < q.std() < 1.4
