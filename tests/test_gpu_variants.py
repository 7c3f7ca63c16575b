"""GPU parity of the compressed-branch variants ("centre": pooled unrotated
keys rotated once at the block centre; "blind": no rotation in the compressed
branch) against the fp64 oracle (pinned in test_oracle_variant_pins.py):
block summaries, the forward (fused and split), the training forward's saved
state, the backward, and packing equivariance.  Same tolerances as the exact
form's tests.
"""

import numpy as np
import pytest
import torch

import synthgen as sg
from oracle import pack3d_oracle as orc
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

GRAD_TOL = 2e-2
NAMES = ("dq", "dk_loc", "dv_loc", "dk_cmp", "dv_cmp", "dgate")
MODES = ("centre", "blind")


def _w(name, grid, hq, hkv, dtype, window=(3, 7, 7), block=(1, 4, 4), packing="random", seed=31):
    return sg.Workload(name, grid, packing, hq, hkv, window, block, dtype, "softmax", seed)


# even and odd block extents (half-integer and integer centres), ragged tiles,
# both dtypes
FWD = [
    _w("f32_ragged", (3, 12, 20), 4, 1, "f32"),
    _w("bf16_ragged", (3, 12, 20), 8, 2, "bf16"),
    _w("bf16_block_2x3x4", (4, 6, 16), 4, 1, "bf16", window=(3, 3, 5), block=(2, 3, 4),
       packing="morton"),
    _w("f32_block_3x3x2", (3, 9, 8), 2, 2, "f32", block=(3, 3, 2)),
]
BWD = [
    _w("c5_4x16x16", (4, 16, 16), 8, 2, "bf16", packing="block", seed=5),
    _w("bwd_block_2x3x4", (4, 6, 16), 4, 1, "bf16", window=(3, 3, 5), block=(2, 3, 4)),
    _w("bwd_g16", (3, 4, 12), 16, 1, "bf16", packing="morton"),
]


def _cases(ws):
    return [w.with_(summary_mode=m) for m in MODES for w in ws]


def _ids(ws):
    return [f"{m}-{w.name}" for m in MODES for w in ws]


@pytest.fixture(scope="module")
def pk():
    from geometry_aware_local_amd import pack3d
    return pack3d


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("w", _cases(FWD), ids=_ids(FWD))
def test_variant_block_summary(pk, w):
    _say("block_summary", w.summary_mode, w.name)
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    ks, vs = pk.pack3d_block_summary(gu.problem(pk, w), d["k_cmp"], d["v_cmp"], d["a"],
                                     d["cell_to_pos"])
    rk, rv = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block,
                                 w.rope_pairs, w.rope_base, mode=w.summary_mode)
    for got, ref in ((gu.host(ks), rk), (gu.host(vs), rv)):
        if w.dtype == "f32":
            assert gu.max_abs(got, ref) <= 1e-5
        else:
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


@pytest.mark.parametrize("w", _cases(FWD), ids=_ids(FWD))
def test_variant_forward(pk, w):
    _say("forward", w.summary_mode, w.name)
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    args = (prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"], d["a"], d["coords"],
            d["cell_to_pos"], d["gate"])
    out = pk.pack3d_forward(*args)
    # split chain: the compressed branch's query is rotated unless blind
    q_rot = pk.pack3d_rope(prob, d["q"], d["coords"])
    q_cmp = d["q"] if w.summary_mode == "blind" else q_rot
    ks, vs = pk.pack3d_block_summary(prob, d["k_cmp"], d["v_cmp"], d["a"], d["cell_to_pos"])
    o_cmp = pk.pack3d_global_attn(prob, q_cmp, ks, vs)
    torch.cuda.synchronize()
    ref = orc.forward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a, inp.coords,
                      inp.gate)
    assert gu.max_abs(gu.host(out), ref["out"]) <= gu.ABS_TOL[w.dtype]
    assert gu.max_rel(gu.host(o_cmp), ref["o_cmp"]) <= gu.REL_TOL[w.dtype]
    # the variants differ from the exact form (the test can tell them apart)
    exact = orc.forward(w.with_(summary_mode="token"), inp.q, inp.k_loc, inp.v_loc, inp.k_cmp,
                        inp.v_cmp, inp.a, inp.coords, inp.gate)
    assert gu.max_rel(exact["o_cmp"], ref["o_cmp"]) > 10 * gu.REL_TOL[w.dtype]


@pytest.mark.parametrize("mode", MODES)
def test_variant_forward_262k_sampled(pk, mode):
    w = sg.WORKLOADS["block_bf16_64x64x64"].with_(summary_mode=mode)
    _say("forward 262k", mode)
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    out = pk.pack3d_forward(gu.problem(pk, w), d["q"], d["k_loc"], d["v_loc"], d["k_cmp"],
                            d["v_cmp"], d["a"], d["coords"], d["cell_to_pos"], d["gate"])
    rows = np.sort(np.random.default_rng(12).choice(w.n_tokens, 512, replace=False))
    ref = orc.forward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a, inp.coords,
                      inp.gate, rows=rows)
    assert gu.max_abs(gu.host(out)[rows], ref["out"]) <= gu.ABS_TOL["bf16"]


def _train(pk, w, inp, dout):
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    args = (prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"], d["a"], d["coords"],
            d["cell_to_pos"], d["gate"])
    out, saved = pk.pack3d_forward_train(*args)
    g = pk.pack3d_backward(*args, saved, gu.dev(dout, torch.bfloat16))
    torch.cuda.synchronize()
    return prob, out, saved, g


def _rel(got, ref):
    return gu.max_abs(got, ref) / max(float(np.abs(ref).max()), 1e-2)


@pytest.mark.parametrize("w", _cases(BWD), ids=_ids(BWD))
def test_variant_backward(pk, w):
    _say("backward", w.summary_mode, w.name)
    inp = sg.make_inputs(w)
    dout = sg.make_upstream_grad(inp)
    prob, out, saved, g = _train(pk, w, inp, dout)
    ref = orc.backward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a, inp.coords,
                       inp.gate, dout)
    errs = {n: _rel(gu.host(g[n]), ref[n]) for n in NAMES}
    _say("  rel errors", {k: f"{v:.2e}" for k, v in errs.items()})
    for n in NAMES:
        assert errs[n] <= GRAD_TOL, n
    f = ref["fwd"]
    assert gu.max_abs(gu.host(out), f["out"]) <= gu.ABS_TOL["bf16"]
    sv = pk.saved_views(prob, saved)
    assert _rel(gu.host(sv["o_cmp"]), f["o_cmp"]) <= GRAD_TOL
    assert gu.max_abs(gu.host(sv["lse_cmp"]), f["lse_cmp"]) <= 2.0 ** -6


@pytest.mark.parametrize("mode", MODES)
def test_variant_packing_equivariance_bitwise(pk, mode):
    """Repacking permutes the forward's output and every gradient bit for bit."""
    w = BWD[0].with_(summary_mode=mode)
    inp = sg.make_inputs(w)
    res = {}
    for kind in ("block", "raster", "random", "morton"):
        x = inp.repacked(kind) if kind != w.packing else inp
        _say("equivariance", mode, kind)
        _, out, _, g = _train(pk, x.workload, x, sg.make_upstream_grad(x))
        res[kind] = (x, out.float().cpu().numpy(),
                     {n: g[n].float().cpu().numpy() for n in NAMES})
    base_inp, base_out, base = res["block"]
    for kind, (x, out, got) in res.items():
        src = base_inp.cell_to_pos[x.order]
        assert np.array_equal(out, base_out[src]), kind
        for n in NAMES:
            assert np.array_equal(got[n], base[n][src]), (kind, n)
