"""GPU parity of the layer around the operator (LayerNorm + the five
projections with RoPE fused into the projection's epilogue; the output
projection + residual; the whole layer) against the fp64 oracle (pinned in
test_oracle_layer_pins.py).

Tolerances (bf16 tensors, fp32 accumulation): each projection output within
1e-2 of its largest magnitude (LayerNorm's output and every product operand
are bf16, relative rounding <= 2^-9 each, and the output is rounded once);
the LayerNorm output itself to one bf16 rounding (fp32 arithmetic on
bf16-exact inputs).  The
whole layer: the output projection is scaled up by 16 (exact in bf16) so the
attention part is of the same size as the residual, and the layer's update
out - h is held to 2e-2 of its largest magnitude plus the output's own bf16
rounding.
"""

import numpy as np
import pytest
import torch

import synthgen as sg
from oracle import pack3d_oracle as orc
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

BF = torch.bfloat16


def _w(name, grid, hq, hkv, window=(3, 7, 7), block=(1, 4, 4), packing="random", seed=51,
       mode="token"):
    return sg.Workload(name, grid, packing, hq, hkv, window, block, "bf16", "softmax", seed,
                       summary_mode=mode)


CASES = [
    (_w("ragged_g4", (3, 12, 20), 8, 2), None),
    (_w("g8_width384", (3, 12, 12), 8, 1, seed=52), 384),
    (_w("g16_width1024", (2, 8, 12), 16, 1, packing="morton", seed=53), 1024),
    (_w("g4_centre", (4, 8, 16), 4, 1, block=(2, 2, 4), seed=54, mode="centre"), 256),
    (_w("g4_blind", (4, 8, 16), 4, 1, seed=55, mode="blind"), None),
]
IDS = [c[0].name for c in CASES]


@pytest.fixture(scope="module")
def pk():
    from geometry_aware_local_amd import pack3d
    return pack3d


def _say(*a):
    print(*a, flush=True)


def _dev_layer(L, w_o_scale=1.0):
    return dict(h=gu.dev(L.h, BF), gamma=gu.dev(L.gamma), beta=gu.dev(L.beta),
                w_qkv=gu.dev(L.w_qkv, BF), w_o=gu.dev(L.w_o * w_o_scale, BF))


def _rel(got, ref):
    return gu.max_abs(got, ref) / float(np.abs(ref).max())


@pytest.mark.parametrize("w,width", CASES, ids=IDS)
def test_layernorm_qkv(pk, w, width):
    _say("layernorm_qkv", w.name, width)
    inp = sg.make_inputs(w)
    L = sg.make_layer_inputs(inp, width)
    d = _dev_layer(L)
    prob = gu.problem(pk, w)
    g = pk.pack3d_layernorm_qkv(prob, d["h"], d["gamma"], d["beta"], d["w_qkv"],
                                gu.dev(inp.coords), with_q_raw=True)
    torch.cuda.synchronize()
    x = orc.layer_norm(L.h, L.gamma, L.beta)
    q, kl, vl, kc, vc = orc.qkv_projection(x, L.w_qkv, w.n_q_heads, w.n_kv_heads)
    # LayerNorm in fp32 on bf16-exact inputs, one bf16 rounding
    xn = gu.host(g["x_norm"])
    assert np.all(np.abs(xn - x) <= 2.0 ** -8 * np.abs(x) + 1e-5)
    refs = dict(q_rot=orc.rotate(q, inp.coords), k_rot=orc.rotate(kl, inp.coords), v_loc=vl,
                k_cmp=kc, v_cmp=vc, q_raw=q)
    for name, ref in refs.items():
        err = _rel(gu.host(g[name]), ref)
        _say(f"  {name} {err:.2e}")
        assert err <= 1e-2, name


def test_out_proj(pk):
    w = CASES[0][0]
    _say("out_proj", w.name)
    rng = np.random.default_rng(9)
    n, hq = w.n_tokens, w.n_q_heads
    for width in (512, 320):
        o = sg.round_to_bf16(rng.standard_normal((n, hq * 64), dtype=np.float32))
        w_o = sg.round_to_bf16((rng.standard_normal((width, hq * 64)) / 16).astype(np.float32))
        res = sg.round_to_bf16(rng.standard_normal((n, width), dtype=np.float32))
        prob = gu.problem(pk, w)
        got = gu.host(pk.pack3d_out_proj(prob, gu.dev(o, BF), gu.dev(w_o, BF), gu.dev(res, BF)))
        upd = o.astype(np.float64) @ w_o.astype(np.float64).T
        ref = res + upd
        # accumulation in fp32, one bf16 rounding of the sum
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-3 * np.abs(upd).max())


def _layer(pk, w, inp, L, scale=16.0):
    d = _dev_layer(L, scale)
    dv = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    out = pk.pack3d_layer_forward(prob, d["h"], d["gamma"], d["beta"], d["w_qkv"], d["w_o"],
                                  dv["a"], dv["coords"], dv["cell_to_pos"], dv["gate"])
    torch.cuda.synchronize()
    return out


def _check_layer(got, ref, h):
    upd_ref = ref - h
    err = np.abs((got - h) - upd_ref)
    bound = 2e-2 * np.abs(upd_ref).max() + 2.0 ** -8 * np.abs(ref)
    _say(f"  layer update error {(err / np.abs(upd_ref).max()).max():.2e} of max |update|")
    assert np.all(err <= bound)


@pytest.mark.parametrize("w,width", CASES, ids=IDS)
def test_layer_forward(pk, w, width):
    _say("layer_forward", w.name, width)
    inp = sg.make_inputs(w)
    L = sg.make_layer_inputs(inp, width)
    got = gu.host(_layer(pk, w, inp, L))
    ref = orc.layer_forward(w, L.h, L.gamma, L.beta, L.w_qkv, L.w_o * 16.0, inp.a, inp.coords,
                            inp.gate)["out"]
    _check_layer(got, ref, L.h.astype(np.float64))


def test_layer_forward_262k_sampled(pk):
    w = sg.WORKLOADS["block_bf16_64x64x64"]
    _say("layer_forward", w.name)
    inp = sg.make_inputs(w)
    L = sg.make_layer_inputs(inp)
    got = gu.host(_layer(pk, w, inp, L))
    rows = np.sort(np.random.default_rng(14).choice(w.n_tokens, 512, replace=False))
    ref = orc.layer_forward(w, L.h, L.gamma, L.beta, L.w_qkv, L.w_o * 16.0, inp.a, inp.coords,
                            inp.gate, rows=rows)["out"]
    _check_layer(got[rows], ref, L.h[rows].astype(np.float64))


def test_layer_is_packing_equivariant_bitwise(pk):
    w = CASES[0][0].with_(packing="raster")
    base = sg.make_inputs(w)
    L = sg.make_layer_inputs(base)
    ref = _layer(pk, w, base, L).float().cpu().numpy()
    for kind in ("block", "morton", "block_morton", "random"):
        inp = base.repacked(kind)
        L2 = sg.make_layer_inputs(inp)
        got = _layer(pk, inp.workload, inp, L2).float().cpu().numpy()
        back = inp.cell_to_pos[base.order]
        assert np.array_equal(got[back], ref), kind
