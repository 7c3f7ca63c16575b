"""GPU parity of the backward: pack3d_forward_train + pack3d_backward against
the fp64 oracle's gradients (oracle/, pinned in test_oracle_bwd_pins.py).

Small lattices are compared in full; the 262 144-token workload on sampled
query rows and keys, plus identities that hold at any size for the summary
gradients.  Tolerance (bf16 tensors, fp32 accumulation): the largest error of
each gradient tensor is at most 2e-2 of its largest magnitude.  Every bf16
operand (rotated q/k, p, ds, the branch upstream gradients) and every bf16
output carries a relative rounding error <= 2^-9; sums of such terms keep
that relative size, so 2e-2 leaves a margin of ~10x while a dropped term,
wrong sign or wrong index shows up at order 1.
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


def _w(name, grid, hq, hkv, window=(3, 7, 7), block=(1, 4, 4), packing="random", seed=5):
    return sg.Workload(name, grid, packing, hq, hkv, window, block, "bf16", "softmax", seed)


C5 = _w("c5_262k", (64, 64, 64), 8, 2, packing="block")
C5_SMALL = _w("c5_4x16x16", (4, 16, 16), 8, 2, packing="block")
CASES = [
    C5_SMALL,
    _w("ragged_g4", (3, 12, 20), 8, 2),
    _w("g8", (3, 12, 12), 8, 1, seed=6),
    _w("g16_morton", (3, 4, 12), 16, 1, packing="morton", seed=7),
    _w("deep_window", (9, 12, 8), 8, 2, window=(7, 3, 5), packing="morton", seed=8),
    _w("window_1", (2, 8, 8), 4, 1, window=(1, 1, 1), packing="raster", seed=9),
    _w("window_3x3x5", (4, 8, 16), 4, 1, window=(3, 3, 5), block=(2, 2, 4), seed=10),
    # 5 040 tokens: the summary-gradient query stream splits into two slices
    # of 2 520 cells (157.5 tiles: a ragged last tile, then padding to whole
    # copy phases); 315 summaries leave a ragged summary tile in both
    # summary-gradient kernels
    _w("multi_slice", (5, 28, 36), 8, 2, seed=14),
    # degenerate lattices: one token (N = M = 1), one summary for the whole
    # lattice (block volume 64), a single row of cells
    _w("single_cell", (1, 1, 1), 4, 1, block=(1, 1, 1), seed=11),
    _w("one_summary", (2, 4, 8), 8, 2, block=(2, 4, 8), seed=12),
    _w("one_row", (1, 1, 24), 16, 1, block=(1, 1, 4), seed=13),
]


@pytest.fixture(scope="module")
def pk():
    from geometry_aware_local_amd import pack3d
    return pack3d


def _say(*a):
    print(*a, flush=True)


def _gate(w, inp, per_head):
    if not per_head:
        return inp.gate
    return np.random.default_rng(w.seed + 3).standard_normal(
        (w.n_tokens, w.n_q_heads, 2)).astype(np.float32)


def _gpu(pk, w, inp, dout, gate):
    d = gu.device_inputs(inp)
    d["gate"] = gu.dev(gate)
    prob = gu.problem(pk, w, gate_per_head=gate.ndim == 3)
    out, saved = pk.pack3d_forward_train(prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"],
                                         d["v_cmp"], d["a"], d["coords"], d["cell_to_pos"],
                                         d["gate"])
    g = pk.pack3d_backward(prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"], d["a"],
                           d["coords"], d["cell_to_pos"], d["gate"], saved,
                           gu.dev(dout, torch.bfloat16))
    torch.cuda.synchronize()
    return prob, d, out, saved, g


def _rel(got, ref):
    # a gradient that is exactly zero (e.g. dk_loc with a 1x1x1 window:
    # softmax over one key has no key gradient) is held to a 1e-2 scale
    return gu.max_abs(got, ref) / max(float(np.abs(ref).max()), 1e-2)


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_backward_small(pk, w):
    _say("backward", w.name)
    inp = sg.make_inputs(w)
    dout = sg.make_upstream_grad(inp)
    prob, d, out, saved, g = _gpu(pk, w, inp, dout, inp.gate)
    ref = orc.backward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a, inp.coords,
                       inp.gate, dout)
    errs = {n: _rel(gu.host(g[n]), ref[n]) for n in NAMES}
    _say("  rel errors", {k: f"{v:.2e}" for k, v in errs.items()})
    _say("  abs errors", {n: f"{gu.max_abs(gu.host(g[n]), ref[n]):.2e}" for n in NAMES},
         "max |ref|", {n: f"{np.abs(ref[n]).max():.2e}" for n in NAMES})
    for n in NAMES:
        assert errs[n] <= GRAD_TOL, n
    # the training forward: same output as the forward, saved state = the
    # oracle's.  End to end the oracle rotates in fp64 while the GPU stores
    # the rotated q, k (and the scaled summaries) in bf16: each logit moves
    # by up to ~2^-8 of |tau q||k|, which shifts lse by the p-weighted mean
    # of those moves; 2^-6 bounds it here (the split-entry tests compare lse
    # on rounded inputs to 2^-8).
    f = ref["fwd"]
    assert gu.max_abs(gu.host(out), f["out"]) <= gu.ABS_TOL["bf16"]
    sv = pk.saved_views(prob, saved)
    assert _rel(gu.host(sv["o_loc"]), f["o_loc"]) <= GRAD_TOL
    assert _rel(gu.host(sv["o_cmp"]), f["o_cmp"]) <= GRAD_TOL
    assert gu.max_abs(gu.host(sv["lse_loc"]), f["lse_loc"]) <= 2.0 ** -6
    assert gu.max_abs(gu.host(sv["lse_cmp"]), f["lse_cmp"]) <= 2.0 ** -6
    plain = pk.pack3d_forward(prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"],
                              d["a"], d["coords"], d["cell_to_pos"], d["gate"])
    assert gu.max_abs(gu.host(plain), gu.host(out)) <= gu.ABS_TOL["bf16"]


def test_backward_gate_per_head(pk):
    w = CASES[1]
    _say("backward, one gate per head", w.name)
    inp = sg.make_inputs(w)
    dout = sg.make_upstream_grad(inp)
    gate = _gate(w, inp, True)
    _, _, _, _, g = _gpu(pk, w, inp, dout, gate)
    ref = orc.backward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a, inp.coords,
                       gate, dout)
    for n in NAMES:
        assert _rel(gu.host(g[n]), ref[n]) <= GRAD_TOL, n


def test_backward_is_packing_equivariant_bitwise(pk):
    """Repacking the inputs permutes every gradient bit for bit (all sums
    run in coordinate order)."""
    w = C5_SMALL
    inp = sg.make_inputs(w)
    res = {}
    for kind in ("block", "raster", "random", "morton", "block_morton"):
        x = inp.repacked(kind) if kind != w.packing else inp
        dout = sg.make_upstream_grad(x)
        _say("backward equivariance", kind)
        _, _, _, _, g = _gpu(pk, x.workload, x, dout, x.gate)
        res[kind] = (x, {n: g[n].float().cpu().numpy() for n in NAMES})
    base_inp, base = res["block"]
    for kind, (x, got) in res.items():
        src = base_inp.cell_to_pos[x.order]
        for n in NAMES:
            assert np.array_equal(got[n], base[n][src]), (kind, n)


def test_backward_deterministic(pk):
    w = CASES[2]
    inp = sg.make_inputs(w)
    dout = sg.make_upstream_grad(inp)
    _, _, _, _, g1 = _gpu(pk, w, inp, dout, inp.gate)
    _, _, _, _, g2 = _gpu(pk, w, inp, dout, inp.gate)
    for n in NAMES:
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("w", [C5_SMALL, CASES[1], CASES[3], CASES[5]], ids=lambda w: w.name)
def test_training_forward_output_is_the_forward_bitwise(pk, w):
    """The training forward mixes the gate in the same epilogue as the
    inference forward, so both give the same O bit for bit; its saved o_cmp
    and lse are those of the compressed branch (checked against the oracle
    through the backward tests)."""
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    args = (prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"], d["a"], d["coords"],
            d["cell_to_pos"], d["gate"])
    out_train, _ = pk.pack3d_forward_train(*args)
    out = pk.pack3d_forward(*args)
    torch.cuda.synchronize()
    assert torch.equal(out_train, out)


def test_backward_262k_sampled(pk):
    """The backward workload at full size: dq and dgate on sampled tokens,
    dk_loc / dv_loc on sampled keys (their whole windows computed by the
    oracle), and the summary-path gradients through identities that hold at
    any size."""
    w = C5
    _say("backward", w.name)
    inp = sg.make_inputs(w)
    dout = sg.make_upstream_grad(inp)
    _, _, _, _, g = _gpu(pk, w, inp, dout, inp.gate)
    got = {n: gu.host(g[n]) for n in NAMES}
    tau = 0.125
    rng = np.random.default_rng(17)
    # --- sampled query rows: dq, dgate
    rows = np.sort(rng.choice(w.n_tokens, 192, replace=False))
    f = orc.forward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a, inp.coords,
                    inp.gate, rows=rows)
    dg, d_loc, d_cmp = orc.gate_backward(inp.gate[rows], dout[rows], f["o_loc"], f["o_cmp"])
    dq_l, _, _ = orc.local_attention_backward(f["q_rot"], f["k_rot"], inp.v_loc, inp.coords,
                                              w.grid, w.window, tau, d_loc, rows,
                                              q_is_rows=True)
    dq_c, _, _ = orc.global_attention_backward(f["q_rot"], f["k_sum"], f["v_sum"], tau, d_cmp)
    dq = orc.rotate_transpose(dq_l + dq_c, inp.coords[rows], w.rope_pairs, w.rope_base)
    _say(f"  dq abs {gu.max_abs(got['dq'][rows], dq):.2e} (max |ref| {np.abs(dq).max():.2e}), "
         f"dgate abs {gu.max_abs(got['dgate'][rows], dg):.2e} (max |ref| {np.abs(dg).max():.2e})")
    assert _rel(got["dq"][rows], dq) <= GRAD_TOL
    assert _rel(got["dgate"][rows], dg) <= GRAD_TOL
    # --- sampled keys: every query of each key's window
    keys = rng.choice(w.n_tokens, 6, replace=False)
    r = np.array(w.window) // 2
    near = np.unique(np.concatenate([
        np.nonzero(np.all(np.abs(inp.coords - inp.coords[k]) <= r, axis=1))[0] for k in keys]))
    f2 = orc.forward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a, inp.coords,
                     inp.gate, rows=near)
    _, d_loc2, _ = orc.gate_backward(inp.gate[near], dout[near], f2["o_loc"], f2["o_cmp"])
    _, dk_r, dv = orc.local_attention_backward(f2["q_rot"], f2["k_rot"], inp.v_loc, inp.coords,
                                               w.grid, w.window, tau, d_loc2, near,
                                               q_is_rows=True)
    dk = orc.rotate_transpose(dk_r[keys], inp.coords[keys], w.rope_pairs, w.rope_base)
    _say(f"  dk_loc abs {gu.max_abs(got['dk_loc'][keys], dk):.2e} "
         f"(max |ref| {np.abs(dk).max():.2e}), dv_loc abs "
         f"{gu.max_abs(got['dv_loc'][keys], dv[keys]):.2e} (max |ref| {np.abs(dv[keys]).max():.2e})")
    assert _rel(got["dk_loc"][keys], dk) <= GRAD_TOL
    assert _rel(got["dv_loc"][keys], dv[keys]) <= GRAD_TOL
    # --- summary path, at any size: sum_u dv_cmp[u, g] = sum over the
    # group's heads of g_cmp * dO (softmax rows sum to one, weights per block
    # sum to one), and sum_u R(c_u) dk_cmp[u, g] = 0 (gradient rows of a
    # softmax sum to zero)
    # The branch gradient g_cmp * dO enters the kernels rounded to bf16; over
    # a million query rows those roundings alone move the sum by ~1, so the
    # identity is taken with the rounded values (as an input, not a result).
    gw = orc.gate_weights(inp.gate)
    grp = w.n_q_heads // w.n_kv_heads
    dco = sg.round_to_bf16((gw[:, 1, None, None] * dout).astype(np.float32)).astype(np.float64)
    want_v = dco.reshape(w.n_tokens, w.n_kv_heads, grp, 64).sum(axis=(0, 2))
    sum_v = got["dv_cmp"].sum(axis=0)
    scale_v = np.sqrt((got["dv_cmp"] ** 2).sum(axis=0)).max()
    assert np.abs(sum_v - want_v).max() <= GRAD_TOL * scale_v + 1e-4 * np.abs(want_v).max()
    rk = orc.rotate(got["dk_cmp"], inp.coords, w.rope_pairs, w.rope_base)
    scale_k = np.sqrt((rk ** 2).sum(axis=0)).max()
    assert np.abs(rk.sum(axis=0)).max() <= GRAD_TOL * scale_k
    # and the gate gradient of every token cancels
    assert np.abs(got["dgate"].sum(axis=1)).max() <= 1e-6
