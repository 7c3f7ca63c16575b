"""Pins of the fp64 oracle's backward against what mathematics fixes.

The pages print no backward: the gradients are the derivatives of the
forward ("Geometry Matters in Packed 3D Attention"; papernotes.org notes, key
designs 1-3 and the flowchart define the forward).  They are pinned here by
the definition of a derivative (central finite differences of the oracle's
forward), by a library routine (torch autograd through float64
scaled_dot_product_attention on the CPU), and by identities every gradient
of a softmax attention obeys at any size.  None of these re-types the
oracle's backward formulas.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synthgen as sg
from oracle import pack3d_oracle as orc

PAIRS, BASE = (11, 11, 10), 10000.0


def _w(grid=(2, 4, 4), hq=2, hkv=1, window=(3, 3, 3), block=(1, 2, 2), packing="raster",
       weights="softmax", seed=21):
    return sg.Workload("b", grid, packing, hq, hkv, window, block, "f32", weights, seed)


def _inputs(w, gate_per_head=False):
    inp = sg.make_inputs(w, explicit_uniform=True)
    f64 = lambda t: None if t is None else np.asarray(t, np.float64)
    x = dict(q=f64(inp.q), k_loc=f64(inp.k_loc), v_loc=f64(inp.v_loc), k_cmp=f64(inp.k_cmp),
             v_cmp=f64(inp.v_cmp), a=f64(inp.a), coords=inp.coords, gate=f64(inp.gate))
    if gate_per_head:
        rng = np.random.default_rng(w.seed + 7)
        x["gate"] = rng.standard_normal((w.n_tokens, w.n_q_heads, 2))
    return inp, x


def _out(w, x):
    return orc.forward(w, x["q"], x["k_loc"], x["v_loc"], x["k_cmp"], x["v_cmp"], x["a"],
                       x["coords"], x["gate"])["out"]


def _bwd(w, x, dout):
    return orc.backward(w, x["q"], x["k_loc"], x["v_loc"], x["k_cmp"], x["v_cmp"], x["a"],
                        x["coords"], x["gate"], dout)


GRADS = [("q", "dq"), ("k_loc", "dk_loc"), ("v_loc", "dv_loc"), ("k_cmp", "dk_cmp"),
         ("v_cmp", "dv_cmp"), ("gate", "dgate")]


def _fd_check(w, x, dout, g, probes=10, eps=1e-5, seed=0):
    """Central differences of L = <dout, out> at random entries of every input."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for name, gname in GRADS:
        arr = x[name]
        for _ in range(probes):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            keep = arr[idx]
            arr[idx] = keep + eps
            lp = float((dout * _out(w, x)).sum())
            arr[idx] = keep - eps
            lm = float((dout * _out(w, x)).sum())
            arr[idx] = keep
            fd = (lp - lm) / (2 * eps)
            worst = max(worst, abs(fd - g[gname][idx]))
    return worst


@pytest.mark.parametrize("gate_per_head", [False, True], ids=["gate_token", "gate_head"])
def test_backward_matches_finite_differences(gate_per_head):
    """Every gradient equals the central difference quotient of <dO, O>
    (truncation ~eps^2, rounding ~1e-16/eps: both far below 1e-7)."""
    w = _w()
    inp, x = _inputs(w, gate_per_head)
    dout = np.random.default_rng(5).standard_normal((w.n_tokens, w.n_q_heads, 64))
    g = _bwd(w, x, dout)
    assert _fd_check(w, x, dout, g) <= 1e-7


def test_fd_check_detects_planted_mistakes(monkeypatch):
    """Negative controls: a transposed inverse rotation (R instead of R^T)
    or swapped gate branches must fail the finite-difference pin."""
    w = _w()
    inp, x = _inputs(w)
    dout = np.random.default_rng(5).standard_normal((w.n_tokens, w.n_q_heads, 64))
    good = _bwd(w, x, dout)
    assert _fd_check(w, x, dout, good, probes=4) <= 1e-7
    with monkeypatch.context() as mp:
        mp.setattr(orc, "rotate_transpose", orc.rotate)
        bad = _bwd(w, x, dout)
    assert _fd_check(w, x, dout, bad, probes=6) > 1e-3
    real = orc.gate_backward
    with monkeypatch.context() as mp:
        def swapped(*a, **k):
            dg, dl, dc = real(*a, **k)
            return dg, dc, dl
        mp.setattr(orc, "gate_backward", swapped)
        bad = _bwd(w, x, dout)
    assert _fd_check(w, x, dout, bad, probes=6) > 1e-3


def _sdpa_grads(q, k, v, dout, mask=None, scale=0.125):
    """torch autograd through float64 SDPA: q [N,Hq,D], k/v [N,Hkv,D]."""
    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None].requires_grad_()
    tq, tk, tv = t(q), t(k), t(v)
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale, enable_gqa=True)
    o.backward(torch.from_numpy(np.ascontiguousarray(dout.transpose(1, 0, 2)))[None])
    g = lambda a: a.grad[0].numpy().transpose(1, 0, 2)
    return g(tq), g(tk), g(tv)


def test_global_backward_equals_autograd_of_library_attention():
    """The query->summary branch is plain softmax attention: its gradients
    equal torch autograd through scaled_dot_product_attention (fp64)."""
    rng = np.random.default_rng(3)
    n, m, hq, hkv = 40, 24, 4, 2
    q = rng.standard_normal((n, hq, 64))
    ks = rng.standard_normal((hkv, m, 64))
    vs = rng.standard_normal((hkv, m, 64))
    dout = rng.standard_normal((n, hq, 64))
    dq, dk, dv = orc.global_attention_backward(q, ks, vs, 0.125, dout)
    # library: keys as a sequence of m "tokens"
    tq, tk, tv = _sdpa_grads(q, ks.transpose(1, 0, 2), vs.transpose(1, 0, 2), dout)
    assert np.abs(dq - tq).max() <= 1e-12
    assert np.abs(dk - tk.transpose(1, 0, 2)).max() <= 1e-12
    assert np.abs(dv - tv.transpose(1, 0, 2)).max() <= 1e-12


def test_local_backward_equals_autograd_of_masked_dense_attention():
    """Brute force on a tiny ragged lattice: the local branch is dense
    attention under the clipped-box mask; gradients equal torch autograd."""
    grid, window = (3, 4, 5), (3, 3, 5)
    cells = sg.lattice_cells(grid)
    n, hq, hkv = len(cells), 4, 2
    rng = np.random.default_rng(4)
    q = rng.standard_normal((n, hq, 64))
    k = rng.standard_normal((n, hkv, 64))
    v = rng.standard_normal((n, hkv, 64))
    dout = rng.standard_normal((n, hq, 64))
    r = np.array(window) // 2
    mask = np.all(np.abs(cells[:, None, :] - cells[None, :, :]) <= r, axis=2)
    dq, dk, dv = orc.local_attention_backward(q, k, v, cells, grid, window, 0.125, dout)
    tq, tk, tv = _sdpa_grads(q, k, v, dout, mask)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(a - b).max() <= 1e-12


def test_local_backward_with_whole_lattice_window_is_dense_backward():
    """A window covering the lattice makes the local branch dense attention
    over all tokens, so its gradients equal the query->summary branch's with
    the tokens themselves as summaries (two separate oracle paths)."""
    grid = (2, 3, 4)
    cells = sg.lattice_cells(grid)
    n, hq, hkv = len(cells), 4, 2
    rng = np.random.default_rng(6)
    q = rng.standard_normal((n, hq, 64))
    k = rng.standard_normal((n, hkv, 64))
    v = rng.standard_normal((n, hkv, 64))
    dout = rng.standard_normal((n, hq, 64))
    big = tuple(2 * g + 1 for g in grid)
    dq, dk, dv = orc.local_attention_backward(q, k, v, cells, grid, big, 0.125, dout)
    gq, gk, gv = orc.global_attention_backward(q, k.transpose(1, 0, 2), v.transpose(1, 0, 2),
                                               0.125, dout)
    assert np.abs(dq - gq).max() <= 1e-12
    assert np.abs(dk - gk.transpose(1, 0, 2)).max() <= 1e-12
    assert np.abs(dv - gv.transpose(1, 0, 2)).max() <= 1e-12


def test_rotate_transpose_is_the_inverse_rotation():
    """R(c)^T R(c) = I: un-rotating a rotated vector returns it, and the
    result matches the transposed matrix of rotation_matrix."""
    rng = np.random.default_rng(8)
    c = rng.integers(0, 200, size=(30, 3))
    x = rng.standard_normal((30, 3, 64))
    back = orc.rotate_transpose(orc.rotate(x, c, PAIRS, BASE), c, PAIRS, BASE)
    assert np.abs(back - x).max() <= 1e-12
    for i in range(5):
        R = orc.rotation_matrix(c[i], 64, PAIRS, BASE)
        y = orc.rotate_transpose(x[i:i + 1], c[i:i + 1], PAIRS, BASE)[0]
        assert np.abs(y - x[i] @ R).max() <= 1e-12   # (R^T x)^T = x^T R


@pytest.fixture(scope="module")
def c5_small():
    """The backward workload's oracle size: 4 x 16 x 16, Hq 8, Hkv 2, 3x7x7."""
    w = sg.Workload("c5s", (4, 16, 16), "block", 8, 2, (3, 7, 7), (1, 4, 4), "bf16",
                    "softmax", 5)
    inp = sg.make_inputs(w)
    dout = sg.make_upstream_grad(inp)
    g = orc.backward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a,
                     inp.coords, inp.gate, dout)
    return w, inp, dout, g


def test_gradient_identities(c5_small):
    """Identities of softmax attention, at any size: sum_j dv~_j is the sum of
    the compressed branch's upstream gradients and sum_j dk~_j = 0 (softmax
    rows sum to one and their gradient rows to zero); likewise for the local
    keys (after rotating back); the gate's two logit gradients cancel; and
    the block sums carry the summary gradients (weights sum to one)."""
    w, inp, dout, g = c5_small
    grp = w.n_q_heads // w.n_kv_heads
    gsum = lambda t: t.reshape(t.shape[0], w.n_kv_heads, grp, -1).sum(axis=(0, 2))
    assert np.abs(g["dv_sum"].sum(axis=1) - gsum(g["d_cmp"])).max() <= 1e-9
    assert np.abs(g["dk_sum"].sum(axis=1)).max() <= 1e-9
    assert np.abs(g["dv_loc"].sum(axis=0) - gsum(g["d_loc"])).max() <= 1e-9
    dk_rot = orc.rotate(g["dk_loc"], inp.coords, PAIRS, BASE)
    assert np.abs(dk_rot.sum(axis=0)).max() <= 1e-9
    assert np.abs(g["dgate"].sum(axis=-1)).max() <= 1e-12
    # sum_u dv_u = sum_j (sum_{u in B_j} a_u) dv~_j; the float32 weights sum
    # to one only up to their rounding, so the block sums are taken as given
    j = orc.block_index(inp.coords, w.grid, w.block)
    asum = np.zeros((w.n_blocks, w.n_kv_heads))
    np.add.at(asum, j, np.asarray(inp.a, np.float64))
    want_v = np.einsum("jg,gjd->gd", asum, g["dv_sum"])
    assert np.abs(g["dv_cmp"].sum(axis=0) - want_v).max() <= 1e-9
    want_k = np.einsum("jg,gjd->gd", asum, g["dk_sum"])
    got_k = orc.rotate(g["dk_cmp"], inp.coords, PAIRS, BASE).sum(axis=0)
    assert np.abs(got_k - want_k).max() <= 1e-9
    assert np.abs(want_k).max() <= 1e-6      # ~ sum_j dk~_j = 0


def test_sampled_rows_match_the_full_backward(c5_small):
    """Restricting the query rows gives the same dq rows, and the same local
    dk/dv at every key whose window lies inside the rows (the window is
    symmetric)."""
    w, inp, dout, g = c5_small
    f = g["fwd"]
    rows = np.sort(np.random.default_rng(2).choice(w.n_tokens, 200, replace=False))
    dq, _, _ = orc.local_attention_backward(f["q_rot"], f["k_rot"], inp.v_loc, inp.coords,
                                            w.grid, w.window, 0.125, g["d_loc"], rows)
    full, _, _ = orc.local_attention_backward(f["q_rot"], f["k_rot"], inp.v_loc, inp.coords,
                                              w.grid, w.window, 0.125, g["d_loc"])
    assert np.abs(dq - full[rows]).max() <= 1e-12
    # keys: one key cell and every query of its window
    key = 300
    r = np.array(w.window) // 2
    near = np.nonzero(np.all(np.abs(inp.coords - inp.coords[key]) <= r, axis=1))[0]
    _, dk, dv = orc.local_attention_backward(f["q_rot"], f["k_rot"], inp.v_loc, inp.coords,
                                             w.grid, w.window, 0.125, g["d_loc"], near)
    _, dkf, dvf = orc.local_attention_backward(f["q_rot"], f["k_rot"], inp.v_loc, inp.coords,
                                               w.grid, w.window, 0.125, g["d_loc"])
    assert np.abs(dk[key] - dkf[key]).max() <= 1e-12
    assert np.abs(dv[key] - dvf[key]).max() <= 1e-12


def test_backward_is_packing_equivariant(c5_small):
    """Proposition 1 carries over to the gradients: repacking the inputs and
    the upstream gradient permutes every gradient the same way."""
    w, inp, dout, g = c5_small
    other = inp.repacked("random")
    dout2 = sg.make_upstream_grad(other)
    g2 = orc.backward(other.workload, other.q, other.k_loc, other.v_loc, other.k_cmp,
                      other.v_cmp, other.a, other.coords, other.gate, dout2)
    src = inp.cell_to_pos[other.order]
    for name in ("dq", "dk_loc", "dv_loc", "dk_cmp", "dv_cmp", "dgate"):
        assert np.abs(g2[name] - g[name][src]).max() <= 1e-11, name
