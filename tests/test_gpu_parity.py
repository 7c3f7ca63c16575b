"""GPU parity: every libpack3d entry point against the fp64 oracle.

The HIP path is called through the C ABI (ctypes binding); expected values come
from ``oracle/`` only.  Small workloads and the 65 536-token workload are
compared element by element in full; the 262 144-, 1 048 576-, 4 194 304- and
8 388 608-token workloads on sampled query rows.  The fused forward (the path
the bench times) is checked branch by branch through the training forward,
which launches the same kernels and also saves each branch's output.
"""

import numpy as np
import pytest
import torch

import synthgen as sg
from oracle import pack3d_oracle as orc
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

W = sg.WORKLOADS
TINY = W["tiny_f32_4x16x16"]
MORTON = W["morton_bf16_16x64x64"]
BLOCK = W["block_bf16_64x64x64"]
RANDOM = W["random_bf16_64x128x128"]


def _w(name, grid, hq, hkv, dtype, window=(3, 7, 7), block=(1, 4, 4), packing="random",
       weights="softmax", seed=7):
    return sg.Workload(name, grid, packing, hq, hkv, window, block, dtype, weights, seed)


# Small cases that span several tiles and ragged tails: Y, X not multiples of
# the 8x8 local tile, M not a multiple of the 64-key summary tile, every
# supported heads-per-group ratio, both dtypes.
SMALL = [
    TINY,
    _w("ragged_f32_g4", (3, 12, 20), 4, 1, "f32"),
    _w("ragged_bf16_g4", (3, 12, 20), 8, 2, "bf16"),
    _w("g1_bf16", (2, 8, 12), 2, 2, "bf16", packing="morton"),
    _w("g8_f32", (4, 8, 8), 8, 1, "f32", window=(3, 3, 5)),
    _w("g16_bf16", (2, 16, 8), 16, 1, "bf16", window=(1, 7, 3)),
    _w("g2_bf16_uniform", (5, 8, 16), 4, 2, "bf16", window=(5, 5, 5), weights="uniform",
       packing="block"),
    _w("tiny_lattice_f32", (1, 4, 4), 4, 2, "f32", window=(3, 7, 7)),
    _w("g8_bf16", (3, 12, 12), 8, 1, "bf16"),
    _w("g16_bf16_full", (3, 4, 12), 16, 1, "bf16", packing="morton"),
    _w("g4_bf16_deep", (9, 12, 8), 8, 2, "bf16", window=(7, 3, 5), packing="morton"),
    _w("g4_bf16_w1", (2, 8, 8), 4, 1, "bf16", window=(1, 1, 1), packing="raster"),
    # windows three planes deep on deeper lattices: the local kernel walks
    # runs of query planes (runs of 4 here, the last one ragged, runs that
    # start inside the lattice) for every heads-per-group ratio
    _w("zrun_bf16_g4", (13, 8, 16), 8, 2, "bf16", window=(3, 5, 7)),
    _w("zrun_bf16_g8", (10, 12, 8), 8, 1, "bf16", window=(3, 7, 3), packing="morton"),
    _w("zrun_bf16_g16", (7, 4, 8), 16, 1, "bf16"),
    _w("zrun_bf16_z2", (2, 8, 8), 8, 2, "bf16", packing="raster"),
]
IDS = [w.name for w in SMALL]


@pytest.fixture(scope="module")
def pk():
    from geometry_aware_local_amd import pack3d
    return pack3d


def _say(*a):
    print(*a, flush=True)


def _rows(w, k, seed=0):
    n = w.n_tokens
    return np.arange(n) if n <= k else np.sort(np.random.default_rng(seed).choice(n, k, False))


# --------------------------------------------------------------------------
# single ops, fed with the oracle's own (rounded) inputs
# --------------------------------------------------------------------------

@pytest.mark.parametrize("w", SMALL + [MORTON], ids=IDS + [MORTON.name])
def test_rope(pk, w):
    _say("rope", w.name)
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    got_q = gu.host(pk.pack3d_rope(prob, d["q"], d["coords"]))
    k = d["k_loc"].clone()
    pk.pack3d_rope(prob, k, d["coords"], out=k)                 # in place
    for got, x in ((got_q, inp.q), (gu.host(k), inp.k_loc)):
        ref = orc.rotate(x, inp.coords, w.rope_pairs, w.rope_base)
        err = np.abs(got - ref)
        if w.dtype == "f32":
            assert err.max() <= 1e-5
        else:
            assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6)


@pytest.mark.parametrize("w", SMALL + [MORTON], ids=IDS + [MORTON.name])
def test_block_summary(pk, w):
    _say("block_summary", w.name)
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    ks, vs = pk.pack3d_block_summary(prob, d["k_cmp"], d["v_cmp"], d["a"], d["cell_to_pos"])
    rk, rv = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block,
                                 w.rope_pairs, w.rope_base)
    for got, ref in ((gu.host(ks), rk), (gu.host(vs), rv)):
        if w.dtype == "f32":
            assert gu.max_abs(got, ref) <= 1e-5
        else:
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


def _rotated(w, inp):
    q = gu.round_like(orc.rotate(inp.q, inp.coords, w.rope_pairs, w.rope_base), w)
    k = gu.round_like(orc.rotate(inp.k_loc, inp.coords, w.rope_pairs, w.rope_base), w)
    return q, k


@pytest.mark.parametrize("w", SMALL + [MORTON], ids=IDS + [MORTON.name])
def test_local_attn(pk, w):
    _say("local_attn", w.name)
    inp = sg.make_inputs(w)
    dt = gu.tdtype(w)
    q, k = _rotated(w, inp)
    prob = gu.problem(pk, w)
    o, lse = pk.pack3d_local_attn(prob, gu.dev(q, dt), gu.dev(k, dt), gu.dev(inp.v_loc, dt),
                                  gu.dev(inp.cell_to_pos), with_lse=True)
    rows = _rows(w, 4096)
    ro, rl = orc.local_attention(q, k, inp.v_loc, inp.coords, w.grid, w.window, 0.125, rows)
    go, gl = gu.host(o)[rows], gu.host(lse)[rows]
    assert gu.max_rel(go, ro) <= gu.REL_TOL[w.dtype]
    assert gu.max_abs(gl, rl) <= gu.LSE_TOL[w.dtype]


@pytest.mark.parametrize("w", SMALL + [MORTON], ids=IDS + [MORTON.name])
def test_global_attn(pk, w):
    _say("global_attn", w.name)
    inp = sg.make_inputs(w)
    dt = gu.tdtype(w)
    q, _ = _rotated(w, inp)
    rk, rv = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block,
                                 w.rope_pairs, w.rope_base)
    rk, rv = gu.round_like(rk, w), gu.round_like(rv, w)
    prob = gu.problem(pk, w)
    o, lse = pk.pack3d_global_attn(prob, gu.dev(q, dt), gu.dev(rk, dt), gu.dev(rv, dt),
                                   with_lse=True)
    rows = _rows(w, 2048)
    ro, rl = orc.global_attention(q, rk, rv, 0.125, rows)
    assert gu.max_rel(gu.host(o)[rows], ro) <= gu.REL_TOL[w.dtype]
    assert gu.max_abs(gu.host(lse)[rows], rl) <= gu.LSE_TOL[w.dtype]


@pytest.mark.parametrize("w", [TINY, MORTON.with_(grid=(4, 16, 16))], ids=["f32", "bf16"])
@pytest.mark.parametrize("per_head", [False, True])
def test_gate_mix(pk, w, per_head):
    _say("gate_mix", w.name, per_head)
    rng = np.random.default_rng(5)
    n, hq = w.n_tokens, w.n_q_heads
    ol = rng.standard_normal((n, hq, 64)).astype(np.float32)
    oc = rng.standard_normal((n, hq, 64)).astype(np.float32)
    g = rng.standard_normal((n, hq, 2) if per_head else (n, 2)).astype(np.float32) * 3
    prob = gu.problem(pk, w, gate_per_head=per_head)
    out = gu.host(pk.pack3d_gate_mix(prob, gu.dev(ol), gu.dev(oc), gu.dev(g)))
    ref = orc.gate_mix(ol, oc, g)
    err = np.abs(out - ref)
    if w.dtype == "f32":
        assert err.max() <= 1e-6
    else:
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6)


# --------------------------------------------------------------------------
# the whole path
# --------------------------------------------------------------------------

def _fargs(pk, w, d, **kw):
    return (gu.problem(pk, w, **kw), d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"],
            d["a"], d["coords"], d["cell_to_pos"], d["gate"])


def _check_fused_branches(pk, prob, fargs, out, ref, rows, dtype):
    """The fused forward the bench times (pre-scaled summaries, the
    per-group norm bound, the gated epilogue) checked branch by branch: the
    training forward launches the same kernels, gives the same output bit
    for bit and also saves each branch's fp32 output."""
    out_t, saved = pk.pack3d_forward_train(*fargs)
    sv = pk.saved_views(prob, saved)
    assert torch.equal(out_t, out)
    idx = torch.from_numpy(np.asarray(rows, np.int64)).cuda()
    o_loc = gu.host(sv["o_loc"][idx])
    o_cmp = gu.host(sv["o_cmp"][idx])
    e_loc, e_cmp = gu.max_rel(o_loc, ref["o_loc"]), gu.max_rel(o_cmp, ref["o_cmp"])
    _say(f"  fused branches: o_loc rel {e_loc:.2e}, o_cmp rel {e_cmp:.2e} "
         f"(max |o_cmp| {np.abs(ref['o_cmp']).max():.3e})")
    assert e_loc <= gu.REL_TOL[dtype]
    assert e_cmp <= gu.REL_TOL[dtype]


def _check_forward(pk, w, inp, rows):
    d = gu.device_inputs(inp)
    fargs = _fargs(pk, w, d)
    prob = fargs[0]
    out = pk.pack3d_forward(*fargs)
    # the same chain through the split entry points, for per-branch checks
    q_rot = pk.pack3d_rope(prob, d["q"], d["coords"])
    k_rot = pk.pack3d_rope(prob, d["k_loc"], d["coords"])
    ks, vs = pk.pack3d_block_summary(prob, d["k_cmp"], d["v_cmp"], d["a"], d["cell_to_pos"])
    o_loc = pk.pack3d_local_attn(prob, q_rot, k_rot, d["v_loc"], d["cell_to_pos"])
    o_cmp = pk.pack3d_global_attn(prob, q_rot, ks, vs)
    torch.cuda.synchronize()
    ref = orc.forward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a, inp.coords,
                      inp.gate, rows=rows)
    got = gu.host(out)[rows]
    err = gu.max_abs(got, ref["out"])
    _say(f"  out max abs {err:.2e} over {len(rows)} rows")
    assert err <= gu.ABS_TOL[w.dtype]
    assert gu.max_rel(gu.host(o_loc)[rows], ref["o_loc"]) <= gu.REL_TOL[w.dtype]
    assert gu.max_rel(gu.host(o_cmp)[rows], ref["o_cmp"]) <= gu.REL_TOL[w.dtype]
    _check_fused_branches(pk, prob, fargs, out, ref, rows, w.dtype)
    # the split chain's gate gives the fused forward's result.  Both take the
    # same local branch (the fused forward rotates Q with k_rope's bits:
    # test_fused_rotations_are_k_rope_bitwise); their compressed branches
    # differ (the fused one streams summaries pre-scaled into log2 units,
    # rounded once more), each within the per-branch bound of the oracle.
    # In bf16 the fused forward also passes the local branch's gated share
    # g_loc * o_loc through the output dtype before adding the compressed
    # share (bf16 keeps 8 significant bits: <= 2^-8 |g_loc o_loc|), and each
    # result carries its final rounding (<= 2^-8 |mix| each).
    mixed = gu.host(pk.pack3d_gate_mix(prob, o_loc, o_cmp, d["gate"]))
    diff = np.abs(mixed - gu.host(out))
    cmp_bound = 2 * gu.REL_TOL[w.dtype] * float(np.abs(gu.host(o_cmp)).max())
    if w.dtype == "f32":
        assert diff.max() <= cmp_bound + 1e-6
    else:
        g = orc.gate_weights(inp.gate)
        g_loc = g[:, None, 0:1] if g.ndim == 2 else g[..., 0:1]
        share = np.abs(g_loc * gu.host(o_loc))
        bound = 2.0 ** -8 * (share + 2 * np.abs(mixed)) + cmp_bound + 1e-6
        worst = float((diff / bound).max())
        _say(f"  split vs fused: largest difference / its bound {worst:.3f}")
        assert worst <= 1.0
    return out, o_loc, o_cmp, ref


@pytest.mark.parametrize("w", [SMALL[1], SMALL[2], SMALL[3], SMALL[12], SMALL[14],
                               MORTON.with_(grid=(4, 32, 32))],
                         ids=lambda w: w.name)
def test_fused_rotations_are_k_rope_bitwise(pk, w):
    """The forward rotates K_loc inside the block pass and Q inside both
    attention kernels (through the rotary table).  The rotated K_loc it
    leaves in the workspace (the section after the table) is what
    pack3d_rope writes, bit for bit; and the training forward's local branch,
    which rotates Q in registers, equals pack3d_local_attn fed pack3d_rope's
    rotated Q, bit for bit (same kernel, same operands)."""
    _say("fused rotations", w.name)
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    fargs = (prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"], d["a"], d["coords"],
             d["cell_to_pos"], d["gate"])
    ws = pk.alloc_workspace(prob, d["q"].device)
    ws.fill_(0xFF)
    pk.pack3d_forward(*fargs, workspace=ws)
    q_rot = pk.pack3d_rope(prob, d["q"], d["coords"])
    k_rot = pk.pack3d_rope(prob, d["k_loc"], d["coords"])
    torch.cuda.synchronize()
    nk = k_rot.numel() * k_rot.element_size()
    ts = max(w.grid)
    k_off = (32 * ts * 8 + 255) // 256 * 256
    assert torch.equal(ws[k_off:k_off + nk], k_rot.view(torch.uint8).reshape(-1))
    _, saved = pk.pack3d_forward_train(*fargs)
    o_loc = pk.pack3d_local_attn(prob, q_rot, k_rot, d["v_loc"], d["cell_to_pos"])
    torch.cuda.synchronize()
    assert torch.equal(pk.saved_views(prob, saved)["o_loc"], o_loc)


@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_forward_small(pk, w):
    _say("forward", w.name)
    inp = sg.make_inputs(w)
    _check_forward(pk, w, inp, np.arange(w.n_tokens))


def test_forward_65k_morton_full(pk):
    """The 65 536-token Morton workload compared in full: every row, every head."""
    _say("forward", MORTON.name, "all rows")
    inp = sg.make_inputs(MORTON)
    _check_forward(pk, MORTON, inp, np.arange(MORTON.n_tokens))


def test_branches_with_peaked_queries(pk):
    """Queries scaled by 4 make both softmaxes far from uniform.  The kernels
    get the rotated queries/keys and summaries as stored on the device (bf16
    values), and so does the oracle, so only the kernels' own arithmetic is
    measured; both branches are held to the relative bound."""
    w = MORTON
    _say("branches peaked", w.name)
    inp = sg.make_inputs(w)
    inp.q = (inp.q * 4.0).astype(np.float32)        # exact in bf16
    dt = gu.tdtype(w)
    q, k = _rotated(w, inp)
    rk, rv = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block)
    rk, rv = gu.round_like(rk, w), gu.round_like(rv, w)
    prob = gu.problem(pk, w)
    o_loc = pk.pack3d_local_attn(prob, gu.dev(q, dt), gu.dev(k, dt), gu.dev(inp.v_loc, dt),
                                 gu.dev(inp.cell_to_pos))
    o_cmp = pk.pack3d_global_attn(prob, gu.dev(q, dt), gu.dev(rk, dt), gu.dev(rv, dt))
    rows = _rows(w, 2048, seed=1)
    ro_loc, _ = orc.local_attention(q, k, inp.v_loc, inp.coords, w.grid, w.window, 0.125, rows)
    ro_cmp, _ = orc.global_attention(q, rk, rv, 0.125, rows)
    assert gu.max_rel(gu.host(o_loc)[rows], ro_loc) <= gu.REL_TOL["bf16"]
    assert gu.max_rel(gu.host(o_cmp)[rows], ro_cmp) <= gu.REL_TOL["bf16"]


def test_forward_softmax_reference_paths(pk):
    """The fused forward picks, per wave, the zero reference (every query's
    logit bound <= 64 in log2 units), a fixed reference (bounds <= 80) or a
    tracked running max.  Queries are scaled per group of 16 tokens (one
    wave's rows) by 1, 8 and 12, and mixed within a group, so all three
    paths and mixed waves run; the gate is forced to the compressed branch.
    The oracle gets the operands as the kernel holds them: rotated queries
    and summaries pre-scaled by tau*log2(e), each rounded to bf16 (computed
    on the host from the oracle's own values), softmax in base 2."""
    w = MORTON.with_(grid=(4, 16, 16))
    _say("softmax reference paths", w.name)
    inp = sg.make_inputs(w)
    n = w.n_tokens
    grp_scale = np.array([1.0, 8.0, 12.0, 0.0])
    scale = grp_scale[(np.arange(n) // 16) % 4]
    mixed = scale == 0.0
    scale[mixed] = np.random.default_rng(3).choice([1.0, 8.0, 12.0], int(mixed.sum()))
    inp.q = sg.round_to_bf16((inp.q * scale[:, None, None]).astype(np.float32))
    inp.gate = np.tile(np.array([[-60.0, 60.0]], np.float32), (n, 1))
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    out = gu.host(pk.pack3d_forward(prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"],
                                    d["a"], d["coords"], d["cell_to_pos"], d["gate"]))
    q_r = gu.round_like(orc.rotate(inp.q, inp.coords), w)
    ks, vs = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block)
    ks2 = gu.round_like(ks * (0.125 / np.log(2.0)), w)
    ref, _ = orc.global_attention(q_r, ks2, gu.round_like(vs, w), np.log(2.0))
    # the three paths are all taken: bounds per token (log2 units)
    kmax = np.sqrt((ks2 ** 2).sum(-1)).max()
    bound = np.sqrt((q_r ** 2).sum(-1)).max(-1) * kmax
    assert (bound <= 60).any() and ((bound > 66) & (bound < 78)).sum() > 64 and (bound > 84).any()
    err = np.abs(out - ref) / np.abs(ref).max()
    for name, sel in (("zero", bound <= 60), ("fixed", (bound > 66) & (bound < 78)),
                      ("tracked", bound > 82)):
        _say(f"  {name}: {int(sel.sum())} tokens, max error {err[sel].max():.2e} of max |o_cmp|")
    assert err.max() <= gu.REL_TOL["bf16"]


def test_forward_262k_block_sampled(pk):
    _say("forward", BLOCK.name)
    inp = sg.make_inputs(BLOCK)
    _check_forward(pk, BLOCK, inp, _rows(BLOCK, 1024, seed=2))


def _reach(pk, w, nrows):
    """The forward at reach sizes: 4 194 304 tokens (M = 262 144) and
    8 388 608 tokens (M = 524 288; element offsets of q pass 2^32), checked
    on sampled rows (the oracle builds every summary)."""
    _say("forward reach", w.name, "generating inputs")
    inp = sg.make_inputs(w, progress=_say)
    rows = _rows(w, nrows, seed=4)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    _say("  gpu forward")
    out = pk.pack3d_forward(prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"], d["a"],
                            d["coords"], d["cell_to_pos"], d["gate"])
    got = gu.host(out[torch.from_numpy(rows).cuda()])
    del out, d
    torch.cuda.empty_cache()
    _say("  oracle on", len(rows), "rows")
    ref = orc.forward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a, inp.coords,
                      inp.gate, rows=rows)
    assert gu.max_abs(got, ref["out"]) <= gu.ABS_TOL["bf16"]


def test_forward_4m_reach_sampled(pk):
    _reach(pk, W["reach_bf16_64x256x256"], 64)


def test_forward_8m_reach_sampled(pk):
    _reach(pk, W["reach_bf16_128x256x256"], 64)


def test_forward_1m_random_sampled(pk):
    """1 048 576 tokens in random packing (M = 65 536): the end-to-end bound
    and both branches of the fused path against the relative bound, on
    sampled rows.  At this size the compressed branch is far below the
    absolute bound, so only the per-branch check could see it break."""
    _say("forward", RANDOM.name)
    inp = sg.make_inputs(RANDOM)
    rows = _rows(RANDOM, 512, seed=3)
    d = gu.device_inputs(inp)
    fargs = _fargs(pk, RANDOM, d)
    out = pk.pack3d_forward(*fargs)
    ref = orc.forward(RANDOM, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a,
                      inp.coords, inp.gate, rows=rows)
    err = gu.max_abs(gu.host(out)[rows], ref["out"])
    _say(f"  out max abs {err:.2e}")
    assert err <= gu.ABS_TOL["bf16"]
    _check_fused_branches(pk, fargs[0], fargs, out, ref, rows, "bf16")


def test_dense_companion_1m_sampled(pk):
    """The dense axial-RoPE attention the bench times beside the forward at
    1 048 576 tokens: the forward with 1x1x1 blocks and a = 1, whose
    compressed branch attends to every rotated key (m = N).  The gate logits
    (-40, +40) select that branch (g_loc = e^-80), so sampled output rows are
    checked against the oracle's dense softmax over all N keys."""
    w = RANDOM
    _say("dense companion", w.name)
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    dprob = gu.problem(pk, w.with_(block=(1, 1, 1)))
    gate = torch.tensor([-40.0, 40.0], dtype=torch.float32).repeat(w.n_tokens, 1).cuda()
    out = pk.pack3d_forward(dprob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"], None,
                            d["coords"], d["cell_to_pos"], gate)
    rows = _rows(w, 48, seed=6)
    got = gu.host(out[torch.from_numpy(rows).cuda()])
    del out, d, gate
    torch.cuda.empty_cache()
    qr = orc.rotate(inp.q[rows], inp.coords[rows])
    rk, rv = orc.block_summaries(inp.k_cmp, inp.v_cmp, None, inp.coords, w.grid, (1, 1, 1))
    ref, _ = orc.global_attention(qr, rk, rv, 0.125, q_is_rows=True)
    e_abs, e_rel = gu.max_abs(got, ref), gu.max_rel(got, ref)
    _say(f"  max abs {e_abs:.2e}, rel {e_rel:.2e}")
    assert e_abs <= gu.ABS_TOL["bf16"]
    assert e_rel <= gu.REL_TOL["bf16"]


# End-to-end error against the logit scale.  The GPU rounds the rotated q, k
# (and the summaries) to bf16 before the products, so each logit carries an
# error that grows with |q||k|; queries scaled by s multiply every logit by s.
# Measured maximum abs errors of the output against the fp64 oracle are
# printed for every scale; the end-to-end bound is asserted up to
# PEAKED_MAX_SCALE.
PEAKED_SCALES = (1.0, 2.0, 3.0, 4.0)
PEAKED_MAX_SCALE = 2.0


@pytest.mark.parametrize("qscale", PEAKED_SCALES)
def test_forward_end_to_end_logit_scale(pk, qscale):
    w = MORTON.with_(grid=(8, 32, 32))
    _say("forward logit scale", qscale, w.name)
    inp = sg.make_inputs(w)
    inp.q = sg.round_to_bf16((inp.q * qscale).astype(np.float32))
    d = gu.device_inputs(inp)
    fargs = _fargs(pk, w, d)
    out = pk.pack3d_forward(*fargs)
    rows = np.arange(w.n_tokens)
    ref = orc.forward(w, inp.q, inp.k_loc, inp.v_loc, inp.k_cmp, inp.v_cmp, inp.a, inp.coords,
                      inp.gate, rows=rows)
    out_t, saved = pk.pack3d_forward_train(*fargs)
    sv = pk.saved_views(fargs[0], saved)
    e = gu.max_abs(gu.host(out), ref["out"])
    e_loc = gu.max_abs(gu.host(sv["o_loc"]), ref["o_loc"])
    e_cmp = gu.max_abs(gu.host(sv["o_cmp"]), ref["o_cmp"])
    _say(f"  scale {qscale}: out max abs {e:.3e}; o_loc {e_loc:.3e}; o_cmp {e_cmp:.3e}")
    if qscale <= PEAKED_MAX_SCALE:
        assert e <= gu.ABS_TOL["bf16"]


# --------------------------------------------------------------------------
# packing equivariance (Proposition 1): repacked outputs are the permuted
# outputs, bit for bit
# --------------------------------------------------------------------------

@pytest.mark.parametrize("w", [BLOCK, TINY], ids=["262k_bf16", "tiny_f32"])
def test_packing_equivariance(pk, w):
    _say("equivariance", w.name)
    base = sg.make_inputs(w.with_(packing="raster"))
    prob = gu.problem(pk, w)
    outs = {}
    for kind in ("raster", "block", "random", "morton", "block_morton"):
        inp = base if kind == "raster" else base.repacked(kind)
        d = gu.device_inputs(inp)
        out = pk.pack3d_forward(prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"],
                                d["a"], d["coords"], d["cell_to_pos"], d["gate"])
        back = torch.from_numpy(inp.cell_to_pos[base.order].astype(np.int64)).cuda()
        outs[kind] = out[back].float()
    for kind in ("block", "random", "morton", "block_morton"):
        diff = (outs[kind] - outs["raster"]).abs().max().item()
        assert diff <= 1e-6, (kind, diff)
        assert torch.equal(outs[kind], outs["raster"]), kind


def test_repeat_runs_are_bitwise_equal(pk):
    _say("determinism", MORTON.name)
    inp = sg.make_inputs(MORTON)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, MORTON)
    args = (d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"], d["a"], d["coords"],
            d["cell_to_pos"], d["gate"])
    a = pk.pack3d_forward(prob, *args)
    b = pk.pack3d_forward(prob, *args)
    assert torch.equal(a, b)


# --------------------------------------------------------------------------
# degenerate cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unit_blocks_give_dense_attention(pk, dtype):
    """1x1x1 blocks with a = 1 turn the compressed branch into dense
    axial-RoPE attention over (R(c)Q, R(c)K_cmp, V_cmp)."""
    w = _w("dense", (4, 8, 10), 8, 2, dtype, block=(1, 1, 1), weights="uniform")
    _say("dense", dtype)
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    q_rot = pk.pack3d_rope(prob, d["q"], d["coords"])
    ks, vs = pk.pack3d_block_summary(prob, d["k_cmp"], d["v_cmp"], None, d["cell_to_pos"])
    assert ks.shape[1] == w.n_tokens
    o = gu.host(pk.pack3d_global_attn(prob, q_rot, ks, vs))
    qr = orc.rotate(inp.q, inp.coords)
    kr = orc.rotate(inp.k_cmp, inp.coords)
    hq, grp = w.n_q_heads, w.n_q_heads // w.n_kv_heads
    ref = np.zeros_like(o)
    for h in range(hq):
        s = 0.125 * qr[:, h] @ kr[:, h // grp].T
        p = np.exp(s - s.max(1, keepdims=True))
        ref[:, h] = (p / p.sum(1, keepdims=True)) @ inp.v_cmp[:, h // grp].astype(np.float64)
    assert gu.max_abs(o, ref) <= gu.ABS_TOL[dtype]
    assert gu.max_rel(o, ref) <= gu.REL_TOL[dtype]


EDGE = [
    _w("single_cell_f32", (1, 1, 1), 4, 1, "f32", block=(1, 1, 1)),
    _w("single_cell_bf16", (1, 1, 1), 8, 2, "bf16", block=(1, 1, 1)),
    _w("one_summary_f32", (2, 4, 8), 4, 2, "f32", block=(2, 4, 8)),
    _w("one_summary_bf16", (2, 4, 8), 8, 2, "bf16", block=(2, 4, 8), packing="morton"),
    _w("one_row_bf16", (1, 1, 24), 16, 1, "bf16", block=(1, 1, 4)),
    _w("one_column_f32", (5, 1, 1), 2, 1, "f32", window=(5, 1, 1), block=(5, 1, 1)),
]


@pytest.mark.parametrize("w", EDGE, ids=[e.name for e in EDGE])
def test_forward_degenerate_lattices(pk, w):
    """One token (N = M = 1), one summary for the whole lattice (M = 1, block
    volume 64), a 1x1xX row and a Zx1x1 column."""
    _say("forward degenerate", w.name)
    inp = sg.make_inputs(w)
    out, o_loc, o_cmp, ref = _check_forward(pk, w, inp, np.arange(w.n_tokens))
    if w.n_blocks == 1:
        # a single summary: every query's compressed branch is that value
        # summary, whatever the logits
        _, vs = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block)
        grp = w.n_q_heads // w.n_kv_heads
        want = np.repeat(vs[:, 0][None], w.n_tokens, 0).repeat(grp, axis=1)
        tol = 1e-5 if w.dtype == "f32" else 2.0 ** -7
        assert np.abs(gu.host(o_cmp) - want).max() <= tol * max(1.0, np.abs(want).max())


def test_window_of_one_cell_returns_values(pk):
    """A 1x1x1 window attends only to the query cell: o_loc = V_loc."""
    w = _w("w1", (3, 8, 12), 4, 2, "f32", window=(1, 1, 1), weights="uniform")
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    o = gu.host(pk.pack3d_local_attn(prob, d["q"], d["k_loc"], d["v_loc"], d["cell_to_pos"]))
    want = np.repeat(inp.v_loc, 2, axis=1)
    assert gu.max_abs(o, want) <= 1e-6


# --------------------------------------------------------------------------
# test power: planted mistakes (in the oracle, on the CPU) must fail the checks
# --------------------------------------------------------------------------

def test_checks_catch_planted_mistakes(pk):
    w = MORTON.with_(grid=(4, 32, 32))
    _say("planted mistakes", w.name)
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    q_rot = pk.pack3d_rope(prob, d["q"], d["coords"])
    ks, vs = pk.pack3d_block_summary(prob, d["k_cmp"], d["v_cmp"], d["a"], d["cell_to_pos"])
    o_cmp = gu.host(pk.pack3d_global_attn(prob, q_rot, ks, vs))
    qr = orc.rotate(inp.q, inp.coords)
    good_k, good_v = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block)
    good, _ = orc.global_attention(qr, good_k, good_v, 0.125)
    assert gu.max_rel(o_cmp, good) <= gu.REL_TOL["bf16"]
    # 1. summaries shuffled (keys paired with another block's values)
    perm = np.random.default_rng(0).permutation(good_v.shape[1])
    bad, _ = orc.global_attention(qr, good_k, good_v[:, perm], 0.125)
    assert gu.max_rel(o_cmp, bad) > gu.REL_TOL["bf16"]
    # 2. keys pooled without rotation
    nz = np.zeros_like(inp.coords)
    bk, bv = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block,
                                 rope_coords=nz)
    bad, _ = orc.global_attention(qr, bk, bv, 0.125)
    assert gu.max_rel(o_cmp, bad) > gu.REL_TOL["bf16"]
    # 3. packed index used as the coordinate of the rotation
    seq = np.stack([np.zeros(w.n_tokens), np.zeros(w.n_tokens), np.arange(w.n_tokens)], 1)
    bad, _ = orc.global_attention(orc.rotate(inp.q, seq.astype(np.int64)), good_k, good_v, 0.125)
    assert gu.max_rel(o_cmp, bad) > gu.REL_TOL["bf16"]
    # 4. the compressed branch dropped altogether is caught by the relative
    #    branch check ...
    assert gu.max_rel(np.zeros_like(o_cmp), good) > gu.REL_TOL["bf16"]
    # ... while at 262 144 tokens the absolute end-to-end bound alone could not
    #     see it: the whole branch is smaller than that bound there
    big = sg.make_inputs(BLOCK)
    rows = _rows(BLOCK, 64, seed=4)
    ref = orc.forward(BLOCK, big.q, big.k_loc, big.v_loc, big.k_cmp, big.v_cmp, big.a,
                      big.coords, big.gate, rows=rows)
    assert np.abs(ref["o_cmp"]).max() < gu.ABS_TOL["bf16"]


# --------------------------------------------------------------------------
# helpers and argument errors on the device path
# --------------------------------------------------------------------------

def test_cell_index_and_packing_check(pk):
    w = MORTON.with_(grid=(4, 16, 16))
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    c2p = pk.pack3d_build_cell_index(prob, d["coords"])
    assert torch.equal(c2p.cpu(), torch.from_numpy(inp.cell_to_pos))
    assert pk.pack3d_check_packing(prob, d["coords"], d["cell_to_pos"]) == 0
    bad = d["cell_to_pos"].clone()
    bad[[3, 7]] = bad[[7, 3]]
    assert pk.pack3d_check_packing(prob, d["coords"], bad) == 2


def test_workspace_too_small_is_rejected(pk):
    inp = sg.make_inputs(TINY)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, TINY)
    ws = torch.empty(pk.pack3d_forward_workspace_size(prob) - 256, dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(pk.Pack3DError, match="ERR_WORKSPACE"):
        pk.pack3d_forward(prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"], d["a"],
                          d["coords"], d["cell_to_pos"], d["gate"], workspace=ws)


def test_forward_timed_matches_forward(pk):
    """The per-stage timed forward launches the same kernels: bitwise equal
    output, and its stage times add up to the whole."""
    w = MORTON.with_(grid=(8, 32, 32))
    _say("forward_timed", w.name)
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    args = (prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"], d["a"], d["coords"],
            d["cell_to_pos"], d["gate"])
    ref = pk.pack3d_forward(*args)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(pk.PACK3D_FORWARD_STAGES + 1)]
    out = pk.pack3d_forward_timed(*args, ev)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    stages = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(ev) - 1)]
    assert all(t >= 0 for t in stages)
    assert abs(sum(stages) - ev[0].elapsed_time(ev[-1])) < 1e-3
    with pytest.raises(ValueError):
        pk.pack3d_forward_timed(*args, ev[:-1])
