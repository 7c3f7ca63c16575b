"""The C ABI on the CPU: the library loads, exports what include/pack3d.h
declares, and rejects bad arguments on the host before any HIP call (no
device is touched by these tests)."""

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pack3d.h")


@pytest.fixture(scope="module")
def pk():
    from geometry_aware_local_amd import pack3d
    return pack3d


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(pack3d_\w+)\s*\(", text,
                                 re.M)))


def test_header_declares_the_entry_points(pk):
    names = _declared()
    for required in ("pack3d_rope", "pack3d_block_summary", "pack3d_local_attn",
                     "pack3d_global_attn", "pack3d_gate_mix", "pack3d_forward"):
        assert required in names
    assert set(names) == set(pk.EXPORTS)


def test_library_exports_every_declared_symbol(pk):
    lib = ctypes.CDLL(pk.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_backend_info(pk):
    assert pk.pack3d_version() == 1
    info = pk.pack3d_backend_info()
    assert "gfx950" in info and "no fallbacks" in info


def _prob(pk, **kw):
    base = dict(grid=(4, 16, 16), n_q_heads=2, n_kv_heads=1, window=(3, 5, 5), block=(1, 4, 4))
    base.update(kw)
    return pk.make_problem(**base)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,code,text", [
    (dict(grid=(0, 16, 16)), -2, "grid"),
    (dict(head_dim=32), -3, "head_dim"),
    (dict(n_q_heads=3, n_kv_heads=2), -2, "multiple"),
    (dict(window=(3, 4, 5)), -2, "odd"),
    (dict(window=(3, 9, 5)), -3, "window"),
    (dict(block=(1, 3, 4)), -2, "divide"),
    (dict(block=(2, 8, 8)), -3, "volume"),
    (dict(rope_pairs=(11, 11, 11)), -2, "rope_pairs"),
    (dict(rope_base=-1.0), -2, "rope_base"),
    (dict(grid=(2048, 1024, 1024)), -2, "int32"),
    (dict(summary_mode=3), -2, "summary_mode"),
    (dict(summary_mode=-1), -2, "summary_mode"),
])
def test_bad_problems_are_rejected_on_the_host(pk, kw, code, text):
    p = _prob(pk, **kw)
    rc = pk.LIB.pack3d_rope(ctypes.byref(p), FAKE, FAKE, 2, FAKE, None)
    assert rc == code
    assert text in pk.pack3d_last_error()
    assert pk.pack3d_forward_workspace_size(p) == 0


def test_problem_struct_matches_the_header(pk):
    """The ctypes mirror has the header's fields in order (the last one is
    the compressed-branch variant) and the C struct's size."""
    text = open(HEADER).read()
    body = re.search(r"typedef struct pack3d_problem \{(.*?)\} pack3d_problem;", text, re.S)
    fields = re.findall(r"^\s*\w+\s+(\w+)(?:\[\d\])?;", body.group(1), re.M)
    assert fields == [f[0] for f in pk.Problem._fields_]
    assert ctypes.sizeof(pk.Problem) == 88
    assert [pk.make_problem((1, 4, 4), 2, 1, summary_mode=m).summary_mode
            for m in pk.SUMMARY_MODES] == [0, 1, 2]


def test_null_arguments_are_rejected(pk):
    p = _prob(pk)
    L, b = pk.LIB, ctypes.byref(p)
    assert L.pack3d_rope(None, FAKE, FAKE, 2, FAKE, None) == -1
    assert L.pack3d_rope(b, None, FAKE, 2, FAKE, None) == -1
    assert L.pack3d_block_summary(b, FAKE, FAKE, None, None, FAKE, FAKE, None) == -1
    assert L.pack3d_local_attn(b, FAKE, FAKE, FAKE, FAKE, None, None, None) == -1
    assert L.pack3d_global_attn(b, FAKE, None, FAKE, 64, FAKE, None, None) == -1
    assert L.pack3d_gate_mix(b, FAKE, FAKE, None, FAKE, None) == -1
    assert L.pack3d_build_cell_index(b, None, FAKE, None) == -1
    assert L.pack3d_check_packing(b, FAKE, FAKE, None, None) == -1
    args = [FAKE] * 5 + [None] + [FAKE] * 4
    assert L.pack3d_forward(b, *args, None, 10 ** 9, None) == -4      # no workspace
    assert "workspace" in pk.pack3d_last_error()
    assert L.pack3d_forward(b, *args, FAKE, 16, None) == -4           # too small
    assert L.pack3d_forward(b, *args, FAKE + 8, 10 ** 9, None) == -4  # misaligned
    assert "aligned" in pk.pack3d_last_error()
    assert L.pack3d_global_attn(b, FAKE, FAKE, FAKE, 0, FAKE, None, None) == -2
    assert L.pack3d_rope(b, FAKE, FAKE, 0, FAKE, None) == -2


def test_unsupported_group_ratio(pk):
    p = _prob(pk, n_q_heads=32, n_kv_heads=1)
    b = ctypes.byref(p)
    assert pk.LIB.pack3d_local_attn(b, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -3
    assert "Hq/Hkv" in pk.pack3d_last_error()


def test_workspace_size_matches_layout(pk):
    p = _prob(pk, grid=(64, 64, 64), n_q_heads=8, n_kv_heads=2, window=(3, 7, 7))
    n, m = 64 ** 3, 64 ** 3 // 16
    a256 = lambda b: (b + 255) // 256 * 256
    # the rotary table (32 pairs x max extent x (sin, cos) fp32), then rotated
    # K_loc, the summaries, their norms and kmax.  Both attention kernels
    # rotate Q in registers (no rotated-Q section) and the local branch
    # writes its gated share into the output (no fp32 o_loc section).
    table = a256(32 * 64 * 2 * 4)
    fp32_parts = a256(4 * 2 * m) + a256(4 * 2)
    bf16 = table + 2 * (n * 2 * 64 + 2 * 2 * m * 64) + fp32_parts
    assert pk.pack3d_forward_workspace_size(p) == bf16
    p.dtype = 0
    assert pk.pack3d_forward_workspace_size(p) == table + 4 * (n * 2 * 64 + 2 * 2 * m * 64) \
        + fp32_parts


def test_error_string_is_per_call(pk):
    p = _prob(pk, head_dim=16)
    assert pk.LIB.pack3d_rope(ctypes.byref(p), FAKE, FAKE, 1, FAKE, None) == -3
    assert pk.pack3d_last_error() != ""
    assert pk.pack3d_forward_workspace_size(_prob(pk)) > 0
    assert pk.pack3d_last_error() == ""


def test_training_entry_points_check_arguments_on_the_host(pk):
    """pack3d_forward_train and pack3d_backward: NULLs, missing or small
    buffers and unsupported problems are rejected before any launch."""
    L = pk.LIB
    p = _prob(pk, n_q_heads=8, n_kv_heads=2)                 # bf16, Hq/Hkv 4
    b = ctypes.byref(p)
    big = 10 ** 12
    fwd = [FAKE] * 5 + [None] + [FAKE] * 4                 # q .. out (a may be NULL)
    assert L.pack3d_forward_train(b, *fwd[:-1], None, FAKE, big, FAKE, big, None) == -1
    assert L.pack3d_forward_train(b, *fwd, None, big, FAKE, big, None) == -4
    assert "saved" in pk.pack3d_last_error()
    assert L.pack3d_forward_train(b, *fwd, FAKE, 16, FAKE, big, None) == -4
    assert L.pack3d_forward_train(b, *fwd, FAKE, big, FAKE + 8, big, None) == -4
    inp = [FAKE] * 5 + [None] + [FAKE] * 3                 # q .. gate
    outs = [FAKE] * 5 + [FAKE]                             # dq .. dv_cmp, dgate
    assert L.pack3d_backward(b, *inp, FAKE, big, None, *outs, FAKE, big, None) == -1
    assert L.pack3d_backward(b, *inp, FAKE, big, FAKE, *outs, None, big, None) == -4
    assert L.pack3d_backward(b, *inp, FAKE, 16, FAKE, *outs, FAKE, big, None) == -4
    f32 = _prob(pk, dtype=torch.float32, n_q_heads=8, n_kv_heads=2)
    assert L.pack3d_backward(ctypes.byref(f32), *inp, FAKE, big, FAKE, *outs, FAKE, big,
                             None) == -3
    assert "bf16" in pk.pack3d_last_error()
    g2 = _prob(pk, n_q_heads=4, n_kv_heads=2)              # Hq/Hkv 2
    assert L.pack3d_backward(ctypes.byref(g2), *inp, FAKE, big, FAKE, *outs, FAKE, big,
                             None) == -3


def test_training_buffer_sizes_match_layout(pk):
    p = _prob(pk, grid=(64, 64, 64), n_q_heads=8, n_kv_heads=2, window=(3, 7, 7))
    n, hq = 64 ** 3, 8
    a256 = lambda b: (b + 255) // 256 * 256
    assert pk.pack3d_saved_size(p) == 2 * a256(n * hq * 64 * 4) + 2 * a256(n * hq * 4)
    assert pk.pack3d_backward_workspace_size(p) > pk.pack3d_saved_size(p)
    bad = _prob(pk, head_dim=16)
    assert pk.pack3d_saved_size(bad) == 0
    assert pk.pack3d_backward_workspace_size(bad) == 0


def test_layer_entry_points_check_arguments_on_the_host(pk):
    """fp32 tensors, a bad width, NULL tensors and a short workspace are
    rejected before any launch."""
    L = pk.LIB
    p32 = _prob(pk, dtype=torch.float32)
    pbf = _prob(pk, dtype=torch.bfloat16, n_q_heads=4, n_kv_heads=1)
    f = ctypes.c_float(1e-5)
    assert L.pack3d_out_proj(ctypes.byref(p32), 512, FAKE, FAKE, FAKE, FAKE, None) == -3
    assert L.pack3d_out_proj(ctypes.byref(pbf), 100, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert "width" in pk.pack3d_last_error()
    assert L.pack3d_out_proj(ctypes.byref(pbf), 512, None, FAKE, FAKE, FAKE, None) == -1
    assert L.pack3d_layernorm_qkv(ctypes.byref(pbf), 512, FAKE, None, None, f, FAKE, FAKE, FAKE,
                                  FAKE, None, FAKE, FAKE, FAKE, None, None) == -1
    assert L.pack3d_layernorm_qkv(ctypes.byref(pbf), 512, FAKE, None, None, ctypes.c_float(0.0),
                                  FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                  None) == -2
    need = pk.pack3d_layer_workspace_size(pbf, 512)
    assert need > 0 and pk.pack3d_layer_workspace_size(p32, 512) == 0
    assert L.pack3d_layer_forward(ctypes.byref(pbf), 512, FAKE, None, None, f, FAKE, FAKE, None,
                                  FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == -4
    assert L.pack3d_layer_forward(ctypes.byref(pbf), 512, FAKE, None, None, f, FAKE, FAKE, None,
                                  FAKE, FAKE, FAKE, FAKE, None, need, None) == -4


def test_layer_workspace_layout(pk):
    """LayerNorm(h), the five projections, summaries, norms and the gated
    output, each section 256-byte aligned (the unrotated Q only for the
    coordinate-blind branch)."""
    a256 = lambda b: (b + 255) // 256 * 256
    p = _prob(pk, dtype=torch.bfloat16, n_q_heads=4, n_kv_heads=1)
    n, m, hq, hkv = 1024, 64, 4, 1
    want = (a256(2 * n * 512) + 2 * a256(2 * n * hq * 64) + 4 * a256(2 * n * hkv * 64)
            + 2 * a256(2 * hkv * m * 64) + a256(4 * hkv * m) + a256(4 * hkv))
    assert pk.pack3d_layer_workspace_size(p, 512) == want
    pb = _prob(pk, dtype=torch.bfloat16, n_q_heads=4, n_kv_heads=1, summary_mode="blind")
    assert pk.pack3d_layer_workspace_size(pb, 512) == want + a256(2 * n * hq * 64)


def test_misaligned_tensors_are_rejected_on_the_host(pk):
    """Every array argument must start on a 16-byte boundary; a misaligned
    pointer (a fake address, never dereferenced) is rejected with
    PACK3D_ERR_SHAPE before any launch, naming the argument."""
    L = pk.LIB
    p = _prob(pk, n_q_heads=8, n_kv_heads=2)
    b = ctypes.byref(p)
    big = 10 ** 12
    bad = FAKE + 8                                         # 8-byte aligned only
    assert L.pack3d_rope(b, FAKE, bad, 2, FAKE, None) == -2
    assert "y is not 16-byte aligned" in pk.pack3d_last_error()
    assert L.pack3d_block_summary(b, FAKE, FAKE, bad, FAKE, FAKE, FAKE, None) == -2
    assert "a is not" in pk.pack3d_last_error()
    assert L.pack3d_local_attn(b, FAKE, FAKE, FAKE, FAKE, FAKE + 4, None, None) == -2
    assert L.pack3d_global_attn(b, FAKE + 2, FAKE, FAKE, 64, FAKE, None, None) == -2
    assert L.pack3d_gate_mix(b, FAKE, FAKE, FAKE, bad, None) == -2
    assert L.pack3d_build_cell_index(b, bad, FAKE, None) == -2
    assert L.pack3d_check_packing(b, FAKE, FAKE, FAKE + 2, None) == -2
    fwd = [FAKE] * 10                                      # q .. out
    for i in range(10):
        args = list(fwd)
        args[i] = bad
        assert L.pack3d_forward(b, *args, FAKE, big, None) == -2, i
        assert "16-byte aligned" in pk.pack3d_last_error()
        assert L.pack3d_forward_train(b, *args, FAKE, big, FAKE, big, None) == -2, i
    inp = [FAKE] * 9                                       # q .. gate
    outs = [FAKE] * 6                                      # dq .. dgate
    assert L.pack3d_backward(b, *inp, FAKE, big, bad, *outs, FAKE, big, None) == -2
    assert "dout" in pk.pack3d_last_error()
    outs[5] = bad
    assert L.pack3d_backward(b, *inp, FAKE, big, FAKE, *outs, FAKE, big, None) == -2
    assert "dgate" in pk.pack3d_last_error()
    pbf = _prob(pk, dtype=torch.bfloat16, n_q_heads=4, n_kv_heads=1)
    assert L.pack3d_out_proj(ctypes.byref(pbf), 512, FAKE, FAKE, bad, FAKE, None) == -2
    assert "residual" in pk.pack3d_last_error()


def test_noalloc_forward_checks_on_the_host(pk):
    """pack3d_forward_noalloc: NULLs, misaligned tensors and problems whose
    workspace exceeds the static scratch array are rejected before the
    device is touched."""
    L = pk.LIB
    small = _prob(pk, n_q_heads=8, n_kv_heads=2)
    big = _prob(pk, grid=(64, 128, 128), n_q_heads=8, n_kv_heads=2, window=(3, 7, 7))
    assert pk.pack3d_forward_workspace_size(small) <= pk.NOALLOC_SCRATCH_BYTES
    assert pk.pack3d_forward_workspace_size(big) > pk.NOALLOC_SCRATCH_BYTES
    fwd = [FAKE] * 10
    assert L.pack3d_forward_noalloc(ctypes.byref(big), *fwd, None) == -4
    assert "static scratch" in pk.pack3d_last_error()
    nul = list(fwd)
    nul[0] = None
    assert L.pack3d_forward_noalloc(ctypes.byref(small), *nul, None) == -1
    mis = list(fwd)
    mis[9] = FAKE + 8
    assert L.pack3d_forward_noalloc(ctypes.byref(small), *mis, None) == -2
    assert "out is not 16-byte aligned" in pk.pack3d_last_error()
    text = open(HEADER).read()
    assert "#define PACK3D_NOALLOC_SCRATCH_BYTES (256u << 20)" in text
    assert pk.NOALLOC_SCRATCH_BYTES == 256 << 20
