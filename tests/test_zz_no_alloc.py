"""GPU: the allocation-free forward (pack3d_forward_noalloc, workspace in the
library's static scratch array) against pack3d_forward (caller workspace):
the same launches and kernels, so the outputs must be equal bit for bit, on
consecutive calls of decreasing size (the array keeps the previous call's
contents), for bf16 and fp32 problems."""

import numpy as np
import pytest
import torch

import synthgen as sg
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

W = sg.WORKLOADS


@pytest.fixture(scope="module")
def pk():
    from geometry_aware_local_amd import pack3d
    return pack3d


def _both(pk, w):
    inp = sg.make_inputs(w)
    d = gu.device_inputs(inp)
    prob = gu.problem(pk, w)
    args = (prob, d["q"], d["k_loc"], d["v_loc"], d["k_cmp"], d["v_cmp"], d["a"], d["coords"],
            d["cell_to_pos"], d["gate"])
    ref = pk.pack3d_forward(*args)
    out = torch.full_like(ref, float("nan"))
    pk.pack3d_forward_noalloc(*args, out=out)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_forward_matches_forward_on_consecutive_calls(pk):
    big = W["block_bf16_64x64x64"]                        # 262 144 tokens, ~76 MB of scratch
    small = big.with_(grid=(4, 16, 24), packing="random")  # 1 536 tokens, reuses the array
    tiny = W["tiny_f32_4x16x16"]                           # fp32, another layout of it
    for w in (big, small, tiny, big):
        print("noalloc forward", w.name, w.grid, flush=True)
        prob = gu.problem(pk, w)
        assert pk.pack3d_forward_workspace_size(prob) <= pk.NOALLOC_SCRATCH_BYTES
        ref, out = _both(pk, w)
        assert torch.equal(out, ref), w.name


def test_noalloc_rejects_problems_beyond_the_scratch_array(pk):
    w = W["random_bf16_64x128x128"]                      # 1 048 576 tokens, ~302 MB
    prob = gu.problem(pk, w)
    assert pk.pack3d_forward_workspace_size(prob) > pk.NOALLOC_SCRATCH_BYTES
    n = w.n_tokens
    q = torch.zeros((n, 8, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((n, 2, 64), dtype=torch.bfloat16, device="cuda")
    coords = torch.zeros((n, 3), dtype=torch.int32, device="cuda")
    c2p = torch.zeros((n,), dtype=torch.int32, device="cuda")
    gate = torch.zeros((n, 2), dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(pk.Pack3DError, match="ERR_WORKSPACE"):
        pk.pack3d_forward_noalloc(prob, q, kv, kv, kv, kv, None, coords, c2p, gate, out=out)
    assert "static scratch" in pk.pack3d_last_error()
