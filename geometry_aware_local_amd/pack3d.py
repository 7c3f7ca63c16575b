"""Python binding of libpack3d: the PACK3D local-global attention operator on MI355X
(forward, training forward and backward, and the layer around it).

Argument marshalling only.  Every step of the operator runs in libpack3d's
HIP kernels; PyTorch provides device memory and the current HIP stream.  The
functions carry the names of the C entry points declared in
``include/pack3d.h`` and take torch tensors in the layouts documented there:

* ``q``            ``[N, Hq, 64]``  float32 or bfloat16, packed token order
* ``k_*``, ``v_*`` ``[N, Hkv, 64]`` same dtype
* ``a``            ``[N, Hkv]``     float32 summary weights, or ``None`` (uniform)
* ``coords``       ``[N, 3]``       int32 (z, y, x)
* ``cell_to_pos``  ``[Z*Y*X]``      int32
* ``gate``         ``[N, 2]`` (or ``[N, Hq, 2]``) float32 logits, index 0 = local

There is no fallback: importing this module fails if ``libpack3d.so`` has not
been built (``python -m geometry_aware_local_amd.build``), and every call
raises :class:`Pack3DError` when the library rejects its arguments.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpack3d.so")

PACK3D_F32, PACK3D_BF16 = 0, 1
SUMMARY_MODES = ("token", "centre", "blind")      # pack3d_summary_mode 0, 1, 2
PACK3D_FORWARD_STAGES = 4
FORWARD_STAGE_NAMES = ("block_pass", "kmax+rope_table", "local_attn", "global_attn+gate")
STATUS = {0: "OK", -1: "ERR_NULL", -2: "ERR_SHAPE", -3: "ERR_UNSUPPORTED", -4: "ERR_WORKSPACE",
          -5: "ERR_PACKING", -6: "ERR_HIP"}

EXPORTS = (
    "pack3d_rope", "pack3d_block_summary", "pack3d_local_attn", "pack3d_global_attn",
    "pack3d_gate_mix", "pack3d_forward", "pack3d_forward_timed", "pack3d_forward_workspace_size",
    "pack3d_build_cell_index", "pack3d_check_packing", "pack3d_last_error",
    "pack3d_backend_info", "pack3d_version", "pack3d_saved_size", "pack3d_forward_train",
    "pack3d_backward_workspace_size", "pack3d_backward", "pack3d_layernorm_qkv",
    "pack3d_out_proj", "pack3d_layer_forward", "pack3d_layer_workspace_size",
    "pack3d_forward_noalloc",
)
NOALLOC_SCRATCH_BYTES = 256 << 20      # PACK3D_NOALLOC_SCRATCH_BYTES


class Pack3DError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libpack3d {STATUS.get(code, code)}: {msg}")
        self.code = code


class Problem(ctypes.Structure):
    """Mirror of ``pack3d_problem``."""
    _fields_ = [
        ("grid", ctypes.c_int32 * 3),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32 * 3),
        ("block", ctypes.c_int32 * 3),
        ("rope_pairs", ctypes.c_int32 * 3),
        ("rope_base", ctypes.c_double),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("gate_per_head", ctypes.c_int32),
        ("summary_mode", ctypes.c_int32),
    ]

    @property
    def n_tokens(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]

    @property
    def n_blocks(self) -> int:
        return self.n_tokens // (self.block[0] * self.block[1] * self.block[2])

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == PACK3D_BF16 else torch.float32


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m geometry_aware_local_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, V, I32, SZ = ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "pack3d_rope": [P, V, V, I32, V, V],
        "pack3d_block_summary": [P, V, V, V, V, V, V, V],
        "pack3d_local_attn": [P, V, V, V, V, V, V, V],
        "pack3d_global_attn": [P, V, V, V, I32, V, V, V],
        "pack3d_gate_mix": [P, V, V, V, V, V],
        "pack3d_forward": [P, V, V, V, V, V, V, V, V, V, V, V, SZ, V],
        "pack3d_forward_noalloc": [P, V, V, V, V, V, V, V, V, V, V, V],
        "pack3d_forward_timed": [P, V, V, V, V, V, V, V, V, V, V, V, SZ, V,
                                 ctypes.POINTER(ctypes.c_void_p), I32],
        "pack3d_build_cell_index": [P, V, V, V],
        "pack3d_check_packing": [P, V, V, V, V],
        "pack3d_forward_train": [P, V, V, V, V, V, V, V, V, V, V, V, SZ, V, SZ, V],
        "pack3d_backward": [P, V, V, V, V, V, V, V, V, V, V, SZ, V, V, V, V, V, V, V, V, SZ, V],
        "pack3d_layernorm_qkv": [P, I32, V, V, V, ctypes.c_float, V, V, V, V, V, V, V, V, V,
                                 V],
        "pack3d_out_proj": [P, I32, V, V, V, V, V],
        "pack3d_layer_forward": [P, I32, V, V, V, ctypes.c_float, V, V, V, V, V, V, V, V, SZ,
                                 V],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = args, ctypes.c_int
    for name in ("pack3d_forward_workspace_size", "pack3d_saved_size",
                 "pack3d_backward_workspace_size"):
        getattr(lib, name).argtypes, getattr(lib, name).restype = [P], ctypes.c_size_t
    for name in ("pack3d_last_error", "pack3d_backend_info"):
        getattr(lib, name).argtypes, getattr(lib, name).restype = [], ctypes.c_char_p
    lib.pack3d_layer_workspace_size.argtypes = [P, I32]
    lib.pack3d_layer_workspace_size.restype = ctypes.c_size_t
    lib.pack3d_version.argtypes, lib.pack3d_version.restype = [], ctypes.c_int
    return lib


LIB = _load()


def make_problem(grid: Sequence[int], n_q_heads: int, n_kv_heads: int,
                 window: Sequence[int] = (3, 7, 7), block: Sequence[int] = (1, 4, 4),
                 dtype: torch.dtype = torch.bfloat16, rope_pairs: Sequence[int] = (11, 11, 10),
                 rope_base: float = 10000.0, scale: float = 0.0, head_dim: int = 64,
                 gate_per_head: bool = False, summary_mode="token") -> Problem:
    """``summary_mode``: "token" (rotation before the block sum, the exact
    form), "centre" (pooled keys rotated at the block centre) or "blind"
    (no rotation in the compressed branch), or the matching int 0/1/2."""
    p = Problem()
    p.grid[:] = list(grid)
    p.n_q_heads, p.n_kv_heads, p.head_dim = n_q_heads, n_kv_heads, head_dim
    p.window[:] = list(window)
    p.block[:] = list(block)
    p.rope_pairs[:] = list(rope_pairs)
    p.rope_base, p.scale = rope_base, scale
    p.dtype = PACK3D_BF16 if dtype == torch.bfloat16 else PACK3D_F32
    p.gate_per_head = int(gate_per_head)
    p.summary_mode = (summary_mode if isinstance(summary_mode, int)
                      else SUMMARY_MODES.index(summary_mode))
    return p


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor], dtype: Optional[torch.dtype] = None,
         shape: Optional[tuple] = None, name: str = "") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name}: tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(rc: int) -> None:
    if rc != 0:
        raise Pack3DError(rc, LIB.pack3d_last_error().decode())


def _empty(shape, dtype, like: torch.Tensor) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=like.device)


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def pack3d_version() -> int:
    return LIB.pack3d_version()


def pack3d_backend_info() -> str:
    return LIB.pack3d_backend_info().decode()


def pack3d_last_error() -> str:
    return LIB.pack3d_last_error().decode()


def pack3d_forward_workspace_size(prob: Problem) -> int:
    return LIB.pack3d_forward_workspace_size(ctypes.byref(prob))


def pack3d_rope(prob: Problem, x: torch.Tensor, coords: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """R(c_i) x[i, h] for every token and head (out may be x: in place)."""
    n, dt = prob.n_tokens, prob.torch_dtype
    if x.dim() != 3:
        raise ValueError("x must be [N, H, 64]")
    heads = x.shape[1]
    out = _empty(x.shape, dt, x) if out is None else out
    _check(LIB.pack3d_rope(ctypes.byref(prob), _ptr(x, dt, (n, heads, 64), "x"),
                           _ptr(out, dt, (n, heads, 64), "out"), heads,
                           _ptr(coords, torch.int32, (n, 3), "coords"), _stream(x.device)))
    return out


def pack3d_block_summary(prob: Problem, k_cmp: torch.Tensor, v_cmp: torch.Tensor,
                         a: Optional[torch.Tensor], cell_to_pos: torch.Tensor):
    """Block summaries (k_sum, v_sum), each [Hkv, M, 64]."""
    n, hkv, m, dt = prob.n_tokens, prob.n_kv_heads, prob.n_blocks, prob.torch_dtype
    ks = _empty((hkv, m, 64), dt, k_cmp)
    vs = _empty((hkv, m, 64), dt, k_cmp)
    _check(LIB.pack3d_block_summary(
        ctypes.byref(prob), _ptr(k_cmp, dt, (n, hkv, 64), "k_cmp"),
        _ptr(v_cmp, dt, (n, hkv, 64), "v_cmp"), _ptr(a, torch.float32, (n, hkv), "a"),
        _ptr(cell_to_pos, torch.int32, (n,), "cell_to_pos"), ks.data_ptr(), vs.data_ptr(),
        _stream(k_cmp.device)))
    return ks, vs


def pack3d_local_attn(prob: Problem, q_rot: torch.Tensor, k_rot: torch.Tensor, v: torch.Tensor,
                      cell_to_pos: torch.Tensor, with_lse: bool = False):
    """Local branch o_loc [N, Hq, 64] fp32 (and lse [N, Hq] if asked)."""
    n, hq, hkv, dt = prob.n_tokens, prob.n_q_heads, prob.n_kv_heads, prob.torch_dtype
    o = _empty((n, hq, 64), torch.float32, q_rot)
    lse = _empty((n, hq), torch.float32, q_rot) if with_lse else None
    _check(LIB.pack3d_local_attn(
        ctypes.byref(prob), _ptr(q_rot, dt, (n, hq, 64), "q_rot"),
        _ptr(k_rot, dt, (n, hkv, 64), "k_rot"), _ptr(v, dt, (n, hkv, 64), "v"),
        _ptr(cell_to_pos, torch.int32, (n,), "cell_to_pos"), o.data_ptr(),
        None if lse is None else lse.data_ptr(), _stream(q_rot.device)))
    return (o, lse) if with_lse else o


def pack3d_global_attn(prob: Problem, q_rot: torch.Tensor, k_sum: torch.Tensor,
                       v_sum: torch.Tensor, with_lse: bool = False):
    """Compressed branch o_cmp [N, Hq, 64] fp32 over all m = k_sum.shape[1] summaries."""
    n, hq, hkv, dt = prob.n_tokens, prob.n_q_heads, prob.n_kv_heads, prob.torch_dtype
    m = k_sum.shape[1]
    o = _empty((n, hq, 64), torch.float32, q_rot)
    lse = _empty((n, hq), torch.float32, q_rot) if with_lse else None
    _check(LIB.pack3d_global_attn(
        ctypes.byref(prob), _ptr(q_rot, dt, (n, hq, 64), "q_rot"),
        _ptr(k_sum, dt, (hkv, m, 64), "k_sum"), _ptr(v_sum, dt, (hkv, m, 64), "v_sum"), m,
        o.data_ptr(), None if lse is None else lse.data_ptr(), _stream(q_rot.device)))
    return (o, lse) if with_lse else o


def pack3d_gate_mix(prob: Problem, o_loc: torch.Tensor, o_cmp: torch.Tensor,
                    gate: torch.Tensor) -> torch.Tensor:
    n, hq, dt = prob.n_tokens, prob.n_q_heads, prob.torch_dtype
    gshape = (n, hq, 2) if prob.gate_per_head else (n, 2)
    out = _empty((n, hq, 64), dt, o_loc)
    _check(LIB.pack3d_gate_mix(
        ctypes.byref(prob), _ptr(o_loc, torch.float32, (n, hq, 64), "o_loc"),
        _ptr(o_cmp, torch.float32, (n, hq, 64), "o_cmp"),
        _ptr(gate, torch.float32, gshape, "gate"), out.data_ptr(), _stream(o_loc.device)))
    return out


def alloc_workspace(prob: Problem, device) -> torch.Tensor:
    """A caller-owned workspace of the size pack3d_forward needs (uint8)."""
    size = pack3d_forward_workspace_size(prob)
    if size == 0:
        _check(LIB.pack3d_forward_workspace_size(ctypes.byref(prob)) or -2)
    return torch.empty(size, dtype=torch.uint8, device=device)


def _forward_args(prob, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos, gate,
                  workspace, out):
    n, hq, hkv, dt = prob.n_tokens, prob.n_q_heads, prob.n_kv_heads, prob.torch_dtype
    gshape = (n, hq, 2) if prob.gate_per_head else (n, 2)
    ws = alloc_workspace(prob, q.device) if workspace is None else workspace
    out = _empty((n, hq, 64), dt, q) if out is None else out
    args = (ctypes.byref(prob), _ptr(q, dt, (n, hq, 64), "q"),
            _ptr(k_loc, dt, (n, hkv, 64), "k_loc"), _ptr(v_loc, dt, (n, hkv, 64), "v_loc"),
            _ptr(k_cmp, dt, (n, hkv, 64), "k_cmp"), _ptr(v_cmp, dt, (n, hkv, 64), "v_cmp"),
            _ptr(a, torch.float32, (n, hkv), "a"), _ptr(coords, torch.int32, (n, 3), "coords"),
            _ptr(cell_to_pos, torch.int32, (n,), "cell_to_pos"),
            _ptr(gate, torch.float32, gshape, "gate"), _ptr(out, dt, (n, hq, 64), "out"),
            ws.data_ptr(), ws.numel(), _stream(q.device))
    # the caller keeps ws alive until the launch: args hold only its address
    return args, out, ws


def pack3d_forward(prob: Problem, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos, gate,
                   workspace: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole forward: out [N, Hq, 64] in the input dtype."""
    args, out, ws = _forward_args(prob, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos,
                                  gate, workspace, out)
    _check(LIB.pack3d_forward(*args))
    del ws
    return out


def pack3d_forward_noalloc(prob: Problem, q, k_loc, v_loc, k_cmp, v_cmp, a, coords,
                           cell_to_pos, gate, out: torch.Tensor) -> torch.Tensor:
    """The forward with the library's static scratch array as its workspace
    (no device allocation in the call; ``out`` is given by the caller)."""
    n, hq, hkv, dt = prob.n_tokens, prob.n_q_heads, prob.n_kv_heads, prob.torch_dtype
    gshape = (n, hq, 2) if prob.gate_per_head else (n, 2)
    _check(LIB.pack3d_forward_noalloc(
        ctypes.byref(prob), _ptr(q, dt, (n, hq, 64), "q"),
        _ptr(k_loc, dt, (n, hkv, 64), "k_loc"), _ptr(v_loc, dt, (n, hkv, 64), "v_loc"),
        _ptr(k_cmp, dt, (n, hkv, 64), "k_cmp"), _ptr(v_cmp, dt, (n, hkv, 64), "v_cmp"),
        _ptr(a, torch.float32, (n, hkv), "a"), _ptr(coords, torch.int32, (n, 3), "coords"),
        _ptr(cell_to_pos, torch.int32, (n,), "cell_to_pos"),
        _ptr(gate, torch.float32, gshape, "gate"), _ptr(out, dt, (n, hq, 64), "out"),
        _stream(q.device)))
    return out


def pack3d_forward_timed(prob: Problem, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos,
                         gate, events, workspace: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """pack3d_forward recording ``events`` (PACK3D_FORWARD_STAGES + 1 timing
    torch.cuda.Event objects) around its stages; stage i lasts
    ``events[i].elapsed_time(events[i + 1])`` ms."""
    if len(events) != PACK3D_FORWARD_STAGES + 1:
        raise ValueError(f"need {PACK3D_FORWARD_STAGES + 1} events")
    for e in events:          # torch creates the HIP event at its first record
        if not e.cuda_event:
            e.record()
    handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    args, out, ws = _forward_args(prob, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos,
                                  gate, workspace, out)
    _check(LIB.pack3d_forward_timed(*args, handles, len(events)))
    del ws
    return out


def pack3d_saved_size(prob: Problem) -> int:
    return int(LIB.pack3d_saved_size(ctypes.byref(prob)))


def pack3d_backward_workspace_size(prob: Problem) -> int:
    return int(LIB.pack3d_backward_workspace_size(ctypes.byref(prob)))


def _buffer(size_fn, prob: Problem, device) -> torch.Tensor:
    size = size_fn(prob)
    if size == 0:
        _check(-2)
    return torch.empty(size, dtype=torch.uint8, device=device)


def pack3d_forward_train(prob: Problem, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos,
                         gate, workspace: Optional[torch.Tensor] = None,
                         saved: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None):
    """The forward for training: returns ``(out, saved)``, ``saved`` holding
    the state pack3d_backward needs (o_loc, o_cmp, lse_loc, lse_cmp)."""
    args, out, ws = _forward_args(prob, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos,
                                  gate, workspace, out)
    saved = _buffer(pack3d_saved_size, prob, q.device) if saved is None else saved
    # C order: ..., out, saved, saved_bytes, workspace, ws_bytes, stream
    _check(LIB.pack3d_forward_train(*args[:11], saved.data_ptr(), saved.numel(), *args[11:]))
    del ws
    return out, saved


def saved_views(prob: Problem, saved: torch.Tensor) -> dict:
    """fp32 views of the saved state: o_loc, o_cmp [N, Hq, 64], lse_loc,
    lse_cmp [N, Hq] (each section 256-byte aligned)."""
    n, hq = prob.n_tokens, prob.n_q_heads
    a256 = lambda b: (b + 255) // 256 * 256
    sizes = [("o_loc", n * hq * 64), ("o_cmp", n * hq * 64), ("lse_loc", n * hq),
             ("lse_cmp", n * hq)]
    out, off = {}, 0
    for name, cnt in sizes:
        t = saved[off:off + cnt * 4].view(torch.float32)
        out[name] = t.view(n, hq, 64) if name.startswith("o_") else t.view(n, hq)
        off += a256(cnt * 4)
    return out


def pack3d_backward(prob: Problem, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos, gate,
                    saved: torch.Tensor, dout: torch.Tensor,
                    workspace: Optional[torch.Tensor] = None,
                    grads: Optional[dict] = None) -> dict:
    """Gradients of the forward's output for upstream ``dout``: a dict with
    dq [N,Hq,64], dk_loc, dv_loc, dk_cmp, dv_cmp [N,Hkv,64] (input dtype) and
    dgate (fp32, the gate logits' shape).  ``grads`` (a dict returned by an
    earlier call) supplies the output tensors to overwrite."""
    n, hq, hkv, dt = prob.n_tokens, prob.n_q_heads, prob.n_kv_heads, prob.torch_dtype
    gshape = (n, hq, 2) if prob.gate_per_head else (n, 2)
    ws = _buffer(pack3d_backward_workspace_size, prob, q.device) if workspace is None else workspace
    if grads is None:
        g = {"dq": _empty((n, hq, 64), dt, q)}
        for name in ("dk_loc", "dv_loc", "dk_cmp", "dv_cmp"):
            g[name] = _empty((n, hkv, 64), dt, q)
        g["dgate"] = _empty(gshape, torch.float32, q)
    else:
        g = grads
        want = {"dq": (n, hq, 64), "dk_loc": (n, hkv, 64), "dv_loc": (n, hkv, 64),
                "dk_cmp": (n, hkv, 64), "dv_cmp": (n, hkv, 64), "dgate": gshape}
        for name, shape in want.items():
            _ptr(g[name], torch.float32 if name == "dgate" else dt, shape, name)
    _check(LIB.pack3d_backward(
        ctypes.byref(prob), _ptr(q, dt, (n, hq, 64), "q"),
        _ptr(k_loc, dt, (n, hkv, 64), "k_loc"), _ptr(v_loc, dt, (n, hkv, 64), "v_loc"),
        _ptr(k_cmp, dt, (n, hkv, 64), "k_cmp"), _ptr(v_cmp, dt, (n, hkv, 64), "v_cmp"),
        _ptr(a, torch.float32, (n, hkv), "a"), _ptr(coords, torch.int32, (n, 3), "coords"),
        _ptr(cell_to_pos, torch.int32, (n,), "cell_to_pos"),
        _ptr(gate, torch.float32, gshape, "gate"), _ptr(saved, torch.uint8, None, "saved"),
        saved.numel(), _ptr(dout, dt, (n, hq, 64), "dout"), g["dq"].data_ptr(),
        g["dk_loc"].data_ptr(), g["dv_loc"].data_ptr(), g["dk_cmp"].data_ptr(),
        g["dv_cmp"].data_ptr(), g["dgate"].data_ptr(), ws.data_ptr(), ws.numel(),
        _stream(q.device)))
    return g


def pack3d_build_cell_index(prob: Problem, coords: torch.Tensor,
                            check: bool = True) -> torch.Tensor:
    """cell_to_pos for ``coords``.  Cells no token maps to keep -1; with
    ``check`` (the default; it synchronises) the index is verified with
    pack3d_check_packing and ``ValueError`` is raised unless coords is a
    bijection onto the lattice, since the kernels dereference every entry."""
    n = prob.n_tokens
    c2p = torch.full((n,), -1, dtype=torch.int32, device=coords.device)
    _check(LIB.pack3d_build_cell_index(ctypes.byref(prob),
                                        _ptr(coords, torch.int32, (n, 3), "coords"),
                                        c2p.data_ptr(), _stream(coords.device)))
    if check:
        bad = pack3d_check_packing(prob, coords, c2p)
        if bad:
            raise ValueError(f"coords is not a bijection onto the lattice: {bad} tokens are "
                             "outside it or share a cell")
    return c2p


def pack3d_check_packing(prob: Problem, coords: torch.Tensor, cell_to_pos: torch.Tensor) -> int:
    """Number of tokens whose coordinates disagree with cell_to_pos (syncs)."""
    n = prob.n_tokens
    bad = torch.empty(1, dtype=torch.int32, device=coords.device)
    _check(LIB.pack3d_check_packing(ctypes.byref(prob),
                                     _ptr(coords, torch.int32, (n, 3), "coords"),
                                     _ptr(cell_to_pos, torch.int32, (n,), "cell_to_pos"),
                                     bad.data_ptr(), _stream(coords.device)))
    return int(bad.item())


# --------------------------------------------------------------------------
# the layer around the operator (bf16): LayerNorm + projections (+ RoPE),
# output projection + residual, and the whole layer
# --------------------------------------------------------------------------

def pack3d_layernorm_qkv(prob: Problem, h, gamma, beta, w_qkv, coords, eps: float = 1e-5,
                         with_q_raw: bool = False) -> dict:
    """LayerNorm(h) projected by the stacked weight ``w_qkv`` [Hq*64 + 4*Hkv*64,
    C]: returns q_rot, k_rot (rotated by R(c)), v_loc, k_cmp, v_cmp, the
    normalised input x_norm [N, C] and, with ``with_q_raw``, q_raw."""
    n, hq, hkv, dt = prob.n_tokens, prob.n_q_heads, prob.n_kv_heads, prob.torch_dtype
    width = h.shape[1]
    out = {"q_rot": _empty((n, hq, 64), dt, h), "k_rot": _empty((n, hkv, 64), dt, h)}
    for name in ("v_loc", "k_cmp", "v_cmp"):
        out[name] = _empty((n, hkv, 64), dt, h)
    out["x_norm"] = _empty((n, width), dt, h)
    if with_q_raw:
        out["q_raw"] = _empty((n, hq, 64), dt, h)
    _check(LIB.pack3d_layernorm_qkv(
        ctypes.byref(prob), width, _ptr(h, dt, (n, width), "h"),
        _ptr(gamma, torch.float32, (width,), "gamma"), _ptr(beta, torch.float32, (width,), "beta"),
        eps, _ptr(w_qkv, dt, ((hq + 4 * hkv) * 64, width), "w_qkv"),
        _ptr(coords, torch.int32, (n, 3), "coords"), out["x_norm"].data_ptr(),
        out["q_rot"].data_ptr(), out["q_raw"].data_ptr() if with_q_raw else None,
        out["k_rot"].data_ptr(), out["v_loc"].data_ptr(), out["k_cmp"].data_ptr(),
        out["v_cmp"].data_ptr(), _stream(h.device)))
    return out


def pack3d_out_proj(prob: Problem, o, w_o, residual) -> torch.Tensor:
    """residual + o W_o^T with o [N, Hq*64] (or [N, Hq, 64]), W_o [C, Hq*64]."""
    n, hq, dt = prob.n_tokens, prob.n_q_heads, prob.torch_dtype
    width = residual.shape[1]
    out = _empty((n, width), dt, residual)
    _check(LIB.pack3d_out_proj(
        ctypes.byref(prob), width, _ptr(o.reshape(n, hq * 64), dt, (n, hq * 64), "o"),
        _ptr(w_o, dt, (width, hq * 64), "w_o"), _ptr(residual, dt, (n, width), "residual"),
        out.data_ptr(), _stream(residual.device)))
    return out


def pack3d_layer_workspace_size(prob: Problem, width: int) -> int:
    return int(LIB.pack3d_layer_workspace_size(ctypes.byref(prob), width))


def pack3d_layer_forward(prob: Problem, h, gamma, beta, w_qkv, w_o, a, coords, cell_to_pos,
                         gate, eps: float = 1e-5, workspace: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """h + PACK3D(projections of LayerNorm(h)) W_o^T, [N, C]."""
    n, hq, hkv, dt = prob.n_tokens, prob.n_q_heads, prob.n_kv_heads, prob.torch_dtype
    width = h.shape[1]
    gshape = (n, hq, 2) if prob.gate_per_head else (n, 2)
    if workspace is None:
        size = pack3d_layer_workspace_size(prob, width)
        if size == 0:
            _check(LIB.pack3d_layer_forward(ctypes.byref(prob), width, None, None, None, eps,
                                            None, None, None, None, None, None, None, None, 0,
                                            None))
        workspace = torch.empty(size, dtype=torch.uint8, device=h.device)
    out = _empty((n, width), dt, h) if out is None else out
    _check(LIB.pack3d_layer_forward(
        ctypes.byref(prob), width, _ptr(h, dt, (n, width), "h"),
        _ptr(gamma, torch.float32, (width,), "gamma"), _ptr(beta, torch.float32, (width,), "beta"),
        eps, _ptr(w_qkv, dt, ((hq + 4 * hkv) * 64, width), "w_qkv"),
        _ptr(w_o, dt, (width, hq * 64), "w_o"), _ptr(a, torch.float32, (n, hkv), "a"),
        _ptr(coords, torch.int32, (n, 3), "coords"),
        _ptr(cell_to_pos, torch.int32, (n,), "cell_to_pos"), _ptr(gate, torch.float32, gshape, "gate"),
        _ptr(out, dt, (n, width), "out"), workspace.data_ptr(), workspace.numel(),
        _stream(h.device)))
    return out
