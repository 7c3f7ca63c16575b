// libpack3d C ABI: argument validation, problem geometry, workspace layout
// and the launch sequence of the forward.  No device memory is allocated and
// no host synchronisation happens here.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <string>

#include "pack3d_internal.h"

using namespace pack3d;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return PACK3D_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PACK3D_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// Validate a problem and derive its geometry.  Host only, reads no device data.
int make_geom(const pack3d_problem* p, Geom* g) {
  if (!p) return fail(PACK3D_ERR_NULL, "problem is NULL");
  for (int a = 0; a < 3; ++a)
    if (p->grid[a] < 1) return fail(PACK3D_ERR_SHAPE, "grid[%d] = %d must be >= 1", a, p->grid[a]);
  const int64_t n = (int64_t)p->grid[0] * p->grid[1] * p->grid[2];
  if (n >= ((int64_t)1 << 31))
    return fail(PACK3D_ERR_SHAPE, "N = %lld tokens does not fit int32 positions", (long long)n);
  if (p->head_dim != kHeadDim)
    return fail(PACK3D_ERR_UNSUPPORTED, "head_dim %d unsupported (only 64)", p->head_dim);
  if (p->n_q_heads < 1 || p->n_kv_heads < 1)
    return fail(PACK3D_ERR_SHAPE, "head counts must be >= 1 (Hq %d, Hkv %d)", p->n_q_heads,
                p->n_kv_heads);
  if (p->n_q_heads % p->n_kv_heads)
    return fail(PACK3D_ERR_SHAPE, "Hq %d is not a multiple of Hkv %d", p->n_q_heads, p->n_kv_heads);
  for (int a = 0; a < 3; ++a) {
    if (p->window[a] < 1 || p->window[a] % 2 == 0)
      return fail(PACK3D_ERR_SHAPE, "window[%d] = %d must be odd and >= 1", a, p->window[a]);
  }
  if (p->window[1] > 7 || p->window[2] > 7 || p->window[0] > 31)
    return fail(PACK3D_ERR_UNSUPPORTED, "window %dx%dx%d unsupported (y, x <= 7; z <= 31)",
                p->window[0], p->window[1], p->window[2]);
  int vol = 1;
  for (int a = 0; a < 3; ++a) {
    if (p->block[a] < 1) return fail(PACK3D_ERR_SHAPE, "block[%d] = %d must be >= 1", a, p->block[a]);
    if (p->grid[a] % p->block[a])
      return fail(PACK3D_ERR_SHAPE, "block[%d] = %d does not divide grid[%d] = %d", a, p->block[a],
                  a, p->grid[a]);
    vol *= p->block[a];
  }
  if (vol > kMaxBlockVol)
    return fail(PACK3D_ERR_UNSUPPORTED, "block volume %d unsupported (max %d)", vol, kMaxBlockVol);
  int pairs = 0;
  for (int a = 0; a < 3; ++a) {
    if (p->rope_pairs[a] < 0) return fail(PACK3D_ERR_SHAPE, "rope_pairs[%d] < 0", a);
    pairs += p->rope_pairs[a];
  }
  if (2 * pairs > p->head_dim)
    return fail(PACK3D_ERR_SHAPE, "2 * sum(rope_pairs) = %d exceeds head_dim", 2 * pairs);
  if (!(p->rope_base > 0.0) || !isfinite(p->rope_base))
    return fail(PACK3D_ERR_SHAPE, "rope_base must be finite and > 0");
  if (p->dtype != PACK3D_F32 && p->dtype != PACK3D_BF16)
    return fail(PACK3D_ERR_UNSUPPORTED, "dtype %d unsupported", p->dtype);
  if (p->gate_per_head != 0 && p->gate_per_head != 1)
    return fail(PACK3D_ERR_SHAPE, "gate_per_head must be 0 or 1");
  if (!isfinite(p->scale)) return fail(PACK3D_ERR_SHAPE, "scale is not finite");
  if (p->summary_mode < PACK3D_SUMMARY_TOKEN || p->summary_mode > PACK3D_SUMMARY_BLIND)
    return fail(PACK3D_ERR_SHAPE, "summary_mode %d unknown (0 token, 1 centre, 2 blind)",
                p->summary_mode);

  g->Z = p->grid[0];
  g->Y = p->grid[1];
  g->X = p->grid[2];
  g->N = n;
  g->Hq = p->n_q_heads;
  g->Hkv = p->n_kv_heads;
  g->G = p->n_q_heads / p->n_kv_heads;
  g->rz = p->window[0] / 2;
  g->ry = p->window[1] / 2;
  g->rx = p->window[2] / 2;
  g->bz = p->block[0];
  g->by = p->block[1];
  g->bx = p->block[2];
  g->bvol = vol;
  g->M = n / vol;
  g->scale = p->scale > 0.0f ? p->scale : (float)(1.0 / sqrt((double)p->head_dim));
  g->bf16 = p->dtype == PACK3D_BF16;
  g->gate_per_head = p->gate_per_head;
  g->summary_mode = p->summary_mode;
  // rotary table: pair p = r-th pair of axis a, omega = base^(-r/m_a), stored
  // in turns (omega / 2pi)
  memset(&g->rope, 0, sizeof g->rope);
  int q = 0;
  for (int a = 0; a < 3; ++a)
    for (int r = 0; r < p->rope_pairs[a]; ++r, ++q) {
      g->rope.axis[q] = a;
      g->rope.nu[q] = pow(p->rope_base, -(double)r / (double)p->rope_pairs[a]) /
                      (2.0 * 3.14159265358979323846);
    }
  g->rope.npairs = q;
  return ok();
}

bool local_supported(const Geom& g) {
  return g.G == 1 || g.G == 2 || g.G == 4 || g.G == 8 || g.G == 16;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// The forward's workspace: the lattice's rotary table, rotated K_loc, the
// summaries (keys pre-scaled), their norms and the per-group maximum norm.
// Both attention kernels rotate Q in registers, so no rotated Q is stored,
// and the local branch writes its gated share straight into the output, so
// no o_loc buffer exists.
struct WsLayout {
  size_t tab, k_rot, k_sum, v_sum, knorm, kmax, total;
};

WsLayout ws_layout(const Geom& g) {
  const size_t es = g.bf16 ? 2 : 4;
  WsLayout w;
  size_t off = 0;
  w.tab = off;
  off += align256(rope_table_bytes(g));
  w.k_rot = off;
  off += align256((size_t)g.N * g.Hkv * 64 * es);
  w.k_sum = off;
  off += align256((size_t)g.Hkv * g.M * 64 * es);
  w.v_sum = off;
  off += align256((size_t)g.Hkv * g.M * 64 * es);
  w.knorm = off;
  off += align256((size_t)g.Hkv * g.M * 4);
  w.kmax = off;
  off += align256((size_t)g.Hkv * 4);
  w.total = off;
  return w;
}

// The forward's saved state for the backward: o_loc, o_cmp fp32 [N, Hq, 64],
// lse_loc, lse_cmp fp32 [N, Hq].
struct SavedLayout {
  size_t o_loc, o_cmp, lse_loc, lse_cmp, total;
};

SavedLayout saved_layout(const Geom& g) {
  SavedLayout l;
  size_t off = 0;
  l.o_loc = off;
  off += align256((size_t)g.N * g.Hq * 64 * 4);
  l.o_cmp = off;
  off += align256((size_t)g.N * g.Hq * 64 * 4);
  l.lse_loc = off;
  off += align256((size_t)g.N * g.Hq * 4);
  l.lse_cmp = off;
  off += align256((size_t)g.N * g.Hq * 4);
  l.total = off;
  return l;
}

struct BwdLayout {
  size_t q_rot, k_rot, k_sum, v_sum, dlo, dco, d_loc, d_cmp, nls_cmp, dq_acc, dk_part, dv_part,
      total;
};

BwdLayout bwd_layout(const Geom& g) {
  BwdLayout w;
  const size_t nsplit = (size_t)glob_dkv_splits(g);
  size_t off = 0;
  auto take = [&](size_t& at, size_t bytes) {
    at = off;
    off += align256(bytes);
  };
  take(w.q_rot, (size_t)g.N * g.Hq * 64 * 2);
  take(w.k_rot, (size_t)g.N * g.Hkv * 64 * 2);
  take(w.k_sum, (size_t)g.Hkv * g.M * 64 * 2);
  take(w.v_sum, (size_t)g.Hkv * g.M * 64 * 2);
  take(w.dlo, (size_t)g.N * g.Hq * 64 * 2);
  take(w.dco, (size_t)g.N * g.Hq * 64 * 2);
  take(w.d_loc, (size_t)g.N * g.Hq * 4);
  take(w.d_cmp, (size_t)g.N * g.Hq * 4);
  take(w.nls_cmp, (size_t)g.N * g.Hq * 4);
  take(w.dq_acc, (size_t)g.N * g.Hq * 64 * 4);
  take(w.dk_part, nsplit * g.Hkv * g.M * 64 * 4);
  take(w.dv_part, nsplit * g.Hkv * g.M * 64 * 4);
  w.total = off;
  return w;
}

// Every device array must start on a 16-byte boundary: the kernels move rows
// with 16-byte vector loads and stores and 16-byte direct-to-LDS copies.
// Host check only (the pointer value), before any launch.
struct Arr {
  const void* p;
  const char* name;
};

int check_aligned(const char* fn, std::initializer_list<Arr> arrs) {
  for (const Arr& a : arrs)
    if (a.p && ((uintptr_t)a.p & 15))
      return fail(PACK3D_ERR_SHAPE, "%s: %s is not 16-byte aligned", fn, a.name);
  return PACK3D_OK;
}

// The operator's inputs and output, as the forward entry points take them.
int check_tensors(const char* fn, const void* q, const void* k_loc, const void* v_loc,
                  const void* k_cmp, const void* v_cmp, const float* a, const int32_t* coords,
                  const int32_t* cell_to_pos, const float* gate_logits, const void* last,
                  const char* last_name = "out") {
  return check_aligned(fn, {{q, "q"}, {k_loc, "k_loc"}, {v_loc, "v_loc"}, {k_cmp, "k_cmp"},
                            {v_cmp, "v_cmp"}, {a, "a"}, {coords, "coords"},
                            {cell_to_pos, "cell_to_pos"}, {gate_logits, "gate_logits"},
                            {last, last_name}});
}

int check_buffer(void* p, size_t have, size_t need, const char* fn, const char* what) {
  if (!p) return fail(PACK3D_ERR_WORKSPACE, "%s: %s is NULL", fn, what);
  if (have < need)
    return fail(PACK3D_ERR_WORKSPACE, "%s: %s %zu bytes < %zu needed", fn, what, have, need);
  if ((uintptr_t)p & 255) return fail(PACK3D_ERR_WORKSPACE, "%s: %s not 256-byte aligned", fn, what);
  return PACK3D_OK;
}

}  // namespace

extern "C" {

int pack3d_version(void) { return PACK3D_VERSION; }

const char* pack3d_last_error(void) { return g_err.c_str(); }

const char* pack3d_backend_info(void) {
  return "libpack3d gfx950: rope=k_rope (VALU, 16B rows); "
         "block_summary=k_block_summary (wave per block, XOR-tree reduction); "
         "local_attn for bf16 with Hq/Hkv in {4,8,16}: k_local_zrun for windows of 3 planes "
         "(runs of query planes, 3-slot LDS ring of K/V planes), else k_local_bf16 (async "
         "double-buffered LDS planes); both transposing V reads, masked-dense MFMA 32x32x16 "
         "bf16; else k_local_attn (LDS plane tiles + halo, masked-dense MFMA 32x32x16 bf16 / "
         "32x32x2 f32); global_attn=k_global_attn (summary tiles in LDS: bf16 copied "
         "asynchronously in phases of 4 tiles, fp32 register-staged double buffers; "
         "MFMA 32x32x16 bf16 / 32x32x2 f32, online softmax, fused gate epilogue in forward); "
         "gate_mix=k_gate_mix; backward (bf16, Hq/Hkv in {4,8,16}): k_bwd_prep, k_loc_dq, "
         "k_glob_dq, k_unrotate, k_loc_dkv, k_glob_dkv, k_sum_bwd (MFMA 32x32x16 bf16); "
         "layer (bf16): k_layernorm, k_gemm<qkv> (RoPE in the epilogue), k_gemm<residual> "
         "(MFMA 32x32x16 bf16, 256x256 tiles of 8 waves, LDS-staged coalesced epilogues); "
         "no fallbacks";
}

size_t pack3d_forward_workspace_size(const pack3d_problem* prob) {
  Geom g;
  if (make_geom(prob, &g) != PACK3D_OK) return 0;
  return ws_layout(g).total;
}

int pack3d_rope(const pack3d_problem* prob, const void* x, void* y, int32_t n_heads,
                const int32_t* coords, void* stream) {
  Geom g;
  int rc = make_geom(prob, &g);
  if (rc) return rc;
  if (!x || !y || !coords) return fail(PACK3D_ERR_NULL, "pack3d_rope: NULL tensor argument");
  if (n_heads < 1) return fail(PACK3D_ERR_SHAPE, "pack3d_rope: n_heads = %d", n_heads);
  if ((rc = check_aligned("pack3d_rope", {{x, "x"}, {y, "y"}, {coords, "coords"}}))) return rc;
  return hip_status(launch_rope(g, x, y, n_heads, coords, (hipStream_t)stream), "k_rope");
}

int pack3d_block_summary(const pack3d_problem* prob, const void* k_cmp, const void* v_cmp,
                         const float* a, const int32_t* cell_to_pos, void* k_sum, void* v_sum,
                         void* stream) {
  Geom g;
  int rc = make_geom(prob, &g);
  if (rc) return rc;
  if (!k_cmp || !v_cmp || !cell_to_pos || !k_sum || !v_sum)
    return fail(PACK3D_ERR_NULL, "pack3d_block_summary: NULL tensor argument");
  if ((rc = check_aligned("pack3d_block_summary",
                          {{k_cmp, "k_cmp"}, {v_cmp, "v_cmp"}, {a, "a"},
                           {cell_to_pos, "cell_to_pos"}, {k_sum, "k_sum"}, {v_sum, "v_sum"}})))
    return rc;
  return hip_status(launch_block_summary(g, k_cmp, v_cmp, a, cell_to_pos, k_sum, v_sum, 1.0f,
                                         nullptr, nullptr, nullptr, (hipStream_t)stream),
                    "k_block_summary");
}

int pack3d_local_attn(const pack3d_problem* prob, const void* q_rot, const void* k_rot,
                      const void* v, const int32_t* cell_to_pos, float* o_loc, float* lse_loc,
                      void* stream) {
  Geom g;
  int rc = make_geom(prob, &g);
  if (rc) return rc;
  if (!q_rot || !k_rot || !v || !cell_to_pos || !o_loc)
    return fail(PACK3D_ERR_NULL, "pack3d_local_attn: NULL tensor argument");
  if (!local_supported(g))
    return fail(PACK3D_ERR_UNSUPPORTED, "pack3d_local_attn: Hq/Hkv = %d unsupported", g.G);
  if ((rc = check_aligned("pack3d_local_attn",
                          {{q_rot, "q_rot"}, {k_rot, "k_rot"}, {v, "v"},
                           {cell_to_pos, "cell_to_pos"}, {o_loc, "o_loc"}, {lse_loc, "lse_loc"}})))
    return rc;
  return hip_status(
      launch_local_attn(g, q_rot, k_rot, v, cell_to_pos, LocalOut{o_loc, lse_loc, nullptr, nullptr},
                        no_qrope(),
                        (hipStream_t)stream),
      "k_local_attn");
}

int pack3d_global_attn(const pack3d_problem* prob, const void* q_rot, const void* k_sum,
                       const void* v_sum, int32_t m, float* o_cmp, float* lse_cmp,
                       void* stream) {
  Geom g;
  int rc = make_geom(prob, &g);
  if (rc) return rc;
  if (!q_rot || !k_sum || !v_sum || !o_cmp)
    return fail(PACK3D_ERR_NULL, "pack3d_global_attn: NULL tensor argument");
  if (m < 1) return fail(PACK3D_ERR_SHAPE, "pack3d_global_attn: m = %d must be >= 1", m);
  if ((rc = check_aligned("pack3d_global_attn", {{q_rot, "q_rot"}, {k_sum, "k_sum"},
                                                 {v_sum, "v_sum"}, {o_cmp, "o_cmp"},
                                                 {lse_cmp, "lse_cmp"}})))
    return rc;
  return hip_status(launch_global_attn(g, q_rot, k_sum, v_sum, m, nullptr, o_cmp, lse_cmp,
                                       nullptr, nullptr, nullptr, no_qrope(),
                                       (hipStream_t)stream),
                    "k_global_attn");
}

int pack3d_gate_mix(const pack3d_problem* prob, const float* o_loc, const float* o_cmp,
                    const float* gate_logits, void* out, void* stream) {
  Geom g;
  int rc = make_geom(prob, &g);
  if (rc) return rc;
  if (!o_loc || !o_cmp || !gate_logits || !out)
    return fail(PACK3D_ERR_NULL, "pack3d_gate_mix: NULL tensor argument");
  if ((rc = check_aligned("pack3d_gate_mix", {{o_loc, "o_loc"}, {o_cmp, "o_cmp"},
                                              {gate_logits, "gate_logits"}, {out, "out"}})))
    return rc;
  return hip_status(launch_gate_mix(g, o_loc, o_cmp, gate_logits, out, (hipStream_t)stream),
                    "k_gate_mix");
}

}  // extern "C"

namespace pack3d {

int api_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

// Host checks of the forward's arguments (everything but the workspace).
int forward_check(const char* fn, const pack3d_problem* prob, const FwdArgs& x, Geom* g) {
  int rc = make_geom(prob, g);
  if (rc) return rc;
  if (!x.q || !x.k_loc || !x.v_loc || !x.k_cmp || !x.v_cmp || !x.coords || !x.cell_to_pos ||
      !x.gate || !x.out)
    return fail(PACK3D_ERR_NULL, "%s: NULL tensor argument", fn);
  if (!local_supported(*g))
    return fail(PACK3D_ERR_UNSUPPORTED, "%s: Hq/Hkv = %d unsupported", fn, g->G);
  return check_tensors(fn, x.q, x.k_loc, x.v_loc, x.k_cmp, x.v_cmp, x.a, x.coords,
                       x.cell_to_pos, x.gate, x.out);
}

size_t forward_workspace_bytes(const Geom& g) { return ws_layout(g).total; }

// The forward's launch sequence on a checked problem and a workspace of at
// least forward_workspace_bytes(g) bytes (256-byte aligned); with `ev`
// (PACK3D_FORWARD_STAGES + 1 events) an event is recorded on the stream
// before the first stage and after each.
int forward_launch(const Geom& g, const FwdArgs& x, void* workspace, hipStream_t s,
                   void* const* ev) {
  const WsLayout w = ws_layout(g);
  char* ws = (char*)workspace;
  float* tab = (float*)(ws + w.tab);
  void* k_rot = ws + w.k_rot;
  void* k_sum = ws + w.k_sum;
  void* v_sum = ws + w.v_sum;
  float* knorm = (float*)(ws + w.knorm);
  float* kmax = (float*)(ws + w.kmax);
  int stage = 0;
  auto mark = [&]() -> hipError_t {
    return ev ? hipEventRecord((hipEvent_t)ev[stage++], s) : hipSuccess;
  };
  hipError_t e;
  if ((e = mark()) != hipSuccess) return hip_status(e, "hipEventRecord");
  // one pass over the blocks: summaries scaled into log2-domain logits, with
  // their norms for the softmax bound of the query->summary kernel, and the
  // rotated K_loc
  if ((e = launch_block_summary(g, x.k_cmp, x.v_cmp, x.a, x.cell_to_pos, k_sum, v_sum,
                                logit_scale(g), knorm, x.k_loc, k_rot, s)) != hipSuccess)
    return hip_status(e, "k_block_summary");
  if ((e = mark()) != hipSuccess) return hip_status(e, "hipEventRecord");
  // the per-group norm bound, and the rotary table both attention kernels
  // rotate Q through
  if ((e = launch_kmax(g, knorm, kmax, tab, s)) != hipSuccess) return hip_status(e, "k_kmax");
  if ((e = mark()) != hipSuccess) return hip_status(e, "hipEventRecord");
  const QRope qr = make_qrope(g, tab);
  // the local branch writes its gated share g_loc * o_loc into out
  if ((e = launch_local_attn(g, x.q, k_rot, x.v_loc, x.cell_to_pos,
                             LocalOut{nullptr, nullptr, x.gate, x.out}, qr, s)) != hipSuccess)
    return hip_status(e, "k_local_attn");
  if ((e = mark()) != hipSuccess) return hip_status(e, "hipEventRecord");
  // the compressed branch adds g_cmp * o_cmp; its query is rotated, or the
  // input q as given when the branch is blind
  const bool blind = g.summary_mode == PACK3D_SUMMARY_BLIND;
  e = launch_global_attn(g, x.q, k_sum, v_sum, g.M, kmax, nullptr, nullptr, x.gate, x.out,
                         x.coords, blind ? no_qrope() : qr, s);
  if (e != hipSuccess) return hip_status(e, "k_global_attn(gated)");
  if ((e = mark()) != hipSuccess) return hip_status(e, "hipEventRecord");
  return ok();
}

}  // namespace pack3d

namespace {

int forward_impl(const char* fn, const pack3d_problem* prob, const FwdArgs& x, void* workspace,
                 size_t ws_bytes, void* stream, void* const* ev, int32_t nev) {
  Geom g;
  int rc = forward_check(fn, prob, x, &g);
  if (rc) return rc;
  const size_t need = forward_workspace_bytes(g);
  if (!workspace) return fail(PACK3D_ERR_WORKSPACE, "%s: workspace is NULL", fn);
  if (ws_bytes < need)
    return fail(PACK3D_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
  if ((uintptr_t)workspace & 255)
    return fail(PACK3D_ERR_WORKSPACE, "%s: workspace not 256-byte aligned", fn);
  if (ev) {
    if (nev != PACK3D_FORWARD_STAGES + 1)
      return fail(PACK3D_ERR_SHAPE, "%s: %d events, need %d", fn, nev, PACK3D_FORWARD_STAGES + 1);
    for (int i = 0; i < nev; ++i)
      if (!ev[i]) return fail(PACK3D_ERR_NULL, "%s: event %d is NULL", fn, i);
  }
  return forward_launch(g, x, workspace, (hipStream_t)stream, ev);
}

}  // namespace

extern "C" {

int pack3d_forward(const pack3d_problem* prob, const void* q, const void* k_loc,
                   const void* v_loc, const void* k_cmp, const void* v_cmp, const float* a,
                   const int32_t* coords, const int32_t* cell_to_pos, const float* gate_logits,
                   void* out, void* workspace, size_t ws_bytes, void* stream) {
  const FwdArgs x{q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos, gate_logits, out};
  return forward_impl("pack3d_forward", prob, x, workspace, ws_bytes, stream, nullptr, 0);
}

int pack3d_forward_timed(const pack3d_problem* prob, const void* q, const void* k_loc,
                         const void* v_loc, const void* k_cmp, const void* v_cmp, const float* a,
                         const int32_t* coords, const int32_t* cell_to_pos,
                         const float* gate_logits, void* out, void* workspace, size_t ws_bytes,
                         void* stream, void* const* events, int32_t n_events) {
  if (!events) return fail(PACK3D_ERR_NULL, "pack3d_forward_timed: events is NULL");
  const FwdArgs x{q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos, gate_logits, out};
  return forward_impl("pack3d_forward_timed", prob, x, workspace, ws_bytes, stream, events,
                      n_events);
}

int pack3d_build_cell_index(const pack3d_problem* prob, const int32_t* coords,
                            int32_t* cell_to_pos, void* stream) {
  Geom g;
  int rc = make_geom(prob, &g);
  if (rc) return rc;
  if (!coords || !cell_to_pos)
    return fail(PACK3D_ERR_NULL, "pack3d_build_cell_index: NULL tensor argument");
  if ((rc = check_aligned("pack3d_build_cell_index",
                          {{coords, "coords"}, {cell_to_pos, "cell_to_pos"}})))
    return rc;
  return hip_status(launch_build_cell_index(g, coords, cell_to_pos, (hipStream_t)stream),
                    "k_cell_index");
}

int pack3d_check_packing(const pack3d_problem* prob, const int32_t* coords,
                         const int32_t* cell_to_pos, int32_t* n_bad_dev, void* stream) {
  Geom g;
  int rc = make_geom(prob, &g);
  if (rc) return rc;
  if (!coords || !cell_to_pos || !n_bad_dev)
    return fail(PACK3D_ERR_NULL, "pack3d_check_packing: NULL tensor argument");
  if ((rc = check_aligned("pack3d_check_packing",
                          {{coords, "coords"}, {cell_to_pos, "cell_to_pos"}})))
    return rc;
  if ((uintptr_t)n_bad_dev & 3)
    return fail(PACK3D_ERR_SHAPE, "pack3d_check_packing: n_bad_dev is not 4-byte aligned");
  return hip_status(launch_check_packing(g, coords, cell_to_pos, n_bad_dev, (hipStream_t)stream),
                    "k_check_packing");
}

}  // extern "C"

extern "C" {

size_t pack3d_saved_size(const pack3d_problem* prob) {
  Geom g;
  if (make_geom(prob, &g) != PACK3D_OK) return 0;
  return saved_layout(g).total;
}

size_t pack3d_backward_workspace_size(const pack3d_problem* prob) {
  Geom g;
  if (make_geom(prob, &g) != PACK3D_OK) return 0;
  return bwd_layout(g).total;
}

int pack3d_forward_train(const pack3d_problem* prob, const void* q, const void* k_loc,
                         const void* v_loc, const void* k_cmp, const void* v_cmp, const float* a,
                         const int32_t* coords, const int32_t* cell_to_pos,
                         const float* gate_logits, void* out, void* saved, size_t saved_bytes,
                         void* workspace, size_t ws_bytes, void* stream) {
  static const char* fn = "pack3d_forward_train";
  Geom g;
  int rc = make_geom(prob, &g);
  if (rc) return rc;
  if (!q || !k_loc || !v_loc || !k_cmp || !v_cmp || !coords || !cell_to_pos || !gate_logits ||
      !out)
    return fail(PACK3D_ERR_NULL, "%s: NULL tensor argument", fn);
  if (!local_supported(g))
    return fail(PACK3D_ERR_UNSUPPORTED, "%s: Hq/Hkv = %d unsupported", fn, g.G);
  if ((rc = check_tensors(fn, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos, gate_logits,
                          out)))
    return rc;
  const WsLayout w = ws_layout(g);
  const SavedLayout sl = saved_layout(g);
  if ((rc = check_buffer(workspace, ws_bytes, w.total, fn, "workspace"))) return rc;
  if ((rc = check_buffer(saved, saved_bytes, sl.total, fn, "saved"))) return rc;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  char* sv = (char*)saved;
  float* tab = (float*)(ws + w.tab);
  void* k_rot = ws + w.k_rot;
  void* k_sum = ws + w.k_sum;
  void* v_sum = ws + w.v_sum;
  float* knorm = (float*)(ws + w.knorm);
  float* kmax = (float*)(ws + w.kmax);
  float* o_loc = (float*)(sv + sl.o_loc);
  float* o_cmp = (float*)(sv + sl.o_cmp);
  float* lse_loc = (float*)(sv + sl.lse_loc);
  float* lse_cmp = (float*)(sv + sl.lse_cmp);
  hipError_t e;
  if ((e = launch_block_summary(g, k_cmp, v_cmp, a, cell_to_pos, k_sum, v_sum,
                                logit_scale(g), knorm, k_loc, k_rot, s)) != hipSuccess)
    return hip_status(e, "k_block_summary");
  if ((e = launch_kmax(g, knorm, kmax, tab, s)) != hipSuccess) return hip_status(e, "k_kmax");
  // the kernels of the inference forward, also saving each branch's output
  // and lse
  const QRope qr = make_qrope(g, tab);
  if ((e = launch_local_attn(g, q, k_rot, v_loc, cell_to_pos,
                             LocalOut{o_loc, lse_loc, gate_logits, out}, qr, s)) != hipSuccess)
    return hip_status(e, "k_local_attn");
  const bool blind = g.summary_mode == PACK3D_SUMMARY_BLIND;
  e = launch_global_attn(g, q, k_sum, v_sum, g.M, kmax, o_cmp, lse_cmp, gate_logits, out, coords,
                         blind ? no_qrope() : qr, s);
  return hip_status(e, "k_global_attn");
}

int pack3d_backward(const pack3d_problem* prob, const void* q, const void* k_loc,
                    const void* v_loc, const void* k_cmp, const void* v_cmp, const float* a,
                    const int32_t* coords, const int32_t* cell_to_pos, const float* gate_logits,
                    const void* saved, size_t saved_bytes, const void* dout, void* dq,
                    void* dk_loc, void* dv_loc, void* dk_cmp, void* dv_cmp, float* dgate,
                    void* workspace, size_t ws_bytes, void* stream) {
  static const char* fn = "pack3d_backward";
  Geom g;
  int rc = make_geom(prob, &g);
  if (rc) return rc;
  if (!q || !k_loc || !v_loc || !k_cmp || !v_cmp || !coords || !cell_to_pos || !gate_logits ||
      !dout || !dq || !dk_loc || !dv_loc || !dk_cmp || !dv_cmp || !dgate)
    return fail(PACK3D_ERR_NULL, "%s: NULL tensor argument", fn);
  if (!backward_supported(g))
    return fail(PACK3D_ERR_UNSUPPORTED,
                "%s: only bf16 with Hq/Hkv in {4, 8, 16} is supported (dtype %d, Hq/Hkv %d)", fn,
                prob->dtype, g.G);
  if ((rc = check_tensors(fn, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, cell_to_pos, gate_logits,
                          dout, "dout")) ||
      (rc = check_aligned(fn, {{dq, "dq"}, {dk_loc, "dk_loc"}, {dv_loc, "dv_loc"},
                               {dk_cmp, "dk_cmp"}, {dv_cmp, "dv_cmp"}, {dgate, "dgate"}})))
    return rc;
  const BwdLayout w = bwd_layout(g);
  const SavedLayout sl = saved_layout(g);
  if ((rc = check_buffer(workspace, ws_bytes, w.total, fn, "workspace"))) return rc;
  if ((rc = check_buffer((void*)saved, saved_bytes, sl.total, fn, "saved"))) return rc;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const char* sv = (const char*)saved;
  BwdBuffers b;
  b.v_loc = v_loc;
  b.a = a;
  b.coords = coords;
  b.c2p = cell_to_pos;
  b.gate = gate_logits;
  b.dout = dout;
  b.o_loc = (const float*)(sv + sl.o_loc);
  b.o_cmp = (const float*)(sv + sl.o_cmp);
  b.lse_loc = (const float*)(sv + sl.lse_loc);
  b.lse_cmp = (const float*)(sv + sl.lse_cmp);
  b.q_rot = ws + w.q_rot;
  b.q_cmp = g.summary_mode == PACK3D_SUMMARY_BLIND ? q : b.q_rot;
  b.k_rot = ws + w.k_rot;
  b.k_sum = ws + w.k_sum;
  b.v_sum = ws + w.v_sum;
  b.dlo = ws + w.dlo;
  b.dco = ws + w.dco;
  b.d_loc = (float*)(ws + w.d_loc);
  b.d_cmp = (float*)(ws + w.d_cmp);
  b.nls_cmp = (float*)(ws + w.nls_cmp);
  b.dq_acc = (float*)(ws + w.dq_acc);
  b.dk_part = (float*)(ws + w.dk_part);
  b.dv_part = (float*)(ws + w.dv_part);
  b.dq = dq;
  b.dk_loc = dk_loc;
  b.dv_loc = dv_loc;
  b.dk_cmp = dk_cmp;
  b.dv_cmp = dv_cmp;
  b.dgate = dgate;
  hipError_t e;
  // recompute the rotations and the summaries (keys scaled into log2-domain
  // logits, as in the forward)
  if ((e = launch_rope(g, q, ws + w.q_rot, g.Hq, coords, s)) != hipSuccess)
    return hip_status(e, "k_rope(q)");
  if ((e = launch_block_summary(g, k_cmp, v_cmp, a, cell_to_pos, ws + w.k_sum, ws + w.v_sum,
                                logit_scale(g), nullptr, k_loc, ws + w.k_rot, s)) != hipSuccess)
    return hip_status(e, "k_block_summary");
  return hip_status(launch_backward(g, b, s), fn);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The layer around the operator: LayerNorm + projections (+ RoPE), the
// operator, the output projection + residual.
// ---------------------------------------------------------------------------
namespace {

int check_width(const Geom& g, int32_t width, const char* fn) {
  if (!g.bf16)
    return fail(PACK3D_ERR_UNSUPPORTED, "%s: only bf16 tensors are supported", fn);
  if (width < 64 || width > 8192 || width % 64)
    return fail(PACK3D_ERR_SHAPE, "%s: width %d must be a multiple of 64 in [64, 8192]", fn,
                width);
  return PACK3D_OK;
}

struct LayerLayout {
  size_t x, q_raw, q_rot, k_rot, v_loc, k_cmp, v_cmp, k_sum, v_sum, knorm, kmax, o, total;
};

LayerLayout layer_layout(const Geom& g, int32_t width) {
  LayerLayout w;
  size_t off = 0;
  auto take = [&](size_t& at, size_t bytes) {
    at = off;
    off += align256(bytes);
  };
  const size_t nq = (size_t)g.N * g.Hq * 64 * 2, nk = (size_t)g.N * g.Hkv * 64 * 2;
  take(w.x, (size_t)g.N * width * 2);
  take(w.q_raw, g.summary_mode == PACK3D_SUMMARY_BLIND ? nq : 0);
  take(w.q_rot, nq);
  take(w.k_rot, nk);
  take(w.v_loc, nk);
  take(w.k_cmp, nk);
  take(w.v_cmp, nk);
  take(w.k_sum, (size_t)g.Hkv * g.M * 64 * 2);
  take(w.v_sum, (size_t)g.Hkv * g.M * 64 * 2);
  take(w.knorm, (size_t)g.Hkv * g.M * 4);
  take(w.kmax, (size_t)g.Hkv * 4);
  take(w.o, nq);
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

int pack3d_layernorm_qkv(const pack3d_problem* prob, int32_t width, const void* h,
                         const float* gamma, const float* beta, float eps, const void* w_qkv,
                         const int32_t* coords, void* x_norm, void* q_rot, void* q_raw,
                         void* k_rot, void* v_loc, void* k_cmp, void* v_cmp, void* stream) {
  static const char* fn = "pack3d_layernorm_qkv";
  Geom g;
  int rc = make_geom(prob, &g);
  if (rc || (rc = check_width(g, width, fn))) return rc;
  if (!h || !w_qkv || !coords || !x_norm || !q_rot || !k_rot || !v_loc || !k_cmp || !v_cmp)
    return fail(PACK3D_ERR_NULL, "%s: NULL tensor argument", fn);
  if (!(eps > 0.0f) || !isfinite(eps)) return fail(PACK3D_ERR_SHAPE, "%s: eps must be > 0", fn);
  if ((rc = check_aligned(fn, {{h, "h"}, {gamma, "gamma"}, {beta, "beta"}, {w_qkv, "w_qkv"},
                               {coords, "coords"}, {x_norm, "x_norm"}, {q_rot, "q_rot"},
                               {q_raw, "q_raw"}, {k_rot, "k_rot"}, {v_loc, "v_loc"},
                               {k_cmp, "k_cmp"}, {v_cmp, "v_cmp"}})))
    return rc;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if ((e = launch_layernorm(g, width, h, gamma, beta, eps, x_norm, s)) != hipSuccess)
    return hip_status(e, "k_layernorm");
  return hip_status(launch_qkv_proj(g, width, x_norm, w_qkv, coords, q_rot, q_raw, k_rot, v_loc,
                                    k_cmp, v_cmp, s),
                    "k_gemm<qkv>");
}

int pack3d_out_proj(const pack3d_problem* prob, int32_t width, const void* o, const void* w_o,
                    const void* residual, void* out, void* stream) {
  static const char* fn = "pack3d_out_proj";
  Geom g;
  int rc = make_geom(prob, &g);
  if (rc || (rc = check_width(g, width, fn))) return rc;
  if (!o || !w_o || !residual || !out) return fail(PACK3D_ERR_NULL, "%s: NULL tensor argument", fn);
  if ((rc = check_aligned(fn, {{o, "o"}, {w_o, "w_o"}, {residual, "residual"}, {out, "out"}})))
    return rc;
  return hip_status(launch_out_proj(g, width, o, w_o, residual, out, (hipStream_t)stream),
                    "k_gemm<residual>");
}

size_t pack3d_layer_workspace_size(const pack3d_problem* prob, int32_t width) {
  Geom g;
  if (make_geom(prob, &g) != PACK3D_OK || check_width(g, width, "pack3d_layer_workspace_size"))
    return 0;
  return layer_layout(g, width).total;
}

int pack3d_layer_forward(const pack3d_problem* prob, int32_t width, const void* h,
                         const float* gamma, const float* beta, float eps, const void* w_qkv,
                         const void* w_o, const float* a, const int32_t* coords,
                         const int32_t* cell_to_pos, const float* gate_logits, void* out,
                         void* workspace, size_t ws_bytes, void* stream) {
  static const char* fn = "pack3d_layer_forward";
  Geom g;
  int rc = make_geom(prob, &g);
  if (rc || (rc = check_width(g, width, fn))) return rc;
  if (!h || !w_qkv || !w_o || !coords || !cell_to_pos || !gate_logits || !out)
    return fail(PACK3D_ERR_NULL, "%s: NULL tensor argument", fn);
  if (!(eps > 0.0f) || !isfinite(eps)) return fail(PACK3D_ERR_SHAPE, "%s: eps must be > 0", fn);
  if (!local_supported(g))
    return fail(PACK3D_ERR_UNSUPPORTED, "%s: Hq/Hkv = %d unsupported", fn, g.G);
  if ((rc = check_aligned(fn, {{h, "h"}, {gamma, "gamma"}, {beta, "beta"}, {w_qkv, "w_qkv"},
                               {w_o, "w_o"}, {a, "a"}, {coords, "coords"},
                               {cell_to_pos, "cell_to_pos"}, {gate_logits, "gate_logits"},
                               {out, "out"}})))
    return rc;
  const LayerLayout w = layer_layout(g, width);
  if ((rc = check_buffer(workspace, ws_bytes, w.total, fn, "workspace"))) return rc;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const bool blind = g.summary_mode == PACK3D_SUMMARY_BLIND;
  void* q_raw = blind ? ws + w.q_raw : nullptr;
  float* knorm = (float*)(ws + w.knorm);
  float* kmax = (float*)(ws + w.kmax);
  hipError_t e;
  if ((e = launch_layernorm(g, width, h, gamma, beta, eps, ws + w.x, s)) != hipSuccess)
    return hip_status(e, "k_layernorm");
  if ((e = launch_qkv_proj(g, width, ws + w.x, w_qkv, coords, ws + w.q_rot, q_raw, ws + w.k_rot,
                           ws + w.v_loc, ws + w.k_cmp, ws + w.v_cmp, s)) != hipSuccess)
    return hip_status(e, "k_gemm<qkv>");
  if ((e = launch_block_summary(g, ws + w.k_cmp, ws + w.v_cmp, a, cell_to_pos, ws + w.k_sum,
                                ws + w.v_sum, logit_scale(g), knorm, nullptr, nullptr, s)) !=
      hipSuccess)
    return hip_status(e, "k_block_summary");
  if ((e = launch_kmax(g, knorm, kmax, nullptr, s)) != hipSuccess) return hip_status(e, "k_kmax");
  // the projection's epilogue rotated Q and K_loc already
  if ((e = launch_local_attn(g, ws + w.q_rot, ws + w.k_rot, ws + w.v_loc, cell_to_pos,
                             LocalOut{nullptr, nullptr, gate_logits, ws + w.o}, no_qrope(), s)) !=
      hipSuccess)
    return hip_status(e, "k_local_attn");
  e = launch_global_attn(g, blind ? q_raw : ws + w.q_rot, ws + w.k_sum, ws + w.v_sum, g.M, kmax,
                         nullptr, nullptr, gate_logits, ws + w.o, nullptr, no_qrope(), s);
  if (e != hipSuccess) return hip_status(e, "k_global_attn(gated)");
  return hip_status(launch_out_proj(g, width, ws + w.o, w_o, h, out, s), "k_gemm<residual>");
}

}  // extern "C"
