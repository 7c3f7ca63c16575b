// Internal declarations shared by the libpack3d translation units: the
// validated problem geometry, the rotary table and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pack3d.h"

namespace pack3d {

constexpr int kHeadDim = 64;
constexpr int kMaxPairs = 32;      // head_dim / 2
constexpr int kMaxBlockVol = 64;
constexpr int kNumXcd = 8;         // MI355X: 8 XCDs, each with its own L2

// Rotary constants: pair p rotates dims (2p, 2p+1) by 2*pi * nu[p] * c[axis[p]]
// (nu = omega / 2pi, computed on the host in double).  Pairs >= npairs are
// the identity block.
struct RopeTab {
  double nu[kMaxPairs];
  int32_t axis[kMaxPairs];
  int32_t npairs;
};

// Everything a kernel needs, derived once from pack3d_problem on the host.
struct Geom {
  int32_t Z, Y, X;
  int64_t N;
  int32_t Hq, Hkv, G;             // G = Hq / Hkv
  int32_t rz, ry, rx;             // window radii
  int32_t bz, by, bx, bvol;       // summary block
  int64_t M;                      // N / bvol
  float scale;                    // softmax scale
  int32_t bf16;                   // 1: bf16 tensors, 0: fp32
  int32_t gate_per_head;
  int32_t summary_mode;           // pack3d_summary_mode
  RopeTab rope;
};

// Launchers (each returns the launch status; no host synchronisation).
hipError_t launch_rope(const Geom& g, const void* x, void* y, int32_t heads,
                       const int32_t* coords, hipStream_t s);
// kscale multiplies the key summaries; knorm (nullable) receives their norms
// [Hkv, M] after scaling.
hipError_t launch_block_summary(const Geom& g, const void* k_cmp, const void* v_cmp,
                                const float* a, const int32_t* cell_to_pos, void* k_sum,
                                void* v_sum, float kscale, float* knorm, hipStream_t s);
// kmax[g] = max over the M key-summary norms of group g.
hipError_t launch_kmax(const Geom& g, const float* knorm, float* kmax, hipStream_t s);
hipError_t launch_local_attn(const Geom& g, const void* q_rot, const void* k_rot,
                             const void* v, const int32_t* cell_to_pos, float* o_loc,
                             float* lse, hipStream_t s);
// The bf16 kernel with compile-time plane geometry serves these group sizes;
// launch_local_attn dispatches to it.
bool local_bf16_serves(int G);
hipError_t launch_local_attn_bf16(const Geom& g, const void* q_rot, const void* k_rot,
                                  const void* v, const int32_t* cell_to_pos, float* o_loc,
                                  float* lse, hipStream_t s);
// out != nullptr: gate-mix epilogue, out = g_loc*o_loc + g_cmp*o_cmp in the
// problem dtype (o_cmp, fp32, also written when non-null).  Otherwise o_cmp
// (fp32) only.  lse != nullptr: natural-log lse per row.  kmax != nullptr:
// the key summaries are pre-scaled by scale*log2(e) and kmax[g] bounds their
// norms (enables the fixed softmax reference); nullptr: unscaled summaries.
hipError_t launch_global_attn(const Geom& g, const void* q_rot, const void* k_sum,
                              const void* v_sum, int64_t m, const float* kmax, float* o_cmp,
                              float* lse, const float* o_loc, const float* gate, void* out,
                              hipStream_t s);
// Backward (bf16).  Inputs, the forward's saved state, workspace buffers and
// outputs of one backward launch sequence.
struct BwdBuffers {
  const void* v_loc;           // [N, Hkv, 64]
  const float* a;              // [N, Hkv] or NULL (uniform)
  const int32_t* coords;       // [N, 3]
  const int32_t* c2p;          // [Z*Y*X]
  const float* gate;           // [N, 2] or [N, Hq, 2]
  const void* dout;            // [N, Hq, 64]
  const float* o_loc;          // saved [N, Hq, 64]
  const float* o_cmp;          // saved [N, Hq, 64]
  const float* lse_loc;        // saved [N, Hq]
  const float* lse_cmp;        // saved [N, Hq]
  const void* q_cmp;           // the compressed branch's query (q_rot, or q if blind)
  const void* q_rot;           // workspace: rotated q, k_loc, unscaled summaries
  const void* k_rot;
  const void* k_sum;
  const void* v_sum;
  void* dlo;                   // workspace: g_loc * dO, g_cmp * dO (bf16)
  void* dco;
  float* d_loc;                // workspace: D of each branch [N, Hq]
  float* d_cmp;
  float* dq_acc;               // workspace: rotated-frame dq [N, Hq, 64]
  float* dk_part;              // workspace: summary gradient partials
  float* dv_part;              //   [splits, Hkv, M, 64]
  void* dq;                    // outputs
  void* dk_loc;
  void* dv_loc;
  void* dk_cmp;
  void* dv_cmp;
  float* dgate;
};
bool backward_supported(const Geom& g);
int64_t glob_dkv_splits(const Geom& g);
hipError_t launch_backward(const Geom& g, const BwdBuffers& b, hipStream_t s);
// The layer around the operator (bf16): x = LayerNorm(h) [N, width]; the
// stacked projection of x with RoPE on Q and K_loc (q_raw: unrotated Q as
// well, nullable); the output projection out = resid + o W_o^T.
hipError_t launch_layernorm(const Geom& g, int32_t width, const void* h, const float* gamma,
                            const float* beta, float eps, void* x, hipStream_t s);
hipError_t launch_qkv_proj(const Geom& g, int32_t width, const void* x, const void* w_qkv,
                           const int32_t* coords, void* q, void* q_raw, void* k_loc,
                           void* v_loc, void* k_cmp, void* v_cmp, hipStream_t s);
hipError_t launch_out_proj(const Geom& g, int32_t width, const void* o, const void* w_o,
                           const void* resid, void* out, hipStream_t s);
hipError_t launch_gate_mix(const Geom& g, const float* o_loc, const float* o_cmp,
                           const float* gate, void* out, hipStream_t s);
hipError_t launch_build_cell_index(const Geom& g, const int32_t* coords, int32_t* c2p,
                                   hipStream_t s);
hipError_t launch_check_packing(const Geom& g, const int32_t* coords, const int32_t* c2p,
                                int32_t* n_bad, hipStream_t s);

}  // namespace pack3d
