/*
 * pack3d.h -- C ABI of libpack3d, the PACK3D local-global attention forward
 * for AMD Instinct MI355X (gfx950).
 *
 * The operator is the one described in "Geometry Matters in Packed 3D
 * Attention" (arXiv 2610.38694).  Citations below name the page and the
 * passage: "notes" = the papernotes.org notes (method section, key designs
 * 1-3, flowchart); "summary" = the ai.info summary (Methodology in Plain
 * English).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tokens are stored in PACKED order: position i of every token-major array
 *   is one lattice cell, coords[i] = (z, y, x) of that cell, and
 *   cell_to_pos[(z*Y + y)*X + x] = i is the inverse map.  A packing is any
 *   bijection between positions and cells (summary, Methodology: raster,
 *   Morton, block-contiguous, random ...).  Results never depend on the
 *   packing (notes, key design 1, Proposition 1): this library computes every
 *   reduction in an order fixed by coordinates, so repacked outputs are the
 *   permuted outputs bit for bit.
 * - Arrays are dense, row-major, contiguous, device memory (HBM), owned by
 *   the caller.  The library never allocates device memory and keeps no
 *   state between calls except a per-thread error string.
 * - Every array argument must start on a 16-byte boundary (the kernels move
 *   rows with 16-byte vector and direct-to-LDS copies); a misaligned pointer
 *   is rejected with PACK3D_ERR_SHAPE before any launch.  Workspaces and the
 *   saved state need 256-byte alignment (PACK3D_ERR_WORKSPACE).
 * - "dtype" arrays hold float (PACK3D_F32) or bf16 (PACK3D_BF16) values as
 *   chosen by pack3d_problem.dtype.  Accumulation is always fp32.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null
 *   stream) and never synchronises the host.
 * - Return value: PACK3D_OK or a negative pack3d_status.  Argument errors are
 *   detected on the host, before any launch and without reading device data;
 *   then nothing is launched and pack3d_last_error() describes the problem.
 *   Unsupported shapes are errors (PACK3D_ERR_UNSUPPORTED); there is no
 *   fallback path.  Data contracts (coordinates consistent with cell_to_pos,
 *   weights normalised per block) are NOT checked on the hot path; use
 *   pack3d_check_packing().  Out-of-range coordinates in coords or
 *   cell_to_pos entries outside [0, N) are undefined behaviour.
 */
#ifndef PACK3D_H
#define PACK3D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PACK3D_VERSION 1

typedef enum pack3d_status {
  PACK3D_OK = 0,
  PACK3D_ERR_NULL = -1,        /* a required pointer is NULL                   */
  PACK3D_ERR_SHAPE = -2,       /* inconsistent sizes (grid, heads, block, ...) */
  PACK3D_ERR_UNSUPPORTED = -3, /* valid but not implemented (e.g. head_dim)    */
  PACK3D_ERR_WORKSPACE = -4,   /* workspace missing or too small               */
  PACK3D_ERR_PACKING = -5,     /* reserved for packing-contract failures       */
  PACK3D_ERR_HIP = -6          /* a HIP launch or runtime call failed          */
} pack3d_status;

typedef enum pack3d_dtype { PACK3D_F32 = 0, PACK3D_BF16 = 1 } pack3d_dtype;

/*
 * Compressed-branch variants (notes, key design 2: rotating every key before
 * the block sum is the exact form; summary, contributions and findings: a
 * cheaper summary-centre placement, and a coordinate-blind compressed branch
 * as the missing control).
 *   TOKEN   k~_j = sum_u a_u R(c_u) k_u; the branch's query is R(c_i) q_i.
 *   CENTRE  k~_j = R(c^_j) sum_u a_u k_u, c^_j the block's geometric centre
 *           (origin + (b - 1)/2 per axis, half-integer for even extents);
 *           the branch's query is R(c_i) q_i.
 *   BLIND   k~_j = sum_u a_u k_u and the branch's query is the unrotated q_i.
 * Values are pooled the same way in all three; the local branch is unchanged.
 */
typedef enum pack3d_summary_mode {
  PACK3D_SUMMARY_TOKEN = 0,
  PACK3D_SUMMARY_CENTRE = 1,
  PACK3D_SUMMARY_BLIND = 2
} pack3d_summary_mode;

/*
 * One operator instance.
 *   grid[3]        lattice extents Z, Y, X (all >= 1); N = Z*Y*X < 2^31.
 *   n_q_heads      Hq; n_kv_heads Hkv; Hq % Hkv == 0 (query head h reads KV
 *                  group h/(Hq/Hkv)); the local branch and the forward take
 *                  Hq/Hkv in {1,2,4,8,16}.
 *   head_dim       d_h; only 64 is supported.
 *   window[3]      odd extents of the local box (notes, key design 3: the
 *                  neighbourhood is a coordinate box); supported up to 3x7x7.
 *                  The box is clipped at the lattice faces and holds the
 *                  query cell itself.
 *   block[3]       summary block shape (notes, key design 2); must divide
 *                  grid; M = N / (block volume); volume <= 64.
 *   rope_pairs[3]  rotary pairs on z, y, x (notes, key design 1: 11/11/10 at
 *                  d_h = 64); 2*(sum) <= head_dim.  Pair p acts on dims
 *                  (2p, 2p+1), z pairs first, with angle
 *                  rope_base^(-r/m_a) * c_a for the r-th pair of axis a.
 *   rope_base      10000 in the pages.
 *   scale          softmax scale; <= 0 selects 1/sqrt(head_dim).
 *   dtype          pack3d_dtype of q/k/v/out.
 *   gate_per_head  0: gate logits are [N, 2]; 1: [N, Hq, 2].
 *   summary_mode   pack3d_summary_mode; 0 (TOKEN) is the pages' exact form.
 */
typedef struct pack3d_problem {
  int32_t grid[3];
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t window[3];
  int32_t block[3];
  int32_t rope_pairs[3];
  double rope_base;
  float scale;
  int32_t dtype;
  int32_t gate_per_head;
  int32_t summary_mode;
} pack3d_problem;

/*
 * Axial grid RoPE (notes, key design 1, the equation for R(c)):
 *   y[i, h, :] = R(coords[i]) x[i, h, :]   for i < N, h < n_heads.
 * x, y: dtype [N, n_heads, head_dim]; y may alias x (in place).
 * coords: int32 [N, 3] (z, y, x) in [0, grid).
 */
int pack3d_rope(const pack3d_problem* prob, const void* x, void* y, int32_t n_heads,
                const int32_t* coords, void* stream);

/*
 * Rotate-before-compression block summaries (notes, key design 2, the
 * equations for k~_j and v~_j):
 *   k_sum[g, j, :] = sum_{u in B_j} a[u, g] R(c_u) k_cmp[u, g, :]
 *   v_sum[g, j, :] = sum_{u in B_j} a[u, g] v_cmp[u, g, :]
 * B_j is the j-th aligned block in block-raster order,
 *   j = ((z/bz)*(Y/by) + y/by)*(X/bx) + x/bx.
 * k_cmp is NOT rotated (the rotation happens inside, before the sum).
 * With summary_mode CENTRE the weighted sum of the unrotated keys is rotated
 * once by R(c^_j); with BLIND it is not rotated.
 * k_cmp, v_cmp: dtype [N, Hkv, head_dim].  a: fp32 [N, Hkv] or NULL for the
 * uniform 1/v (normalisation is the caller's contract).  cell_to_pos: int32
 * [N].  k_sum, v_sum: dtype [Hkv, M, head_dim], rounded once from fp32.
 */
int pack3d_block_summary(const pack3d_problem* prob, const void* k_cmp, const void* v_cmp,
                         const float* a, const int32_t* cell_to_pos, void* k_sum,
                         void* v_sum, void* stream);

/*
 * Exact local-neighbourhood attention (notes, key design 3; summary,
 * Methodology, first contract):
 *   o_loc[i, h] = sum_{u in N(i)} softmax_u(scale <q_rot[i,h], k_rot[u,g]>) v[u,g]
 * with N(i) the clipped box window around coords[i].  q_rot: dtype
 * [N, Hq, head_dim]; k_rot, v: dtype [N, Hkv, head_dim] (pre-rotated by
 * pack3d_rope; v is never rotated).  o_loc: fp32 [N, Hq, head_dim];
 * lse_loc: fp32 [N, Hq] natural-log log-sum-exp of the scaled logits, or NULL.
 */
int pack3d_local_attn(const pack3d_problem* prob, const void* q_rot, const void* k_rot,
                      const void* v, const int32_t* cell_to_pos, float* o_loc,
                      float* lse_loc, void* stream);

/*
 * Query -> all-summaries attention, streamed with an online softmax (notes,
 * key design 3; summary, Methodology, second contract):
 *   o_cmp[i, h] = sum_{j < m} softmax_j(scale <q_rot[i,h], k_sum[g,j]>) v_sum[g,j]
 * q_rot: dtype [N, Hq, head_dim]; k_sum, v_sum: dtype [Hkv, m, head_dim]
 * (m >= 1 is explicit, so m = N with 1x1x1 blocks is dense attention).
 * The query operand is the compressed branch's query: rotated for TOKEN and
 * CENTRE, the unrotated q for BLIND (the caller passes it).
 * o_cmp: fp32 [N, Hq, head_dim]; lse_cmp: fp32 [N, Hq] or NULL.
 */
int pack3d_global_attn(const pack3d_problem* prob, const void* q_rot, const void* k_sum,
                       const void* v_sum, int32_t m, float* o_cmp, float* lse_cmp,
                       void* stream);

/*
 * Tokenwise softmax gate (notes, flowchart node F and overall framework):
 *   (g_loc, g_cmp) = softmax(gate_logits[i] or gate_logits[i, h])
 *   out[i, h] = g_loc * o_loc[i, h] + g_cmp * o_cmp[i, h]
 * Index 0 of the logits is the local branch.  o_loc, o_cmp: fp32
 * [N, Hq, head_dim]; gate_logits: fp32 [N, 2] or [N, Hq, 2]; out: dtype.
 */
int pack3d_gate_mix(const pack3d_problem* prob, const float* o_loc, const float* o_cmp,
                    const float* gate_logits, void* out, void* stream);

/*
 * The whole forward (notes, overall framework and flowchart): RoPE on Q and
 * K_loc, block summaries of (K_cmp, V_cmp), local attention, query->summary
 * attention and the gate, in four launches on `stream`:
 *   1. one pass over the blocks: the summaries (keys scaled into log2-domain
 *      logits) with their norms, and R(c) K_loc for every token;
 *   2. the per-group maximum summary norm, and the lattice's rotary
 *      (sin, cos) table;
 *   3. local attention, rotating its query fragments in registers through
 *      the table; writes the gated share g_loc * o_loc to out;
 *   4. query->summary attention, rotating its query fragments likewise;
 *      adds g_cmp * o_cmp to out.
 * q: dtype [N, Hq, 64]; k_loc, v_loc, k_cmp, v_cmp: dtype [N, Hkv, 64], all
 * unrotated.  a: fp32 [N, Hkv] or NULL; coords: int32 [N, 3]; cell_to_pos:
 * int32 [N]; gate_logits: fp32 [N, 2] or [N, Hq, 2]; out: dtype [N, Hq, 64]
 * (its prior contents are overwritten).  workspace: device memory of at
 * least pack3d_forward_workspace_size() bytes, 256-byte aligned,
 * caller-owned; it holds the rotary table, the rotated K_loc, the summaries
 * and their norms between the launches.
 */
int pack3d_forward(const pack3d_problem* prob, const void* q, const void* k_loc,
                   const void* v_loc, const void* k_cmp, const void* v_cmp, const float* a,
                   const int32_t* coords, const int32_t* cell_to_pos,
                   const float* gate_logits, void* out, void* workspace, size_t ws_bytes,
                   void* stream);

/*
 * The forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, launches, kernels and result as
 * pack3d_forward, with the workspace in a static device array of
 * PACK3D_NOALLOC_SCRATCH_BYTES (256 MiB) that every GPU the library runs on
 * holds until the process ends.  The call allocates nothing.
 *   - Problems whose pack3d_forward_workspace_size() exceeds that size are
 *     rejected with PACK3D_ERR_WORKSPACE before any launch (at 8 query heads,
 *     2 KV groups and bf16, about 288.5 bytes per token: up to ~930 000
 *     tokens).
 *   - Every call on a GPU shares that GPU's array, which keeps the last
 *     call's contents (the forward writes every part it reads, so nothing
 *     needs clearing): calls that overlap on one GPU (different streams, no
 *     ordering between them) race and give undefined results.
 *   - The first call on each device looks up the array's device address
 *     (hipGetSymbolAddress) with that device current.
 */
#define PACK3D_NOALLOC_SCRATCH_BYTES (256u << 20)
int pack3d_forward_noalloc(const pack3d_problem* prob, const void* q, const void* k_loc,
                           const void* v_loc, const void* k_cmp, const void* v_cmp,
                           const float* a, const int32_t* coords, const int32_t* cell_to_pos,
                           const float* gate_logits, void* out, void* stream);

/*
 * pack3d_forward with per-stage timing: the same launches, plus an event
 * recorded on `stream` before the first stage and after each of the
 * PACK3D_FORWARD_STAGES stages, in this order (pack3d_forward's launches):
 *   0 block pass (summaries, their norms, RoPE of k_loc), 1 per-group max
 *   summary norm and the rotary table, 2 local attention (with RoPE of q,
 *   writing its gated share), 3 query->summary attention (with RoPE of q,
 *   adding its gated share).
 * events: PACK3D_FORWARD_STAGES + 1 hipEvent_t handles created by the caller
 * (timing enabled); n_events must equal that count.  The elapsed time
 * between events i and i+1 is stage i.  Errors as pack3d_forward.
 */
#define PACK3D_FORWARD_STAGES 4
int pack3d_forward_timed(const pack3d_problem* prob, const void* q, const void* k_loc,
                         const void* v_loc, const void* k_cmp, const void* v_cmp, const float* a,
                         const int32_t* coords, const int32_t* cell_to_pos,
                         const float* gate_logits, void* out, void* workspace, size_t ws_bytes,
                         void* stream, void* const* events, int32_t n_events);

/*
 * Training forward: the same output as pack3d_forward, plus, in `saved`, the
 * state pack3d_backward needs: o_loc fp32 [N, Hq, 64], o_cmp fp32
 * [N, Hq, 64], lse_loc fp32 [N, Hq], lse_cmp fp32 [N, Hq] (natural-log
 * log-sum-exp of each branch's scaled logits), in that order, each section
 * starting on a 256-byte boundary.  saved: device memory of at least
 * pack3d_saved_size() bytes, 256-byte aligned, caller-owned.  The gate is
 * applied in the compressed branch's epilogue, as in pack3d_forward, so out
 * is bit for bit the same as pack3d_forward's.  Errors as
 * pack3d_forward (PACK3D_ERR_WORKSPACE also for `saved`).
 */
int pack3d_forward_train(const pack3d_problem* prob, const void* q, const void* k_loc,
                         const void* v_loc, const void* k_cmp, const void* v_cmp, const float* a,
                         const int32_t* coords, const int32_t* cell_to_pos,
                         const float* gate_logits, void* out, void* saved, size_t saved_bytes,
                         void* workspace, size_t ws_bytes, void* stream);

/* Bytes of the saved state pack3d_forward_train writes (0 if invalid). */
size_t pack3d_saved_size(const pack3d_problem* prob);

/*
 * Backward of the forward: the exact derivatives of out with respect to its
 * inputs for the upstream gradient dout [N, Hq, 64] (dtype).  The pages state
 * the forward (notes, overall framework and key designs 1-3) and use it as a
 * trained block (notes, the loss/training paragraph); the gradients follow
 * by the chain rule through the gate softmax, the two softmax attentions,
 * the rotate-before-pool block sums and the rotations.
 *   dq: dtype [N, Hq, 64]; dk_loc, dv_loc, dk_cmp, dv_cmp: dtype [N, Hkv, 64];
 *   dgate: fp32, the shape of gate_logits.  No gradient for `a`.
 * The inputs are those given to pack3d_forward_train, with its `saved`
 * state (saved_bytes >= pack3d_saved_size()).  workspace: at least
 * pack3d_backward_workspace_size() bytes, 256-byte aligned, caller-owned.
 * Supported: bf16 with Hq/Hkv in {4, 8, 16} (else PACK3D_ERR_UNSUPPORTED).
 * Every sum runs in an order fixed by coordinates, so repacked inputs give
 * the permuted gradients bit for bit.
 */
int pack3d_backward(const pack3d_problem* prob, const void* q, const void* k_loc,
                    const void* v_loc, const void* k_cmp, const void* v_cmp, const float* a,
                    const int32_t* coords, const int32_t* cell_to_pos, const float* gate_logits,
                    const void* saved, size_t saved_bytes, const void* dout, void* dq,
                    void* dk_loc, void* dv_loc, void* dk_cmp, void* dv_cmp, float* dgate,
                    void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace pack3d_backward needs for this problem (0 if invalid). */
size_t pack3d_backward_workspace_size(const pack3d_problem* prob);

/*
 * The layer around the operator (notes, flowchart node B "linear projection
 * and layer normalisation produce Q, K_loc, V_loc, K_cmp, V_cmp" and node G
 * "residual output"; key design 1 writes q = R(c) W_Q LN(h),
 * k^b = R(c) W_K^b LN(h), v^b = W_V^b LN(h)).  bf16 tensors only; the
 * model width is `width` (a multiple of 64 in [64, 8192]).
 *
 * pack3d_layernorm_qkv: x = LayerNorm(h) over the width (biased variance,
 * x = (h - mean) / sqrt(var + eps) * gamma + beta; gamma/beta fp32 [width]
 * or NULL for 1/0), then the bias-free projections y = x W_qkv^T with
 * W_qkv bf16 [Hq*64 + 4*Hkv*64, width] row-major, its rows stacked in the
 * order Q, K_loc, V_loc, K_cmp, V_cmp.  Q and K_loc are rotated by R(c_i)
 * before their single rounding: q_rot [N, Hq, 64], k_rot [N, Hkv, 64];
 * v_loc, k_cmp, v_cmp [N, Hkv, 64] unrotated (k_cmp is rotated per cell
 * inside the summaries).  q_raw (nullable) also receives the unrotated Q (the
 * coordinate-blind compressed branch reads it).  h bf16 [N, width];
 * x_norm bf16 [N, width] receives LayerNorm(h) (the projections' input).
 */
int pack3d_layernorm_qkv(const pack3d_problem* prob, int32_t width, const void* h,
                         const float* gamma, const float* beta, float eps, const void* w_qkv,
                         const int32_t* coords, void* x_norm, void* q_rot, void* q_raw,
                         void* k_rot, void* v_loc, void* k_cmp, void* v_cmp, void* stream);

/*
 * Output projection with the residual (notes, flowchart node G):
 *   out[i, :] = residual[i, :] + o[i, :] W_o^T
 * o bf16 [N, Hq*64] (the heads' gated outputs, concatenated); W_o bf16
 * [width, Hq*64]; residual, out bf16 [N, width] (out must not alias o).
 */
int pack3d_out_proj(const pack3d_problem* prob, int32_t width, const void* o, const void* w_o,
                    const void* residual, void* out, void* stream);

/*
 * The whole layer: h' = h + PACK3D(LayerNorm(h) projections) W_o^T, i.e.
 * pack3d_layernorm_qkv, the block summaries, local attention, the
 * query->summary attention with the gate, and pack3d_out_proj, on one
 * stream.  a, coords, cell_to_pos, gate_logits as in pack3d_forward;
 * out bf16 [N, width] (must not alias h).  workspace: at least
 * pack3d_layer_workspace_size() bytes, 256-byte aligned, caller-owned.
 */
int pack3d_layer_forward(const pack3d_problem* prob, int32_t width, const void* h,
                         const float* gamma, const float* beta, float eps, const void* w_qkv,
                         const void* w_o, const float* a, const int32_t* coords,
                         const int32_t* cell_to_pos, const float* gate_logits, void* out,
                         void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace pack3d_layer_forward needs (0 if invalid). */
size_t pack3d_layer_workspace_size(const pack3d_problem* prob, int32_t width);

/* Bytes of workspace pack3d_forward needs for this problem (0 if invalid). */
size_t pack3d_forward_workspace_size(const pack3d_problem* prob);

/* cell_to_pos[(z*Y + y)*X + x] = i for every i < N.  Tokens whose
 * coordinates lie outside the lattice are skipped, and entries of cells no
 * token maps to are left unwritten, so the result is a valid index (one the
 * kernels may dereference) only when coords is a bijection onto the lattice:
 * fill cell_to_pos with -1 first and call pack3d_check_packing(), which must
 * report 0, before passing it to any other entry point. */
int pack3d_build_cell_index(const pack3d_problem* prob, const int32_t* coords,
                            int32_t* cell_to_pos, void* stream);

/* Counts, into *n_bad_dev (device int32, overwritten), the tokens whose
 * coordinates are outside the lattice or disagree with cell_to_pos. */
int pack3d_check_packing(const pack3d_problem* prob, const int32_t* coords,
                         const int32_t* cell_to_pos, int32_t* n_bad_dev, void* stream);

/* Text of the last error on this thread ("" if none). */
const char* pack3d_last_error(void);

/* Which kernel variant serves each op (there are no fallbacks). */
const char* pack3d_backend_info(void);

/* PACK3D_VERSION of the built library. */
int pack3d_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PACK3D_H */
