// Axial grid RoPE and the rotate-before-compression block summaries.
//
// "Geometry Matters in Packed 3D Attention", papernotes.org notes:
//   key design 1 - R(c) is a direct sum over the axes z, y, x of 2x2
//     rotations by omega_{a,r} * c_a, applied to queries and keys only;
//   key design 2 - each block summary is the normalised weighted sum of the
//     ROTATED keys of its cells (and of the unrotated values), so the
//     query-summary logit keeps every cell's displacement from the query.
//
// Both kernels are HBM streams: lanes own 16-byte chunks (8 dims) of token
// rows, so every wave moves whole 128-byte rows.
#include "pack3d_device.h"

namespace pack3d {

// ---------------------------------------------------------------------------
// k_rope: y[i, h, :] = R(coords[i]) x[i, h, :].
// 8 lanes per token, lane c owns dims 8c..8c+7 (4 rotary pairs) of every head:
// its 4 sines/cosines are computed once and reused for all heads.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_rope(const T* __restrict__ x, T* y, int64_t n,
                                              int32_t heads, const int32_t* __restrict__ coords,
                                              RopeTab rt) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tok = gid >> 3;
  const int chunk = (int)(gid & 7);
  if (tok >= n) return;
  const int z = coords[3 * tok], yy = coords[3 * tok + 1], xx = coords[3 * tok + 2];
  float sn[4], cs[4];
  chunk_sincos(rt, chunk, z, yy, xx, sn, cs);
  const T* src = x + tok * heads * 64 + chunk * 8;
  T* dst = y + tok * heads * 64 + chunk * 8;
  for (int h = 0; h < heads; ++h) {
    float v[8];
    load8<T>(src + h * 64, v);
    rotate8(v, sn, cs);
    store8<T>(dst + h * 64, v);
  }
}

hipError_t launch_rope(const Geom& g, const void* x, void* y, int32_t heads,
                       const int32_t* coords, hipStream_t s) {
  const int64_t threads = g.N * 8;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (g.bf16)
    hipLaunchKernelGGL(k_rope<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)x, (bf16_t*)y,
                       g.N, heads, coords, g.rope);
  else
    hipLaunchKernelGGL(k_rope<float>, grid, dim3(256), 0, s, (const float*)x, (float*)y, g.N,
                       heads, coords, g.rope);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// k_block_summary: one wave per block j.
// Lane = (cell slot u8 = lane/8, chunk = lane%8).  The block's cells are taken
// in raster order, 8 per pass; each lane rotates its K chunk by its cell's
// coordinates (rotation before the weighted sum), weights K and V by a, and
// accumulates in fp32.  The 8 cell slots are then reduced with a fixed XOR
// tree, so the summation order depends only on cell positions.  The
// summary-centre variant rotates the reduced sum once at the block centre
// instead; the coordinate-blind variant does not rotate.
//
// In the forward the same pass also rotates the local branch's keys: every
// token lies in exactly one block, so rotating K_loc of the block's cells
// with the cells' sines and cosines (already at hand) covers the lattice and
// writes the rows k_rope would write, in one HBM pre-pass instead of two.
// ---------------------------------------------------------------------------
constexpr int kSumWaves = 4;

// The forward asks for the key summaries multiplied by kscale (the softmax
// scale in log2 units, applied once before the single rounding) and for the
// norm of every scaled key summary in knorm [Hkv, M].
// P = passes of 8 cells (block volume <= 8 P), fixed at compile time so the
// per-cell rotations of small blocks take few registers.
// kl / kr (nullable): K_loc in, R(c) K_loc out, both [N, Hkv, 64].
// Raw 8-element row chunks, loaded first and converted when used, so every
// row a lane needs is in flight before any of them is waited for.
template <typename T> struct Row8 { u32x4 w[sizeof(T) / 2]; };
template <typename T>
__device__ __forceinline__ void ld_row8(Row8<T>& r, const T* p) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) r.w[i] = ld16(p + i * (16 / sizeof(T)));
}
template <typename T>
__device__ __forceinline__ void cvt_row8(const Row8<T>& r, float* v) {
  if constexpr (std::is_same<T, float>::value) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_bit_cast(f32x4, r.w[i / 4])[i % 4];
  } else {
    const bf16x8 b = __builtin_bit_cast(bf16x8, r.w[0]);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)b[i];
  }
}

// Sines and cosines of the 4 pairs of dim-chunk `chunk` at (z, y, x), from
// the rotary parameters staged in LDS (the same values and arithmetic as
// chunk_sincos).
__device__ __forceinline__ void chunk_sincos_lds(const double* nu, const int32_t* ax, int npairs,
                                                 int chunk, double z, double y, double x,
                                                 float* sn, float* cs) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = chunk * 4 + i;
    if (p < npairs) {
      const int a = ax[p];
      rope_sincos(nu[p], a == 0 ? z : (a == 1 ? y : x), sn[i], cs[i]);
    } else {
      sn[i] = 0.0f;
      cs[i] = 1.0f;
    }
  }
}

// KG: KV groups whose rows are loaded together (1 or 2); kA: weights given
// (else uniform); kL: K_loc given (rotate it too).  Every load is
// unconditional (clamped addresses, results selected afterwards), so the
// compiler's memory-counter waits come only where the values are used.
template <typename T, int P, int KG, bool kA, bool kL>
__global__ __launch_bounds__(64 * kSumWaves) void k_block_summary(
    const T* __restrict__ kc, const T* __restrict__ vc, const float* __restrict__ a,
    const int32_t* __restrict__ c2p, T* __restrict__ ks, T* __restrict__ vs, Geom g,
    float kscale, float* __restrict__ knorm, const T* __restrict__ kl, T* __restrict__ kr) {
  // the rotary parameters, staged once per workgroup: indexed by a per-lane
  // pair, the kernel arguments would be read through vector memory, one
  // dependent read after another
  __shared__ double s_nu[kMaxPairs];
  __shared__ int32_t s_ax[kMaxPairs];
  if (threadIdx.x < kMaxPairs) {
    s_nu[threadIdx.x] = g.rope.nu[threadIdx.x];
    s_ax[threadIdx.x] = g.rope.axis[threadIdx.x];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * kSumWaves + (threadIdx.x >> 6);
  if (j >= g.M) return;
  const int slot = lane >> 3, chunk = lane & 7;
  const int nbx = g.X / g.bx, nby = g.Y / g.by;
  const int jx = (int)(j % nbx), jy = (int)((j / nbx) % nby), jz = (int)(j / ((int64_t)nbx * nby));
  const float uniform = 1.0f / (float)g.bvol;
  const bool per_cell = g.summary_mode == PACK3D_SUMMARY_TOKEN;
  const bool cell_rot = per_cell || kL;

  // positions of the lane's cells (one per pass), then their rotations while
  // the positions are in flight
  int64_t pos[P];
  bool cok[P];
  int cz[P], cy[P], cx[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int u0 = p * 8 + slot;
    cok[p] = u0 < g.bvol;
    const int u = cok[p] ? u0 : 0;
    const int ux = u % g.bx, uy = (u / g.bx) % g.by, uz = u / (g.bx * g.by);
    cz[p] = jz * g.bz + uz;
    cy[p] = jy * g.by + uy;
    cx[p] = jx * g.bx + ux;
    pos[p] = c2p[((int64_t)cz[p] * g.Y + cy[p]) * g.X + cx[p]];
  }
  float sn[P][4], cs[P][4];
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (cell_rot)
      chunk_sincos_lds(s_nu, s_ax, g.rope.npairs, chunk, cz[p], cy[p], cx[p], sn[p], cs[p]);

  for (int g0 = 0; g0 < g.Hkv; g0 += KG) {
    // every row of these groups and passes in flight before any is used
    Row8<T> rk[KG][P], rv[KG][P], rl[KG][P];
    float w[KG][P];
#pragma unroll
    for (int gi = 0; gi < KG; ++gi)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int grp = g0 + gi < g.Hkv ? g0 + gi : g.Hkv - 1;
        const int64_t row = (pos[p] * g.Hkv + grp) * 64 + chunk * 8;
        ld_row8<T>(rk[gi][p], kc + row);
        ld_row8<T>(rv[gi][p], vc + row);
        if constexpr (kL) ld_row8<T>(rl[gi][p], kl + row);
        if constexpr (kA) w[gi][p] = a[pos[p] * g.Hkv + grp];
        else w[gi][p] = uniform;
      }
#pragma unroll
    for (int gi = 0; gi < KG; ++gi) {
      const int grp = g0 + gi;
      if (grp >= g.Hkv) break;
      float ak[8], av[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ak[i] = av[i] = 0.0f;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if (cok[p]) {
          const int64_t row = (pos[p] * g.Hkv + grp) * 64 + chunk * 8;
          float kv[8], vv[8];
          cvt_row8<T>(rk[gi][p], kv);
          cvt_row8<T>(rv[gi][p], vv);
          if constexpr (kL) {
            float lv[8];
            cvt_row8<T>(rl[gi][p], lv);
            rotate8(lv, sn[p], cs[p]);
            store8<T>(kr + row, lv);
          }
          if (per_cell) rotate8(kv, sn[p], cs[p]);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            ak[i] += w[gi][p] * kv[i];
            av[i] += w[gi][p] * vv[i];
          }
        }
      }
#pragma unroll
      for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ak[i] += __shfl_xor(ak[i], off);
          av[i] += __shfl_xor(av[i], off);
        }
      }
      if (g.summary_mode == PACK3D_SUMMARY_CENTRE) {
        // the block's geometric centre (half-integers are exact in double)
        float csn[4], ccs[4];
        chunk_sincos_lds(s_nu, s_ax, g.rope.npairs, chunk, jz * g.bz + 0.5 * (g.bz - 1),
                         jy * g.by + 0.5 * (g.by - 1), jx * g.bx + 0.5 * (g.bx - 1), csn, ccs);
        rotate8(ak, csn, ccs);
      }
      float n2 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ak[i] *= kscale;
        n2 = fmaf(ak[i], ak[i], n2);
      }
      if (slot == 0) {
        const int64_t o = ((int64_t)grp * g.M + j) * 64 + chunk * 8;
        store8<T>(ks + o, ak);
        store8<T>(vs + o, av);
      }
      if (knorm) {
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) n2 += __shfl_xor(n2, off);
        if (lane == 0) knorm[(int64_t)grp * g.M + j] = sqrtf(n2);
      }
    }
  }
}

template <typename T>
static void launch_sum_t(const Geom& g, const void* k_cmp, const void* v_cmp, const float* a,
                         const int32_t* c2p, void* k_sum, void* v_sum, float kscale,
                         float* knorm, const void* k_loc, void* k_rot, hipStream_t s) {
  const dim3 grid((unsigned)((g.M + kSumWaves - 1) / kSumWaves));
  const dim3 block(64 * kSumWaves);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, (const T*)k_cmp, (const T*)v_cmp, a, c2p,
                       (T*)k_sum, (T*)v_sum, g, kscale, knorm, (const T*)k_loc, (T*)k_rot);
  };
  static_assert(kMaxBlockVol <= 64, "block volume");
  // two KV groups' rows in flight together where the registers allow
  constexpr int KG = std::is_same<T, float>::value ? 1 : 2;
  auto by_vol = [&](auto kA, auto kL) {
    constexpr bool A_ = decltype(kA)::value, L_ = decltype(kL)::value;
    if (g.bvol <= 8) go(k_block_summary<T, 1, KG, A_, L_>);
    else if (g.bvol <= 16) go(k_block_summary<T, 2, KG, A_, L_>);
    else if (g.bvol <= 32) go(k_block_summary<T, 4, 1, A_, L_>);
    else go(k_block_summary<T, 8, 1, A_, L_>);
  };
  using yes = std::true_type;
  using no = std::false_type;
  if (a && k_loc) by_vol(yes{}, yes{});
  else if (a) by_vol(yes{}, no{});
  else if (k_loc) by_vol(no{}, yes{});
  else by_vol(no{}, no{});
}

hipError_t launch_block_summary(const Geom& g, const void* k_cmp, const void* v_cmp,
                                const float* a, const int32_t* c2p, void* k_sum, void* v_sum,
                                float kscale, float* knorm, const void* k_loc, void* k_rot,
                                hipStream_t s) {
  if (g.bf16)
    launch_sum_t<bf16_t>(g, k_cmp, v_cmp, a, c2p, k_sum, v_sum, kscale, knorm, k_loc, k_rot, s);
  else
    launch_sum_t<float>(g, k_cmp, v_cmp, a, c2p, k_sum, v_sum, kscale, knorm, k_loc, k_rot, s);
  return hipGetLastError();
}

}  // namespace pack3d
