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
// ---------------------------------------------------------------------------
constexpr int kSumWaves = 4;

// The forward asks for the key summaries multiplied by kscale (the softmax
// scale in log2 units, applied once before the single rounding) and for the
// norm of every scaled key summary in knorm [Hkv, M].
// P = passes of 8 cells (block volume <= 8 P), fixed at compile time so the
// per-cell rotations of small blocks take few registers.
template <typename T, int P>
__global__ __launch_bounds__(64 * kSumWaves) void k_block_summary(
    const T* __restrict__ kc, const T* __restrict__ vc, const float* __restrict__ a,
    const int32_t* __restrict__ c2p, T* __restrict__ ks, T* __restrict__ vs, Geom g,
    float kscale, float* __restrict__ knorm) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * kSumWaves + (threadIdx.x >> 6);
  if (j >= g.M) return;
  const int slot = lane >> 3, chunk = lane & 7;
  const int nbx = g.X / g.bx, nby = g.Y / g.by;
  const int jx = (int)(j % nbx), jy = (int)((j / nbx) % nby), jz = (int)(j / ((int64_t)nbx * nby));
  const float uniform = 1.0f / (float)g.bvol;
  const bool per_cell = g.summary_mode == PACK3D_SUMMARY_TOKEN;

  // positions and rotations of the lane's cells (one per pass)
  int64_t pos[P];
  float sn[P][4], cs[P][4];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    pos[p] = -1;
    const int u = p * 8 + slot;
    if (u < g.bvol) {
      const int ux = u % g.bx, uy = (u / g.bx) % g.by, uz = u / (g.bx * g.by);
      const int z = jz * g.bz + uz, y = jy * g.by + uy, x = jx * g.bx + ux;
      pos[p] = c2p[((int64_t)z * g.Y + y) * g.X + x];
      if (per_cell) chunk_sincos(g.rope, chunk, z, y, x, sn[p], cs[p]);
    }
  }

  for (int grp = 0; grp < g.Hkv; ++grp) {
    float ak[8], av[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ak[i] = av[i] = 0.0f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (pos[p] >= 0) {
        const int64_t row = (pos[p] * g.Hkv + grp) * 64 + chunk * 8;
        float kv[8], vv[8];
        load8<T>(kc + row, kv);
        load8<T>(vc + row, vv);
        const float w = a ? a[pos[p] * g.Hkv + grp] : uniform;
        if (per_cell) rotate8(kv, sn[p], cs[p]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ak[i] += w * kv[i];
          av[i] += w * vv[i];
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
      float csn[4], ccs[4];
      summary_sincos(g, chunk, jz * g.bz, jy * g.by, jx * g.bx, csn, ccs);
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

template <typename T>
static void launch_sum_t(const Geom& g, const void* k_cmp, const void* v_cmp, const float* a,
                         const int32_t* c2p, void* k_sum, void* v_sum, float kscale,
                         float* knorm, hipStream_t s) {
  const dim3 grid((unsigned)((g.M + kSumWaves - 1) / kSumWaves));
  const dim3 block(64 * kSumWaves);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, (const T*)k_cmp, (const T*)v_cmp, a, c2p,
                       (T*)k_sum, (T*)v_sum, g, kscale, knorm);
  };
  static_assert(kMaxBlockVol <= 64, "block volume");
  if (g.bvol <= 8) go(k_block_summary<T, 1>);
  else if (g.bvol <= 16) go(k_block_summary<T, 2>);
  else if (g.bvol <= 32) go(k_block_summary<T, 4>);
  else go(k_block_summary<T, 8>);
}

hipError_t launch_block_summary(const Geom& g, const void* k_cmp, const void* v_cmp,
                                const float* a, const int32_t* c2p, void* k_sum, void* v_sum,
                                float kscale, float* knorm, hipStream_t s) {
  if (g.bf16)
    launch_sum_t<bf16_t>(g, k_cmp, v_cmp, a, c2p, k_sum, v_sum, kscale, knorm, s);
  else
    launch_sum_t<float>(g, k_cmp, v_cmp, a, c2p, k_sum, v_sum, kscale, knorm, s);
  return hipGetLastError();
}

}  // namespace pack3d
