// The layer around the operator: LayerNorm, the five projections with the
// axial RoPE applied in the projection's epilogue, and the output
// projection with the residual.
//
// "Geometry Matters in Packed 3D Attention", papernotes.org notes: flowchart
// node B (linear projection and layer normalisation produce Q, K_loc, V_loc,
// K_cmp, V_cmp), node G (residual output), key design 1 (q = R(c) W_Q LN(h),
// k^b = R(c) W_K^b LN(h), v^b = W_V^b LN(h)).
//
//   k_ln_stats  per token: mean and 1/sqrt(var + eps) over the model width
//               (two passes over the row, biased variance)
//   k_gemm<E>   Y^T = W X^T for row-major W [F, K] and X [T, K], bf16 MFMA
//               32x32x16 with fp32 accumulation.  The X operand is
//               normalised on its way into LDS when LayerNorm statistics are
//               given.  Epilogues: E = kQkv splits the F = Hq*64 + 4*Hkv*64
//               outputs into Q, K_loc, V_loc, K_cmp, V_cmp (per-head layouts)
//               and rotates Q and K_loc by R(c) in fp32 before the single
//               rounding; E = kResidual writes residual + Y.
//
// Feature rows are the MFMA rows, so a lane's accumulators hold 4
// consecutive features of one token: rotary pairs (2p, 2p+1) stay in the
// lane.
#include "pack3d_device.h"

namespace pack3d {

namespace ly {

typedef KLds<bf16_t> TL;            // 64-element rows, bank-swizzled chunks

constexpr int kT = 128;             // tokens per workgroup tile
constexpr int kF = 128;             // features per workgroup tile
constexpr int kK = 64;              // contraction step (one LDS row)
constexpr int kWaves = 4;           // 2 x 2 waves, 64 x 64 outputs each
constexpr int kStage = kT * 8 / (64 * kWaves);   // 16-byte chunks per thread per operand

enum Epi { kQkv = 0, kResidual = 1 };

struct GemmArgs {
  const bf16_t* w;                  // [F, K]
  const bf16_t* x;                  // [T, K]
  const float* stats;               // [T, 2] (mean, rstd) or NULL: X used as is
  const float* gamma;               // [K] or NULL (1)
  const float* beta;                // [K] or NULL (0)
  int64_t t_rows;
  int32_t f_rows, k;
  int64_t nt;                       // token tiles, padded to a multiple of 8
  int32_t nf;                       // feature tiles
  // kQkv
  bf16_t* q;                        // [T, Hq, 64] rotated
  bf16_t* q_raw;                    // [T, Hq, 64] unrotated, or NULL
  bf16_t* k_loc;                    // [T, Hkv, 64] rotated
  bf16_t* v_loc;
  bf16_t* k_cmp;                    // unrotated (summaries rotate per cell)
  bf16_t* v_cmp;
  int32_t hq, hkv;
  const int32_t* coords;            // [T, 3]
  RopeTab rope;
  // kResidual
  const bf16_t* resid;              // [T, F]
  bf16_t* y;                        // [T, F]
};

__device__ __forceinline__ void row_frags(const bf16_t* t, int row, int h, bf16x8 (&f)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    f[s] = *reinterpret_cast<const bf16x8*>(t + TL::chunk_off(row, h * 4 + s));
}

// cos/sin of rotary pair p at cell (z, y, x); identity past the rotary pairs
__device__ __forceinline__ void pair_sincos(const RopeTab& rt, int p, int z, int y, int x,
                                            float& sn, float& cs) {
  if (p < rt.npairs) {
    const int ax = rt.axis[p];
    rope_sincos(rt.nu[p], ax == 0 ? z : (ax == 1 ? y : x), sn, cs);
  } else {
    sn = 0.0f;
    cs = 1.0f;
  }
}

template <int E>
__global__ __launch_bounds__(64 * kWaves) void k_gemm(GemmArgs A) {
  __shared__ __attribute__((aligned(16))) bf16_t w_l[2][kF * kK];
  __shared__ __attribute__((aligned(16))) bf16_t x_l[2][kT * kK];
  // XCD-aware order: the workgroups an XCD receives sweep every feature tile
  // of one token tile before the next, so the token tile stays in its L2
  const int64_t bid = blockIdx.x;
  const int xcd = (int)(bid % kNumXcd);
  const int64_t k8 = bid / kNumXcd;
  const int ft = (int)(k8 % A.nf);
  const int64_t tt = (k8 / A.nf) * kNumXcd + xcd;
  if (tt * kT >= A.t_rows) return;
  const int64_t t0 = tt * kT;
  const int f0 = ft * kF;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, col = lane & 31;
  const int fw = (wave & 1) * 64, tw = (wave >> 1) * 64;

  // staging: thread = (row tid/8 + 32 i, 16-byte chunk tid % 8)
  const int sch = tid & 7;
  float mu[kStage], rs[kStage];
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const int64_t t = t0 + (tid >> 3) + 32 * i;
    mu[i] = 0.0f;
    rs[i] = 1.0f;
    if (A.stats && t < A.t_rows) {
      mu[i] = A.stats[2 * t];
      rs[i] = A.stats[2 * t + 1];
    }
  }
  u32x4 sw[kStage], sx[kStage];
  auto load = [&](int kk) {
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const int fr = f0 + r;
      const int64_t tr = t0 + r;
      sw[i] = fr < A.f_rows ? ld16(A.w + (int64_t)fr * A.k + kk + sch * 8) : u32x4{0, 0, 0, 0};
      sx[i] = tr < A.t_rows ? ld16(A.x + tr * A.k + kk + sch * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int b, int kk) {
    float g[8], be[8];
    if (A.stats) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        g[e] = A.gamma ? A.gamma[kk + sch * 8 + e] : 1.0f;
        be[e] = A.beta ? A.beta[kk + sch * 8 + e] : 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const int r = (tid >> 3) + 32 * i;
      st16(w_l[b] + TL::chunk_off(r, sch), sw[i]);
      u32x4 xv = sx[i];
      if (A.stats && t0 + r < A.t_rows) {
        const bf16x8 raw = __builtin_bit_cast(bf16x8, sx[i]);
        bf16x8 nv;
#pragma unroll
        for (int e = 0; e < 8; ++e) nv[e] = (bf16_t)(((float)raw[e] - mu[i]) * rs[i] * g[e] + be[e]);
        xv = __builtin_bit_cast(u32x4, nv);
      }
      st16(x_l[b] + TL::chunk_off(r, sch), xv);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x16{};
  const int nk = A.k / kK;
  load(0);
  for (int ks = 0; ks < nk; ++ks) {
    const int b = ks & 1;
    store(b, ks * kK);
    __syncthreads();
    if (ks + 1 < nk) load((ks + 1) * kK);
    bf16x8 af[2][4], xf[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) row_frags(w_l[b], fw + 32 * i + col, h, af[i]);
#pragma unroll
    for (int j = 0; j < 2; ++j) row_frags(x_l[b], tw + 32 * j + col, h, xf[j]);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = Mma<bf16_t>::mma(af[i][s], xf[j][s], acc[i][j]);
  }

  // epilogue: lane = token (column), accumulator v = feature
  // fb + 8*(v/4) + 4*h + (v%4) of the 32-feature block fb
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t t = t0 + tw + 32 * j + col;
    if (t >= A.t_rows) continue;
    int cz = 0, cy = 0, cx = 0;
    if (E == kQkv) {
      cz = A.coords[3 * t];
      cy = A.coords[3 * t + 1];
      cx = A.coords[3 * t + 2];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int fb = f0 + fw + 32 * i;
      if (fb >= A.f_rows) continue;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q4 + e];
        const int f = fb + 8 * q4 + 4 * h;          // first of 4 consecutive features
        if (E == kResidual) {
          const int64_t o = t * A.f_rows + f;
          const bf16x4 r = *reinterpret_cast<const bf16x4*>(A.resid + o);
          bf16x4 out;
#pragma unroll
          for (int e = 0; e < 4; ++e) out[e] = (bf16_t)((float)r[e] + v[e]);
          *reinterpret_cast<bf16x4*>(A.y + o) = out;
        } else {
          // which projection, which head, which dims
          const int seg = f >> 6, dim = f & 63;
          bf16_t* dst;
          int heads, head;
          bool rot = false;
          if (seg < A.hq) {
            dst = A.q, heads = A.hq, head = seg, rot = true;
          } else {
            const int s2 = seg - A.hq, part = s2 / A.hkv;
            heads = A.hkv, head = s2 % A.hkv;
            dst = part == 0 ? A.k_loc : part == 1 ? A.v_loc : part == 2 ? A.k_cmp : A.v_cmp;
            rot = part == 0;
          }
          const int64_t o = (t * heads + head) * 64 + dim;
          if (seg < A.hq && A.q_raw) {
            bf16x4 raw;
#pragma unroll
            for (int e = 0; e < 4; ++e) raw[e] = (bf16_t)v[e];
            *reinterpret_cast<bf16x4*>(A.q_raw + o) = raw;
          }
          if (rot) {
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              float sn, cs;
              pair_sincos(A.rope, (dim >> 1) + pp, cz, cy, cx, sn, cs);
              const float x0 = v[2 * pp], x1 = v[2 * pp + 1];
              v[2 * pp] = cs * x0 - sn * x1;
              v[2 * pp + 1] = sn * x0 + cs * x1;
            }
          }
          bf16x4 out;
#pragma unroll
          for (int e = 0; e < 4; ++e) out[e] = (bf16_t)v[e];
          *reinterpret_cast<bf16x4*>(dst + o) = out;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_ln_stats: one wave per token; lane = 16-byte chunks lane, lane + 64, ...
// of the row.  Pass 1: mean; pass 2: mean square deviation (biased).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_ln_stats(const bf16_t* __restrict__ h, int64_t n,
                                                  int32_t width, float eps,
                                                  float* __restrict__ stats) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;
  const bf16_t* row = h + t * width;
  const int nch = width >> 3;
  float s = 0.0f;
  for (int c = lane; c < nch; c += 64) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(row + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)v[e];
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s += __shfl_xor(s, m);
  const float mean = s / (float)width;
  float d2 = 0.0f;
  for (int c = lane; c < nch; c += 64) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(row + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = (float)v[e] - mean;
      d2 = fmaf(d, d, d2);
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) d2 += __shfl_xor(d2, m);
  if (lane == 0) {
    stats[2 * t] = mean;
    stats[2 * t + 1] = 1.0f / sqrtf(d2 / (float)width + eps);
  }
}

}  // namespace ly

hipError_t launch_ln_stats(const Geom& g, int32_t width, const void* h, float eps, float* stats,
                           hipStream_t s) {
  hipLaunchKernelGGL(ly::k_ln_stats, dim3((unsigned)((g.N + 3) / 4)), dim3(256), 0, s,
                     (const bf16_t*)h, g.N, width, eps, stats);
  return hipGetLastError();
}

static void gemm_grid(ly::GemmArgs& A, int64_t t_rows, int32_t f_rows, int32_t k) {
  A.t_rows = t_rows;
  A.f_rows = f_rows;
  A.k = k;
  const int64_t tiles = (t_rows + ly::kT - 1) / ly::kT;
  A.nt = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
  A.nf = (f_rows + ly::kF - 1) / ly::kF;
}

hipError_t launch_qkv_proj(const Geom& g, int32_t width, const void* h, const float* stats,
                           const float* gamma, const float* beta, const void* w_qkv,
                           const int32_t* coords, void* q, void* q_raw, void* k_loc,
                           void* v_loc, void* k_cmp, void* v_cmp, hipStream_t s) {
  ly::GemmArgs A = {};
  A.w = (const bf16_t*)w_qkv;
  A.x = (const bf16_t*)h;
  A.stats = stats;
  A.gamma = gamma;
  A.beta = beta;
  gemm_grid(A, g.N, (g.Hq + 4 * g.Hkv) * 64, width);
  A.q = (bf16_t*)q;
  A.q_raw = (bf16_t*)q_raw;
  A.k_loc = (bf16_t*)k_loc;
  A.v_loc = (bf16_t*)v_loc;
  A.k_cmp = (bf16_t*)k_cmp;
  A.v_cmp = (bf16_t*)v_cmp;
  A.hq = g.Hq;
  A.hkv = g.Hkv;
  A.coords = coords;
  A.rope = g.rope;
  hipLaunchKernelGGL(ly::k_gemm<ly::kQkv>, dim3((unsigned)(A.nt * A.nf)), dim3(64 * ly::kWaves),
                     0, s, A);
  return hipGetLastError();
}

hipError_t launch_out_proj(const Geom& g, int32_t width, const void* o, const void* w_o,
                           const void* resid, void* out, hipStream_t s) {
  ly::GemmArgs A = {};
  A.w = (const bf16_t*)w_o;
  A.x = (const bf16_t*)o;
  gemm_grid(A, g.N, width, g.Hq * 64);
  A.resid = (const bf16_t*)resid;
  A.y = (bf16_t*)out;
  hipLaunchKernelGGL(ly::k_gemm<ly::kResidual>, dim3((unsigned)(A.nt * A.nf)),
                     dim3(64 * ly::kWaves), 0, s, A);
  return hipGetLastError();
}

}  // namespace pack3d
