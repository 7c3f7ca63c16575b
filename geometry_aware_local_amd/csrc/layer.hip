// The layer around the operator: LayerNorm, the five projections with the
// axial RoPE applied in the projection's epilogue, and the output
// projection with the residual.
//
// "Geometry Matters in Packed 3D Attention", papernotes.org notes: flowchart
// node B (linear projection and layer normalisation produce Q, K_loc, V_loc,
// K_cmp, V_cmp), node G (residual output), key design 1 (q = R(c) W_Q LN(h),
// k^b = R(c) W_K^b LN(h), v^b = W_V^b LN(h)).
//
//   k_layernorm per token: x = (h - mean) / sqrt(var + eps) * gamma + beta
//               over the model width (biased variance), once per token
//   k_gemm<E>   Y^T = W X^T for row-major W [F, K] and X [T, K], bf16 MFMA
//               32x32x16 with fp32 accumulation.  Epilogues: E = kQkv splits
//               the F = Hq*64 + 4*Hkv*64 outputs into Q, K_loc, V_loc, K_cmp,
//               V_cmp (per-head layouts) and rotates Q and K_loc by R(c) in
//               fp32 before the single rounding; E = kResidual writes
//               residual + Y.  The output tile is staged through LDS so every
//               global store moves whole 16-byte chunks of 128-byte rows.
//               256 x 256 tiles (8 waves of 64 features x 128 tokens): each
//               token tile is read once per 256 features and each weight
//               tile once per 256 tokens, which is what bounds a contraction
//               this short (K = the model width) on this part.
//
// Feature rows are the MFMA rows, so a lane's accumulators hold 4
// consecutive features of one token: rotary pairs (2p, 2p+1) stay in the
// lane.
#include "pack3d_device.h"

namespace pack3d {

namespace ly {

typedef KLds<bf16_t> TL;            // 64-element rows, bank-swizzled chunks

constexpr int kK = 64;              // contraction step (one LDS row)

// Tile shape: WF x WT waves, each 64 features x 32*NJ tokens; the workgroup
// covers 64*WF features x 32*NJ*WT tokens.
template <int WF, int WT, int NJ>
struct GTile {
  static constexpr int W = WF * WT;
  static constexpr int F = 64 * WF, T = 32 * NJ * WT;
  static constexpr int SW = F * 8 / (64 * W), SX = T * 8 / (64 * W);   // chunks per thread
  static_assert(F * 8 % (64 * W) == 0 && T * 8 % (64 * W) == 0, "whole chunks per thread");
};
// Both projections use 256 features x 256 tokens (8 waves).  Against 128 x
// 128 tiles this halves the operand re-reads from L2 (the bound of a
// contraction as short as the model width); the layer measured 0.67 -> 0.58
// ms for LayerNorm + the stacked projection and 0.29 -> 0.25 ms for the
// output projection at 262,144 tokens, width 512.
typedef GTile<4, 2, 4> QkvTile;
typedef GTile<4, 2, 4> OutTile;

enum Epi { kQkv = 0, kResidual = 1 };

struct GemmArgs {
  const bf16_t* w;                  // [F, K]
  const bf16_t* x;                  // [T, K]
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

// cos/sin of rotary pair p at cell (z, y, x) from the workgroup's copy of
// the rotary table in LDS (axis -1: past the rotary pairs, the identity).
__device__ __forceinline__ void pair_sincos(const double* nu, const int* axis, int p, int z,
                                            int y, int x, float& sn, float& cs) {
  const int ax = axis[p];
  rope_sincos(nu[p], ax == 0 ? z : (ax == 1 ? y : x), sn, cs);
  sn = ax < 0 ? 0.0f : sn;
  cs = ax < 0 ? 1.0f : cs;
}

template <int E, class Tile>
__global__ __launch_bounds__(64 * Tile::W) void k_gemm(GemmArgs A) {
  constexpr int W = Tile::W, kF = Tile::F, kT = Tile::T, NJ = kT / 32 / (W / (kF / 64));
  // operand tiles (double-buffered); after the contraction the same memory
  // stages the output tile for coalesced stores
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * (kF + kT) * kK];
  __shared__ double nu_l[kMaxPairs];
  __shared__ int ax_l[kMaxPairs];
  auto w_l = [&](int b) { return lds + b * kF * kK; };
  auto x_l = [&](int b) { return lds + 2 * kF * kK + b * kT * kK; };
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
  const int fw = (wave % (kF / 64)) * 64, tw = (wave / (kF / 64)) * (32 * NJ);
  if (E == kQkv && tid < kMaxPairs) {        // read after the first barrier below
    const bool on = tid < A.rope.npairs;
    nu_l[tid] = on ? A.rope.nu[tid] : 0.0;
    ax_l[tid] = on ? A.rope.axis[tid] : -1;
  }

  // staging: thread = (row tid/8 + 8W i, 16-byte chunk tid % 8)
  const int sch = tid & 7;
  u32x4 sw[Tile::SW], sx[Tile::SX];
  auto load = [&](int kk) {
#pragma unroll
    for (int i = 0; i < Tile::SW; ++i) {
      const int fr = f0 + (tid >> 3) + 8 * W * i;
      sw[i] = fr < A.f_rows ? ld16(A.w + (int64_t)fr * A.k + kk + sch * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < Tile::SX; ++i) {
      const int64_t tr = t0 + (tid >> 3) + 8 * W * i;
      sx[i] = tr < A.t_rows ? ld16(A.x + tr * A.k + kk + sch * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int i = 0; i < Tile::SW; ++i)
      st16(w_l(b) + TL::chunk_off((tid >> 3) + 8 * W * i, sch), sw[i]);
#pragma unroll
    for (int i = 0; i < Tile::SX; ++i)
      st16(x_l(b) + TL::chunk_off((tid >> 3) + 8 * W * i, sch), sx[i]);
  };

  f32x16 acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  const int nk = A.k / kK;
  load(0);
  for (int ks = 0; ks < nk; ++ks) {
    const int b = ks & 1;
    store(b);
    __syncthreads();
    if (ks + 1 < nk) load((ks + 1) * kK);
    bf16x8 af[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) row_frags(w_l(b), fw + 32 * i + col, h, af[i]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      bf16x8 xf[4];
      row_frags(x_l(b), tw + 32 * j + col, h, xf);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][j] = Mma<bf16_t>::mma(af[i][s], xf[s], acc[i][j]);
    }
  }
  __syncthreads();                  // operand tiles free: reuse for the output

  // Accumulator layout: lane = token tw + 32 j + col, element 4 q4 + e =
  // feature fw + 32 i + 8 q4 + 4 h + e of the tile.
  // The output is staged in rounds; round r holds token blocks JR r ..
  // JR r + JR - 1 of every wave, so all waves work in every round.  Staged
  // row sr is token t0 + (sr / (32 JR)) (32 NJ) + 32 JR r + sr % (32 JR).
  constexpr int kWT = W / (kF / 64);
  if (E == kResidual) {
    constexpr int JR = 1, RR = kWT * 32 * JR;      // rows per round
    constexpr int kOS32 = kF + 4;
    static_assert(NJ % JR == 0 && RR * kF / 8 % (64 * W) == 0, "whole rounds");
    static_assert(RR * kOS32 * 4 <= (int)sizeof(lds), "staging fits the operand tiles");
    float* ot = reinterpret_cast<float*>(lds);
#pragma unroll 1
    for (int r = 0; r < NJ / JR; ++r) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (j / JR != r) continue;
        const int sr = (tw / (32 * NJ)) * 32 * JR + (j % JR) * 32 + col;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q4 + e];
            *reinterpret_cast<f32x4*>(ot + sr * kOS32 + fw + 32 * i + 8 * q4 + 4 * h) = v;
          }
      }
      __syncthreads();
#pragma unroll
      for (int c8 = 0; c8 < RR * kF / 8 / (64 * W); ++c8) {
        const int c = tid + 64 * W * c8, sr = c / (kF / 8), fc = (c % (kF / 8)) * 8;
        const int64_t t = t0 + (sr / (32 * JR)) * 32 * NJ + 32 * JR * r + sr % (32 * JR);
        const int f = f0 + fc;
        if (t < A.t_rows && f < A.f_rows) {
          const f32x4 a0 = *reinterpret_cast<const f32x4*>(ot + sr * kOS32 + fc);
          const f32x4 a1 = *reinterpret_cast<const f32x4*>(ot + sr * kOS32 + fc + 4);
          const int64_t o = t * A.f_rows + f;
          const bf16x8 rs = *reinterpret_cast<const bf16x8*>(A.resid + o);
          bf16x8 out;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            out[e] = (bf16_t)((float)rs[e] + a0[e]);
            out[4 + e] = (bf16_t)((float)rs[4 + e] + a1[e]);
          }
          *reinterpret_cast<bf16x8*>(A.y + o) = out;
        }
      }
      __syncthreads();
    }
  } else {
    // bf16 staging in rounds of 128 tokens: [128][kOS16], then 16-byte stores
    // of each (token, projection head) 128-byte row.  With q_raw the
    // unrotated Q is staged and stored first.
    constexpr int JR = 2, RR = kWT * 32 * JR;      // rows per round
    constexpr int kOS16 = kF + 8;
    static_assert(NJ % JR == 0 && RR * kF / 8 % (64 * W) == 0, "whole rounds");
    static_assert(RR * kOS16 * 2 <= (int)sizeof(lds), "staging fits the operand tiles");
    // The round's rotary table follows the staging area: row sr holds (sin,
    // cos) of every pair for the token of staged row sr, computed once per
    // workgroup instead of once per head (rows padded by 16 bytes so the 32
    // lanes of a half-wave read different banks).
    constexpr int kTabS = 2 * 32 + 4;
    static_assert(RR * kOS16 * 2 + RR * kTabS * 4 <= (int)sizeof(lds), "table fits");
    static_assert(RR * 4 == 64 * W, "one table task per thread");
    bf16_t* ot = lds;
    float* tab = reinterpret_cast<float*>(lds + RR * kOS16);
    const int seg = (f0 + fw) >> 6;               // the wave's 64 features: one head
    const bool rotatable = (seg < A.hq || (seg - A.hq) / A.hkv == 0) && seg < A.hq + 4 * A.hkv;
    const bool any_rot = f0 < (A.hq + A.hkv) * 64;  // the tile holds a Q or K_loc head
    const bool raw_pass = A.q_raw != nullptr && f0 < A.hq * 64;
#pragma unroll 1
    for (int pass = raw_pass ? 0 : 1; pass < 2; ++pass) {
      const bool rotate = pass == 1;
#pragma unroll 1
      for (int r = 0; r < NJ / JR; ++r) {
        if (rotate && any_rot) {
          // task: staged row tid / 4, pairs 8 (tid % 4) .. + 7
          const int sr = tid >> 2, pg = tid & 3;
          const int64_t t = t0 + (sr / (32 * JR)) * 32 * NJ + 32 * JR * r + sr % (32 * JR);
          int cz = 0, cy = 0, cx = 0;
          if (t < A.t_rows) {
            cz = A.coords[3 * t];
            cy = A.coords[3 * t + 1];
            cx = A.coords[3 * t + 2];
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float s0, c0, s1, c1;
            pair_sincos(nu_l, ax_l, 8 * pg + 2 * u, cz, cy, cx, s0, c0);
            pair_sincos(nu_l, ax_l, 8 * pg + 2 * u + 1, cz, cy, cx, s1, c1);
            *reinterpret_cast<f32x4*>(tab + sr * kTabS + 16 * pg + 4 * u) = f32x4{s0, c0, s1, c1};
          }
          __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (j / JR != r) continue;
          const int sr = (tw / (32 * NJ)) * 32 * JR + (j % JR) * 32 + col;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q4 + e];
              if (rotate && rotatable) {
                // dims 32 i + 8 q4 + 4 h .. +3: pairs p and p + 1
                const int p = 16 * i + 4 * q4 + 2 * h;
                const f32x4 w = *reinterpret_cast<const f32x4*>(tab + sr * kTabS + 2 * p);
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                  const float sn = w[2 * pp], cs = w[2 * pp + 1];
                  const float x0 = v[2 * pp], x1 = v[2 * pp + 1];
                  v[2 * pp] = cs * x0 - sn * x1;
                  v[2 * pp + 1] = sn * x0 + cs * x1;
                }
              }
              bf16x4 o;
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = (bf16_t)v[e];
              *reinterpret_cast<bf16x4*>(ot + sr * kOS16 + fw + 32 * i + 8 * q4 + 4 * h) = o;
            }
        }
        __syncthreads();
#pragma unroll
        for (int c8 = 0; c8 < RR * kF / 8 / (64 * W); ++c8) {
          const int c = tid + 64 * W * c8, sr = c / (kF / 8), fc = (c % (kF / 8)) * 8;
          const int64_t t = t0 + (sr / (32 * JR)) * 32 * NJ + 32 * JR * r + sr % (32 * JR);
          const int f = f0 + fc;
          if (t >= A.t_rows || f >= A.f_rows) continue;
          const int sg = f >> 6, dim = f & 63;
          bf16_t* dst;
          int heads, head;
          if (sg < A.hq) {
            dst = rotate ? A.q : A.q_raw, heads = A.hq, head = sg;
          } else {
            if (!rotate) continue;
            const int s2 = sg - A.hq, part = s2 / A.hkv;
            heads = A.hkv, head = s2 % A.hkv;
            dst = part == 0 ? A.k_loc : part == 1 ? A.v_loc : part == 2 ? A.k_cmp : A.v_cmp;
          }
          st16(dst + (t * heads + head) * 64 + dim, ld16(ot + sr * kOS16 + fc));
        }
        __syncthreads();
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_layernorm: x = (h - mean) / sqrt(var + eps) * gamma + beta, one wave per
// token.  The row is read once into registers (lane = 16-byte chunks
// lane + 64 u, u < U = ceil(width / 512), chosen at launch so short rows keep
// few registers); mean, then the mean square deviation (biased) of the held
// values, then the normalised row.
// ---------------------------------------------------------------------------
template <int U>                      // chunks per lane: width <= 512 U
__global__ __launch_bounds__(256) void k_layernorm(const bf16_t* __restrict__ h,
                                                   const float* __restrict__ gamma,
                                                   const float* __restrict__ beta, int64_t n,
                                                   int32_t width, float eps,
                                                   bf16_t* __restrict__ x) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;
  const bf16_t* row = h + t * width;
  const int nch = width >> 3;
  bf16x8 v[U];
  float s = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = lane + 64 * u;
    if (c < nch) {
      v[u] = *reinterpret_cast<const bf16x8*>(row + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (float)v[u][e];
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s += __shfl_xor(s, m);
  const float mean = s / (float)width;
  float d2 = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = lane + 64 * u;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = (float)v[u][e] - mean;
        d2 = fmaf(d, d, d2);
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) d2 += __shfl_xor(d2, m);
  const float rstd = 1.0f / sqrtf(d2 / (float)width + eps);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = lane + 64 * u;
    if (c < nch) {
      f32x4 g[2] = {f32x4{1.0f, 1.0f, 1.0f, 1.0f}, f32x4{1.0f, 1.0f, 1.0f, 1.0f}};
      f32x4 b[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
      if (gamma) {
        g[0] = *reinterpret_cast<const f32x4*>(gamma + 8 * c);
        g[1] = *reinterpret_cast<const f32x4*>(gamma + 8 * c + 4);
      }
      if (beta) {
        b[0] = *reinterpret_cast<const f32x4*>(beta + 8 * c);
        b[1] = *reinterpret_cast<const f32x4*>(beta + 8 * c + 4);
      }
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = (bf16_t)(((float)v[u][e] - mean) * rstd * g[e >> 2][e & 3] + b[e >> 2][e & 3]);
      *reinterpret_cast<bf16x8*>(x + t * width + 8 * c) = o;
    }
  }
}

}  // namespace ly

hipError_t launch_layernorm(const Geom& g, int32_t width, const void* h, const float* gamma,
                            const float* beta, float eps, void* x, hipStream_t s) {
  const dim3 grid((unsigned)((g.N + 3) / 4)), block(256);
  const int u = (width + 511) / 512;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, (const bf16_t*)h, gamma, beta, g.N, width, eps,
                       (bf16_t*)x);
  };
  if (u <= 1) go(ly::k_layernorm<1>);
  else if (u <= 2) go(ly::k_layernorm<2>);
  else if (u <= 4) go(ly::k_layernorm<4>);
  else if (u <= 8) go(ly::k_layernorm<8>);
  else go(ly::k_layernorm<16>);
  return hipGetLastError();
}

template <class Tile>
static void gemm_grid(ly::GemmArgs& A, int64_t t_rows, int32_t f_rows, int32_t k) {
  A.t_rows = t_rows;
  A.f_rows = f_rows;
  A.k = k;
  const int64_t tiles = (t_rows + Tile::T - 1) / Tile::T;
  A.nt = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
  A.nf = (f_rows + Tile::F - 1) / Tile::F;
}

hipError_t launch_qkv_proj(const Geom& g, int32_t width, const void* x, const void* w_qkv,
                           const int32_t* coords, void* q, void* q_raw, void* k_loc,
                           void* v_loc, void* k_cmp, void* v_cmp, hipStream_t s) {
  ly::GemmArgs A = {};
  A.w = (const bf16_t*)w_qkv;
  A.x = (const bf16_t*)x;
  typedef ly::QkvTile Tile;
  gemm_grid<Tile>(A, g.N, (g.Hq + 4 * g.Hkv) * 64, width);
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
  hipLaunchKernelGGL((ly::k_gemm<ly::kQkv, Tile>), dim3((unsigned)(A.nt * A.nf)), dim3(64 * Tile::W),
                     0, s, A);
  return hipGetLastError();
}

hipError_t launch_out_proj(const Geom& g, int32_t width, const void* o, const void* w_o,
                           const void* resid, void* out, hipStream_t s) {
  ly::GemmArgs A = {};
  A.w = (const bf16_t*)w_o;
  A.x = (const bf16_t*)o;
  typedef ly::OutTile Tile;
  gemm_grid<Tile>(A, g.N, width, g.Hq * 64);
  A.resid = (const bf16_t*)resid;
  A.y = (bf16_t*)out;
  hipLaunchKernelGGL((ly::k_gemm<ly::kResidual, Tile>), dim3((unsigned)(A.nt * A.nf)),
                     dim3(64 * Tile::W), 0, s, A);
  return hipGetLastError();
}

}  // namespace pack3d
