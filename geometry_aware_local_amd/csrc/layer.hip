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

template <int E>
__global__ __launch_bounds__(64 * kWaves) void k_gemm(GemmArgs A) {
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
  const int fw = (wave & 1) * 64, tw = (wave >> 1) * 64;
  if (E == kQkv && tid < kMaxPairs) {        // read after the first barrier below
    const bool on = tid < A.rope.npairs;
    nu_l[tid] = on ? A.rope.nu[tid] : 0.0;
    ax_l[tid] = on ? A.rope.axis[tid] : -1;
  }

  // staging: thread = (row tid/8 + 32 i, 16-byte chunk tid % 8)
  const int sch = tid & 7;
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
  auto store = [&](int b) {
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const int r = (tid >> 3) + 32 * i;
      st16(w_l(b) + TL::chunk_off(r, sch), sw[i]);
      st16(x_l(b) + TL::chunk_off(r, sch), sx[i]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x16{};
  const int nk = A.k / kK;
  load(0);
  for (int ks = 0; ks < nk; ++ks) {
    const int b = ks & 1;
    store(b);
    __syncthreads();
    if (ks + 1 < nk) load((ks + 1) * kK);
    bf16x8 af[2][4], xf[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) row_frags(w_l(b), fw + 32 * i + col, h, af[i]);
#pragma unroll
    for (int j = 0; j < 2; ++j) row_frags(x_l(b), tw + 32 * j + col, h, xf[j]);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = Mma<bf16_t>::mma(af[i][s], xf[j][s], acc[i][j]);
  }
  __syncthreads();                  // operand tiles free: reuse for the output

  // Accumulator layout: lane = token tw + 32 j + col, element 4 q4 + e =
  // feature fw + 32 i + 8 q4 + 4 h + e of the tile.
  if (E == kResidual) {
    // fp32 staging in two halves of 64 tokens: [64][kOS32] floats
    constexpr int kOS32 = kF + 4;
    float* ot = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (tw == 64 * half) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              f32x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q4 + e];
              *reinterpret_cast<f32x4*>(ot + (32 * j + col) * kOS32 + fw + 32 * i + 8 * q4 +
                                        4 * h) = v;
            }
      }
      __syncthreads();
      // 64 tokens x 16 chunks of 8 features; 4 chunks per thread
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int c = tid + 256 * c4, tl = c >> 4, fc = (c & 15) * 8;
        const int64_t t = t0 + 64 * half + tl;
        const int f = f0 + fc;
        if (t < A.t_rows && f < A.f_rows) {
          const f32x4 a0 = *reinterpret_cast<const f32x4*>(ot + tl * kOS32 + fc);
          const f32x4 a1 = *reinterpret_cast<const f32x4*>(ot + tl * kOS32 + fc + 4);
          const int64_t o = t * A.f_rows + f;
          const bf16x8 r = *reinterpret_cast<const bf16x8*>(A.resid + o);
          bf16x8 out;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            out[e] = (bf16_t)((float)r[e] + a0[e]);
            out[4 + e] = (bf16_t)((float)r[4 + e] + a1[e]);
          }
          *reinterpret_cast<bf16x8*>(A.y + o) = out;
        }
      }
      __syncthreads();
    }
  } else {
    // bf16 staging of the whole tile: [128 tokens][kOS16], then 16-byte
    // stores of each (token, projection head) 128-byte row.  With q_raw the
    // unrotated Q tile is staged and stored first.
    constexpr int kOS16 = kF + 8;
    bf16_t* ot = lds;
    int cz[2], cy[2], cx[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t t = t0 + tw + 32 * j + col;
      cz[j] = cy[j] = cx[j] = 0;
      if (t < A.t_rows) {
        cz[j] = A.coords[3 * t];
        cy[j] = A.coords[3 * t + 1];
        cx[j] = A.coords[3 * t + 2];
      }
    }
    const bool raw_pass = A.q_raw != nullptr && f0 < A.hq * 64;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const bool rotate = pass == 1;
      if (!rotate && !raw_pass) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int seg = (f0 + fw) >> 6;         // the wave's 64 features: one head
          const bool rot = rotate && (seg < A.hq || (seg - A.hq) / A.hkv == 0) &&
                           seg < A.hq + 4 * A.hkv;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q4 + e];
            if (rot) {
              // dims 32 i + 8 q4 + 4 h .. +3: pairs p and p + 1
              const int p = 16 * i + 4 * q4 + 2 * h;
#pragma unroll
              for (int pp = 0; pp < 2; ++pp) {
                float sn, cs;
                pair_sincos(nu_l, ax_l, p + pp, cz[j], cy[j], cx[j], sn, cs);
                const float x0 = v[2 * pp], x1 = v[2 * pp + 1];
                v[2 * pp] = cs * x0 - sn * x1;
                v[2 * pp + 1] = sn * x0 + cs * x1;
              }
            }
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (bf16_t)v[e];
            *reinterpret_cast<bf16x4*>(ot + (tw + 32 * j + col) * kOS16 + fw + 32 * i + 8 * q4 +
                                       4 * h) = o;
          }
        }
      __syncthreads();
      // 128 tokens x 16 chunks of 8 features; 8 chunks per thread
#pragma unroll
      for (int c8 = 0; c8 < 8; ++c8) {
        const int c = tid + 256 * c8, tl = c >> 4, fc = (c & 15) * 8;
        const int64_t t = t0 + tl;
        const int f = f0 + fc;
        if (t >= A.t_rows || f >= A.f_rows) continue;
        const int seg = f >> 6, dim = f & 63;
        bf16_t* dst;
        int heads, head;
        if (seg < A.hq) {
          dst = rotate ? A.q : A.q_raw, heads = A.hq, head = seg;
        } else {
          if (!rotate) continue;
          const int s2 = seg - A.hq, part = s2 / A.hkv;
          heads = A.hkv, head = s2 % A.hkv;
          dst = part == 0 ? A.k_loc : part == 1 ? A.v_loc : part == 2 ? A.k_cmp : A.v_cmp;
        }
        st16(dst + (t * heads + head) * 64 + dim, ld16(ot + tl * kOS16 + fc));
      }
      __syncthreads();
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

static void gemm_grid(ly::GemmArgs& A, int64_t t_rows, int32_t f_rows, int32_t k) {
  A.t_rows = t_rows;
  A.f_rows = f_rows;
  A.k = k;
  const int64_t tiles = (t_rows + ly::kT - 1) / ly::kT;
  A.nt = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
  A.nf = (f_rows + ly::kF - 1) / ly::kF;
}

hipError_t launch_qkv_proj(const Geom& g, int32_t width, const void* x, const void* w_qkv,
                           const int32_t* coords, void* q, void* q_raw, void* k_loc,
                           void* v_loc, void* k_cmp, void* v_cmp, hipStream_t s) {
  ly::GemmArgs A = {};
  A.w = (const bf16_t*)w_qkv;
  A.x = (const bf16_t*)x;
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
