// Device-side helpers shared by the libpack3d kernels: element types, vector
// loads, the rotary sine/cosine, and the gfx950 MFMA tile primitives used by
// both attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pack3d_internal.h"

namespace pack3d {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return (float)v; }
template <typename T>
__device__ __forceinline__ T from_f32(float v) { return (T)v; }

// 16-byte vector load/store through plain (vector-memory) instructions.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---------------------------------------------------------------------------
// Rotary sine and cosine of 2*pi*nu*c.
//
// The angle is reduced in double to the nearest quarter turn, so the float
// argument is |x| <= pi/4 whatever the coordinate; sin and cos of x are then
// the Taylor series to x^9 and x^10 (truncation below 2e-9 on |x| <= pi/4),
// and the quarter-turn index k selects and signs the pair.  Depends only on
// (nu, c), so every kernel rotates a given cell identically.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rope_sincos(double nu, double c, float& sn, float& cs) {
  const double t = nu * c;                              // turns
  const double q = rint(4.0 * t);                       // quarter turns
  const float x = (float)((t - 0.25 * q) * 6.283185307179586);
  const int k = ((int)q) & 3;
  const float x2 = x * x;
  const float s = x + x * x2 * (-1.0f / 6.0f + x2 * (1.0f / 120.0f +
                  x2 * (-1.0f / 5040.0f + x2 * (1.0f / 362880.0f))));
  const float c0 = 1.0f + x2 * (-0.5f + x2 * (1.0f / 24.0f + x2 * (-1.0f / 720.0f +
                   x2 * (1.0f / 40320.0f + x2 * (-1.0f / 3628800.0f)))));
  // sin(x + k pi/2), cos(x + k pi/2)
  const float a = (k & 1) ? c0 : s;
  const float b = (k & 1) ? s : c0;
  sn = (k & 2) ? -a : a;
  cs = ((k + 1) & 2) ? -b : b;
}

// Rotate 4 consecutive pairs (dims 8*chunk .. 8*chunk+7) held as floats.
// The fused multiply-adds are written out, so every kernel that rotates a
// row (whatever the compiler would contract) produces the same bits.
__device__ __forceinline__ void rotate8(float* v, const float* sn, const float* cs) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = v[2 * i], x1 = v[2 * i + 1];
    v[2 * i] = fmaf(cs[i], x0, -(sn[i] * x1));
    v[2 * i + 1] = fmaf(sn[i], x0, cs[i] * x1);
  }
}

// cos/sin for the 4 pairs of dim-chunk `chunk` (8 dims) at point (z, y, x):
// a lattice cell, or a block centre (half-integers are exact in double).
__device__ __forceinline__ void chunk_sincos(const RopeTab& rt, int chunk, double z, double y,
                                             double x, float* sn, float* cs) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = chunk * 4 + i;
    if (p < rt.npairs) {
      const int ax = rt.axis[p];
      const double c = ax == 0 ? z : (ax == 1 ? y : x);
      rope_sincos(rt.nu[p], c, sn[i], cs[i]);
    } else {
      sn[i] = 0.0f;
      cs[i] = 1.0f;
    }
  }
}

// The rotation a key summary carries for the token at cell (z, y, x) of
// block (jz, jy, jx): R(c_u) for the exact form, R(c^_j) at the block's
// geometric centre for the summary-centre variant, none when blind.
__device__ __forceinline__ void summary_sincos(const Geom& g, int chunk, int z, int y, int x,
                                               float* sn, float* cs) {
  if (g.summary_mode == PACK3D_SUMMARY_TOKEN) {
    chunk_sincos(g.rope, chunk, z, y, x, sn, cs);
  } else if (g.summary_mode == PACK3D_SUMMARY_CENTRE) {
    chunk_sincos(g.rope, chunk, (z / g.bz) * g.bz + 0.5 * (g.bz - 1),
                 (y / g.by) * g.by + 0.5 * (g.by - 1), (x / g.bx) * g.bx + 0.5 * (g.bx - 1), sn,
                 cs);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sn[i] = 0.0f;
      cs[i] = 1.0f;
    }
  }
}

// The tokenwise gate (notes, flowchart node F): a 2-way softmax over the
// logits of token tok (or of token tok and head `head` when per_head), index
// 0 the local branch, 1 the compressed one.  Every kernel that applies the
// gate goes through this function, so g_loc and g_cmp have the same bits
// wherever they are computed.
__device__ __forceinline__ void gate_weights(const float* gate, int64_t tok, int head, int hq,
                                             int per_head, float& g0, float& g1) {
  const float* gl = gate + (per_head ? (tok * hq + head) * 2 : tok * 2);
  const float l0 = gl[0], l1 = gl[1];
  const float mx = fmaxf(l0, l1);
  const float e0 = expf(l0 - mx), e1 = expf(l1 - mx);
  g0 = e0 / (e0 + e1);
  g1 = e1 / (e0 + e1);
}

// The local branch's share of the output: out[row, d0 .. d0+3] = g * r,
// rounded to the output dtype (the compressed branch's epilogue adds its
// share to it with add_gated4).
template <typename T>
__device__ __forceinline__ void store_gated4(T* out, const f32x4& r, float g0) {
  if constexpr (std::is_same<T, float>::value) {
    f32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = g0 * r[j];
    *reinterpret_cast<f32x4*>(out) = w;
  } else {
    bf16x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (bf16_t)(g0 * r[j]);
    *reinterpret_cast<bf16x4*>(out) = w;
  }
}

// out[row, d0 .. d0+3] += g * r, rounded once to the output dtype.
template <typename T>
__device__ __forceinline__ void add_gated4(T* out, const f32x4& r, float g) {
  if constexpr (std::is_same<T, float>::value) {
    f32x4 w = *reinterpret_cast<const f32x4*>(out);
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = w[j] + g * r[j];
    *reinterpret_cast<f32x4*>(out) = w;
  } else {
    bf16x4 w = *reinterpret_cast<const bf16x4*>(out);
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (bf16_t)((float)w[j] + g * r[j]);
    *reinterpret_cast<bf16x4*>(out) = w;
  }
}

// Load / store 8 consecutive elements as floats.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v) {
  if constexpr (std::is_same<T, float>::value) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  } else {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float* v) {
  if constexpr (std::is_same<T, float>::value) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
    *reinterpret_cast<f32x4*>(p) = a;
    *reinterpret_cast<f32x4*>(p + 4) = b;
  } else {
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (bf16_t)v[i];
    *reinterpret_cast<bf16x8*>(p) = a;
  }
}

// ---------------------------------------------------------------------------
// MFMA tile primitives (gfx950, wave64).
//
// Both attention kernels compute S^T = K Q^T and O^T = V^T P^T with 32x32
// output tiles: keys (or head dims) are MFMA rows, query rows are MFMA
// columns.  Accumulator element v (0..15) of lane l holds row
// 8*(v/4) + 4*(l/32) + (v%4) of column l%32.
//
// QK^T contraction over the 64 head dims: lane half h = l/32 supplies dims
// h*32 .. h*32+31 of its key row (A) and of its query row (B), in the same
// order, so any internal k ordering of the instruction is immaterial.
//   bf16: 4 x v_mfma_f32_32x32x16_bf16, step s takes dims h*32 + 8s .. +7
//   fp32: 32 x v_mfma_f32_32x32x2_f32,  step s takes dim  h*32 + s
// PV contraction over 32 keys: the B operand is the lane's own accumulator
// (the P^T column), so the A operand (V^T) must hold, for element e of step
// t, the value of key kr(t, e, h) below.
//   bf16: 2 steps x 8 elements;  fp32: 16 steps x 1 element.
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<bf16_t> {
  static constexpr int kQkSteps = 4;
  static constexpr int kPvSteps = 2;
  static constexpr int kPerStep = 8;
  typedef bf16x8 frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // key row (within the 32-key block) of PV step t, element e, lane half h
  __device__ static __forceinline__ int kr(int t, int e, int h) {
    return 16 * t + 8 * (e >> 2) + 4 * h + (e & 3);
  }
  // B operand of PV step t from the accumulator (P^T column)
  __device__ static __forceinline__ frag p_frag(const f32x16& p, int t) {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16_t)p[8 * t + e];
    return f;
  }
};

template <> struct Mma<float> {
  static constexpr int kQkSteps = 32;
  static constexpr int kPvSteps = 16;
  static constexpr int kPerStep = 1;
  typedef float frag;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ int kr(int t, int e, int h) {
    (void)e;
    return 8 * (t >> 2) + 4 * h + (t & 3);
  }
  __device__ static __forceinline__ frag p_frag(const f32x16& p, int t) { return p[t]; }
};

// Query fragment: the lane's 32 dims (h*32 ..) of one query row, as the MFMA
// B operand of every QK^T step.
template <typename T>
struct QFrag {
  typename Mma<T>::frag f[Mma<T>::kQkSteps];
};

template <typename T>
__device__ __forceinline__ void load_qfrag(QFrag<T>& q, const T* row_h /* row + h*32 */,
                                           bool valid) {
  if constexpr (std::is_same<T, float>::value) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f32x4 v = valid ? *reinterpret_cast<const f32x4*>(row_h + 4 * i) : f32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) q.f[4 * i + j] = v[j];
    }
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 v;
      if (valid) {
        v = *reinterpret_cast<const bf16x8*>(row_h + 8 * s);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16_t)0.0f;
      }
      q.f[s] = v;
    }
  }
}

// The query fragment rotated by R(z, y, x) (notes, key design 1) and rounded
// to its dtype.  The lane's dims h*32 .. h*32+31 are rotary pairs 16h .. 16h+15;
// each pair's (sin, cos) at its axis' coordinate comes from the lattice's
// rotary table (k_rope's values), and rotate8 is k_rope's arithmetic, so the
// bits equal the rows k_rope writes.  (z, y, x) must lie in the lattice.
// qrope_load and qrope_apply split the table reads from the arithmetic, so a
// kernel can issue the reads early.
struct QRopeCS {
  float sn[16], cs[16];
};
// The axes of the lane's 16 pairs (2 bits each).  The two words are read as
// scalars, so selecting one is a register select, not a per-lane load from
// the kernel arguments (whose wait would also wait for every copy in flight).
__device__ __forceinline__ uint32_t qrope_lane_axes(const QRope& r, int h) {
  const uint32_t a0 = __builtin_amdgcn_readfirstlane(r.axes[0]);
  const uint32_t a1 = __builtin_amdgcn_readfirstlane(r.axes[1]);
  return h ? a1 : a0;
}
__device__ __forceinline__ void qrope_load(QRopeCS& t, const QRope& r, uint32_t ab, int h, int z,
                                           int y, int x) {
  const float* tab = r.tab + (size_t)(16 * h) * r.ts * 2;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t ax = (ab >> (2 * k)) & 3u;
    const int c = ax == 0 ? z : (ax == 1 ? y : x);
    const float* e = tab + ((size_t)k * r.ts + c) * 2;
    t.sn[k] = e[0];
    t.cs[k] = e[1];
  }
}
template <typename T>
__device__ __forceinline__ void qrope_apply(QFrag<T>& q, const QRopeCS& t) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float v[8];
    if constexpr (std::is_same<T, float>::value) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = q.f[8 * s + e];
      rotate8(v, t.sn + 4 * s, t.cs + 4 * s);
#pragma unroll
      for (int e = 0; e < 8; ++e) q.f[8 * s + e] = v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (float)q.f[s][e];
      rotate8(v, t.sn + 4 * s, t.cs + 4 * s);
#pragma unroll
      for (int e = 0; e < 8; ++e) q.f[s][e] = (bf16_t)v[e];
    }
  }
}
template <typename T>
__device__ __forceinline__ void rotate_qfrag(QFrag<T>& q, const QRope& r, int h, int z, int y,
                                             int x) {
  QRopeCS t;
  qrope_load(t, r, qrope_lane_axes(r, h), h, z, y, x);
  qrope_apply<T>(q, t);
}

// ---------------------------------------------------------------------------
// LDS tile layouts.
//
// K rows: [rows][64] elements with the 16-byte chunks of each row XOR-
// swizzled so that the rows read by one MFMA operand spread over all banks.
// gfx950 LDS has 64 four-byte banks (256 bytes) and serves a 128-bit read 16
// lanes at a time: a bf16 row is 128 bytes, so rows r and r+1 sit in
// different bank halves and the 8 rows of one parity among 16 consecutive
// rows need distinct chunk positions: the swizzle is a bijection of
// (r >> 1) & 7.  The same bf16 tiles are also read transposed (the 8-byte
// transposing read, 32 lanes at a time: rows 4i .. 4i+3, the same 4 aligned
// chunks of each); rows 4i and 4i+2 then need chunk positions in different
// 4-chunk halves, so bit 2 of the swizzle follows bit 1 of r:
// sw(r) = 4 * ((r >> 1) & 1) + ((r >> 2) & 3).  An fp32 row is 256 bytes and
// 16 consecutive rows need distinct positions (r & 15).
// V^T: [64 dims][ld] elements, ld = key capacity + 4, so consecutive dims
// start on different banks.
// ---------------------------------------------------------------------------
template <typename T>
struct KLds {
  static constexpr int kChunkElems = 16 / sizeof(T);       // elements per 16 B
  static constexpr int kChunks = 64 / kChunkElems;          // chunks per row
  __device__ static __forceinline__ int chunk_off(int row, int chunk) {
    const int sw = sizeof(T) == 2 ? (((row >> 1) & 1) << 2) | ((row >> 2) & 3) : row & 15;
    return row * 64 + ((chunk ^ sw) * kChunkElems);
  }
};

// A operand of QK^T step s for key row `row` (lane half h).
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag k_frag(const T* ks, int row, int h, int s) {
  if constexpr (std::is_same<T, float>::value) {
    const int dim = h * 32 + s;
    return ks[KLds<T>::chunk_off(row, dim >> 2) + (dim & 3)];
  } else {
    const int chunk = h * 4 + s;
    return *reinterpret_cast<const bf16x8*>(ks + KLds<T>::chunk_off(row, chunk));
  }
}

// Full K fragment set for one key row: all QK^T steps (fp32 reads 8 chunks).
template <typename T>
struct KFrag {
  typename Mma<T>::frag f[Mma<T>::kQkSteps];
};

template <typename T>
__device__ __forceinline__ void load_kfrag(KFrag<T>& k, const T* ks, int row, int h) {
  if constexpr (std::is_same<T, float>::value) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(ks + KLds<T>::chunk_off(row, h * 8 + i));
#pragma unroll
      for (int j = 0; j < 4; ++j) k.f[4 * i + j] = v[j];
    }
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) k.f[s] = k_frag<T>(ks, row, h, s);
  }
}

template <typename T>
__device__ __forceinline__ f32x16 qk_tile(const KFrag<T>& k, const QFrag<T>& q) {
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < Mma<T>::kQkSteps; ++s) acc = Mma<T>::mma(k.f[s], q.f[s], acc);
  return acc;
}

// Lanes l and l+32 hold the same MFMA column: combine their values.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum of the 8 probabilities of a bf16 PV operand (as rounded for the MFMA).
__device__ __forceinline__ float frag_sum(const bf16x8& f, float acc) {
  const bf16x2 one = {(bf16_t)1.0f, (bf16_t)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {f[2 * i], f[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float frag_sum(float f, float acc) { return acc + f; }

// Online-softmax state of one query column (per lane; lanes l and l+32 hold
// the same column and always agree on m).
struct SoftmaxState {
  float m;   // running reference max, in scaled log2 units
  float l;   // this lane's partial sum of exponentials
};

// Lazy rescaling: the reference max only moves when a tile's max exceeds it
// by more than kRescaleSlack (log2 units), so exponentials stay below
// 2^kRescaleSlack.  The decision is per column; skipping the O update when no
// column moves changes no value (the factor would be exactly 1).
constexpr float kRescaleSlack = 8.0f;

// Softmax references of the query->summary kernels.  Given the largest
// summary norm kmax of a group, every logit of query q lies within
// +-|q| kmax (Cauchy-Schwarz); a column whose bound B (with a margin for the
// bf16 rounding of q and k~ and the fp32 sums) is at most kSafeBound uses the
// fixed reference max(0, B - kRefHeadroom), so its exponentials stay in
// [2^-96, 2^64]; other columns track a lazily updated running max.
constexpr float kRefHeadroom = 64.0f;
constexpr float kSafeBound = 80.0f;
constexpr float kBoundMargin = 1.015625f;
enum GMode : int { kGeneral = 0, kFixedRef = 1, kZeroRef = 2 };

}  // namespace pack3d
