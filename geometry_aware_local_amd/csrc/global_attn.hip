// Query -> all-summaries attention with the gate fused into the epilogue.
//
// "Geometry Matters in Packed 3D Attention", papernotes.org notes, key
// design 3: every query attends to all M block summaries; the softmax is
// streamed (online) so no N x M score matrix exists, and only the M summary
// vectors are materialised.  The gate (flowchart node F) mixes the result
// with the local branch per token.
//
// Design (gfx950): one workgroup = 8 waves = one KV group and 512 (bf16) query
// rows, where a query row is a (token, head) pair of that group, so the G
// heads sharing the group's summaries are stacked as MFMA columns and every
// summary tile staged in LDS feeds all of them.  Summary tiles of 64 keys are
// double-buffered in LDS (K row-major swizzled, V transposed); each wave
// computes S^T = K Q^T and O^T += V^T P^T with 32x32 MFMA tiles (see
// pack3d_device.h) and keeps its softmax state in registers.  Workgroups are
// ordered so that all the workgroups an XCD receives read the same KV group,
// keeping one group's summaries resident in that XCD's L2.
#include "pack3d_device.h"

namespace pack3d {

constexpr int kGWaves = 8;
constexpr int kGKt = 64;           // keys per LDS tile
constexpr int kGVld = kGKt + 4;    // V^T row pitch (elements)

template <typename T> struct GCfg { static constexpr int kCb = 2; };   // column blocks / wave
template <> struct GCfg<float> { static constexpr int kCb = 1; };

template <typename T>
struct GArgs {
  const T* q;
  const T* ks;
  const T* vs;
  int64_t m;
  int64_t n;
  int32_t hq, hkv, grp;
  float c;                 // softmax scale * log2(e)
  float* o_cmp;
  float* lse;
  const float* o_loc;
  const float* gate;
  T* out;
  int32_t gate_per_head;
  int64_t tiles;           // query tiles per KV group
  int32_t xcd_per;         // consecutive XCDs sharing a group (0: plain order)
};

template <typename T>
struct GStage {
  static constexpr int kE = 16 / sizeof(T);               // elements per 16-byte chunk
  static constexpr int kChunks = kGKt * 64 / kE;           // chunks per tile
  static constexpr int kPer = kChunks / (kGWaves * 64);    // chunks per thread
  u32x4 k[kPer], v[kPer];
};

template <typename T>
__device__ __forceinline__ void g_load(GStage<T>& st, const T* ks, const T* vs, int64_t k0,
                                       int64_t m, int tid) {
#pragma unroll
  for (int c = 0; c < GStage<T>::kPer; ++c) {
    const int idx = tid + c * kGWaves * 64;
    const int row = idx / (64 / GStage<T>::kE), ch = idx % (64 / GStage<T>::kE);
    const int64_t key = k0 + row;
    if (key < m) {
      st.k[c] = ld16(ks + key * 64 + ch * GStage<T>::kE);
      st.v[c] = ld16(vs + key * 64 + ch * GStage<T>::kE);
    } else {
      st.k[c] = u32x4{0, 0, 0, 0};
      st.v[c] = u32x4{0, 0, 0, 0};
    }
  }
}

template <typename T>
__device__ __forceinline__ void g_store(const GStage<T>& st, T* kl, T* vl, int tid) {
#pragma unroll
  for (int c = 0; c < GStage<T>::kPer; ++c) {
    const int idx = tid + c * kGWaves * 64;
    const int row = idx / (64 / GStage<T>::kE), ch = idx % (64 / GStage<T>::kE);
    st16(kl + KLds<T>::chunk_off(row, ch), st.k[c]);
    const T* e = reinterpret_cast<const T*>(&st.v[c]);
#pragma unroll
    for (int i = 0; i < GStage<T>::kE; ++i) vl[(ch * GStage<T>::kE + i) * kGVld + row] = e[i];
  }
}

// A operand of PV step t for head dim `dim`, key block starting at kb0.
template <typename T>
__device__ __forceinline__ void v_frags(typename Mma<T>::frag* f, const T* vl, int dim, int kb0,
                                        int h) {
  const T* r = vl + dim * kGVld + kb0;
  if constexpr (std::is_same<T, float>::value) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(r + 8 * q + 4 * h);
#pragma unroll
      for (int j = 0; j < 4; ++j) f[4 * q + j] = x[j];
    }
  } else {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x4 lo = *reinterpret_cast<const bf16x4*>(r + 16 * t + 4 * h);
      const bf16x4 hi = *reinterpret_cast<const bf16x4*>(r + 16 * t + 8 + 4 * h);
      bf16x8 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) { x[j] = lo[j]; x[4 + j] = hi[j]; }
      f[t] = x;
    }
  }
}

template <typename T, bool kGate>
__global__ __launch_bounds__(64 * kGWaves) void k_global_attn(GArgs<T> A) {
  constexpr int CB = GCfg<T>::kCb;
  constexpr int ROWS = kGWaves * CB * 32;
  __shared__ __attribute__((aligned(16))) T k_lds[2][kGKt * 64];
  __shared__ __attribute__((aligned(16))) T v_lds[2][64 * kGVld];

  // workgroup -> (KV group, query tile), XCD-aware
  const int64_t bid = blockIdx.x;
  int grp;
  int64_t tile;
  if (A.xcd_per > 0) {
    const int x = (int)(bid % kNumXcd);
    grp = x / A.xcd_per;
    tile = (bid / kNumXcd) * A.xcd_per + x % A.xcd_per;
  } else {
    grp = (int)(bid % A.hkv);
    tile = bid / A.hkv;
  }
  if (tile >= A.tiles) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, col = lane & 31;
  const int64_t nrows = A.n * A.grp;
  const T* ksg = A.ks + (int64_t)grp * A.m * 64;
  const T* vsg = A.vs + (int64_t)grp * A.m * 64;

  // query fragments of this lane's columns
  QFrag<T> qf[CB];
  int64_t tok[CB];
  int head[CB];
  bool valid[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int64_t row = tile * ROWS + (int64_t)(wave * CB + cb) * 32 + col;
    valid[cb] = row < nrows;
    tok[cb] = valid[cb] ? row / A.grp : 0;
    head[cb] = grp * A.grp + (valid[cb] ? (int)(row % A.grp) : 0);
    load_qfrag<T>(qf[cb], A.q + (tok[cb] * A.hq + head[cb]) * 64 + h * 32, valid[cb]);
  }

  f32x16 o[CB][2];
  SoftmaxState sm[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    o[cb][0] = f32x16{};
    o[cb][1] = f32x16{};
    sm[cb].m = kNegInf;
    sm[cb].l = 0.0f;
  }

  const int64_t nt = (A.m + kGKt - 1) / kGKt;
  GStage<T> stage;
  g_load<T>(stage, ksg, vsg, 0, A.m, tid);
  for (int64_t t = 0; t < nt; ++t) {
    const int b = (int)(t & 1);
    g_store<T>(stage, k_lds[b], v_lds[b], tid);
    __syncthreads();
    if (t + 1 < nt) g_load<T>(stage, ksg, vsg, (t + 1) * kGKt, A.m, tid);

    const T* kl = k_lds[b];
    const T* vl = v_lds[b];
    const int64_t k0 = t * kGKt;

    f32x16 s[2][CB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      KFrag<T> kf;
      load_kfrag<T>(kf, kl, kb * 32 + col, h);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) s[kb][cb] = qk_tile<T>(kf, qf[cb]);
    }
    if (k0 + kGKt > A.m) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t key = k0 + kb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
          if (key >= A.m)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) s[kb][cb][v] = kNegInf;
        }
    }

    typename Mma<T>::frag pf[2][CB][Mma<T>::kPvSteps];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][cb][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mt = mx * A.c;
      const bool upd = mt > sm[cb].m + kRescaleSlack;
      if (__any(upd)) {
        const float mn = upd ? mt : sm[cb].m;
        const float alpha = upd ? __builtin_amdgcn_exp2f(sm[cb].m - mn) : 1.0f;
        sm[cb].m = mn;
        sm[cb].l *= alpha;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          o[cb][0][v] *= alpha;
          o[cb][1][v] *= alpha;
        }
      }
      const float mu = sm[cb].m == kNegInf ? 0.0f : sm[cb].m;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][cb][v], A.c, -mu));
          s[kb][cb][v] = p;
          sm[cb].l += p;
        }
#pragma unroll
        for (int st = 0; st < Mma<T>::kPvSteps; ++st) pf[kb][cb][st] = Mma<T>::p_frag(s[kb][cb], st);
      }
    }

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        typename Mma<T>::frag vf[Mma<T>::kPvSteps];
        v_frags<T>(vf, vl, db * 32 + col, kb * 32, h);
#pragma unroll
        for (int st = 0; st < Mma<T>::kPvSteps; ++st)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) o[cb][db] = Mma<T>::mma(vf[st], pf[kb][cb][st], o[cb][db]);
      }
  }

  // epilogue: normalise, write o_cmp or the gated output
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const float l = sm[cb].l + __shfl_xor(sm[cb].l, 32);
    if (!valid[cb]) continue;
    const float inv = 1.0f / l;
    const int64_t rbase = (tok[cb] * A.hq + head[cb]) * 64;
    if (A.lse && h == 0) A.lse[tok[cb] * A.hq + head[cb]] = (sm[cb].m + __log2f(l)) * kLn2;
    float g0 = 0.0f, g1 = 0.0f;
    if constexpr (kGate) {
      const float* gl = A.gate + (A.gate_per_head ? (tok[cb] * A.hq + head[cb]) * 2 : tok[cb] * 2);
      const float l0 = gl[0], l1 = gl[1];
      const float mx = fmaxf(l0, l1);
      const float e0 = expf(l0 - mx), e1 = expf(l1 - mx);
      g0 = e0 / (e0 + e1);
      g1 = e1 / (e0 + e1);
    }
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * h;
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = o[cb][db][4 * q4 + j] * inv;
        if constexpr (kGate) {
          const f32x4 ol = *reinterpret_cast<const f32x4*>(A.o_loc + rbase + d0);
          if constexpr (std::is_same<T, float>::value) {
            f32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = g0 * ol[j] + g1 * r[j];
            *reinterpret_cast<f32x4*>(A.out + rbase + d0) = w;
          } else {
            bf16x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = (bf16_t)(g0 * ol[j] + g1 * r[j]);
            *reinterpret_cast<bf16x4*>(A.out + rbase + d0) = w;
          }
        } else {
          *reinterpret_cast<f32x4*>(A.o_cmp + rbase + d0) = r;
        }
      }
  }
}

template <typename T, bool kGate>
static hipError_t launch_g(const Geom& g, const void* q, const void* ks, const void* vs,
                           int64_t m, float* o_cmp, float* lse, const float* o_loc,
                           const float* gate, void* out, hipStream_t s) {
  constexpr int ROWS = kGWaves * GCfg<T>::kCb * 32;
  GArgs<T> A;
  A.q = (const T*)q;
  A.ks = (const T*)ks;
  A.vs = (const T*)vs;
  A.m = m;
  A.n = g.N;
  A.hq = g.Hq;
  A.hkv = g.Hkv;
  A.grp = g.G;
  A.c = g.scale * kLog2e;
  A.o_cmp = o_cmp;
  A.lse = lse;
  A.o_loc = o_loc;
  A.gate = gate;
  A.out = (T*)out;
  A.gate_per_head = g.gate_per_head;
  A.tiles = (g.N * g.G + ROWS - 1) / ROWS;
  int64_t blocks;
  if (g.Hkv <= kNumXcd && kNumXcd % g.Hkv == 0) {
    A.xcd_per = kNumXcd / g.Hkv;
    blocks = (A.tiles + A.xcd_per - 1) / A.xcd_per * kNumXcd;
  } else {
    A.xcd_per = 0;
    blocks = A.tiles * g.Hkv;
  }
  hipLaunchKernelGGL((k_global_attn<T, kGate>), dim3((unsigned)blocks), dim3(64 * kGWaves), 0, s,
                     A);
  return hipGetLastError();
}

hipError_t launch_global_attn(const Geom& g, const void* q_rot, const void* k_sum,
                              const void* v_sum, int64_t m, float* o_cmp, float* lse,
                              const float* o_loc, const float* gate, void* out,
                              hipStream_t s) {
  const bool gated = o_cmp == nullptr;
  if (g.bf16)
    return gated ? launch_g<bf16_t, true>(g, q_rot, k_sum, v_sum, m, o_cmp, lse, o_loc, gate, out, s)
                 : launch_g<bf16_t, false>(g, q_rot, k_sum, v_sum, m, o_cmp, lse, o_loc, gate, out, s);
  return gated ? launch_g<float, true>(g, q_rot, k_sum, v_sum, m, o_cmp, lse, o_loc, gate, out, s)
               : launch_g<float, false>(g, q_rot, k_sum, v_sum, m, o_cmp, lse, o_loc, gate, out, s);
}

}  // namespace pack3d
