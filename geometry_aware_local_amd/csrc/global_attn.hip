// Query -> all-summaries attention with the gate fused into the epilogue.
//
// "Geometry Matters in Packed 3D Attention", papernotes.org notes, key
// design 3: every query attends to all M block summaries; the softmax is
// streamed (online) so no N x M score matrix exists, and only the M summary
// vectors are materialised.  The gate (flowchart node F) mixes the result
// with the local branch per token: the local branch's kernel has already
// written its gated share g_loc * o_loc into the output, and this kernel's
// epilogue adds g_cmp * o_cmp to it.
//
// In the forward the kernel takes the unrotated queries and rotates each
// query fragment by R(c) (key design 1) once, in registers, through the
// lattice's rotary table, so no rotated copy of Q is ever stored.
//
// Design (gfx950):
// * One workgroup = 8 waves = one KV group and 512 (bf16) query rows, a query
//   row being a (token, head) pair of that group: the G heads sharing the
//   group's summaries are stacked as MFMA columns, so every summary tile
//   staged in LDS feeds all of them.
// * Summary tiles of 64 keys live in LDS as plain row-major copies (16-byte
//   chunks XOR-swizzled against bank conflicts).  bf16: phases of 4 tiles,
//   copied global -> LDS asynchronously one phase ahead, one barrier per
//   phase; fp32: register-staged double buffering.  Each wave
//   computes S^T = K Q^T and O^T += V^T P^T with 32x32 MFMA tiles (see
//   pack3d_device.h); the V^T operand comes straight from the row-major tile
//   through the gfx950 transposing LDS read (ds_read_b64_tr_b16).
// * Softmax reference.  The kernel is bound by the VALU work per logit, so
//   the running max is avoided where a bound allows: given the largest
//   summary norm of the group (kmax), every logit of query q lies within
//   +-|q| kmax (Cauchy-Schwarz).  A query whose bound B is small uses the
//   fixed reference max(0, B - 64) for the whole stream (its exponentials
//   stay in [2^-96, 2^64]); only queries with a large bound track a lazily
//   updated running max.  The choice is per query, so results do not depend
//   on which queries share a wave (packing equivariance stays bitwise).
// * Workgroups are ordered so that all the workgroups an XCD receives read
//   the same KV group, keeping one group's summaries resident in its L2.
#include "pack3d_device.h"
#include "local_tiles.h"

namespace pack3d {

constexpr int kGWaves = 8;
constexpr int kGKt = 64;           // keys per LDS tile
constexpr int kGVld = kGKt + 4;    // fp32 V^T row pitch (elements)

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
  float c;                 // multiplier of q.k~ giving log2-domain logits
  float* o_cmp;
  float* lse;
  const float* gate;
  T* out;                  // gated: holds g_loc * o_loc on entry
  const float* kmax;       // [Hkv] max_j c |k~_j| (NULL: always track the max)
  const int32_t* coords;   // [N, 3], with qrope.tab: q is unrotated
  QRope qrope;
  int32_t gate_per_head;
  int64_t tiles;           // query tiles per KV group
  int32_t xcd_per;         // consecutive XCDs sharing a group (0: plain order)
};

// ---------------------------------------------------------------------------
// LDS tiles.  bf16: K and V both row-major [64 keys][64 dims], chunk c of key
// row r stored at chunk c ^ sw(r) (K, see KLds) or c ^ (2r & 6) (V:
// the transposing read takes 4 consecutive keys x 16 dims per 16 lanes).
// fp32: K as above, V transposed [64 dims][kGVld].
// ---------------------------------------------------------------------------
template <typename T>
struct GLds {
  static constexpr bool kF32 = std::is_same<T, float>::value;
  static constexpr int kVElems = kF32 ? 64 * kGVld : kGKt * 64;
};

__device__ __forceinline__ int v_swz(int row, int chunk) { return chunk ^ ((2 * row) & 6); }

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
    if constexpr (GLds<T>::kF32) {
      const T* e = reinterpret_cast<const T*>(&st.v[c]);
#pragma unroll
      for (int i = 0; i < GStage<T>::kE; ++i) vl[(ch * GStage<T>::kE + i) * kGVld + row] = e[i];
    } else {
      st16(vl + row * 64 + v_swz(row, ch) * 8, st.v[c]);
    }
  }
}

// A operand (V^T) of PV step t for head dim `dim` = db*32 + lane%32, key block
// kb0 .. kb0+31.
template <typename T>
__device__ __forceinline__ void v_frags(typename Mma<T>::frag* f, const T* vl, int db, int kb0,
                                        int lane) {
  const int h = lane >> 5;
  if constexpr (GLds<T>::kF32) {
    const T* r = vl + (db * 32 + (lane & 31)) * kGVld + kb0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(r + 8 * q + 4 * h);
#pragma unroll
      for (int j = 0; j < 4; ++j) f[4 * q + j] = x[j];
    }
  } else {
    // ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element
    // (i % 4) of the 8-byte chunks addressed by lanes i/4, i/4+4, i/4+8,
    // i/4+12.  Lane r addresses key K0 + r/4, dims base + 4*(r%4) .. +3, so
    // lane i receives dim base + i of keys K0 .. K0+3.
    const int r = lane & 15;
    const int dim = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (r & 3);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x4 part[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int key = kb0 + 16 * t + 8 * half + 4 * h + (r >> 2);
        const T* p = vl + key * 64 + v_swz(key, dim >> 3) * 8 + (dim & 7);
        part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(
                (__attribute__((address_space(3))) char*)p));
      }
      bf16x8 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = part[0][j];
        x[4 + j] = part[1][j];
      }
      f[t] = x;
    }
  }
}

// Per-column softmax state.
struct GCol {
  float m;       // reference (log2 units)
  float l;       // fp32: this lane's partial sum
  f32x4 lm;      // bf16: the column's sum, accumulated on the matrix cores
  bool track;    // true: lazily tracked running max; false: fixed reference
};

// bf16 row sums on the matrix cores.  The P fragment of a PV step (lane l
// holds P[col = l % 32][keys 8(l/32) .. +7] of 16 keys) taken as the B
// operand of a 16x16x32 MFMA is B[k = 8(l/16) + e][n = l % 16] =
// P[16((l/16) % 2) + n][8((l/16)/2) + e]; with A[m][8g + e] = 1 exactly when
// g % 2 == (m/4) % 2, D[m][n] sums the 16 keys of column 16((m/4) % 2) + n,
// and lane l's accumulator rows m = 4(l/16) .. +3 are its own column's sum.
// The sum thus costs one small MFMA per 16 keys instead of four v_dot2 per
// lane, which on this part do not overlap the other wave's MFMAs.
__device__ __forceinline__ bf16x8 rowsum_ones(int lane) {
  const int g = lane >> 4, m = lane & 15;
  const bf16_t v = ((g & 1) == ((m >> 2) & 1)) ? (bf16_t)1.0f : (bf16_t)0.0f;
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = v;
  return a;
}

// One 64-key tile for all of the wave's column blocks.
template <typename T, int CB, int MODE, bool kFull = false>
__device__ __forceinline__ void g_tile(const T* __restrict__ kl, const T* __restrict__ vl,
                                       int k0, int m,
                                       float c, const QFrag<T> (&qf)[CB], GCol (&st)[CB],
                                       f32x16 (&o)[CB][2], int lane, const bf16x8& ones) {
  const int h = lane >> 5, col = lane & 31;
  if constexpr (MODE != kGeneral) {
    // no tile maximum needed: each 32-key half runs logits -> exponentials
    // -> PV on its own (half the live logits and probabilities)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sk[CB];
      {
        KFrag<T> kf;
        load_kfrag<T>(kf, kl, kb * 32 + col, h);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) sk[cb] = qk_tile<T>(kf, qf[cb]);
      }
      if (!kFull && k0 + kGKt > m) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + kb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
          if (key >= m)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) sk[cb][v] = kNegInf;
        }
      }
      typename Mma<T>::frag pk[CB][Mma<T>::kPvSteps];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float mu = st[cb].m == kNegInf ? 0.0f : st[cb].m;
        f32x16 p;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if constexpr (MODE == kZeroRef)
            p[v] = __builtin_amdgcn_exp2f(sk[cb][v]);
          else
            p[v] = __builtin_amdgcn_exp2f(fmaf(sk[cb][v], c, -mu));
        }
#pragma unroll
        for (int t = 0; t < Mma<T>::kPvSteps; ++t) {
          pk[cb][t] = Mma<T>::p_frag(p, t);
          if constexpr (GLds<T>::kF32)
            st[cb].l = frag_sum(pk[cb][t], st[cb].l);
          else
            st[cb].lm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pk[cb][t], st[cb].lm,
                                                                0, 0, 0);
        }
      }
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        typename Mma<T>::frag vf[Mma<T>::kPvSteps];
        v_frags<T>(vf, vl, db, kb * 32, lane);
#pragma unroll
        for (int t = 0; t < Mma<T>::kPvSteps; ++t)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) o[cb][db] = Mma<T>::mma(vf[t], pk[cb][t], o[cb][db]);
      }
    }
    return;
  }
  f32x16 s[2][CB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    KFrag<T> kf;
    load_kfrag<T>(kf, kl, kb * 32 + col, h);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) s[kb][cb] = qk_tile<T>(kf, qf[cb]);
  }
  if (!kFull && k0 + kGKt > m) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = k0 + kb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (key >= m)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) s[kb][cb][v] = kNegInf;
      }
  }

  typename Mma<T>::frag pf[2][CB][Mma<T>::kPvSteps];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if constexpr (MODE == kGeneral) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][cb][v]);
      const float mt = pair_max(mx) * c;
      const bool upd = st[cb].track && mt > st[cb].m + kRescaleSlack;
      if (__any(upd)) {
        const float mn = upd ? mt : st[cb].m;
        const float alpha = upd ? __builtin_amdgcn_exp2f(st[cb].m - mn) : 1.0f;
        st[cb].m = mn;
        st[cb].l *= alpha;
        st[cb].lm *= alpha;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          o[cb][0][v] *= alpha;
          o[cb][1][v] *= alpha;
        }
      }
    }
    const float mu = st[cb].m == kNegInf ? 0.0f : st[cb].m;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 p;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if constexpr (MODE == kZeroRef)
          p[v] = __builtin_amdgcn_exp2f(s[kb][cb][v]);
        else
          p[v] = __builtin_amdgcn_exp2f(fmaf(s[kb][cb][v], c, -mu));
      }
#pragma unroll
      for (int t = 0; t < Mma<T>::kPvSteps; ++t) {
        pf[kb][cb][t] = Mma<T>::p_frag(p, t);
        if constexpr (GLds<T>::kF32)
          st[cb].l = frag_sum(pf[kb][cb][t], st[cb].l);
        else
          st[cb].lm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[kb][cb][t], st[cb].lm,
                                                              0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      typename Mma<T>::frag vf[Mma<T>::kPvSteps];
      v_frags<T>(vf, vl, db, kb * 32, lane);
#pragma unroll
      for (int t = 0; t < Mma<T>::kPvSteps; ++t)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) o[cb][db] = Mma<T>::mma(vf[t], pf[kb][cb][t], o[cb][db]);
    }
}

template <typename T, int CB, int MODE>
__device__ __forceinline__ void g_stream(T (&k_lds)[2][kGKt * 64],
                                         T (&v_lds)[2][GLds<T>::kVElems], GStage<T>& stage,
                                         const T* ksg, const T* vsg, const GArgs<T>& A,
                                         const QFrag<T> (&qf)[CB], GCol (&st)[CB],
                                         f32x16 (&o)[CB][2], int tid, int lane) {
  const int m = (int)A.m;
  const int nt = (m + kGKt - 1) / kGKt;
  for (int t = 0; t < nt; ++t) {
    const int b = (int)(t & 1);
    g_store<T>(stage, k_lds[b], v_lds[b], tid);
    __syncthreads();
    if (t + 1 < nt) g_load<T>(stage, ksg, vsg, (t + 1) * kGKt, A.m, tid);
    g_tile<T, CB, MODE>(k_lds[b], v_lds[b], t * kGKt, m, A.c, qf, st, o, lane, bf16x8{});
  }
}

// bf16 stream: phases of kPhR tiles.  The tiles of the next phase are copied
// global -> LDS asynchronously (one 1 KB copy of 8 key rows per wave and
// operand) while the waves work through the current phase with no barrier
// between its tiles; one barrier per phase publishes the copies and frees
// the previous phase's buffers.  Keys past M read the last summary (finite)
// and are masked to p = 0.  Two separate LDS arrays hold the two phases so
// the compiler can tell the copies in flight from the tiles being read.
constexpr int kPhR = 4;                      // tiles per phase
constexpr int kPhTile = 2 * kGKt * 64;       // K then V, elements

template <int I>
__device__ __forceinline__ bf16_t* ph_buf() {
  __shared__ __attribute__((aligned(16))) bf16_t buf[kPhR * kPhTile];
  return buf;
}

__device__ __forceinline__ void g_issue_ph(bf16_t* __restrict__ buf, int ph, const bf16_t* ksg,
                                           const bf16_t* vsg, int m, int nt, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int row = wave * 8 + (lane >> 3), pos = lane & 7;
  const int ksw = pos ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  const int vsw = pos ^ ((2 * row) & 6);
#pragma unroll
  for (int i = 0; i < kPhR; ++i) {
    const int t = ph * kPhR + i;
    if (t < nt) {
      const int key = t * kGKt + row;
      const int kc = key < m ? key : m - 1;
      bf16_t* dst = buf + i * kPhTile + wave * 512;
      const int64_t off = (int64_t)kc * 64;
      __builtin_amdgcn_global_load_lds((const void*)(ksg + off + ksw * 8), (lb::lds_ptr)dst, 16, 0,
                                       0);
      __builtin_amdgcn_global_load_lds((const void*)(vsg + off + vsw * 8),
                                       (lb::lds_ptr)(dst + kGKt * 64), 16, 0, 0);
    }
  }
}

template <int CB, int MODE>
__device__ __forceinline__ void g_stream_ph(const bf16_t* ksg, const bf16_t* vsg,
                                            const GArgs<bf16_t>& A,
                                            const QFrag<bf16_t> (&qf)[CB], GCol (&st)[CB],
                                            f32x16 (&o)[CB][2], int tid, int lane) {
  // tile and key indices in 32 bits (M < 2^31): their compares then run on
  // the scalar unit (gfx9 has no 64-bit scalar ordered compare)
  const int m = (int)A.m;
  const int nt = (m + kGKt - 1) / kGKt;
  const int nph = (nt + kPhR - 1) / kPhR;
  const bf16x8 ones = rowsum_ones(lane);
  // full tiles run without the key mask; a ragged last tile runs once after
  // the stream, from its phase's buffer (nothing overwrites it after the
  // last phase's barrier)
  const int ntf = m / kGKt;
  auto phase = [&](int ph, bf16_t* __restrict__ cur, bf16_t* __restrict__ nxt) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ph + 1 < nph) g_issue_ph(nxt, ph + 1, ksg, vsg, m, nt, tid);
#pragma unroll
    for (int i = 0; i < kPhR; ++i) {
      const int t = ph * kPhR + i;
      if (t < ntf)
        g_tile<bf16_t, CB, MODE, true>(cur + i * kPhTile, cur + i * kPhTile + kGKt * 64,
                                       t * kGKt, m, A.c, qf, st, o, lane, ones);
    }
  };
  for (int ph = 0; ph < nph; ph += 2) {
    phase(ph, ph_buf<0>(), ph_buf<1>());
    if (ph + 1 < nph) phase(ph + 1, ph_buf<1>(), ph_buf<0>());
  }
  if (ntf < nt) {
    const int t = nt - 1, i = t % kPhR;
    bf16_t* buf = ((t / kPhR) & 1) ? ph_buf<1>() : ph_buf<0>();
    g_tile<bf16_t, CB, MODE, false>(buf + i * kPhTile, buf + i * kPhTile + kGKt * 64, t * kGKt, m,
                                    A.c, qf, st, o, lane, ones);
  }
}

template <typename T, bool kGate>
__global__ __launch_bounds__(64 * kGWaves) void k_global_attn(GArgs<T> A) {
  constexpr int CB = GCfg<T>::kCb;
  constexpr int ROWS = kGWaves * CB * 32;
  constexpr bool kAsync = !GLds<T>::kF32;
  typedef T KTile[2][kGKt * 64];
  typedef T VTile[2][GLds<T>::kVElems];
  __shared__ __attribute__((aligned(16))) KTile k_lds_f32;
  __shared__ __attribute__((aligned(16))) VTile v_lds_f32;

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

  GStage<T> stage;
  if constexpr (kAsync)
    g_issue_ph(ph_buf<0>(), 0, ksg, vsg, (int)A.m, (int)((A.m + kGKt - 1) / kGKt), tid);
  else
    g_load<T>(stage, ksg, vsg, 0, A.m, tid);

  // query fragments of this lane's columns, and their softmax references
  QFrag<T> qf[CB];
  int64_t tok[CB];
  int head[CB];
  bool valid[CB];
  GCol st[CB];
  const float kmax = A.kmax ? A.kmax[grp] : 0.0f;
  bool all_fixed = true, all_zero = true;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int64_t row = tile * ROWS + (int64_t)(wave * CB + cb) * 32 + col;
    valid[cb] = row < nrows;
    tok[cb] = valid[cb] ? row / A.grp : 0;
    head[cb] = grp * A.grp + (valid[cb] ? (int)(row % A.grp) : 0);
    load_qfrag<T>(qf[cb], A.q + (tok[cb] * A.hq + head[cb]) * 64 + h * 32, valid[cb]);
    if (A.qrope.tab) {
      const int32_t* c3 = A.coords + 3 * tok[cb];
      rotate_qfrag<T>(qf[cb], A.qrope, h, c3[0], c3[1], c3[2]);
    }
    st[cb].l = 0.0f;
    st[cb].lm = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    st[cb].m = kNegInf;
    st[cb].track = true;
    if (A.kmax) {
      float q2 = 0.0f;
#pragma unroll
      for (int s = 0; s < Mma<T>::kQkSteps; ++s) {
        if constexpr (GLds<T>::kF32) {
          q2 = fmaf(qf[cb].f[s], qf[cb].f[s], q2);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) q2 = fmaf((float)qf[cb].f[s][e], (float)qf[cb].f[s][e], q2);
        }
      }
      const float bound = sqrtf(pair_sum(q2)) * kmax * kBoundMargin;
      if (bound <= kSafeBound) {
        st[cb].track = false;
        st[cb].m = fmaxf(bound - kRefHeadroom, 0.0f);
      }
    }
    all_fixed = all_fixed && !st[cb].track;
    all_zero = all_zero && !st[cb].track && st[cb].m == 0.0f;
  }

  f32x16 o[CB][2];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    o[cb][0] = f32x16{};
    o[cb][1] = f32x16{};
  }

  // one code path per wave; each query's arithmetic is the same in all of them
  if constexpr (kAsync) {
    if (A.kmax && __all(all_zero))
      g_stream_ph<CB, kZeroRef>(ksg, vsg, A, qf, st, o, tid, lane);
    else if (A.kmax && __all(all_fixed))
      g_stream_ph<CB, kFixedRef>(ksg, vsg, A, qf, st, o, tid, lane);
    else
      g_stream_ph<CB, kGeneral>(ksg, vsg, A, qf, st, o, tid, lane);
  } else {
    if (A.kmax && __all(all_zero))
      g_stream<T, CB, kZeroRef>(k_lds_f32, v_lds_f32, stage, ksg, vsg, A, qf, st, o, tid, lane);
    else if (A.kmax && __all(all_fixed))
      g_stream<T, CB, kFixedRef>(k_lds_f32, v_lds_f32, stage, ksg, vsg, A, qf, st, o, tid, lane);
    else
      g_stream<T, CB, kGeneral>(k_lds_f32, v_lds_f32, stage, ksg, vsg, A, qf, st, o, tid, lane);
  }

  // epilogue: normalise, write o_cmp or the gated output
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    // bf16: the matrix cores summed both lane halves already
    const float l = GLds<T>::kF32 ? pair_sum(st[cb].l) : st[cb].lm[0];
    if (!valid[cb]) continue;
    const float inv = 1.0f / l;
    const int64_t rbase = (tok[cb] * A.hq + head[cb]) * 64;
    if (A.lse && h == 0) A.lse[tok[cb] * A.hq + head[cb]] = (st[cb].m + __log2f(l)) * kLn2;
    float g0 = 0.0f, g1 = 0.0f;
    if constexpr (kGate) gate_weights(A.gate, tok[cb], head[cb], A.hq, A.gate_per_head, g0, g1);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * h;
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = o[cb][db][4 * q4 + j] * inv;
        if constexpr (kGate) {
          // the local branch's kernel wrote its gated share g_loc * o_loc
          // into the output; add this branch's share
          if (A.o_cmp) *reinterpret_cast<f32x4*>(A.o_cmp + rbase + d0) = r;
          add_gated4<T>(A.out + rbase + d0, r, g1);
        } else {
          *reinterpret_cast<f32x4*>(A.o_cmp + rbase + d0) = r;
        }
      }
  }
}

// kmax[g] = max_j part[g][j] over nparts per-block summary norms (blocks
// 0 .. Hkv-1).  The blocks after them fill the lattice's rotary table, one
// (pair, coordinate) entry per thread, with k_rope's sines and cosines.
__global__ __launch_bounds__(1024) void k_kmax(const float* __restrict__ part, int64_t nparts,
                                               int32_t groups, float* kmax, float* tab, int32_t ts,
                                               RopeTab rt) {
  if ((int)blockIdx.x >= groups) {
    const int e = ((int)blockIdx.x - groups) * 1024 + (int)threadIdx.x;
    if (e >= kMaxPairs * ts) return;
    const int p = e / ts, c = e % ts;
    float sn = 0.0f, cs = 1.0f;
    if (p < rt.npairs) rope_sincos(rt.nu[p], (double)c, sn, cs);
    tab[2 * e] = sn;
    tab[2 * e + 1] = cs;
    return;
  }
  __shared__ float red[1024];
  const float* p = part + (int64_t)blockIdx.x * nparts;
  float x = 0.0f;
  for (int64_t i = threadIdx.x; i < nparts; i += blockDim.x) x = fmaxf(x, p[i]);
  red[threadIdx.x] = x;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
    __syncthreads();
  }
  if (threadIdx.x == 0) kmax[blockIdx.x] = red[0];
}

hipError_t launch_kmax(const Geom& g, const float* knorm, float* kmax, float* tab, hipStream_t s) {
  const int ts = rope_table_stride(g);
  const int extra = tab ? (kMaxPairs * ts + 1023) / 1024 : 0;
  hipLaunchKernelGGL(k_kmax, dim3(g.Hkv + extra), dim3(1024), 0, s, knorm, (int64_t)g.M, g.Hkv,
                     kmax, tab, ts, g.rope);
  return hipGetLastError();
}

template <typename T, bool kGate>
static hipError_t launch_g(const Geom& g, const void* q, const void* ks, const void* vs,
                           int64_t m, float c, const float* kmax, float* o_cmp, float* lse,
                           const float* gate, void* out, const int32_t* coords,
                           const QRope& qr, hipStream_t s) {
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
  A.c = c;
  A.o_cmp = o_cmp;
  A.lse = lse;
  A.gate = gate;
  A.out = (T*)out;
  A.kmax = kmax;
  A.gate_per_head = g.gate_per_head;
  A.coords = coords;
  A.qrope = qr;
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

hipError_t launch_global_attn(const Geom& g, const void* q, const void* k_sum, const void* v_sum,
                              int64_t m, const float* kmax, float* o_cmp, float* lse,
                              const float* gate, void* out, const int32_t* coords,
                              const QRope& qr, hipStream_t s) {
  // gated: the epilogue adds this branch's gated share to the local branch's
  // in out (and writes o_cmp too when given, for the backward)
  const bool gated = out != nullptr;
  // with kmax the summaries carry the softmax scale in log2 units already
  const float c = kmax ? 1.0f : g.scale * kLog2e;
  if (g.bf16)
    return gated ? launch_g<bf16_t, true>(g, q, k_sum, v_sum, m, c, kmax, o_cmp, lse, gate, out,
                                          coords, qr, s)
                 : launch_g<bf16_t, false>(g, q, k_sum, v_sum, m, c, kmax, o_cmp, lse, gate, out,
                                           coords, qr, s);
  return gated ? launch_g<float, true>(g, q, k_sum, v_sum, m, c, kmax, o_cmp, lse, gate, out,
                                       coords, qr, s)
               : launch_g<float, false>(g, q, k_sum, v_sum, m, c, kmax, o_cmp, lse, gate, out,
                                        coords, qr, s);
}

}  // namespace pack3d
