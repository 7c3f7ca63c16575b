// Backward of the PACK3D forward (bf16 tensors, fp32 accumulation).
//
// The pages define the forward ("Geometry Matters in Packed 3D Attention",
// papernotes.org notes: key designs 1-3 and the flowchart); the operator is a
// block of a trained network (the notes' loss / training paragraph), so its
// gradients are the forward's derivatives.  For one softmax attention with
// probabilities p_u = exp(tau <q, k_u> - lse) and upstream gradient g:
//   dp_u = <g, v_u>,  D = <g, o>,  ds_u = p_u (dp_u - D),
//   dq = tau sum_u ds_u k_u,  dk_u = tau ds_u q,  dv_u = p_u g.
// The forward saved o and lse of both branches, so p is recomputed directly
// (no running max).
//
// Kernels:
//   k_bwd_prep   per token: gate weights, the branch upstream gradients
//                g_b * dO (bf16), D of both branches, the gate-logit gradient
//   k_glob_dq    query -> summary dq (queries stationary, summaries streamed
//                through LDS; S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T)
//   k_glob_dkv   summary gradients (summaries stationary in registers, the
//                group's query rows streamed in raster-cell order;
//                S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS), one
//                partial per slice of the query stream
//   k_loc_dq     local dq over the coordinate planes of the window
//   k_loc_dkv    local dk / dv: keys stationary, the window's query cells
//                (symmetric window) streamed one plane and head at a time
//   k_unrotate   dq = R(c)^T (local + summary dq)
//   k_sum_bwd    dk_cmp = a R(c)^T dk~, dv_cmp = a dv~ (partials summed in a
//                fixed order)
// Every sum runs in an order fixed by coordinates, never by packing.
#include <utility>

#include "local_tiles.h"

namespace pack3d {

namespace bw {

typedef KLds<bf16_t> TL;     // row layout of every 64 x 64 bf16 tile here

// A operand of a contraction over head dims: rows of a row-major tile.
__device__ __forceinline__ void row_frags(const bf16_t* t, int row, int h, bf16x8 (&f)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    f[s] = *reinterpret_cast<const bf16x8*>(t + TL::chunk_off(row, h * 4 + s));
}

// A operand of a contraction over tile rows (the transposed tile): for
// output row dim = 32*db + l%32, element e of step t holds
// tile[row0 + kr(t, e, h)][dim], read with the transposing LDS load (in each
// group of 16 lanes, lane i receives element i%4 of the 8-byte chunks
// addressed by lanes i/4 + 4j).
__device__ __forceinline__ void tr_frags(const bf16_t* t, int row0, int db, int lane,
                                         bf16x8 (&f)[2]) {
  const int h = lane >> 5, r = lane & 15;
  const int dim = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (r & 3);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = row0 + 16 * tt + 8 * half + 4 * h + (r >> 2);
      const bf16x4 part = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(
              (__attribute__((address_space(3))) bf16_t*)(t + TL::chunk_off(row, dim >> 3) +
                                                         (dim & 7))));
#pragma unroll
      for (int j = 0; j < 4; ++j) f[tt][4 * half + j] = part[j];
    }
}

__device__ __forceinline__ f32x16 contract_dims(const bf16x8 (&a)[4], const QFrag<bf16_t>& b,
                                                 f32x16 acc = f32x16{}) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = Mma<bf16_t>::mma(a[s], b.f[s], acc);
  return acc;
}

// 4 consecutive fp32 outputs of an accumulator column: dims d0 .. d0+3 with
// d0 = 32*db + 8*q4 + 4h hold elements 4*q4 .. 4*q4+3.
__device__ __forceinline__ f32x4 acc4(const f32x16& a, int q4, float s) {
  f32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = a[4 * q4 + j] * s;
  return r;
}

// ---------------------------------------------------------------------------
// k_bwd_prep: one wave per token.  Lane = 16-byte chunk (8 dims) of one
// head's row; the 8 lanes of a head reduce with XOR shuffles.  The
// compressed branch's D is stored negated, next to -lse * log2(e): the
// starting values of its kernels' accumulators.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void softmax2(float l0, float l1, float& g0, float& g1) {
  const float mx = fmaxf(l0, l1);
  const float e0 = expf(l0 - mx), e1 = expf(l1 - mx);
  g0 = e0 / (e0 + e1);
  g1 = e1 / (e0 + e1);
}

__global__ __launch_bounds__(256) void k_bwd_prep(const bf16_t* __restrict__ dout,
                                                  const float* __restrict__ o_loc,
                                                  const float* __restrict__ o_cmp,
                                                  const float* __restrict__ gate,
                                                  const float* __restrict__ lse_c, int64_t n,
                                                  int32_t hq, int32_t per_head, bf16_t* dlo,
                                                  bf16_t* dco, float* dl, float* dc, float* nls,
                                                  float* dgate) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;
  float g0 = 0.0f, g1 = 0.0f;
  if (!per_head) softmax2(gate[2 * t], gate[2 * t + 1], g0, g1);
  float tot0 = 0.0f, tot1 = 0.0f;
  const int nch = hq * 8;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + lane, head = c >> 3;
    const bool ok = c < nch;
    float gl = g0, gc = g1;
    if (per_head && ok) softmax2(gate[(t * hq + head) * 2], gate[(t * hq + head) * 2 + 1], gl, gc);
    float sl = 0.0f, sc = 0.0f, pl = 0.0f, pc = 0.0f;
    if (ok) {
      const int64_t base = t * hq * 64 + (int64_t)c * 8;
      const bf16x8 d = *reinterpret_cast<const bf16x8*>(dout + base);
      const f32x4 ol0 = *reinterpret_cast<const f32x4*>(o_loc + base);
      const f32x4 ol1 = *reinterpret_cast<const f32x4*>(o_loc + base + 4);
      const f32x4 oc0 = *reinterpret_cast<const f32x4*>(o_cmp + base);
      const f32x4 oc1 = *reinterpret_cast<const f32x4*>(o_cmp + base + 4);
      bf16x8 bl, bc;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)d[e];
        const float ol = e < 4 ? ol0[e] : ol1[e - 4];
        const float oc = e < 4 ? oc0[e] : oc1[e - 4];
        bl[e] = (bf16_t)(gl * x);
        bc[e] = (bf16_t)(gc * x);
        // D pairs the rounded branch gradient (the MFMA operand) with o
        sl = fmaf((float)bl[e], ol, sl);
        sc = fmaf((float)bc[e], oc, sc);
        pl = fmaf(x, ol, pl);
        pc = fmaf(x, oc, pc);
      }
      *reinterpret_cast<bf16x8*>(dlo + base) = bl;
      *reinterpret_cast<bf16x8*>(dco + base) = bc;
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
      sl += __shfl_xor(sl, m);
      sc += __shfl_xor(sc, m);
      pl += __shfl_xor(pl, m);
      pc += __shfl_xor(pc, m);
    }
    if (ok && (lane & 7) == 0) {
      dl[t * hq + head] = sl;
      dc[t * hq + head] = -sc;
      nls[t * hq + head] = -(lse_c[t * hq + head] * kLog2e);
      if (per_head) {
        // two-logit softmax Jacobian: d l0 = g0 g1 (dg0 - dg1) = -d l1
        const float d0 = gl * gc * (pl - pc);
        dgate[(t * hq + head) * 2] = d0;
        dgate[(t * hq + head) * 2 + 1] = -d0;
      }
      tot0 += pl;
      tot1 += pc;
    }
  }
  if (!per_head) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      tot0 += __shfl_xor(tot0, m);
      tot1 += __shfl_xor(tot1, m);
    }
    if (lane == 0) {
      const float d0 = g0 * g1 * (tot0 - tot1);
      dgate[2 * t] = d0;
      dgate[2 * t + 1] = -d0;
    }
  }
}

// ---------------------------------------------------------------------------
// k_glob_dq: workgroup = 8 waves = one KV group x 512 query rows (two
// 32-column blocks per wave), summaries streamed in 64-key tiles double-
// buffered in LDS through registers (the next tile's loads are issued after
// the barrier and land while the current tile is computed).
// ---------------------------------------------------------------------------
constexpr int kGW = 8, kGCb = 2, kGRows = kGW * kGCb * 32, kGKt = 64;

struct GdqArgs {
  const bf16_t* q;         // rotated queries [N, Hq, 64]
  const bf16_t* dco;       // g_cmp * dO [N, Hq, 64]
  const bf16_t* ks;        // key summaries [Hkv, M, 64]
  const bf16_t* vs;
  const float* lse;        // lse_cmp [N, Hq]
  const float* ndd;        // -D_cmp [N, Hq]
  float* dq;               // in: local dq (tau included); out: + summary dq
  int64_t m, n;
  int32_t hq, hkv, grp;
  float c;                 // q . ks * c = the log2-domain logit
  float tau;               // tau * sum dS ks = dq
  int64_t tiles;
  int32_t xcd_per;
};

__global__ __launch_bounds__(64 * kGW) void k_glob_dq(GdqArgs A) {
  __shared__ __attribute__((aligned(16))) bf16_t k_l[2][kGKt * 64];
  __shared__ __attribute__((aligned(16))) bf16_t v_l[2][kGKt * 64];
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
  const bf16_t* ksg = A.ks + (int64_t)grp * A.m * 64;
  const bf16_t* vsg = A.vs + (int64_t)grp * A.m * 64;

  QFrag<bf16_t> qf[kGCb], df[kGCb];
  int64_t tok[kGCb];
  int head[kGCb];
  bool valid[kGCb];
  float lse2[kGCb], nddv[kGCb];
#pragma unroll
  for (int cb = 0; cb < kGCb; ++cb) {
    const int64_t row = tile * kGRows + (int64_t)(wave * kGCb + cb) * 32 + col;
    valid[cb] = row < nrows;
    tok[cb] = valid[cb] ? row / A.grp : 0;
    head[cb] = grp * A.grp + (valid[cb] ? (int)(row % A.grp) : 0);
    const int64_t r = tok[cb] * A.hq + head[cb];
    load_qfrag<bf16_t>(qf[cb], A.q + r * 64 + h * 32, valid[cb]);
    load_qfrag<bf16_t>(df[cb], A.dco + r * 64 + h * 32, valid[cb]);
    lse2[cb] = valid[cb] ? A.lse[r] * kLog2e : 0.0f;
    nddv[cb] = valid[cb] ? A.ndd[r] : 0.0f;
  }
  f32x16 acc[kGCb][2];
#pragma unroll
  for (int cb = 0; cb < kGCb; ++cb) acc[cb][0] = acc[cb][1] = f32x16{};

  // one 16-byte chunk of K and of V per thread per tile
  const int srow = tid >> 3, sch = tid & 7;
  // Tile base pointers are uniform and lane offsets 32-bit, so no 64-bit
  // address stays live across the loop.  Keys past M read the last summary
  // (finite; M >= 1 since the block divides the grid); their p is masked to 0.
  auto load = [&](int64_t t, u32x4& sk, u32x4& sv) {
    const int64_t k0 = t * kGKt;
    const int64_t left = A.m - 1 - k0;
    const int lim = left < kGKt - 1 ? (int)left : kGKt - 1;
    const uint32_t off = (uint32_t)(srow < lim ? srow : lim) * 128u + (uint32_t)sch * 16u;
    sk = ld16(reinterpret_cast<const bf16_t*>(reinterpret_cast<const char*>(ksg + k0 * 64) + off));
    sv = ld16(reinterpret_cast<const bf16_t*>(reinterpret_cast<const char*>(vsg + k0 * 64) + off));
  };
  u32x4 sk, sv;
  load(0, sk, sv);
  const int64_t nt = (A.m + kGKt - 1) / kGKt;
  for (int64_t t = 0; t < nt; ++t) {
    const int b = (int)(t & 1);
    st16(k_l[b] + TL::chunk_off(srow, sch), sk);
    st16(v_l[b] + TL::chunk_off(srow, sch), sv);
    __syncthreads();
    if (t + 1 < nt) load(t + 1, sk, sv);
    const bool full = (t + 1) * kGKt <= A.m;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8 kf[4], vf[4];
      row_frags(k_l[b], kb * 32 + col, h, kf);
      row_frags(v_l[b], kb * 32 + col, h, vf);
      bf16x8 dsf[kGCb][2];
#pragma unroll
      for (int cb = 0; cb < kGCb; ++cb) {
        const f32x16 s = contract_dims(kf, qf[cb]);
        const f32x16 dp = contract_dims(vf, df[cb]);
        f32x16 ds;
        if (full) {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            ds[v] = __builtin_amdgcn_exp2f(fmaf(s[v], A.c, -lse2[cb])) * (dp[v] + nddv[cb]);
        } else {
          // keys past M: p = 0
          const int lim = (int)(A.m - t * kGKt) - kb * 32 - 4 * h;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const bool ok = 8 * (v >> 2) + (v & 3) < lim;
            const float p = ok ? __builtin_amdgcn_exp2f(fmaf(s[v], A.c, -lse2[cb])) : 0.0f;
            ds[v] = p * (dp[v] + nddv[cb]);
          }
        }
        dsf[cb][0] = Mma<bf16_t>::p_frag(ds, 0);
        dsf[cb][1] = Mma<bf16_t>::p_frag(ds, 1);
      }
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        bf16x8 kt[2];
        tr_frags(k_l[b], kb * 32, db, lane, kt);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int cb = 0; cb < kGCb; ++cb)
            acc[cb][db] = Mma<bf16_t>::mma(kt[tt], dsf[cb][tt], acc[cb][db]);
      }
    }
  }
#pragma unroll
  for (int cb = 0; cb < kGCb; ++cb) {
    if (!valid[cb]) continue;
    float* o = A.dq + (tok[cb] * A.hq + head[cb]) * 64;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * h;
        f32x4 r = acc4(acc[cb][db], q4, A.tau);
        const f32x4 prev = *reinterpret_cast<const f32x4*>(o + d0);
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] += prev[j];
        *reinterpret_cast<f32x4*>(o + d0) = r;
      }
  }
}

// ---------------------------------------------------------------------------
// k_glob_dkv: workgroup = 8 waves = 256 summaries of one group (32 per wave,
// held in registers as MFMA B operands) x one slice of the group's query
// stream.  The stream runs over lattice cells in raster order, 64 query rows
// (64/G cells x G heads) per tile, gathered through cell_to_pos.  Tiles are
// copied global -> LDS asynchronously in phases of kKPh tiles (rows, their
// lse and -D): the copies of the next phase are issued at the start of a
// phase and land while its tiles are computed; one wait + barrier per phase
// publishes them and frees the previous phase's buffer.
// ---------------------------------------------------------------------------
constexpr int kKW = 8, kKKeys = kKW * 32, kKRows = 64;
constexpr int kKPh = 4;                                  // tiles per phase
constexpr int kKTileElems = kKRows * 64;                 // one 64 x 64 bf16 tile

struct GkvArgs {
  const bf16_t* q;
  const bf16_t* dco;
  const bf16_t* ks;
  const bf16_t* vs;
  const float* nls;        // -lse * log2(e) of the compressed branch [N, Hq]
  const float* ndd;        // -D of the compressed branch [N, Hq]
  const int32_t* c2p;
  float* dk;               // partials [nsplit, Hkv, M, 64]
  float* dv;
  int64_t m, ncell;
  int32_t hq, hkv, grp;
  float tau;
  int64_t nkt;             // key tiles (of 256) per group
  int32_t nsplit;
  int64_t cps;             // cells per slice
};

// Separate LDS arrays hold the two phases, so the compiler can tell the
// copies in flight from the tiles being read: q and dO rows of the phase's
// tiles, then per tile the 64 values of -lse*log2(e) and of -D.
template <int I>
struct KvBuf {
  __device__ static __forceinline__ bf16_t* q() {
    __shared__ __attribute__((aligned(16))) bf16_t b[kKPh * kKTileElems];
    return b;
  }
  __device__ static __forceinline__ bf16_t* d() {
    __shared__ __attribute__((aligned(16))) bf16_t b[kKPh * kKTileElems];
    return b;
  }
  __device__ static __forceinline__ float* ld() {
    __shared__ __attribute__((aligned(16))) float b[kKPh * 2 * kKRows];
    return b;
  }
};

// What a row past the slice reads: zero q and dO, -lse*log2(e) = -inf (so
// p = 0) and -D = 0.
struct __attribute__((aligned(16))) KvPad {
  float zero[32];
  float ninf;
  float zero1[3];
};
__device__ KvPad g_kv_pad = {{}, -__builtin_inff(), {}};

__global__ __launch_bounds__(64 * kKW) void k_glob_dkv(GkvArgs A) {
  const int64_t bid = blockIdx.x;
  const int split = (int)(bid % A.nsplit);
  const int grp = (int)((bid / A.nsplit) % A.hkv);
  const int64_t kt = bid / ((int64_t)A.nsplit * A.hkv);
  if (kt >= A.nkt) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, col = lane & 31;
  const int64_t key = kt * kKKeys + wave * 32 + col;
  const bool kok = key < A.m;
  QFrag<bf16_t> kq, vq;
  load_qfrag<bf16_t>(kq, A.ks + ((int64_t)grp * A.m + (kok ? key : 0)) * 64 + h * 32, kok);
  load_qfrag<bf16_t>(vq, A.vs + ((int64_t)grp * A.m + (kok ? key : 0)) * 64 + h * 32, kok);
  f32x16 dk[2] = {f32x16{}, f32x16{}}, dv[2] = {f32x16{}, f32x16{}};

  const int64_t c0 = (int64_t)split * A.cps;
  const int64_t c1 = c0 + A.cps < A.ncell ? c0 + A.cps : A.ncell;
  const int cpt = kKRows / A.grp;                    // cells per tile
  const int64_t nt = c1 > c0 ? (c1 - c0 + cpt - 1) / cpt : 0;
  const int64_t nph = (nt + kKPh - 1) / kKPh;
  const int head0 = grp * A.grp;

  // Copy assignment.  Rows: copy i of a wave moves 8 rows of tile i (row
  // 8*wave + lane/8, 16-byte chunk lane%8 of its LDS row; the tile swizzle is
  // applied on the source side).  -lse*log2(e) / -D: wave w moves the 64
  // values of array w%2 of tile w/2.  A position is the raw table entry plus a
  // validity flag computed from the cell index alone, so nothing waits for
  // the entry until the copies that use it are issued, a phase later.
  const int crow = wave * 8 + (lane >> 3);
  const int cch = (lane & 7) ^ ((((crow >> 1) & 1) << 2) | ((crow >> 2) & 3));
  const int chead = head0 + crow % A.grp;
  const int lhead = head0 + lane % A.grp;
  struct Pos {
    int32_t p[kKPh];
    bool ok[kKPh];
    int32_t lp;
    bool lok;
  };
  auto position = [&](int64_t c) -> int32_t { return A.c2p[c < c1 ? c : c1 - 1]; };
  auto positions = [&](int64_t ph, Pos& P) {
#pragma unroll
    for (int i = 0; i < kKPh; ++i) {
      const int64_t cell = c0 + (ph * kKPh + i) * cpt + crow / A.grp;
      P.p[i] = position(cell);
      P.ok[i] = cell < c1;
    }
    const int64_t cell = c0 + (ph * kKPh + (wave >> 1)) * cpt + lane / A.grp;
    P.lp = position(cell);
    P.lok = cell < c1;
  };
  auto issue = [&](bf16_t* bq, bf16_t* bd, float* bl, const Pos& P) {
#pragma unroll
    for (int i = 0; i < kKPh; ++i) {
      const int64_t r = (int64_t)P.p[i] * A.hq + chead;
      const void* sq = P.ok[i] ? (const void*)(A.q + r * 64 + cch * 8) : (const void*)g_kv_pad.zero;
      const void* sd = P.ok[i] ? (const void*)(A.dco + r * 64 + cch * 8) : (const void*)g_kv_pad.zero;
      __builtin_amdgcn_global_load_lds(sq, (lb::lds_ptr)(bq + i * kKTileElems + wave * 512), 16, 0,
                                       0);
      __builtin_amdgcn_global_load_lds(sd, (lb::lds_ptr)(bd + i * kKTileElems + wave * 512), 16, 0,
                                       0);
    }
    const int64_t r = (int64_t)P.lp * A.hq + lhead;
    const float* src = (wave & 1) ? A.ndd : A.nls;
    const void* sl = P.lok ? (const void*)(src + r)
                           : (const void*)((wave & 1) ? g_kv_pad.zero1 : &g_kv_pad.ninf);
    __builtin_amdgcn_global_load_lds(sl, (lb::lds_ptr)(bl + wave * 64), 4, 0, 0);
  };
  auto tile = [&](const bf16_t* q_l, const bf16_t* d_l, const float* ls_l) {
    const float* dd_l = ls_l + kKRows;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      bf16x8 qr[4], dr[4];
      row_frags(q_l, rb * 32 + col, h, qr);
      row_frags(d_l, rb * 32 + col, h, dr);
      // accumulator element v holds query row rb*32 + 8*(v/4) + 4h + v%4:
      // start S at -lse (log2 units) and dP at -D, so the products come out
      // as the exponent of p and as dP - D
      f32x16 nl, nd;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r0 = rb * 32 + 8 * q4 + 4 * h;
        const f32x4 L = *reinterpret_cast<const f32x4*>(&ls_l[r0]);
        const f32x4 D = *reinterpret_cast<const f32x4*>(&dd_l[r0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          nl[4 * q4 + j] = L[j];
          nd[4 * q4 + j] = D[j];
        }
      }
      const f32x16 s = contract_dims(qr, kq, nl);
      const f32x16 dp = contract_dims(dr, vq, nd);
      f32x16 p, ds;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        p[v] = __builtin_amdgcn_exp2f(s[v]);
        ds[v] = p[v] * dp[v];
      }
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        pf[tt] = Mma<bf16_t>::p_frag(p, tt);
        dsf[tt] = Mma<bf16_t>::p_frag(ds, tt);
      }
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        bf16x8 dt[2], qt[2];
        tr_frags(d_l, rb * 32, db, lane, dt);
        tr_frags(q_l, rb * 32, db, lane, qt);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          dv[db] = Mma<bf16_t>::mma(dt[tt], pf[tt], dv[db]);
          dk[db] = Mma<bf16_t>::mma(qt[tt], dsf[tt], dk[db]);
        }
      }
    }
  };
  // The stream is padded to whole phases: a padding tile has no rows (p = 0,
  // adding exact zeros).
  auto phase = [&](auto cur, auto nxt, int64_t ph, const Pos& pn, Pos& pf) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ph + 1 < nph) issue(decltype(nxt)::q(), decltype(nxt)::d(), decltype(nxt)::ld(), pn);
    if (ph + 2 < nph) positions(ph + 2, pf);
#pragma unroll
    for (int i = 0; i < kKPh; ++i)
      tile(decltype(cur)::q() + i * kKTileElems, decltype(cur)::d() + i * kKTileElems,
           decltype(cur)::ld() + i * 2 * kKRows);
  };
  if (nph > 0) {
    Pos pa, pb;
    positions(0, pa);
    issue(KvBuf<0>::q(), KvBuf<0>::d(), KvBuf<0>::ld(), pa);
    if (nph > 1) positions(1, pb);
    for (int64_t ph = 0; ph < nph; ph += 2) {
      phase(KvBuf<0>{}, KvBuf<1>{}, ph, pb, pa);
      if (ph + 1 < nph) phase(KvBuf<1>{}, KvBuf<0>{}, ph + 1, pa, pb);
    }
  }
  if (!kok) return;
  const int64_t ob = (((int64_t)split * A.hkv + grp) * A.m + key) * 64;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = db * 32 + 8 * q4 + 4 * h;
      *reinterpret_cast<f32x4*>(A.dk + ob + d0) = acc4(dk[db], q4, A.tau);
      *reinterpret_cast<f32x4*>(A.dv + ob + d0) = acc4(dv[db], q4, 1.0f);
    }
}

// ---------------------------------------------------------------------------
// k_loc_dq: the local forward's tiling (plane slots, masks, XCD order), with
// p recomputed from the saved lse and dq accumulated instead of o.
// ---------------------------------------------------------------------------
struct LdqArgs {
  const bf16_t* q;         // rotated
  const bf16_t* k;         // rotated
  const bf16_t* v;
  const bf16_t* dlo;       // g_loc * dO
  const float* lse;        // lse_loc
  const float* dd;         // D_loc
  const int32_t* c2p;
  float* dq;               // out: tau * local dq (rotated frame)
  int32_t Z, Y, X, hq, hkv;
  int32_t rz, ry, rx;
  float c, tau;
  int32_t tiles_y, tiles_x;
  int64_t nblocks;
  int64_t per_xcd;
};

template <int G>
__global__ __launch_bounds__(64 * lb::Cfg<G>::W) void k_loc_dq(LdqArgs A) {
  using namespace lb;
  using C = Cfg<G>;
  constexpr int PY = C::PY, PX = C::PX, TX = C::TX, NKB = C::NKB, KY = C::KY, RX = C::RX,
                RC = C::RC, RCP = C::RCP, RCA = C::RCA, W = C::W, NT = 64 * W;
  __shared__ __attribute__((aligned(16))) bf16_t k_lds0[RCA * 64];
  __shared__ __attribute__((aligned(16))) bf16_t k_lds1[RCA * 64];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds0[RCA * 64];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds1[RCA * 64];

  const int64_t bid = blockIdx.x;
  const int64_t lin = (bid % kNumXcd) * A.per_xcd + bid / kNumXcd;
  if (lin >= A.nblocks) return;
  const int tx = (int)(lin % A.tiles_x);
  const int ty = (int)((lin / A.tiles_x) % A.tiles_y);
  const int z0 = (int)((lin / ((int64_t)A.tiles_x * A.tiles_y)) % A.Z);
  const int grp = (int)(lin / ((int64_t)A.tiles_x * A.tiles_y * A.Z));
  const int y0 = ty * C::TY, x0 = tx * TX;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = col % G, cip = col / G, qy = cip / PX, qx = cip % PX;
  const int py0 = (wave / (TX / PX)) * PY, px0 = (wave % (TX / PX)) * PX;

  constexpr int NPC = (RCP / 8 + W - 1) / W;
  auto load_pos = [&](int zz, int32_t (&pos)[NPC]) {
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int cell = (wave + W * i) * 8 + (lane >> 3);
      const int yy = y0 - kHalo + cell / RX, xx = x0 - kHalo + cell % RX;
      pos[i] = cell < RC && yy >= 0 && yy < A.Y && xx >= 0 && xx < A.X
                   ? A.c2p[((int64_t)zz * A.Y + yy) * A.X + xx]
                   : 0;
    }
  };
  const bf16_t* kg = A.k + (int64_t)grp * 64;
  const bf16_t* vg = A.v + (int64_t)grp * 64;
  const int64_t rstride = (int64_t)A.hkv * 64;
  auto issue_loads = [&](const int32_t (&pos)[NPC], bf16_t* kl, bf16_t* vl) {
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int pc = wave + W * i;
      if (pc < RCP / 8) {
        const int cell = pc * 8 + (lane >> 3), cp = lane & 7;
        const int64_t row = (int64_t)pos[i] * rstride;
        __builtin_amdgcn_global_load_lds(
            (const void*)(kg + row + kv_swz(cell / RX, cell % RX, cp) * 8),
            (lds_ptr)(kl + pc * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vg + row + kv_swz(cell / RX, cell % RX, cp) * 8),
                                         (lds_ptr)(vl + pc * 512), 16, 0, 0);
      }
    }
  };

  const int yq = y0 + py0 + qy, xq = x0 + px0 + qx;
  const bool qok = yq < A.Y && xq < A.X;
  const int64_t qpos = qok ? (int64_t)A.c2p[((int64_t)z0 * A.Y + yq) * A.X + xq] : 0;
  const int64_t qrow = qpos * A.hq + grp * G + hh;
  QFrag<bf16_t> qf, df;
  load_qfrag<bf16_t>(qf, A.q + qrow * 64 + h * 32, qok);
  load_qfrag<bf16_t>(df, A.dlo + qrow * 64 + h * 32, qok);
  const float lse2 = qok ? A.lse[qrow] * kLog2e : 0.0f;
  const float ddv = qok ? A.dd[qrow] : 0.0f;

  // window mask, as in the forward: key row 4kb + e/4, key column 4h + e%4
  bool rv[NKB * 4], cv[4];
#pragma unroll
  for (int r = 0; r < NKB * 4; ++r) {
    const int dy = r - kHalo - qy, yk = y0 + py0 + r - kHalo;
    rv[r] = qok && r < KY && dy >= -A.ry && dy <= A.ry && yk >= 0 && yk < A.Y;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int kx = 4 * h + c, dx = kx - kHalo - qx, xk = x0 + px0 + kx - kHalo;
    cv[c] = dx >= -A.rx && dx <= A.rx && xk >= 0 && xk < A.X;
  }

  // lane offsets: K and V rows (A operands of S and dP) and K^T (A operand of dQ)
  const int ky0 = py0 + col / 8, kx0 = px0 + col % 8, kcell = ky0 * RX + kx0;
  int koff[4], voff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    koff[st] = kcell * 64 + kv_swz(ky0, kx0, h * 4 + st) * 8;
    voff[st] = kcell * 64 + kv_swz(ky0, kx0, h * 4 + st) * 8;
  }
  const int r4 = lane & 15;
  int toff[2][2];   // [half][db]: K^T rows, + (4kb + 2t) region rows per step
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int ty_ = py0 + half, tx_ = px0 + 4 * h + (r4 >> 2), cell = ty_ * RX + tx_;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int dim = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (r4 & 3);
      toff[half][db] = cell * 64 + kv_swz(ty_, tx_, dim >> 3) * 8 + (dim & 7);
    }
  }

  f32x16 acc0 = {}, acc1 = {};
  auto compute_plane = [&](const bf16_t* kl, const bf16_t* vl) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      bf16x8 kf[4], vf[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        kf[st] = *reinterpret_cast<const bf16x8*>(kl + 4 * RX * 64 * kb + koff[st]);
        vf[st] = *reinterpret_cast<const bf16x8*>(vl + 4 * RX * 64 * kb + voff[st]);
      }
      const f32x16 s = contract_dims(kf, qf);
      const f32x16 dp = contract_dims(vf, df);
      f32x16 ds;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = (rv[4 * kb + e / 4] && cv[e % 4])
                            ? __builtin_amdgcn_exp2f(fmaf(s[e], A.c, -lse2))
                            : 0.0f;
        ds[e] = p * (dp[e] - ddv);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (4 * kb + 2 * t >= KY) continue;   // both key rows are padding
        const bf16x8 dsf = Mma<bf16_t>::p_frag(ds, t);
        const bf16_t* rows = kl + (4 * kb + 2 * t) * RX * 64;
        bf16x8 kt[2];
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const bf16x4 part = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(
                    (__attribute__((address_space(3))) bf16_t*)(rows + toff[half][db])));
#pragma unroll
            for (int j = 0; j < 4; ++j) kt[db][4 * half + j] = part[j];
          }
        acc0 = Mma<bf16_t>::mma(kt[0], dsf, acc0);
        acc1 = Mma<bf16_t>::mma(kt[1], dsf, acc1);
      }
    }
  };

  // planes, double-buffered exactly as in the forward
  for (int i = RCP * 8 + tid; i < RCA * 8; i += NT) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    st16(k_lds0 + 8 * i, z);
    st16(k_lds1 + 8 * i, z);
    st16(v_lds0 + 8 * i, z);
    st16(v_lds1 + 8 * i, z);
  }
  const int zlo = z0 - A.rz < 0 ? 0 : z0 - A.rz;
  const int zhi = z0 + A.rz >= A.Z ? A.Z - 1 : z0 + A.rz;
  const int np = zhi - zlo + 1;
  int32_t pos_a[NPC], pos_b[NPC];
  load_pos(zlo, pos_a);
  __builtin_amdgcn_s_waitcnt(0);
  issue_loads(pos_a, k_lds0, v_lds0);
  if (np > 1) load_pos(zlo + 1, pos_a);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int p = 0; p < np; p += 2) {
    if (p + 1 < np) issue_loads(pos_a, k_lds1, v_lds1);
    if (p + 2 < np) load_pos(zlo + p + 2, pos_b);
    compute_plane(k_lds0, v_lds0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (p + 1 >= np) break;
    if (p + 2 < np) issue_loads(pos_b, k_lds0, v_lds0);
    if (p + 3 < np) load_pos(zlo + p + 3, pos_a);
    compute_plane(k_lds1, v_lds1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (!qok) return;
  float* o = A.dq + qrow * 64;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    *reinterpret_cast<f32x4*>(o + 8 * q4 + 4 * h) = acc4(acc0, q4, A.tau);
    *reinterpret_cast<f32x4*>(o + 32 + 8 * q4 + 4 * h) = acc4(acc1, q4, A.tau);
  }
}

// ---------------------------------------------------------------------------
// k_loc_dkv: workgroup = 4 waves = an 8 x 8 tile of key cells of one z-plane
// and one KV group; waves w and w + 2 own the 4 x 8 patch of rows
// 4(w%2) .. 4(w%2)+3 (its 32 key cells are the MFMA columns, held in
// registers).  The window is symmetric, so a key's gradient sums over the
// queries in the box around it: for every plane of the window and every head
// of the group the workgroup copies the q and g_loc * dO rows of the 14 x 16
// region (tile plus a 3-cell halo, padded to 16 columns) into LDS, with lse
// and D per cell.  A patch's 10 x 16 query slots form five 32-slot blocks;
// its two waves split them 3 + 2 (which wave takes three alternates between
// workgroups), so two workgroups share each SIMD and one computes while the
// other waits for its copies; the two partial sums meet in LDS at the end.
// ---------------------------------------------------------------------------
constexpr int kDW = 4, kDTY = 8, kDTX = 8, kDRY = kDTY + 2 * lb::kHalo, kDRX = 16;
constexpr int kDRC = kDRY * kDRX;      // 224 region cells
constexpr int kDSY = 4 + 2 * lb::kHalo;  // query slot rows per wave (10)
constexpr int kDBlk = kDSY * kDRX / 32;  // 32-slot blocks per wave (5)
static_assert(kDSY * kDRX % 32 == 0, "whole slot blocks");
static_assert(kDRC % 8 == 0, "1 KB pieces");

// chunk position in a region cell's row (cells numbered row-major, 16 per
// region row).  Row reads take 16 consecutive cells per 16 lanes, the
// transposing reads 4 consecutive cells x 4 aligned chunks per 32 lanes; the
// tile swizzle 4 ((cell >> 1) & 1) + ((cell >> 2) & 3) serves both without
// bank conflicts (cells c and c + 2 land in different 4-chunk halves).
__device__ __forceinline__ int q_swz(int cell, int chunk) {
  return chunk ^ ((((cell >> 1) & 1) << 2) | ((cell >> 2) & 3));
}

struct LkvArgs {
  const bf16_t* q;         // rotated queries
  const bf16_t* dlo;       // g_loc * dO
  const float* lse;        // lse_loc
  const float* dd;         // D_loc
  const bf16_t* k;         // rotated keys
  const bf16_t* v;
  const int32_t* c2p;
  bf16_t* dk;              // out: dk_loc (unrotated frame)
  bf16_t* dv;              // out: dv_loc
  int32_t Z, Y, X, hq, hkv, G;
  int32_t rz, ry, rx;
  float c, tau;
  int32_t tiles_y, tiles_x;
  int64_t nblocks;
  int64_t per_xcd;
  RopeTab rope;
};

__global__ __launch_bounds__(64 * kDW) void k_loc_dkv(LkvArgs A) {
  __shared__ __attribute__((aligned(16))) bf16_t q_l[kDRC * 64];
  __shared__ __attribute__((aligned(16))) bf16_t d_l[kDRC * 64];
  __shared__ __attribute__((aligned(16))) float ls_l[kDRC];
  __shared__ __attribute__((aligned(16))) float dd_l[kDRC];
  __shared__ int32_t pos_l[2][kDRC];
  const int64_t bid = blockIdx.x;
  const int64_t lin = (bid % kNumXcd) * A.per_xcd + bid / kNumXcd;
  if (lin >= A.nblocks) return;
  const int tx = (int)(lin % A.tiles_x);
  const int ty = (int)((lin / A.tiles_x) % A.tiles_y);
  const int z0 = (int)((lin / ((int64_t)A.tiles_x * A.tiles_y)) % A.Z);
  const int grp = (int)(lin / ((int64_t)A.tiles_x * A.tiles_y * A.Z));
  const int y0 = ty * kDTY, x0 = tx * kDTX;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 1, part = wave >> 1;
  const int split = (lin & 1) ? 2 : 3;   // part 0: blocks < split, part 1: the rest
  const int py0 = 4 * kw;
  const int ky = col / 8, kx = col % 8;
  const int yk = y0 + py0 + ky, xk = x0 + kx;
  const bool kok = yk < A.Y && xk < A.X;
  const int64_t kpos = kok ? (int64_t)A.c2p[((int64_t)z0 * A.Y + yk) * A.X + xk] : 0;
  const int64_t krow = kpos * A.hkv + grp;
  QFrag<bf16_t> kq, vq;
  load_qfrag<bf16_t>(kq, A.k + krow * 64 + h * 32, kok);
  load_qfrag<bf16_t>(vq, A.v + krow * 64 + h * 32, kok);

  // query slot (sy, sx), sy < 10, sx < 16 of this wave is region cell
  // (py0 + sy, sx): lattice cell (y0 - 3 + py0 + sy, x0 - 3 + sx).  In block
  // blk, element v on lane half h is slot 32 blk + 8(v/4) + 4h + v%4, i.e.
  // sy = 2 blk + (v >= 8), sx = 8((v/4) % 2) + 4h + v%4.
  bool rok[kDSY], cok[8];
#pragma unroll
  for (int sy = 0; sy < kDSY; ++sy) {
    const int dy = sy - lb::kHalo - ky;
    rok[sy] = kok && dy >= -A.ry && dy <= A.ry;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sx = 8 * (i >> 2) + 4 * h + (i & 3), dx = sx - lb::kHalo - kx;
    cok[i] = dx >= -A.rx && dx <= A.rx;
  }
  // lane offsets: row fragments of slot col of block 0; transposed reads
  const int rcell = (py0 + col / 16) * kDRX + col % 16;
  int roff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) roff[st] = rcell * 64 + q_swz(rcell, h * 4 + st) * 8;
  const int r4 = lane & 15;
  int toff[2][2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int cell = py0 * kDRX + 8 * half + 4 * h + (r4 >> 2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int dim = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (r4 & 3);
      toff[half][db] = cell * 64 + q_swz(cell, dim >> 3) * 8 + (dim & 7);
    }
  }

  f32x16 dk[2] = {f32x16{}, f32x16{}}, dv[2] = {f32x16{}, f32x16{}};
  const int zlo = z0 - A.rz < 0 ? 0 : z0 - A.rz;
  const int zhi = z0 + A.rz >= A.Z ? A.Z - 1 : z0 + A.rz;
  constexpr int kPieces = kDRC / 8;
  // Packed positions of the region's cells in the current plane (-1: off the
  // lattice) sit in LDS, read once per plane: the next plane's load during
  // the current plane's last head and are stored after its compute, so each
  // plane-and-head step waits for one round of loads (rows, lse, D) only.
  constexpr int kPosPer = (kDRC + 64 * kDW - 1) / (64 * kDW);
  auto region_pos = [&](int zz, int cell) -> int32_t {
    const int yy = y0 - lb::kHalo + cell / kDRX, xx = x0 - lb::kHalo + cell % kDRX;
    const bool ok = cell < kDRC && yy >= 0 && yy < A.Y && xx >= 0 && xx < A.X;
    return ok ? A.c2p[((int64_t)zz * A.Y + yy) * A.X + xx] : -1;
  };
  {
    int32_t p0[kPosPer];
#pragma unroll
    for (int k = 0; k < kPosPer; ++k) p0[k] = region_pos(zlo, tid + 64 * kDW * k);
#pragma unroll
    for (int k = 0; k < kPosPer; ++k)
      if (tid + 64 * kDW * k < kDRC) pos_l[0][tid + 64 * kDW * k] = p0[k];
  }
  __syncthreads();
  int pb = 0;
  for (int zz = zlo; zz <= zhi; ++zz) {
    for (int hd = 0; hd < A.G; ++hd) {
      const int head = grp * A.G + hd;
      const int32_t* pos = pos_l[pb];
      // copies of the region's q and g_loc*dO rows for this plane and head
      // (cells off the lattice copy row 0: finite, and masked to p = 0)
      for (int pc = wave; pc < kPieces; pc += kDW) {
        const int cell = pc * 8 + (lane >> 3), cp = lane & 7;
        const int32_t pp = pos[cell];
        const int64_t r = (int64_t)(pp >= 0 ? pp : 0) * A.hq + head;
        const int src = q_swz(cell, cp);
        __builtin_amdgcn_global_load_lds((const void*)(A.q + r * 64 + src * 8),
                                         (lb::lds_ptr)(q_l + pc * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(A.dlo + r * 64 + src * 8),
                                         (lb::lds_ptr)(d_l + pc * 512), 16, 0, 0);
      }
      for (int cell = tid; cell < kDRC; cell += 64 * kDW) {
        const int32_t pp = pos[cell];
        float l = __builtin_inff(), d = 0.0f;   // off the lattice: p = 0
        if (pp >= 0) {
          const int64_t r = (int64_t)pp * A.hq + head;
          l = A.lse[r] * kLog2e;
          d = A.dd[r];
        }
        ls_l[cell] = l;
        dd_l[cell] = d;
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const bool next_plane = hd == A.G - 1 && zz < zhi;
      int32_t np[kPosPer];
#pragma unroll
      for (int k = 0; k < kPosPer; ++k) np[k] = next_plane ? region_pos(zz + 1, tid + 64 * kDW * k) : -1;
#pragma unroll
      for (int blk = 0; blk < kDBlk; ++blk) {
        if ((blk < split) != (part == 0)) continue;
        const int boff = 2 * blk * kDRX * 64;    // two region rows per block
        bf16x8 qr[4], dr[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          qr[st] = *reinterpret_cast<const bf16x8*>(q_l + boff + roff[st]);
          dr[st] = *reinterpret_cast<const bf16x8*>(d_l + boff + roff[st]);
        }
        const f32x16 s = contract_dims(qr, kq);
        const f32x16 dp = contract_dims(dr, vq);
        f32x16 p, ds;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int sy = 2 * blk + (q4 >= 2);
          const int cell = (py0 + sy) * kDRX + 8 * (q4 & 1) + 4 * h;
          const f32x4 L = *reinterpret_cast<const f32x4*>(&ls_l[cell]);
          const f32x4 D = *reinterpret_cast<const f32x4*>(&dd_l[cell]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int v = 4 * q4 + j;
            const bool in = rok[sy] && cok[4 * (q4 & 1) + j];
            p[v] = in ? __builtin_amdgcn_exp2f(fmaf(s[v], A.c, -L[j])) : 0.0f;
            ds[v] = p[v] * (dp[v] - D[j]);
          }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const bf16x8 pf = Mma<bf16_t>::p_frag(p, tt);
          const bf16x8 dsf = Mma<bf16_t>::p_frag(ds, tt);
          const int rows = boff + tt * kDRX * 64;   // slot rows 2blk + tt
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            bf16x8 dt, qt;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                  (__attribute__((address_space(3))) bf16x4*)(
                      (__attribute__((address_space(3))) bf16_t*)(d_l + rows + toff[half][db])));
              const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                  (__attribute__((address_space(3))) bf16x4*)(
                      (__attribute__((address_space(3))) bf16_t*)(q_l + rows + toff[half][db])));
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                dt[4 * half + j] = a[j];
                qt[4 * half + j] = b[j];
              }
            }
            dv[db] = Mma<bf16_t>::mma(dt, pf, dv[db]);
            dk[db] = Mma<bf16_t>::mma(qt, dsf, dk[db]);
          }
        }
      }
      if (next_plane) {
#pragma unroll
        for (int k = 0; k < kPosPer; ++k)
          if (tid + 64 * kDW * k < kDRC) pos_l[pb ^ 1][tid + 64 * kDW * k] = np[k];
      }
      __syncthreads();
    }
    pb ^= 1;
  }

  // part 1 leaves its partial sums in the region buffers (free after the
  // last step's barrier); part 0 adds them, always in this order
  f32x4* red_k = reinterpret_cast<f32x4*>(q_l);
  f32x4* red_v = reinterpret_cast<f32x4*>(d_l);
  static_assert(2 * 2 * 4 * 64 * sizeof(f32x4) <= sizeof(q_l), "reduction fits");
  if (part == 1) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int i = ((kw * 2 + db) * 4 + q4) * 64 + lane;
        red_k[i] = f32x4{dk[db][4 * q4], dk[db][4 * q4 + 1], dk[db][4 * q4 + 2], dk[db][4 * q4 + 3]};
        red_v[i] = f32x4{dv[db][4 * q4], dv[db][4 * q4 + 1], dv[db][4 * q4 + 2], dv[db][4 * q4 + 3]};
      }
  }
  __syncthreads();
  if (part == 1 || !kok) return;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int i = ((kw * 2 + db) * 4 + q4) * 64 + lane;
      const f32x4 ek = red_k[i], ev = red_v[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dk[db][4 * q4 + j] += ek[j];
        dv[db][4 * q4 + j] += ev[j];
      }
    }
  // dk_loc = R(c)^T (tau dk^R); pairs (2p, 2p+1) are adjacent elements
  const int kc[3] = {z0, yk, xk};
  bf16_t* ok_ = A.dk + krow * 64;
  bf16_t* ov = A.dv + krow * 64;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = db * 32 + 8 * q4 + 4 * h;
      bf16x4 wk, wv;
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const int pr = (d0 + j) >> 1;
        float sn = 0.0f, cs = 1.0f;
        if (pr < A.rope.npairs) rope_sincos(A.rope.nu[pr], kc[A.rope.axis[pr]], sn, cs);
        const float x0_ = A.tau * dk[db][4 * q4 + j], x1_ = A.tau * dk[db][4 * q4 + j + 1];
        wk[j] = (bf16_t)(cs * x0_ + sn * x1_);
        wk[j + 1] = (bf16_t)(cs * x1_ - sn * x0_);
        wv[j] = (bf16_t)dv[db][4 * q4 + j];
        wv[j + 1] = (bf16_t)dv[db][4 * q4 + j + 1];
      }
      *reinterpret_cast<bf16x4*>(ok_ + d0) = wk;
      *reinterpret_cast<bf16x4*>(ov + d0) = wv;
    }
}

// ---------------------------------------------------------------------------
// k_unrotate: y = R(c)^T x (kRot) or y = x for fp32 x [N, H, 64] -> y of
// type TO (bf16 output, or fp32 in place); 8 lanes per token, lane = 16-byte
// chunk (4 pairs) of every head.
// ---------------------------------------------------------------------------
template <bool kRot, typename TO>
__global__ __launch_bounds__(256) void k_unrotate(const float* x, TO* y, int64_t n,
                                                  int32_t heads,
                                                  const int32_t* __restrict__ coords,
                                                  RopeTab rt) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tok = gid >> 3;
  const int chunk = (int)(gid & 7);
  if (tok >= n) return;
  float sn[4], cs[4];
  if (kRot)
    chunk_sincos(rt, chunk, coords[3 * tok], coords[3 * tok + 1], coords[3 * tok + 2], sn, cs);
  for (int hd = 0; hd < heads; ++hd) {
    float v[8];
    load8<float>(x + (tok * heads + hd) * 64 + chunk * 8, v);
    if (kRot) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = v[2 * i], x1 = v[2 * i + 1];
        v[2 * i] = cs[i] * x0 + sn[i] * x1;
        v[2 * i + 1] = cs[i] * x1 - sn[i] * x0;
      }
    }
    store8<TO>(y + (tok * heads + hd) * 64 + chunk * 8, v);
  }
}

// ---------------------------------------------------------------------------
// k_sum_bwd: dk_cmp[u, g] = a[u, g] R^T sum_s dk~_s[g, j(u)] with R = R(c_u)
// (exact form), R(c^_j) (summary centre) or the identity (blind),
// dv_cmp[u, g] = a[u, g] sum_s dv~_s[g, j(u)] (s = slices of the query
// stream, summed in order); 8 lanes per token, lane = 16-byte chunk.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sum_bwd(const float* __restrict__ dks,
                                                 const float* __restrict__ dvs, int32_t nsplit,
                                                 const float* __restrict__ a,
                                                 const int32_t* __restrict__ coords, Geom g,
                                                 bf16_t* dk, bf16_t* dv) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tok = gid >> 3;
  const int chunk = (int)(gid & 7);
  if (tok >= g.N) return;
  const int z = coords[3 * tok], yy = coords[3 * tok + 1], xx = coords[3 * tok + 2];
  const int64_t j = ((int64_t)(z / g.bz) * (g.Y / g.by) + yy / g.by) * (g.X / g.bx) + xx / g.bx;
  float sn[4], cs[4];
  summary_sincos(g, chunk, z, yy, xx, sn, cs);
  for (int gr = 0; gr < g.Hkv; ++gr) {
    float sk[8] = {}, sv[8] = {};
    for (int s = 0; s < nsplit; ++s) {
      const int64_t off = (((int64_t)s * g.Hkv + gr) * g.M + j) * 64 + chunk * 8;
      float tk[8], tv[8];
      load8<float>(dks + off, tk);
      load8<float>(dvs + off, tv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sk[e] += tk[e];
        sv[e] += tv[e];
      }
    }
    const float w = a ? a[tok * g.Hkv + gr] : 1.0f / (float)g.bvol;
    float ok_[8], ov[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = w * sk[2 * i], x1 = w * sk[2 * i + 1];
      ok_[2 * i] = cs[i] * x0 + sn[i] * x1;
      ok_[2 * i + 1] = cs[i] * x1 - sn[i] * x0;
      ov[2 * i] = w * sv[2 * i];
      ov[2 * i + 1] = w * sv[2 * i + 1];
    }
    store8<bf16_t>(dk + (tok * g.Hkv + gr) * 64 + chunk * 8, ok_);
    store8<bf16_t>(dv + (tok * g.Hkv + gr) * 64 + chunk * 8, ov);
  }
}

template <int G>
static hipError_t launch_loc_dq_g(const Geom& g, const BwdBuffers& b, hipStream_t s) {
  using C = lb::Cfg<G>;
  LdqArgs A;
  A.q = (const bf16_t*)b.q_rot;
  A.k = (const bf16_t*)b.k_rot;
  A.v = (const bf16_t*)b.v_loc;
  A.dlo = (const bf16_t*)b.dlo;
  A.lse = b.lse_loc;
  A.dd = b.d_loc;
  A.c2p = b.c2p;
  A.dq = b.dq_acc;
  A.Z = g.Z;
  A.Y = g.Y;
  A.X = g.X;
  A.hq = g.Hq;
  A.hkv = g.Hkv;
  A.rz = g.rz;
  A.ry = g.ry;
  A.rx = g.rx;
  A.c = g.scale * kLog2e;
  A.tau = g.scale;
  A.tiles_y = (g.Y + C::TY - 1) / C::TY;
  A.tiles_x = (g.X + C::TX - 1) / C::TX;
  A.nblocks = (int64_t)A.tiles_x * A.tiles_y * g.Z * g.Hkv;
  A.per_xcd = (A.nblocks + kNumXcd - 1) / kNumXcd;
  hipLaunchKernelGGL(k_loc_dq<G>, dim3((unsigned)(A.per_xcd * kNumXcd)), dim3(64 * C::W), 0, s,
                     A);
  return hipGetLastError();
}

}  // namespace bw

bool backward_supported(const Geom& g) {
  return g.bf16 && (g.G == 4 || g.G == 8 || g.G == 16) && g.ry <= lb::kHalo &&
         g.rx <= lb::kHalo;
}

int64_t glob_dkv_splits(const Geom& g) {
  // enough workgroups to cover the chip twice, at most one slice per 4096 cells
  const int64_t nkt = (g.M + bw::kKKeys - 1) / bw::kKKeys;
  int64_t s = (2 * 256 + nkt * g.Hkv - 1) / (nkt * g.Hkv);
  const int64_t cap = (g.N + 4095) / 4096;
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

hipError_t launch_backward(const Geom& g, const BwdBuffers& b, hipStream_t s) {
  hipError_t e;
  // 1. per-token prep
  hipLaunchKernelGGL(bw::k_bwd_prep, dim3((unsigned)((g.N + 3) / 4)), dim3(256), 0, s,
                     (const bf16_t*)b.dout, b.o_loc, b.o_cmp, b.gate, b.lse_cmp, g.N, g.Hq,
                     g.gate_per_head, (bf16_t*)b.dlo, (bf16_t*)b.dco, b.d_loc, b.d_cmp, b.nls_cmp,
                     b.dgate);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 2. local dq (first writer of dq_acc), 3. summary dq (adds)
  switch (g.G) {
    case 4: e = bw::launch_loc_dq_g<4>(g, b, s); break;
    case 8: e = bw::launch_loc_dq_g<8>(g, b, s); break;
    case 16: e = bw::launch_loc_dq_g<16>(g, b, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const dim3 tok_grid((unsigned)((g.N * 8 + 255) / 256));
  const bool blind = g.summary_mode == PACK3D_SUMMARY_BLIND;
  if (blind) {
    // the compressed branch saw the unrotated query: un-rotate the local dq
    // first (in place, fp32), then add the summary dq
    hipLaunchKernelGGL((bw::k_unrotate<true, float>), tok_grid, dim3(256), 0, s, b.dq_acc,
                       b.dq_acc, g.N, g.Hq, b.coords, g.rope);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    bw::GdqArgs A;
    A.q = (const bf16_t*)b.q_cmp;
    A.dco = (const bf16_t*)b.dco;
    A.ks = (const bf16_t*)b.k_sum;
    A.vs = (const bf16_t*)b.v_sum;
    A.lse = b.lse_cmp;
    A.ndd = b.d_cmp;
    A.dq = b.dq_acc;
    A.m = g.M;
    A.n = g.N;
    A.hq = g.Hq;
    A.hkv = g.Hkv;
    A.grp = g.G;
    // the summaries carry tau * log2(e): logits need no factor, and
    // sum dS k~ takes tau / (tau log2(e)) to give dq
    A.c = 1.0f;
    A.tau = g.scale / logit_scale(g);
    A.tiles = (g.N * g.G + bw::kGRows - 1) / bw::kGRows;
    int64_t blocks;
    if (g.Hkv <= kNumXcd && kNumXcd % g.Hkv == 0) {
      A.xcd_per = kNumXcd / g.Hkv;
      blocks = (A.tiles + A.xcd_per - 1) / A.xcd_per * kNumXcd;
    } else {
      A.xcd_per = 0;
      blocks = A.tiles * g.Hkv;
    }
    hipLaunchKernelGGL(bw::k_glob_dq, dim3((unsigned)blocks), dim3(64 * bw::kGW), 0, s, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 4. dq = R^T dq_acc (blind: already un-rotated, only rounded to bf16)
  if (blind)
    hipLaunchKernelGGL((bw::k_unrotate<false, bf16_t>), tok_grid, dim3(256), 0, s, b.dq_acc,
                       (bf16_t*)b.dq, g.N, g.Hq, b.coords, g.rope);
  else
    hipLaunchKernelGGL((bw::k_unrotate<true, bf16_t>), tok_grid, dim3(256), 0, s, b.dq_acc,
                       (bf16_t*)b.dq, g.N, g.Hq, b.coords, g.rope);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 5. local dk / dv
  {
    bw::LkvArgs A;
    A.q = (const bf16_t*)b.q_rot;
    A.dlo = (const bf16_t*)b.dlo;
    A.lse = b.lse_loc;
    A.dd = b.d_loc;
    A.k = (const bf16_t*)b.k_rot;
    A.v = (const bf16_t*)b.v_loc;
    A.c2p = b.c2p;
    A.dk = (bf16_t*)b.dk_loc;
    A.dv = (bf16_t*)b.dv_loc;
    A.Z = g.Z;
    A.Y = g.Y;
    A.X = g.X;
    A.hq = g.Hq;
    A.hkv = g.Hkv;
    A.G = g.G;
    A.rz = g.rz;
    A.ry = g.ry;
    A.rx = g.rx;
    A.c = g.scale * kLog2e;
    A.tau = g.scale;
    A.tiles_y = (g.Y + bw::kDTY - 1) / bw::kDTY;
    A.tiles_x = (g.X + bw::kDTX - 1) / bw::kDTX;
    A.nblocks = (int64_t)A.tiles_x * A.tiles_y * g.Z * g.Hkv;
    A.per_xcd = (A.nblocks + kNumXcd - 1) / kNumXcd;
    A.rope = g.rope;
    hipLaunchKernelGGL(bw::k_loc_dkv, dim3((unsigned)(A.per_xcd * kNumXcd)), dim3(64 * bw::kDW),
                       0, s, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 6. summary gradients (partials per slice of the query stream)
  const int64_t nsplit = glob_dkv_splits(g);
  {
    bw::GkvArgs A;
    A.q = (const bf16_t*)b.q_cmp;
    A.dco = (const bf16_t*)b.dco;
    A.ks = (const bf16_t*)b.k_sum;
    A.vs = (const bf16_t*)b.v_sum;
    A.nls = b.nls_cmp;
    A.ndd = b.d_cmp;
    A.c2p = b.c2p;
    A.dk = b.dk_part;
    A.dv = b.dv_part;
    A.m = g.M;
    A.ncell = g.N;
    A.hq = g.Hq;
    A.hkv = g.Hkv;
    A.grp = g.G;
    A.tau = g.scale;
    A.nkt = (g.M + bw::kKKeys - 1) / bw::kKKeys;
    A.nsplit = (int32_t)nsplit;
    A.cps = (g.N + nsplit - 1) / nsplit;
    hipLaunchKernelGGL(bw::k_glob_dkv, dim3((unsigned)(A.nkt * g.Hkv * nsplit)),
                       dim3(64 * bw::kKW), 0, s, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 7. through the block sums and the rotation
  hipLaunchKernelGGL(bw::k_sum_bwd, dim3((unsigned)((g.N * 8 + 255) / 256)), dim3(256), 0, s,
                     b.dk_part, b.dv_part, (int32_t)nsplit, b.a, b.coords, g, (bf16_t*)b.dk_cmp,
                     (bf16_t*)b.dv_cmp);
  return hipGetLastError();
}

}  // namespace pack3d
