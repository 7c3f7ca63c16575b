// Exact local-neighbourhood attention, bf16 kernel for query-group sizes
// G = Hq/Hkv of 4, 8 and 16.
//
// "Geometry Matters in Packed 3D Attention", papernotes.org notes, key
// design 3: the neighbourhood N(i) is a box of lattice coordinates, local K/V
// tiles are streamed through on-chip memory, and no gathered neighbour
// tensor is ever materialised.
//
// A workgroup owns a 1 x TY x TX tile of query cells of one z-plane and one
// KV group, split into patches of 32/G cells (two cells wide); a patch's
// (cell, head) pairs are the 32 columns of an MFMA block, so the G heads of
// the group share every key fragment.  For every z-plane of the window the
// workgroup copies the rotated K and the V rows of the tile plus a 3-cell
// halo into LDS, gathering rows through cell_to_pos (by coordinate) with
// asynchronous global->LDS copies, double-buffered so the next plane's
// copies are in flight while this plane is computed.  A patch treats the
// union of its cells' windows in that plane, for the largest supported
// radius, as a dense 8-wide key set (so all shapes are compile-time):
// S^T = K Q^T and O^T += V^T P^T on 32x32x16 bf16 MFMA, V^T read from the
// row-major tile with the transposing LDS load.  Keys outside a query's
// window or outside the lattice are masked to -inf and an online softmax
// carries the state across planes.  Every reduction order is fixed by
// coordinates, never by packing.
//
// Windows of three planes (z radius 1, the pages' 3 x k x k) use k_local_zrun
// below: the same tiles and arithmetic, walking runs of query planes with a
// ring of three K / V plane slots, one new plane per query plane.
#include "local_tiles.h"

namespace pack3d {

namespace lb {

struct Args {
  const bf16_t* q;         // rotated, or unrotated with qrope.tab
  QRope qrope;
  const bf16_t* k;
  const bf16_t* v;
  const int32_t* c2p;
  float* o;                // fp32 o_loc (nullable)
  float* lse;
  const float* gate;
  bf16_t* out;             // gated share g_loc * o_loc (nullable)
  int32_t gate_per_head;
  int32_t Z, Y, X, hq, hkv;
  int32_t rz, ry, rx;
  float c;                 // scale * log2(e)
  int32_t tiles_y, tiles_x;
  int64_t nblocks;
  int64_t per_xcd;
  int32_t zrun;            // k_local_zrun: query planes per workgroup
};

template <int G>
__global__ __launch_bounds__(64 * Cfg<G>::W) void k_local_bf16(Args A) {
  using C = Cfg<G>;
  constexpr int PY = C::PY, PX = C::PX, TX = C::TX, NKB = C::NKB, KY = C::KY, RX = C::RX,
                RC = C::RC, RCP = C::RCP, RCA = C::RCA, W = C::W, NT = 64 * W;
  // two plane slots, as separate arrays so copies into one are known not to
  // alias reads of the other
  __shared__ __attribute__((aligned(16))) bf16_t k_lds0[RCA * 64];
  __shared__ __attribute__((aligned(16))) bf16_t k_lds1[RCA * 64];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds0[RCA * 64];
  __shared__ __attribute__((aligned(16))) bf16_t v_lds1[RCA * 64];

  // workgroup -> (group, z, tile y, tile x); each XCD takes a contiguous range
  const int64_t bid = blockIdx.x;
  const int64_t lin = (bid % kNumXcd) * A.per_xcd + bid / kNumXcd;
  if (lin >= A.nblocks) return;
  const int tx = (int)(lin % A.tiles_x);
  const int ty = (int)((lin / A.tiles_x) % A.tiles_y);
  const int z0 = (int)((lin / ((int64_t)A.tiles_x * A.tiles_y)) % A.Z);
  const int grp = (int)(lin / ((int64_t)A.tiles_x * A.tiles_y * A.Z));
  const int y0 = ty * C::TY, x0 = tx * TX;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, col = lane & 31;
  const int hh = col % G, cip = col / G, qy = cip / PX, qx = cip % PX;
  const int py0 = (wave / (TX / PX)) * PY, px0 = (wave % (TX / PX)) * PX;

  // Region cells are copied in 1 KB pieces (8 cells): wave w owns pieces
  // w, w + W, ...; lane l of a piece fills cell 8*piece + l/8 at chunk
  // position l%8, which holds data chunk swz(cell, l%8) (the swizzles are
  // involutions).  The packed positions of a plane's cells are gathered
  // into registers one plane ahead of its copies.
  constexpr int NPC = (RCP / 8 + W - 1) / W;   // pieces per wave
  auto load_pos = [&](int zz, int32_t (&pos)[NPC]) {
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int cell = (wave + W * i) * 8 + (lane >> 3);
      const int yy = y0 - kHalo + cell / RX, xx = x0 - kHalo + cell % RX;
      // off the lattice (or past the region): token 0, finite and masked
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
        __builtin_amdgcn_global_load_lds((const void*)(kg + row + kv_swz(cell / RX, cell % RX, cp) * 8),
                                         (lds_ptr)(kl + pc * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vg + row + kv_swz(cell / RX, cell % RX, cp) * 8),
                                         (lds_ptr)(vl + pc * 512), 16, 0, 0);
      }
    }
  };

  // this lane's query column
  const int yq = y0 + py0 + qy, xq = x0 + px0 + qx;
  const bool qok = yq < A.Y && xq < A.X;
  const int64_t qpos = qok ? (int64_t)A.c2p[((int64_t)z0 * A.Y + yq) * A.X + xq] : -1;
  QFrag<bf16_t> qf;
  load_qfrag<bf16_t>(qf, A.q + (qpos * A.hq + grp * G + hh) * 64 + h * 32, qok);
  // unrotated query: rotate it here (lanes past the lattice hold zeros and
  // read the table at a cell inside it)
  if (A.qrope.tab) rotate_qfrag<bf16_t>(qf, A.qrope, h, z0, qok ? yq : 0, qok ? xq : 0);

  // Window mask.  Key slot s of the patch is region cell (py0 + s/8, px0 +
  // s%8); accumulator element e of 32-key block kb on lane half h is slot
  // kb*32 + 8*(e/4) + 4h + e%4, i.e. key row 4kb + e/4 and key column
  // 4h + e%4.  The key is valid iff its row and its column are.
  bool rv[NKB * 4], cv[4];
#pragma unroll
  for (int r = 0; r < NKB * 4; ++r) {
    const int dy = r - kHalo - qy, yk = y0 + py0 + r - kHalo;
    rv[r] = r < KY && dy >= -A.ry && dy <= A.ry && yk >= 0 && yk < A.Y;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int kx = 4 * h + c, dx = kx - kHalo - qx, xk = x0 + px0 + kx - kHalo;
    cv[c] = dx >= -A.rx && dx <= A.rx && xk >= 0 && xk < A.X;
  }

  f32x16 o0 = {}, o1 = {};
  SoftmaxState sm;
  sm.m = kNegInf;
  sm.l = 0.0f;

  // LDS element offsets of this lane's operand rows within a slot
  // + 4*RX cells per key block (4 rows: the row parity, hence the swizzle, stays)
  const int ky0 = py0 + col / 8, kx0 = px0 + col % 8, kcell = ky0 * RX + kx0;
  int koff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) koff[st] = kcell * 64 + kv_swz(ky0, kx0, h * 4 + st) * 8;
  const int r4 = lane & 15;
  int voff[2][2];   // [half][dim block]; + (4*kb + 2t)*RX cells per PV step
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int vy = py0 + half, vx = px0 + 4 * h + (r4 >> 2), cell = vy * RX + vx;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int dim = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (r4 & 3);
      voff[half][db] = cell * 64 + kv_swz(vy, vx, dim >> 3) * 8 + (dim & 7);
    }
  }

  auto compute_plane = [&](const bf16_t* kl, const bf16_t* vl) {
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      KFrag<bf16_t> kf;
#pragma unroll
      for (int st = 0; st < 4; ++st)
        kf.f[st] = *reinterpret_cast<const bf16x8*>(kl + 4 * RX * 64 * kb + koff[st]);
      s[kb] = qk_tile<bf16_t>(kf, qf);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (!(rv[4 * kb + e / 4] && cv[e % 4])) s[kb][e] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    const float mt = pair_max(mx) * A.c;
    const bool upd = mt > sm.m + kRescaleSlack;
    if (__any(upd)) {
      const float mn = upd ? mt : sm.m;
      const float alpha = upd ? __builtin_amdgcn_exp2f(sm.m - mn) : 1.0f;
      sm.m = mn;
      sm.l *= alpha;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        o0[e] *= alpha;
        o1[e] *= alpha;
      }
    }
    const float mu = sm.m == kNegInf ? 0.0f : sm.m;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (4 * kb + 2 * t >= KY) continue;   // both key rows are padding: P = 0
        f32x16 pr;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pr[8 * t + e] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * t + e], A.c, -mu));
        const bf16x8 pf = Mma<bf16_t>::p_frag(pr, t);
        sm.l = frag_sum(pf, sm.l);
        const bf16_t* vrows = vl + (4 * kb + 2 * t) * RX * 64;
        bf16x8 vf[2];
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const bf16x4 part = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(
                    (__attribute__((address_space(3))) bf16_t*)(vrows + voff[half][db])));
#pragma unroll
            for (int j = 0; j < 4; ++j) vf[db][4 * half + j] = part[j];
          }
        o0 = Mma<bf16_t>::mma(vf[0], pf, o0);
        o1 = Mma<bf16_t>::mma(vf[1], pf, o1);
      }
    }
  };

  // planes of the window inside the lattice (z0 itself always is)
  const int zlo = z0 - A.rz < 0 ? 0 : z0 - A.rz;
  const int zhi = z0 + A.rz >= A.Z ? A.Z - 1 : z0 + A.rz;
  const int np = zhi - zlo + 1;

  // zero the rows past the copied region once (they stay untouched)
  for (int i = RCP * 8 + tid; i < RCA * 8; i += NT) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    st16(k_lds0 + 8 * i, z);
    st16(k_lds1 + 8 * i, z);
    st16(v_lds0 + 8 * i, z);
    st16(v_lds1 + 8 * i, z);
  }
  int32_t pos_a[NPC], pos_b[NPC];   // positions of the next two planes
  load_pos(zlo, pos_a);
  __builtin_amdgcn_s_waitcnt(0);
  issue_loads(pos_a, k_lds0, v_lds0);
  if (np > 1) load_pos(zlo + 1, pos_a);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // plane p lives in slot p & 1; while it is computed the next plane's copies
  // are in flight into the other slot and the positions of plane p + 2 are
  // being gathered
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

  const float l = pair_sum(sm.l);
  if (qpos < 0) return;
  const float inv = 1.0f / l;
  const int head = grp * G + hh;
  const int64_t rbase = (qpos * A.hq + head) * 64;
  if (A.lse && h == 0) A.lse[qpos * A.hq + head] = (sm.m + __log2f(l)) * kLn2;
  float g0 = 0.0f, g1 = 0.0f;
  if (A.out) gate_weights(A.gate, qpos, head, A.hq, A.gate_per_head, g0, g1);
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    f32x4 r0, r1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r0[j] = o0[4 * q4 + j] * inv;
      r1[j] = o1[4 * q4 + j] * inv;
    }
    const int64_t a0 = rbase + 8 * q4 + 4 * h, a1 = a0 + 32;
    if (A.o) {
      *reinterpret_cast<f32x4*>(A.o + a0) = r0;
      *reinterpret_cast<f32x4*>(A.o + a1) = r1;
    }
    if (A.out) {
      store_gated4<bf16_t>(A.out + a0, r0, g0);
      store_gated4<bf16_t>(A.out + a1, r1, g0);
    }
  }
}

// ---------------------------------------------------------------------------
// k_local_zrun: the tile, patches, masks and per-plane arithmetic of
// k_local_bf16, for windows of three planes (z radius 1).  A
// workgroup walks a run of consecutive query planes of its (y, x) tile.  The
// K / V planes live in a ring of three LDS slots: while query plane z is
// computed against planes z - 1, z, z + 1, plane z + 2 is copied into the
// slot plane z - 1 leaves once it has been used (first in the window), so
// each query plane brings one new plane instead of three, and its copies
// overlap three planes of compute.  The planes are visited in the same order
// as in k_local_bf16, so the results are the same bit for bit.
// ---------------------------------------------------------------------------
// kRot: the query is unrotated; its fragments are rotated through A.qrope.
template <int G, bool kRot>
__global__ __launch_bounds__(64 * Cfg<G>::W) void k_local_zrun(Args A) {
  using C = Cfg<G>;
  constexpr int PY = C::PY, PX = C::PX, TX = C::TX, NKB = C::NKB, KY = C::KY, RX = C::RX,
                RC = C::RC, RCP = C::RCP, RCA = C::RCA, W = C::W, NT = 64 * W;
  // three plane slots per operand, as separate arrays so the copies into one
  // are known not to alias the reads of another; K slots hold RCA cells (the
  // key blocks read that far), V slots the RC region cells
  __shared__ __attribute__((aligned(16))) bf16_t k_l0[RCA * 64];
  __shared__ __attribute__((aligned(16))) bf16_t k_l1[RCA * 64];
  __shared__ __attribute__((aligned(16))) bf16_t k_l2[RCA * 64];
  __shared__ __attribute__((aligned(16))) bf16_t v_l0[RC * 64];
  __shared__ __attribute__((aligned(16))) bf16_t v_l1[RC * 64];
  __shared__ __attribute__((aligned(16))) bf16_t v_l2[RC * 64];

  // workgroup -> (group, run of planes, tile y, tile x); each XCD takes a
  // contiguous range
  const int64_t bid = blockIdx.x;
  const int64_t lin = (bid % kNumXcd) * A.per_xcd + bid / kNumXcd;
  if (lin >= A.nblocks) return;
  const int nruns = (A.Z + A.zrun - 1) / A.zrun;
  const int tx = (int)(lin % A.tiles_x);
  const int ty = (int)((lin / A.tiles_x) % A.tiles_y);
  const int run = (int)((lin / ((int64_t)A.tiles_x * A.tiles_y)) % nruns);
  const int grp = (int)(lin / ((int64_t)A.tiles_x * A.tiles_y * nruns));
  const int zs = run * A.zrun, ze = zs + A.zrun < A.Z ? zs + A.zrun : A.Z;
  const int y0 = ty * C::TY, x0 = tx * TX;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, col = lane & 31;
  const int hh = col % G, cip = col / G, qy = cip / PX, qx = cip % PX;
  const int py0 = (wave / (TX / PX)) * PY, px0 = (wave % (TX / PX)) * PX;

  // copies in 1 KB pieces of 8 region cells, as in k_local_bf16; V lanes
  // past the region cells copy nothing (V slots hold RC cells)
  constexpr int NPC = (RCP / 8 + W - 1) / W;
  auto load_pos = [&](int zz, int32_t (&pos)[NPC]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int cell = (wave + W * i) * 8 + (lane >> 3);
      const int yy = y0 - kHalo + cell / RX, xx = x0 - kHalo + cell % RX;
      // 32-bit cell index (lattices hold < 2^31 cells): base + offset
      // addressing, nothing 64-bit to keep live across the run
      pos[i] = cell < RC && yy >= 0 && yy < A.Y && xx >= 0 && xx < A.X
                   ? A.c2p[(uint32_t)((zz * A.Y + yy) * A.X + xx)]
                   : 0;
    }
  };
  const bf16_t* kg = A.k + (int64_t)grp * 64;
  const bf16_t* vg = A.v + (int64_t)grp * 64;
  const int64_t rstride = (int64_t)A.hkv * 64;
  auto issue_loads = [&](const int32_t (&pos)[NPC], bf16_t* __restrict__ kl,
                         bf16_t* __restrict__ vl) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int pc = wave + W * i;
      if (pc < RCP / 8) {
        const int cell = pc * 8 + (lane >> 3), cp = lane & 7;
        const int64_t row = (int64_t)pos[i] * rstride;
        __builtin_amdgcn_global_load_lds((const void*)(kg + row + kv_swz(cell / RX, cell % RX, cp) * 8),
                                         (lds_ptr)(kl + pc * 512), 16, 0, 0);
        if (cell < RC)
          __builtin_amdgcn_global_load_lds((const void*)(vg + row + kv_swz(cell / RX, cell % RX, cp) * 8),
                                           (lds_ptr)(vl + pc * 512), 16, 0, 0);
      }
    }
  };

  // this lane's query column: (yq, xq) of every plane of the run
  const int yq = y0 + py0 + qy, xq = x0 + px0 + qx;
  const bool qok = yq < A.Y && xq < A.X;
  const int yc = qok ? yq : 0, xc = qok ? xq : 0;     // in-lattice table coordinates
  const uint32_t rab = qrope_lane_axes(A.qrope, h);
  const uint32_t qcell = qok ? (uint32_t)(yq * A.X + xq) : 0u;
  const uint32_t plane_cells = (uint32_t)(A.Y * A.X);
  const bf16_t* qg = A.q + (int64_t)(grp * G + hh) * 64 + h * 32;
  auto qrow = [&](int32_t pos) __attribute__((always_inline)) { return qg + (int64_t)pos * A.hq * 64; };

  // window mask (as in k_local_bf16)
  bool rv[NKB * 4], cv[4];
#pragma unroll
  for (int r = 0; r < NKB * 4; ++r) {
    const int dy = r - kHalo - qy, yk = y0 + py0 + r - kHalo;
    rv[r] = r < KY && dy >= -A.ry && dy <= A.ry && yk >= 0 && yk < A.Y;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int kx = 4 * h + c, dx = kx - kHalo - qx, xk = x0 + px0 + kx - kHalo;
    cv[c] = dx >= -A.rx && dx <= A.rx && xk >= 0 && xk < A.X;
  }

  const int ky0 = py0 + col / 8, kx0 = px0 + col % 8, kcell = ky0 * RX + kx0;
  int koff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) koff[st] = kcell * 64 + kv_swz(ky0, kx0, h * 4 + st) * 8;
  const int r4 = lane & 15;
  int voff[2][2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int vy = py0 + half, vx = px0 + 4 * h + (r4 >> 2), cell = vy * RX + vx;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int dim = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (r4 & 3);
      voff[half][db] = cell * 64 + kv_swz(vy, vx, dim >> 3) * 8 + (dim & 7);
    }
  }

  QFrag<bf16_t> qf, qf_n;
  f32x16 o0 = {}, o1 = {};
  SoftmaxState sm;
  sm.m = kNegInf;
  sm.l = 0.0f;

  auto compute_plane = [&](const QFrag<bf16_t>& qf, const bf16_t* __restrict__ kl,
                           const bf16_t* __restrict__ vl) __attribute__((always_inline)) {
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      KFrag<bf16_t> kf;
#pragma unroll
      for (int st = 0; st < 4; ++st)
        kf.f[st] = *reinterpret_cast<const bf16x8*>(kl + 4 * RX * 64 * kb + koff[st]);
      s[kb] = qk_tile<bf16_t>(kf, qf);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (!(rv[4 * kb + e / 4] && cv[e % 4])) s[kb][e] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    const float mt = pair_max(mx) * A.c;
    const bool upd = mt > sm.m + kRescaleSlack;
    if (__any(upd)) {
      const float mn = upd ? mt : sm.m;
      const float alpha = upd ? __builtin_amdgcn_exp2f(sm.m - mn) : 1.0f;
      sm.m = mn;
      sm.l *= alpha;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        o0[e] *= alpha;
        o1[e] *= alpha;
      }
    }
    const float mu = sm.m == kNegInf ? 0.0f : sm.m;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (4 * kb + 2 * t >= KY) continue;   // both key rows are padding: P = 0
        f32x16 pr;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pr[8 * t + e] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * t + e], A.c, -mu));
        const bf16x8 pf = Mma<bf16_t>::p_frag(pr, t);
        sm.l = frag_sum(pf, sm.l);
        const bf16_t* vrows = vl + (4 * kb + 2 * t) * RX * 64;
        bf16x8 vf[2];
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const bf16x4 part = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(
                    (__attribute__((address_space(3))) bf16_t*)(vrows + voff[half][db])));
#pragma unroll
            for (int j = 0; j < 4; ++j) vf[db][4 * half + j] = part[j];
          }
        o0 = Mma<bf16_t>::mma(vf[0], pf, o0);
        o1 = Mma<bf16_t>::mma(vf[1], pf, o1);
      }
    }
  };

  auto finish = [&](int32_t qpos) __attribute__((always_inline)) {
    const float l = pair_sum(sm.l);
    if (qok) {
      const float inv = 1.0f / l;
      const int head = grp * G + hh;
      const int64_t rbase = ((int64_t)qpos * A.hq + head) * 64;
      if (A.lse && h == 0) A.lse[(int64_t)qpos * A.hq + head] = (sm.m + __log2f(l)) * kLn2;
      float g0 = 0.0f, g1 = 0.0f;
      if (A.out) gate_weights(A.gate, qpos, head, A.hq, A.gate_per_head, g0, g1);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 r0, r1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          r0[j] = o0[4 * q4 + j] * inv;
          r1[j] = o1[4 * q4 + j] * inv;
        }
        const int64_t a0 = rbase + 8 * q4 + 4 * h, a1 = a0 + 32;
        if (A.o) {
          *reinterpret_cast<f32x4*>(A.o + a0) = r0;
          *reinterpret_cast<f32x4*>(A.o + a1) = r1;
        }
        if (A.out) {
          store_gated4<bf16_t>(A.out + a0, r0, g0);
          store_gated4<bf16_t>(A.out + a1, r1, g0);
        }
      }
    }
    o0 = f32x16{};
    o1 = f32x16{};
    sm.m = kNegInf;
    sm.l = 0.0f;
  };

  // K rows past the copied cells are read by the last key block and always
  // masked; zero them once so they hold finite values
  for (int i = RCP * 8 + tid; i < RCA * 8; i += NT) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    st16(k_l0 + 8 * i, z);
    st16(k_l1 + 8 * i, z);
    st16(k_l2 + 8 * i, z);
  }

  // prologue: planes zs - 1, zs, zs + 1 into slots 0, 1, 2
  int32_t pos_n[NPC];
  {
    int32_t p0[NPC], p1[NPC], p2[NPC];
    if (zs > 0) load_pos(zs - 1, p0);
    load_pos(zs, p1);
    if (zs + 1 < A.Z) load_pos(zs + 1, p2);
    __builtin_amdgcn_s_waitcnt(0);
    if (zs > 0) issue_loads(p0, k_l0, v_l0);
    issue_loads(p1, k_l1, v_l1);
    if (zs + 1 < A.Z) issue_loads(p2, k_l2, v_l2);
  }
  if (zs + 2 < A.Z && zs + 1 < ze) load_pos(zs + 2, pos_n);
  // query positions one plane ahead of their fragments
  int32_t qpos = A.c2p[(uint32_t)zs * plane_cells + qcell];
  int32_t qpos_n = A.c2p[(uint32_t)(zs + 1 < A.Z ? zs + 1 : zs) * plane_cells + qcell];
  __builtin_amdgcn_s_waitcnt(0);
  load_qfrag<bf16_t>(qf, qrow(qpos), qok);
  if constexpr (kRot) rotate_qfrag<bf16_t>(qf, A.qrope, h, zs, yc, xc);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // query plane z0 = zs + j with j = 3i + R: planes z0 - 1, z0, z0 + 1 sit in
  // slots R, R + 1, R + 2 (mod 3); plane z0 + 2 goes into slot R.  The next
  // query plane's fragments are loaded at the start of a step and have
  // landed by its barrier; the plane copies issued after the barrier are
  // waited for only at the next step's barrier.
  auto step = [&](int z0, bf16_t* __restrict__ ka, bf16_t* __restrict__ va,
                  bf16_t* __restrict__ kb_, bf16_t* __restrict__ vb, bf16_t* __restrict__ kc,
                  bf16_t* __restrict__ vc) __attribute__((always_inline)) {
    if (z0 + 1 < ze) load_qfrag<bf16_t>(qf_n, qrow(qpos_n), qok);
    // unconditional (a plane past the run reads the last one, unused): no
    // branch that would pin the load's use next to it
    const int zq = z0 + 2 < A.Z ? z0 + 2 : A.Z - 1;
    const int32_t qpos_nn = A.c2p[(uint32_t)zq * plane_cells + qcell];
    if (z0 > 0) compute_plane(qf, ka, va);
    // the copies of plane z0 + 1 have landed; every wave is done with slot R
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // unrotated queries: rotate the next plane's fragments (landed at the
    // barrier) before this step's plane copies are issued, so waiting for
    // the table reads never waits for the copies (a plane past the lattice
    // reads the last one's (sin, cos), unused)
    if constexpr (kRot) {
      QRopeCS rcs;
      qrope_load(rcs, A.qrope, rab, h, z0 + 1 < A.Z ? z0 + 1 : z0, yc, xc);
      qrope_apply<bf16_t>(qf_n, rcs);
      // keep the rotation (and its wait) ahead of the copies: an empty asm
      // that takes the rotated fragments pins their computation here
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 w = __builtin_bit_cast(u32x4, qf_n.f[q]);
        asm volatile("" : "+v"(w));
        qf_n.f[q] = __builtin_bit_cast(bf16x8, w);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (z0 + 2 < A.Z && z0 + 1 < ze) issue_loads(pos_n, ka, va);
    if (z0 + 3 < A.Z && z0 + 2 < ze) load_pos(z0 + 3, pos_n);
    compute_plane(qf, kb_, vb);
    if (z0 + 1 < A.Z) compute_plane(qf, kc, vc);
    finish(qpos);
    qf = qf_n;
    qpos = qpos_n;
    qpos_n = qpos_nn;
  };
  for (int z0 = zs; z0 < ze; z0 += 3) {
    step(z0, k_l0, v_l0, k_l1, v_l1, k_l2, v_l2);
    if (z0 + 1 >= ze) break;
    step(z0 + 1, k_l1, v_l1, k_l2, v_l2, k_l0, v_l0);
    if (z0 + 2 >= ze) break;
    step(z0 + 2, k_l2, v_l2, k_l0, v_l0, k_l1, v_l1);
  }
}

template <int G>
hipError_t launch(const Geom& g, const void* q, const void* k, const void* v, const int32_t* c2p,
                  const LocalOut& lo, const QRope& qr, hipStream_t s) {
  using C = Cfg<G>;
  Args A;
  A.q = (const bf16_t*)q;
  A.qrope = qr;
  A.k = (const bf16_t*)k;
  A.v = (const bf16_t*)v;
  A.c2p = c2p;
  A.o = lo.o_loc;
  A.lse = lo.lse;
  A.gate = lo.gate;
  A.out = (bf16_t*)lo.out;
  A.gate_per_head = g.gate_per_head;
  A.Z = g.Z;
  A.Y = g.Y;
  A.X = g.X;
  A.hq = g.Hq;
  A.hkv = g.Hkv;
  A.rz = g.rz;
  A.ry = g.ry;
  A.rx = g.rx;
  A.c = g.scale * kLog2e;
  A.tiles_y = (g.Y + C::TY - 1) / C::TY;
  A.tiles_x = (g.X + C::TX - 1) / C::TX;
  if (g.rz == 1) {
    // runs of planes: about 1 024 workgroups (one per CU at a time), runs
    // of at least 4 planes
    const int64_t cols = (int64_t)A.tiles_x * A.tiles_y * g.Hkv;
    int64_t nruns = (1024 + cols - 1) / cols;
    if (nruns > (g.Z + 3) / 4) nruns = (g.Z + 3) / 4;
    if (nruns < 1) nruns = 1;
    A.zrun = (int32_t)((g.Z + nruns - 1) / nruns);
    nruns = (g.Z + A.zrun - 1) / A.zrun;
    A.nblocks = cols * nruns;
    A.per_xcd = (A.nblocks + kNumXcd - 1) / kNumXcd;
    if (qr.tab)
      hipLaunchKernelGGL((k_local_zrun<G, true>), dim3((unsigned)(A.per_xcd * kNumXcd)),
                         dim3(64 * C::W), 0, s, A);
    else
      hipLaunchKernelGGL((k_local_zrun<G, false>), dim3((unsigned)(A.per_xcd * kNumXcd)),
                         dim3(64 * C::W), 0, s, A);
    return hipGetLastError();
  }
  A.zrun = 1;
  A.nblocks = (int64_t)A.tiles_x * A.tiles_y * g.Z * g.Hkv;
  A.per_xcd = (A.nblocks + kNumXcd - 1) / kNumXcd;
  hipLaunchKernelGGL(k_local_bf16<G>, dim3((unsigned)(A.per_xcd * kNumXcd)), dim3(64 * C::W), 0,
                     s, A);
  return hipGetLastError();
}

}  // namespace lb

bool local_bf16_serves(int G) { return G == 4 || G == 8 || G == 16; }

hipError_t launch_local_attn_bf16(const Geom& g, const void* q, const void* k_rot,
                                  const void* v, const int32_t* c2p, const LocalOut& lo,
                                  const QRope& qr, hipStream_t s) {
  switch (g.G) {
    case 4: return lb::launch<4>(g, q, k_rot, v, c2p, lo, qr, s);
    case 8: return lb::launch<8>(g, q, k_rot, v, c2p, lo, qr, s);
    case 16: return lb::launch<16>(g, q, k_rot, v, c2p, lo, qr, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pack3d
