// Exact local-neighbourhood attention over a coordinate-defined box window.
//
// "Geometry Matters in Packed 3D Attention", papernotes.org notes, key
// design 3: the neighbourhood N(i) is defined by lattice coordinates, never
// by packed-index windows, and local K/V tiles are streamed through on-chip
// memory so no gathered neighbour tensor is ever materialised.
//
// Design (gfx950): a workgroup owns a 1 x 8 x 8 tile of query cells of one
// z-plane and one KV group.  The tile is split into patches of 32/G cells;
// a patch's (cell, head) pairs are the 32 columns of one MFMA column block,
// so the G heads of the group share every key fragment.  For each z-offset
// of the window the workgroup stages the rotated K (row-major, swizzled) and
// V (transposed) of the tile plus its y/x halo in LDS, reading rows through
// cell_to_pos, i.e. by coordinate.  Each patch then treats the union of its
// cells' windows in that plane as a dense key set (masked-dense MFMA: S^T =
// K Q^T, O^T += V^T P^T), with the out-of-window and out-of-lattice keys
// masked to -inf; an online softmax carries the state across z-offsets.
// Every reduction order is fixed by coordinates, never by packing.
#include "pack3d_device.h"

namespace pack3d {

constexpr int kTile = 8;                 // tile is 1 x kTile x kTile cells
constexpr int kMaxR = 3;                 // max y/x window radius
constexpr int kRegionCells = (kTile + 2 * kMaxR) * (kTile + 2 * kMaxR + 2);  // 14 x 16
constexpr int kVtPitch = kRegionCells + 4;

template <int G> struct Patch;           // (PY, PX): 32/G cells
template <> struct Patch<1> { static constexpr int PY = 4, PX = 8; };
template <> struct Patch<2> { static constexpr int PY = 4, PX = 4; };
template <> struct Patch<4> { static constexpr int PY = 4, PX = 2; };
template <> struct Patch<8> { static constexpr int PY = 2, PX = 2; };
template <> struct Patch<16> { static constexpr int PY = 1, PX = 2; };

template <int G>
struct LCfg {
  static constexpr int PY = Patch<G>::PY, PX = Patch<G>::PX;
  static constexpr int NP = kTile * kTile / (PY * PX);              // patches per tile = 2G
  static constexpr int W = NP < 8 ? NP : 8;                          // waves
  static constexpr int CBW = NP / W;                                 // patches per wave
  static constexpr int KXMAX = (PX + 2 * kMaxR + 3) / 4 * 4;
  static constexpr int KYMAX = PY + 2 * kMaxR;
  static constexpr int NKB = (KYMAX * KXMAX + 31) / 32;              // key blocks per plane
  static constexpr int MWORDS = (NKB * 16 + 31) / 32;
};

template <typename T>
struct LArgs {
  const T* q;              // rotated, or unrotated with qrope.tab
  QRope qrope;
  const T* k;
  const T* v;
  const int32_t* c2p;
  float* o;
  float* lse;
  const float* gate;
  T* out;
  int32_t gate_per_head;
  int32_t Z, Y, X, hq, hkv;
  int32_t rz, ry, rx;
  float c;                 // scale * log2(e)
  int32_t tiles_y, tiles_x;
  int64_t nblocks;         // real workgroups (before XCD padding)
  int64_t per_xcd;
};

template <typename T, int G>
__global__ __launch_bounds__(64 * LCfg<G>::W) void k_local_attn(LArgs<T> A) {
  using C = LCfg<G>;
  constexpr int PY = C::PY, PX = C::PX, CBW = C::CBW, NKB = C::NKB;
  constexpr int NT = 64 * C::W;
  constexpr int E = 16 / sizeof(T);
  __shared__ __attribute__((aligned(16))) T k_lds[kRegionCells * 64];
  __shared__ __attribute__((aligned(16))) T v_lds[64 * kVtPitch];

  // workgroup -> (group, z, tile y, tile x): each XCD gets a contiguous range
  const int64_t bid = blockIdx.x;
  const int64_t lin = (bid % kNumXcd) * A.per_xcd + bid / kNumXcd;
  if (lin >= A.nblocks) return;
  const int tx = (int)(lin % A.tiles_x);
  const int ty = (int)((lin / A.tiles_x) % A.tiles_y);
  const int z0 = (int)((lin / ((int64_t)A.tiles_x * A.tiles_y)) % A.Z);
  const int grp = (int)(lin / ((int64_t)A.tiles_x * A.tiles_y * A.Z));
  const int y0 = ty * kTile, x0 = tx * kTile;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, col = lane & 31;
  const int ry = A.ry, rx = A.rx;
  const int KX = (PX + 2 * rx + 3) / 4 * 4;       // slots per key row (multiple of 4)
  const int KY = PY + 2 * ry;
  const int nslots = KY * KX;
  const int RX = kTile - PX + KX;                  // region width (even)
  const int RY = kTile + 2 * ry;
  const int nkb = (nslots + 31) / 32;
  const int cell_in_patch = col / G, hh = col % G;
  const int qy = cell_in_patch / PX, qx = cell_in_patch % PX;

  QFrag<T> qf[CBW];
  int64_t qpos[CBW];
  int py0[CBW], px0[CBW];
  uint32_t mbits[CBW][C::MWORDS];
#pragma unroll
  for (int cb = 0; cb < CBW; ++cb) {
    const int pi = wave * CBW + cb;
    py0[cb] = (pi / (kTile / PX)) * PY;
    px0[cb] = (pi % (kTile / PX)) * PX;
    const int yq = y0 + py0[cb] + qy, xq = x0 + px0[cb] + qx;
    const bool ok = yq < A.Y && xq < A.X;
    qpos[cb] = ok ? (int64_t)A.c2p[((int64_t)z0 * A.Y + yq) * A.X + xq] : -1;
    load_qfrag<T>(qf[cb], A.q + (qpos[cb] * A.hq + grp * G + hh) * 64 + h * 32, ok);
    if (A.qrope.tab) rotate_qfrag<T>(qf[cb], A.qrope, h, z0, ok ? yq : 0, ok ? xq : 0);
    // window and lattice mask of each (key block, accumulator element)
#pragma unroll
    for (int w = 0; w < C::MWORDS; ++w) mbits[cb][w] = 0;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int slot = kb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        const int ky = slot / KX, kx = slot % KX;
        const int yk = y0 - ry + py0[cb] + ky, xk = x0 - rx + px0[cb] + kx;
        const bool in = kb < nkb && (unsigned)(ky - qy) <= (unsigned)(2 * ry) &&
                        (unsigned)(kx - qx) <= (unsigned)(2 * rx) && yk >= 0 && yk < A.Y &&
                        xk >= 0 && xk < A.X;
        if (in) mbits[cb][(kb * 16 + v) >> 5] |= 1u << ((kb * 16 + v) & 31);
      }
  }

  f32x16 o[CBW][2];
  SoftmaxState sm[CBW];
#pragma unroll
  for (int cb = 0; cb < CBW; ++cb) {
    o[cb][0] = f32x16{};
    o[cb][1] = f32x16{};
    sm[cb].m = kNegInf;
    sm[cb].l = 0.0f;
  }

  const T* kg = A.k + (int64_t)grp * 64;
  const T* vg = A.v + (int64_t)grp * 64;
  const int64_t rstride = (int64_t)A.hkv * 64;

  for (int dz = -A.rz; dz <= A.rz; ++dz) {
    const int zz = z0 + dz;
    if (zz < 0 || zz >= A.Z) continue;
    // stage the plane's region: K rows (swizzled) and V transposed
    const int nch = RY * RX * (64 / E);
    for (int idx = tid; idx < nch; idx += NT) {
      const int cell = idx / (64 / E), ch = idx % (64 / E);
      const int yy = y0 - ry + cell / RX, xx = x0 - rx + cell % RX;
      u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (yy >= 0 && yy < A.Y && xx >= 0 && xx < A.X) {
        const int64_t pos = A.c2p[((int64_t)zz * A.Y + yy) * A.X + xx];
        kv = ld16(kg + pos * rstride + ch * E);
        vv = ld16(vg + pos * rstride + ch * E);
      }
      st16(k_lds + KLds<T>::chunk_off(cell, ch), kv);
      const T* e = reinterpret_cast<const T*>(&vv);
#pragma unroll
      for (int i = 0; i < E; ++i) v_lds[(ch * E + i) * kVtPitch + cell] = e[i];
    }
    __syncthreads();

#pragma unroll
    for (int cb = 0; cb < CBW; ++cb) {
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if (kb < nkb) {
          const int slot = kb * 32 + col;
          const int cell = slot < nslots ? (py0[cb] + slot / KX) * RX + px0[cb] + slot % KX : 0;
          KFrag<T> kf;
          load_kfrag<T>(kf, k_lds, cell, h);
          s[kb] = qk_tile<T>(kf, qf[cb]);
        } else {
          s[kb] = f32x16{};
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int bit = kb * 16 + v;
          if (!((mbits[cb][bit >> 5] >> (bit & 31)) & 1u)) s[kb][v] = kNegInf;
        }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
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
      for (int kb = 0; kb < NKB; ++kb) {
        if (kb >= nkb) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][v], A.c, -mu));
          s[kb][v] = p;
          sm[cb].l += p;
        }
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int dim = db * 32 + col;
#pragma unroll
          for (int st = 0; st < Mma<T>::kPvSteps; ++st) {
            typename Mma<T>::frag vf;
            if constexpr (std::is_same<T, float>::value) {
              const int slot = kb * 32 + Mma<T>::kr(st, 0, h);
              const int cell =
                  slot < nslots ? (py0[cb] + slot / KX) * RX + px0[cb] + slot % KX : 0;
              vf = v_lds[dim * kVtPitch + cell];
            } else {
#pragma unroll
              for (int half = 0; half < 2; ++half) {
                const int slot = kb * 32 + 16 * st + 8 * half + 4 * h;
                const int cell =
                    slot < nslots ? (py0[cb] + slot / KX) * RX + px0[cb] + slot % KX : 0;
                const bf16x2 a = *reinterpret_cast<const bf16x2*>(v_lds + dim * kVtPitch + cell);
                const bf16x2 b =
                    *reinterpret_cast<const bf16x2*>(v_lds + dim * kVtPitch + cell + 2);
                vf[4 * half + 0] = a[0];
                vf[4 * half + 1] = a[1];
                vf[4 * half + 2] = b[0];
                vf[4 * half + 3] = b[1];
              }
            }
            o[cb][db] = Mma<T>::mma(vf, Mma<T>::p_frag(s[kb], st), o[cb][db]);
          }
        }
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int cb = 0; cb < CBW; ++cb) {
    const float l = sm[cb].l + __shfl_xor(sm[cb].l, 32);
    if (qpos[cb] < 0) continue;
    const float inv = 1.0f / l;
    const int head = grp * G + hh;
    const int64_t rbase = (qpos[cb] * A.hq + head) * 64;
    if (A.lse && h == 0) A.lse[qpos[cb] * A.hq + head] = (sm[cb].m + __log2f(l)) * kLn2;
    float g0 = 0.0f, g1 = 0.0f;
    if (A.out) gate_weights(A.gate, qpos[cb], head, A.hq, A.gate_per_head, g0, g1);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = o[cb][db][4 * q4 + j] * inv;
        const int64_t at = rbase + db * 32 + 8 * q4 + 4 * h;
        if (A.o) *reinterpret_cast<f32x4*>(A.o + at) = r;
        if (A.out) store_gated4<T>(A.out + at, r, g0);
      }
  }
}

template <typename T, int G>
static hipError_t launch_l(const Geom& g, const void* q, const void* k, const void* v,
                           const int32_t* c2p, const LocalOut& lo, const QRope& qr,
                           hipStream_t s) {
  LArgs<T> A;
  A.q = (const T*)q;
  A.qrope = qr;
  A.k = (const T*)k;
  A.v = (const T*)v;
  A.c2p = c2p;
  A.o = lo.o_loc;
  A.lse = lo.lse;
  A.gate = lo.gate;
  A.out = (T*)lo.out;
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
  A.tiles_y = (g.Y + kTile - 1) / kTile;
  A.tiles_x = (g.X + kTile - 1) / kTile;
  A.nblocks = (int64_t)A.tiles_x * A.tiles_y * g.Z * g.Hkv;
  A.per_xcd = (A.nblocks + kNumXcd - 1) / kNumXcd;
  hipLaunchKernelGGL((k_local_attn<T, G>), dim3((unsigned)(A.per_xcd * kNumXcd)),
                     dim3(64 * LCfg<G>::W), 0, s, A);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_lt(const Geom& g, const void* q, const void* k, const void* v,
                            const int32_t* c2p, const LocalOut& lo, const QRope& qr,
                            hipStream_t s) {
  switch (g.G) {
    case 1: return launch_l<T, 1>(g, q, k, v, c2p, lo, qr, s);
    case 2: return launch_l<T, 2>(g, q, k, v, c2p, lo, qr, s);
    case 4: return launch_l<T, 4>(g, q, k, v, c2p, lo, qr, s);
    case 8: return launch_l<T, 8>(g, q, k, v, c2p, lo, qr, s);
    case 16: return launch_l<T, 16>(g, q, k, v, c2p, lo, qr, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_local_attn(const Geom& g, const void* q, const void* k_rot, const void* v,
                             const int32_t* c2p, const LocalOut& lo, const QRope& qr,
                             hipStream_t s) {
  if (g.bf16 && local_bf16_serves(g.G))
    return launch_local_attn_bf16(g, q, k_rot, v, c2p, lo, qr, s);
  if (g.bf16) return launch_lt<bf16_t>(g, q, k_rot, v, c2p, lo, qr, s);
  return launch_lt<float>(g, q, k_rot, v, c2p, lo, qr, s);
}

}  // namespace pack3d
