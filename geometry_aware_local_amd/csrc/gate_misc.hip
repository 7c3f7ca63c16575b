// Standalone tokenwise gate and the packing helpers.
//
// Gate: "Geometry Matters in Packed 3D Attention", papernotes.org notes,
// flowchart node F: a learned per-token softmax over the two branches mixes
// the local and compressed outputs before the residual.
#include "pack3d_device.h"

namespace pack3d {

// out[i, h, :] = g_loc * o_loc + g_cmp * o_cmp; one thread per 4 dims.
template <typename T>
__global__ __launch_bounds__(256) void k_gate_mix(const float* __restrict__ ol,
                                                  const float* __restrict__ oc,
                                                  const float* __restrict__ gate, T* out,
                                                  int64_t n, int32_t hq, int32_t per_head) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid >> 4;          // (token, head)
  if (row >= n * hq) return;
  const int d0 = (int)(gid & 15) * 4;
  float g0, g1;
  gate_weights(gate, row / hq, (int)(row % hq), hq, per_head, g0, g1);
  const f32x4 a = *reinterpret_cast<const f32x4*>(ol + row * 64 + d0);
  const f32x4 b = *reinterpret_cast<const f32x4*>(oc + row * 64 + d0);
  if constexpr (std::is_same<T, float>::value) {
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = g0 * a[j] + g1 * b[j];
    *reinterpret_cast<f32x4*>(out + row * 64 + d0) = r;
  } else {
    bf16x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (bf16_t)(g0 * a[j] + g1 * b[j]);
    *reinterpret_cast<bf16x4*>(out + row * 64 + d0) = r;
  }
}

hipError_t launch_gate_mix(const Geom& g, const float* o_loc, const float* o_cmp,
                           const float* gate, void* out, hipStream_t s) {
  const int64_t threads = g.N * g.Hq * 16;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (g.bf16)
    hipLaunchKernelGGL(k_gate_mix<bf16_t>, grid, dim3(256), 0, s, o_loc, o_cmp, gate,
                       (bf16_t*)out, g.N, g.Hq, g.gate_per_head);
  else
    hipLaunchKernelGGL(k_gate_mix<float>, grid, dim3(256), 0, s, o_loc, o_cmp, gate,
                       (float*)out, g.N, g.Hq, g.gate_per_head);
  return hipGetLastError();
}

// cell_to_pos[cell(coords[i])] = i (coordinates outside the lattice are skipped).
__global__ __launch_bounds__(256) void k_cell_index(const int32_t* __restrict__ coords,
                                                    int32_t* c2p, int64_t n, int32_t Z, int32_t Y,
                                                    int32_t X) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int z = coords[3 * i], y = coords[3 * i + 1], x = coords[3 * i + 2];
  if (z < 0 || z >= Z || y < 0 || y >= Y || x < 0 || x >= X) return;
  c2p[((int64_t)z * Y + y) * X + x] = (int32_t)i;
}

hipError_t launch_build_cell_index(const Geom& g, const int32_t* coords, int32_t* c2p,
                                   hipStream_t s) {
  hipLaunchKernelGGL(k_cell_index, dim3((unsigned)((g.N + 255) / 256)), dim3(256), 0, s, coords,
                     c2p, g.N, g.Z, g.Y, g.X);
  return hipGetLastError();
}

// Counts tokens whose coordinates are outside the lattice or whose cell does
// not map back to them.  Single workgroup: block-local reduction, no atomics
// on device memory, and the count is written (not accumulated), so no
// separate clearing step is needed.
__global__ __launch_bounds__(1024) void k_check_packing(const int32_t* __restrict__ coords,
                                                        const int32_t* __restrict__ c2p,
                                                        int32_t* n_bad, int64_t n, int32_t Z,
                                                        int32_t Y, int32_t X) {
  __shared__ int32_t part[1024];
  int32_t bad = 0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int z = coords[3 * i], y = coords[3 * i + 1], x = coords[3 * i + 2];
    if (z < 0 || z >= Z || y < 0 || y >= Y || x < 0 || x >= X) {
      ++bad;
      continue;
    }
    const int32_t p = c2p[((int64_t)z * Y + y) * X + x];
    bad += p != (int32_t)i;
  }
  part[threadIdx.x] = bad;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_bad = part[0];
}

hipError_t launch_check_packing(const Geom& g, const int32_t* coords, const int32_t* c2p,
                                int32_t* n_bad, hipStream_t s) {
  hipLaunchKernelGGL(k_check_packing, dim3(1), dim3(1024), 0, s, coords, c2p, n_bad, g.N, g.Z,
                     g.Y, g.X);
  return hipGetLastError();
}

}  // namespace pack3d
