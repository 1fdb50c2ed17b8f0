// The read floor of the decode step's tile gather, for measurement (kvs_gather_read_floor): the same
// K and V tiles read with nothing else done, so that the attention launches' time can be set against
// what reading their bytes alone takes on this device.  None of the method's arithmetic is here.
#include "kvs_device.h"
#include "kvs_launch.h"

namespace kvs {

// Workgroup x reads tile ids[x] (phys * Hkv + h: kBlock * kDim fp16 values, contiguous in each pool)
// of K and of V: lane t takes 16 bytes at t * 16 of every 4 KiB, all 16 loads issued before any is
// used (as an attention tile's), and the workgroup writes the fp32 sum of the tile's values to out[x]
// so that no load is dead.  An id outside [0, pool_tiles) reads nothing and writes NaN.  The dynamic
// LDS is only reserved: it sets how many workgroups share a CU.
__global__ __launch_bounds__(256) void gather_read_kernel(const uint16_t* __restrict__ k_pool,
                                                          const uint16_t* __restrict__ v_pool,
                                                          int pool_tiles, const int32_t* __restrict__ ids,
                                                          float* __restrict__ out) {
  __shared__ float part[4];
  constexpr int kTile = kBlock * kDim;       // fp16 values of one tile
  constexpr int kLoads = kTile / (256 * 8);  // 16-byte loads per lane and pool
  const int id = ids[blockIdx.x];
  if (id < 0 || id >= pool_tiles) {
    if (threadIdx.x == 0) out[blockIdx.x] = __builtin_nanf("");
    return;
  }
  const size_t base = (size_t)id * kTile + threadIdx.x * 8;
  uint4 kr[kLoads], vr[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    kr[u] = ld_stream16(k_pool + base + (size_t)u * 256 * 8);
    vr[u] = ld_stream16(v_pool + base + (size_t)u * 256 * 8);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    float f[8], g[8];
    unpack8(kr[u], f);
    unpack8(vr[u], g);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += f[e] + g[e];
  }
  s = wave_sum_f32(s);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = (part[0] + part[1]) + (part[2] + part[3]);
}

hipError_t launch_gather_read(const void* k_pool, const void* v_pool, int pool_tiles, const int32_t* ids,
                              int n, int lds_bytes, float* out, hipStream_t s) {
  if (n <= 0) return hipGetLastError();
  hipLaunchKernelGGL(gather_read_kernel, dim3(n), dim3(256), (size_t)lds_bytes, s,
                     static_cast<const uint16_t*>(k_pool), static_cast<const uint16_t*>(v_pool), pool_tiles,
                     ids, out);
  return hipGetLastError();
}

}  // namespace kvs
