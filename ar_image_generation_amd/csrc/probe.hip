// Measurement kernel: streaming read of a device buffer, the attainable-HBM
// reference the decode kernel's kept-byte bandwidth is compared with.
//
// Each thread reads 16-byte chunks with nontemporal loads (the data is read
// once), UNROLL independent loads in flight per iteration, grid-stride; the
// XOR of everything read is written once per workgroup so the loads cannot
// be removed.
#include "common.h"

namespace da {

template <int UNROLL>
__global__ void __launch_bounds__(256) read_probe_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace da

using namespace da;

extern "C" int da_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid,
                                 int32_t loads_in_flight, void* stream) {
  if (!buf || !sink) return fail(DA_EINVAL, "probe: NULL buffer or sink");
  if (bytes < 16 || bytes % 16 || (uintptr_t)buf % 16)
    return fail(DA_EINVAL, "probe: bytes must be a positive multiple of 16, buffer 16-byte aligned");
  if (grid < 1) return fail(DA_EINVAL, "probe: grid=%d < 1", grid);
  void (*k)(const u32x4*, int64_t, uint32_t*);
  switch (loads_in_flight) {
    case 1: k = read_probe_kernel<1>; break;
    case 2: k = read_probe_kernel<2>; break;
    case 4: k = read_probe_kernel<4>; break;
    case 8: k = read_probe_kernel<8>; break;
    case 16: k = read_probe_kernel<16>; break;
    default: return fail(DA_EINVAL, "probe: loads_in_flight=%d not in {1, 2, 4, 8, 16}", loads_in_flight);
  }
  clear_error();
  hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, (hipStream_t)stream, reinterpret_cast<const u32x4*>(buf),
                     bytes / 16, sink);
  return check_launch("read_probe_kernel");
}
