// Measurement kernels: a streaming read of a device buffer, and a gather of
// exactly the K/V rows a decode step keeps -- the attainable-HBM references
// the decode kernel's kept-byte bandwidth is compared with.
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

// Gather probe: reads the rows at n_rows byte offsets (the kept K/V rows of
// a decode step, resolved through its lists and block table beforehand) of
// two buffers, K and V, and nothing else -- the attainable rate of the
// decode's access pattern without its arithmetic or its own address chain.
// One group of row_bytes / 16 lanes reads one row of K and of V; UNROLL rows
// a group in flight, grid-stride over the rows; the next iteration's offsets
// are fetched while this iteration's rows are in flight.  Offsets are
// clamped into [0, max_off] and rounded down to 16 bytes, so no offset
// reads outside the buffers.
template <int UNROLL>
__global__ void __launch_bounds__(256) gather_probe_kernel(const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                                                           const int64_t* __restrict__ offs, int64_t n_rows,
                                                           int64_t max_off, int lpr_shift, uint32_t* __restrict__ sink) {
  auto fetch = [&](int64_t r) -> int64_t {
    if (r >= n_rows) return -1;
    const int64_t o = offs[r];
    return (o < 0 ? 0 : o > max_off ? max_off : o) & ~int64_t(15);
  };
  const int lane = threadIdx.x & 63;
  const int grp = lane >> lpr_shift;
  const int sub = lane & ((1 << lpr_shift) - 1);
  const int64_t upw = 64 >> lpr_shift;                      // rows a wave reads at once
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t step = (((int64_t)gridDim.x * blockDim.x) >> 6) * upw * UNROLL;
  int64_t base = wave * upw * UNROLL;
  int64_t nxt[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    nxt[u] = fetch(base + u * upw + grp);
  }
  uint32_t acc = 0;
  for (; base < n_rows; base += step) {
    u32x4 kk[UNROLL], vv[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      kk[u] = vv[u] = u32x4{0u, 0u, 0u, 0u};
      if (nxt[u] >= 0) {
        kk[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + nxt[u] + sub * 16));
        vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + nxt[u] + sub * 16));
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      nxt[u] = fetch(base + step + u * upw + grp);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= kk[u][0] ^ kk[u][1] ^ kk[u][2] ^ kk[u][3] ^ vv[u][0] ^ vv[u][1] ^ vv[u][2] ^ vv[u][3];
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

extern "C" int da_gather_read_probe(const void* k, const void* v, const int64_t* offsets, int64_t n_rows,
                                    int32_t row_bytes, int64_t span_bytes, uint32_t* sink, int32_t grid,
                                    int32_t loads_in_flight, void* stream) {
  if (row_bytes != 128 && row_bytes != 256 && row_bytes != 512)
    return fail(DA_ENOTSUP, "gather probe: a row of %d bytes (128, 256 or 512)", row_bytes);
  if (n_rows < 0 || span_bytes < 0) return fail(DA_EINVAL, "gather probe: n_rows=%lld span=%lld",
                                                (long long)n_rows, (long long)span_bytes);
  if (grid < 1) return fail(DA_EINVAL, "gather probe: grid=%d < 1", grid);
  if (n_rows > 0 && (!k || !v || !offsets || !sink)) return fail(DA_EINVAL, "gather probe: NULL buffer, offsets or sink");
  if (n_rows > 0 && span_bytes < row_bytes) return fail(DA_EINVAL, "gather probe: span below one row");
  if (((uintptr_t)k | (uintptr_t)v) % 16) return fail(DA_EINVAL, "gather probe: K and V must be 16-byte aligned");
  void (*kfn)(const uint8_t*, const uint8_t*, const int64_t*, int64_t, int64_t, int, uint32_t*);
  switch (loads_in_flight) {
    case 1: kfn = gather_probe_kernel<1>; break;
    case 2: kfn = gather_probe_kernel<2>; break;
    case 4: kfn = gather_probe_kernel<4>; break;
    default: return fail(DA_EINVAL, "gather probe: loads_in_flight=%d not in {1, 2, 4}", loads_in_flight);
  }
  clear_error();
  if (n_rows == 0) return DA_OK;
  hipLaunchKernelGGL(kfn, dim3(grid), dim3(256), 0, (hipStream_t)stream, reinterpret_cast<const uint8_t*>(k),
                     reinterpret_cast<const uint8_t*>(v), offsets, n_rows, span_bytes - row_bytes,
                     row_bytes == 128 ? 3 : row_bytes == 256 ? 4 : 5, sink);
  return check_launch("gather_probe_kernel");
}

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
