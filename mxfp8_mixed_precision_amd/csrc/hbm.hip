// HBM ceiling kernels: the read, write and copy rates this chip sustains, measured with the
// access patterns that reach them (16-byte lanes, contiguous kilobyte per wavefront
// instruction, grid-stride over the whole buffer). The HBM-bound kernels of the library (the
// quantizers, the dequantizer) are reported against these as well as against the 8 TB/s data
// sheet figure.
//
// Launch shapes (measured on MI355X over 1 GiB; each the fastest of 1, 2, 4, 8 or 16 blocks
// per CU and 4 or 8 loads in flight per lane):
//   read:  one block per CU, eight 16-byte non-temporal loads in flight per lane (7.0-7.3 TB/s)
//   write: one block per CU, four 16-byte stores per lane and iteration (5.9 TB/s)
//   copy:  two blocks per CU, four 16-byte non-temporal loads, then stores (5.8-6.1 TB/s)
#include "kernels.h"
#include "mx_device.h"

namespace mxf {

typedef unsigned hb_u4 __attribute__((ext_vector_type(4)));

// Read: every 16-byte word of src once, XOR-reduced over the block; block b then XORs its
// partial into 16-byte slot b % 64 of dst (one vector-memory atomic per word position: atomics
// from many blocks to the same address serialise and would dominate the time). The XOR of
// dst's 64 slots is the XOR of all of src's words, so the loads are not dead and the result
// is checkable.
template <int U>
__global__ __launch_bounds__(256) void hbm_read_kernel(const hb_u4* __restrict__ src, int64_t n, uint32_t* dst) {
  __shared__ hb_u4 part[4];
  hb_u4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * 256 * U;
  for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
    hb_u4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      v[u] = i < n ? __builtin_nontemporal_load(src + i) : hb_u4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  // wavefront XOR reduction, then one atomic per word position and wavefront
  for (int off = 32; off >= 1; off >>= 1) {
    acc.x ^= (uint32_t)__shfl_xor((int)acc.x, off);
    acc.y ^= (uint32_t)__shfl_xor((int)acc.y, off);
    acc.z ^= (uint32_t)__shfl_xor((int)acc.z, off);
    acc.w ^= (uint32_t)__shfl_xor((int)acc.w, off);
  }
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const hb_u4 b = part[0] ^ part[1] ^ part[2] ^ part[3];
    uint32_t* slot = dst + 4 * (blockIdx.x & 63);
    atomicXor(slot + 0, b.x);
    atomicXor(slot + 1, b.y);
    atomicXor(slot + 2, b.z);
    atomicXor(slot + 3, b.w);
  }
}

// Write: 16-byte word i of dst (i counted from the buffer start) becomes {i, i, i, i} (low 32
// bits of i).
template <int U>
__global__ __launch_bounds__(256) void hbm_write_kernel(hb_u4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256 * U;
  for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      const uint32_t w = (uint32_t)i;
      if (i < n) dst[i] = hb_u4{w, w, w, w};
    }
  }
}

// Copy: dst = src, U non-temporal loads per lane in flight, then U non-temporal stores.
template <int U>
__global__ __launch_bounds__(256) void hbm_copy_kernel(const hb_u4* __restrict__ src, hb_u4* __restrict__ dst,
                                                       int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256 * U;
  for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
    hb_u4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

}  // namespace mxf

// mode 0: read src (XOR of its 16-byte words spread over dst's 64 16-byte slots, which the
// caller zeroes);
// 1: write dst; 2: copy src to dst. bytes is a positive multiple of 16; buffers 16-byte aligned.
hipError_t mxf_launch_hbm_probe(int mode, const void* src, void* dst, int64_t bytes, int ncu, hipStream_t st) {
  using namespace mxf;
  const int64_t n = bytes / 16;
  if (n <= 0 || ncu <= 0) return hipErrorInvalidValue;
  if (mode == 0) {
    hipLaunchKernelGGL(hbm_read_kernel<8>, dim3((unsigned)ncu), dim3(256), 0, st,
                       reinterpret_cast<const hb_u4*>(src), n, reinterpret_cast<uint32_t*>(dst));
  } else if (mode == 1) {
    hipLaunchKernelGGL(hbm_write_kernel<4>, dim3((unsigned)ncu), dim3(256), 0, st, reinterpret_cast<hb_u4*>(dst), n);
  } else if (mode == 2) {
    hipLaunchKernelGGL(hbm_copy_kernel<4>, dim3((unsigned)(2 * ncu)), dim3(256), 0, st,
                       reinterpret_cast<const hb_u4*>(src), reinterpret_cast<hb_u4*>(dst), n);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
