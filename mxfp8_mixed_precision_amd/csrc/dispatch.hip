// Expert-major dispatch of routed tokens into the padded token layout, for gfx950.
//
// The fully fused MLP needs every expert's rows in one contiguous segment whose length is a
// multiple of pad_multiple, pad rows zero (torchtitan PR #12 "Wire the fully-fused grouped-GEMM
// MXFP8 plan behind fusion_plan", section "What it adds": the padded dispatcher that the
// kernels' hard per-expert alignment requires; torchtitan PR #2, section "Summary"). Inside a
// segment rows follow the assignment index a = t * topk + k (a stable counting sort), so the
// layout is unique.
//
//  * route_plan_kernel (one workgroup of 16 wavefronts): wavefront w owns a contiguous chunk of
//    the assignments. Pass 1 counts its chunk per expert in its own LDS row; then one thread
//    per expert turns the 16 rows into per-wavefront bases and the padded segment lengths are
//    scanned into offs. Pass 2 walks the chunk again 64 assignments at a time: lanes routed to
//    the same expert find each other with log2(E) ballots, take their rank among themselves,
//    and the lowest of them advances the wavefront's counter for that expert -- so the order
//    is the assignment order without any cross-wavefront atomics. Launch cost is a few
//    microseconds at tens of thousands of assignments; the plan is latency-bound, not
//    bandwidth-bound.
//  * permute_kernel: one wavefront per padded row copies the token's BF16 row (16-byte
//    loads and stores) or writes zeros for a pad row.
// The fused gather + dual quantization (no BF16 copy) is a kind of the quantizer
// (quantize.hip).
#include "kernels.h"

namespace mxf {

constexpr int kPlanWaves = 16;

__global__ __launch_bounds__(1024) void route_plan_kernel(const int32_t* __restrict__ idx, int32_t n, int E,
                                                          int pad, int64_t mcap, int32_t* __restrict__ offs,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ row_assign,
                                                          int32_t* __restrict__ assign_row, int32_t* status) {
  extern __shared__ int32_t lds[];
  int32_t* cnt = lds;                        // [kPlanWaves][E]: per-wavefront counts, then bases
  int32_t* ecnt = cnt + kPlanWaves * E;      // [E] routed rows per expert
  int32_t* eoff = ecnt + E;                  // [E + 1] segment starts
  __shared__ int32_t wsum[kPlanWaves];
  __shared__ int32_t bad_flag;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kPlanWaves * E; i += 1024) cnt[i] = 0;
  if (tid == 0) bad_flag = 0;
  __syncthreads();

  const int chunk = (int)(((int64_t)n + kPlanWaves * 64 - 1) / (kPlanWaves * 64) * 64);
  const int a0 = (int)min<int64_t>((int64_t)w * chunk, n);
  const int a1 = (int)min<int64_t>((int64_t)a0 + chunk, n);
  int32_t* mine = cnt + w * E;
  bool bad = false;
  for (int a = a0 + lane; a < a1; a += 64) {
    const int e = idx[a];
    if ((unsigned)e < (unsigned)E) atomicAdd(&mine[e], 1);
    else bad = true;
  }
  if (bad) bad_flag = 1;
  __syncthreads();

  // per expert: total, and each wavefront's base inside the expert's segment
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int ww = 0; ww < kPlanWaves; ++ww) {
      const int c = cnt[ww * E + e];
      cnt[ww * E + e] = run;
      run += c;
    }
    ecnt[e] = run;
  }
  __syncthreads();

  // exclusive scan of the padded segment lengths (E <= 1024: one expert per thread)
  const int c = tid < E ? ecnt[tid] : 0;
  const int seg = (c + pad - 1) / pad * pad;
  int incl = seg;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d);
    if (lane >= d) incl += t;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int wbase = 0;
  for (int ww = 0; ww < w; ++ww) wbase += wsum[ww];
  if (tid < E) {
    eoff[tid] = wbase + incl - seg;
    offs[tid] = wbase + incl - seg;
    counts[tid] = c;
  }
  if (tid == 1023) {
    eoff[E] = wbase + incl;
    offs[E] = wbase + incl;
  }
  __syncthreads();

  // stable placement, 64 assignments of the chunk at a time
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  for (int base = a0; base < a1; base += 64) {
    const int a = base + lane;
    const bool in = a < a1;
    const int e = in ? idx[a] : -1;
    const bool ok = in && (unsigned)e < (unsigned)E;
    uint64_t peers = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    const int leader = ok ? __ffsll((unsigned long long)peers) - 1 : lane;
    int first = 0;
    if (ok && lane == leader) first = atomicAdd(&mine[e], __popcll(peers));
    first = __shfl(first, leader);
    if (in) {
      int row = -1;
      if (ok) {
        const int64_t r = (int64_t)eoff[e] + first + rank;
        if (r < mcap) {
          row = (int)r;
          row_assign[r] = a;
        }
      }
      assign_row[a] = row;
    }
  }

  // pad rows of each expert (inside the capacity) map to -1
  for (int e = w; e < E; e += kPlanWaves) {
    const int64_t r1 = min<int64_t>(eoff[e + 1], mcap);
    for (int64_t r = (int64_t)eoff[e] + ecnt[e] + lane; r < r1; r += 64) row_assign[r] = -1;
  }
  if (tid == 0 && status) *status = bad_flag ? 2 : ((int64_t)eoff[E] > mcap ? 3 : 0);
}

// One wavefront per row of the padded layout: row r < min(offs[E], mcap) gets token
// row_assign[r] / topk, or zeros for a pad row (or an index outside the token range).
__global__ __launch_bounds__(256) void permute_kernel(const uint16_t* __restrict__ x, int64_t n_assign, int topk,
                                                      int64_t D, const int32_t* __restrict__ offs, int E,
                                                      const int32_t* __restrict__ row_assign, int64_t mcap,
                                                      uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t mend = min<int64_t>(offs[E], mcap);
  if (r >= mend) return;
  const int a = row_assign[r];
  const bool real = a >= 0 && a < n_assign;
  const uint4* src = reinterpret_cast<const uint4*>(x + (real ? (int64_t)(a / topk) * D : 0));
  uint4* dst = reinterpret_cast<uint4*>(out + r * D);
  const int64_t chunks = D >> 3;
  int64_t i = lane;
  for (; i + 192 < chunks; i += 256) {
    uint4 v0 = {0, 0, 0, 0}, v1 = v0, v2 = v0, v3 = v0;
    if (real) {
      v0 = src[i]; v1 = src[i + 64]; v2 = src[i + 128]; v3 = src[i + 192];
    }
    dst[i] = v0; dst[i + 64] = v1; dst[i + 128] = v2; dst[i + 192] = v3;
  }
  for (; i < chunks; i += 64) dst[i] = real ? src[i] : make_uint4(0, 0, 0, 0);
}

}  // namespace mxf

size_t mxf_route_plan_lds_bytes(int E) { return (size_t)(mxf::kPlanWaves * E + 2 * E + 1) * sizeof(int32_t); }

hipError_t mxf_launch_route_plan(const int32_t* idx, int32_t n, int E, int pad, int64_t mcap, int32_t* offs,
                                 int32_t* counts, int32_t* row_assign, int32_t* assign_row, int32_t* status,
                                 hipStream_t st) {
  const size_t lds = mxf_route_plan_lds_bytes(E);
  if (lds > 65536) {
    // above 64 KiB of dynamic LDS (E > 900) the kernel must opt in (gfx950 has 160 KiB per CU)
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&mxf::route_plan_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(mxf::route_plan_kernel, dim3(1), dim3(1024), lds, st, idx, n, E, pad, mcap, offs, counts,
                     row_assign, assign_row, status);
  return hipGetLastError();
}

hipError_t mxf_launch_permute(const void* x, int64_t n_assign, int topk, int64_t D, const int32_t* offs, int E,
                              const int32_t* row_assign, int64_t mcap, void* out, hipStream_t st) {
  if (mcap == 0) return hipSuccess;
  const int64_t blocks = (mcap + 3) / 4;
  hipLaunchKernelGGL(mxf::permute_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint16_t*)x, n_assign,
                     topk, D, offs, E, row_assign, mcap, (uint16_t*)out);
  return hipGetLastError();
}
