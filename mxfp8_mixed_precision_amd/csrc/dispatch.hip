// Expert-major dispatch of routed tokens into the padded token layout, for gfx950.
//
// The fully fused MLP needs every expert's rows in one contiguous segment whose length is a
// multiple of pad_multiple, pad rows zero (torchtitan PR #12 "Wire the fully-fused grouped-GEMM
// MXFP8 plan behind fusion_plan", section "What it adds": the padded dispatcher that the
// kernels' hard per-expert alignment requires; torchtitan PR #2, section "Summary"). Inside a
// segment rows follow the assignment index a = t * topk + k (a stable counting sort), so the
// layout is unique.
//
//  * The plan is a stable counting sort in three launches. Workgroup b of the first and last
//    owns assignments [1024 b, 1024 b + 1024), 256 per wavefront, read as 4 ids per lane with
//    all loads in flight. Lanes routed to the same expert find each other with one ballot per
//    bit of the id, so each LDS counter is advanced once per group of equal ids (same-address
//    LDS atomics from 64 lanes would serialize).
//      route_hist:  per-workgroup histogram (plus a count of out-of-range ids) -> workspace
//                   [B][E+1];
//      route_scan:  one workgroup: per expert, the exclusive prefix over workgroups (in place)
//                   and the total; the padded segment lengths scanned into offs; the status;
//      route_place: each workgroup re-counts its chunk per wavefront, takes its bases from
//                   offs + the prefix, and places 64 assignments at a time in assignment order
//                   (rank among equal ids + one LDS add per group); it also marks the pad rows
//                   of the experts e = b, b + B, ... with -1.
//    Bound by memory latency and launch overhead (three short launches), not bandwidth.
//  * permute_kernel: one wavefront per padded row copies the token's BF16 row (16-byte
//    loads and stores) or writes zeros for a pad row.
// The fused gather + dual quantization (no BF16 copy) is a kind of the quantizer
// (quantize.hip).
#include <mutex>

#include "kernels.h"
#include "mxfp8.h"

// Per-workgroup histograms of the allocation-free routing plan (mxf_route_plan_noalloc): a
// file-scope device array instead of a caller workspace. Each GPU the library runs on holds
// its own copy until the process ends. Host code never passes this name to a kernel (on the
// host it is only a stand-in symbol): it looks the device address up once per device with
// hipGetSymbolAddress and uses that.
static __device__ __align__(256) int32_t scratch[MXF_ROUTE_NOALLOC_MAX_BYTES / sizeof(int32_t)];

namespace mxf {

constexpr int kPlanChunk = 1024;  // assignments per workgroup (4 wavefronts x 4 x 64)

// Lanes (with ok set) whose expert id equals this lane's: one ballot per bit of the id.
__device__ __forceinline__ uint64_t same_expert(int e, bool ok, int nbits) {
  uint64_t peers = __ballot(ok);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

__device__ __forceinline__ int plan_nbits(int E) { return E > 1 ? 32 - __clz(E - 1) : 0; }

// The 4 ids of this lane in its wavefront's quarter of workgroup b's chunk (-1 past n).
__device__ __forceinline__ void load_ids(const int32_t* idx, int32_t n, int b, int w, int lane, int (&ev)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t a = (int64_t)b * kPlanChunk + w * 256 + u * 64 + lane;
    ev[u] = a < n ? idx[a] : -1;
  }
}

// Per-wavefront counts of its 256 ids into cnt[E] (cnt[E] counts ids outside [0, E)).
__device__ __forceinline__ void count_ids(const int (&ev)[4], int32_t n, int b, int w, int lane, int E,
                                          int32_t* cnt) {
  const int nbits = plan_nbits(E);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t a = (int64_t)b * kPlanChunk + w * 256 + u * 64 + lane;
    const bool in = a < n;
    const bool ok = in && (unsigned)ev[u] < (unsigned)E;
    const uint64_t peers = same_expert(ev[u], ok, nbits);
    if (ok && __ffsll((unsigned long long)peers) - 1 == lane) atomicAdd(&cnt[ev[u]], __popcll(peers));
    const uint64_t badm = __ballot(in && !ok);
    if (badm && lane == 0) atomicAdd(&cnt[E], __popcll(badm));
  }
}

__global__ __launch_bounds__(256) void route_hist_kernel(const int32_t* __restrict__ idx, int32_t n, int E,
                                                         int32_t* __restrict__ hist) {
  extern __shared__ int32_t lds[];  // [E + 1]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, b = blockIdx.x;
  int ev[4];
  load_ids(idx, n, b, w, lane, ev);
  for (int e = tid; e <= E; e += 256) lds[e] = 0;
  __syncthreads();
  count_ids(ev, n, b, w, lane, E, lds);
  __syncthreads();
  for (int e = tid; e <= E; e += 256) hist[(int64_t)b * (E + 1) + e] = lds[e];
}

// One workgroup of 1024 threads; thread e <= E owns column e of hist [B][E+1].
__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t* __restrict__ hist, int B, int E, int pad,
                                                          int64_t mcap, int32_t* __restrict__ offs,
                                                          int32_t* __restrict__ counts, int32_t* status) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t etot[1025];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int col = tid; col <= E; col += 1024) {
    int total = 0;
    int b = 0;
    for (; b + 8 <= B; b += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = hist[(int64_t)(b + i) * (E + 1) + col];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hist[(int64_t)(b + i) * (E + 1) + col] = total;
        total += v[i];
      }
    }
    for (; b < B; ++b) {
      const int v = hist[(int64_t)b * (E + 1) + col];
      hist[(int64_t)b * (E + 1) + col] = total;
      total += v;
    }
    etot[col] = total;
  }
  __syncthreads();
  // exclusive scan of the padded segment lengths over experts (E <= 1024: one per thread)
  const int c = tid < E ? etot[tid] : 0;
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
    offs[tid] = wbase + incl - seg;
    counts[tid] = c;
  }
  if (tid == 1023) {
    offs[E] = wbase + incl;
    if (status) *status = etot[E] ? 2 : ((int64_t)(wbase + incl) > mcap ? 3 : 0);
  }
}

__global__ __launch_bounds__(256) void route_place_kernel(const int32_t* __restrict__ idx, int32_t n, int E,
                                                          int64_t mcap, const int32_t* __restrict__ hist,
                                                          const int32_t* __restrict__ offs,
                                                          const int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ row_assign,
                                                          int32_t* __restrict__ assign_row) {
  extern __shared__ int32_t lds[];
  int32_t* wc = lds;                 // [4][E + 1] per-wavefront counts, then bases
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, b = blockIdx.x;
  int ev[4];
  load_ids(idx, n, b, w, lane, ev);
  for (int i = tid; i < 4 * (E + 1); i += 256) wc[i] = 0;
  __syncthreads();
  count_ids(ev, n, b, w, lane, E, wc + w * (E + 1));
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int run = offs[e] + hist[(int64_t)b * (E + 1) + e];
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const int t = wc[ww * (E + 1) + e];
      wc[ww * (E + 1) + e] = run;
      run += t;
    }
  }
  __syncthreads();
  int32_t* mine = wc + w * (E + 1);
  const int nbits = plan_nbits(E);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t a = (int64_t)b * kPlanChunk + w * 256 + u * 64 + lane;
    const bool in = a < n;
    const int e = ev[u];
    const bool ok = in && (unsigned)e < (unsigned)E;
    const uint64_t peers = same_expert(e, ok, nbits);
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    const int leader = ok ? __ffsll((unsigned long long)peers) - 1 : lane;
    int first = 0;
    if (ok && lane == leader) first = atomicAdd(&mine[e], __popcll(peers));
    first = __shfl(first, leader);
    if (in) {
      int row = -1;
      if (ok) {
        const int64_t r = (int64_t)first + rank;
        if (r < mcap) {
          row = (int)r;
          row_assign[r] = (int)a;
        }
      }
      assign_row[a] = row;
    }
  }
  // pad rows (inside the capacity) of the experts e = b, b + B, ... map to -1
  for (int e = b; e < E; e += gridDim.x) {
    const int64_t r1 = min<int64_t>(offs[e + 1], mcap);
    for (int64_t r = (int64_t)offs[e] + counts[e] + tid; r < r1; r += 256) row_assign[r] = -1;
  }
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

static int64_t plan_blocks(int64_t n) { return n > 0 ? (n + mxf::kPlanChunk - 1) / mxf::kPlanChunk : 1; }

size_t mxf_route_plan_workspace_bytes(int64_t n, int E) { return (size_t)plan_blocks(n) * (E + 1) * sizeof(int32_t); }

hipError_t mxf_launch_route_plan(const int32_t* idx, int32_t n, int E, int pad, int64_t mcap, int32_t* offs,
                                 int32_t* counts, int32_t* row_assign, int32_t* assign_row, int32_t* status,
                                 void* workspace, hipStream_t st) {
  const int B = (int)plan_blocks(n);
  int32_t* hist = (int32_t*)workspace;
  hipLaunchKernelGGL(mxf::route_hist_kernel, dim3(B), dim3(256), (E + 1) * sizeof(int32_t), st, idx, n, E, hist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mxf::route_scan_kernel, dim3(1), dim3(1024), 0, st, hist, B, E, pad, mcap, offs, counts,
                     status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mxf::route_place_kernel, dim3(B), dim3(256), 4 * (E + 1) * sizeof(int32_t), st, idx, n, E,
                     mcap, hist, offs, counts, row_assign, assign_row);
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

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // device address of `scratch`, per device ordinal
}  // namespace

// Device address and size of the routing plan's static scratch array on the current device,
// looked up on the first call per device (with that device current) and cached.
hipError_t mxf_route_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}
