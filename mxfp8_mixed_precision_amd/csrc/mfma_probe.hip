// Matrix-core ceiling kernels: the MXFP8 contraction rate this chip sustains, measured with the
// grouped GEMM's own instruction mix, so the GEMMs can be reported against a measured rate as
// well as against the data-sheet peak (as the quantizers are against the HBM probe kernels).
//
// Both run one 256-thread block per CU (four wavefronts in a 2 x 2 grid, each owning a 128 x 128
// tile of 32 x 32 fragments, i.e. a 256 x 256 block tile) and count 64-k stages: per stage every
// wavefront issues 16 v_mfma_scale_f32_32x32x64_f8f6f4 (256 x 256 x 64 x 2 FLOP per block).
//   MODE 0 (matrix only): the fragments are read from LDS once; the loop is the 16 matrix
//          instructions per stage with nothing beside them. Under the socket's power limit this
//          is the highest rate the matrix cores reach on real operand bits.
//   MODE 1 (whole stage): the GEMM main loop's stage without the tile bookkeeping: a four-slot
//          LDS ring filled by direct global->LDS loads (eight 1 KB operand loads per wavefront
//          and stage, two 256-byte scale-word loads every other stage), the next stage's 16
//          fragment reads and 8 scale-byte reads interleaved with the current stage's matrix
//          instructions, one block barrier per stage. Stage s of block b reads the 32 KB chunk
//          (37 b + s) mod (bytes / 32 KB) of the source window: a window of a few MB stays in
//          each XCD's L2, a window of hundreds of MB streams from HBM.
// The E8M0 scales are read as bytes from an LDS area holding 127 (a factor of 1), so with every
// operand code 0x38 (E4M3 1.0) each accumulator gains 64 per stage and every thread's output
// (the sum of the first accumulator of its 16 fragments) is exactly 1024 * stages.
#include "kernels.h"

namespace mxf {
namespace mfp {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4_t lds_u4;
typedef __attribute__((address_space(3))) const uint8_t lds_u8;
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int STAGE = 32768;       // one stage: 256 A rows + 256 B rows of 64 bytes
constexpr int S = 4;               // ring slots
constexpr int SC_OFF = S * STAGE;  // scale bytes (read) at +0, scale-word landing area at +4096
constexpr int LDS = S * STAGE + 8192;

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr)p; }
__device__ __forceinline__ lds_u4* lds16_at(uint32_t a) { return (lds_u4*)(uintptr_t)a; }
__device__ __forceinline__ lds_u8* lds8_at(uint32_t a) { return (lds_u8*)(uintptr_t)a; }
// 16-byte chunk c of 64-byte row r at chunk c ^ ((r / 4) % 4), as in the GEMM's LDS tiles
__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// direct global->LDS loads (lane l's bytes land at M0 + size * l); the kernel waits on vmcnt itself
template <int OFF>
__device__ __forceinline__ void g2lds16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3" ::"s"(lds), "v"(voff), "s"(sbase),
               "i"(OFF) : "memory", "m0");
}
__device__ __forceinline__ void g2lds16_q(int q, const void* sbase, uint32_t voff, uint32_t lds) {
  switch (q & 3) {
    case 0: g2lds16<0>(sbase, voff, lds); break;
    case 1: g2lds16<1024>(sbase, voff, lds); break;
    case 2: g2lds16<2048>(sbase, voff, lds); break;
    default: g2lds16<3072>(sbase, voff, lds); break;
  }
}
__device__ __forceinline__ void g2lds4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}

template <int MODE>
__global__ __launch_bounds__(256, 1) void mfma_probe_kernel(const uint8_t* __restrict__ src, uint32_t nchunk,
                                                            int stages, float* __restrict__ out) {
  extern __shared__ __align__(1024) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int r32 = lane & 31, g = lane >> 5;
  const uint32_t lds0 = lds_addr(smem);
  // the ring starts with the window's first four chunks; scale bytes 127
  for (int i = tid; i < S * STAGE / 16; i += 256)
    reinterpret_cast<uint4*>(smem)[i] = reinterpret_cast<const uint4*>(src)[i];
  for (int i = tid; i < 4096; i += 256) smem[SC_OFF + i] = 127;
  __syncthreads();

  const uint32_t wid_u = (uint32_t)__builtin_amdgcn_readfirstlane(wid);
  // lane l of a 1 KB load: row l / 4 of 16, chunk (l % 4) ^ (l / 16) (the swizzle on the global side)
  const uint32_t voff = (uint32_t)(lane >> 2) * 64 + ((uint32_t)((lane & 3) ^ (lane >> 4)) << 4);
  const uint32_t rd_a0 = lds0 + swz(wm * 128 + r32, g), rd_a1 = lds0 + swz(wm * 128 + r32, 2 + g);
  const uint32_t rd_b0 = lds0 + 16384 + swz(wn * 128 + r32, g), rd_b1 = lds0 + 16384 + swz(wn * 128 + r32, 2 + g);
  const uint32_t rd_sa = lds0 + SC_OFF + (wm * 128 + r32) * 4 + g;
  const uint32_t rd_sb = lds0 + SC_OFF + 2048 + (wn * 128 + r32) * 4 + g;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  v8i fa[2][4], fb[2][4];
  uint32_t sa[2][4], sb[2][4];
  // read r of a stage: r < 8 A fragment r / 2 (k half r % 2), then 8 B reads
  auto read_frag = [&](int r, uint32_t so, int B) {
    const int i = (r >> 1) & 3, hi = r & 1;
    const u32x4_t v = lds16_at((r < 8 ? (hi ? rd_a1 : rd_a0) : (hi ? rd_b1 : rd_b0)) + so)[i * 128];
    v8i& f = r < 8 ? fa[B][i] : fb[B][i];
    f[4 * hi] = (int)v.x; f[4 * hi + 1] = (int)v.y; f[4 * hi + 2] = (int)v.z; f[4 * hi + 3] = (int)v.w;
  };
  auto read_scale = [&](int q, int B) {  // q < 4: A fragment q, else B fragment q - 4
    if (q < 4) sa[B][q] = lds8_at(rd_sa)[q * 128 + 2 * B];
    else sb[B][q - 4] = lds8_at(rd_sb)[(q - 4) * 128 + 2 * B];
  };
#pragma unroll
  for (int r = 0; r < 16; ++r) read_frag(r, 0, 0);
#pragma unroll
  for (int q = 0; q < 8; ++q) read_scale(q, 0);

  if constexpr (MODE == 0) {
    for (int kt = 0; kt < stages; ++kt) {
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int i = m >> 2, j = m & 3;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[0][i], fb[0][j], acc[i][j], 0, 0, 0,
                                                                    (int)sa[0][i], 0, (int)sb[0][j]);
      }
    }
  } else {
    uint32_t chunk = (uint32_t)(((uint64_t)blockIdx.x * 37u) % nchunk);
    // step kt (P = kt % 2): stage kt+1 has landed once at most the loads of stages kt+2 and
    // kt+3 (one even stage: 10, one odd: 8) are pending; after the barrier every wavefront has
    // stage kt in registers, so slot kt % 4 takes stage kt+4's loads
    auto step = [&](int kt, auto par) {
      constexpr int P = decltype(par)::value;
      wait_vmcnt<18>();
      __syncthreads();
      const uint32_t so_next = (uint32_t)((kt + 1) % S) * STAGE;
      const uint32_t slot = lds0 + (uint32_t)(kt % S) * STAGE;
      const uint8_t* gb = src + (uint64_t)chunk * STAGE + wid_u * 4096;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int i = m >> 2, j = m & 3;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[P][i], fb[P][j], acc[i][j], 0, 0, 0,
                                                                    (int)sa[P][i], 0, (int)sb[P][j]);
        read_frag(m, so_next, 1 - P);
        if ((m & 1) == 0) read_scale(m >> 1, 1 - P);
        if (m < 8) g2lds16_q(m, gb + (m < 4 ? 0 : 16384), voff, slot + (m < 4 ? 0 : 16384) + wid_u * 4096);
        if (P == 0 && m == 9) {  // the scale words of a 128-k block (landing area only)
          g2lds4(gb + 8192, (uint32_t)lane * 4, lds0 + SC_OFF + 4096 + wid_u * 512);
          g2lds4(gb + 9216, (uint32_t)lane * 4, lds0 + SC_OFF + 4096 + wid_u * 512 + 256);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      chunk = chunk + 1 == nchunk ? 0 : chunk + 1;
    };
    for (int kt = 0; kt < stages; kt += 2) {
      step(kt, std::integral_constant<int, 0>());
      step(kt + 1, std::integral_constant<int, 1>());
    }
    wait_vmcnt<0>();
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[i][j][0];
  out[(size_t)blockIdx.x * 256 + tid] = s;
}

}  // namespace mfp
}  // namespace mxf

// mode 0: matrix instructions only; 1: whole GEMM stage over the source window. bytes is a
// multiple of 32 KB and at least 128 KB; stages even and positive; out holds blocks * 256 floats.
hipError_t mxf_launch_mfma_probe(int mode, const void* src, int64_t bytes, int stages, int blocks, float* out,
                                 hipStream_t st) {
  using namespace mxf::mfp;
  const int64_t nchunk = bytes / STAGE;
  if (nchunk < S || bytes % STAGE || nchunk > 0xFFFFFFFFll || stages <= 0 || stages % 2 || blocks <= 0)
    return hipErrorInvalidValue;
  auto k = mode == 0 ? mfma_probe_kernel<0> : mfma_probe_kernel<1>;
  hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(256), LDS, st, reinterpret_cast<const uint8_t*>(src),
                     (uint32_t)nchunk, stages, out);
  return hipGetLastError();
}
