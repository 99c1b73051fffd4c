// Block-scaled MXFP8 grouped GEMM for gfx950, with the MLP's fused epilogues.
//
// Every GEMM of the routed-experts MLP (torchtitan PR #12 "Wire the fully-fused grouped-GEMM
// MXFP8 plan behind fusion_plan", section "What it adds": FC1 grouped GEMM + SwiGLU + dual
// MXFP8 quantization, FC2 GEMM, fused dSwiGLU backward, wgrad) has the form
//     C[m, n] = sum_k A[m, k] * B[n, k]
// with both operands stored K-contiguous as E4M3 codes plus one E8M0 scale per 32 k, and
// fp32 accumulation. The contraction runs on v_mfma_scale_f32_32x32x64_f8f6f4, which applies
// the per-32-k scales of both operands inside the matrix core.
//
// Operand layout in registers (checked on the hardware with a single-instruction test):
// for a 32x32x64 step, lane l = r + 32g (r < 32, g < 2) holds row r's bytes
// k in [16g, 16g+16) in VGPRs 0-3 and k in [32+16g, 32+16g+16) in VGPRs 4-7, and supplies
// the E8M0 scale of 32-k group g of row r (byte op_sel of its scale register). The
// accumulator lane l holds column l%32, rows 8(j/4) + 4(l/32) + (j%4) for j < 16.
//
// Tiling: block tile BM x BN, K step 128 (four scale groups), WM x WN wavefronts each
// owning a (BM/WM) x (BN/WN) tile of 32x32 MFMA fragments. A and B tiles are staged
// through LDS with double buffering (global loads for step k+1 are in flight while step k
// computes). LDS rows are 128 bytes; the 16-byte chunk index is XOR-swizzled with (row % 8)
// so that the 32 lanes reading 16 bytes from 32 consecutive rows spread over all banks.
//
// Schedulers (expert-offset driven; no host synchronisation):
//   M-grouped (FC1, FC2, both dgrads): A rows are the padded expert-major tokens; the block
//     at row tile m0 finds its expert e from the device offsets (offs[e] <= m0 < offs[e+1])
//     and multiplies by expert e's B. Tiles at or past offs[E] exit. BM divides
//     pad_multiple, so no tile straddles two experts.
//   K-grouped (both wgrads): blockIdx.z = expert; K runs over the expert's token segment
//     (the real rows rounded up to 128; pad rows are zero codes). A zero-token expert runs
//     no K step and stores zeros.
#include "kernels.h"
#include "mx_device.h"

namespace mxf {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

enum GemmSched { SCHED_MGROUP = 0, SCHED_KGROUP = 1 };
enum GemmEpi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2, EPI_UNPACK13 = 3 };



template <int BM, int BN, int WM, int WN>
struct Tile {
  static constexpr int BK = 128;
  static constexpr int NT = WM * WN * 64;
  static constexpr int TM = BM / WM;
  static constexpr int TN = BN / WN;
  static constexpr int FM = TM / 32;
  static constexpr int FN = TN / 32;
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = BM * BK;
  static constexpr int SA_OFF = (BM + BN) * BK;
  static constexpr int SB_OFF = SA_OFF + BM * 4;
  static constexpr int STAGE = SB_OFF + BN * 4;
  static constexpr int CA = BM * 8 / NT;  // 16-byte A chunks per thread per K step
  static constexpr int CB = BN * 8 / NT;
  // epilogue staging (per wavefront, bf16 elements): SwiGLU h tile TM x (TN/2 + 8),
  // dSwiGLU packed tile TM x (2TN + 8)
  static constexpr int EPI_SW = TM * (TN / 2 + 8) * 2;
  static constexpr int EPI_DSW = TM * (2 * TN + 8) * 2;
  static constexpr int LDS_MAIN = 2 * STAGE;
  static constexpr int LDS = LDS_MAIN > EPI_DSW * WM * WN ? LDS_MAIN : EPI_DSW * WM * WN;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/thread mismatch");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 fragments");
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ void store_out(void* C, int64_t idx, float v, int f32) {
  if (f32) reinterpret_cast<float*>(C)[idx] = v;
  else reinterpret_cast<uint16_t*>(C)[idx] = (uint16_t)bf16_bits(v);
}

template <int BM, int BN, int WM, int WN, int SCHED, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void gemm_mx_kernel(GemmParams p) {
  using T = Tile<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[T::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid / WN;
  const int wn = wid % WN;

  if (!offsets_valid(p.offs, p.counts, p.E, p.pad, p.mcap)) return;

  int e;
  int64_t m0, n0, kbeg, kend;
  const uint8_t *Ag, *Asg, *Bg, *Bsg;
  if (SCHED == SCHED_MGROUP) {
    m0 = (int64_t)blockIdx.x * BM;
    n0 = (int64_t)blockIdx.y * BN;
    if (m0 >= p.offs[p.E]) return;
    e = expert_of_row(p.offs, p.E, m0);
    kbeg = 0;
    kend = p.K;
    Ag = p.A + m0 * p.lda;
    Asg = p.As + m0 * p.ldas;
    Bg = p.B + e * p.b_es + n0 * p.ldb;
    Bsg = p.Bs + e * p.bs_es + n0 * p.ldbs;
  } else {
    e = blockIdx.z;
    m0 = (int64_t)blockIdx.x * BM;
    n0 = (int64_t)blockIdx.y * BN;
    const int64_t seg = p.offs[e + 1] - p.offs[e];
    const int64_t real = p.counts ? p.counts[e] : seg;
    kbeg = p.offs[e];
    kend = kbeg + min(seg, (real + 127) / 128 * 128);
    Ag = p.A + m0 * p.lda + kbeg;
    Asg = p.As + m0 * p.ldas + kbeg / 32;
    Bg = p.B + n0 * p.ldb + kbeg;
    Bsg = p.Bs + n0 * p.ldbs + kbeg / 32;
  }
  const int KT = (int)((kend - kbeg) / T::BK);

  v16f acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  uint4 ra[T::CA], rb[T::CB];
  uint32_t rsa = 0, rsb = 0;

  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * T::BK;
#pragma unroll
    for (int i = 0; i < T::CA; ++i) {
      const int q = tid + i * T::NT;
      ra[i] = *reinterpret_cast<const uint4*>(Ag + (int64_t)(q >> 3) * p.lda + k0 + ((q & 7) << 4));
    }
#pragma unroll
    for (int i = 0; i < T::CB; ++i) {
      const int q = tid + i * T::NT;
      rb[i] = *reinterpret_cast<const uint4*>(Bg + (int64_t)(q >> 3) * p.ldb + k0 + ((q & 7) << 4));
    }
    if (tid < BM) rsa = *reinterpret_cast<const uint32_t*>(Asg + (int64_t)tid * p.ldas + k0 / 32);
    if (tid < BN) rsb = *reinterpret_cast<const uint32_t*>(Bsg + (int64_t)tid * p.ldbs + k0 / 32);
  };
  auto sstore = [&](int stage) {
    uint8_t* base = smem + stage * T::STAGE;
#pragma unroll
    for (int i = 0; i < T::CA; ++i) {
      const int q = tid + i * T::NT;
      *reinterpret_cast<uint4*>(base + T::A_OFF + swz(q >> 3, q & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < T::CB; ++i) {
      const int q = tid + i * T::NT;
      *reinterpret_cast<uint4*>(base + T::B_OFF + swz(q >> 3, q & 7)) = rb[i];
    }
    if (tid < BM) *reinterpret_cast<uint32_t*>(base + T::SA_OFF + tid * 4) = rsa;
    if (tid < BN) *reinterpret_cast<uint32_t*>(base + T::SB_OFF + tid * 4) = rsb;
  };

  const int r32 = lane & 31;
  const int g = lane >> 5;
  if (KT > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
  }
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint8_t* base = smem + cur * T::STAGE;
    uint32_t sa[T::FM], sb[T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
      sa[i] = *reinterpret_cast<const uint32_t*>(base + T::SA_OFF + (wm * T::TM + i * 32 + r32) * 4) >> (8 * g);
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
      sb[j] = *reinterpret_cast<const uint32_t*>(base + T::SB_OFF + (wn * T::TN + j * 32 + r32) * 4) >> (8 * g);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8i af[T::FM], bf[T::FN];
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        const int row = wm * T::TM + i * 32 + r32;
        const uint4 lo = *reinterpret_cast<const uint4*>(base + T::A_OFF + swz(row, 4 * s + g));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + T::A_OFF + swz(row, 4 * s + 2 + g));
        af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        const int row = wn * T::TN + j * 32 + r32;
        const uint4 lo = *reinterpret_cast<const uint4*>(base + T::B_OFF + swz(row, 4 * s + g));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + T::B_OFF + swz(row, 4 * s + 2 + g));
        bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
          if (s == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0,
                                                                        (int)sa[i], 0, (int)sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 2,
                                                                        (int)sa[i], 2, (int)sb[j]);
        }
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogues
  const int64_t wrow0 = m0 + wm * T::TM;  // first output row of this wavefront
  const int64_t wcol0 = n0 + wn * T::TN;  // first output column of this wavefront

  if (EPI == EPI_STORE || EPI == EPI_UNPACK13) {
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int64_t row = wrow0 + i * 32 + 8 * (q >> 2) + 4 * g + (q & 3);
          const int64_t col = wcol0 + j * 32 + r32;
          if (EPI == EPI_STORE) {
            const int64_t base = (SCHED == SCHED_KGROUP) ? (int64_t)e * p.c_es : 0;
            store_out(p.C, base + row * p.ldc + col, acc[i][j][q], p.out_f32);
          } else {
            // row = packed W13 row n -> dW1 / dW3 row 32*(n/64) + n%32 of expert e
            void* dst = (row & 32) ? p.C2 : p.C;
            const int64_t frow = (row >> 6) * 32 + (row & 31);
            store_out(dst, (int64_t)e * p.c_es + frow * p.ldc + col, acc[i][j][q], p.out_f32);
          }
        }
    return;
  }

  if (EPI == EPI_SWIGLU) {
    // N = 2F (packed gate/up columns): fragment pair (2c, 2c+1) of a wavefront holds gate and
    // up columns of the same 32 h columns. g, u are rounded to BF16 (saved for backward),
    // h = BF16(silu(g) * u) is staged in LDS and quantized along rows and along columns.
    static_assert(T::FN % 2 == 0, "SwiGLU epilogue needs whole gate/up column pairs");
    constexpr int HC = T::TN / 2;       // h columns per wavefront
    constexpr int HP = HC + 8;          // LDS pitch (bf16 elements)
    const int64_t ldn = p.N;            // 2F
    const int64_t F = p.N / 2;
    __syncthreads();                    // main-loop LDS no longer needed
    uint16_t* hs = reinterpret_cast<uint16_t*>(smem) + wid * (T::TM * HP);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int jp = 0; jp < T::FN / 2; ++jp)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int rl = i * 32 + 8 * (q >> 2) + 4 * g + (q & 3);
          const int64_t row = wrow0 + rl;
          const int64_t cg = wcol0 + (2 * jp) * 32 + r32;  // gate column (packed)
          const float gv = acc[i][2 * jp][q];
          const float uv = acc[i][2 * jp + 1][q];
          const uint32_t gb = bf16_bits(gv), ub = bf16_bits(uv);
          p.h13[row * ldn + cg] = (uint16_t)gb;
          p.h13[row * ldn + cg + 32] = (uint16_t)ub;
          if (p.dbg) {
            p.dbg[row * ldn + cg] = gv;
            p.dbg[row * ldn + cg + 32] = uv;
          }
          const float gf = bf16_to_f32(gb), uf = bf16_to_f32(ub);
          const float h = gf * sigmoid_f(gf) * uf;
          hs[rl * HP + jp * 32 + r32] = (uint16_t)bf16_bits(h);
        }
    __syncthreads();
    const int64_t hcol0 = wcol0 / 2;
    // row-wise groups: (row, 32-column group)
    for (int q = lane; q < T::TM * (HC / 32); q += 64) {
      const int rl = q / (HC / 32), gi = q % (HC / 32);
      uint32_t v[16], cd[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint4 x = *reinterpret_cast<const uint4*>(hs + rl * HP + gi * 32 + t * 8);
        v[4 * t] = x.x; v[4 * t + 1] = x.y; v[4 * t + 2] = x.z; v[4 * t + 3] = x.w;
      }
      const uint32_t byte = quant32(v, cd);
      const int64_t row = wrow0 + rl;
      uint8_t* dst = p.q_r + row * F + hcol0 + gi * 32;
      *reinterpret_cast<uint4*>(dst) = make_uint4(cd[0], cd[1], cd[2], cd[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(cd[4], cd[5], cd[6], cd[7]);
      p.s_r[row * (F / 32) + (hcol0 >> 5) + gi] = (uint8_t)byte;
    }
    // column-wise groups: (column, 32-row group)
    for (int q = lane; q < HC * (T::TM / 32); q += 64) {
      const int cl = q % HC, rg = q / HC;
      uint32_t v[16], cd[8];
#pragma unroll
      for (int t = 0; t < 16; ++t)
        v[t] = (uint32_t)hs[(rg * 32 + 2 * t) * HP + cl] | ((uint32_t)hs[(rg * 32 + 2 * t + 1) * HP + cl] << 16);
      const uint32_t byte = quant32(v, cd);
      const int64_t hc = hcol0 + cl;
      uint8_t* dst = p.q_c + hc * p.mcap + wrow0 + rg * 32;
      *reinterpret_cast<uint4*>(dst) = make_uint4(cd[0], cd[1], cd[2], cd[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(cd[4], cd[5], cd[6], cd[7]);
      p.s_c[hc * (p.mcap / 32) + (wrow0 >> 5) + rg] = (uint8_t)byte;
    }
    return;
  }

  if (EPI == EPI_DSWIGLU) {
    // N = F: acc = dh. dh -> BF16; with the saved BF16 g, u: dG = dh u s (1 + g (1 - s)),
    // dU = dh g s (s = sigmoid(g)), each -> BF16, written into a packed [TM, 2TN] LDS tile
    // (gate group then up group per 32 columns) and quantized along rows and columns.
    constexpr int PC = 2 * T::TN;   // packed columns per wavefront
    constexpr int HP = PC + 8;
    const int64_t F = p.N;
    const int64_t ld13 = 2 * F;
    __syncthreads();
    uint16_t* hs = reinterpret_cast<uint16_t*>(smem) + wid * (T::TM * HP);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int rl = i * 32 + 8 * (q >> 2) + 4 * g + (q & 3);
          const int64_t row = wrow0 + rl;
          const int64_t f = wcol0 + j * 32 + r32;
          const float dv = acc[i][j][q];
          if (p.dbg) p.dbg[row * F + f] = dv;
          const float dh = bf16_to_f32(bf16_bits(dv));
          const int64_t pc = (f >> 5) * 64 + (f & 31);
          const float gf = bf16_to_f32(p.h13[row * ld13 + pc]);
          const float uf = bf16_to_f32(p.h13[row * ld13 + pc + 32]);
          const float sg = sigmoid_f(gf);
          const float dg = dh * uf * sg * (1.0f + gf * (1.0f - sg));
          const float du = dh * gf * sg;
          hs[rl * HP + j * 64 + r32] = (uint16_t)bf16_bits(dg);
          hs[rl * HP + j * 64 + 32 + r32] = (uint16_t)bf16_bits(du);
        }
    __syncthreads();
    const int64_t pcol0 = 2 * wcol0;
    for (int q = lane; q < T::TM * (PC / 32); q += 64) {
      const int rl = q / (PC / 32), gi = q % (PC / 32);
      uint32_t v[16], cd[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint4 x = *reinterpret_cast<const uint4*>(hs + rl * HP + gi * 32 + t * 8);
        v[4 * t] = x.x; v[4 * t + 1] = x.y; v[4 * t + 2] = x.z; v[4 * t + 3] = x.w;
      }
      const uint32_t byte = quant32(v, cd);
      const int64_t row = wrow0 + rl;
      uint8_t* dst = p.q_r + row * ld13 + pcol0 + gi * 32;
      *reinterpret_cast<uint4*>(dst) = make_uint4(cd[0], cd[1], cd[2], cd[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(cd[4], cd[5], cd[6], cd[7]);
      p.s_r[row * (ld13 / 32) + (pcol0 >> 5) + gi] = (uint8_t)byte;
    }
    for (int q = lane; q < PC * (T::TM / 32); q += 64) {
      const int cl = q % PC, rg = q / PC;
      uint32_t v[16], cd[8];
#pragma unroll
      for (int t = 0; t < 16; ++t)
        v[t] = (uint32_t)hs[(rg * 32 + 2 * t) * HP + cl] | ((uint32_t)hs[(rg * 32 + 2 * t + 1) * HP + cl] << 16);
      const uint32_t byte = quant32(v, cd);
      const int64_t pcg = pcol0 + cl;
      uint8_t* dst = p.q_c + pcg * p.mcap + wrow0 + rg * 32;
      *reinterpret_cast<uint4*>(dst) = make_uint4(cd[0], cd[1], cd[2], cd[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(cd[4], cd[5], cd[6], cd[7]);
      p.s_c[pcg * (p.mcap / 32) + (wrow0 >> 5) + rg] = (uint8_t)byte;
    }
    return;
  }
}

// ------------------------------------------------------------------ host launchers

constexpr int GBM = 128, GBN = 128, GWM = 2, GWN = 2;

template <int SCHED, int EPI>
static hipError_t launch(const GemmParams& p, dim3 grid, hipStream_t st) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_mx_kernel<GBM, GBN, GWM, GWN, SCHED, EPI>), grid, dim3(GWM * GWN * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace mxf

// M-grouped: C[m, n] = sum_k A[m, k] B_e[n, k] for m in expert e's segment.
// epi: 0 store (C, ldc, out_f32), 1 SwiGLU + dual quant, 2 dSwiGLU + dual quant.
hipError_t mxf_launch_gemm_mgroup(int epi, const mxf::GemmParams& p, hipStream_t st) {
  using namespace mxf;
  if (p.mcap % GBM || p.N % GBN || p.K % 128) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.mcap / GBM), (unsigned)(p.N / GBN), 1);
  switch (epi) {
    case EPI_STORE: return launch<SCHED_MGROUP, EPI_STORE>(p, grid, st);
    case EPI_SWIGLU: return launch<SCHED_MGROUP, EPI_SWIGLU>(p, grid, st);
    case EPI_DSWIGLU: return launch<SCHED_MGROUP, EPI_DSWIGLU>(p, grid, st);
    default: return hipErrorInvalidValue;
  }
}

// K-grouped: C_e[m, n] = sum over expert e's tokens k of A[m, k] B[n, k].
// epi: 0 store into C + e * c_es, 3 store with the W13 row unpack into C (dW1) / C2 (dW3).
hipError_t mxf_launch_gemm_kgroup(int epi, const mxf::GemmParams& p, hipStream_t st) {
  using namespace mxf;
  if (p.M % GBM || p.N % GBN) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.M / GBM), (unsigned)(p.N / GBN), (unsigned)p.E);
  switch (epi) {
    case EPI_STORE: return launch<SCHED_KGROUP, EPI_STORE>(p, grid, st);
    case EPI_UNPACK13: return launch<SCHED_KGROUP, EPI_UNPACK13>(p, grid, st);
    default: return hipErrorInvalidValue;
  }
}
