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
  static constexpr int SB_OFF = SA_OFF + (BM > NT ? BM : NT) * 4;  // every thread stores a scale
  static constexpr int STAGE = SB_OFF + (BN > NT ? BN : NT) * 4;   // word (extra ones are unused)
  static constexpr int CA = BM * 8 / NT;  // 16-byte A chunks per thread per K step
  static constexpr int CB = BN * 8 / NT;
  // epilogue staging (per wavefront, bf16 elements): SwiGLU h tile TM x (TN/2 + 8),
  // dSwiGLU packed tile TM x (2TN + 8)
  static constexpr int EPI_ROWS = 64;  // epilogues stage 64 rows of a wavefront tile at a time
  static constexpr int EPI_SW = EPI_ROWS * (TN / 2 + 8) * 2;
  static constexpr int EPI_DSW = EPI_ROWS * ((TN + 8) + (2 * TN + 8)) * 2;
  static constexpr int LDS_MAIN = 2 * STAGE;
  static constexpr int imax(int a, int b) { return a > b ? a : b; }
  // LDS of a kernel instance: the main loop's two stages or its epilogue's staging
  static constexpr int lds(int epi) {
    return imax(LDS_MAIN, epi == 2 ? EPI_DSW * WM * WN : epi == 1 ? EPI_SW * WM * WN : 0);
  }
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/thread mismatch");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 fragments");
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ void store_out(void* C, int64_t idx, float v, int f32) {
  if (f32) reinterpret_cast<float*>(C)[idx] = v;
  else reinterpret_cast<uint16_t*>(C)[idx] = (uint16_t)bf16_bits(v);
}

// Staging registers of one K step, held in vector registers (4 dwords per 16-byte chunk).
template <int N>
struct Stage {
  typedef unsigned int vec __attribute__((ext_vector_type(4 * N)));
};

// Global loads of one K step into the staging registers (see the kernel for the chunk map).
template <int CA, int CB>
__device__ __forceinline__ void gload(typename Stage<CA>::vec& ra, typename Stage<CB>::vec& rb,
                                      uint32_t& rsa, uint32_t& rsb, const uint8_t* a_src,
                                      const uint8_t* b_src, int64_t a_step, int64_t b_step,
                                      const uint8_t* sa_src, const uint8_t* sb_src, int64_t k0) {
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const uint4 v = *reinterpret_cast<const uint4*>(a_src + i * a_step + k0);
    ra[4 * i] = v.x; ra[4 * i + 1] = v.y; ra[4 * i + 2] = v.z; ra[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const uint4 v = *reinterpret_cast<const uint4*>(b_src + i * b_step + k0);
    rb[4 * i] = v.x; rb[4 * i + 1] = v.y; rb[4 * i + 2] = v.z; rb[4 * i + 3] = v.w;
  }
  rsa = *reinterpret_cast<const uint32_t*>(sa_src + k0 / 32);
  rsb = *reinterpret_cast<const uint32_t*>(sb_src + k0 / 32);
}

// Staging registers -> one LDS stage (A/B tiles swizzled, scale words per row).
template <int CA, int CB, int BM, int BN, int RSTEP>
__device__ __forceinline__ void sstore(uint8_t* a_lds, uint8_t* b_lds, uint8_t* sa_lds, uint8_t* sb_lds,
                                       const typename Stage<CA>::vec& ra, const typename Stage<CB>::vec& rb,
                                       uint32_t rsa, uint32_t rsb, int ab_dst, int tid) {
#pragma unroll
  for (int i = 0; i < CA; ++i)
    *reinterpret_cast<uint4*>(a_lds + ab_dst + i * RSTEP * 128) =
        make_uint4(ra[4 * i], ra[4 * i + 1], ra[4 * i + 2], ra[4 * i + 3]);
#pragma unroll
  for (int i = 0; i < CB; ++i)
    *reinterpret_cast<uint4*>(b_lds + ab_dst + i * RSTEP * 128) =
        make_uint4(rb[4 * i], rb[4 * i + 1], rb[4 * i + 2], rb[4 * i + 3]);
  *reinterpret_cast<uint32_t*>(sa_lds + tid * 4) = rsa;  // branch-free: rows >= BM / BN land
  *reinterpret_cast<uint32_t*>(sb_lds + tid * 4) = rsb;  // in unused padding
}

template <int BM, int BN, int WM, int WN, int SCHED, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void gemm_mx_kernel(GemmParams p) {
  using T = Tile<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[T::lds(EPI)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid / WN;
  const int wn = wid % WN;

  if (!offsets_valid(p.offs, p.counts, p.E, p.pad, p.mcap)) return;

  int e;
  int64_t m0, n0, kbeg, kend;
  const uint8_t *Ag, *Asg, *Bg, *Bsg;
  const int ntn = (int)(p.N / BN);
  if (SCHED == SCHED_MGROUP) {
    // Only the row tiles before offs[E] carry work: the grid is sized for m_capacity and the
    // surplus blocks exit. Blocks are dispatched round-robin over the 8 XCDs (block b runs on
    // XCD b % 8), so tile t is taken from a contiguous per-XCD range, and inside it tiles go in
    // groups of GM row tiles x all column tiles: the ~32 blocks an XCD runs at once share a
    // few A row panels and B column panels in that XCD's L2.
    constexpr int GM = 4;
    const int64_t mtu = p.offs[p.E] / BM;
    const int64_t ntiles = mtu * ntn;
    const int64_t b = blockIdx.x;
    if (b >= ntiles) return;
    const int64_t q8 = ntiles / 8, r8 = ntiles % 8, x8 = b % 8, s8 = b / 8;
    const int64_t t = x8 < r8 ? x8 * (q8 + 1) + s8 : r8 * (q8 + 1) + (x8 - r8) * q8 + s8;
    const int64_t grp = t / (GM * ntn);
    const int64_t first = grp * GM;
    const int64_t gsz = min((int64_t)GM, mtu - first);
    const int64_t within = t - grp * GM * ntn;
    m0 = (first + within % gsz) * BM;
    n0 = (within / gsz) * BN;
    e = expert_of_row(p.offs, p.E, m0);
    kbeg = 0;
    kend = p.K;
    Ag = p.A + m0 * p.lda;
    Asg = p.As + m0 * p.ldas;
    Bg = p.B + e * p.b_es + n0 * p.ldb;
    Bsg = p.Bs + e * p.bs_es + n0 * p.ldbs;
  } else {
    // Experts are taken longest-K first (their tiles start earliest, which shortens the tail);
    // within an expert, tiles go 8 row tiles fastest, so consecutive blocks -- one per XCD --
    // each keep one A row panel in their L2 while sweeping the column tiles.
    int* ksp = reinterpret_cast<int*>(smem);  // per-expert K span, then the order (LDS scratch)
    int* order = ksp + p.E;
    for (int i = tid; i < p.E; i += T::NT) {
      const int seg = p.offs[i + 1] - p.offs[i];
      const int real = p.counts ? p.counts[i] : seg;
      ksp[i] = min(seg, (real + 127) / 128 * 128);
    }
    __syncthreads();
    for (int i = tid; i < p.E; i += T::NT) {
      const int ki = ksp[i];
      int rank = 0;
      for (int j = 0; j < p.E; ++j) {
        const int kj = ksp[j];
        rank += (kj > ki) || (kj == ki && j < i);
      }
      order[rank] = i;
    }
    __syncthreads();
    const int mtn = (int)(p.M / BM);
    const int64_t per = (int64_t)mtn * ntn;
    const int64_t t = blockIdx.x;
    e = order[t / per];
    const int64_t w = t % per;
    constexpr int GMK = 8;
    const int64_t first = (w / (GMK * ntn)) * GMK;
    const int64_t gsz = min((int64_t)GMK, mtn - first);
    const int64_t within = w - first * ntn;
    m0 = (first + within % gsz) * BM;
    n0 = (within / gsz) * BN;
    kbeg = p.offs[e];
    kend = kbeg + ksp[e];
    __syncthreads();  // the LDS scratch is reused by the main loop
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

  // global -> register staging of the next K step, then register -> LDS with the XOR swizzle.
  // Chunk q = tid + i * NT of a tile is row q / 8, bytes 16 * (q % 8); since NT / 8 is a
  // multiple of 8, row % 8 and q % 8 depend on tid only, so every chunk of a thread is its
  // first chunk plus i rows-of-NT/8.
  constexpr int RSTEP = T::NT / 8;  // rows between a thread's chunks
  static_assert(RSTEP % 8 == 0, "swizzle assumes NT / 8 is a multiple of 8");
  typename Stage<T::CA>::vec ra;
  typename Stage<T::CB>::vec rb;
  uint32_t rsa = 0, rsb = 0;
  const uint8_t* a_src = Ag + (int64_t)(tid >> 3) * p.lda + ((tid & 7) << 4);
  const uint8_t* b_src = Bg + (int64_t)(tid >> 3) * p.ldb + ((tid & 7) << 4);
  const int64_t a_step = (int64_t)RSTEP * p.lda;
  const int64_t b_step = (int64_t)RSTEP * p.ldb;
  const int ab_dst = swz(tid >> 3, tid & 7);  // A and B share the in-tile layout
  const uint8_t* sa_src = Asg + (int64_t)(tid % BM) * p.ldas;  // threads past BM/BN re-read a
  const uint8_t* sb_src = Bsg + (int64_t)(tid % BN) * p.ldbs;  // valid row (stored to padding)

#define MXF_GLOAD(kt_) gload<T::CA, T::CB>(ra, rb, rsa, rsb, a_src, b_src, a_step, b_step, sa_src, sb_src, (int64_t)(kt_) * T::BK)
#define MXF_SSTORE(stage_) sstore<T::CA, T::CB, BM, BN, RSTEP>(smem + (stage_) * T::STAGE + T::A_OFF, smem + (stage_) * T::STAGE + T::B_OFF, smem + (stage_) * T::STAGE + T::SA_OFF, smem + (stage_) * T::STAGE + T::SB_OFF, ra, rb, rsa, rsb, ab_dst, tid)

  const int r32 = lane & 31;
  const int g = lane >> 5;
  if (KT > 0) {
    MXF_GLOAD(0);
    MXF_SSTORE(0);
    __syncthreads();
  }
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    // prefetch the next K step (the last iteration re-reads its own step; nothing is stored)
    MXF_GLOAD(kt + 1 < KT ? kt + 1 : kt);
    __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before this step's LDS reads / MFMAs
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
    // keep the MFMAs ahead of the LDS stores of the prefetched step, so the global-load
    // latency overlaps the matrix work instead of stalling before it
    __builtin_amdgcn_sched_barrier(0);
    // unconditional, so the K step stays one basic block: on the last step this rewrites the
    // idle buffer (last read one step earlier, before the previous barrier) and nobody reads it
    MXF_SSTORE(cur ^ 1);
    __syncthreads();
  }
#undef MXF_GLOAD
#undef MXF_SSTORE

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
    // h = BF16(silu(g) * u) is staged in LDS (64 rows at a time) and quantized along rows
    // (32-column groups) and along columns (32-row groups).
    static_assert(T::FN % 2 == 0, "SwiGLU epilogue needs whole gate/up column pairs");
    constexpr int HC = T::TN / 2;                 // h columns per wavefront
    constexpr int HP = HC + 8;                    // LDS pitch (bf16 elements)
    constexpr int RC = T::TM < 64 ? T::TM : 64;   // rows per chunk
    constexpr int FC = RC / 32;                   // fragments per chunk
    const int64_t ldn = p.N;                      // 2F
    const int64_t F = p.N / 2;
    const int64_t hcol0 = wcol0 / 2;
    uint16_t* hs = reinterpret_cast<uint16_t*>(smem) + wid * (RC * HP);
#pragma unroll
    for (int ic = 0; ic < T::FM; ic += FC) {
      __syncthreads();  // LDS free (main loop or previous chunk)
#pragma unroll
      for (int ii = 0; ii < FC; ++ii)
#pragma unroll
        for (int jp = 0; jp < T::FN / 2; ++jp)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int i = ic + ii;
            const int rl = ii * 32 + 8 * (q >> 2) + 4 * g + (q & 3);  // row within the chunk
            const int64_t row = wrow0 + i * 32 + 8 * (q >> 2) + 4 * g + (q & 3);
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
      const int64_t crow0 = wrow0 + ic * 32;  // first output row of the chunk
      for (int q = lane; q < RC * (HC / 32); q += 64) {
        const int rl = q / (HC / 32), gi = q % (HC / 32);
        uint32_t v[16], cd[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint4 x = *reinterpret_cast<const uint4*>(hs + rl * HP + gi * 32 + t * 8);
          v[4 * t] = x.x; v[4 * t + 1] = x.y; v[4 * t + 2] = x.z; v[4 * t + 3] = x.w;
        }
        const uint32_t byte = quant32(v, cd);
        const int64_t row = crow0 + rl;
        uint8_t* dst = p.q_r + row * F + hcol0 + gi * 32;
        *reinterpret_cast<uint4*>(dst) = make_uint4(cd[0], cd[1], cd[2], cd[3]);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(cd[4], cd[5], cd[6], cd[7]);
        p.s_r[row * (F / 32) + (hcol0 >> 5) + gi] = (uint8_t)byte;
      }
      for (int q = lane; q < HC * FC; q += 64) {
        const int cl = q % HC, rg = q / HC;
        uint32_t v[16], cd[8];
#pragma unroll
        for (int t = 0; t < 16; ++t)
          v[t] = (uint32_t)hs[(rg * 32 + 2 * t) * HP + cl] | ((uint32_t)hs[(rg * 32 + 2 * t + 1) * HP + cl] << 16);
        const uint32_t byte = quant32(v, cd);
        const int64_t hc = hcol0 + cl;
        uint8_t* dst = p.q_c + hc * p.mcap + crow0 + rg * 32;
        *reinterpret_cast<uint4*>(dst) = make_uint4(cd[0], cd[1], cd[2], cd[3]);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(cd[4], cd[5], cd[6], cd[7]);
        p.s_c[hc * (p.mcap / 32) + (crow0 >> 5) + rg] = (uint8_t)byte;
      }
    }
    return;
  }

  if (EPI == EPI_DSWIGLU) {
    // N = F: acc = dh. Per 64-row chunk of the wavefront tile:
    //  1. dh -> BF16 into an LDS tile [64, TN];
    //  2. row pass, one (row, 32-column group) per lane task: 16-byte loads of the saved BF16
    //     g and u (contiguous in the packed h13), dG = dh u s (1 + g (1 - s)), dU = dh g s with
    //     s = sigmoid(g), each -> BF16; both row-wise groups quantized and stored; dG, dU
    //     written into a packed LDS tile [64, 2TN] (gate group then up group per 32 columns);
    //  3. column pass over the packed tile: column-wise groups quantized and stored.
    constexpr int DP = T::TN + 8;   // dh tile pitch (bf16 elements)
    constexpr int PC = 2 * T::TN;   // packed columns per wavefront
    constexpr int HP = PC + 8;
    constexpr int RC = T::TM < 64 ? T::TM : 64;
    constexpr int FC = RC / 32;
    const int64_t F = p.N;
    const int64_t ld13 = 2 * F;
    const int64_t pcol0 = 2 * wcol0;
    uint16_t* dhs = reinterpret_cast<uint16_t*>(smem) + wid * (RC * (DP + HP));
    uint16_t* hs = dhs + RC * DP;
#pragma unroll
    for (int ic = 0; ic < T::FM; ic += FC) {
      __syncthreads();
#pragma unroll
      for (int ii = 0; ii < FC; ++ii)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int i = ic + ii;
            const int rl = ii * 32 + 8 * (q >> 2) + 4 * g + (q & 3);
            const float dv = acc[i][j][q];
            if (p.dbg) p.dbg[(wrow0 + ic * 32 + rl) * F + wcol0 + j * 32 + r32] = dv;
            dhs[rl * DP + j * 32 + r32] = (uint16_t)bf16_bits(dv);
          }
      __syncthreads();
      const int64_t crow0 = wrow0 + ic * 32;
      for (int q = lane; q < RC * (T::TN / 32); q += 64) {
        const int rl = q / (T::TN / 32), gi = q % (T::TN / 32);
        const int64_t row = crow0 + rl;
        const uint16_t* gsrc = p.h13 + row * ld13 + pcol0 + gi * 64;  // g group, then u group
        uint32_t gv[16], uv[16], dgv[16], duv[16], cd[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint4 a = *reinterpret_cast<const uint4*>(gsrc + t * 8);
          const uint4 b = *reinterpret_cast<const uint4*>(gsrc + 32 + t * 8);
          gv[4 * t] = a.x; gv[4 * t + 1] = a.y; gv[4 * t + 2] = a.z; gv[4 * t + 3] = a.w;
          uv[4 * t] = b.x; uv[4 * t + 1] = b.y; uv[4 * t + 2] = b.z; uv[4 * t + 3] = b.w;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const uint32_t d2 = *reinterpret_cast<const uint32_t*>(dhs + rl * DP + gi * 32 + 2 * t);
          uint32_t og = 0, ou = 0;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float dh = bf16_to_f32((d2 >> (16 * h)) & 0xFFFFu);
            const float gf = bf16_to_f32((gv[t] >> (16 * h)) & 0xFFFFu);
            const float uf = bf16_to_f32((uv[t] >> (16 * h)) & 0xFFFFu);
            const float sg = sigmoid_f(gf);
            og |= bf16_bits(dh * uf * sg * (1.0f + gf * (1.0f - sg))) << (16 * h);
            ou |= bf16_bits(dh * gf * sg) << (16 * h);
          }
          dgv[t] = og;
          duv[t] = ou;
        }
        uint8_t* dst = p.q_r + row * ld13 + pcol0 + gi * 64;
        uint32_t byte = quant32(dgv, cd);
        *reinterpret_cast<uint4*>(dst) = make_uint4(cd[0], cd[1], cd[2], cd[3]);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(cd[4], cd[5], cd[6], cd[7]);
        p.s_r[row * (ld13 / 32) + (pcol0 >> 5) + 2 * gi] = (uint8_t)byte;
        byte = quant32(duv, cd);
        *reinterpret_cast<uint4*>(dst + 32) = make_uint4(cd[0], cd[1], cd[2], cd[3]);
        *reinterpret_cast<uint4*>(dst + 48) = make_uint4(cd[4], cd[5], cd[6], cd[7]);
        p.s_r[row * (ld13 / 32) + (pcol0 >> 5) + 2 * gi + 1] = (uint8_t)byte;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          *reinterpret_cast<uint4*>(hs + rl * HP + gi * 64 + t * 8) =
              make_uint4(dgv[4 * t], dgv[4 * t + 1], dgv[4 * t + 2], dgv[4 * t + 3]);
          *reinterpret_cast<uint4*>(hs + rl * HP + gi * 64 + 32 + t * 8) =
              make_uint4(duv[4 * t], duv[4 * t + 1], duv[4 * t + 2], duv[4 * t + 3]);
        }
      }
      __syncthreads();
      for (int q = lane; q < PC * FC; q += 64) {
        const int cl = q % PC, rg = q / PC;
        uint32_t v[16], cd[8];
#pragma unroll
        for (int t = 0; t < 16; ++t)
          v[t] = (uint32_t)hs[(rg * 32 + 2 * t) * HP + cl] | ((uint32_t)hs[(rg * 32 + 2 * t + 1) * HP + cl] << 16);
        const uint32_t byte = quant32(v, cd);
        const int64_t pcg = pcol0 + cl;
        uint8_t* dst = p.q_c + pcg * p.mcap + crow0 + rg * 32;
        *reinterpret_cast<uint4*>(dst) = make_uint4(cd[0], cd[1], cd[2], cd[3]);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(cd[4], cd[5], cd[6], cd[7]);
        p.s_c[pcg * (p.mcap / 32) + (crow0 >> 5) + rg] = (uint8_t)byte;
      }
    }
    return;
  }
}

// ------------------------------------------------------------------ host launchers

// Tile configurations: 256x128 (wavefront tile 128x64) where the dimensions allow it, else
// 128x128 (wavefront tile 64x64). M-grouped tiles must divide pad_multiple.
template <int BM, int BN, int SCHED, int EPI>
static hipError_t launch_cfg(const GemmParams& p, hipStream_t st) {
  // 1-D grids: the kernel maps block ids to tiles (see the schedulers)
  int64_t nblk;
  if (SCHED == SCHED_MGROUP)
    nblk = (p.mcap / BM) * (p.N / BN);
  else
    nblk = (p.M / BM) * (p.N / BN) * p.E;
  if (nblk == 0) return hipSuccess;
  if (nblk > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nblk);
  hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, 2, 2, SCHED, EPI>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int SCHED, int EPI>
static hipError_t launch(const GemmParams& p, bool big_m, hipStream_t st) {
  if (big_m) return launch_cfg<256, 128, SCHED, EPI>(p, st);
  return launch_cfg<128, 128, SCHED, EPI>(p, st);
}

}  // namespace mxf

// M-grouped: C[m, n] = sum_k A[m, k] B_e[n, k] for m in expert e's segment.
// epi: 0 store (C, ldc, out_f32), 1 SwiGLU + dual quant, 2 dSwiGLU + dual quant.
hipError_t mxf_launch_gemm_mgroup(int epi, const mxf::GemmParams& p, hipStream_t st) {
  using namespace mxf;
  if (p.mcap % 128 || p.N % 128 || p.K % 128) return hipErrorInvalidValue;
  const bool big = (p.pad % 256 == 0) && (p.mcap % 256 == 0);
  switch (epi) {
    case EPI_STORE: return launch<SCHED_MGROUP, EPI_STORE>(p, big, st);
    case EPI_SWIGLU: return launch<SCHED_MGROUP, EPI_SWIGLU>(p, big, st);
    case EPI_DSWIGLU: return launch<SCHED_MGROUP, EPI_DSWIGLU>(p, big, st);
    default: return hipErrorInvalidValue;
  }
}

// K-grouped: C_e[m, n] = sum over expert e's tokens k of A[m, k] B[n, k].
// epi: 0 store into C + e * c_es, 3 store with the W13 row unpack into C (dW1) / C2 (dW3).
hipError_t mxf_launch_gemm_kgroup(int epi, const mxf::GemmParams& p, hipStream_t st) {
  using namespace mxf;
  if (p.M % 128 || p.N % 128) return hipErrorInvalidValue;
  const bool big = (p.M % 256 == 0);
  switch (epi) {
    case EPI_STORE: return launch<SCHED_KGROUP, EPI_STORE>(p, big, st);
    case EPI_UNPACK13: return launch<SCHED_KGROUP, EPI_UNPACK13>(p, big, st);
    default: return hipErrorInvalidValue;
  }
}
