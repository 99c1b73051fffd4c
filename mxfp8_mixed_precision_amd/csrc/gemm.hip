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
  static constexpr int NW = WM * WN;
  static constexpr int TM = BM / WM;
  static constexpr int TN = BN / WN;
  static constexpr int FM = TM / 32;
  static constexpr int FN = TN / 32;
  // one pipeline stage: A tile [BM][128 B], B tile [BN][128 B], then one 256-byte slot of
  // scale words per wavefront for A and for B (rows beyond BM / BN land in unused slots)
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = BM * BK;
  static constexpr int SA_OFF = (BM + BN) * BK;
  static constexpr int SB_OFF = SA_OFF + NW * 256;
  static constexpr int STAGE = SB_OFF + NW * 256;
  static constexpr int LDS_BYTES = 160 * 1024;
  static constexpr int S = LDS_BYTES / STAGE >= 4 ? 4 : LDS_BYTES / STAGE;  // stages (S-1 steps in flight)
  static constexpr int IA = BM / 8 / NW;  // 1 KB direct-to-LDS loads of the A tile, per wavefront
  static constexpr int IB = BN / 8 / NW;
  static constexpr int L = IA + IB + 2;   // loads per wavefront per K step (with the scale words)
  static constexpr int EPI_ROWS = TN > 64 ? 32 : 64;  // rows of a wavefront tile staged at a time
  static constexpr int EPI_SW = EPI_ROWS * (TN / 2 + 8) * 2;
  static constexpr int EPI_DSW = EPI_ROWS * ((TN + 8) + (2 * TN + 8)) * 2;
  static constexpr int LDS_MAIN = S * STAGE;
  static constexpr int imax(int a, int b) { return a > b ? a : b; }
  // LDS of a kernel instance: the main loop's stages or its epilogue's staging
  static constexpr int lds(int epi) {
    return imax(LDS_MAIN, epi == 2 ? EPI_DSW * NW : epi == 1 ? EPI_SW * NW : 0);
  }
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile/wavefront mismatch");
  static_assert(BM <= 64 * NW && BN <= 64 * NW, "one scale-word load per wavefront and operand");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 fragments");
  static_assert(S * STAGE <= LDS_BYTES && S >= 2, "pipeline does not fit in LDS");
  static_assert(IA % 2 == 0 && IB % 2 == 0, "the swizzle alternates between load pairs");
};

// LDS tile layout: 128-byte rows, 16-byte chunk c of row r stored at chunk c ^ ((r / 2) % 8). A
// 16-lane phase of ds_read_b128 reads 16 consecutive rows at one chunk index; with 64 banks
// (256 bytes) the even rows then cover bank slots 0-7 and the odd rows slots 8-15 once each.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

__device__ __forceinline__ void store_out(void* C, int64_t idx, float v, int f32) {
  if (f32) reinterpret_cast<float*>(C)[idx] = v;
  else reinterpret_cast<uint16_t*>(C)[idx] = (uint16_t)bf16_bits(v);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt low bits
// [3:0] and high bits [15:14]; expcnt 7 and lgkmcnt 15 mean "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Direct global -> LDS loads (gfx950 global_load_lds_dword{,x4}): lane l's bytes land at LDS
// address m0 + size * l. Written as inline asm so that the compiler's wait insertion does not
// treat every LDS read as aliasing the in-flight fills (it would drain the pipeline with
// vmcnt(0) before each read); the kernel waits on vmcnt itself. M0 is set in the same asm
// block and clobbered; the instruction has no destination VGPRs.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr)p;
}
// Address = wavefront-uniform 64-bit base (SGPRs) + per-lane 32-bit offset (one VGPR).
__device__ __forceinline__ void g2lds16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}
__device__ __forceinline__ void g2lds4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
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

  // Pipeline: S LDS stages in a ring, filled by direct global->LDS loads (no register
  // staging), S-1 K steps in flight. A wavefront's 1 KB load writes LDS bytes
  // [base, base + 1024) in lane order (16 bytes per lane), so the swizzle of the tile layout
  // is applied on the global side: the lane that lands on LDS chunk (row, c) fetches global
  // chunk (row, c ^ ((row / 2) % 8)). A load covers 8 consecutive tile rows starting at a
  // multiple of 8, lane l at row offset l / 8; so (row / 2) % 8 = 4 * (load index % 2) + l / 16
  // and the source chunk only alternates between even and odd loads.
  const int r32 = lane & 31;
  const int g = lane >> 5;
  const int64_t lrow = lane >> 3;  // row within a 1 KB load
  const uint32_t lcol0 = (uint32_t)(((lane & 7) ^ (lane >> 4)) << 4);        // even loads
  const uint32_t lcol1 = (uint32_t)(((lane & 7) ^ (4 | (lane >> 4))) << 4);  // odd loads
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);  // wavefront-uniform (SGPR) copy
  const uint8_t* a_s = Ag + (int64_t)wid_u * T::IA * 8 * p.lda;  // this wavefront's first rows
  const uint8_t* b_s = Bg + (int64_t)wid_u * T::IB * 8 * p.ldb;
  const uint32_t a_v0 = (uint32_t)(lrow * p.lda) + lcol0, a_v1 = (uint32_t)(lrow * p.lda) + lcol1;
  const uint32_t b_v0 = (uint32_t)(lrow * p.ldb) + lcol0, b_v1 = (uint32_t)(lrow * p.ldb) + lcol1;
  const uint32_t sa_v = (uint32_t)(((wid * 64 + lane) % BM) * p.ldas);
  const uint32_t sb_v = (uint32_t)(((wid * 64 + lane) % BN) * p.ldbs);
  const int64_t a8 = 8 * p.lda, b8 = 8 * p.ldb;
  const uint32_t lds0 = lds_addr(smem);
  // One of the L direct-to-LDS loads of a K step: q < IA are A-tile loads, then IB B-tile
  // loads, then the A and B scale words. q is a compile-time constant at every call.
  auto issue_one = [&](int q, int64_t k0, uint32_t st) {
    if (q < T::IA) {
      g2lds16(a_s + q * a8 + k0, (q & 1) ? a_v1 : a_v0, st + T::A_OFF + (wid_u * T::IA + q) * 1024);
    } else if (q < T::IA + T::IB) {
      const int i = q - T::IA;
      g2lds16(b_s + i * b8 + k0, (i & 1) ? b_v1 : b_v0, st + T::B_OFF + (wid_u * T::IB + i) * 1024);
    } else if (q == T::IA + T::IB) {
      g2lds4(Asg + k0 / 32, sa_v, st + T::SA_OFF + wid_u * 256);
    } else {
      g2lds4(Bsg + k0 / 32, sb_v, st + T::SB_OFF + wid_u * 256);
    }
  };

  if (KT > 0) {
    // prologue: steps 0 .. S-2 (clamped to the last step; a surplus load fills a stage that
    // is never read, which keeps every wavefront's load count per step fixed)
#pragma unroll
    for (int st = 0; st < T::S - 1; ++st) {
      const int64_t k0 = (int64_t)(st < KT ? st : KT - 1) * T::BK;
#pragma unroll
      for (int q = 0; q < T::L; ++q) issue_one(q, k0, lds0 + st * T::STAGE);
    }
  }
  constexpr int NMF = 2 * T::FM * T::FN;  // MFMAs per K step
  for (int kt = 0; kt < KT; ++kt) {
    // this wavefront's loads of step kt are done once at most (S-2) steps' loads remain
    wait_vmcnt<(T::S - 2) * T::L>();
    __syncthreads();  // every wavefront's step-kt data is in LDS; step kt-1 fully consumed
    const uint8_t* base = smem + (kt % T::S) * T::STAGE;
    // all fragments and scales of the step are read up front (LDS latency overlaps the MFMAs)
    uint32_t sa[T::FM], sb[T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
      sa[i] = *reinterpret_cast<const uint32_t*>(base + T::SA_OFF + (wm * T::TM + i * 32 + r32) * 4) >> (8 * g);
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
      sb[j] = *reinterpret_cast<const uint32_t*>(base + T::SB_OFF + (wn * T::TN + j * 32 + r32) * 4) >> (8 * g);
    v8i af[2][T::FM], bf[2][T::FN];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        const int row = wm * T::TM + i * 32 + r32;
        const uint4 lo = *reinterpret_cast<const uint4*>(base + T::A_OFF + swz(row, 4 * h + g));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + T::A_OFF + swz(row, 4 * h + 2 + g));
        af[h][i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        const int row = wn * T::TN + j * 32 + r32;
        const uint4 lo = *reinterpret_cast<const uint4*>(base + T::B_OFF + swz(row, 4 * h + g));
        const uint4 hi = *reinterpret_cast<const uint4*>(base + T::B_OFF + swz(row, 4 * h + 2 + g));
        bf[h][j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
    // MFMAs with the refill of the stage consumed at step kt-1 interleaved one load after each
    // MFMA, so that a full load queue never holds the wavefront before its matrix work
    const int nxt = kt + T::S - 1;
    const int64_t nk0 = (int64_t)(nxt < KT ? nxt : KT - 1) * T::BK;
    const uint32_t nst = lds0 + (nxt % T::S) * T::STAGE;
#pragma unroll
    for (int m = 0; m < NMF; ++m) {
      const int h = m / (T::FM * T::FN), i = (m / T::FN) % T::FM, j = m % T::FN;
      if (h == 0)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[0][i], bf[0][j], acc[i][j], 0, 0, 0,
                                                                    (int)sa[i], 0, (int)sb[j]);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[1][i], bf[1][j], acc[i][j], 0, 0, 2,
                                                                    (int)sa[i], 2, (int)sb[j]);
      if (m < T::L) issue_one(m, nk0, nst);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = NMF; q < T::L; ++q) issue_one(q, nk0, nst);  // loads beyond the MFMA count
  }
  if (KT > 0) {
    wait_vmcnt<0>();  // surplus loads must land before the epilogue reuses LDS
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
    // h = BF16(silu(g) * u) is staged in LDS (64 rows at a time) and quantized along rows
    // (32-column groups) and along columns (32-row groups).
    static_assert(T::FN % 2 == 0, "SwiGLU epilogue needs whole gate/up column pairs");
    constexpr int HC = T::TN / 2;                 // h columns per wavefront
    constexpr int HP = HC + 8;                    // LDS pitch (bf16 elements)
    constexpr int RC = T::TM < T::EPI_ROWS ? T::TM : T::EPI_ROWS;  // rows per chunk
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
    constexpr int RC = T::TM < T::EPI_ROWS ? T::TM : T::EPI_ROWS;
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

// Tile configurations (4 wavefronts): 256x128 (wavefront tile 128x64) where the dimensions
// allow, else 128x128 (64x64). M-grouped row tiles divide pad_multiple. (256x256 with a
// 128x128 wavefront tile measured slower: only two LDS stages fit and its epilogues spill.)
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
