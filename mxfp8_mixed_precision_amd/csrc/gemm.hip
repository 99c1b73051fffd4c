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
// Operands in HBM: codes in 64-k panels (64 k of 16 consecutive rows are one contiguous
// kilobyte), scales in 128-k planes (the four scale bytes of a row for 128 k are one word;
// consecutive rows' words are adjacent) -- see kernels.h.
//
// Tiling: block tile BM x BN (256 x 256, 256 x 128 or 128 x 128), four wavefronts in a 2 x 2
// grid, each owning a (BM/2) x (BN/2) tile of 32x32 MFMA fragments (accumulators in AGPRs).
// K advances in 64-k stages through a ring of four LDS stages filled by direct global->LDS
// loads (one 1 KB load per 16 rows; three stages in flight while one is consumed); the
// fragments of the next stage are read into a second register set while the matrix
// instructions of the current one run. The dSwiGLU GEMM instead runs two blocks per CU (a
// three-stage ring in 80 KB, fragments read at the start of each stage, at most 256 registers),
// so that each block's long epilogue runs beside the other block's matrix instructions. LDS rows are 64 bytes; the 16-byte chunk index is
// XOR-swizzled with (row / 4) % 4 so that a 16-lane phase of ds_read_b128 over 16
// consecutive rows hits 16 distinct bank groups.
//
// Schedulers (expert-offset driven; no host synchronisation):
//   M-grouped (FC1, FC2, both dgrads): A rows are the padded expert-major tokens; the block
//     at row tile m0 finds its expert e from the device offsets (offs[e] <= m0 < offs[e+1])
//     and multiplies by expert e's B. Tiles at or past offs[E] exit. BM divides
//     pad_multiple, so no tile straddles two experts. Tiles are ordered per XCD for L2
//     reuse, and the last (T mod #CU) tiles are split into sub-tiles (see TailCfg).
//   K-grouped (both wgrads): one tile grid per expert, experts longest-K first (index order
//     from 64 experts on); K runs over
//     the expert's token segment (the real rows rounded up to 128; pad rows are zero codes).
//     A zero-token expert runs no K step and stores zeros.
#include <atomic>
#include <type_traits>

#include "kernels.h"
#include "mx_device.h"

namespace mxf {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

enum GemmSched { SCHED_MGROUP = 0, SCHED_KGROUP = 1 };
enum GemmEpi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2, EPI_UNPACK13 = 3 };



// OCC = blocks resident per CU. OCC 1: a four-stage ring in up to 160 KB of LDS, fragments
// double-buffered in registers. OCC 2: a three-stage ring in at most 80 KB and at most 256
// registers per lane, so a second block shares every SIMD and its matrix instructions run while
// this block waits on loads or works through its epilogue.
template <int BM, int BN, int WM, int WN, int OCC = 1>
struct Tile {
  static constexpr int BK = 64;   // K per pipeline stage (one MFMA K step)
  static constexpr int S = OCC == 2 ? 3 : 4;  // stages in the LDS ring
  static constexpr int NT = WM * WN * 64;
  static constexpr int NW = WM * WN;
  static constexpr int TM = BM / WM;
  static constexpr int TN = BN / WN;
  static constexpr int FM = TM / 32;
  static constexpr int FN = TN / 32;
  // one stage: A tile [BM][64 B], B tile [BN][64 B]. The scale words (four E8M0 bytes of
  // 128 k per row) of a 128-k block serve its two stages: the even stage loads them into a
  // ring of NSC scale slots after the stage slots (one 256-byte piece per wavefront for A,
  // then for B; rows beyond BM / BN land in unused bytes), the odd stage reads the same slot.
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = BM * BK;
  static constexpr int STAGE = (BM + BN) * BK;
  static constexpr int NSC = OCC == 2 ? 3 : 4;  // scale slots (a power of two where LDS allows)
  static constexpr int SC_OFF = S * STAGE;
  static constexpr int SC_SLOT = 2 * NW * 256;
  static constexpr int LDS_BYTES = 160 * 1024 / OCC;
  static constexpr int IA = BM / 16 / NW;  // 1 KB direct-to-LDS loads (16 rows) of A, per wavefront
  static constexpr int IB = BN / 16 / NW;
  static constexpr int LO = IA + IB;       // loads per wavefront for an odd stage
  static constexpr int L = LO + 2;         // for an even stage (with the scale words)
  // epilogue staging: BF16 output tile; SwiGLU: row-major h tile + transposed codes + scales;
  // dSwiGLU (one wavefront row at a time): packed dG/dU tile + transposed codes + scales
  static constexpr int EPI_ST = BM * (BN + 8) * 2;
  static constexpr int EPI_SW = BM * (BN / 2 + 8) * 2 + (BN / 2) * (BM + 8) + (BN / 2) * (BM / 32);
  // dSwiGLU passes: a wavefront's fragment rows in two halves (dSwiGLU runs on 64-column
  // wavefront tiles, FN <= 2); under OCC 2 one fragment row per pass (the staging then fits
  // the smaller LDS share)
  static constexpr int DSW_NP = (OCC == 2 && FM >= 2) ? FM : 2;
  static constexpr int DSW_SR = WM * (TM / DSW_NP);  // staged rows per pass
  // passes of 32 rows per wavefront keep two passes' column codes (whole 64-token panel rows)
  static constexpr int DSW_PAIR = (TM / DSW_NP == 32 && DSW_NP % 2 == 0) ? 2 : 1;
  static constexpr int EPI_DSW = DSW_SR * (2 * BN + 8) * 2 + 2 * BN * (DSW_PAIR * DSW_SR + 8) +
                                 2 * BN * (DSW_PAIR * DSW_SR / 32);
  static constexpr int LDS_MAIN = S * STAGE + NSC * SC_SLOT;
  static constexpr int imax(int a, int b) { return a > b ? a : b; }
  // LDS of a kernel instance: the main loop's stages or its epilogue's staging
  static constexpr int lds(int epi) {
    return imax(LDS_MAIN, epi == 2 ? EPI_DSW : epi == 1 ? EPI_SW : EPI_ST);
  }
  static_assert(BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "tile/wavefront mismatch");
  static_assert(BM <= 64 * NW && BN <= 64 * NW, "one scale-word load per wavefront and operand");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 fragments");
  static_assert(IA <= 4 && IB <= 4, "runs of at most four 1 KB loads per operand and wavefront");
  static_assert(LDS_MAIN <= LDS_BYTES, "pipeline does not fit in LDS");
  static_assert(OCC == 2 ? (S == 3 && L + LO <= 63) : (S % 2 == 0 && (S / 2) * (L + LO) <= 63),
                "loads in flight exceed the vmcnt range");
};

// LDS tile layout: 64-byte rows, 16-byte chunk c of row r stored at chunk c ^ ((r / 4) % 4). A
// 16-lane phase of ds_read_b128 reads 16 consecutive rows at one chunk index; four rows share
// a 256-byte bank window and the XOR spreads the four windows' chunks, so the 16 reads hit
// 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

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
__device__ __forceinline__ void g2lds4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
}
// Kilobyte q of a run of consecutive 1 KB loads that share one global base and one M0: the
// instruction offset (1024 q) moves both the global and the LDS address, so a whole operand of
// a stage needs one 64-bit base and one M0 value. q is a compile-time constant after unrolling.
template <int OFF>
__device__ __forceinline__ void g2lds16_off(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3" ::"s"(lds), "v"(voff), "s"(sbase),
               "i"(OFF) : "memory", "m0");
}
__device__ __forceinline__ void g2lds16_q(int q, const void* sbase, uint32_t voff, uint32_t lds) {
  switch (q) {
    case 0: g2lds16_off<0>(sbase, voff, lds); break;
    case 1: g2lds16_off<1024>(sbase, voff, lds); break;
    case 2: g2lds16_off<2048>(sbase, voff, lds); break;
    default: g2lds16_off<3072>(sbase, voff, lds); break;
  }
}

// LDS reads through a 32-bit LDS byte address; constant offsets added to the returned pointer
// fold into the instruction's offset field.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4_t lds_u4;
typedef __attribute__((address_space(3))) const uint8_t lds_u8;
__device__ __forceinline__ lds_u4* lds16_at(uint32_t a) { return (lds_u4*)(uintptr_t)a; }
__device__ __forceinline__ lds_u8* lds8_at(uint32_t a) { return (lds_u8*)(uintptr_t)a; }

// One output tile (rows [m0, m0 + BM), columns [n0, n0 + BN), contraction over [kbeg, kend)):
// the pipelined main loop and the epilogue. smem holds Tile<BM, BN, WM, WN>::lds(EPI) bytes.
// DBG: the fused epilogues also write the FP32 accumulator to p.dbg (a test option, launched
// only when p.dbg is set). Run-time-dead paths compiled into the product kernels cost time even
// when not taken: with the debug stores and the 64-or-more-experts offsets path (BIGE in
// gemm_block) as template choices, FC1 + SwiGLU measured 156.0 against 160.1 us, FC2 76.6
// against 78.1, FC2 dgrad + dSwiGLU 127.3 against 128.6 (three A/B pairs).
template <int BM, int BN, int WM, int WN, int SCHED, int EPI, int OCC, bool DBG = false>
__device__ __forceinline__ void tile_run(const GemmParams& p, uint8_t* smem, int e, int64_t m0, int64_t n0,
                                         int64_t kbeg, int64_t kend) {
  using T = Tile<BM, BN, WM, WN, OCC>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid / WN;
  const int wn = wid % WN;
  // operand panels of the tile (M-grouped: kbeg = 0 and B is expert e's; K-grouped: b_es = 0)
  const uint8_t* Ag = p.A + m0 * 64 + (kbeg >> 6) * p.akp;
  const uint8_t* Asg = p.As + m0 * p.ldas + (kbeg >> 7) * p.kbsa;
  const uint8_t* Bg = p.B + e * p.b_es + n0 * 64 + (kbeg >> 6) * p.bkp;
  const uint8_t* Bsg = p.Bs + e * p.bs_es + n0 * p.ldbs + (kbeg >> 7) * p.kbsb;
  const int tr0 = wm * T::TM;  // first row / column of this wavefront within the block tile
  const int tc0 = wn * T::TN;
  const int KT = (int)((kend - kbeg) / T::BK);  // stages (even: K is a multiple of 128)

  // Accumulator layout. Fragment (i, j) covers tile rows tr0 + 32 i + [0, 32) and columns
  // tc0 + 32 j + [0, 32). Normal: lane (r32, g) holds column r32, rows 8 (q / 4) + 4 g + q % 4
  // of it. Transposed (TRACC: the operands swap places in the matrix instruction, which then
  // computes the fragment of C^T): lane (r32, g) holds row r32, columns 8 (q / 4) + 4 g + q % 4,
  // so each group of four accumulators is four consecutive columns of one row -- one 8-byte
  // BF16 write. The plain-store epilogues use it; SwiGLU and dSwiGLU pair gate/up fragments
  // column-wise and keep the normal layout.
  constexpr bool TRACC = (EPI == EPI_STORE || EPI == EPI_UNPACK13);
  v16f acc[T::FM][T::FN];
  // zeroed after the first loads are issued (a few hundred cycles that then overlap their latency)
  auto zero_acc = [&]() {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  };

  // Direct global->LDS loads: a wavefront's 1 KB load covers 16 consecutive tile rows (starting
  // at a multiple of 16) of one 64-k panel -- one contiguous kilobyte of the operand -- and
  // writes LDS bytes [base, base + 1024) in lane order, 16 bytes per lane: lane l lands on row
  // l / 4, LDS chunk l % 4. The swizzle is applied on the global side: that lane fetches chunk
  // (l % 4) ^ ((row / 4) % 4) = (l % 4) ^ (l / 16), the same for every load, so one per-lane
  // offset serves them all.
  const int r32 = lane & 31;
  const int g = lane >> 5;
  const int64_t lrow = lane >> 2;
  const uint32_t lcol = (uint32_t)(((lane & 3) ^ (lane >> 4)) << 4);
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);  // wavefront-uniform (SGPR) copy
  const uint8_t* a_s = Ag + (int64_t)wid_u * T::IA * 1024;  // this wavefront's first rows
  const uint8_t* b_s = Bg + (int64_t)wid_u * T::IB * 1024;
  const uint32_t a_v = (uint32_t)(lrow * 64) + lcol;
  const uint32_t b_v = a_v;
  const uint32_t sa_v = (uint32_t)(((wid * 64 + lane) % BM) * p.ldas);
  const uint32_t sb_v = (uint32_t)(((wid * 64 + lane) % BN) * p.ldbs);
  const uint32_t lds0 = lds_addr(smem);
  // One of the direct-to-LDS loads of stage ks into the LDS slot of stage kt (ks == kt, or
  // a surplus load of the last stage into a free slot, which keeps every step's load count
  // and waits the same): q < IA are A-tile loads, then IB B-tile loads, then (even stages
  // only) the A and B scale words of the 128-k block holding the stage, into scale slot
  // (kt / 2) % NSC. q is a compile-time constant.
  // A wavefront's IA (IB) kilobytes of an operand are consecutive in HBM and in LDS, so they
  // share one global base and one M0 value (g2lds16_q adds 1024 q to both).
  auto issue_one = [&](int q, int ks, int kt) {
    const uint64_t ku = (uint32_t)ks;  // 0 <= ks < KT
    const uint32_t st = lds0 + (kt % T::S) * T::STAGE;
    const uint32_t sc = lds0 + T::SC_OFF + ((kt >> 1) % T::NSC) * T::SC_SLOT;
    if (q < T::IA) {
      g2lds16_q(q, a_s + ku * (uint64_t)p.akp, a_v, st + T::A_OFF + wid_u * T::IA * 1024);
    } else if (q < T::IA + T::IB) {
      g2lds16_q(q - T::IA, b_s + ku * (uint64_t)p.bkp, b_v, st + T::B_OFF + wid_u * T::IB * 1024);
    } else if (q == T::IA + T::IB) {
      g2lds4(Asg + (ku >> 1) * (uint64_t)p.kbsa, sa_v, sc + wid_u * 256);
    } else {
      g2lds4(Bsg + (ku >> 1) * (uint64_t)p.kbsb, sb_v, sc + T::NW * 256 + wid_u * 256);
    }
  };

  constexpr int NMF = T::FM * T::FN;  // MFMAs per stage
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if constexpr (OCC == 2) {
    // Three-slot ring, one register set. Step kt: wait until stage kt has landed (stage kt+1's
    // loads may still be in flight), pass the block barrier (every wavefront has consumed stage
    // kt-1, whose slot is (kt+2) % 3), issue stage kt+2 into that slot, read stage kt's
    // fragments and run its matrix instructions. The LDS read latency and the load waits are
    // covered by the other block on the same SIMDs. Past the end a surplus copy of the last
    // stage is loaded, so every step's loads and waits are the same.
    v8i fa[T::FM], fb[T::FN];
    uint32_t sa[T::FM], sb[T::FN];
    auto read_stage = [&](int kt, auto par) {
      constexpr int B = decltype(par)::value;  // kt % 2: which 32-k groups of the scale word
      const uint8_t* base = smem + (kt % T::S) * T::STAGE;
      const uint8_t* sbase = smem + T::SC_OFF + ((kt >> 1) % T::NSC) * T::SC_SLOT;
#pragma unroll
      for (int i = 0; i < T::FM; ++i) sa[i] = sbase[(tr0 + i * 32 + r32) * 4 + 2 * B + g];
#pragma unroll
      for (int j = 0; j < T::FN; ++j) sb[j] = sbase[T::NW * 256 + (tc0 + j * 32 + r32) * 4 + 2 * B + g];
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
          const uint4 v = *reinterpret_cast<const uint4*>(base + T::B_OFF + swz(tc0 + j * 32 + r32, 2 * hi + g));
          fb[j][4 * hi] = (int)v.x; fb[j][4 * hi + 1] = (int)v.y;
          fb[j][4 * hi + 2] = (int)v.z; fb[j][4 * hi + 3] = (int)v.w;
        }
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
          const uint4 v = *reinterpret_cast<const uint4*>(base + T::A_OFF + swz(tr0 + i * 32 + r32, 2 * hi + g));
          fa[i][4 * hi] = (int)v.x; fa[i][4 * hi + 1] = (int)v.y;
          fa[i][4 * hi + 2] = (int)v.z; fa[i][4 * hi + 3] = (int)v.w;
        }
    };
    if (KT > 0) {  // stages 0 and 1 (KT is even, so stage 1 exists)
#pragma unroll
      for (int q = 0; q < T::L; ++q) issue_one(q, 0, 0);
#pragma unroll
      for (int q = 0; q < T::LO; ++q) issue_one(q, 1, 1);
    }
    zero_acc();
    auto step2 = [&](int kt, auto par) {
      constexpr int P = decltype(par)::value;
      wait_vmcnt<P ? T::L : T::LO>();  // stage kt landed; stage kt+1 (odd: LO loads) may be in flight
      __syncthreads();
      const int ks = kt + 2 < KT ? kt + 2 : KT - 1;
#pragma unroll
      for (int q = 0; q < (P ? T::LO : T::L); ++q) issue_one(q, ks, kt + 2);  // stage kt+2 has parity P
      read_stage(kt, par);
#pragma unroll
      for (int m = 0; m < NMF; ++m) {
        const int i = m / T::FN, j = m % T::FN;
        if constexpr (TRACC)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0, (int)sb[j], 0,
                                                                      (int)sa[i]);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, (int)sa[i], 0,
                                                                      (int)sb[j]);
      }
    };
    for (int kt = 0; kt < KT; kt += 2) {
      step2(kt, I0());
      step2(kt + 1, I1());
    }
    if (KT > 0) wait_vmcnt<0>();  // no load may still target LDS when the epilogue reuses it
  } else {
  // Fragments of one stage in registers: A/B operands and this lane's two E8M0 scale bytes
  // (its 32-k group of the stage: byte 2 * (kt % 2) + g of the row's scale word, read alone so
  // that the matrix instruction takes it with op_sel 0).
  v8i fa[2][T::FM], fb[2][T::FN];
  uint32_t sa[2][T::FM], sb[2][T::FN];
  // LDS reads of stage kt into register set kt % 2, as a list of NR reads so that they can be
  // interleaved with the matrix instructions of the previous stage. Read r < 2 FM: A fragment
  // r / 2, half r % 2 (k bytes [16g, 16g+16) or [32+16g, 32+16g+16)); then 2 FN B reads; then
  // FM + FN scale bytes.
  constexpr int NR = 2 * (T::FM + T::FN) + T::FM + T::FN;
  // This lane's LDS byte addresses in ring slot 0 and scale slot 0: fragment rows tr0 + r32
  // (A) and tc0 + r32 (B) in k half hi, and the row's scale word at byte g. Fragment i (j) is
  // 2048 i bytes further (whole 32-row steps keep the swizzle) and its scale word 128 i further,
  // so per stage only the slot offsets change and every read takes a constant offset.
  const uint32_t rd_a0 = lds0 + T::A_OFF + swz(tr0 + r32, g), rd_a1 = lds0 + T::A_OFF + swz(tr0 + r32, 2 + g);
  const uint32_t rd_b0 = lds0 + T::B_OFF + swz(tc0 + r32, g), rd_b1 = lds0 + T::B_OFF + swz(tc0 + r32, 2 + g);
  const uint32_t rd_sa = lds0 + T::SC_OFF + (tr0 + r32) * 4 + g;
  const uint32_t rd_sb = lds0 + T::SC_OFF + T::NW * 256 + (tc0 + r32) * 4 + g;
  struct ReadBase { uint32_t a0, a1, b0, b1, sa, sb; };
  auto read_base = [&](int kt) {  // addresses of stage kt's slots
    const uint32_t so = (uint32_t)(kt % T::S) * T::STAGE;
    const uint32_t sc = (uint32_t)((kt >> 1) % T::NSC) * T::SC_SLOT;
    return ReadBase{rd_a0 + so, rd_a1 + so, rd_b0 + so, rd_b1 + so, rd_sa + sc, rd_sb + sc};
  };
  auto read_one = [&](int r, const ReadBase& rb, auto par) {
    constexpr int B = decltype(par)::value;  // kt % 2
    if (r < 2 * T::FM) {
      const int i = r >> 1, hi = r & 1;
      const u32x4_t v = lds16_at(hi ? rb.a1 : rb.a0)[i * 128];
      fa[B][i][4 * hi] = (int)v.x; fa[B][i][4 * hi + 1] = (int)v.y;
      fa[B][i][4 * hi + 2] = (int)v.z; fa[B][i][4 * hi + 3] = (int)v.w;
    } else if (r < 2 * (T::FM + T::FN)) {
      const int j = (r - 2 * T::FM) >> 1, hi = r & 1;
      const u32x4_t v = lds16_at(hi ? rb.b1 : rb.b0)[j * 128];
      fb[B][j][4 * hi] = (int)v.x; fb[B][j][4 * hi + 1] = (int)v.y;
      fb[B][j][4 * hi + 2] = (int)v.z; fb[B][j][4 * hi + 3] = (int)v.w;
    } else if (r < 2 * (T::FM + T::FN) + T::FM) {
      const int i = r - 2 * (T::FM + T::FN);
      sa[B][i] = lds8_at(rb.sa)[i * 128 + 2 * B];
    } else {
      const int j = r - 2 * (T::FM + T::FN) - T::FM;
      sb[B][j] = lds8_at(rb.sb)[j * 128 + 2 * B];
    }
  };

  // Pipeline (S = 4 stages in an LDS ring, register double buffering): at step kt the
  // wavefront waits until stage kt+1 has landed (the loads of stages kt+2 and kt+3 may remain
  // in flight) and passes the block barrier, after which stage kt+1 is visible to all and
  // every wavefront holds stage kt in registers (its LDS reads completed before the barrier),
  // so stage kt's slot takes the loads of stage kt+4. The MFMAs on stage kt are interleaved
  // with the LDS reads of stage kt+1 and those loads. Every step but the last two loads a
  // stage (past the end: a surplus copy of the last stage), so the waits are the same
  // everywhere; steps are instantiated with compile-time flags so that each interleaved
  // sequence is one basic block.
  if (KT > 0) {
#pragma unroll
    for (int st = 0; st < T::S; ++st) {
#pragma unroll
      for (int q = 0; q < ((st & 1) ? T::LO : T::L); ++q) issue_one(q, st < KT ? st : KT - 1, st);
    }
  }
  zero_acc();
  if (KT > 0) {
    wait_vmcnt<2 * T::LO + T::L>();  // stage 0 landed; stages 1 - 3 may be in flight
    __syncthreads();
    const ReadBase rb0 = read_base(0);
#pragma unroll
    for (int r = 0; r < NR; ++r) read_one(r, rb0, I0());
  }
  // step kt (P = kt % 2); MORE: stage kt+1 exists; LOAD: load stage kt+4 (clamped)
  auto step = [&](int kt, auto par, auto more, auto load) {
    constexpr int P = decltype(par)::value;
    constexpr bool MORE = decltype(more)::value, LOAD = decltype(load)::value;
    constexpr int LL = P ? T::LO : T::L;  // loads of stage kt + 4 (same parity as kt)
    if (MORE) wait_vmcnt<T::L + T::LO>();  // stage kt+1 landed; kt+2 and kt+3 may be in flight
    __syncthreads();
    const int ks = kt + 4 < KT ? kt + 4 : KT - 1;
    const ReadBase rb = read_base(kt + 1);
#pragma unroll
    for (int m = 0; m < NMF; ++m) {
      const int i = m / T::FN, j = m % T::FN;
      if constexpr (TRACC)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[P][j], fa[P][i], acc[i][j], 0, 0, 0,
                                                                    (int)sb[P][j], 0, (int)sa[P][i]);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[P][i], fb[P][j], acc[i][j], 0, 0, 0,
                                                                    (int)sa[P][i], 0, (int)sb[P][j]);
      if (MORE) {
#pragma unroll
        for (int r = m * NR / NMF; r < (m + 1) * NR / NMF; ++r)
          read_one(r, rb, std::integral_constant<int, 1 - P>());
      }
      if (LOAD && m < LL) issue_one(m, ks, kt + 4);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (LOAD) {
#pragma unroll
      for (int q = NMF; q < LL; ++q) issue_one(q, ks, kt + 4);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  int kt = 0;
  for (; kt + 2 < KT; kt += 2) {
    step(kt, I0(), T_(), T_());
    step(kt + 1, I1(), T_(), T_());
  }
  if (KT > 0) {  // the last two stages (KT is even)
    step(kt, I0(), T_(), F_());
    step(kt + 1, I1(), F_(), F_());
  }
  if (KT > 0) {
    wait_vmcnt<0>();  // no load may still target LDS when the epilogue reuses it
  }
  }

  // ------------------------------------------------------------------ epilogues
  // The pipeline LDS is idle after the main loop; every epilogue stages through it so that
  // global stores are 16-byte, row-contiguous runs (a wavefront store covers whole lines).
  const int64_t wrow0 = m0 + wm * T::TM;  // first output row of this wavefront
  const int64_t wcol0 = n0 + wn * T::TN;  // first output column of this wavefront
  __syncthreads();  // every wavefront has finished reading the last stage

  if (EPI == EPI_STORE || EPI == EPI_UNPACK13) {
    const int64_t ebase = (SCHED == SCHED_KGROUP) ? (int64_t)e * p.c_es : 0;
    if (p.out_f32) {
      // fp32 output (a test/debug option): direct stores from the accumulator layout
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        // fragment rows are 32-aligned: a packed W13 row n goes to dW1 (n % 64 < 32) or dW3,
        // row 32 * (n / 64) + n % 32 of expert e
        const int64_t fr = wrow0 + i * 32;
        float* base = (EPI == EPI_STORE)
                          ? reinterpret_cast<float*>(p.C) + ebase + fr * p.ldc
                          : reinterpret_cast<float*>((fr & 32) ? p.C2 : p.C) + ebase + (fr >> 6) * 32 * p.ldc;
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q)
            base[r32 * p.ldc + wcol0 + j * 32 + 8 * (q >> 2) + 4 * g + (q & 3)] = acc[i][j][q];
      }
      return;
    }
    // BF16 tile [BM][BN] in LDS (8-byte writes of four columns), then 16-byte row-contiguous
    // copies. Row stride BN + 8 elements: 16-byte aligned rows for the copy-out reads.
    constexpr int CP = BN + 8;
    uint16_t* cs = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        // the fragment stays in its AGPRs until here: its copies to VGPRs are made one fragment
        // at a time, not all 256 ahead of the branch above (which spilled)
        asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t lo = bf16x2_bits(acc[i][j][4 * c], acc[i][j][4 * c + 1]);
          const uint32_t hi = bf16x2_bits(acc[i][j][4 * c + 2], acc[i][j][4 * c + 3]);
          *reinterpret_cast<uint2*>(cs + (tr0 + i * 32 + r32) * CP + tc0 + j * 32 + 8 * c + 4 * g) =
              make_uint2(lo, hi);
        }
      }
    __syncthreads();
    constexpr int CPR = BN / 8;  // 16-byte chunks per row
    static_assert((BM * CPR) % T::NT == 0, "whole copy rounds");
#pragma unroll 2
    for (int it = 0; it < BM * CPR / T::NT; ++it) {
      const int t = it * T::NT + tid;
      const int r = t / CPR, c = t % CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(cs + r * CP + c * 8);
      const int64_t row = m0 + r, col = n0 + c * 8;
      uint16_t* dst;
      if (EPI == EPI_STORE) {
        dst = reinterpret_cast<uint16_t*>(p.C) + ebase + row * p.ldc + col;
      } else {
        dst = reinterpret_cast<uint16_t*>((row & 32) ? p.C2 : p.C) + ebase +
              ((row >> 6) * 32 + (row & 31)) * p.ldc + col;
      }
      store16_nt(dst, v);  // y, dx, dW are not read again by the library
    }
    return;
  }

  if (EPI == EPI_SWIGLU) {
    // N = 2F (packed gate/up columns): fragment pair (2c, 2c+1) of a wavefront holds the gate
    // and up columns of the same 32 h columns, in the same accumulator slots. Per pair:
    //  * g, u are rounded to BF16 and saved (for the backward pass) as one 4 KB record in
    //    accumulator order: four contiguous-kilobyte stores, no staging;
    //  * h = BF16(silu(g) * u); its column-wise groups (32 rows of one column: this lane's 16
    //    slots plus lane l^32's) are quantized in registers and the codes staged, transposed,
    //    in LDS; h itself is staged row-major for the row-wise groups.
    // Then the whole block quantizes the row-wise groups and copies the column codes out.
    static_assert(T::FN % 2 == 0, "SwiGLU epilogue needs whole gate/up column pairs");
    constexpr int HCB = BN / 2;   // h columns of the block
    constexpr int HP = HCB + 8;   // row-major h tile pitch (bf16)
    constexpr int QP = BM + 8;    // transposed code tile pitch (bytes)
    constexpr int SG = BM / 32;   // column-wise groups per column in the block
    const int64_t F = p.N / 2;
    const int64_t hc0 = n0 / 2;
    uint16_t* hR = reinterpret_cast<uint16_t*>(smem);
    uint8_t* qT = smem + BM * HP * 2;
    uint8_t* sT = qT + HCB * QP;
    // Row staging two columns at a time: word t of a lane holds rows R, R+1 of its column
    // (slots 2t, 2t+1), lane l ^ 1 the same rows of the neighbouring column. After one lane
    // swap, an even lane writes row R of columns (c, c+1), an odd lane row R+1 of (c-1, c):
    // one 4-byte LDS write per word instead of two 2-byte writes.
    const bool odd_lane = (lane & 1) != 0;
    const uint32_t pr_sel = odd_lane ? 0x03020706u : 0x05040100u;  // {swapped, mine} byte picks
    const int pr_off = odd_lane ? HP - 1 : 0;
    if (DBG && p.dbg) {
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q)
            p.dbg[(wrow0 + i * 32 + 8 * (q >> 2) + 4 * g + (q & 3)) * p.N + wcol0 + j * 32 + r32] = acc[i][j][q];
    }
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
#pragma unroll
      for (int jp = 0; jp < T::FN / 2; ++jp) {
        const int hcl = tc0 / 2 + jp * 32 + r32;  // h column within the block
        uint32_t gw[8], uw[8], hw[8];  // slots 2t, 2t+1 as packed BF16 pairs
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          gw[t] = bf16x2_bits(acc[i][2 * jp][2 * t], acc[i][2 * jp][2 * t + 1]);
          uw[t] = bf16x2_bits(acc[i][2 * jp + 1][2 * t], acc[i][2 * jp + 1][2 * t + 1]);
          hw[t] = swiglu_h2(gw[t], uw[t]);
        }
        const int64_t rec = ((wrow0 + i * 32) >> 5) * (F >> 5) + ((hc0 + tc0 / 2 + jp * 32) >> 5);
        // record layout: four 1 KB runs (gate slots 0-7, gate 8-15, up 0-7, up 8-15), lane l's
        // 16 bytes at 16 l in each, so every store is one contiguous kilobyte
        uint4* dg = reinterpret_cast<uint4*>(p.h13 + rec * 2048) + lane;
        // saved for the backward pass: non-temporal (keeps the L2 for the GEMM operands)
        store16_nt(dg, make_uint4(gw[0], gw[1], gw[2], gw[3]));
        store16_nt(dg + 64, make_uint4(gw[4], gw[5], gw[6], gw[7]));
        store16_nt(dg + 128, make_uint4(uw[0], uw[1], uw[2], uw[3]));
        store16_nt(dg + 192, make_uint4(uw[4], uw[5], uw[6], uw[7]));
        uint32_t am = amax16(hw);
        am = max(am, (uint32_t)__shfl_xor((int)am, 32));
        const Scale s = scale_from_amax(am);
        const int rl = tr0 + i * 32 + 4 * g;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          *reinterpret_cast<uint32_t*>(qT + hcl * QP + rl + 8 * k) = cvt4(hw[2 * k], hw[2 * k + 1], s);
        sT[hcl * SG + (tr0 >> 5) + i] = (uint8_t)s.byte;  // lanes l and l ^ 32 write the same byte
#pragma unroll
        for (int t = 0; t < 8; ++t)
          *reinterpret_cast<uint32_t*>(hR + (rl + 8 * (t >> 1) + 2 * (t & 1)) * HP + hcl + pr_off) =
              __builtin_amdgcn_perm(dpp_xor1(hw[t]), hw[t], pr_sel);
      }
    }
    __syncthreads();
    // row-wise groups: one task = 16 columns of a row, four tasks (four lanes) per 64-column
    // panel row, consecutive rows on consecutive lane quads, so a wavefront stores a contiguous
    // kilobyte of a panel; lanes 2c and 2c+1 hold one group
    // A quad handles one row in each of the NPAN panels of the tile (the panel loop is inner),
    // so its first lane gathers the row's 2 NPAN scale bytes (group 2P+1 from lane 2 of the
    // quad) and stores them as one word (NPAN = 2) or halfword (NPAN = 1) of the 128-k plane.
    constexpr int CPR = HCB / 16;
    constexpr int NPAN = CPR / 4;  // 64-column panels of the tile's h columns (1 or 2)
    static_assert(BM % 64 == 0 && T::NT == 256 && CPR % 4 == 0 && (NPAN == 1 || NPAN == 2),
                  "row pass: 64 rows per round, one or two panels");
    const int64_t M = p.mcap;
    const int64_t g0 = hc0 >> 5;  // first 32-column group of the tile (a multiple of 2 NPAN)
#pragma unroll 1
    for (int rg = 0; rg < BM / 64; ++rg) {
      const int r = rg * 64 + (tid >> 2);
      const int64_t row = m0 + r;
      uint32_t wsc = 0;
#pragma unroll
      for (int P = 0; P < NPAN; ++P) {
        const int c = P * 4 + (tid & 3);
        const uint4 a = *reinterpret_cast<const uint4*>(hR + r * HP + c * 16);
        const uint4 b = *reinterpret_cast<const uint4*>(hR + r * HP + c * 16 + 8);
        const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t am = amax16(v);
        am = max(am, dpp_xor1(am));
        const Scale s = scale_from_amax(am);
        const int64_t hcol = hc0 + c * 16;
        *reinterpret_cast<uint4*>(p.q_r + (hcol >> 6) * 64 * M + row * 64 + (hcol & 63)) =
            make_uint4(cvt4(v[0], v[1], s), cvt4(v[2], v[3], s), cvt4(v[4], v[5], s), cvt4(v[6], v[7], s));
        wsc |= (s.byte | (dpp_xor2(s.byte) << 8)) << (16 * P);  // lane 0 of the quad: groups 2P, 2P+1
      }
      if ((tid & 3) == 0) {
        uint8_t* d = p.s_r + row * p.sr_rs + (g0 >> 2) * p.sr_kbs + (g0 & 3);
        if constexpr (NPAN == 2) *reinterpret_cast<uint32_t*>(d) = wsc;
        else *reinterpret_cast<uint16_t*>(d) = (uint16_t)wsc;
      }
    }
    // column-wise codes (hq_c [F, mcap], 64-token panels): four lanes per column and panel,
    // consecutive columns on consecutive lane quads (contiguous kilobytes)
    constexpr int CPC = BM / 16;
    static_assert((HCB * CPC) % T::NT == 0 && CPC % 4 == 0, "whole column-copy rounds");
#pragma unroll 2
    for (int it = 0; it < HCB * CPC / T::NT; ++it) {
      const int t = it * T::NT + tid;
      const int hc = (t >> 2) % HCB, c = ((t >> 2) / HCB) * 4 + (t & 3);
      const uint2 a = *reinterpret_cast<const uint2*>(qT + hc * QP + c * 16);
      const uint2 b = *reinterpret_cast<const uint2*>(qT + hc * QP + c * 16 + 8);
      const int64_t tok = m0 + c * 16;
      store16_nt(p.q_c + (tok >> 6) * 64 * F + (hc0 + hc) * 64 + (tok & 63),  // saved for backward
                 make_uint4(a.x, a.y, b.x, b.y));
    }
    // column scales: SG groups per column (whole 128-row planes: m0 is a multiple of 128)
    for (int t = tid; t < HCB * (SG / 4); t += T::NT) {
      const int hc = t / (SG / 4), w4 = t % (SG / 4);
      *reinterpret_cast<uint32_t*>(p.s_c + (hc0 + hc) * p.sc_rs + ((m0 >> 7) + w4) * p.sc_kbs) =
          *reinterpret_cast<const uint32_t*>(sT + hc * SG + 4 * w4);
    }
    return;
  }

  if (EPI == EPI_DSWIGLU) {
    // N = F: acc = dh. NP = 2 passes; in pass hh every wavefront takes its fragment rows
    // [hh FH, (hh+1) FH) (all SIMDs busy): dG = dh u s (1 + g (1 - s)), dU = dh g s with
    // s = sigmoid(g), from the saved g, u (4 KB records in accumulator order, so each lane's
    // slots arrive in its own registers), each rounded to BF16. Their column-wise groups are
    // quantized in registers (codes staged transposed in LDS) and the BF16 values staged
    // row-major in the packed order (gate group, then up group, per 32 columns); then the block
    // quantizes the staged rows' row-wise groups and copies the column codes out.
    constexpr int NP = T::DSW_NP;     // passes (the staging of a pass fits the pipeline LDS)
    static_assert(T::FM % NP == 0, "passes of whole fragment rows");
    constexpr int FH = T::FM / NP;    // fragment rows per wavefront per pass
    constexpr int RH = T::TM / NP;    // rows per wavefront per pass
    constexpr int SR = T::DSW_SR;     // staged rows per pass (WM * RH)
    constexpr int PCB = 2 * BN;       // packed columns of the block
    constexpr int DP = PCB + 8;       // row-major tile pitch (bf16)
    // Column codes are staged for PAIR consecutive passes (PAIR = 2 when a pass holds 32 rows
    // per wavefront), then copied out together: each wavefront's 2 x 32 rows of a pass pair are
    // one whole 64-token panel row per column, so every 16-byte store is a quarter of a 64-byte
    // run instead of half of a 32-byte one (half the store instructions and lines touched).
    constexpr int PAIR = T::DSW_PAIR;
    constexpr int QP = PAIR * SR + 8;  // transposed code tile pitch (bytes)
    constexpr int SG = PAIR * SR / 32; // column groups staged per pass pair
    const int64_t F = p.N;
    const int64_t ld13 = 2 * F;
    const int64_t pc0 = 2 * n0;
    uint16_t* dR = reinterpret_cast<uint16_t*>(smem);
    uint8_t* qT = smem + SR * DP * 2;
    uint8_t* sT = qT + PCB * QP;
    // row staging two columns at a time (as in the SwiGLU epilogue)
    const bool odd_lane = (lane & 1) != 0;
    const uint32_t pr_sel = odd_lane ? 0x03020706u : 0x05040100u;
    const int pr_off = odd_lane ? DP - 1 : 0;
    // staged row lr of pass hh is block row (lr / RH) * TM + hh * RH + lr % RH
    auto brow = [&](int hh, int lr) { return (lr / RH) * T::TM + hh * RH + lr % RH; };
    // g, u of the fragments in flight, a ring of GR fragment slots in processing order
    // (f = i FN + j): fragment f + GR - 1 is requested when fragment f is taken up
    constexpr int NF = T::FM * T::FN;
    static_assert(EPI != EPI_DSWIGLU || T::FN <= 2, "dSwiGLU runs on 64-column wavefront tiles");
    constexpr int GR = OCC == 2 ? 3 : 4;
    uint4 gs[GR][2], us[GR][2];
    auto load_gu = [&](int f) {
      const int i = f / T::FN, j = f % T::FN, slot = f % GR;
      const int64_t rec = ((wrow0 + i * 32) >> 5) * (F >> 5) + ((wcol0 + j * 32) >> 5);
      const uint4* src = reinterpret_cast<const uint4*>(p.h13 + rec * 2048) + lane;  // as written
      gs[slot][0] = load16_nt(src);  // read once: non-temporal
      gs[slot][1] = load16_nt(src + 64);
      us[slot][0] = load16_nt(src + 128);
      us[slot][1] = load16_nt(src + 192);
    };
#pragma unroll
    for (int f = 0; f < GR - 1 && f < NF; ++f) load_gu(f);
    if (DBG && p.dbg) {
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q)
            p.dbg[(wrow0 + i * 32 + 8 * (q >> 2) + 4 * g + (q & 3)) * F + wcol0 + j * 32 + r32] = acc[i][j][q];
    }
#pragma unroll
    for (int hh = 0; hh < NP; ++hh) {
#pragma unroll
      for (int ii = 0; ii < FH; ++ii) {
        const int i = hh * FH + ii;
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
          const int f = i * T::FN + j, b = f % GR;
          if (f + GR - 1 < NF) load_gu(f + GR - 1);
          const uint32_t gw[8] = {gs[b][0].x, gs[b][0].y, gs[b][0].z, gs[b][0].w,
                                  gs[b][1].x, gs[b][1].y, gs[b][1].z, gs[b][1].w};
          const uint32_t uw[8] = {us[b][0].x, us[b][0].y, us[b][0].z, us[b][0].w,
                                  us[b][1].x, us[b][1].y, us[b][1].z, us[b][1].w};
          uint32_t dgw[8], duw[8];
#pragma unroll
          for (int t = 0; t < 8; ++t)
            dswiglu2(bf16x2_bits(acc[i][j][2 * t], acc[i][j][2 * t + 1]), gw[t], uw[t], dgw[t], duw[t]);
          const int pcg = 2 * (tc0 + j * 32) + r32;  // packed column of dG (dU: + 32)
          const int rl = wm * RH + ii * 32 + 4 * g;  // staged row of slot 0
          // its row in the column-code staging: wavefront run wm, pass hh % PAIR within it
          const int rq = wm * PAIR * RH + (hh % PAIR) * RH + ii * 32 + 4 * g;
#pragma unroll
          for (int part = 0; part < 2; ++part) {
            const uint32_t* w = part ? duw : dgw;
            const int pcl = pcg + 32 * part;
            uint32_t am = amax16(w);
            am = max(am, (uint32_t)__shfl_xor((int)am, 32));
            const Scale s = scale_from_amax(am);
#pragma unroll
            for (int k = 0; k < 4; ++k)
              *reinterpret_cast<uint32_t*>(qT + pcl * QP + rq + 8 * k) = cvt4(w[2 * k], w[2 * k + 1], s);
            sT[pcl * SG + wm * PAIR * FH + (hh % PAIR) * FH + ii] = (uint8_t)s.byte;  // lanes l and l ^ 32: same byte
#pragma unroll
            for (int t = 0; t < 8; ++t)
              *reinterpret_cast<uint32_t*>(dR + (rl + 8 * (t >> 1) + 2 * (t & 1)) * DP + pcl + pr_off) =
                  __builtin_amdgcn_perm(dpp_xor1(w[t]), w[t], pr_sel);
          }
        }
      }
      __syncthreads();
      // four lanes per 64-column panel row, consecutive rows on consecutive lane quads; a quad
      // takes one row through all NPAN panels (inner loop), its first lane gathering the row's
      // scale bytes and storing each 128-k plane word (two panels) whole
      constexpr int CPR = PCB / 16;
      constexpr int NPAN = CPR / 4;  // 64-column panels of the packed columns (an even number)
      static_assert(SR % 64 == 0 && T::NT == 256 && CPR % 4 == 0 && NPAN % 2 == 0,
                    "row pass: 64 rows per round, whole 128-column scale words");
#pragma unroll 2
      for (int rg = 0; rg < SR / 64; ++rg) {
        const int r = rg * 64 + (tid >> 2);
        const int64_t row = m0 + brow(hh, r);
        uint32_t wsc = 0;
#pragma unroll
        for (int P = 0; P < NPAN; ++P) {
          const int c = P * 4 + (tid & 3);
          const uint4 a = *reinterpret_cast<const uint4*>(dR + r * DP + c * 16);
          const uint4 b = *reinterpret_cast<const uint4*>(dR + r * DP + c * 16 + 8);
          const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
          uint32_t am = amax16(v);
          am = max(am, dpp_xor1(am));
          const Scale s = scale_from_amax(am);
          const int64_t pcol = pc0 + c * 16;
          *reinterpret_cast<uint4*>(p.q_r + (pcol >> 6) * 64 * p.mcap + row * 64 + (pcol & 63)) =
              make_uint4(cvt4(v[0], v[1], s), cvt4(v[2], v[3], s), cvt4(v[4], v[5], s), cvt4(v[6], v[7], s));
          wsc |= (s.byte | (dpp_xor2(s.byte) << 8)) << (16 * (P & 1));  // groups 2P, 2P+1
          if ((P & 1) && (tid & 3) == 0) {
            const int64_t grp = (pc0 >> 5) + 2 * (P - 1);  // first group of the word (a multiple of 4)
            *reinterpret_cast<uint32_t*>(p.s_r + row * p.sr_rs + (grp >> 2) * p.sr_kbs) = wsc;
          }
          if (P & 1) wsc = 0;
        }
      }
      if (hh % PAIR == PAIR - 1) {
        // dhq_c [2F, mcap] in 64-token panels: a wavefront run of the staged passes is PAIR * RH
        // consecutive block rows, one panel row (64) or half of one (32); G lanes cover a
        // column's run, consecutive columns on consecutive lane groups. Staged row cr of the
        // pass group is block row (cr / (PAIR RH)) TM + h0 RH + cr % (PAIR RH), h0 its first pass.
        constexpr int RUN = PAIR * RH;
        constexpr int CPC = PAIR * SR / 16;
        constexpr int G = RUN >= 64 ? 4 : RUN / 16;
        static_assert((PCB * CPC) % T::NT == 0 && RH % 16 == 0 && CPC % G == 0, "whole column-copy rounds");
        const int h0 = hh - (PAIR - 1);
        auto crow = [&](int cr) { return (cr / RUN) * T::TM + h0 * RH + cr % RUN; };
#pragma unroll 2
        for (int it = 0; it < PCB * CPC / T::NT; ++it) {
          const int t = it * T::NT + tid;
          const int pc = (t / G) % PCB, c = ((t / G) / PCB) * G + (t % G);
          const uint2 a = *reinterpret_cast<const uint2*>(qT + pc * QP + c * 16);
          const uint2 b = *reinterpret_cast<const uint2*>(qT + pc * QP + c * 16 + 8);
          const int64_t tok = m0 + crow(c * 16);
          *reinterpret_cast<uint4*>(p.q_c + (tok >> 6) * 64 * ld13 + (pc0 + pc) * 64 + (tok & 63)) =
              make_uint4(a.x, a.y, b.x, b.y);
        }
        for (int t = tid; t < PCB * SG; t += T::NT) {
          const int pc = t / SG, gi = t % SG;
          const int64_t rg = (m0 + crow(gi * 32)) >> 5;
          p.s_c[(pc0 + pc) * p.sc_rs + (rg >> 2) * p.sc_kbs + (rg & 3)] = sT[pc * SG + gi];
        }
      }
      __syncthreads();  // the row staging is rewritten in the next pass (the code staging after PAIR)
    }
    return;
  }
}

// Tail sub-tiles (M-grouped): when the tile count T is not a multiple of the CU count, the last
// R = T mod #CU tiles (in raster order) would leave most CUs idle in a final round. Each of them
// is split into Q sub-tiles (Q = 4 when 4R <= #CU, else 2 when 2R <= #CU): BM/2 x BN/2, or
// BM x BN/2 (BN >= 256) / BM/2 x BN, computed by separate blocks with the same pipeline.
template <int BM, int BN>
struct TailCfg {
  static constexpr bool Q2 = BM == 256;                 // sub-tiles keep >= 128 rows
  static constexpr bool Q4 = BM == 256 && BN == 256;
  static constexpr int BM2 = BN >= 256 ? BM : BM / 2;   // Q = 2
  static constexpr int BN2 = BN >= 256 ? BN / 2 : BN;
  static constexpr int BM4 = BM / 2, BN4 = BN / 2;      // Q = 4
};

// LDS of one GEMM's blocks: its tile's main loop or epilogue staging, and those of its tail
// sub-tiles (M-grouped).
template <int BM, int BN, int WM, int WN, int SCHED, int EPI, int OCC>
constexpr int gemm_lds() {
  using T = Tile<BM, BN, WM, WN, OCC>;
  using TC = TailCfg<BM, BN>;
  return (SCHED == SCHED_MGROUP && TC::Q2)
             ? T::imax(T::lds(EPI), T::imax(Tile<TC::BM2, TC::BN2, WM, WN, OCC>::lds(EPI),
                                            Tile<TC::BM4, TC::BN4, WM, WN, OCC>::lds(EPI)))
             : T::lds(EPI);
}

// One block of a grouped GEMM: bid is the block's index within the GEMM's own grid (block bid
// runs on XCD bid % 8, which the tile orders assume: a GEMM sharing a launch starts at a
// multiple of 8). TAILS false compiles the M-grouped tail sub-tiles out, for a launch that never
// splits (p.ncu == 0): the merged backward launch measured 2 us faster without the dead paths.
// BIGE: the launch has 64 or more experts (p.E >= 64, chosen by the launcher): the offsets go
// through LDS as described below; otherwise one wavefront's lanes hold them.
template <int BM, int BN, int WM, int WN, int SCHED, int EPI, int OCC, bool TAILS = true, bool DBG = false,
          bool BIGE = false>
__device__ __forceinline__ void gemm_block(const GemmParams& p, uint32_t bid, uint8_t* smem) {
  using T = Tile<BM, BN, WM, WN, OCC>;
  using TC = TailCfg<BM, BN>;
  constexpr bool SPLIT = SCHED == SCHED_MGROUP && TC::Q2 && TAILS;

  const int tid = threadIdx.x;
  // Token offsets (validated on the device; a violation leaves every output untouched). E < 64:
  // one wavefront's lanes hold them (one round of loads; row lookups by ballot). E >= 64: the
  // block copies offs and counts into LDS in one round of coalesced loads, checks them in
  // parallel and looks rows up in LDS (the wavefront helpers would loop over E with a load per
  // step and binary-search global memory). The copy sits after the K-grouped scratch (2E ints).
  constexpr bool big_e = BIGE;
  int32_t* olds = reinterpret_cast<int32_t*>(smem) + 2 * p.E;  // offs [0, E], counts [E + 1, 2E]
  Offsets ofs = {};
  int64_t mend;
  if (!big_e) {
    ofs = read_offsets(p.offs, p.counts, p.E, p.pad, p.mcap);
    if (!ofs.ok) return;
    mend = ofs.mend;
  } else {
    for (int i = tid; i <= p.E; i += T::NT) olds[i] = p.offs[i];
    if (p.counts)
      for (int i = tid; i < p.E; i += T::NT) olds[p.E + 1 + i] = p.counts[i];
    __syncthreads();
    bool bad = false;
    for (int i = tid; i <= p.E; i += T::NT) {
      const int32_t o = olds[i];
      if (o % p.pad != 0 || o < 0 || (int64_t)o > p.mcap) bad = true;
      if (i == 0 && o != 0) bad = true;
      if (i > 0) {
        const int32_t pr = olds[i - 1];
        if (o < pr) bad = true;
        if (p.counts) {
          const int32_t c = olds[p.E + i];  // counts[i - 1]
          if (c < 0 || c > o - pr) bad = true;
        }
      }
    }
    if (__syncthreads_or(bad)) return;
    mend = olds[p.E];
  }
  // expert that owns row m (offs[e] <= m < offs[e + 1]; requires m < offs[E])
  auto expert_of = [&](int64_t m) -> int {
    if (!big_e) return ofs.expert(m);
    int lo = 0, hi = p.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)olds[mid] <= m) lo = mid; else hi = mid;
    }
    return lo;
  };

  int e;
  int64_t m0, n0, kbeg, kend;
  const int ntn = (int)(p.N / BN);
  if (SCHED == SCHED_MGROUP) {
    // Only the row tiles before offs[E] carry work: the grid is sized for m_capacity (plus the
    // tail sub-tiles) and the surplus blocks exit. Blocks are dispatched round-robin over the 8
    // XCDs (block b runs on XCD b % 8), so raster position t is taken from a contiguous per-XCD
    // range, and positions go in groups of GM row tiles x all column tiles: the ~32 blocks an
    // XCD runs at once share a few A row panels and B column panels in that XCD's L2.
    // 32-bit arithmetic throughout (tile counts stay below 2^31, which the launcher checks):
    // 64-bit divisions by run-time values cost about a microsecond per block.
    // GM measured per epilogue (settled clocks, GM 2, 3, 4, 8): 4 for FC1 + SwiGLU (164 against
    // 166-168 us), 2 for the others (FC2 dgrad + dSwiGLU 131 against 133, FC2 78.3 against 78.7)
    constexpr uint32_t GM = EPI == EPI_SWIGLU ? 4 : 2;
    const uint32_t mtu = (uint32_t)(mend / BM);
    const uint32_t ntiles = mtu * (uint32_t)ntn;
    uint32_t nfull = ntiles, rem = 0;
    uint32_t qs = 0;  // log2 of the sub-tiles per tail tile
    if (SPLIT && p.ncu > 0) {
      const uint32_t slots = (uint32_t)p.ncu * OCC;  // blocks resident at once
      rem = ntiles % slots;
      if (rem && TC::Q4 && 4 * rem <= slots) qs = 2;
      else if (rem && 2 * rem <= slots) qs = 1;
      if (qs) nfull = ntiles - rem;
      else rem = 0;
    }
    const uint32_t q = 1u << qs;
    // The sub-tile blocks take the lowest block ids (padded to whole rounds of the 8 XCDs):
    // they finish early and their CUs move on to whole tiles out of phase with the rest, which
    // spreads the epilogues' store bursts over time.
    const uint32_t nsub = (rem * q + 7) / 8 * 8;
    const uint32_t b = bid;
    const bool tail = b < nsub;  // a sub-tile of one of the last rem tiles (raster order)
    uint32_t t, part = 0;
    if (!tail) {
      const uint32_t f = b - nsub;  // whole tile f; f % 8 is still the block's XCD
      if (f >= nfull) return;
      const uint32_t q8 = nfull / 8, r8 = nfull % 8, x8 = f % 8, s8 = f / 8;
      t = x8 < r8 ? x8 * (q8 + 1) + s8 : r8 * (q8 + 1) + (x8 - r8) * q8 + s8;
    } else {
      if (b >= rem * q) return;
      t = nfull + (b >> qs);
      part = b & (q - 1);
    }
    const uint32_t gstride = GM * (uint32_t)ntn;
    const uint32_t grp = t / gstride;
    const uint32_t first = grp * GM;
    const uint32_t gsz = min(GM, mtu - first);
    const uint32_t within = t - grp * gstride;
    m0 = (int64_t)(first + within % gsz) * BM;
    n0 = (int64_t)(within / gsz) * BN;
    kbeg = 0;
    kend = p.K;
    if constexpr (SPLIT) {
      if constexpr (TC::Q4) {
        if (tail && q == 4) {
          m0 += (part >> 1) * TC::BM4;
          n0 += (part & 1) * TC::BN4;
          e = expert_of(m0);
          if (big_e) __syncthreads();  // the LDS copy of the offsets is reused by the main loop
          tile_run<TC::BM4, TC::BN4, WM, WN, SCHED, EPI, OCC, DBG>(p, smem, e, m0, n0, kbeg, kend);
          return;
        }
      }
      if (tail && q == 2) {
        if (TC::BM2 == BM) n0 += part * TC::BN2;
        else m0 += part * TC::BM2;
        e = expert_of(m0);
        if (big_e) __syncthreads();
        tile_run<TC::BM2, TC::BN2, WM, WN, SCHED, EPI, OCC, DBG>(p, smem, e, m0, n0, kbeg, kend);
        return;
      }
    }
    e = expert_of(m0);
    if (big_e) __syncthreads();
  } else {
    // Experts are taken longest-K first (their tiles start earliest, which shortens the tail;
    // with 64 or more experts in index order, see below).
    // Within an expert every tile streams the whole K range, so what matters is how many A
    // row panels and B column panels each XCD's L2 must hold: block l of the expert runs on
    // XCD l % 8, each XCD takes a contiguous run of positions, and positions walk the tile
    // grid in strips 3 tiles wide across the smaller dimension, so a run covers a compact
    // patch instead of whole rows of the grid.
    // 32-bit arithmetic (as in the M-grouped order)
    const uint32_t mtn = (uint32_t)(p.M / BM);
    const uint32_t per = mtn * (uint32_t)ntn;
    const uint32_t t = bid;
    if (t >= per * (uint32_t)p.E) return;  // blocks that round a shared launch's section up
    int ke;  // K span of expert e: its real rows rounded up to 128, within its segment
    if (!big_e) {
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
      e = order[t / per];
      ke = ksp[e];
      kbeg = p.offs[e];
    } else {
      // many experts: index order (the rank sort costs O(E^2 / threads) per block, and the
      // longest-first order matters less when each expert is a small share of the work)
      e = (int)(t / per);
      const int seg = olds[e + 1] - olds[e];
      const int real = p.counts ? olds[p.E + 1 + e] : seg;
      ke = min(seg, (real + 127) / 128 * 128);
      kbeg = olds[e];
    }
    const uint32_t l = t % per;
    const uint32_t q8 = per / 8, r8 = per % 8, x8 = l % 8, s8 = l / 8;
    const uint32_t pos = (x8 < r8 ? x8 * (q8 + 1) : r8 * (q8 + 1) + (x8 - r8) * q8) + s8;
    // strips of width W across the smaller grid dimension; the longer one runs inside a strip
    const bool mlong = mtn >= (uint32_t)ntn;
    const uint32_t nlong = mlong ? mtn : ntn, nshort = mlong ? ntn : mtn;
    // W measured in the merged backward launch (settled clocks, three A/B pairs): 3 gives
    // 354.4-355.6 us against 357.8-358.5 for 4; 2 and 4 are alike, 8 is 6 us slower
    constexpr uint32_t W = 3;
    const uint32_t nstrip = (nshort + W - 1) / W;
    const uint32_t strip = min(pos / (W * nlong), nstrip - 1);
    const uint32_t sw = min(W, nshort - strip * W);  // width of this strip
    const uint32_t within = pos - strip * W * nlong;
    const uint32_t il = within / sw, is = strip * W + within % sw;
    m0 = (int64_t)(mlong ? il : is) * BM;
    n0 = (int64_t)(mlong ? is : il) * BN;
    kend = kbeg + ke;
    __syncthreads();  // the LDS scratch is reused by the main loop
  }
  tile_run<BM, BN, WM, WN, SCHED, EPI, OCC, DBG>(p, smem, e, m0, n0, kbeg, kend);
}

template <int BM, int BN, int WM, int WN, int SCHED, int EPI, int OCC, bool DBG = false, bool BIGE = false>
__global__ __launch_bounds__(WM * WN * 64, OCC) void gemm_mx_kernel(GemmParams p) {
  constexpr int LDSZ = gemm_lds<BM, BN, WM, WN, SCHED, EPI, OCC>();
  static_assert(LDSZ <= Tile<BM, BN, WM, WN, OCC>::LDS_BYTES, "LDS of the kernel exceeds its share of the CU");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDSZ];
  gemm_block<BM, BN, WM, WN, SCHED, EPI, OCC, true, DBG, BIGE>(p, blockIdx.x, smem);
}

// The three GEMMs of the backward pass that follow FC2 dgrad -- FC1 dgrad, FC1 wgrad (with the
// W13 row unpack) and FC2 wgrad -- read only operands that exist once dH13 does and write
// disjoint outputs, so they share one launch: three sections of one 1-D grid, each block
// running one block of its section's GEMM. One kernel boundary replaces three, and the CUs
// that finish one section's last tiles start the next section's at once instead of waiting
// for the slowest tile. FC1 dgrad's tiles (all of one length, no tail sub-tiles: the rounds of
// the launch do not start with its section) come first; then the weight gradients, whose
// experts are taken longest-K first, FC1 wgrad (the larger tiles) before FC2 wgrad, so the
// launch ends on the shortest tiles. Measured against FC1 dgrad last with its tail sub-tiles:
// 362.5-363.4 against 368.9-371.4 us on the DSv3 rank shape. Section sizes are rounded up to
// multiples of 8 (surplus blocks exit) so that every section keeps the XCD mapping its tile
// order assumes.
struct GemmTrio {
  GemmParams d1, w1, w2;  // FC1 dgrad (ncu 0: no tail sub-tiles), FC1 wgrad, FC2 wgrad
  uint32_t n1, n2;        // blocks of the first two sections
};
template <int BN2, bool BIGE>
__global__ __launch_bounds__(256, 1) void gemm_bwd3_kernel(GemmTrio g) {
  constexpr int L1 = gemm_lds<256, 256, 2, 2, SCHED_KGROUP, EPI_UNPACK13, 1>();
  constexpr int L2 = gemm_lds<256, BN2, 2, 2, SCHED_KGROUP, EPI_STORE, 1>();
  constexpr int L3 = gemm_lds<256, 256, 2, 2, SCHED_MGROUP, EPI_STORE, 1>();
  constexpr int LDSZ = L1 > L2 ? (L1 > L3 ? L1 : L3) : (L2 > L3 ? L2 : L3);
  static_assert(LDSZ <= 160 * 1024, "LDS of the kernel exceeds the CU");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDSZ];
  uint32_t b = blockIdx.x;
  if (b < g.n1) {
    gemm_block<256, 256, 2, 2, SCHED_MGROUP, EPI_STORE, 1, false, false, BIGE>(g.d1, b, smem);  // d1.ncu == 0
    return;
  }
  b -= g.n1;
  if (b < g.n2) {
    gemm_block<256, 256, 2, 2, SCHED_KGROUP, EPI_UNPACK13, 1, true, false, BIGE>(g.w1, b, smem);
    return;
  }
  b -= g.n2;
  gemm_block<256, BN2, 2, 2, SCHED_KGROUP, EPI_STORE, 1, true, false, BIGE>(g.w2, b, smem);
}

// ------------------------------------------------------------------ host launchers

// Tile configurations (4 wavefronts): 256x256 (wavefront tile 128x128) when the rows allow
// 256-row tiles (M-grouped: pad_multiple 256) and N is a multiple of 256; 256x128 otherwise,
// 128x128 for pad_multiple 128. M-grouped row tiles divide pad_multiple. dSwiGLU stays on
// 256x128: with 256 accumulators per wavefront its epilogue has registers for one fragment of
// g/u lookahead only, and the exposed h13 read latency made it slower than 256x128 (measured).
template <int BM, int BN, int SCHED, int EPI, int OCC = 1>
static hipError_t launch_cfg(const GemmParams& p, hipStream_t st) {
  // 1-D grids: the kernel maps block ids to tiles (see the schedulers)
  int64_t nblk;
  if (SCHED == SCHED_MGROUP)
    nblk = (p.mcap / BM) * (p.N / BN) + (TailCfg<BM, BN>::Q2 ? 3 * p.ncu * OCC : 0);  // + tail sub-tiles
  else
    nblk = (p.M / BM) * (p.N / BN) * p.E;
  if (nblk == 0) return hipSuccess;
  if (nblk > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nblk);
  const bool big_e = p.E >= 64;
  if constexpr (EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU) {
    if (p.dbg) {
      if (big_e) hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, 2, 2, SCHED, EPI, OCC, true, true>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, 2, 2, SCHED, EPI, OCC, true, false>), grid, dim3(256), 0, st, p);
      return hipGetLastError();
    }
  }
  if (big_e) hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, 2, 2, SCHED, EPI, OCC, false, true>), grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, 2, 2, SCHED, EPI, OCC, false, false>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int SCHED, int EPI>
static hipError_t launch(const GemmParams& p, bool big_m, hipStream_t st) {
  if constexpr (EPI == EPI_DSWIGLU) {
    // two blocks per CU: one block's dSwiGLU epilogue (sigmoid, saved g/u reads, dual
    // quantization) runs beside the other block's matrix instructions; measured 13% faster
    // than one 256 x 128 block per CU on the DSv3 rank shape (FC2 dgrad: 141 against 165 us)
    if (big_m) return launch_cfg<256, 128, SCHED, EPI, 2>(p, st);
  } else {
    if (big_m && p.N % 256 == 0) return launch_cfg<256, 256, SCHED, EPI>(p, st);
    if (big_m) return launch_cfg<256, 128, SCHED, EPI>(p, st);
  }
  return launch_cfg<128, 128, SCHED, EPI>(p, st);
}

}  // namespace mxf

// M-grouped: C[m, n] = sum_k A[m, k] B_e[n, k] for m in expert e's segment.
// epi: 0 store (C, ldc, out_f32), 1 SwiGLU + dual quant, 2 dSwiGLU + dual quant.
namespace {
// compute units per device, looked up once (the tail sub-tiling balances the last round over them)
std::atomic<int> g_ncu[64];
hipError_t device_cus(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int n = g_ncu[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n <= 0) return hipErrorInvalidValue;
    g_ncu[dev].store(n, std::memory_order_relaxed);
  }
  *out = n;
  return hipSuccess;
}
}  // namespace

hipError_t mxf_launch_gemm_mgroup(int epi, const mxf::GemmParams& pin, hipStream_t st) {
  using namespace mxf;
  if (pin.mcap % 128 || pin.N % 128 || pin.K % 128 || pin.ldc % 8) return hipErrorInvalidValue;
  GemmParams p = pin;
  const hipError_t ce = device_cus(&p.ncu);
  if (ce != hipSuccess) return ce;
  const bool big = (p.pad % 256 == 0) && (p.mcap % 256 == 0);
  // the fused epilogues store whole scale words of 128-k planes
  if ((epi == EPI_SWIGLU || epi == EPI_DSWIGLU) && (p.sr_rs != 4 || p.sc_rs != 4)) return hipErrorInvalidValue;
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
  if (p.M % 128 || p.N % 128 || p.ldc % 8) return hipErrorInvalidValue;
  const bool big = (p.M % 256 == 0);
  switch (epi) {
    case EPI_STORE: return launch<SCHED_KGROUP, EPI_STORE>(p, big, st);
    case EPI_UNPACK13: return launch<SCHED_KGROUP, EPI_UNPACK13>(p, big, st);
    default: return hipErrorInvalidValue;
  }
}

bool mxf_gemm_bwd3_fits(const mxf::GemmParams& w1, const mxf::GemmParams& w2, const mxf::GemmParams& d1) {
  return w1.M % 256 == 0 && w1.N % 256 == 0 && w2.M % 256 == 0 && d1.pad % 256 == 0 && d1.mcap % 256 == 0 &&
         d1.N % 256 == 0;
}

hipError_t mxf_launch_gemm_bwd3(const mxf::GemmParams& w1, const mxf::GemmParams& w2, const mxf::GemmParams& d1,
                                hipStream_t st) {
  using namespace mxf;
  // the single launches' shape checks
  if (w1.M % 128 || w1.N % 128 || w1.ldc % 8 || w2.M % 128 || w2.N % 128 || w2.ldc % 8) return hipErrorInvalidValue;
  if (d1.mcap % 128 || d1.N % 128 || d1.K % 128 || d1.ldc % 8) return hipErrorInvalidValue;
  // the tiles the single launches would choose: 256 x 256 for FC1 wgrad and FC1 dgrad, 256 x 256
  // or 256 x 128 for FC2 wgrad
  if (!mxf_gemm_bwd3_fits(w1, w2, d1)) return hipErrorInvalidValue;
  GemmTrio g;
  g.d1 = d1;
  g.d1.ncu = 0;  // no tail sub-tiles
  g.w1 = w1;
  g.w2 = w2;
  const bool wide2 = w2.N % 256 == 0;
  const int64_t n1 = (d1.mcap / 256) * (d1.N / 256);
  const int64_t n2 = (w1.M / 256) * (w1.N / 256) * w1.E;
  const int64_t n3 = (w2.M / 256) * (w2.N / (wide2 ? 256 : 128)) * w2.E;
  const int64_t r1 = (n1 + 7) / 8 * 8, r2 = (n2 + 7) / 8 * 8;
  if (r1 + r2 + n3 > 0x7FFFFFFF) return hipErrorInvalidValue;
  g.n1 = (uint32_t)r1;
  g.n2 = (uint32_t)r2;
  const dim3 grid((unsigned)(r1 + r2 + n3));
  const bool big_e = d1.E >= 64;  // the three GEMMs share the experts
  if (wide2 && big_e) hipLaunchKernelGGL((gemm_bwd3_kernel<256, true>), grid, dim3(256), 0, st, g);
  else if (wide2) hipLaunchKernelGGL((gemm_bwd3_kernel<256, false>), grid, dim3(256), 0, st, g);
  else if (big_e) hipLaunchKernelGGL((gemm_bwd3_kernel<128, true>), grid, dim3(256), 0, st, g);
  else hipLaunchKernelGGL((gemm_bwd3_kernel<128, false>), grid, dim3(256), 0, st, g);
  return hipGetLastError();
}
