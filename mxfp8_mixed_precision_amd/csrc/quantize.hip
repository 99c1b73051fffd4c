// MXFP8 dual (row-wise + column-wise) quantization kernels for gfx950.
//
// Dual quantization is torchtitan PR #12 "Wire the fully-fused grouped-GEMM MXFP8 plan behind
// fusion_plan", section "What it adds": each operand is quantized in 32-element groups along
// the axis its GEMM contracts over, so one BF16 matrix yields row-wise codes [R, C] (+ scales
// [R, C/32]) and column-wise codes stored transposed [C, R] (+ scales [C, R/32]).
//
// Work decomposition (HBM-bound: 2 bytes in, ~2.06 bytes out per element for dual):
//   * block = 4 wavefronts = 128 rows x 128 columns; each wavefront owns 32 rows x 128 cols,
//     so every column-wise 32-group lies inside one wavefront and no LDS or block barrier is
//     needed;
//   * lane l: row octet s = l / 16 (rows 8s .. 8s+7 of the wavefront), column octet
//     c = l % 16 (cols 8c .. 8c+7). Each lane loads 8 rows x 16 bytes: a wavefront load
//     instruction covers 4 rows x 256 contiguous bytes;
//   * a row-wise group (32 cols) is 4 adjacent lanes: amax by two DPP quad swaps; lanes 2t and
//     2t+1 swap halves of rows j and j+1 so that each writes 16 codes of one row (16 bytes: a
//     wavefront store covers 8 rows x 128 bytes, 512 contiguous bytes of a 64-k panel);
//   * a column-wise group (32 rows) is the 4 lanes l, l^16, l^32, l^48: amax by two
//     cross-lane swaps; each lane writes 8 contiguous codes per column (the 4 lanes, and
//     the 4 wavefronts of the block, complete 128 contiguous bytes of every column).
#include "kernels.h"
#include "mx_device.h"

namespace mxf {

// QK_SWIGLU / QK_DSWIGLU are the standalone SwiGLU / dSwiGLU + dual-quantization kernels of the
// unfused plan: they read the BF16 FC1 output (and dh) that the plain GEMMs wrote, apply the
// same rounding points as the fused epilogues, and quantize like QK_MASKED.
// QK_GATHER is the fused dispatch: row r of the padded token layout is read from the token
// row_assign[r] / topk of the unpermuted token matrix (no BF16 copy of the permuted matrix),
// then quantized like QK_MASKED.
enum QuantKind { QK_PLAIN = 0, QK_MASKED = 1, QK_PACK13 = 2, QK_SWIGLU = 3, QK_DSWIGLU = 4, QK_GATHER = 5 };

struct QuantParams {
  const uint16_t* src;   // BF16 bits; QK_PACK13: w1 [E, F, D]
  const uint16_t* src2;  // QK_PACK13: w3 [E, F, D]; QK_DSWIGLU: g | u [rows, cols] (packed order)
  int64_t rows, cols;    // logical matrix per batch entry (QK_PACK13: rows = 2F, cols = D)
  int64_t src_bs;        // elements between batch entries of src / src2
  uint8_t* q_r;
  uint8_t* s_r;          // scale byte (r, g) at r * sr_rs + (g / 4) * sr_kbs + g % 4
  uint8_t* q_c;
  uint8_t* s_c;          // scale byte (column c, row group g) at c * sc_rs + (g / 4) * sc_kbs + g % 4
  int64_t sr_rs, sr_kbs, sc_rs, sc_kbs;
  int64_t qr_bs, sr_bs, qc_bs, sc_bs;  // bytes between batch entries of each output
  int64_t ldc;                          // row pitch (bytes) of q_c; multiple of 32
  const int32_t* offs;                  // QK_MASKED: token offsets [E+1]
  const int32_t* counts;                // QK_MASKED: real rows per expert [E] or null
  int E, pad;
  int32_t* status;                      // QK_MASKED, QK_GATHER: device status word (block 0 writes it)
  const int32_t* row_assign;            // QK_GATHER: assignment of each padded row (-1: pad)
  int64_t n_assign;                     // QK_GATHER: tokens * topk
  int topk;                             // QK_GATHER
  int col_fast;                         // grid x walks column tiles (set by the launcher)
  int macro8;                           // 1-D grid of 8x8-tile macro-tiles per XCD (launcher)
  int nt_c;                             // column codes saved for the backward pass: non-temporal stores
  int blk;                              // codes in 64-k panels (the MLP's GEMM operands): q_r byte
                                        // (r, c) at (c/64)*64*rows + 64r + c%64, q_c byte (c, r) at
                                        // (r/64)*64*cols + 64c + r%64; else row-major
};


// Column codes of a block, transposed [128 columns][QTP bytes], and its scale words (4 groups of
// a row / of a column), staged in LDS so that every global store is a 16-byte (codes) or 4-byte
// (scales) piece of a contiguous run.
constexpr int QTP = 128 + 8;
struct QuantLds {
  uint8_t qT[128 * QTP];
  uint32_t srow[128];
  uint32_t scol[128];
};

// One 128 x 128 tile of one batch entry: (bx, by, bz) is the tile's position in the launch grid
// of its kind (see grid_of), so the same body serves a kernel of one kind and the combined
// forward kernel.
template <int KIND, bool ROW, bool COL, int FMT = FMT_E4M3>
__device__ __forceinline__ void quant_tile(const QuantParams& p, int64_t bx, int64_t by, int64_t bz, QuantLds& L) {
  uint8_t* qT = L.qT;
  uint32_t* srow = L.srow;
  uint32_t* scol = L.scol;
  uint8_t* srow_b = reinterpret_cast<uint8_t*>(srow);
  uint8_t* scol_b = reinterpret_cast<uint8_t*>(scol);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int s = lane >> 4;
  const int c = lane & 15;
  const int64_t e = bz;
  // with col_fast, consecutive blocks take the column tiles of one 128-row band, so the blocks
  // resident at a time read and write a few contiguous bands
  int64_t row0 = (p.col_fast ? by : bx) * 128;
  int64_t col0 = (p.col_fast ? bx : by) * 128;
  if (p.macro8) {
    // Row-major scales of a single matrix: a row's 32-byte scale sector spans 8 column tiles
    // and a column's spans 8 row bands. Block L runs on XCD L % 8; each XCD takes whole
    // macro-tiles of 8 bands x 8 column tiles, so every sector is filled inside one XCD's L2
    // (split over XCDs, each L2 writes its few bytes back as a partial sector).
    const uint32_t L = (uint32_t)bx, x = L & 7, sq = L >> 3;  // 32-bit: tiles < 2^31
    const uint32_t m = x + 8 * (sq >> 6);                    // macro-tile of the XCD's sq-th block
    const uint32_t w = sq & 63;                              // tile within it, band-major
    const uint32_t mcols = (uint32_t)((p.cols + 1023) >> 10);  // macro-tiles across
    const uint32_t mr = m / mcols;
    row0 = (int64_t)(mr * 8 + (w >> 3)) * 128;
    col0 = (int64_t)((m - mr * mcols) * 8 + (w & 7)) * 128;
  }
  const int64_t col = col0 + c * 8;
  const int64_t rw0 = row0 + w * 32;  // first row of this wavefront
  const int64_t r0 = rw0 + 8 * s;     // first row of this lane

  int64_t valid_end = p.rows;  // rows at or past this read as zero
  const uint16_t* src = p.src + e * p.src_bs;
  int64_t src_row0 = rw0;      // source row of the wavefront's first row
  if (KIND == QK_MASKED || KIND == QK_SWIGLU || KIND == QK_DSWIGLU || KIND == QK_GATHER) {
    // every wavefront reads the offsets (same answers everywhere); mend and the block's rows
    // are multiples of 128, so a block is either wholly before offs[E] or wholly past it
    const Offsets ofs = read_offsets(p.offs, p.counts, p.E, p.pad, p.rows);
    if ((KIND == QK_MASKED || KIND == QK_GATHER) && bx == 0 && by == 0 && threadIdx.x == 0)
      *p.status = ofs.ok ? 0 : 1;
    if (!ofs.ok) return;
    if (row0 >= ofs.mend) return;  // tail rows: never read or written
    const int ex = ofs.expert(rw0);
    valid_end = ofs.real_end(ex);
  } else if (KIND == QK_PACK13) {
    // packed row n of [2F, D]: groups of 32 rows alternate between w1 and w3
    const int64_t grp = rw0 >> 5;
    src = ((grp & 1) ? p.src2 : p.src) + e * p.src_bs;
    src_row0 = (grp >> 1) * 32;
  }
  const bool colok = col < p.cols;
  const int64_t rend = valid_end < p.rows ? valid_end : p.rows;

  uint32_t x[8][4];
  int tok[8];  // QK_GATHER: token row of each of the lane's rows (-1: zero row)
  if (KIND == QK_GATHER) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t r = r0 + j;
      const int a = (colok && r < rend) ? p.row_assign[r] : -1;
      tok[j] = (a >= 0 && a < p.n_assign) ? a / p.topk : -1;
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t r = r0 + j;
    if (KIND == QK_GATHER) {
      if (tok[j] >= 0) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t)tok[j] * p.cols + col);
        x[j][0] = v.x; x[j][1] = v.y; x[j][2] = v.z; x[j][3] = v.w;
      } else {
        x[j][0] = x[j][1] = x[j][2] = x[j][3] = 0u;
      }
    } else if (colok && r < rend && KIND == QK_SWIGLU) {
      // h column col of row r: gate at packed column 64 (col / 32) + col % 32, up 32 further
      const uint16_t* row = src + r * (2 * p.cols) + (col >> 5) * 64 + (col & 31);
      const uint4 gv = *reinterpret_cast<const uint4*>(row);
      const uint4 uv = *reinterpret_cast<const uint4*>(row + 32);
      const uint32_t g4[4] = {gv.x, gv.y, gv.z, gv.w}, u4[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        x[j][k] = swiglu_h2(g4[k], u4[k]);
    } else if (colok && r < rend && KIND == QK_DSWIGLU) {
      // packed column col: dG (col % 64 < 32) or dU of dh column 32 (col / 64) + col % 32
      const int64_t F = p.cols >> 1;
      const int64_t j32 = col >> 6, cc = col & 31;
      const uint4 dv = *reinterpret_cast<const uint4*>(src + r * F + j32 * 32 + cc);
      const uint16_t* gu = p.src2 + r * p.cols + j32 * 64 + cc;
      const uint4 gv = *reinterpret_cast<const uint4*>(gu);
      const uint4 uv = *reinterpret_cast<const uint4*>(gu + 32);
      const uint32_t d4[4] = {dv.x, dv.y, dv.z, dv.w}, g4[4] = {gv.x, gv.y, gv.z, gv.w}, u4[4] = {uv.x, uv.y, uv.z, uv.w};
      const bool up = (col & 32) != 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t dg2, du2;
        dswiglu2(d4[k], g4[k], u4[k], dg2, du2);
        x[j][k] = up ? du2 : dg2;
      }
    } else if (colok && r < rend) {
      // the BF16 input is read exactly once: non-temporal, so it does not evict the L2 lines of a
      // GEMM running beside this kernel
      const uint4 v = load16_nt(src + (src_row0 + 8 * s + j) * p.cols + col);
      x[j][0] = v.x; x[j][1] = v.y; x[j][2] = v.z; x[j][3] = v.w;
    } else {
      x[j][0] = x[j][1] = x[j][2] = x[j][3] = 0u;
    }
  }

  if (ROW) {
    uint8_t* q_r = p.q_r + e * p.qr_bs;
    // rows j and j+1 in pairs: lanes 2t and 2t+1 (column octets c, c+1 of one 16-column run)
    // swap halves, so the even lane stores row j's 16 codes of the run and the odd lane row
    // j+1's: one 16-byte store per lane and row pair instead of two 8-byte stores
    const bool odd = (c & 1) != 0;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      uint32_t w[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t m = pk_max_u16(pk_max_u16(mag2(x[j + h][0]), mag2(x[j + h][1])),
                                pk_max_u16(mag2(x[j + h][2]), mag2(x[j + h][3])));
        m = max(m & 0xFFFFu, m >> 16);
        m = max(m, dpp_xor1(m));
        m = max(m, dpp_xor2(m));
        const Scale sc = scale_from_amax<FMT>(m);
        w[h][0] = cvt4<FMT>(x[j + h][0], x[j + h][1], sc);
        w[h][1] = cvt4<FMT>(x[j + h][2], x[j + h][3], sc);
        if ((c & 3) == 0) srow_b[(r0 + j + h - row0) * 4 + (c >> 2)] = (uint8_t)sc.byte;
      }
      // even lane keeps row j and takes the odd neighbour's row j; odd lane keeps row j+1
      const uint32_t s0 = odd ? w[0][0] : w[1][0], s1 = odd ? w[0][1] : w[1][1];
      const uint32_t r0w = dpp_xor1(s0), r1w = dpp_xor1(s1);
      const int64_t r = r0 + j + (odd ? 1 : 0);
      const int64_t cc = col - (odd ? 8 : 0);  // first column of the 16-column run
      const uint4 v = odd ? make_uint4(r0w, r1w, w[1][0], w[1][1]) : make_uint4(w[0][0], w[0][1], r0w, r1w);
      if (cc < p.cols && r < p.rows) {
        const int64_t o = p.blk ? (cc >> 6) * 64 * p.rows + r * 64 + (cc & 63) : r * p.cols + cc;
        *reinterpret_cast<uint4*>(q_r + o) = v;
      }
    }
  }

  if (COL) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t m = mag2(x[0][k]);
#pragma unroll
      for (int j = 1; j < 8; ++j) m = pk_max_u16(m, mag2(x[j][k]));
      m = pk_max_u16(m, (uint32_t)__shfl_xor((int)m, 16));
      m = pk_max_u16(m, (uint32_t)__shfl_xor((int)m, 32));
      const Scale slo = scale_from_amax<FMT>(m & 0xFFFFu);
      const Scale shi = scale_from_amax<FMT>(m >> 16);
      const uint32_t a0 = cvt4<FMT>(pack_lo(x[0][k], x[1][k]), pack_lo(x[2][k], x[3][k]), slo);
      const uint32_t a1 = cvt4<FMT>(pack_lo(x[4][k], x[5][k]), pack_lo(x[6][k], x[7][k]), slo);
      const uint32_t b0 = cvt4<FMT>(pack_hi(x[0][k], x[1][k]), pack_hi(x[2][k], x[3][k]), shi);
      const uint32_t b1 = cvt4<FMT>(pack_hi(x[4][k], x[5][k]), pack_hi(x[6][k], x[7][k]), shi);
      const int cl = c * 8 + 2 * k;  // block-local column
      const int rl = w * 32 + 8 * s;  // block-local row
      *reinterpret_cast<uint2*>(qT + cl * QTP + rl) = make_uint2(a0, a1);
      *reinterpret_cast<uint2*>(qT + (cl + 1) * QTP + rl) = make_uint2(b0, b1);
      if (s == 0) {
        scol_b[cl * 4 + w] = (uint8_t)slo.byte;
        scol_b[(cl + 1) * 4 + w] = (uint8_t)shi.byte;
      }
    }
  }
  __syncthreads();

  if (ROW && tid < 128) {
    // the block's 4 row groups of row r are one word in the 128-k plane layout
    const int64_t r = row0 + tid;
    const int64_t g0 = col0 >> 5;
    const int64_t ng = (p.cols - col0) >> 5;  // valid groups in the block (>= 1)
    uint8_t* dst = p.s_r + e * p.sr_bs + r * p.sr_rs + (g0 >> 2) * p.sr_kbs;
    if (r < p.rows) {
      // one word store only where the four bytes are a naturally aligned word (the scale
      // array's base may sit at any byte)
      if (ng >= 4 && ((uintptr_t)dst & 3) == 0 && (p.sr_rs & 3) == 0 && (p.sr_kbs & 3) == 0) {
        *reinterpret_cast<uint32_t*>(dst) = srow[tid];
      } else {
        for (int g = 0; g < 4 && g < ng; ++g) dst[g] = srow_b[tid * 4 + g];
      }
    }
  }
  if (COL) {
    uint8_t* q_c = p.q_c + e * p.qc_bs;
    // 16 bytes (one column, 16 rows) per task. Row-major: a column's codes for the block's rows
    // are contiguous, eight tasks per column. 64-k panels: four tasks per column and panel,
    // consecutive columns on consecutive lane quads (contiguous kilobytes).
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int t = it * 256 + tid;
      const int cl = p.blk ? (t >> 2) & 127 : t >> 3;
      const int ch = p.blk ? (t >> 9) * 4 + (t & 3) : t & 7;
      if (col0 + cl < p.cols && row0 + ch * 16 < p.rows) {
        const uint2 a = *reinterpret_cast<const uint2*>(qT + cl * QTP + ch * 16);
        const uint2 b = *reinterpret_cast<const uint2*>(qT + cl * QTP + ch * 16 + 8);
        const int64_t r = row0 + ch * 16;
        const int64_t o = p.blk ? (r >> 6) * 64 * p.cols + (col0 + cl) * 64 + (r & 63) : (col0 + cl) * p.ldc + r;
        if (p.nt_c) store16_nt(q_c + o, make_uint4(a.x, a.y, b.x, b.y));
        else *reinterpret_cast<uint4*>(q_c + o) = make_uint4(a.x, a.y, b.x, b.y);
      }
    }
    if (tid < 128 && col0 + tid < p.cols) {
      const int64_t g0 = row0 >> 5;
      const int64_t ng = (p.rows - row0) >> 5;
      uint8_t* dst = p.s_c + e * p.sc_bs + (col0 + tid) * p.sc_rs + (g0 >> 2) * p.sc_kbs;
      if (ng >= 4 && ((uintptr_t)dst & 3) == 0 && (p.sc_rs & 3) == 0 && (p.sc_kbs & 3) == 0) {
        *reinterpret_cast<uint32_t*>(dst) = scol[tid];
      } else {
        for (int g = 0; g < 4 && g < ng; ++g) dst[g] = scol_b[tid * 4 + g];
      }
    }
  }
}

template <int KIND, bool ROW, bool COL, int FMT = FMT_E4M3>
__global__ __launch_bounds__(256) void quant_dual_kernel(QuantParams p) {
  __shared__ __attribute__((aligned(16))) QuantLds L;
  quant_tile<KIND, ROW, COL, FMT>(p, blockIdx.x, blockIdx.y, blockIdx.z, L);
}

// Launch grid of one quantization (tiles of 128 x 128, batch entries along z); sets the
// parameters' block-order fields. Shared by the single-kind launches and the combined forward
// kernel.
struct QGrid {
  int64_t x, y, z;
};
static QGrid grid_of(int kind, QuantParams& p, int64_t batch) {
  const int64_t rt = std::max<int64_t>((p.rows + 127) / 128, 1), ct = std::max<int64_t>((p.cols + 127) / 128, 1);
  // Block order: column tiles fastest unless the matrix is much wider than tall or a batch of
  // small matrices (measured on MI355X: 10-20% faster for tall operands such as [26112, 2048],
  // slightly slower for [2048, 26112] and for the expert weight batches); grid y and z are
  // limited to 65535.
  p.col_fast = (batch == 1 && rt * 8 >= ct && rt <= 65535) || ct > 65535;
  // a single matrix with row-major scales on both sides: macro-tile order (see the kernel)
  p.macro8 = kind == QK_PLAIN && batch == 1 && !p.blk && rt % 8 == 0 && ct % 8 == 0 &&
             ((rt / 8) * (ct / 8)) % 8 == 0 && rt * ct <= 0x7FFFFFFF;
  if (p.macro8) return {rt * ct, 1, 1};
  return {p.col_fast ? ct : rt, p.col_fast ? rt : ct, batch > 0 ? batch : 1};
}

// The forward's operand quantizations in one launch: W13 (pack + dual, a batch of experts), W2
// (dual, a batch of experts) and, unless X's codes were written by the fused dispatch, X (dual
// under the token layout; its first block writes the status word). One grid of n13 + n2 + nx
// blocks, each section walking its own tile grid; one launch instead of three fills the
// compute units through the last round of tiles.
struct QuantFwd {
  QuantParams w13, w2, x;
  QGrid g13, g2, gx;
  int64_t n13, n2, nx;
};
__global__ __launch_bounds__(256) void quant_fwd_kernel(QuantFwd f) {
  __shared__ __attribute__((aligned(16))) QuantLds L;
  uint32_t b = blockIdx.x;
  // 32-bit arithmetic (block counts stay below 2^31; 64-bit divisions by run-time values are
  // long scalar sequences)
  auto split = [](uint32_t i, const QGrid& g, int64_t& bx, int64_t& by, int64_t& bz) {
    const uint32_t gx = (uint32_t)g.x, gy = (uint32_t)g.y;
    const uint32_t q = i / gx;
    bx = i - q * gx;
    by = q % gy;
    bz = q / gy;
  };
  int64_t bx, by, bz;
  if (b < f.n13) {
    split(b, f.g13, bx, by, bz);
    quant_tile<QK_PACK13, true, true>(f.w13, bx, by, bz, L);
    return;
  }
  b -= f.n13;
  if (b < f.n2) {
    split(b, f.g2, bx, by, bz);
    quant_tile<QK_PLAIN, true, true>(f.w2, bx, by, bz, L);
    return;
  }
  b -= f.n2;
  if (b < f.nx) {
    split(b, f.gx, bx, by, bz);
    quant_tile<QK_MASKED, true, true>(f.x, bx, by, bz, L);
  }
}

// ------------------------------------------------------------------ dequantization

// E4M3 code -> its exact fp32 value, from the bit fields (OCP FP8): exponent field 0 is m * 2^-9,
// S.1111.111 is NaN, otherwise (1 + m/8) * 2^(e-7), i.e. fp32 exponent field e + 120.
__device__ __forceinline__ float e4m3_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  const uint32_t normal = sign | ((e + 120u) << 23) | (m << 20);
  const uint32_t sub = sign | __float_as_uint((float)m * 0.001953125f);  // m * 2^-9, exact
  const uint32_t nan = sign | 0x7FC00000u;
  return __uint_as_float((c & 0x7Fu) == 0x7Fu ? nan : (e == 0 ? sub : normal));
}

// E5M2 code -> its exact fp32 value, from the bit fields (OCP FP8): exponent field 0 is m * 2^-16,
// field 31 is infinity (m = 0) or NaN, otherwise (1 + m/4) * 2^(e-15), i.e. fp32 exponent field
// e + 112.
__device__ __forceinline__ float e5m2_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t e = (c >> 2) & 0x1Fu, m = c & 3u;
  const uint32_t normal = sign | ((e + 112u) << 23) | (m << 21);
  const uint32_t sub = sign | __float_as_uint((float)m * 1.52587890625e-05f);  // m * 2^-16, exact
  const uint32_t special = sign | (m == 0 ? 0x7F800000u : 0x7FC00000u);
  return __uint_as_float(e == 31u ? special : (e == 0 ? sub : normal));
}

template <int FMT>
__device__ __forceinline__ float code_f32(uint32_t c) {
  if constexpr (FMT == FMT_E5M2) return e5m2_f32(c);
  else return e4m3_f32(c);
}

// Two codes (bytes 0-1, or 2-3 with HI) of a word -> their exact fp32 values, by the gfx950
// hardware conversion of the OCP formats (the same values as code_f32; NaN codes give a NaN).
template <int FMT, bool HI>
__device__ __forceinline__ f32x2 code_pk_f32(uint32_t w) {
  if constexpr (FMT == FMT_E5M2) return __builtin_amdgcn_cvt_pk_f32_bf8((int)w, HI);
  else return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

// E8M0 byte -> 2^(b - 127) as fp32: 0x00 is the subnormal 2^-127 (bits 0x00400000), 0xFF is NaN.
__device__ __forceinline__ float e8m0_f32(uint32_t b) {
  return __uint_as_float(b == 0xFFu ? 0x7FC00000u : (b == 0u ? 0x00400000u : b << 23));
}

// out[r, c] = code(q[r, c]) * E8M0(s[r, c / 32]) rounded once to BF16 or FP32, the code being
// E4M3 or E5M2. The fp32 product of a code (at most 4 significant bits) and a power of two is
// exact whenever it is in range (down to 2^-136 = 2^-9 * 2^-127 for E4M3 and 2^-143 for E5M2,
// fp32 subnormals), so the only rounding is the output conversion. Rows of 16-multiple width
// take 16 codes per thread; other widths one code per thread.
template <bool BF16, int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* q, const uint8_t* s, int64_t rows,
                                                      int64_t cols, void* out) {
  const int64_t G = (cols + 31) >> 5;  // scale bytes per row (the last group may be short)
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if ((cols & 15) == 0) {
    const int64_t cpr = cols >> 4;
    const int64_t total = rows * cpr;
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    // (row, 16-code chunk) of t, stepped by the grid stride without a division per step
    int64_t r = t / cpr, c16 = t - r * cpr;
    const int64_t sr = stride / cpr, sc16 = stride - sr * cpr;
    for (; t < total; t += stride) {
      const uint4 v = load16_nt(q + r * cols + c16 * 16);  // the codes are read once
      const float sc = e8m0_f32(s[r * G + (c16 >> 1)]);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      float f[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // the hardware OCP decode of bytes 0-1 and 2-3 of the word (exact in fp32)
        const f32x2 lo = code_pk_f32<FMT, false>(w[k]), hi = code_pk_f32<FMT, true>(w[k]);
        f[4 * k] = lo.x * sc;
        f[4 * k + 1] = lo.y * sc;
        f[4 * k + 2] = hi.x * sc;
        f[4 * k + 3] = hi.y * sc;
      }
      if (BF16) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = bf16x2_bits(f[2 * i], f[2 * i + 1]);
        uint4* o = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + r * cols + c16 * 16);
        o[0] = make_uint4(h[0], h[1], h[2], h[3]);
        o[1] = make_uint4(h[4], h[5], h[6], h[7]);
      } else {
        float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + r * cols + c16 * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = make_float4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
      }
      r += sr;
      c16 += sc16;
      if (c16 >= cpr) {
        c16 -= cpr;
        ++r;
      }
    }
  } else {
    const int64_t total = rows * cols;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
      const int64_t r = t / cols, c = t - r * cols;
      const float f = code_f32<FMT>(q[t]) * e8m0_f32(s[r * G + (c >> 5)]);
      if (BF16) reinterpret_cast<uint16_t*>(out)[t] = (uint16_t)bf16_bits(f);
      else reinterpret_cast<float*>(out)[t] = f;
    }
  }
}

// 32-row-block interleave of w1/w3 into [E, 2F, D] and back (BF16, 16-byte copies).
template <bool PACK>
__global__ __launch_bounds__(256) void pack13_kernel(const uint16_t* a, const uint16_t* b,
                                                     uint16_t* w13, uint16_t* w1, uint16_t* w3,
                                                     int64_t E, int64_t F, int64_t D) {
  const int64_t chunks_per_row = D / 8;
  const int64_t total = E * 2 * F * chunks_per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t ch = i % chunks_per_row;
    const int64_t n = (i / chunks_per_row) % (2 * F);
    const int64_t e = i / (chunks_per_row * 2 * F);
    const int64_t f = (n >> 6) * 32 + (n & 31);
    const bool up = (n & 32) != 0;
    const int64_t src_off = (e * F + f) * D + ch * 8;
    const int64_t dst_off = (e * 2 * F + n) * D + ch * 8;
    if (PACK) {
      const uint16_t* s = up ? b : a;
      *reinterpret_cast<uint4*>(w13 + dst_off) = *reinterpret_cast<const uint4*>(s + src_off);
    } else {
      uint16_t* d = up ? w3 : w1;
      *reinterpret_cast<uint4*>(d + src_off) = *reinterpret_cast<const uint4*>(a + dst_off);
    }
  }
}

// ------------------------------------------------------------------ host launchers

static hipError_t launch_quant(int kind, uint32_t mode, const QuantParams& pin, int64_t batch,
                               hipStream_t st, bool e5m2 = false) {
  // the token-layout kind always runs (its first block writes the status word)
  if ((pin.rows == 0 || pin.cols == 0 || batch == 0) && kind != QK_MASKED && kind != QK_GATHER) return hipSuccess;
  QuantParams p = pin;
  const QGrid g = grid_of(kind, p, batch);
  const dim3 grid((unsigned)g.x, (unsigned)g.y, (unsigned)g.z);
  const dim3 block(256);
#define MXF_QLAUNCH(K, R, C) hipLaunchKernelGGL((quant_dual_kernel<K, R, C>), grid, block, 0, st, p)
  if (kind == QK_PLAIN && e5m2) {
    if (mode == 3) hipLaunchKernelGGL((quant_dual_kernel<QK_PLAIN, true, true, FMT_E5M2>), grid, block, 0, st, p);
    else if (mode == 1) hipLaunchKernelGGL((quant_dual_kernel<QK_PLAIN, true, false, FMT_E5M2>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((quant_dual_kernel<QK_PLAIN, false, true, FMT_E5M2>), grid, block, 0, st, p);
  } else if (kind == QK_PLAIN) {
    if (mode == 3) MXF_QLAUNCH(QK_PLAIN, true, true);
    else if (mode == 1) MXF_QLAUNCH(QK_PLAIN, true, false);
    else MXF_QLAUNCH(QK_PLAIN, false, true);
  } else if (kind == QK_MASKED) {
    MXF_QLAUNCH(QK_MASKED, true, true);
  } else if (kind == QK_SWIGLU) {
    MXF_QLAUNCH(QK_SWIGLU, true, true);
  } else if (kind == QK_DSWIGLU) {
    MXF_QLAUNCH(QK_DSWIGLU, true, true);
  } else if (kind == QK_GATHER) {
    MXF_QLAUNCH(QK_GATHER, true, true);
  } else {
    MXF_QLAUNCH(QK_PACK13, true, true);
  }
#undef MXF_QLAUNCH
  return hipGetLastError();
}

}  // namespace mxf

// Internal entry points used by the C ABI layer (abi.hip).
hipError_t mxf_launch_quantize(const void* x, int64_t rows, int64_t cols, uint32_t mode, bool e5m2, void* q_row,
                               void* s_row, void* q_col, void* s_col, hipStream_t st) {
  mxf::QuantParams p = {};
  p.src = (const uint16_t*)x;
  p.rows = rows;
  p.cols = cols;
  p.q_r = (uint8_t*)q_row;
  p.s_r = (uint8_t*)s_row;
  p.q_c = (uint8_t*)q_col;
  p.s_c = (uint8_t*)s_col;
  p.ldc = rows;
  p.sr_rs = cols / 32; p.sr_kbs = 4;  // row-major scales
  p.sc_rs = rows / 32; p.sc_kbs = 4;
  return mxf::launch_quant(mxf::QK_PLAIN, mode, p, 1, st, e5m2);
}

// Dual quantization of the activation-like operand x [mcap, D] under the token layout
// (pad rows read as zero, rows >= offs[E] skipped); writes the status word. Scales in 128-k
// planes (row-wise [D/128][mcap][4], column-wise [mcap/128][D][4]).
static mxf::QuantParams token_params(const void* x, int64_t mcap, int64_t D, const int32_t* offs,
                                     const int32_t* counts, int E, int pad, void* q_r, void* s_r, void* q_c,
                                     void* s_c, int32_t* status, bool saved_c) {
  mxf::QuantParams p = {};
  p.blk = 1;  // GEMM operands: codes in 64-k panels
  p.nt_c = saved_c;
  p.src = (const uint16_t*)x;
  p.rows = mcap;
  p.cols = D;
  p.q_r = (uint8_t*)q_r;
  p.s_r = (uint8_t*)s_r;
  p.q_c = (uint8_t*)q_c;
  p.s_c = (uint8_t*)s_c;
  p.ldc = mcap;
  p.sr_rs = 4; p.sr_kbs = 4 * mcap;  // 128-k planes
  p.sc_rs = 4; p.sc_kbs = 4 * D;
  p.offs = offs;
  p.counts = counts;
  p.E = E;
  p.pad = pad;
  p.status = status;
  return p;
}

hipError_t mxf_launch_quant_tokens(const void* x, int64_t mcap, int64_t D, const int32_t* offs,
                                   const int32_t* counts, int E, int pad, void* q_r, void* s_r,
                                   void* q_c, void* s_c, int32_t* status, bool saved_c, hipStream_t st) {
  return mxf::launch_quant(mxf::QK_MASKED, 3,
                           token_params(x, mcap, D, offs, counts, E, pad, q_r, s_r, q_c, s_c, status, saved_c), 1, st);
}

// Fused dispatch: dual quantization of the padded token layout [mcap, D] gathered from the token
// matrix x_tokens [n_assign / topk, D] through row_assign (row r: token row_assign[r] / topk;
// pad rows zero; rows >= offs[E] skipped); same outputs and status word as
// mxf_launch_quant_tokens on the permuted matrix.
hipError_t mxf_launch_quant_gather(const void* x_tokens, int64_t n_assign, int topk, const int32_t* row_assign,
                                   int64_t mcap, int64_t D, const int32_t* offs, const int32_t* counts, int E,
                                   int pad, void* q_r, void* s_r, void* q_c, void* s_c, int32_t* status,
                                   hipStream_t st) {
  mxf::QuantParams p = {};
  p.blk = 1;  // GEMM operands: codes in 64-k panels
  p.nt_c = 1;  // column codes are saved for the backward pass
  p.src = (const uint16_t*)x_tokens;
  p.rows = mcap;
  p.cols = D;
  p.q_r = (uint8_t*)q_r; p.s_r = (uint8_t*)s_r; p.q_c = (uint8_t*)q_c; p.s_c = (uint8_t*)s_c;
  p.ldc = mcap;
  p.sr_rs = 4; p.sr_kbs = 4 * mcap;
  p.sc_rs = 4; p.sc_kbs = 4 * D;
  p.offs = offs; p.counts = counts; p.E = E; p.pad = pad;
  p.status = status;
  p.row_assign = row_assign;
  p.n_assign = n_assign;
  p.topk = topk;
  return mxf::launch_quant(mxf::QK_GATHER, 3, p, 1, st);
}

// Unfused plan: h = SwiGLU of the BF16 FC1 output h13 [mcap, 2F] (packed gate/up order),
// dual-quantized like the token operands (hq_r [mcap, F], hq_c [F, mcap], 128-k plane scales).
hipError_t mxf_launch_swiglu_quant(const void* h13, int64_t mcap, int64_t F, const int32_t* offs,
                                   const int32_t* counts, int E, int pad, void* q_r, void* s_r, void* q_c,
                                   void* s_c, hipStream_t st) {
  mxf::QuantParams p = {};
  p.blk = 1;  // GEMM operands: codes in 64-k panels
  p.nt_c = 1;  // column codes are saved for the backward pass
  p.src = (const uint16_t*)h13;
  p.rows = mcap;
  p.cols = F;
  p.q_r = (uint8_t*)q_r; p.s_r = (uint8_t*)s_r; p.q_c = (uint8_t*)q_c; p.s_c = (uint8_t*)s_c;
  p.ldc = mcap;
  p.sr_rs = 4; p.sr_kbs = 4 * mcap;
  p.sc_rs = 4; p.sc_kbs = 4 * F;
  p.offs = offs; p.counts = counts; p.E = E; p.pad = pad;
  return mxf::launch_quant(mxf::QK_SWIGLU, 3, p, 1, st);
}

// Unfused plan: dH13 = pack(dG, dU) from the BF16 dh [mcap, F] and h13 [mcap, 2F], dual-quantized
// (dhq_r [mcap, 2F], dhq_c [2F, mcap], 128-k plane scales).
hipError_t mxf_launch_dswiglu_quant(const void* dh, const void* h13, int64_t mcap, int64_t F, const int32_t* offs,
                                    const int32_t* counts, int E, int pad, void* q_r, void* s_r, void* q_c,
                                    void* s_c, hipStream_t st) {
  mxf::QuantParams p = {};
  p.blk = 1;  // GEMM operands: codes in 64-k panels
  p.src = (const uint16_t*)dh;
  p.src2 = (const uint16_t*)h13;
  p.rows = mcap;
  p.cols = 2 * F;
  p.q_r = (uint8_t*)q_r; p.s_r = (uint8_t*)s_r; p.q_c = (uint8_t*)q_c; p.s_c = (uint8_t*)s_c;
  p.ldc = mcap;
  p.sr_rs = 4; p.sr_kbs = 4 * mcap;
  p.sc_rs = 4; p.sc_kbs = 4 * 2 * F;
  p.offs = offs; p.counts = counts; p.E = E; p.pad = pad;
  return mxf::launch_quant(mxf::QK_DSWIGLU, 3, p, 1, st);
}

// Dual quantization of a batch of E weight matrices [rows, cols], scales in 128-k planes per
// matrix ([cols/128][rows][4] and [rows/128][cols][4]). pack13 = true reads w1/w3
// [E, rows/2, cols] and quantizes their [E, rows, cols] 32-block interleave.
static mxf::QuantParams weight_params(const void* w, const void* w3, bool pack13, int64_t rows, int64_t cols,
                                      void* q_r, void* s_r, void* q_c, void* s_c) {
  mxf::QuantParams p = {};
  p.blk = 1;  // GEMM operands: codes in 64-k panels
  p.nt_c = 1;  // column codes are saved for the backward pass
  p.src = (const uint16_t*)w;
  p.src2 = (const uint16_t*)w3;
  p.rows = rows;
  p.cols = cols;
  p.src_bs = pack13 ? (rows / 2) * cols : rows * cols;
  p.q_r = (uint8_t*)q_r;
  p.s_r = (uint8_t*)s_r;
  p.q_c = (uint8_t*)q_c;
  p.s_c = (uint8_t*)s_c;
  p.qr_bs = rows * cols;
  p.sr_bs = rows * (cols / 32);
  p.qc_bs = rows * cols;
  p.sc_bs = cols * (rows / 32);
  p.ldc = rows;
  p.sr_rs = 4; p.sr_kbs = 4 * rows;  // 128-k planes per matrix
  p.sc_rs = 4; p.sc_kbs = 4 * cols;
  return p;
}

hipError_t mxf_launch_quant_weights(const void* w, const void* w3, bool pack13, int64_t E, int64_t rows,
                                    int64_t cols, void* q_r, void* s_r, void* q_c, void* s_c,
                                    hipStream_t st) {
  return mxf::launch_quant(pack13 ? mxf::QK_PACK13 : mxf::QK_PLAIN, 3,
                           weight_params(w, w3, pack13, rows, cols, q_r, s_r, q_c, s_c), E, st);
}

// The forward's three quantizations (W13 pack + dual, W2 dual, X dual under the token layout)
// in one launch (quant_fwd_kernel); x == nullptr leaves X out (its codes were written by the
// fused dispatch). Same outputs as mxf_launch_quant_weights (twice) and mxf_launch_quant_tokens.
hipError_t mxf_launch_quant_fwd(const void* w1, const void* w3, const void* w2, int64_t E, int64_t D, int64_t F,
                                void* w13q_r, void* w13s_r, void* w13q_c, void* w13s_c, void* w2q_r, void* w2s_r,
                                void* w2q_c, void* w2s_c, const void* x, int64_t mcap, const int32_t* offs,
                                const int32_t* counts, int pad, void* xq_r, void* xs_r, void* xq_c, void* xs_c,
                                int32_t* status, hipStream_t st) {
  mxf::QuantFwd f = {};
  f.w13 = weight_params(w1, w3, true, 2 * F, D, w13q_r, w13s_r, w13q_c, w13s_c);
  f.w2 = weight_params(w2, nullptr, false, D, F, w2q_r, w2s_r, w2q_c, w2s_c);
  f.g13 = mxf::grid_of(mxf::QK_PACK13, f.w13, E);
  f.g2 = mxf::grid_of(mxf::QK_PLAIN, f.w2, E);
  f.n13 = f.g13.x * f.g13.y * f.g13.z;
  f.n2 = f.g2.x * f.g2.y * f.g2.z;
  if (x) {
    f.x = token_params(x, mcap, D, offs, counts, (int)E, pad, xq_r, xs_r, xq_c, xs_c, status, true);
    f.gx = mxf::grid_of(mxf::QK_MASKED, f.x, 1);
    f.nx = f.gx.x * f.gx.y * f.gx.z;
  }
  const int64_t n = f.n13 + f.n2 + f.nx;
  if (n == 0) return hipSuccess;
  if (n > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mxf::quant_fwd_kernel, dim3((unsigned)n), dim3(256), 0, st, f);
  return hipGetLastError();
}

hipError_t mxf_launch_dequantize(const void* q, const void* s, int64_t rows, int64_t cols, bool bf16, bool e5m2,
                                 void* out, hipStream_t st) {
  const int64_t units = (cols % 16 == 0) ? rows * (cols / 16) : rows * cols;
  if (units == 0) return hipSuccess;
  // one unit per thread up to 2^24 units; the grid-stride loop covers larger inputs (a grid capped
  // at 8192 workgroups, each thread looping 3-4 times, measured 15% slower on [16384, 7168])
  const dim3 grid((unsigned)std::min<int64_t>((units + 255) / 256, 65536));
  const uint8_t* qq = (const uint8_t*)q;
  const uint8_t* ss = (const uint8_t*)s;
  if (bf16 && !e5m2)
    hipLaunchKernelGGL((mxf::dequant_kernel<true, mxf::FMT_E4M3>), grid, dim3(256), 0, st, qq, ss, rows, cols, out);
  else if (!e5m2)
    hipLaunchKernelGGL((mxf::dequant_kernel<false, mxf::FMT_E4M3>), grid, dim3(256), 0, st, qq, ss, rows, cols, out);
  else if (bf16)
    hipLaunchKernelGGL((mxf::dequant_kernel<true, mxf::FMT_E5M2>), grid, dim3(256), 0, st, qq, ss, rows, cols, out);
  else
    hipLaunchKernelGGL((mxf::dequant_kernel<false, mxf::FMT_E5M2>), grid, dim3(256), 0, st, qq, ss, rows, cols, out);
  return hipGetLastError();
}

hipError_t mxf_launch_pack13(const void* w1, const void* w3, void* w13, int64_t E, int64_t F,
                             int64_t D, bool pack, hipStream_t st) {
  const int64_t total = E * 2 * F * (D / 8);
  if (total == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 65536);
  if (pack)
    hipLaunchKernelGGL(mxf::pack13_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint16_t*)w1, (const uint16_t*)w3, (uint16_t*)w13, nullptr, nullptr, E, F, D);
  else
    hipLaunchKernelGGL(mxf::pack13_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint16_t*)w13, nullptr, nullptr, (uint16_t*)w1, (uint16_t*)w3, E, F, D);
  return hipGetLastError();
}
