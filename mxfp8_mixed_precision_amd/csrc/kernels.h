// Internal interface between the C ABI layer and the HIP kernels (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxf {

// Code addressing of the MLP's GEMM operands (64-k panels): a code matrix with R rows and K
// columns (K the contraction axis) is stored as K/64 panels [R][64]: the byte of (r, k) is at
// (k / 64) * 64R + 64 r + k % 64. A GEMM stage (64 k of 16 consecutive rows) is then one
// contiguous kilobyte.
// Scale addressing (every E8M0 tensor): the byte of (row r, 32-group g) is at
// r * rs + (g / 4) * kbs + g % 4. Row-major [R][G]: rs = G, kbs = 4. The MLP's operands use
// 128-k planes [G/4][R][4] (rs = 4, kbs = 4R): the scale words of consecutive rows for one
// 128-k block are contiguous, so a tile's scales for a K step are one contiguous run.
struct GemmParams {
  const uint8_t* A;   // codes in 64-k panels, panel stride akp (= 64 x rows of A)
  const uint8_t* As;  // scales: row stride ldas, 128-k plane stride kbsa
  const uint8_t* B;   // codes in 64-k panels, panel stride bkp (per expert for M-grouped B)
  const uint8_t* Bs;
  int64_t akp, ldas, bkp, ldbs;
  int64_t kbsa, kbsb;
  int64_t b_es, bs_es;  // M-grouped: bytes between experts in B / Bs
  int64_t M, N, K;      // M-grouped: M = m_capacity. K-grouped: output [M, N] per expert
  const int32_t* offs;
  const int32_t* counts;
  int E, pad;
  int64_t mcap;
  int ncu;           // compute units of the device (set by the launcher; tail sub-tiling; 0: none)
  // epilogue
  void* C;           // STORE: [M, N] (+ e * c_es for K-grouped); UNPACK13: dW1
  void* C2;          // UNPACK13: dW3
  int64_t ldc, c_es;
  int out_f32;
  uint16_t* h13;     // SWIGLU: written, DSWIGLU: read; fragment-tiled (4 KB per 32x32 h block)
  uint8_t* q_r;      // SWIGLU: hq_r [mcap, F];  DSWIGLU: dhq_r [mcap, 2F] (64-k panels)
  uint8_t* s_r;      // their scales: row stride sr_rs, plane stride sr_kbs
  uint8_t* q_c;      // SWIGLU: hq_c [F, mcap];  DSWIGLU: dhq_c [2F, mcap] (64-k panels)
  uint8_t* s_c;      // row stride sc_rs, plane stride sc_kbs
  int64_t sr_rs, sr_kbs, sc_rs, sc_kbs;
  float* dbg;        // optional fp32 copy of the accumulator ([mcap, N])
};

}  // namespace mxf

// quantize.hip
hipError_t mxf_launch_quantize(const void* x, int64_t rows, int64_t cols, uint32_t mode, bool e5m2, void* q_row,
                               void* s_row, void* q_col, void* s_col, hipStream_t st);
hipError_t mxf_launch_quant_tokens(const void* x, int64_t mcap, int64_t D, const int32_t* offs,
                                   const int32_t* counts, int E, int pad, void* q_r, void* s_r,
                                   void* q_c, void* s_c, int32_t* status, bool saved_c, hipStream_t st);
hipError_t mxf_launch_quant_weights(const void* w, const void* w3, bool pack13, int64_t E, int64_t rows,
                                    int64_t cols, void* q_r, void* s_r, void* q_c, void* s_c,
                                    hipStream_t st);
hipError_t mxf_launch_quant_fwd(const void* w1, const void* w3, const void* w2, int64_t E, int64_t D, int64_t F,
                                void* w13q_r, void* w13s_r, void* w13q_c, void* w13s_c, void* w2q_r, void* w2s_r,
                                void* w2q_c, void* w2s_c, const void* x, int64_t mcap, const int32_t* offs,
                                const int32_t* counts, int pad, void* xq_r, void* xs_r, void* xq_c, void* xs_c,
                                int32_t* status, hipStream_t st);
hipError_t mxf_launch_swiglu_quant(const void* h13, int64_t mcap, int64_t F, const int32_t* offs,
                                   const int32_t* counts, int E, int pad, void* q_r, void* s_r, void* q_c,
                                   void* s_c, hipStream_t st);
hipError_t mxf_launch_dswiglu_quant(const void* dh, const void* h13, int64_t mcap, int64_t F, const int32_t* offs,
                                    const int32_t* counts, int E, int pad, void* q_r, void* s_r, void* q_c,
                                    void* s_c, hipStream_t st);
hipError_t mxf_launch_quant_gather(const void* x_tokens, int64_t n_assign, int topk, const int32_t* row_assign,
                                   int64_t mcap, int64_t D, const int32_t* offs, const int32_t* counts, int E,
                                   int pad, void* q_r, void* s_r, void* q_c, void* s_c, int32_t* status,
                                   hipStream_t st);
hipError_t mxf_launch_dequantize(const void* q, const void* s, int64_t rows, int64_t cols, bool bf16, bool e5m2,
                                 void* out, hipStream_t st);
hipError_t mxf_launch_pack13(const void* w1, const void* w3, void* w13, int64_t E, int64_t F,
                             int64_t D, bool pack, hipStream_t st);
// dispatch.hip
size_t mxf_route_plan_workspace_bytes(int64_t n, int E);
hipError_t mxf_route_scratch(void** ptr, size_t* bytes);
hipError_t mxf_launch_route_plan(const int32_t* idx, int32_t n, int E, int pad, int64_t mcap, int32_t* offs,
                                 int32_t* counts, int32_t* row_assign, int32_t* assign_row, int32_t* status,
                                 void* workspace, hipStream_t st);
hipError_t mxf_launch_permute(const void* x, int64_t n_assign, int topk, int64_t D, const int32_t* offs, int E,
                              const int32_t* row_assign, int64_t mcap, void* out, hipStream_t st);
// gemm.hip
hipError_t mxf_launch_gemm_mgroup(int epi, const mxf::GemmParams& p, hipStream_t st);
hipError_t mxf_launch_gemm_kgroup(int epi, const mxf::GemmParams& p, hipStream_t st);
// FC1 dgrad (M-grouped, plain store), FC1 wgrad (K-grouped, W13 unpack) and FC2 wgrad
// (K-grouped, plain store) in one launch, where each of them runs on 256-row tiles
// (mxf_gemm_bwd3_fits; otherwise the launcher returns hipErrorInvalidValue and the caller
// launches them one by one).
bool mxf_gemm_bwd3_fits(const mxf::GemmParams& w1, const mxf::GemmParams& w2, const mxf::GemmParams& d1);
hipError_t mxf_launch_gemm_bwd3(const mxf::GemmParams& w1, const mxf::GemmParams& w2, const mxf::GemmParams& d1,
                                hipStream_t st);
// hbm.hip
hipError_t mxf_launch_hbm_probe(int mode, const void* src, void* dst, int64_t bytes, int ncu, hipStream_t st);
// mfma_probe.hip
hipError_t mxf_launch_mfma_probe(int mode, const void* src, int64_t bytes, int stages, int blocks, float* out,
                                 hipStream_t st);
