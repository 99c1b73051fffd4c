/*
 * mxfp8.h -- C ABI of the MI355X (gfx950) MXFP8 routed-experts SwiGLU MLP library.
 *
 * What the library computes, with the passages that define it:
 *
 *  - MXFP8 block quantization: tensors are split in groups of 32 consecutive
 *    elements (afd-plugin PR #475 "quantize the A2E FFN transport to MXFP8",
 *    sections "Purpose" and "Test Plan"); each group stores one E8M0 scale byte
 *    and 32 E4M3 codes. The scale exponent is floor(log2(amax)) - 8 clamped to
 *    [-127, 127] and the codes are round-to-nearest-even saturated to +-448 (the
 *    OCP MX v1.0 MXFP8 rule). An all-zero group gets scale byte 0x00; a group
 *    holding NaN or Inf gets 0xFF and NaN codes (0x7F | sign).
 *    E8M0 byte b means 2^(b-127); 0x00 is 2^-127 and 0xFF is NaN (PR #475,
 *    review on E8M0 endpoint decoding).
 *  - "Dual" quantization (torchtitan PR #12 "Wire the fully-fused grouped-GEMM
 *    MXFP8 plan behind fusion_plan", section "What it adds"): the same matrix
 *    quantized along rows (q_row [rows, cols], s_row [rows, cols/32]) and along
 *    columns, stored transposed (q_col [cols, rows], s_col [cols, rows/32]).
 *  - The routed-experts SwiGLU MLP as four fused ops (same section): FC1
 *    grouped GEMM + SwiGLU + dual MXFP8 quantization, FC2 GEMM, fused dSwiGLU
 *    backward, wgrad -- over a padded expert-major token layout with per-expert
 *    alignment pad_multiple (128 or 256). Parameters are stock: w1 (gate) and
 *    w3 (up) [E, F, D], w2 [E, D, F], all BF16; the library packs w1/w3 into a
 *    [E, 2F, D] 32-block order internally. The BF16 post-activation is never
 *    written (torchtitan PR #2 "fused gated-activation (SwiGLU) + MXFP8
 *    quantization kernel override", section "Summary").
 *
 * Conventions (torchtitan PR #2, section "Fail-loud contract"):
 *  - Every pointer argument is a DEVICE pointer unless marked "host".
 *  - The caller owns every buffer. The library never allocates or frees device
 *    memory, never synchronises (except mxf_read_status and mxf_profile_end)
 *    and keeps no pointer after a call returns.
 *  - Library-owned state: besides the thread-local error string, the library
 *    keeps, per host thread, (a) two helper streams and three events per device,
 *    created on the first MLP call with MXF_CONCURRENT and kept until the
 *    process ends, and (b) the timing events of mxf_profile_begin (kept and
 *    reused until the thread ends), plus a per-device cache of the device's
 *    architecture and compute-unit count. Without MXF_CONCURRENT and without
 *    profiling no stream or event is created.
 *  - All arguments are validated on the host before anything is launched. On
 *    failure nothing is launched, a status code is returned and
 *    mxf_last_error() names the offending argument and value. There is no
 *    fallback path: an unsupported configuration is an error.
 *  - Token offsets live on the device and are checked there (non-decreasing,
 *    multiples of pad_multiple, within capacity, counts <= segment). A
 *    violation makes every kernel of the call skip its work and records a
 *    non-zero status word in the workspace, read with mxf_read_status.
 *  - All work is enqueued on the given stream (a hipStream_t passed as void*;
 *    NULL is the default stream). Calls that share a workspace must not overlap.
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXF_ABI_VERSION 1

/* Status codes. There is no dtype code: every argument's element type is fixed by the entry
 * point (BF16 inputs, u8 codes and scales, int32 offsets; the output type is chosen by a flag),
 * and no workspace-size code: workspace and saved sizes are derived from the descriptor by
 * mxf_mlp_workspace_bytes / mxf_mlp_saved_bytes, not passed in. */
typedef enum {
  MXF_OK = 0,
  MXF_E_NULL = 1,      /* a required pointer is NULL */
  MXF_E_SHAPE = 2,     /* a dimension is negative, not a required multiple, or too large */
  MXF_E_ALIGN = 3,     /* a pointer is not aligned as required (16 bytes; int32 arrays 4) */
  MXF_E_DEVICE = 4,    /* the current device is not a gfx950 GPU */
  MXF_E_ARG = 5,       /* an enum/flag argument is out of range */
  MXF_E_HIP = 6        /* the HIP runtime reported an error (message in mxf_last_error) */
} mxf_status;

/* Device-side status word values (mxf_read_status). */
#define MXF_DEV_OK 0
#define MXF_DEV_BAD_OFFSETS 1   /* offs/counts violate the layout contract; no output was written */
#define MXF_DEV_BAD_EXPERT 2    /* mxf_route_plan: an expert id outside [0, E); it was dropped */
#define MXF_DEV_OVERFLOW 3      /* mxf_route_plan: the padded layout exceeds m_capacity */

/* ABI version of the loaded library; equals MXF_ABI_VERSION of the header it was built with. */
int mxf_abi_version(void);

/* Capability query for a device ordinal. On success *caps gets bit 0 set when the device is
 * a gfx950 GPU (block-scaled FP8 MFMA), which every compute entry point requires.
 * Errors: MXF_E_NULL (caps), MXF_E_HIP (bad ordinal). */
#define MXF_CAP_GFX950 1u
mxf_status mxf_query_device(int device, uint32_t* caps /* host */);

/* Thread-local, NUL-terminated description of the last error on this thread ("" if none).
 * Valid until the next library call on the same thread. */
const char* mxf_last_error(void);

/* ------------------------------------------------------------------ standalone quantizer */

#define MXF_ROW 1u   /* groups along each row    -> q_row [rows, cols], s_row [rows, cols/32] */
#define MXF_COL 2u   /* groups along each column -> q_col [cols, rows], s_col [cols, rows/32] */
#define MXF_E5M2 4u  /* mode flag: E5M2 elements instead of E4M3 (see below) */

/* MXFP8 quantization of a row-major BF16 matrix x [rows, cols] (see top of file).
 * mode: MXF_ROW, MXF_COL or both (dual: x is read once), optionally | MXF_E5M2: E5M2 elements
 * (the alternative element format afd-plugin PR #475 offers for the transport, under the same
 * E8M0 scale): scale exponent floor(log2(amax)) - 15, codes RNE saturated to +-57344
 * (0x7B | sign), NaN groups 0xFF with codes 0x7F | sign.
 * Requires cols % 32 == 0; with MXF_COL also rows % 32 == 0; rows, cols >= 0. An empty matrix
 * (rows or cols 0) is a no-op that accepts NULL pointers.
 * Outputs not selected by mode may be NULL. All outputs are dense row-major u8 arrays.
 * Pointers must be 16-byte aligned (scale arrays: any alignment).
 * Errors: MXF_E_NULL, MXF_E_SHAPE, MXF_E_ALIGN, MXF_E_ARG (mode), MXF_E_DEVICE, MXF_E_HIP. */
mxf_status mxfp8_quantize(const void* x, int64_t rows, int64_t cols, uint32_t mode,
                          void* q_row, void* s_row, void* q_col, void* s_col, void* stream);

/* ------------------------------------------------------------------ dequantization */

#define MXF_DEQ_BF16 0u  /* out is BF16 */
#define MXF_DEQ_F32 1u   /* out is FP32 */
#define MXF_DEQ_E5M2 2u  /* flag: the codes are E5M2 (field 31: +-Inf for mantissa 0, else NaN) */

/* Decode of row-wise MXFP8 (the receive side of an MXFP8 transport; afd-plugin PR #475
 * "quantize the A2E FFN transport to MXFP8", third review on E8M0 decoding and on hidden sizes
 * that are not a multiple of 32).
 * q [rows, cols] u8 E4M3 codes; s [rows, ceil(cols/32)] u8 E8M0 bytes: element (r, c) uses
 * s[r, c / 32], so when cols % 32 != 0 the last group of a row is short and has its own byte.
 * out [rows, cols] row-major = E4M3(q) * 2^(s - 127) rounded once (RNE) to BF16 or FP32
 * (out_type MXF_DEQ_BF16 / MXF_DEQ_F32, | MXF_DEQ_E5M2 for E5M2 codes); overflow gives +-Inf. Scale byte 0x00 is 2^-127
 * (not zero), 0xFF is NaN (the whole group decodes to NaN); codes 0x7F / 0xFF are NaN (the sign
 * and payload of a NaN result are unspecified).
 * Any rows, cols >= 0 (empty is a no-op accepting NULL); q and out 16-byte aligned.
 * Errors: MXF_E_NULL, MXF_E_SHAPE, MXF_E_ALIGN, MXF_E_ARG (out_type), MXF_E_DEVICE, MXF_E_HIP. */
mxf_status mxfp8_dequantize(const void* q, const void* s, int64_t rows, int64_t cols, uint32_t out_type,
                            void* out, void* stream);

/* ------------------------------------------------------------------ routed-experts MLP */

#define MXF_OUT_F32 1u     /* y, dx, dw1, dw3, dw2 are FP32 instead of BF16 */
#define MXF_DEBUG_F32 2u   /* also store the FP32 FC1 output and FP32 dh (FC2 dgrad) in the
                              workspace (tensors MXF_T_H13_F32, MXF_T_DH_F32) */
#define MXF_UNFUSED 8u     /* the unfused plan, for A/B comparison: FC1 and FC2 dgrad write BF16
                              (the FC1 output g | u row-major into MXF_T_H13, dh into MXF_T_DH16)
                              and standalone SwiGLU / dSwiGLU + dual-quantization kernels read
                              them back; same results as the fused plan. Not with MXF_DEBUG_F32. */
#define MXF_X_QUANTIZED 16u /* grouped_mlp_fwd: X's dual codes were already written into saved /
                              workspace by mxfp8_dispatch_quantize (same desc, offs, counts);
                              x is not read and may be NULL */
#define MXF_SERIAL 4u      /* launch every kernel on the caller's stream, one after another:
                              the default, stated explicitly (not with MXF_CONCURRENT). The
                              backward's FC1 wgrad, FC2 wgrad and FC1 dgrad then share one launch
                              where all three run on 256-row tiles (pad_multiple 256, D and 2F
                              multiples of 256) */
#define MXF_CONCURRENT 32u /* run independent launches concurrently on two helper streams forked
                              from and joined into the caller's stream (the backward's FC2 wgrad,
                              FC1 wgrad and FC1 dgrad as three launches beside each other). Measured
                              on MI355X it is slower than the serial order for the DSv3 rank
                              shape (the GEMMs then share their L2 panels); kept for A/B runs */

typedef struct {
  int32_t E;             /* local experts, 1 .. 1024 */
  int32_t D;             /* model dim, multiple of 128 */
  int32_t F;             /* expert hidden dim, multiple of 128 */
  int32_t pad_multiple;  /* 128 or 256: every expert segment is a multiple of this */
  int64_t m_capacity;    /* rows allocated in x/y/dy/dx; multiple of pad_multiple */
  uint32_t flags;        /* MXF_OUT_F32 | MXF_DEBUG_F32 | MXF_SERIAL | MXF_CONCURRENT | MXF_UNFUSED |
                            MXF_X_QUANTIZED */
} mxf_mlp_desc;

/* Tensors held in the caller's buffers (for tests and inspection). Region: 0 = workspace,
 * 1 = saved (forward -> backward context). Codes u8, scales u8 (E8M0), h13 BF16.
 *
 * MXF_T_H13 (the BF16-rounded FC1 output g | u, kept for the backward pass) is row-major
 * [Mcap, 2F] in packed order under MXF_UNFUSED; otherwise it is stored fragment-tiled, in the order the matrix-core accumulators produce and consume it: records
 * of 2048 BF16 values, record R * (F/32) + J holding rows 32R .. 32R+31 and h columns
 * 32J .. 32J+31; inside a record, index ((2 s + (k >> 1)) * 64 + c + 32 b) * 8 + 4 (k & 1) + j
 * (s = 0 gate, 1 up; b < 2, c < 32, k < 4, j < 4) holds row 32R + 8k + 4b + j, column 32J + c
 * of the gate (s = 0) or up (s = 1) projection. Same size as [Mcap, 2F].
 *
 * Every code tensor below (…Q_R, …Q_C; the shapes listed are [R, K], per expert for the
 * weights, K the axis the 32-groups run along) is stored in 64-k panels, the order the GEMM
 * loads it in: the byte of (row r, column k) is at (k / 64) * 64R + 64r + k % 64, so 64 k of
 * 16 consecutive rows are one contiguous kilobyte. Same size as [R, K].
 *
 * Every scale tensor below (…S_R, …S_C) holds the E8M0 bytes of a code tensor with R rows
 * and K columns (the shapes listed are [R, K/32], per expert for the weights) in 128-k
 * planes, the order the GEMM loads them in: the byte of (row r, 32-group g) is at
 * (g / 4) * 4R + 4r + g % 4, so the four scale bytes of a row for one 128-wide block of K
 * are a word and the words of consecutive rows are adjacent. Same size as [R, K/32]. */
typedef enum {
  MXF_T_STATUS = 0,                                       /* int32 status word (workspace) */
  MXF_T_XQ_R, MXF_T_XS_R,                                 /* [Mcap, D], [Mcap, D/32]       (ws)    */
  MXF_T_XQ_C, MXF_T_XS_C,                                 /* [D, Mcap], [D, Mcap/32]       (saved) */
  MXF_T_W13Q_R, MXF_T_W13S_R,                             /* [E, 2F, D], [E, 2F, D/32]     (ws)    */
  MXF_T_W13Q_C, MXF_T_W13S_C,                             /* [E, D, 2F], [E, D, 2F/32]     (saved) */
  MXF_T_W2Q_R, MXF_T_W2S_R,                               /* [E, D, F], [E, D, F/32]       (ws)    */
  MXF_T_W2Q_C, MXF_T_W2S_C,                               /* [E, F, D], [E, F, D/32]       (saved) */
  MXF_T_H13,                                              /* Mcap*2F BF16, fragment-tiled (saved) */
  MXF_T_HQ_R, MXF_T_HS_R,                                 /* [Mcap, F], [Mcap, F/32]       (ws)    */
  MXF_T_HQ_C, MXF_T_HS_C,                                 /* [F, Mcap], [F, Mcap/32]       (saved) */
  MXF_T_DYQ_R, MXF_T_DYS_R, MXF_T_DYQ_C, MXF_T_DYS_C,     /* like X                        (ws)    */
  MXF_T_DHQ_R, MXF_T_DHS_R,                               /* [Mcap, 2F], [Mcap, 2F/32]     (ws)    */
  MXF_T_DHQ_C, MXF_T_DHS_C,                               /* [2F, Mcap], [2F, Mcap/32]     (ws)    */
  MXF_T_H13_F32,                                          /* [Mcap, 2F] FP32 (ws, MXF_DEBUG_F32)   */
  MXF_T_DH_F32,                                           /* [Mcap, F] FP32  (ws, MXF_DEBUG_F32)   */
  MXF_T_DH16,                                             /* [Mcap, F] BF16  (ws, MXF_UNFUSED)     */
  MXF_T_COUNT
} mxf_tensor;

/* Bytes the caller must provide for `saved` and for `workspace` (one workspace serves both
 * grouped_mlp_fwd and grouped_mlp_bwd). Return 0 when the descriptor is invalid. */
size_t mxf_mlp_saved_bytes(const mxf_mlp_desc* desc /* host */);
size_t mxf_mlp_workspace_bytes(const mxf_mlp_desc* desc /* host */);

/* Where tensor `which` lives: *region (0 workspace, 1 saved), *offset and *bytes in it.
 * Errors: MXF_E_NULL, MXF_E_SHAPE (desc), MXF_E_ARG (which). */
mxf_status mxf_mlp_tensor(const mxf_mlp_desc* desc /* host */, int which, int* region /* host */,
                          size_t* offset /* host */, size_t* bytes /* host */);

/* Streams: fwd and bwd enqueue their kernels asynchronously on `stream`. With MXF_CONCURRENT
 * some backward kernels run on two helper streams owned by the calling host thread (one pair per
 * device);
 * the helpers start after everything previously enqueued on `stream` and `stream` waits for them
 * before the call returns, so the call behaves as one ordered unit of work on `stream`.
 *
 * Forward. offs: int32 [E+1] (offs[0] = 0, non-decreasing, multiples of pad_multiple,
 * offs[E] <= m_capacity); expert e owns rows [offs[e], offs[e+1]). counts: int32 [E] real
 * rows per expert (counts[e] <= offs[e+1]-offs[e]) or NULL (every row real). Rows in
 * [offs[e]+counts[e], offs[e+1]) are pad: read as zero, written as zero. Rows at or after
 * offs[E] are never read or written.
 * x [m_capacity, D] BF16; w1, w3 [E, F, D] BF16; w2 [E, D, F] BF16;
 * y [m_capacity, D] BF16 (FP32 with MXF_OUT_F32).
 * saved: mxf_mlp_saved_bytes; keep it unchanged until grouped_mlp_bwd has run.
 * workspace: mxf_mlp_workspace_bytes. Tensor pointers 16-byte aligned; offs and counts
 * 4-byte aligned. */
mxf_status grouped_mlp_fwd(const mxf_mlp_desc* desc /* host */, const int32_t* offs,
                           const int32_t* counts, const void* x, const void* w1, const void* w3,
                           const void* w2, void* y, void* saved, void* workspace, void* stream);

/* Backward (straight-through quantization). dy [m_capacity, D] BF16 (pad rows read as zero);
 * saved as written by grouped_mlp_fwd with the same desc/offs/counts.
 * dx [m_capacity, D]; dw1, dw3 [E, F, D]; dw2 [E, D, F] -- BF16, or FP32 with MXF_OUT_F32.
 * Weight gradients are overwritten (not accumulated); an expert with no routed rows gets
 * exact zeros. */
mxf_status grouped_mlp_bwd(const mxf_mlp_desc* desc /* host */, const int32_t* offs,
                           const int32_t* counts, const void* dy, const void* saved, void* dx,
                           void* dw1, void* dw3, void* dw2, void* workspace, void* stream);

/* ------------------------------------------------------------------ dispatch */

/* Dispatch of routed tokens into the padded expert-major layout the MLP consumes: every
 * expert's rows form one segment whose length is a multiple of pad_multiple, pad rows zero
 * (torchtitan PR #12 "Wire the fully-fused grouped-GEMM MXFP8 plan behind fusion_plan",
 * section "What it adds": the padded dispatcher that the kernels' per-expert alignment
 * requires; torchtitan PR #2, section "Summary"). Inside a segment, rows follow the
 * assignment index a = t * topk + k (token t's k-th choice), so the layout is unique.
 *
 * Routing plan. expert_idx: int32 [tokens, topk], each in [0, E) (a token may name an expert
 * more than once: each assignment gets its own row). Outputs (int32, caller-owned):
 *   offs [E+1], counts [E] -- as grouped_mlp_fwd takes them (counts[e] = assignments routed to
 *     e, offs[e+1] - offs[e] = counts[e] rounded up to pad_multiple);
 *   row_assign [m_capacity] -- assignment held by row r, -1 for a pad row; rows at or past
 *     offs[E] are not written;
 *   assign_row [tokens * topk] -- row of assignment a, or -1 (dropped, or past m_capacity).
 *   status (may be NULL): MXF_DEV_OK; MXF_DEV_BAD_EXPERT if an id is outside [0, E) (the
 *     assignment is dropped, the rest is placed); else MXF_DEV_OVERFLOW if offs[E] >
 *     m_capacity (offs and counts still describe the whole layout; rows past the capacity
 *     are not written, so the MLP's offsets check rejects these offs).
 *   workspace: device scratch of mxf_route_plan_workspace_bytes(tokens, topk, E) bytes
 *     (4 * (E + 1) per 1024 assignments); its contents on entry do not matter.
 * tokens * topk <= 2^30, 1 <= topk <= 64, 1 <= E <= 1024, 1 <= pad_multiple <= 4096,
 * 0 <= m_capacity <= 2^30; int32 pointers and workspace 4-byte aligned. Three short launches.
 * Errors: MXF_E_NULL, MXF_E_SHAPE, MXF_E_ALIGN, MXF_E_DEVICE, MXF_E_HIP. */
size_t mxf_route_plan_workspace_bytes(int64_t tokens, int32_t topk, int32_t E); /* 0 if invalid */
mxf_status mxf_route_plan(const int32_t* expert_idx, int64_t tokens, int32_t topk, int32_t E,
                          int32_t pad_multiple, int64_t m_capacity, int32_t* offs, int32_t* counts,
                          int32_t* row_assign, int32_t* assign_row, int32_t* status, void* workspace,
                          void* stream);

/* Allocation-free variant of mxf_route_plan, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same plan, with the same arguments and outputs minus `workspace`. Its per-workgroup
 * histograms live in a static device array of MXF_ROUTE_NOALLOC_MAX_BYTES that the library
 * holds on each GPU it runs on until the process ends (the address is looked up on the first
 * call per device). The call allocates nothing. Limit: mxf_route_plan_workspace_bytes(tokens,
 * topk, E) <= MXF_ROUTE_NOALLOC_MAX_BYTES (e.g. E = 16: up to 120M assignments; E = 1024: up to
 * 2M), else MXF_E_SHAPE before any launch. Every call on one GPU shares that array: calls that
 * overlap on one GPU (other streams, other host threads) race and give undefined results;
 * calls ordered on one stream are safe (the array's contents on entry do not matter).
 * Errors: as mxf_route_plan. */
#define MXF_ROUTE_NOALLOC_MAX_BYTES (8u << 20)
mxf_status mxf_route_plan_noalloc(const int32_t* expert_idx, int64_t tokens, int32_t topk, int32_t E,
                                  int32_t pad_multiple, int64_t m_capacity, int32_t* offs,
                                  int32_t* counts, int32_t* row_assign, int32_t* assign_row,
                                  int32_t* status, void* stream);

/* BF16 permute: x_out [m_capacity, D] row r (r < min(offs[E], m_capacity)) = x_tokens
 * [tokens, D] row row_assign[r] / topk, or zeros where row_assign[r] is -1 (or outside
 * [0, tokens * topk)). Rows at or past offs[E] are not written. offs and row_assign as
 * written by mxf_route_plan. D % 8 == 0; x_tokens, x_out 16-byte aligned.
 * Errors: MXF_E_NULL, MXF_E_SHAPE, MXF_E_ALIGN, MXF_E_DEVICE, MXF_E_HIP. */
mxf_status mxf_dispatch_permute(const void* x_tokens, int64_t tokens, int32_t topk, int64_t D, int32_t E,
                                const int32_t* offs, const int32_t* row_assign, int64_t m_capacity,
                                void* x_out, void* stream);

/* Fused dispatch + Q_X: writes the MLP's X operand (MXF_T_XQ_R/XS_R in workspace,
 * MXF_T_XQ_C/XS_C in saved) straight from the token rows, bit-identical to what
 * grouped_mlp_fwd computes from the permuted BF16 matrix, and sets the workspace status word
 * from the offsets check. Follow it with grouped_mlp_fwd under MXF_X_QUANTIZED (same desc
 * otherwise, same offs and counts). x_tokens [tokens, desc->D] BF16, 16-byte aligned;
 * offs, counts and row_assign as written by mxf_route_plan with desc's E, pad_multiple and
 * m_capacity. Errors: as grouped_mlp_fwd plus MXF_E_SHAPE for tokens / topk. */
mxf_status mxfp8_dispatch_quantize(const mxf_mlp_desc* desc /* host */, const int32_t* offs,
                                   const int32_t* counts, const int32_t* row_assign,
                                   const void* x_tokens, int64_t tokens, int32_t topk, void* saved,
                                   void* workspace, void* stream);

/* Synchronises `stream` and copies the device status word of the last fwd/bwd call that
 * used `workspace` into *device_status (MXF_DEV_OK or MXF_DEV_BAD_OFFSETS). */
mxf_status mxf_read_status(const void* workspace, void* stream, int32_t* device_status /* host */);

/* ------------------------------------------------------------------ kernel timing */

/* Per-kernel timing for benchmarks. mxf_profile_begin(capacity) starts recording on the
 * calling thread: each kernel that this thread's later library calls launch is bracketed by
 * two HIP events recorded on the same stream (at most `capacity` launches; the events are
 * created here, not in the timed calls). mxf_profile_end waits for the recorded events and
 * returns, per kernel name, the number of launches and their summed duration in ms; it
 * fills at most max_out entries and sets *n_out to the number filled, then stops recording.
 * Kernel names: quant_fwd (W13, W2 and X quantized in one launch), fc1_swiglu, fc2, quant_dy,
 * fc2_dgrad_dswiglu, bwd_gemms (FC1 wgrad, FC2 wgrad and FC1 dgrad in one launch, on 256-row
 * tiles: pad_multiple 256, D and 2F multiples of 256, not with MXF_CONCURRENT; otherwise
 * fc2_wgrad, fc1_wgrad, fc1_dgrad) (MXF_UNFUSED: fc1, swiglu_quant, fc2_dgrad, dswiglu_quant),
 * quantize, dequantize, route_plan, permute, dispatch_quant_x, hbm_read, hbm_write, hbm_copy.
 * Errors: MXF_E_ARG (capacity < 1 or > 1<<20, or end without begin), MXF_E_NULL, MXF_E_HIP. */
typedef struct {
  char name[32];
  int32_t launches;
  double total_ms;
} mxf_kernel_time;
mxf_status mxf_profile_begin(int32_t capacity);
mxf_status mxf_profile_end(mxf_kernel_time* out /* host */, int32_t max_out, int32_t* n_out /* host */);

/* HBM ceiling kernels (measurement): the read, write and copy rates the device sustains with
 * the access pattern that reaches them (16-byte lanes, one contiguous kilobyte per wavefront
 * instruction, grid-stride over the buffer). The HBM-bound kernels of the library are reported
 * against these rates as well as against the data-sheet bandwidth. Device buffers, 16-byte
 * aligned; bytes a positive multiple of 16 (at most 2^40).
 *   mode 0 (read):  every 16-byte word of src is read once; dst (caller-owned, 1024 bytes:
 *                   64 slots of 16 bytes, zero them first) receives partial XORs, and the
 *                   XOR of its 64 slots is the XOR of all of src's 16-byte words.
 *   mode 1 (write): 16-byte word i of dst becomes four copies of the low 32 bits of i; src unused.
 *   mode 2 (copy):  dst = src (bytes each; the buffers must not overlap).
 * Errors: MXF_E_ARG (mode), MXF_E_SHAPE (bytes), MXF_E_NULL, MXF_E_ALIGN, MXF_E_DEVICE,
 * MXF_E_HIP. Timed under the profiling name hbm_read / hbm_write / hbm_copy. */
mxf_status mxf_hbm_probe(int32_t mode, const void* src, void* dst, int64_t bytes, void* stream);

/* Matrix-core ceiling kernels (measurement): the MXFP8 contraction rate the device sustains
 * with the grouped GEMM's instruction mix, so the GEMMs can be reported against a measured rate
 * as well as against the data-sheet peak. One 256-thread block per CU is the intended launch
 * (blocks = the CU count); each block works a 256 x 256 tile in 64-k stages with
 * v_mfma_scale_f32_32x32x64_f8f6f4 (8,388,608 FLOP per block and stage).
 *   mode 0 (matrix only):  operands read once into registers; the loop is the matrix
 *                          instructions alone.
 *   mode 1 (whole stage):  the GEMM main loop's stage: direct global->LDS operand and scale
 *                          loads into a four-stage ring, LDS fragment reads beside the matrix
 *                          instructions, one barrier per stage. Stage s of block b reads the
 *                          32 KB chunk (37 b + s) mod (bytes / 32768) of src.
 * src: device buffer of bytes E4M3 codes (16-byte aligned; bytes a multiple of 32768, at least
 * 131072, at most 2^40); its first 128 KB also seed the LDS ring. Scales are 127 (a factor of 1).
 * out: device, blocks * 256 floats (16-byte aligned); thread t of block b writes out[256 b + t],
 * the sum of the first accumulator of its 16 fragments -- with every code 0x38 (E4M3 1.0)
 * exactly 1024 * stages. stages: even, in [2, 2^24]; blocks in [1, 65535].
 * Errors: MXF_E_ARG (mode), MXF_E_SHAPE (bytes, stages, blocks), MXF_E_NULL, MXF_E_ALIGN,
 * MXF_E_DEVICE, MXF_E_HIP. Timed under the profiling name mfma_matrix / mfma_stage. */
mxf_status mxf_mfma_probe(int32_t mode, const void* src, int64_t bytes, int32_t stages, int32_t blocks,
                          float* out, void* stream);

/* Test helpers for the [E, 2F, D] 32-block packing: w13[e, 64j+i] = w1[e, 32j+i] and
 * w13[e, 64j+32+i] = w3[e, 32j+i] (i < 32), BF16, and its inverse. F % 32 == 0. */
mxf_status mxf_pack_w13(const void* w1, const void* w3, void* w13, int32_t E, int32_t F,
                        int32_t D, void* stream);
mxf_status mxf_unpack_w13(const void* w13, void* w1, void* w3, int32_t E, int32_t F, int32_t D,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MXFP8_H */
