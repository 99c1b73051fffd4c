// C ABI of the MXFP8 routed-experts MLP library: argument validation, buffer layout and
// launch sequencing. The public contract (argument meaning, layout, ownership, errors) is
// documented in include/mxfp8.h.
//
// Fail-loud contract (torchtitan PR #2 "[mxfp8 training] fused gated-activation (SwiGLU) +
// MXFP8 quantization kernel override", section "Fail-loud contract"): every unsupported
// configuration is rejected before anything is launched, with a message naming the offending
// value; there is no fallback path. Data-dependent token counts are checked on the device
// (the analogue of deferred asserts): the kernels skip their work and a status word records
// the violation.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"
#include "mxfp8.h"

namespace {

thread_local std::string g_err;

mxf_status fail(mxf_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

mxf_status hip_fail(hipError_t e, const char* what) {
  return fail(MXF_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MXF_HIP(call, what)                      \
  do {                                           \
    hipError_t _e = (call);                      \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_cap[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

mxf_status check_device() {
  int dev = 0;
  MXF_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MXF_E_DEVICE, "device ordinal %d out of range", dev);
  int c = g_dev_cap[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    hipDeviceProp_t prop;
    MXF_HIP(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties");
    c = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_cap[dev].store(c, std::memory_order_relaxed);
    if (c == 2) return fail(MXF_E_DEVICE, "device %d is %s; this library runs only on gfx950", dev, prop.gcnArchName);
  }
  if (c != 1) return fail(MXF_E_DEVICE, "device %d is not a gfx950 GPU", dev);
  return MXF_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// The token offsets and counts are int32 arrays read by every kernel of an MLP call.
mxf_status check_offs_ptrs(const int32_t* offs, const int32_t* counts) {
  if (!offs) return fail(MXF_E_NULL, "offs is NULL");
  if (!aligned4(offs)) return fail(MXF_E_ALIGN, "offs is not 4-byte aligned");
  if (counts && !aligned4(counts)) return fail(MXF_E_ALIGN, "counts is not 4-byte aligned");
  return MXF_OK;
}

// ------------------------------------------------------------------ kernel timing

struct Profile {
  bool on = false;
  int used = 0;
  std::vector<hipEvent_t> ev;     // 2 per launch
  std::vector<const char*> name;  // per launch
  ~Profile() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
};
thread_local Profile g_prof;

// Brackets one kernel launch with events when profiling is on; `launch` returns hipError_t.
template <class Fn>
hipError_t timed(const char* name, hipStream_t st, Fn&& launch) {
  Profile& P = g_prof;
  const bool rec = P.on && P.used < (int)P.name.size();
  if (rec) {
    hipError_t e = hipEventRecord(P.ev[2 * P.used], st);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (e != hipSuccess) return e;
  if (rec) {
    e = hipEventRecord(P.ev[2 * P.used + 1], st);
    if (e != hipSuccess) return e;
    P.name[P.used++] = name;
  }
  return hipSuccess;
}

// ------------------------------------------------------------------ helper streams

// Launches of one MLP call that do not depend on each other run on two helper streams, forked
// from and joined back into the caller's stream with events (no host synchronisation, and the
// fork/join pattern is legal under stream capture). Each host thread owns its own helpers per
// device, created on first use at the default priority and kept until the process ends.
struct Helpers {
  bool ready = false;
  hipStream_t s[2];
  hipEvent_t fork;
  hipEvent_t join[2];
};
thread_local Helpers g_helpers[kMaxDevices];

// Unless MXF_CONCURRENT is set, the "helpers" are the caller's stream itself (no fork, no join).
mxf_status get_helpers(Helpers** out, uint32_t flags, hipStream_t st) {
  if (!(flags & MXF_CONCURRENT)) {
    thread_local Helpers serial;
    serial.ready = true;
    serial.s[0] = serial.s[1] = st;
    *out = &serial;
    return MXF_OK;
  }
  int dev = 0;
  MXF_HIP(hipGetDevice(&dev), "hipGetDevice");
  Helpers& h = g_helpers[dev];
  if (!h.ready) {
    for (int i = 0; i < 2; ++i) {
      MXF_HIP(hipStreamCreateWithFlags(&h.s[i], hipStreamNonBlocking), "hipStreamCreateWithFlags");
      MXF_HIP(hipEventCreateWithFlags(&h.join[i], hipEventDisableTiming), "hipEventCreateWithFlags");
    }
    MXF_HIP(hipEventCreateWithFlags(&h.fork, hipEventDisableTiming), "hipEventCreateWithFlags");
    h.ready = true;
  }
  *out = &h;
  return MXF_OK;
}

// ------------------------------------------------------------------ MLP buffer layout

struct Layout {
  size_t off[MXF_T_COUNT];
  size_t bytes[MXF_T_COUNT];
  int region[MXF_T_COUNT];
  size_t saved_total;
  size_t ws_total;
};

mxf_status check_desc(const mxf_mlp_desc* d) {
  if (!d) return fail(MXF_E_NULL, "desc is NULL");
  if (d->E < 1 || d->E > 1024) return fail(MXF_E_SHAPE, "E = %d: must be in [1, 1024]", d->E);
  if (d->D <= 0 || d->D % 128) return fail(MXF_E_SHAPE, "D = %d: must be a positive multiple of 128", d->D);
  if (d->F <= 0 || d->F % 128) return fail(MXF_E_SHAPE, "F = %d: must be a positive multiple of 128", d->F);
  if (d->pad_multiple != 128 && d->pad_multiple != 256)
    return fail(MXF_E_SHAPE, "pad_multiple = %d: must be 128 or 256", d->pad_multiple);
  if (d->m_capacity < 0 || d->m_capacity % d->pad_multiple)
    return fail(MXF_E_SHAPE, "m_capacity = %lld: must be a non-negative multiple of pad_multiple (%d)",
                (long long)d->m_capacity, d->pad_multiple);
  if (d->m_capacity > (int64_t)1 << 30)
    return fail(MXF_E_SHAPE, "m_capacity = %lld: larger than 2^30 rows", (long long)d->m_capacity);
  if (d->flags & ~(uint32_t)(MXF_OUT_F32 | MXF_DEBUG_F32 | MXF_SERIAL | MXF_CONCURRENT | MXF_UNFUSED |
                             MXF_X_QUANTIZED))
    return fail(MXF_E_ARG, "flags = 0x%x: unknown bits", d->flags);
  if ((d->flags & MXF_SERIAL) && (d->flags & MXF_CONCURRENT))
    return fail(MXF_E_ARG, "flags = 0x%x: MXF_SERIAL and MXF_CONCURRENT together", d->flags);
  if ((d->flags & MXF_UNFUSED) && (d->flags & MXF_DEBUG_F32))
    return fail(MXF_E_ARG, "flags = 0x%x: MXF_DEBUG_F32 is not available with MXF_UNFUSED", d->flags);
  return MXF_OK;
}

void make_layout(const mxf_mlp_desc* d, Layout* L) {
  const size_t M = (size_t)d->m_capacity, D = (size_t)d->D, F = (size_t)d->F, E = (size_t)d->E;
  const bool dbg = (d->flags & MXF_DEBUG_F32) != 0;
  memset(L, 0, sizeof(*L));
  auto put = [&](int t, int region, size_t* cursor, size_t bytes) {
    L->region[t] = region;
    L->off[t] = *cursor;
    L->bytes[t] = bytes;
    *cursor += (bytes + 255) / 256 * 256;
  };
  size_t sv = 0;
  put(MXF_T_XQ_C, 1, &sv, D * M);
  put(MXF_T_XS_C, 1, &sv, D * M / 32);
  put(MXF_T_W13Q_C, 1, &sv, E * D * 2 * F);
  put(MXF_T_W13S_C, 1, &sv, E * D * 2 * F / 32);
  put(MXF_T_W2Q_C, 1, &sv, E * F * D);
  put(MXF_T_W2S_C, 1, &sv, E * F * D / 32);
  put(MXF_T_H13, 1, &sv, M * 2 * F * 2);
  put(MXF_T_HQ_C, 1, &sv, F * M);
  put(MXF_T_HS_C, 1, &sv, F * M / 32);
  L->saved_total = sv;
  size_t fw = 0;
  put(MXF_T_STATUS, 0, &fw, 4);
  const size_t after_status = fw;
  put(MXF_T_XQ_R, 0, &fw, M * D);
  put(MXF_T_XS_R, 0, &fw, M * D / 32);
  put(MXF_T_W13Q_R, 0, &fw, E * 2 * F * D);
  put(MXF_T_W13S_R, 0, &fw, E * 2 * F * D / 32);
  put(MXF_T_W2Q_R, 0, &fw, E * D * F);
  put(MXF_T_W2S_R, 0, &fw, E * D * F / 32);
  put(MXF_T_HQ_R, 0, &fw, M * F);
  put(MXF_T_HS_R, 0, &fw, M * F / 32);
  put(MXF_T_H13_F32, 0, &fw, dbg ? M * 2 * F * 4 : 0);
  size_t bw = after_status;  // backward tensors reuse the forward-only workspace
  put(MXF_T_DYQ_R, 0, &bw, M * D);
  put(MXF_T_DYS_R, 0, &bw, M * D / 32);
  put(MXF_T_DYQ_C, 0, &bw, D * M);
  put(MXF_T_DYS_C, 0, &bw, D * M / 32);
  put(MXF_T_DHQ_R, 0, &bw, M * 2 * F);
  put(MXF_T_DHS_R, 0, &bw, M * 2 * F / 32);
  put(MXF_T_DHQ_C, 0, &bw, 2 * F * M);
  put(MXF_T_DHS_C, 0, &bw, 2 * F * M / 32);
  put(MXF_T_DH_F32, 0, &bw, dbg ? M * F * 4 : 0);
  put(MXF_T_DH16, 0, &bw, (d->flags & MXF_UNFUSED) ? M * F * 2 : 0);
  L->ws_total = fw > bw ? fw : bw;
}

}  // namespace

// ------------------------------------------------------------------ exported entry points

extern "C" {

int mxf_abi_version(void) { return MXF_ABI_VERSION; }

const char* mxf_last_error(void) { return g_err.c_str(); }

mxf_status mxf_query_device(int device, uint32_t* caps) {
  g_err.clear();
  if (!caps) return fail(MXF_E_NULL, "caps is NULL");
  *caps = 0;
  hipDeviceProp_t prop;
  MXF_HIP(hipGetDeviceProperties(&prop, device), "hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) == 0) *caps |= MXF_CAP_GFX950;
  return MXF_OK;
}

mxf_status mxfp8_quantize(const void* x, int64_t rows, int64_t cols, uint32_t mode, void* q_row,
                          void* s_row, void* q_col, void* s_col, void* stream) {
  g_err.clear();
  if ((mode & (MXF_ROW | MXF_COL)) == 0 || (mode & ~(uint32_t)(MXF_ROW | MXF_COL | MXF_E5M2)))
    return fail(MXF_E_ARG, "mode = %u: must be MXF_ROW, MXF_COL or both, optionally | MXF_E5M2", mode);
  const bool e5m2 = (mode & MXF_E5M2) != 0;
  mode &= MXF_ROW | MXF_COL;
  if (rows < 0 || cols < 0) return fail(MXF_E_SHAPE, "rows = %lld, cols = %lld: negative", (long long)rows, (long long)cols);
  if (cols % 32) return fail(MXF_E_SHAPE, "cols = %lld: must be a multiple of 32", (long long)cols);
  if ((mode & MXF_COL) && rows % 32)
    return fail(MXF_E_SHAPE, "rows = %lld: must be a multiple of 32 for column-wise groups", (long long)rows);
  if ((rows + 127) / 128 > 0x7FFFFFFFLL || (cols + 127) / 128 > 65535)
    return fail(MXF_E_SHAPE, "rows = %lld, cols = %lld: too large", (long long)rows, (long long)cols);
  if (rows == 0 || cols == 0) return MXF_OK;  // nothing to read or write
  if (!x) return fail(MXF_E_NULL, "x is NULL");
  if ((mode & MXF_ROW) && (!q_row || !s_row)) return fail(MXF_E_NULL, "q_row/s_row is NULL with MXF_ROW");
  if ((mode & MXF_COL) && (!q_col || !s_col)) return fail(MXF_E_NULL, "q_col/s_col is NULL with MXF_COL");
  if (!aligned16(x)) return fail(MXF_E_ALIGN, "x is not 16-byte aligned");
  if ((mode & MXF_ROW) && !aligned16(q_row)) return fail(MXF_E_ALIGN, "q_row is not 16-byte aligned");
  if ((mode & MXF_COL) && !aligned16(q_col)) return fail(MXF_E_ALIGN, "q_col is not 16-byte aligned");
  mxf_status s = check_device();
  if (s != MXF_OK) return s;
  MXF_HIP(timed("quantize", (hipStream_t)stream, [&] {
            return mxf_launch_quantize(x, rows, cols, mode, e5m2, q_row, s_row, q_col, s_col, (hipStream_t)stream);
          }), "quantize launch");
  return MXF_OK;
}

mxf_status mxfp8_dequantize(const void* q, const void* s, int64_t rows, int64_t cols, uint32_t out_type,
                            void* out, void* stream) {
  g_err.clear();
  if (out_type & ~(uint32_t)(MXF_DEQ_F32 | MXF_DEQ_E5M2))
    return fail(MXF_E_ARG, "out_type = %u: must be MXF_DEQ_BF16 or MXF_DEQ_F32, optionally | MXF_DEQ_E5M2", out_type);
  if (rows < 0 || cols < 0) return fail(MXF_E_SHAPE, "rows = %lld, cols = %lld: negative", (long long)rows, (long long)cols);
  if (rows > ((int64_t)1 << 40) / (cols > 0 ? cols : 1))
    return fail(MXF_E_SHAPE, "rows = %lld, cols = %lld: more than 2^40 elements", (long long)rows, (long long)cols);
  if (rows == 0 || cols == 0) return MXF_OK;
  if (!q || !s || !out) return fail(MXF_E_NULL, "q, s or out is NULL");
  if (!aligned16(q)) return fail(MXF_E_ALIGN, "q is not 16-byte aligned");
  if (!aligned16(out)) return fail(MXF_E_ALIGN, "out is not 16-byte aligned");
  mxf_status st = check_device();
  if (st != MXF_OK) return st;
  MXF_HIP(timed("dequantize", (hipStream_t)stream, [&] {
            return mxf_launch_dequantize(q, s, rows, cols, (out_type & MXF_DEQ_F32) == 0, (out_type & MXF_DEQ_E5M2) != 0,
                                         out, (hipStream_t)stream);
          }), "dequantize launch");
  return MXF_OK;
}

size_t mxf_mlp_saved_bytes(const mxf_mlp_desc* desc) {
  if (check_desc(desc) != MXF_OK) return 0;
  Layout L;
  make_layout(desc, &L);
  return L.saved_total;
}

size_t mxf_mlp_workspace_bytes(const mxf_mlp_desc* desc) {
  if (check_desc(desc) != MXF_OK) return 0;
  Layout L;
  make_layout(desc, &L);
  return L.ws_total;
}

mxf_status mxf_mlp_tensor(const mxf_mlp_desc* desc, int which, int* region, size_t* offset, size_t* bytes) {
  g_err.clear();
  mxf_status s = check_desc(desc);
  if (s != MXF_OK) return s;
  if (!region || !offset || !bytes) return fail(MXF_E_NULL, "region/offset/bytes is NULL");
  if (which < 0 || which >= MXF_T_COUNT) return fail(MXF_E_ARG, "tensor id %d out of range", which);
  Layout L;
  make_layout(desc, &L);
  *region = L.region[which];
  *offset = L.off[which];
  *bytes = L.bytes[which];
  return MXF_OK;
}

static mxf_status check_mlp_ptrs(const void* const* ptrs, const char* const* names, int n) {
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) return fail(MXF_E_NULL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(MXF_E_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  return MXF_OK;
}

mxf_status grouped_mlp_fwd(const mxf_mlp_desc* desc, const int32_t* offs, const int32_t* counts,
                           const void* x, const void* w1, const void* w3, const void* w2, void* y,
                           void* saved, void* workspace, void* stream) {
  g_err.clear();
  mxf_status s = check_desc(desc);
  if (s != MXF_OK) return s;
  // with MXF_X_QUANTIZED, X's codes are already in saved / workspace and x is not read
  const bool xq = (desc->flags & MXF_X_QUANTIZED) != 0;
  const void* ptrs[] = {w1, w3, w2, y, saved, workspace, x};
  const char* names[] = {"w1", "w3", "w2", "y", "saved", "workspace", "x"};
  if ((s = check_mlp_ptrs(ptrs, names, xq ? 6 : 7)) != MXF_OK) return s;
  if ((s = check_offs_ptrs(offs, counts)) != MXF_OK) return s;
  if ((s = check_device()) != MXF_OK) return s;

  Layout L;
  make_layout(desc, &L);
  hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  uint8_t* sv = (uint8_t*)saved;
  auto T = [&](int t) -> uint8_t* { return (L.region[t] ? sv : ws) + L.off[t]; };
  const int64_t M = desc->m_capacity, D = desc->D, F = desc->F, E = desc->E;
  const bool dbg = (desc->flags & MXF_DEBUG_F32) != 0;

  // W13 (pack + dual), W2 (dual) and X (dual, unless the fused dispatch wrote its codes) in
  // one launch
  MXF_HIP(timed("quant_fwd", st, [&] {
            return mxf_launch_quant_fwd(w1, w3, w2, E, D, F, T(MXF_T_W13Q_R), T(MXF_T_W13S_R), T(MXF_T_W13Q_C),
                                        T(MXF_T_W13S_C), T(MXF_T_W2Q_R), T(MXF_T_W2S_R), T(MXF_T_W2Q_C),
                                        T(MXF_T_W2S_C), xq ? nullptr : x, M, offs, counts, desc->pad_multiple,
                                        T(MXF_T_XQ_R), T(MXF_T_XS_R), T(MXF_T_XQ_C), T(MXF_T_XS_C),
                                        (int32_t*)T(MXF_T_STATUS), st);
          }), "forward quantize launch");

  mxf::GemmParams p = {};
  p.offs = offs;
  p.counts = counts;
  p.E = (int)E;
  p.pad = desc->pad_multiple;
  p.mcap = M;
  p.M = M;
  // FC1 + SwiGLU + dual quantization of h
  // every scale tensor is in 128-k planes: row stride 4, plane stride 4 x rows
  p.A = T(MXF_T_XQ_R); p.As = T(MXF_T_XS_R); p.akp = 64 * M; p.ldas = 4; p.kbsa = 4 * M;
  p.B = T(MXF_T_W13Q_R); p.Bs = T(MXF_T_W13S_R); p.bkp = 64 * 2 * F; p.ldbs = 4; p.kbsb = 4 * 2 * F;
  p.b_es = 2 * F * D; p.bs_es = 2 * F * D / 32;
  p.N = 2 * F; p.K = D;
  p.h13 = (uint16_t*)T(MXF_T_H13);
  p.q_r = T(MXF_T_HQ_R); p.s_r = T(MXF_T_HS_R); p.q_c = T(MXF_T_HQ_C); p.s_c = T(MXF_T_HS_C);
  p.sr_rs = 4; p.sr_kbs = 4 * M; p.sc_rs = 4; p.sc_kbs = 4 * F;
  p.dbg = dbg ? (float*)T(MXF_T_H13_F32) : nullptr;
  if (desc->flags & MXF_UNFUSED) {
    // plain FC1 into the BF16 h13 (row-major), then the standalone SwiGLU + dual quantization
    mxf::GemmParams q1 = p;
    q1.C = T(MXF_T_H13); q1.ldc = 2 * F; q1.out_f32 = 0;
    MXF_HIP(timed("fc1", st, [&] { return mxf_launch_gemm_mgroup(0, q1, st); }), "FC1 launch");
    MXF_HIP(timed("swiglu_quant", st, [&] {
              return mxf_launch_swiglu_quant(T(MXF_T_H13), M, F, offs, counts, (int)E, desc->pad_multiple,
                                             T(MXF_T_HQ_R), T(MXF_T_HS_R), T(MXF_T_HQ_C), T(MXF_T_HS_C), st);
            }), "SwiGLU quantize launch");
  } else {
    MXF_HIP(timed("fc1_swiglu", st, [&] { return mxf_launch_gemm_mgroup(1, p, st); }), "FC1 launch");
  }
  // FC2
  p.A = T(MXF_T_HQ_R); p.As = T(MXF_T_HS_R); p.akp = 64 * M; p.ldas = 4; p.kbsa = 4 * M;
  p.B = T(MXF_T_W2Q_R); p.Bs = T(MXF_T_W2S_R); p.bkp = 64 * D; p.ldbs = 4; p.kbsb = 4 * D;
  p.b_es = D * F; p.bs_es = D * F / 32;
  p.N = D; p.K = F;
  p.C = y; p.ldc = D; p.out_f32 = (desc->flags & MXF_OUT_F32) ? 1 : 0;
  p.dbg = nullptr;
  MXF_HIP(timed("fc2", st, [&] { return mxf_launch_gemm_mgroup(0, p, st); }), "FC2 launch");
  return MXF_OK;
}

mxf_status grouped_mlp_bwd(const mxf_mlp_desc* desc, const int32_t* offs, const int32_t* counts,
                           const void* dy, const void* saved, void* dx, void* dw1, void* dw3, void* dw2,
                           void* workspace, void* stream) {
  g_err.clear();
  mxf_status s = check_desc(desc);
  if (s != MXF_OK) return s;
  const void* ptrs[] = {dy, saved, dx, dw1, dw3, dw2, workspace};
  const char* names[] = {"dy", "saved", "dx", "dw1", "dw3", "dw2", "workspace"};
  if ((s = check_mlp_ptrs(ptrs, names, 7)) != MXF_OK) return s;
  if ((s = check_offs_ptrs(offs, counts)) != MXF_OK) return s;
  if ((s = check_device()) != MXF_OK) return s;

  Layout L;
  make_layout(desc, &L);
  hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  uint8_t* sv = (uint8_t*)const_cast<void*>(saved);
  auto T = [&](int t) -> uint8_t* { return (L.region[t] ? sv : ws) + L.off[t]; };
  const int64_t M = desc->m_capacity, D = desc->D, F = desc->F, E = desc->E;
  const bool dbg = (desc->flags & MXF_DEBUG_F32) != 0;
  const int of32 = (desc->flags & MXF_OUT_F32) ? 1 : 0;

  MXF_HIP(timed("quant_dy", st, [&] {
            return mxf_launch_quant_tokens(dy, M, D, offs, counts, (int)E, desc->pad_multiple, T(MXF_T_DYQ_R),
                                           T(MXF_T_DYS_R), T(MXF_T_DYQ_C), T(MXF_T_DYS_C),
                                           (int32_t*)T(MXF_T_STATUS), false, st);
          }), "dY quantize launch");
  mxf::GemmParams base = {};
  base.offs = offs;
  base.counts = counts;
  base.E = (int)E;
  base.pad = desc->pad_multiple;
  base.mcap = M;
  base.out_f32 = of32;
  // After dY's quantization the backward is a small graph: FC2 wgrad needs only dY and the
  // saved h; FC1 wgrad and FC1 dgrad need dH13 from FC2 dgrad. Serial launches (the default):
  // FC2 dgrad, then the three others in one launch where all run on 256-row tiles (one kernel
  // boundary instead of three; CUs done with one GEMM's tiles start the next GEMM's), else one
  // after another. MXF_CONCURRENT: FC2 wgrad on a helper stream beside FC2 dgrad, then FC1
  // wgrad (second helper) beside FC1 dgrad (caller's stream).
  Helpers* H = nullptr;
  if ((s = get_helpers(&H, desc->flags, st)) != MXF_OK) return s;
  const bool fork = H->s[0] != st;
  // FC2 wgrad: dW2[e] = dY^T h over the expert's tokens
  mxf::GemmParams pw2 = base;
  // every scale tensor is in 128-k planes: row stride 4, plane stride 4 x rows
  pw2.A = T(MXF_T_DYQ_C); pw2.As = T(MXF_T_DYS_C); pw2.akp = 64 * D; pw2.ldas = 4; pw2.kbsa = 4 * D;
  pw2.B = T(MXF_T_HQ_C); pw2.Bs = T(MXF_T_HS_C); pw2.bkp = 64 * F; pw2.ldbs = 4; pw2.kbsb = 4 * F;
  pw2.M = D; pw2.N = F; pw2.K = M;
  pw2.C = dw2; pw2.ldc = F; pw2.c_es = D * F;
  if (fork) {
    MXF_HIP(hipEventRecord(H->fork, st), "hipEventRecord");
    MXF_HIP(hipStreamWaitEvent(H->s[0], H->fork, 0), "hipStreamWaitEvent");
    MXF_HIP(timed("fc2_wgrad", H->s[0], [&] { return mxf_launch_gemm_kgroup(0, pw2, H->s[0]); }),
            "FC2 wgrad launch");
    MXF_HIP(hipEventRecord(H->join[0], H->s[0]), "hipEventRecord");
  }
  // FC2 dgrad + dSwiGLU + dual quantization of dH13
  {
    mxf::GemmParams p = base;
    p.M = M;
    p.A = T(MXF_T_DYQ_R); p.As = T(MXF_T_DYS_R); p.akp = 64 * M; p.ldas = 4; p.kbsa = 4 * M;
    p.B = T(MXF_T_W2Q_C); p.Bs = T(MXF_T_W2S_C); p.bkp = 64 * F; p.ldbs = 4; p.kbsb = 4 * F;
    p.b_es = F * D; p.bs_es = F * D / 32;
    p.N = F; p.K = D;
    p.h13 = (uint16_t*)T(MXF_T_H13);
    p.q_r = T(MXF_T_DHQ_R); p.s_r = T(MXF_T_DHS_R); p.q_c = T(MXF_T_DHQ_C); p.s_c = T(MXF_T_DHS_C);
    p.sr_rs = 4; p.sr_kbs = 4 * M; p.sc_rs = 4; p.sc_kbs = 4 * 2 * F;
    p.dbg = dbg ? (float*)T(MXF_T_DH_F32) : nullptr;
    if (desc->flags & MXF_UNFUSED) {
      // plain FC2 dgrad into the BF16 dh, then the standalone dSwiGLU + dual quantization
      p.C = T(MXF_T_DH16); p.ldc = F; p.out_f32 = 0;
      MXF_HIP(timed("fc2_dgrad", st, [&] { return mxf_launch_gemm_mgroup(0, p, st); }), "FC2 dgrad launch");
      MXF_HIP(timed("dswiglu_quant", st, [&] {
                return mxf_launch_dswiglu_quant(T(MXF_T_DH16), T(MXF_T_H13), M, F, offs, counts, (int)E,
                                                desc->pad_multiple, T(MXF_T_DHQ_R), T(MXF_T_DHS_R), T(MXF_T_DHQ_C),
                                                T(MXF_T_DHS_C), st);
              }), "dSwiGLU quantize launch");
    } else {
      MXF_HIP(timed("fc2_dgrad_dswiglu", st, [&] { return mxf_launch_gemm_mgroup(2, p, st); }), "FC2 dgrad launch");
    }
  }
  // FC1 wgrad: dW13[e] = dH13^T X over the expert's tokens, unpacked into dW1 / dW3
  mxf::GemmParams pw1 = base;
  pw1.A = T(MXF_T_DHQ_C); pw1.As = T(MXF_T_DHS_C); pw1.akp = 64 * 2 * F; pw1.ldas = 4; pw1.kbsa = 4 * 2 * F;
  pw1.B = T(MXF_T_XQ_C); pw1.Bs = T(MXF_T_XS_C); pw1.bkp = 64 * D; pw1.ldbs = 4; pw1.kbsb = 4 * D;
  pw1.M = 2 * F; pw1.N = D; pw1.K = M;
  pw1.C = dw1; pw1.C2 = dw3; pw1.ldc = D; pw1.c_es = F * D;
  // FC1 dgrad: dX = dH13 W13
  mxf::GemmParams pd1 = base;
  pd1.M = M;
  pd1.A = T(MXF_T_DHQ_R); pd1.As = T(MXF_T_DHS_R); pd1.akp = 64 * M; pd1.ldas = 4; pd1.kbsa = 4 * M;
  pd1.B = T(MXF_T_W13Q_C); pd1.Bs = T(MXF_T_W13S_C); pd1.bkp = 64 * D; pd1.ldbs = 4; pd1.kbsb = 4 * D;
  pd1.b_es = D * 2 * F; pd1.bs_es = D * 2 * F / 32;
  pd1.N = D; pd1.K = 2 * F;
  pd1.C = dx; pd1.ldc = D;
  if (!fork && mxf_gemm_bwd3_fits(pw1, pw2, pd1)) {
    // serial launches: the three GEMMs in one launch
    MXF_HIP(timed("bwd_gemms", st, [&] { return mxf_launch_gemm_bwd3(pw1, pw2, pd1, st); }),
            "FC1 wgrad + FC2 wgrad + FC1 dgrad launch");
  } else {
    if (!fork)
      MXF_HIP(timed("fc2_wgrad", st, [&] { return mxf_launch_gemm_kgroup(0, pw2, st); }), "FC2 wgrad launch");
    if (fork) {
      MXF_HIP(hipEventRecord(H->fork, st), "hipEventRecord");
      MXF_HIP(hipStreamWaitEvent(H->s[1], H->fork, 0), "hipStreamWaitEvent");
    }
    MXF_HIP(timed("fc1_wgrad", H->s[1], [&] { return mxf_launch_gemm_kgroup(3, pw1, H->s[1]); }),
            "FC1 wgrad launch");
    if (fork) MXF_HIP(hipEventRecord(H->join[1], H->s[1]), "hipEventRecord");
    MXF_HIP(timed("fc1_dgrad", st, [&] { return mxf_launch_gemm_mgroup(0, pd1, st); }), "FC1 dgrad launch");
  }
  if (fork) {
    MXF_HIP(hipStreamWaitEvent(st, H->join[0], 0), "hipStreamWaitEvent");
    MXF_HIP(hipStreamWaitEvent(st, H->join[1], 0), "hipStreamWaitEvent");
  }
  return MXF_OK;
}

// ------------------------------------------------------------------ dispatch

static mxf_status check_plan_sizes(int64_t tokens, int32_t topk, int32_t E) {
  if (tokens < 0) return fail(MXF_E_SHAPE, "tokens = %lld: negative", (long long)tokens);
  if (topk < 1 || topk > 64) return fail(MXF_E_SHAPE, "topk = %d: must be in [1, 64]", topk);
  if (tokens * topk > ((int64_t)1 << 30))
    return fail(MXF_E_SHAPE, "tokens * topk = %lld: more than 2^30 assignments", (long long)(tokens * topk));
  if (E < 1 || E > 1024) return fail(MXF_E_SHAPE, "E = %d: must be in [1, 1024]", E);
  return MXF_OK;
}

size_t mxf_route_plan_workspace_bytes(int64_t tokens, int32_t topk, int32_t E) {
  if (check_plan_sizes(tokens, topk, E) != MXF_OK) return 0;
  return mxf_route_plan_workspace_bytes(tokens * topk, E);
}

// Host-side checks shared by the two routing-plan entry points (workspace: the caller's buffer,
// or the library's static scratch for the allocation-free variant, which passes a non-null
// placeholder here and checks the size itself).
static mxf_status check_route_plan(const int32_t* expert_idx, int64_t tokens, int32_t topk, int32_t E,
                                   int32_t pad_multiple, int64_t m_capacity, const int32_t* offs,
                                   const int32_t* counts, const int32_t* row_assign, const int32_t* assign_row,
                                   const int32_t* status, const void* workspace) {
  mxf_status s = check_plan_sizes(tokens, topk, E);
  if (s != MXF_OK) return s;
  if (pad_multiple < 1 || pad_multiple > 4096)
    return fail(MXF_E_SHAPE, "pad_multiple = %d: must be in [1, 4096]", pad_multiple);
  if (m_capacity < 0 || m_capacity > ((int64_t)1 << 30))
    return fail(MXF_E_SHAPE, "m_capacity = %lld: must be in [0, 2^30]", (long long)m_capacity);
  const int64_t n = tokens * topk;
  if (!offs || !counts) return fail(MXF_E_NULL, "offs/counts is NULL");
  if (!workspace) return fail(MXF_E_NULL, "workspace is NULL");
  if (n > 0 && (!expert_idx || !assign_row)) return fail(MXF_E_NULL, "expert_idx/assign_row is NULL");
  if (m_capacity > 0 && !row_assign) return fail(MXF_E_NULL, "row_assign is NULL");
  const void* al[] = {expert_idx, offs, counts, row_assign, assign_row, status, workspace};
  const char* an[] = {"expert_idx", "offs", "counts", "row_assign", "assign_row", "status", "workspace"};
  for (int i = 0; i < 7; ++i)
    if (!aligned4(al[i])) return fail(MXF_E_ALIGN, "%s is not 4-byte aligned", an[i]);
  return MXF_OK;
}

mxf_status mxf_route_plan(const int32_t* expert_idx, int64_t tokens, int32_t topk, int32_t E, int32_t pad_multiple,
                          int64_t m_capacity, int32_t* offs, int32_t* counts, int32_t* row_assign,
                          int32_t* assign_row, int32_t* status, void* workspace, void* stream) {
  g_err.clear();
  mxf_status s = check_route_plan(expert_idx, tokens, topk, E, pad_multiple, m_capacity, offs, counts, row_assign,
                                  assign_row, status, workspace);
  if (s != MXF_OK) return s;
  if ((s = check_device()) != MXF_OK) return s;
  MXF_HIP(timed("route_plan", (hipStream_t)stream, [&] {
            return mxf_launch_route_plan(expert_idx, (int32_t)(tokens * topk), E, pad_multiple, m_capacity, offs,
                                         counts, row_assign, assign_row, status, workspace, (hipStream_t)stream);
          }), "route plan launch");
  return MXF_OK;
}

mxf_status mxf_route_plan_noalloc(const int32_t* expert_idx, int64_t tokens, int32_t topk, int32_t E,
                                  int32_t pad_multiple, int64_t m_capacity, int32_t* offs, int32_t* counts,
                                  int32_t* row_assign, int32_t* assign_row, int32_t* status, void* stream) {
  g_err.clear();
  static const int32_t placeholder = 0;  // stands for the scratch array in the shared host checks
  mxf_status s = check_route_plan(expert_idx, tokens, topk, E, pad_multiple, m_capacity, offs, counts, row_assign,
                                  assign_row, status, &placeholder);
  if (s != MXF_OK) return s;
  const size_t need = mxf_route_plan_workspace_bytes(tokens * topk, E);
  if (need > (size_t)MXF_ROUTE_NOALLOC_MAX_BYTES)
    return fail(MXF_E_SHAPE,
                "tokens * topk = %lld with E = %d needs %zu bytes of plan scratch; the allocation-free plan holds "
                "at most %zu (use mxf_route_plan with a workspace)",
                (long long)(tokens * topk), E, need, (size_t)MXF_ROUTE_NOALLOC_MAX_BYTES);
  if ((s = check_device()) != MXF_OK) return s;
  void* ws = nullptr;
  size_t cap = 0;
  MXF_HIP(mxf_route_scratch(&ws, &cap), "route plan scratch lookup");
  if (need > cap) return fail(MXF_E_SHAPE, "plan scratch of %zu bytes exceeds the static %zu", need, cap);
  MXF_HIP(timed("route_plan", (hipStream_t)stream, [&] {
            return mxf_launch_route_plan(expert_idx, (int32_t)(tokens * topk), E, pad_multiple, m_capacity, offs,
                                         counts, row_assign, assign_row, status, ws, (hipStream_t)stream);
          }), "route plan launch");
  return MXF_OK;
}

static mxf_status check_dispatch(const void* x_tokens, int64_t tokens, int32_t topk, const int32_t* offs,
                                 const int32_t* row_assign, int64_t m_capacity) {
  if (tokens < 0) return fail(MXF_E_SHAPE, "tokens = %lld: negative", (long long)tokens);
  if (topk < 1 || topk > 64) return fail(MXF_E_SHAPE, "topk = %d: must be in [1, 64]", topk);
  if (tokens * topk > ((int64_t)1 << 30))
    return fail(MXF_E_SHAPE, "tokens * topk = %lld: more than 2^30 assignments", (long long)(tokens * topk));
  if (!offs) return fail(MXF_E_NULL, "offs is NULL");
  if (m_capacity > 0 && !row_assign) return fail(MXF_E_NULL, "row_assign is NULL");
  if (tokens > 0 && !x_tokens) return fail(MXF_E_NULL, "x_tokens is NULL");
  if (!aligned16(x_tokens)) return fail(MXF_E_ALIGN, "x_tokens is not 16-byte aligned");
  if (!aligned4(offs) || !aligned4(row_assign)) return fail(MXF_E_ALIGN, "offs/row_assign is not 4-byte aligned");
  return MXF_OK;
}

mxf_status mxf_dispatch_permute(const void* x_tokens, int64_t tokens, int32_t topk, int64_t D, int32_t E,
                                const int32_t* offs, const int32_t* row_assign, int64_t m_capacity, void* x_out,
                                void* stream) {
  g_err.clear();
  if (D < 0 || D % 8) return fail(MXF_E_SHAPE, "D = %lld: must be a non-negative multiple of 8", (long long)D);
  if (E < 1 || E > 1024) return fail(MXF_E_SHAPE, "E = %d: must be in [1, 1024]", E);
  if (m_capacity < 0 || m_capacity > ((int64_t)1 << 30))
    return fail(MXF_E_SHAPE, "m_capacity = %lld: must be in [0, 2^30]", (long long)m_capacity);
  mxf_status s = check_dispatch(x_tokens, tokens, topk, offs, row_assign, m_capacity);
  if (s != MXF_OK) return s;
  if (m_capacity > 0 && D > 0 && !x_out) return fail(MXF_E_NULL, "x_out is NULL");
  if (!aligned16(x_out)) return fail(MXF_E_ALIGN, "x_out is not 16-byte aligned");
  if (m_capacity == 0 || D == 0) return MXF_OK;
  if ((s = check_device()) != MXF_OK) return s;
  MXF_HIP(timed("permute", (hipStream_t)stream, [&] {
            return mxf_launch_permute(x_tokens, tokens * topk, topk, D, offs, E, row_assign, m_capacity, x_out,
                                      (hipStream_t)stream);
          }), "permute launch");
  return MXF_OK;
}

mxf_status mxfp8_dispatch_quantize(const mxf_mlp_desc* desc, const int32_t* offs, const int32_t* counts,
                                   const int32_t* row_assign, const void* x_tokens, int64_t tokens, int32_t topk,
                                   void* saved, void* workspace, void* stream) {
  g_err.clear();
  mxf_status s = check_desc(desc);
  if (s != MXF_OK) return s;
  if ((s = check_dispatch(x_tokens, tokens, topk, offs, row_assign, desc->m_capacity)) != MXF_OK) return s;
  if ((s = check_offs_ptrs(offs, counts)) != MXF_OK) return s;
  const void* ptrs[] = {saved, workspace};
  const char* names[] = {"saved", "workspace"};
  if ((s = check_mlp_ptrs(ptrs, names, 2)) != MXF_OK) return s;
  if ((s = check_device()) != MXF_OK) return s;
  Layout L;
  make_layout(desc, &L);
  hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  uint8_t* sv = (uint8_t*)saved;
  auto T = [&](int t) -> uint8_t* { return (L.region[t] ? sv : ws) + L.off[t]; };
  MXF_HIP(timed("dispatch_quant_x", st, [&] {
            return mxf_launch_quant_gather(x_tokens, tokens * topk, topk, row_assign, desc->m_capacity, desc->D,
                                           offs, counts, desc->E, desc->pad_multiple, T(MXF_T_XQ_R), T(MXF_T_XS_R),
                                           T(MXF_T_XQ_C), T(MXF_T_XS_C), (int32_t*)T(MXF_T_STATUS), st);
          }), "dispatch quantize launch");
  return MXF_OK;
}

mxf_status mxf_read_status(const void* workspace, void* stream, int32_t* device_status) {
  g_err.clear();
  if (!workspace || !device_status) return fail(MXF_E_NULL, "workspace/device_status is NULL");
  MXF_HIP(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize");
  MXF_HIP(hipMemcpy(device_status, workspace, sizeof(int32_t), hipMemcpyDeviceToHost), "hipMemcpy");
  return MXF_OK;
}

mxf_status mxf_profile_begin(int32_t capacity) {
  g_err.clear();
  if (capacity < 1 || capacity > (1 << 20)) return fail(MXF_E_ARG, "capacity = %d: must be in [1, 2^20]", capacity);
  Profile& P = g_prof;
  while ((int)P.ev.size() < 2 * capacity) {
    hipEvent_t e;
    MXF_HIP(hipEventCreate(&e), "hipEventCreate");
    P.ev.push_back(e);
  }
  P.name.assign(capacity, nullptr);
  P.used = 0;
  P.on = true;
  return MXF_OK;
}

mxf_status mxf_profile_end(mxf_kernel_time* out, int32_t max_out, int32_t* n_out) {
  g_err.clear();
  Profile& P = g_prof;
  if (!P.on) return fail(MXF_E_ARG, "mxf_profile_end without mxf_profile_begin on this thread");
  if (!out || !n_out) return fail(MXF_E_NULL, "out/n_out is NULL");
  P.on = false;
  int n = 0;
  for (int i = 0; i < P.used; ++i) {
    MXF_HIP(hipEventSynchronize(P.ev[2 * i + 1]), "hipEventSynchronize");
    float ms = 0.0f;
    MXF_HIP(hipEventElapsedTime(&ms, P.ev[2 * i], P.ev[2 * i + 1]), "hipEventElapsedTime");
    int k = 0;
    while (k < n && strcmp(out[k].name, P.name[i]) != 0) ++k;
    if (k == n) {
      if (n == max_out) continue;
      memset(&out[k], 0, sizeof(out[k]));
      snprintf(out[k].name, sizeof(out[k].name), "%s", P.name[i]);
      ++n;
    }
    out[k].launches += 1;
    out[k].total_ms += ms;
  }
  *n_out = n;
  P.used = 0;
  return MXF_OK;
}

static mxf_status pack_common(const void* a, const void* b, const void* c, int32_t E, int32_t F, int32_t D) {
  if (!a || !b || !c) return fail(MXF_E_NULL, "a weight pointer is NULL");
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return fail(MXF_E_ALIGN, "a weight pointer is not 16-byte aligned");
  if (E < 0 || F < 0 || D < 0 || F % 32 || D % 8)
    return fail(MXF_E_SHAPE, "E = %d, F = %d, D = %d: need F %% 32 == 0 and D %% 8 == 0", E, F, D);
  return check_device();
}

mxf_status mxf_hbm_probe(int32_t mode, const void* src, void* dst, int64_t bytes, void* stream) {
  g_err.clear();
  if (mode < 0 || mode > 2) return fail(MXF_E_ARG, "mode = %d: must be 0 (read), 1 (write) or 2 (copy)", mode);
  if (bytes <= 0 || bytes % 16 != 0 || bytes > ((int64_t)1 << 40))
    return fail(MXF_E_SHAPE, "bytes = %lld: must be a positive multiple of 16, at most 2^40", (long long)bytes);
  if ((mode != 1 && !src) || !dst) return fail(MXF_E_NULL, "src or dst is NULL");
  if ((mode != 1 && !aligned16(src)) || !aligned16(dst)) return fail(MXF_E_ALIGN, "src or dst is not 16-byte aligned");
  mxf_status st = check_device();
  if (st != MXF_OK) return st;
  int dev = 0, ncu = 0;
  MXF_HIP(hipGetDevice(&dev), "hipGetDevice");
  MXF_HIP(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev), "CU count");
  static const char* const names[3] = {"hbm_read", "hbm_write", "hbm_copy"};
  MXF_HIP(timed(names[mode], (hipStream_t)stream,
                [&] { return mxf_launch_hbm_probe(mode, src, dst, bytes, ncu, (hipStream_t)stream); }),
          "HBM probe launch");
  return MXF_OK;
}

mxf_status mxf_mfma_probe(int32_t mode, const void* src, int64_t bytes, int32_t stages, int32_t blocks, float* out,
                          void* stream) {
  g_err.clear();
  if (mode < 0 || mode > 1) return fail(MXF_E_ARG, "mode = %d: must be 0 (matrix only) or 1 (whole stage)", mode);
  if (bytes < 131072 || bytes % 32768 != 0 || bytes > ((int64_t)1 << 40))
    return fail(MXF_E_SHAPE, "bytes = %lld: must be a multiple of 32768, at least 131072, at most 2^40",
                (long long)bytes);
  if (stages <= 0 || stages % 2 != 0 || stages > (1 << 24))
    return fail(MXF_E_SHAPE, "stages = %d: must be even, positive and at most 2^24", stages);
  if (blocks <= 0 || blocks > 65535) return fail(MXF_E_SHAPE, "blocks = %d: must be in [1, 65535]", blocks);
  if (!src || !out) return fail(MXF_E_NULL, "src or out is NULL");
  if (!aligned16(src) || !aligned16(out)) return fail(MXF_E_ALIGN, "src or out is not 16-byte aligned");
  mxf_status st = check_device();
  if (st != MXF_OK) return st;
  static const char* const names[2] = {"mfma_matrix", "mfma_stage"};
  MXF_HIP(timed(names[mode], (hipStream_t)stream,
                [&] { return mxf_launch_mfma_probe(mode, src, bytes, stages, blocks, out, (hipStream_t)stream); }),
          "matrix-core probe launch");
  return MXF_OK;
}

mxf_status mxf_pack_w13(const void* w1, const void* w3, void* w13, int32_t E, int32_t F, int32_t D, void* stream) {
  g_err.clear();
  mxf_status s = pack_common(w1, w3, w13, E, F, D);
  if (s != MXF_OK) return s;
  MXF_HIP(mxf_launch_pack13(w1, w3, w13, E, F, D, true, (hipStream_t)stream), "pack launch");
  return MXF_OK;
}

mxf_status mxf_unpack_w13(const void* w13, void* w1, void* w3, int32_t E, int32_t F, int32_t D, void* stream) {
  g_err.clear();
  mxf_status s = pack_common(w1, w3, w13, E, F, D);
  if (s != MXF_OK) return s;
  MXF_HIP(mxf_launch_pack13(w1, w3, const_cast<void*>(w13), E, F, D, false, (hipStream_t)stream), "unpack launch");
  return MXF_OK;
}

}  // extern "C"
