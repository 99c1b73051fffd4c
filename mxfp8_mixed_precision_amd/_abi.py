"""ctypes binding of libmxfp8.so (the C ABI declared in include/mxfp8.h).

Argument marshalling only: every step of the computation runs in the HIP
library. Torch tensors are accepted for convenience (their device pointers and
the current HIP stream are passed through); torch is used for device memory and
streams, nothing else. If the library is missing or cannot be loaded, every call
raises -- there is no fallback path.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmxfp8.so")

ABI_VERSION = 1

# status codes
OK, E_NULL, E_SHAPE, E_ALIGN, E_DEVICE, E_ARG, E_HIP = range(7)
STATUS_NAMES = {OK: "MXF_OK", E_NULL: "MXF_E_NULL", E_SHAPE: "MXF_E_SHAPE", E_ALIGN: "MXF_E_ALIGN",
                E_DEVICE: "MXF_E_DEVICE", E_ARG: "MXF_E_ARG", E_HIP: "MXF_E_HIP"}
DEV_OK, DEV_BAD_OFFSETS, DEV_BAD_EXPERT, DEV_OVERFLOW = 0, 1, 2, 3
CAP_GFX950 = 1
ROW, COL, E5M2 = 1, 2, 4
OUT_F32, DEBUG_F32, SERIAL, UNFUSED, X_QUANTIZED, CONCURRENT = 1, 2, 4, 8, 16, 32
DEQ_BF16, DEQ_F32, DEQ_E5M2 = 0, 1, 2

# tensor ids (mxf_tensor)
TENSORS = ["STATUS", "XQ_R", "XS_R", "XQ_C", "XS_C", "W13Q_R", "W13S_R", "W13Q_C", "W13S_C",
           "W2Q_R", "W2S_R", "W2Q_C", "W2S_C", "H13", "HQ_R", "HS_R", "HQ_C", "HS_C",
           "DYQ_R", "DYS_R", "DYQ_C", "DYS_C", "DHQ_R", "DHS_R", "DHQ_C", "DHS_C",
           "H13_F32", "DH_F32", "DH16"]
T = {name: i for i, name in enumerate(TENSORS)}

EXPORTS = ["mxf_abi_version", "mxf_query_device", "mxf_last_error", "mxfp8_quantize", "mxfp8_dequantize",
           "mxf_mlp_saved_bytes", "mxf_mlp_workspace_bytes", "mxf_mlp_tensor", "grouped_mlp_fwd",
           "grouped_mlp_bwd", "mxf_read_status", "mxf_profile_begin", "mxf_profile_end",
           "mxf_pack_w13", "mxf_unpack_w13", "mxf_route_plan_workspace_bytes", "mxf_route_plan", "mxf_route_plan_noalloc",
           "mxf_dispatch_permute",
           "mxfp8_dispatch_quantize", "mxf_hbm_probe", "mxf_mfma_probe"]


class MxfError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


class MlpDesc(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("D", ctypes.c_int32), ("F", ctypes.c_int32),
                ("pad_multiple", ctypes.c_int32), ("m_capacity", ctypes.c_int64),
                ("flags", ctypes.c_uint32)]


_lib = None


def lib():
    """Load libmxfp8.so (once). Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m mxfp8_mixed_precision_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
        sz = ctypes.c_size_t
        pdesc = ctypes.POINTER(MlpDesc)
        sig = {
            "mxf_abi_version": (ctypes.c_int, []),
            "mxf_query_device": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(u32)]),
            "mxf_last_error": (ctypes.c_char_p, []),
            "mxfp8_quantize": (ctypes.c_int, [vp, i64, i64, u32, vp, vp, vp, vp, vp]),
            "mxfp8_dequantize": (ctypes.c_int, [vp, vp, i64, i64, u32, vp, vp]),
            "mxf_mlp_saved_bytes": (sz, [pdesc]),
            "mxf_mlp_workspace_bytes": (sz, [pdesc]),
            "mxf_mlp_tensor": (ctypes.c_int, [pdesc, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                              ctypes.POINTER(sz), ctypes.POINTER(sz)]),
            "grouped_mlp_fwd": (ctypes.c_int, [pdesc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "grouped_mlp_bwd": (ctypes.c_int, [pdesc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "mxf_read_status": (ctypes.c_int, [vp, vp, ctypes.POINTER(i32)]),
            "mxf_profile_begin": (ctypes.c_int, [i32]),
            "mxf_profile_end": (ctypes.c_int, [ctypes.POINTER(KernelTime), i32, ctypes.POINTER(i32)]),
            "mxf_pack_w13": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp]),
            "mxf_unpack_w13": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp]),
            "mxf_route_plan_workspace_bytes": (sz, [i64, i32, i32]),
            "mxf_route_plan": (ctypes.c_int, [vp, i64, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp]),
            "mxf_route_plan_noalloc": (ctypes.c_int, [vp, i64, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp]),
            "mxf_dispatch_permute": (ctypes.c_int, [vp, i64, i32, i64, i32, vp, vp, i64, vp, vp]),
            "mxfp8_dispatch_quantize": (ctypes.c_int, [pdesc, vp, vp, vp, vp, i64, i32, vp, vp, vp]),
            "mxf_hbm_probe": (ctypes.c_int, [i32, vp, vp, i64, vp]),
            "mxf_mfma_probe": (ctypes.c_int, [i32, vp, i64, i32, i32, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.mxf_abi_version() != ABI_VERSION:
            raise RuntimeError(f"libmxfp8.so ABI version {L.mxf_abi_version()} != {ABI_VERSION}")
        _lib = L
    return _lib


def last_error():
    return lib().mxf_last_error().decode()


def _check(status):
    if status != OK:
        raise MxfError(status, last_error())


def _ptr(t):
    """Device pointer of a tensor (or None / int passed through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ entry points

def abi_version():
    return lib().mxf_abi_version()


def query_device(device=0):
    caps = ctypes.c_uint32(0)
    _check(lib().mxf_query_device(device, ctypes.byref(caps)))
    return caps.value


def mxfp8_quantize(x, rows, cols, mode, q_row=None, s_row=None, q_col=None, s_col=None, stream=None):
    """Raw call: pointers (tensors or ints) and sizes, as in the C header."""
    _check(lib().mxfp8_quantize(_ptr(x), rows, cols, mode, _ptr(q_row), _ptr(s_row), _ptr(q_col),
                                _ptr(s_col), _stream(stream)))


def quantize(x, mode=ROW | COL, stream=None):
    """Quantize a 2-D BF16 CUDA tensor (mode may include E5M2); allocates and returns
    (q_row, s_row, q_col, s_col)."""
    import torch
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()
    rows, cols = x.shape
    dev = x.device
    q_row = s_row = q_col = s_col = None
    if mode & ROW:
        q_row = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        s_row = torch.empty((rows, max(cols // 32, 0)), dtype=torch.uint8, device=dev)
    if mode & COL:
        q_col = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
        s_col = torch.empty((cols, max(rows // 32, 0)), dtype=torch.uint8, device=dev)
    mxfp8_quantize(x, rows, cols, mode, q_row, s_row, q_col, s_col, stream)
    return q_row, s_row, q_col, s_col


def mxfp8_dequantize(q, s, rows, cols, out_type, out, stream=None):
    """Raw call: pointers (tensors or ints) and sizes, as in the C header."""
    _check(lib().mxfp8_dequantize(_ptr(q), _ptr(s), rows, cols, out_type, _ptr(out), _stream(stream)))


def dequantize(q, s, out_dtype=None, e5m2=False, stream=None):
    """Decode row-wise MXFP8 codes q [rows, cols] u8 (E4M3, or E5M2 with e5m2=True) with
    scales s [rows, ceil(cols/32)] u8 (CUDA tensors); allocates and returns a BF16 (default)
    or FP32 tensor."""
    import torch
    out_dtype = out_dtype or torch.bfloat16
    assert q.dtype == torch.uint8 and q.dim() == 2 and q.is_contiguous()
    rows, cols = q.shape
    assert s.dtype == torch.uint8 and s.is_contiguous() and tuple(s.shape) == (rows, -(-cols // 32))
    out = torch.empty((rows, cols), dtype=out_dtype, device=q.device)
    kind = (DEQ_BF16 if out_dtype == torch.bfloat16 else DEQ_F32) | (DEQ_E5M2 if e5m2 else 0)
    mxfp8_dequantize(q, s, rows, cols, kind, out, stream)
    return out


def make_desc(E, D, F, pad_multiple, m_capacity, flags=0):
    return MlpDesc(E, D, F, pad_multiple, m_capacity, flags)


def mlp_saved_bytes(desc):
    return lib().mxf_mlp_saved_bytes(ctypes.byref(desc))


def mlp_workspace_bytes(desc):
    return lib().mxf_mlp_workspace_bytes(ctypes.byref(desc))


def mlp_tensor(desc, which):
    """(region, offset, bytes) of tensor `which` (name or id): region 0 workspace, 1 saved."""
    if isinstance(which, str):
        which = T[which]
    region, off, nb = ctypes.c_int(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().mxf_mlp_tensor(ctypes.byref(desc), which, ctypes.byref(region), ctypes.byref(off),
                                ctypes.byref(nb)))
    return region.value, off.value, nb.value


def grouped_mlp_fwd(desc, offs, counts, x, w1, w3, w2, y, saved, workspace, stream=None):
    _check(lib().grouped_mlp_fwd(ctypes.byref(desc), _ptr(offs), _ptr(counts), _ptr(x), _ptr(w1),
                                 _ptr(w3), _ptr(w2), _ptr(y), _ptr(saved), _ptr(workspace),
                                 _stream(stream)))


def grouped_mlp_bwd(desc, offs, counts, dy, saved, dx, dw1, dw3, dw2, workspace, stream=None):
    _check(lib().grouped_mlp_bwd(ctypes.byref(desc), _ptr(offs), _ptr(counts), _ptr(dy), _ptr(saved),
                                 _ptr(dx), _ptr(dw1), _ptr(dw3), _ptr(dw2), _ptr(workspace),
                                 _stream(stream)))


def route_plan_workspace_bytes(tokens, topk, E):
    return lib().mxf_route_plan_workspace_bytes(tokens, topk, E)


def mxf_route_plan(expert_idx, tokens, topk, E, pad_multiple, m_capacity, offs, counts, row_assign, assign_row,
                   status, workspace, stream=None):
    """Raw call: pointers (tensors or ints) and sizes, as in the C header."""
    _check(lib().mxf_route_plan(_ptr(expert_idx), tokens, topk, E, pad_multiple, m_capacity, _ptr(offs),
                                _ptr(counts), _ptr(row_assign), _ptr(assign_row), _ptr(status), _ptr(workspace),
                                _stream(stream)))


ROUTE_NOALLOC_MAX_BYTES = 8 << 20


def mxf_route_plan_noalloc(expert_idx, tokens, topk, E, pad_multiple, m_capacity, offs, counts, row_assign,
                           assign_row, status, stream=None):
    """Raw call of the allocation-free routing plan (no workspace argument)."""
    _check(lib().mxf_route_plan_noalloc(_ptr(expert_idx), tokens, topk, E, pad_multiple, m_capacity, _ptr(offs),
                                        _ptr(counts), _ptr(row_assign), _ptr(assign_row), _ptr(status),
                                        _stream(stream)))


def route_plan(expert_idx, E, pad_multiple, m_capacity, stream=None):
    """Routing plan of expert ids [tokens, topk] (int32 CUDA tensor); allocates and returns
    dict(offs, counts, row_assign, assign_row, status) as int32 CUDA tensors."""
    import torch
    assert expert_idx.dtype == torch.int32 and expert_idx.dim() == 2 and expert_idx.is_contiguous()
    tokens, topk = expert_idx.shape
    dev = expert_idx.device
    out = {"offs": torch.empty(E + 1, dtype=torch.int32, device=dev),
           "counts": torch.empty(E, dtype=torch.int32, device=dev),
           "row_assign": torch.empty(max(m_capacity, 1), dtype=torch.int32, device=dev),
           "assign_row": torch.empty(max(tokens * topk, 1), dtype=torch.int32, device=dev),
           "status": torch.empty(1, dtype=torch.int32, device=dev)}
    ws = torch.empty(route_plan_workspace_bytes(tokens, topk, E), dtype=torch.uint8, device=dev)
    mxf_route_plan(expert_idx, tokens, topk, E, pad_multiple, m_capacity, out["offs"], out["counts"],
                   out["row_assign"], out["assign_row"], out["status"], ws, stream)
    out["row_assign"] = out["row_assign"][:m_capacity]
    out["assign_row"] = out["assign_row"][:tokens * topk]
    return out


def mxf_dispatch_permute(x_tokens, tokens, topk, D, E, offs, row_assign, m_capacity, x_out, stream=None):
    """Raw call: pointers (tensors or ints) and sizes, as in the C header."""
    _check(lib().mxf_dispatch_permute(_ptr(x_tokens), tokens, topk, D, E, _ptr(offs), _ptr(row_assign), m_capacity,
                                      _ptr(x_out), _stream(stream)))


def mxfp8_dispatch_quantize(desc, offs, counts, row_assign, x_tokens, tokens, topk, saved, workspace, stream=None):
    """Raw call: pointers (tensors or ints) and sizes, as in the C header."""
    _check(lib().mxfp8_dispatch_quantize(ctypes.byref(desc), _ptr(offs), _ptr(counts), _ptr(row_assign),
                                         _ptr(x_tokens), tokens, topk, _ptr(saved), _ptr(workspace),
                                         _stream(stream)))


def read_status(workspace, stream=None):
    st = ctypes.c_int32(-1)
    _check(lib().mxf_read_status(_ptr(workspace), _stream(stream), ctypes.byref(st)))
    return st.value


def pack_w13(w1, w3, w13, E, F, D, stream=None):
    _check(lib().mxf_pack_w13(_ptr(w1), _ptr(w3), _ptr(w13), E, F, D, _stream(stream)))


def unpack_w13(w13, w1, w3, E, F, D, stream=None):
    _check(lib().mxf_unpack_w13(_ptr(w13), _ptr(w1), _ptr(w3), E, F, D, _stream(stream)))


HBM_READ, HBM_WRITE, HBM_COPY = 0, 1, 2


def hbm_probe(mode, src, dst, nbytes, stream=None):
    """HBM ceiling kernel (see mxf_hbm_probe): mode HBM_READ, HBM_WRITE or HBM_COPY."""
    _check(lib().mxf_hbm_probe(mode, _ptr(src) if src is not None else None, _ptr(dst), nbytes, _stream(stream)))


MFMA_MATRIX, MFMA_STAGE = 0, 1


def mfma_probe(mode, src, nbytes, stages, blocks, out, stream=None):
    """Matrix-core ceiling kernel (see mxf_mfma_probe): mode MFMA_MATRIX or MFMA_STAGE."""
    _check(lib().mxf_mfma_probe(mode, _ptr(src), nbytes, stages, blocks, _ptr(out), _stream(stream)))


def profile_begin(capacity=4096):
    """Start per-kernel event timing on this thread (see mxf_profile_begin)."""
    _check(lib().mxf_profile_begin(capacity))


def profile_end():
    """Stop timing; returns {kernel name: (launches, total_ms)}."""
    buf = (KernelTime * 64)()
    n = ctypes.c_int32(0)
    _check(lib().mxf_profile_end(buf, 64, ctypes.byref(n)))
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(n.value)}
