"""MXFP8 routed-experts SwiGLU MLP for MI355X (gfx950).

The compute lives in the HIP library ``libmxfp8.so`` (C ABI: include/mxfp8.h);
this package is its Python binding. ``MlpContext`` allocates the caller-owned
``saved`` and ``workspace`` buffers with torch and exposes the library's
documented intermediate tensors as views, for tests and inspection.
"""
from ._abi import (CAP_GFX950, COL, DEBUG_F32, DEQ_BF16, DEQ_E5M2, DEQ_F32, E5M2, DEV_BAD_EXPERT, DEV_BAD_OFFSETS, DEV_OK,
                   CONCURRENT, DEV_OVERFLOW, EXPORTS, LIB_PATH, OUT_F32, SERIAL, UNFUSED, X_QUANTIZED, dequantize,
                   mxf_dispatch_permute, mxf_route_plan, mxf_route_plan_noalloc, ROUTE_NOALLOC_MAX_BYTES, route_plan_workspace_bytes, mxfp8_dequantize, mxfp8_dispatch_quantize, route_plan,
                   ROW, T, TENSORS, MlpDesc, MxfError, abi_version, grouped_mlp_bwd, grouped_mlp_fwd,
                   last_error, lib, make_desc, mlp_saved_bytes, mlp_tensor, mlp_workspace_bytes,
                   mxfp8_quantize, pack_w13, profile_begin, profile_end, quantize, query_device,
                   read_status, unpack_w13, hbm_probe, HBM_READ, HBM_WRITE, HBM_COPY,
                   mfma_probe, MFMA_MATRIX, MFMA_STAGE)

# shapes of the documented tensors, as functions of (E, D, F, m_capacity)
_SHAPES = {
    "XQ_R": lambda E, D, F, M: (M, D), "XS_R": lambda E, D, F, M: (M, D // 32),
    "XQ_C": lambda E, D, F, M: (D, M), "XS_C": lambda E, D, F, M: (D, M // 32),
    "W13Q_R": lambda E, D, F, M: (E, 2 * F, D), "W13S_R": lambda E, D, F, M: (E, 2 * F, D // 32),
    "W13Q_C": lambda E, D, F, M: (E, D, 2 * F), "W13S_C": lambda E, D, F, M: (E, D, 2 * F // 32),
    "W2Q_R": lambda E, D, F, M: (E, D, F), "W2S_R": lambda E, D, F, M: (E, D, F // 32),
    "W2Q_C": lambda E, D, F, M: (E, F, D), "W2S_C": lambda E, D, F, M: (E, F, D // 32),
    "H13": lambda E, D, F, M: (M, 2 * F),
    "HQ_R": lambda E, D, F, M: (M, F), "HS_R": lambda E, D, F, M: (M, F // 32),
    "HQ_C": lambda E, D, F, M: (F, M), "HS_C": lambda E, D, F, M: (F, M // 32),
    "DYQ_R": lambda E, D, F, M: (M, D), "DYS_R": lambda E, D, F, M: (M, D // 32),
    "DYQ_C": lambda E, D, F, M: (D, M), "DYS_C": lambda E, D, F, M: (D, M // 32),
    "DHQ_R": lambda E, D, F, M: (M, 2 * F), "DHS_R": lambda E, D, F, M: (M, 2 * F // 32),
    "DHQ_C": lambda E, D, F, M: (2 * F, M), "DHS_C": lambda E, D, F, M: (2 * F, M // 32),
    "H13_F32": lambda E, D, F, M: (M, 2 * F), "DH_F32": lambda E, D, F, M: (M, F),
    "DH16": lambda E, D, F, M: (M, F),
    "STATUS": lambda E, D, F, M: (1,),
}


_PANEL_CODES = ("XQ_R", "XQ_C", "W13Q_R", "W13Q_C", "W2Q_R", "W2Q_C", "HQ_R", "HQ_C", "DYQ_R", "DYQ_C",
                "DHQ_R", "DHQ_C")

_PLANE_SCALES = ("XS_R", "XS_C", "W13S_R", "W13S_C", "W2S_R", "W2S_C", "HS_R", "HS_C", "DYS_R", "DYS_C",
                 "DHS_R", "DHS_C")


def scales_rowmajor(planes, shape):
    """Row-major copy [..., R, G] of a scale tensor stored in 128-k planes [..., G/4, R, 4]
    (byte of row r, group g at (g / 4) * 4R + 4r + g % 4; leading dims are experts)."""
    *lead, R, G = shape
    t = planes.reshape(*lead, G // 4, R, 4)
    n = len(lead)
    return t.permute(*range(n), n + 1, n, n + 2).reshape(*lead, R, G)


def codes_rowmajor(panels, shape):
    """Row-major copy [..., R, K] of a code tensor stored in 64-k panels [..., K/64, R, 64]
    (byte of row r, column k at (k / 64) * 64R + 64r + k % 64; leading dims are experts)."""
    *lead, R, K = shape
    t = panels.reshape(*lead, K // 64, R, 64)
    n = len(lead)
    return t.permute(*range(n), n + 1, n, n + 2).reshape(*lead, R, K)


def h13_rowmajor(tiled, F):
    """Row-major [M, 2F] copy of the fragment-tiled saved h13 (BF16, flat or any shape).

    Stored order: 4096-byte records, record (R, J) = rows 32R..32R+31 x h columns
    32J..32J+31, at record index R * (F/32) + J; inside a record, element
    (s, kh, b, c, kl, j) -- s = 0 gate / 1 up, lane c + 32b, slot 4k + j with
    k = 2 kh + kl -- is row 32R + 8k + 4b + j, packed column 64J + 32s + c.
    """
    t = tiled.reshape(-1, F // 32, 2, 2, 2, 32, 2, 4)     # R, J, s, kh, b, c, kl, j
    M = t.shape[0] * 32
    return t.permute(0, 3, 6, 4, 7, 1, 2, 5).reshape(M, 2 * F)  # R, kh, kl, b, j | J, s, c


class MlpContext:
    """Descriptor plus caller-owned device buffers for one MLP configuration."""

    def __init__(self, E, D, F, pad_multiple, m_capacity, flags=0, device="cuda"):
        import torch
        self.E, self.D, self.F, self.pad, self.m_capacity, self.flags = E, D, F, pad_multiple, m_capacity, flags
        self.desc = make_desc(E, D, F, pad_multiple, m_capacity, flags)
        self.desc_xq = make_desc(E, D, F, pad_multiple, m_capacity, flags | X_QUANTIZED)
        nsaved = mlp_saved_bytes(self.desc)
        nws = mlp_workspace_bytes(self.desc)
        if nsaved == 0 or nws == 0:
            raise MxfError(2, f"invalid descriptor E={E} D={D} F={F} pad={pad_multiple} m={m_capacity}")
        self.saved = torch.empty(nsaved, dtype=torch.uint8, device=device)
        self.workspace = torch.empty(nws, dtype=torch.uint8, device=device)

    def view_raw(self, name):
        """The bytes of documented tensor `name` inside saved / workspace (uint8, flat)."""
        region, off, nbytes = mlp_tensor(self.desc, name)
        buf = self.saved if region == 1 else self.workspace
        return buf[off:off + nbytes]

    def view(self, name):
        """A typed view of documented tensor `name` inside saved / workspace. H13 (stored
        fragment-tiled), the code tensors (stored in 64-k panels) and the scale tensors (stored
        in 128-k planes; include/mxfp8.h) are returned as row-major copies: [m_capacity, 2F]
        BF16, [..., R, K] and [..., R, K/32] bytes."""
        import torch
        raw = self.view_raw(name)
        shape = _SHAPES[name](self.E, self.D, self.F, self.m_capacity)
        if name == "H13":
            if self.flags & UNFUSED:
                return raw.view(torch.bfloat16).view(shape)
            return h13_rowmajor(raw.view(torch.bfloat16), self.F)
        if name == "DH16":
            return raw.view(torch.bfloat16).view(shape)
        if name in _PLANE_SCALES:
            return scales_rowmajor(raw, shape)
        if name in _PANEL_CODES:
            return codes_rowmajor(raw, shape)
        if name in ("H13_F32", "DH_F32"):
            return raw.view(torch.float32).view(shape)
        if name == "STATUS":
            return raw.view(torch.int32)
        return raw.view(shape)

    def fwd(self, offs, counts, x, w1, w3, w2, y, stream=None):
        """Forward; x=None means X was already quantized by dispatch_quantize (MXF_X_QUANTIZED)."""
        desc = self.desc if x is not None else self.desc_xq
        grouped_mlp_fwd(desc, offs, counts, x, w1, w3, w2, y, self.saved, self.workspace, stream)

    def dispatch_quantize(self, offs, counts, row_assign, x_tokens, topk, stream=None):
        """Fused dispatch + dual quantization of X from the token rows x_tokens [tokens, D]."""
        mxfp8_dispatch_quantize(self.desc, offs, counts, row_assign, x_tokens, x_tokens.shape[0], topk, self.saved,
                                self.workspace, stream)

    def bwd(self, offs, counts, dy, dx, dw1, dw3, dw2, stream=None):
        grouped_mlp_bwd(self.desc, offs, counts, dy, self.saved, dx, dw1, dw3, dw2, self.workspace, stream)

    def status(self, stream=None):
        return read_status(self.workspace, stream)
