"""Expert-major dispatch of routed tokens into the padded layout (oracle; test infrastructure).

What is computed, and where it comes from:

* torchtitan PR #12 "Wire the fully-fused grouped-GEMM MXFP8 plan behind
  fusion_plan", section "What it adds": the fully fused plan needs a token
  dispatcher whose per-expert segments are aligned to pad_multiple 256 (the
  kernels' hard per-expert alignment); torchtitan PR #2 "[mxfp8 training] fused
  gated-activation (SwiGLU) + MXFP8 quantization kernel override", section
  "Summary", swaps in the padded dispatcher with pad_multiple 128. The routed
  rows of expert e form one contiguous segment; each segment is padded with
  zero rows up to a multiple of pad_multiple.
* The MLP's first operand is then quantized in both directions (X -> dual
  MXFP8, the Q_X step of the fused forward); a fused dispatch computes the same
  codes from the token rows without storing the permuted BF16 matrix.

Readings of points the pages leave open:

* Input: expert ids [tokens, topk] (int), assignment a = t * topk + k routes
  token t's k-th choice to expert ids[t, k]. A token may name the same expert
  twice; each assignment is then its own row.
* Order inside a segment: ascending assignment index (a stable counting sort by
  expert), which makes the layout unique.
* An expert id outside [0, E) is an error: the assignment is dropped (no row),
  and the status is MXF_DEV_BAD_EXPERT (2).
* If the padded total exceeds the row capacity, offs and counts still describe
  the full layout, rows at or past the capacity are not written, their
  assignments map to -1, and the status is MXF_DEV_OVERFLOW (3) (a bad expert id
  takes precedence).
* Pad rows map to assignment -1 and read as zero. Rows at or past offs[E] are
  not part of the layout.
"""
import numpy as np

STATUS_OK, STATUS_BAD_EXPERT, STATUS_OVERFLOW = 0, 2, 3


def route_plan(expert_idx, E, pad_multiple, m_capacity):
    """Padded expert-major layout of the routed assignments.

    Returns dict(offs [E+1], counts [E], row_assign [min(offs[E], m_capacity)],
    assign_row [n], status): row_assign[r] is the assignment in row r (-1 for
    pad rows), assign_row[a] the row of assignment a (-1 if dropped or past the
    capacity).
    """
    ids = np.asarray(expert_idx, dtype=np.int64).reshape(-1)
    n = ids.size
    bad = bool(np.any((ids < 0) | (ids >= E)))
    members = [[] for _ in range(E)]          # assignments of each expert, in ascending order
    for a in range(n):
        if 0 <= ids[a] < E:
            members[ids[a]].append(a)
    counts = np.array([len(m) for m in members], dtype=np.int64)
    offs = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        seg = -(-int(counts[e]) // pad_multiple) * pad_multiple
        offs[e + 1] = offs[e] + seg
    rows = int(min(offs[E], m_capacity))
    row_assign = np.full(rows, -1, dtype=np.int64)
    assign_row = np.full(n, -1, dtype=np.int64)
    for e in range(E):
        for i, a in enumerate(members[e]):
            r = int(offs[e]) + i
            if r < m_capacity:
                row_assign[r] = a
                assign_row[a] = r
    status = STATUS_BAD_EXPERT if bad else (STATUS_OVERFLOW if offs[E] > m_capacity else STATUS_OK)
    return dict(offs=offs, counts=counts, row_assign=row_assign, assign_row=assign_row, status=status)


def permute(x_tokens, row_assign, topk, m_rows):
    """Padded expert-major matrix [m_rows, D]: row r holds the token of its assignment
    (token index = assignment // topk), pad rows are zero. Any dtype (BF16 bit patterns
    stay bit patterns); rows at or past len(row_assign) are zero here (outside the layout)."""
    x_tokens = np.asarray(x_tokens)
    out = np.zeros((m_rows, x_tokens.shape[1]), dtype=x_tokens.dtype)
    for r, a in enumerate(row_assign):
        if a >= 0:
            out[r] = x_tokens[a // topk]
    return out
