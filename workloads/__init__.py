"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
quantization or MLP arithmetic. Both the CPU oracle and the HIP path are fed
from here, so that they see identical inputs.

Workloads (all synthetic; no dataset is involved):

  tiny          E=4 experts, D=256, F=256. 512 tokens ~N(0,1), each routed to
                2 distinct experts chosen uniformly at random (1024 rows),
                expert-major, every segment padded to a multiple of 128.
  quant         [16384, 7168] BF16 ~N(0,1); independently per row-wise
                32-group: with p=0.01 scaled by 2^+20 or 2^-20 (coin flip),
                with p=0.001 set to zero; 0.1% of aligned 32x32 tiles zeroed
                (so column-wise all-zero groups exist too).
  dense         one expert (a dense llama-style FFN): 8192 rows, D=4096,
                F=14336.
  dsv3_rank     one expert-parallel rank of a DeepSeek-V3-16B-like MoE: 16
                local experts, D=2048, F=1408; 24576 routed rows whose counts
                follow Zipf(1.1) over 14 experts (largest-remainder rounding)
                with 2 zero-token experts; segments padded to 256.
  large_expert  8 experts, D=7168, F=2048; 32768 routed rows with counts from
                Dirichlet(alpha=0.5) (largest remainder); padded to 256.

Activations and output gradients are ~N(0,1), weights ~N(0, 0.02); float32
normals rounded to BF16. Expert counts come from numpy's default_rng(42);
values from torch generators seeded with the given seed. The per-expert counts
are regenerated here and asserted against their known lists, to catch RNG
drift.
"""
import numpy as np
import torch

MLP_CONFIGS = {
    "tiny": dict(E=4, D=256, F=256, pad=128),
    "dense": dict(E=1, D=4096, F=14336, pad=256),
    "dsv3_rank": dict(E=16, D=2048, F=1408, pad=256),
    "large_expert": dict(E=8, D=7168, F=2048, pad=256),
}
QUANT_CONFIG = dict(rows=16384, cols=7168)

KNOWN_COUNTS = {
    "tiny": [258, 248, 268, 250],
    "dense": [8192],
    "dsv3_rank": [1428, 545, 748, 1825, 666, 851, 0, 1168, 460, 2504, 3911, 8385, 986, 499, 600, 0],
    "large_expert": [7006, 11149, 77, 6582, 143, 1197, 3905, 2709],
}


def largest_remainder(weights, total):
    """Integer counts proportional to weights that sum exactly to total."""
    w = np.asarray(weights, dtype=np.float64)
    q = w / w.sum() * total
    base = np.floor(q).astype(np.int64)
    rem = int(total - base.sum())
    order = np.argsort(-(q - base), kind="stable")
    base[order[:rem]] += 1
    return base


def tiny_routing(seed=42, tokens=512, experts=4, topk=2):
    """Per-token expert choices for the tiny workload: [tokens, topk] distinct experts."""
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(experts, topk, replace=False) for _ in range(tokens)])


def expert_counts(name):
    if name == "tiny":
        choice = tiny_routing()
        counts = np.bincount(choice.ravel(), minlength=4)
    elif name == "dense":
        counts = np.array([8192])
    elif name == "dsv3_rank":
        ranks = largest_remainder(1.0 / np.arange(1, 15) ** 1.1, 24576)
        perm = np.random.default_rng(42).permutation(16)
        counts = np.zeros(16, dtype=np.int64)
        counts[perm[2:]] = ranks           # perm[0], perm[1] are the zero-token experts
    elif name == "large_expert":
        rng = np.random.default_rng(42)
        counts = largest_remainder(rng.dirichlet(np.full(8, 0.5)), 32768)
    else:
        raise KeyError(name)
    counts = [int(c) for c in counts]
    assert counts == KNOWN_COUNTS[name], (name, counts)
    return counts


def padded_offsets(counts, pad):
    """offs[e+1] - offs[e] = counts[e] rounded up to a multiple of pad."""
    offs = [0]
    for c in counts:
        offs.append(offs[-1] + (int(c) + pad - 1) // pad * pad)
    return offs


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn_bf16(shape, std, gen, device):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t = t * std
    return t.to(torch.bfloat16)


def mlp_problem(name="tiny", seed=42, device="cpu", m_capacity=None, pad_fill=0.0, tail_fill=0.0,
                counts=None, E=None, D=None, F=None, pad=None):
    """Inputs for one routed-experts MLP call.

    Returns a dict: x [m_capacity, D] bf16, w1/w3 [E, F, D] bf16, w2 [E, D, F]
    bf16, dy [m_capacity, D] bf16, offs (list, E+1), counts (list, E), E, D, F,
    pad, m_capacity. Real rows ~N(0,1); pad rows hold pad_fill and rows past
    offs[E] hold tail_fill (NaN fills build the poisoned-pad controls).
    A custom shape is built when counts/E/D/F/pad are given.
    """
    if counts is None:
        cfg = MLP_CONFIGS[name]
        E, D, F, pad = cfg["E"], cfg["D"], cfg["F"], cfg["pad"]
        counts = expert_counts(name)
    offs = padded_offsets(counts, pad)
    m = offs[-1]
    mcap = m if m_capacity is None else int(m_capacity)
    assert mcap >= m
    gen = _gen(seed, device)
    x = torch.full((mcap, D), tail_fill, dtype=torch.bfloat16, device=device)
    dy = torch.full((mcap, D), tail_fill, dtype=torch.bfloat16, device=device)
    if name == "tiny" and counts == KNOWN_COUNTS["tiny"]:
        # each token row appears once in every expert it was routed to
        choice = tiny_routing()
        tok = randn_bf16((choice.shape[0], D), 1.0, gen, device)  # same draw as routed_tokens("tiny")
        for e in range(E):
            ids = torch.from_numpy(np.nonzero((choice == e).any(axis=1))[0]).to(device)
            x[offs[e]:offs[e] + counts[e]] = tok[ids]
    else:
        for e in range(E):
            if counts[e]:
                x[offs[e]:offs[e] + counts[e]] = randn_bf16((counts[e], D), 1.0, gen, device)
    w1 = randn_bf16((E, F, D), 0.02, gen, device)
    w3 = randn_bf16((E, F, D), 0.02, gen, device)
    w2 = randn_bf16((E, D, F), 0.02, gen, device)
    for e in range(E):
        if counts[e]:
            dy[offs[e]:offs[e] + counts[e]] = randn_bf16((counts[e], D), 1.0, gen, device)
        x[offs[e] + counts[e]:offs[e + 1]] = pad_fill
        dy[offs[e] + counts[e]:offs[e + 1]] = pad_fill
    return dict(x=x, w1=w1, w3=w3, w2=w2, dy=dy, offs=offs, counts=list(counts), E=E, D=D, F=F,
                pad=pad, m_capacity=mcap)


DISPATCH_TOPK = {"tiny": 2, "dense": 1, "dsv3_rank": 6, "large_expert": 8}


def routed_tokens(name="tiny", seed=42, device="cpu"):
    """Token rows and their expert choices before dispatch: (x_tokens [T, D] bf16,
    expert_idx [T, topk] int32 numpy).

    tiny: the 512 tokens and top-2 choices that mlp_problem("tiny") lays out (same
    generator draw). Other workloads: T = routed rows / topk tokens ~N(0,1), the expert ids
    a seeded random permutation of each expert repeated counts[e] times (so a token may
    name an expert twice), reshaped [T, topk].
    """
    cfg = MLP_CONFIGS[name]
    counts = expert_counts(name)
    topk = DISPATCH_TOPK[name]
    if name == "tiny":
        idx = tiny_routing().astype(np.int32)
    else:
        flat = np.repeat(np.arange(cfg["E"], dtype=np.int32), counts)
        assert flat.size % topk == 0
        idx = np.random.default_rng(seed).permutation(flat).reshape(-1, topk)
    gen = _gen(seed, device)
    x = randn_bf16((idx.shape[0], cfg["D"]), 1.0, gen, device)
    return x, idx


def quant_matrix(rows=QUANT_CONFIG["rows"], cols=QUANT_CONFIG["cols"], seed=42, device="cpu"):
    """The standalone-quantizer workload: BF16 [rows, cols] with scaled and zeroed groups."""
    assert rows % 32 == 0 and cols % 32 == 0
    gen = _gen(seed, device)
    a = torch.randn((rows, cols), generator=gen, device=device, dtype=torch.float32)
    nb = cols // 32
    u = torch.rand((rows, nb), generator=gen, device=device)
    coin = torch.rand((rows, nb), generator=gen, device=device) < 0.5
    z = torch.rand((rows, nb), generator=gen, device=device) < 0.001
    factor = torch.ones((rows, nb), device=device)
    factor[(u < 0.01) & coin] = 2.0 ** 20
    factor[(u < 0.01) & ~coin] = 2.0 ** -20
    factor[z] = 0.0
    a = (a.view(rows, nb, 32) * factor[:, :, None]).view(rows, cols)
    tz = torch.rand((rows // 32, nb), generator=gen, device=device) < 0.001
    a = (a.view(rows // 32, 32, nb, 32) * (~tz).float()[:, None, :, None]).view(rows, cols)
    return a.to(torch.bfloat16)


def bf16_bits(t):
    """uint16 numpy view of a CPU bf16 tensor's bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
