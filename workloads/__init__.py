"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the tests, the bench and the smoke check; it holds
no arithmetic of the method (no scores, softmax or products), only the
recipes that draw Q, K and V.  Both the HIP path and the CPU oracle consume
exactly the tensors returned here.

Recipe (all workloads): a CPU ``torch.Generator`` seeded with ``seed`` draws
float32 standard normals in the order Q, K, V, each of shape [B, H, N, d];
the stress workload then draws one offset per query row.  The float32 values
are cast to the workload's dtype with round-to-nearest-even, and the oracle
upcasts those rounded values exactly to float64.

The pages benchmark on synthetic inputs only (a sweep over sequence lengths),
so no dataset is stood in for.
"""

from dataclasses import dataclass
import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "fp32", "bf16" or "fp16"
    causal: bool
    stress: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[self.dtype]

    def describe(self) -> str:
        mask = "causal" if self.causal else "non-causal"
        extra = ", stress logits" if self.stress else ""
        return (f"{self.name}: B={self.B} H={self.H} N={self.N} d={self.d} "
                f"{self.dtype} {mask}{extra}")


# The five workloads: a tiny fp32 case, multi-head bf16, causal bf16 at
# N=4096/d=128, a long sequence, and a numerical-stress case.
TINY_FP32 = Workload("tiny_fp32_b1h1n256d64", 1, 1, 256, 64, "fp32", False)
MULTIHEAD = Workload("mha_bf16_b4h16n1024d64", 4, 16, 1024, 64, "bf16", False)
CAUSAL_4K = Workload("causal_bf16_b2h32n4096d128", 2, 32, 4096, 128, "bf16", True)
LONG_16K = Workload("long_bf16_b1h16n16384d128", 1, 16, 16384, 128, "bf16", False)
STRESS = Workload("stress_bf16_b16h16n2048d64", 16, 16, 2048, 64, "bf16", False,
                  stress=True)

ALL = (TINY_FP32, MULTIHEAD, CAUSAL_4K, LONG_16K, STRESS)

# Few query tiles: 32 or 64 tiles of 256 rows cover only part of the chip's
# 256 compute units, so fa_fwd runs them as 128-row workgroups, two per CU.
LOWOCC_8K = Workload("lowocc_bf16_b1h4n8192d128", 1, 4, 8192, 128, "bf16", False)
LOWOCC_8K_CAUSAL = Workload("lowocc_causal_bf16_b1h8n8192d128", 1, 8, 8192, 128, "bf16", True)
FEW_TILES = (LOWOCC_8K, LOWOCC_8K_CAUSAL)

# Key-range split workloads: a single head at N = 16384, where even 128-row
# workgroups leave half the CUs idle (and, causal, the last query tile alone
# streams every key).  Each entry names the shape and the number of key
# ranges the split path uses.
ONEHEAD_16K = Workload("lowocc_bf16_b1h1n16384d128", 1, 1, 16384, 128, "bf16", False)
ONEHEAD_16K_CAUSAL = Workload("lowocc_causal_bf16_b1h1n16384d128", 1, 1, 16384, 128, "bf16",
                              True)
SPLIT = ((ONEHEAD_16K, 4), (ONEHEAD_16K_CAUSAL, 8))

BY_NAME = {w.name: w for w in ALL + FEW_TILES + tuple(w for w, _ in SPLIT)}
SPLITS_OF = {w.name: s for w, s in SPLIT}

# The stress workload: Q and K drawn with standard deviation 3, and a per-row
# offset c ~ U(-20, 20) added to every component of the *scaled* query, i.e.
# Q <- Q + c / scale before rounding, so that logits reach several hundred.
STRESS_SD = 3.0
STRESS_OFFSET = 20.0


def make_inputs(w: Workload, seed: int, device="cpu"):
    """(q, k, v) for workload ``w`` drawn from ``seed``, in w's dtype."""
    return make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, seed,
                    stress=w.stress, scale=w.scale, device=device)


def make_qkv(B, H, N, d, dtype, seed, stress=False, scale=None, device="cpu"):
    """Seeded Q, K, V of shape [B, H, N, d]; see the module docstring."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if stress:
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        q.mul_(STRESS_SD)
        k.mul_(STRESS_SD)
        c = torch.rand((B, H, N, 1), generator=g, dtype=torch.float32)
        c = c.mul_(2.0 * STRESS_OFFSET).sub_(STRESS_OFFSET)
        q.add_(c / scale)
    q, k, v = (t.to(dtype) for t in (q, k, v))
    if device != "cpu":
        q, k, v = (t.to(device) for t in (q, k, v))
    return q, k, v


def to_f64_numpy(t):
    """Exact float64 copy of a (CPU or device) tensor for the oracle."""
    return t.detach().to("cpu", torch.float32).double().numpy()


# ---------------------------------------------------------------------------
# Block masks for block-sparse attention (64 x 64 blocks).  Inputs only: these
# draw which blocks are on; they compute nothing of the method.

def random_block_mask(nb, density, seed, heads=None, device="cpu"):
    """uint8 [nb, nb] (or [heads, nb, nb]) with each block on with probability
    ``density``, from a seeded CPU generator."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (nb, nb) if heads is None else (heads, nb, nb)
    m = (torch.rand(shape, generator=g) < density).to(torch.uint8)
    return m.to(device)


def local_global_block_mask(nb, window, n_global, device="cpu"):
    """uint8 [nb, nb]: block (i, j) on when |i - j| <= window (a band of
    2 window + 1 blocks around the diagonal) or when i or j is one of the
    first n_global blocks (global rows and columns), the sliding-window plus
    global-token pattern of long-sequence sparse attention."""
    i = torch.arange(nb)[:, None]
    j = torch.arange(nb)[None, :]
    on = ((i - j).abs() <= window) | (i < n_global) | (j < n_global)
    return on.to(torch.uint8).to(device)


# The block-sparse workload: B=2, H=32, N=4096, d=128 (the causal workload's
# shape) with a local-global mask: a band of 3 blocks on each side of the
# diagonal and 2 global blocks, 64 x 64 blocks.
SPARSE_4K = Workload("blocksparse_bf16_b2h32n4096d128", 2, 32, 4096, 128, "bf16", False)
SPARSE_4K_WINDOW, SPARSE_4K_GLOBAL = 3, 2
BY_NAME[SPARSE_4K.name] = SPARSE_4K


# ---------------------------------------------------------------------------
# Backward pass: the output gradient dO is drawn like V (standard normal, then
# rounded to the workload's dtype) from its own seeded generator.

def make_grad(B, H, N, d, dtype, seed, device="cpu"):
    """Seeded dO of shape [B, H, N, d]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 1_000_003)
    return torch.randn((B, H, N, d), generator=g, dtype=torch.float32).to(dtype).to(device)


# The backward workload: the causal shape B=2, H=32, N=4096, d=128 in bf16.
BWD_CAUSAL_4K = Workload("bwd_causal_bf16_b2h32n4096d128", 2, 32, 4096, 128, "bf16", True)
BY_NAME[BWD_CAUSAL_4K.name] = BWD_CAUSAL_4K


# More element types and head dimensions: the causal shape in fp16, d = 32
# at B=4, H=32, N=2048, and d = 256 at B=2, H=16, N=4096.
CAUSAL_4K_FP16 = Workload("causal_fp16_b2h32n4096d128", 2, 32, 4096, 128, "fp16", True)
MHA_D32 = Workload("mha_bf16_b4h32n2048d32", 4, 32, 2048, 32, "bf16", False)
MHA_D256 = Workload("mha_bf16_b2h16n4096d256", 2, 16, 4096, 256, "bf16", False)
for _w in (CAUSAL_4K_FP16, MHA_D32, MHA_D256):
    BY_NAME[_w.name] = _w
