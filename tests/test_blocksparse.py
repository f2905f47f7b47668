"""GPU parity of the block-sparse forward (fa_fwd_blocksparse) against the oracle.

The oracle is ``oracle.attention_block_sparse`` (hidden scores are -inf before
the softmax; a row with no visible key has O = 0, L = -inf), element by element
on small shapes that span several tiles and ragged tails, and
``oracle.attention_block_sparse_rows`` on sampled rows at the full size of the
block-sparse bench workload.  Masks come from ``workloads``: seeded random
masks of several densities (with empty block rows forced in), the local-global
band, all-ones and all-zeros, shared by all heads, per head and per (batch,
head).

Tolerances: those of the dense path (O <= 1e-4 for float32, <= 2e-2 for
bfloat16, L <= 1e-3, max-abs); rows with no visible key must be exactly
O = 0, L = -inf.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import make_inputs, make_qkv, to_f64_numpy

pytestmark = pytest.mark.gpu

TOL_O = {"fp32": 1e-4, "bf16": 2e-2, "fp16": 5e-3}
TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}
TOL_L = 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _mask(kind, nb, B, H, seed):
    if kind == "ones":
        return torch.ones((nb, nb), dtype=torch.uint8)
    if kind == "zeros":
        return torch.zeros((nb, nb), dtype=torch.uint8)
    if kind == "local":
        return workloads.local_global_block_mask(nb, 1, 1)
    density = float(kind[1:]) / 10  # "r3" -> 0.3
    m = workloads.random_block_mask(nb, density, seed, heads=H)
    m[0, min(1, nb - 1), :] = 0  # head 0: an empty block row
    return m if H > 1 else m[0]


def compare(O, L, q, k, v, scale, causal, mask, dtype):
    Or, Lr = oracle.attention_block_sparse(to_f64_numpy(q), to_f64_numpy(k), to_f64_numpy(v),
                                           scale, causal, mask.numpy())
    Og = to_f64_numpy(O)
    Lg = L.cpu().double().numpy()
    dead = np.isneginf(Lr)
    assert np.array_equal(np.isneginf(Lg), dead), "rows with no visible key differ"
    assert np.all(Og[dead] == 0), "a row with no visible key has O != 0"
    assert np.isfinite(Og).all()
    eo = np.abs(Og - Or).max()
    el = np.abs(np.where(dead, 0.0, Lg - np.where(dead, 0.0, Lr))).max()
    assert eo <= TOL_O[dtype], f"max |O - O_ref| = {eo}"
    assert el <= TOL_L, f"max |L - L_ref| = {el}"
    return eo, el


SMALL = [
    # (B, H, N, d, dtype, causal, mask kind)
    (1, 1, 1, 64, "bf16", False, "ones"),
    (1, 2, 200, 64, "bf16", False, "r5"),
    (1, 2, 300, 128, "bf16", True, "r5"),
    (2, 2, 513, 128, "bf16", False, "r3"),
    (1, 3, 1000, 64, "bf16", True, "r7"),
    (1, 2, 1024, 128, "bf16", False, "local"),
    (1, 2, 777, 128, "bf16", True, "local"),
    (1, 1, 640, 64, "bf16", False, "zeros"),
    (1, 2, 2048, 128, "bf16", True, "r1"),
    (1, 1, 100, 64, "fp32", False, "r5"),
    (1, 2, 333, 128, "fp32", True, "r5"),
    (2, 1, 300, 64, "fp32", False, "local"),
    (1, 2, 700, 128, "fp16", True, "r5"),
    (1, 1, 1024, 64, "fp16", False, "local"),
    (1, 2, 777, 32, "bf16", True, "r5"),
    (1, 1, 200, 32, "fp32", False, "r5"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b{}h{}n{}d{}-{}-{}-{}".format(
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full", c[6]))
def test_blocksparse_small(gpu_lib, case):
    B, H, N, d, dt, causal, kind = case
    _say(f"[sparse] small {case}")
    nb = -(-N // 64)
    q, k, v = make_qkv(B, H, N, d, TORCH_DTYPE[dt], seed=N + d)
    mask = _mask(kind, nb, B, H, seed=N)
    scale = 1.0 / math.sqrt(d)
    O, L = gpu_lib.fwd_blocksparse(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), scale=scale,
                                   causal=causal)
    torch.cuda.synchronize()
    compare(O, L, q, k, v, scale, causal, mask, dt)


@pytest.mark.parametrize("layout", ["shared", "per_head", "per_batch_head"])
def test_blocksparse_mask_layouts(gpu_lib, layout):
    _say(f"[sparse] mask layout {layout}")
    B, H, N, d = 2, 3, 450, 64
    nb = -(-N // 64)
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=31)
    if layout == "shared":
        mask = workloads.random_block_mask(nb, 0.5, 1)
    elif layout == "per_head":
        mask = workloads.random_block_mask(nb, 0.5, 2, heads=H)
    else:
        mask = workloads.random_block_mask(nb, 0.5, 3, heads=B * H).view(B, H, nb, nb)
    O, L = gpu_lib.fwd_blocksparse(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), causal=True)
    torch.cuda.synchronize()
    compare(O, L, q, k, v, 1 / math.sqrt(d), True, mask, "bf16")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_equals_dense(gpu_lib, dt, causal):
    """Every block on: the same tiles in the same order as fa_fwd, bit for bit."""
    _say(f"[sparse] all-ones vs dense {dt} causal={causal}")
    B, H, N, d = 2, 2, 700, 128
    q, k, v = make_qkv(B, H, N, d, dt, seed=13, device="cuda")
    ones = torch.ones((-(-N // 64),) * 2, dtype=torch.uint8, device="cuda")
    O1, L1 = gpu_lib.fwd(q, k, v, causal=causal)
    O2, L2 = gpu_lib.fwd_blocksparse(q, k, v, ones, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_blocksparse_workload(gpu_lib):
    """The bench workload at full size, sampled rows against the oracle."""
    w = workloads.SPARSE_4K
    _say(f"[sparse] {w.describe()} local-global mask")
    q, k, v = make_inputs(w, 1)
    nb = w.N // 64
    mask = workloads.local_global_block_mask(nb, workloads.SPARSE_4K_WINDOW,
                                             workloads.SPARSE_4K_GLOBAL)
    O, L = gpu_lib.fwd_blocksparse(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), scale=w.scale,
                                   causal=w.causal)
    torch.cuda.synchronize()
    assert torch.isfinite(O.float()).all() and torch.isfinite(L).all()
    rng = np.random.default_rng(1)
    rows = []
    for b in range(w.B):
        for h in range(w.H):
            picks = {0, 63, 64, 127, 128, 1000, w.N - 1}
            picks |= set(int(i) for i in rng.integers(0, w.N, size=6))
            rows += [(b, h, i) for i in sorted(picks)]
    idx = torch.tensor(rows, dtype=torch.long)
    Og = O[idx[:, 0], idx[:, 1], idx[:, 2]].double().cpu().numpy()
    Lg = L[idx[:, 0], idx[:, 1], idx[:, 2]].double().cpu().numpy()
    Or, Lr = oracle.attention_block_sparse_rows(to_f64_numpy(q), to_f64_numpy(k),
                                                to_f64_numpy(v), w.scale, w.causal,
                                                mask.numpy(), rows)
    eo, el = np.abs(Og - Or).max(), np.abs(Lg - Lr).max()
    _say(f"[sparse]   rows={len(rows)} max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= TOL_O["bf16"] and el <= TOL_L


def test_blocksparse_deterministic_and_guarded(gpu_lib):
    _say("[sparse] determinism and guard bands")
    B, H, N, d = 2, 3, 333, 64
    nb = -(-N // 64)
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=6, device="cuda")
    mask = workloads.random_block_mask(nb, 0.4, 9, heads=H).cuda()
    n_o, n_l, pad = B * H * N * d, B * H * N, 4096
    o_buf = torch.full((n_o + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((n_l + 2 * pad,), float("nan"), dtype=torch.float32, device="cuda")
    O = o_buf[pad:pad + n_o].view(B, H, N, d)
    L = l_buf[pad:pad + n_l].view(B, H, N)
    gpu_lib.fwd_blocksparse(q, k, v, mask, causal=True, out=O, lse=L)
    O2, L2 = gpu_lib.fwd_blocksparse(q, k, v, mask, causal=True)
    torch.cuda.synchronize()
    assert torch.isnan(o_buf[:pad].float()).all() and torch.isnan(o_buf[-pad:].float()).all()
    assert torch.isnan(l_buf[:pad]).all() and torch.isnan(l_buf[-pad:]).all()
    assert not torch.isnan(O.float()).any() and not torch.isnan(L).any()
    assert torch.equal(O, O2) and torch.equal(L, L2)


def test_blocksparse_error_status_raises(gpu_lib):
    q = torch.zeros((1, 2, 100, 64), dtype=torch.bfloat16, device="cuda")
    bad = torch.ones((3, 3), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        gpu_lib.fwd_blocksparse(q, q.clone(), q.clone(), bad)
