"""GPU parity of the backward pass (fa_bwd) against the float64 oracle.

The GPU forward supplies O and L (as in training); fa_bwd then returns dQ,
dK, dV, compared with ``oracle.attention_backward`` on the same rounded
inputs.  Small shapes element by element (several tiles, ragged tails, both
masks, both head dimensions, both dtypes, large logits); at the full size of
the backward bench workload, two whole heads.

Tolerance (no figure is set for gradients, so it follows the arithmetic):
each of dQ, dK, dV must satisfy max |g - g_ref| <= tol * max |g_ref| with
tol = 2e-2 for bfloat16 (P and dS enter the products rounded to bf16, 2^-9
relative, and the outputs are rounded to bf16), 1e-2 for float16 (2^-11) and
tol = 1e-4 for float32.  The largest bf16 term is D = rowsum(dO o O) taken
from the forward's bf16 O: where P is peaked, dP - D cancels and carries
O's rounding into dS.  On the large-logit case it alone puts dK near 1.4e-2
(a float64 emulation of the same roundings), which the kernels match.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import make_grad, make_inputs, make_qkv, to_f64_numpy

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2, "fp16": 1e-2}
TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(fa, q, k, v, do, scale, causal):
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    O, L = fa.fwd(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = fa.bwd(qd, kd, vd, O, dod, L, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(grads, refs, dtype, where=""):
    for name, g, r in zip(("dQ", "dK", "dV"), grads, refs):
        gn = to_f64_numpy(g)
        assert np.isfinite(gn).all(), f"{where} {name} not finite"
        err = np.abs(gn - r).max()
        ref = np.abs(r).max()
        _say(f"[bwd]   {where} {name}: max err {err:.3e}, max |ref| {ref:.3e}")
        assert err <= TOL[dtype] * ref + 1e-6, f"{where} {name}: {err} > {TOL[dtype]} * {ref}"


SMALL = [
    # (B, H, N, d, dtype, causal)
    (1, 1, 1, 64, "bf16", False),
    (1, 2, 77, 128, "bf16", True),
    (1, 2, 200, 64, "bf16", False),
    (2, 2, 300, 128, "bf16", True),
    (1, 1, 513, 64, "bf16", True),
    (1, 2, 1000, 128, "bf16", False),
    (1, 1, 1, 64, "fp32", False),
    (1, 2, 100, 64, "fp32", True),
    (2, 1, 129, 128, "fp32", False),
    (1, 2, 333, 128, "fp32", True),
    (1, 2, 300, 128, "fp16", True),
    (2, 1, 513, 64, "fp16", False),
    (1, 2, 300, 32, "bf16", True),
    (2, 1, 129, 32, "bf16", False),
    (1, 2, 100, 32, "fp32", True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b{}h{}n{}d{}-{}-{}".format(
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full"))
def test_backward_small(gpu_lib, case):
    B, H, N, d, dt, causal = case
    _say(f"[bwd] small {case}")
    tdt = TORCH_DTYPE[dt]
    q, k, v = make_qkv(B, H, N, d, tdt, seed=N + d)
    do = make_grad(B, H, N, d, tdt, seed=N + d)
    scale = 1.0 / math.sqrt(d)
    grads = run(gpu_lib, q, k, v, do, scale, causal)
    refs = oracle.attention_backward(to_f64_numpy(q), to_f64_numpy(k), to_f64_numpy(v),
                                     to_f64_numpy(do), scale, causal)
    check(grads, refs, dt, str(case))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_large_logits(gpu_lib, causal):
    _say(f"[bwd] stress logits causal={causal}")
    q, k, v = make_qkv(2, 2, 333, 64, torch.bfloat16, seed=5, stress=True)
    do = make_grad(2, 2, 333, 64, torch.bfloat16, seed=5)
    grads = run(gpu_lib, q, k, v, do, 0.125, causal)
    refs = oracle.attention_backward(to_f64_numpy(q), to_f64_numpy(k), to_f64_numpy(v),
                                     to_f64_numpy(do), 0.125, causal)
    check(grads, refs, "bf16", "stress")


def test_backward_workload_two_heads(gpu_lib):
    """The bench workload at full size; two whole heads against the oracle."""
    w = workloads.BWD_CAUSAL_4K
    _say(f"[bwd] {w.describe()}")
    q, k, v = make_inputs(w, 1)
    do = make_grad(w.B, w.H, w.N, w.d, w.torch_dtype, seed=1)
    grads = run(gpu_lib, q, k, v, do, w.scale, w.causal)
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        refs = oracle.attention_backward(to_f64_numpy(q[sl]), to_f64_numpy(k[sl]),
                                         to_f64_numpy(v[sl]), to_f64_numpy(do[sl]), w.scale,
                                         w.causal)
        check(tuple(g[sl] for g in grads), refs, w.dtype, f"head ({b},{h})")


def test_backward_deterministic(gpu_lib):
    _say("[bwd] determinism")
    q, k, v = make_qkv(2, 3, 700, 128, torch.bfloat16, seed=4, device="cuda")
    do = make_grad(2, 3, 700, 128, torch.bfloat16, seed=4, device="cuda")
    O, L = gpu_lib.fwd(q, k, v, causal=True)
    g1 = gpu_lib.bwd(q, k, v, O, do, L, causal=True)
    g2 = gpu_lib.bwd(q, k, v, O, do, L, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_backward_error_status_raises(gpu_lib):
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    O, L = gpu_lib.fwd(q, q.clone(), q.clone())
    small = torch.empty(4, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu_lib.FaError) as ei:
        gpu_lib.bwd(q, q.clone(), q.clone(), O, q.clone(), L, workspace=small)
    assert ei.value.status == gpu_lib.FA_ERR_WORKSPACE
