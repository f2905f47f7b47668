"""fa_fwd_splitkv_noalloc (the entry point that allocates nothing) on the GPU.

Through the C ABI: each call is compared element by element with
fa_fwd_splitkv on the same inputs and the same number of key ranges, run
with a caller-owned workspace.  Both run the same kernels on the same
partials, so the outputs must agree bitwise (which implies the bf16 bar of
2e-2 on O and 1e-3 on L, and the float32 bar of 1e-4).  Calls follow one
another on one device, so the later ones reuse the library's scratch buffer
after a larger call has left its contents there.
"""

import math
import sys

import pytest
import torch

from workloads import make_qkv

pytestmark = pytest.mark.gpu

# (B, H, N, d, dtype, causal, splits): a large call, then smaller ones.
CASES = [(2, 4, 1000, 128, torch.bfloat16, True, 4),
         (1, 2, 300, 64, torch.bfloat16, False, 3),
         (1, 1, 129, 64, torch.float32, True, 2)]
DTYPE_CODE = {torch.bfloat16: 0, torch.float32: 1}


def _run_noalloc(fa, q, k, v, S, causal):
    B, H, N, d = q.shape
    O = torch.full_like(q, float("nan"))
    L = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device)
    rc = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), O.data_ptr(),
                                   L.data_ptr(), B, H, N, d, 1.0 / math.sqrt(d),
                                   1 if causal else 0, stream.cuda_stream, DTYPE_CODE[q.dtype], S)
    assert rc == fa.FA_OK, fa.fa_strerror(rc)
    return O, L


def test_noalloc_matches_splitkv_on_consecutive_calls(gpu_lib):
    fa = gpu_lib
    dev = torch.device("cuda:0")
    for B, H, N, d, dt, causal, S in CASES:
        print(f"noalloc case B={B} H={H} N={N} d={d} {dt} causal={causal} S={S}", flush=True)
        sys.stdout.flush()
        assert fa.fa_fwd_splitkv_workspace(B, H, N, d, S) <= fa.NOALLOC_SCRATCH_BYTES
        q, k, v = (t.to(dev) for t in make_qkv(B, H, N, d, dt, seed=7))
        O, L = _run_noalloc(fa, q, k, v, S, causal)
        Oref, Lref, _ = fa.fwd_splitkv(q, k, v, S, scale=1.0 / math.sqrt(d), causal=causal)
        torch.cuda.synchronize()
        tol = 1e-4 if dt == torch.float32 else 2e-2
        assert torch.isfinite(O).all() and torch.isfinite(L).all()
        assert (O.double() - Oref.double()).abs().max().item() <= tol
        assert (L.double() - Lref.double()).abs().max().item() <= 1e-3
        assert torch.equal(O, Oref) and torch.equal(L, Lref)


def test_noalloc_rejects_more_than_its_scratch(gpu_lib):
    fa = gpu_lib
    S, d = 4, 128
    N = fa.NOALLOC_SCRATCH_BYTES // (S * (d + 1) * 4) + 1
    q = torch.zeros(1, 1, N, d, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(fa.FaError) as e:
        fa.fwd_splitkv_noalloc(q, q.clone(), q.clone(), S)
    assert e.value.status == fa.FA_ERR_SCRATCH
