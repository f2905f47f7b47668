"""GPU parity of the key-range split forward (fa_fwd_splitkv) and its merge.

Through the C ABI against the float64 CPU oracle:
  * the merged O and L against ``oracle.attention`` (element by element on
    small shapes; sampled rows via ``oracle.attention_rows`` at full size);
  * every partial O_s, L_s left in the workspace against
    ``oracle.attention_partial`` over the same key range, so that the split
    kernel and the merge kernel are each pinned on their own;
  * empty ranges (more ranges than key tiles, causal ranges past the
    diagonal), ragged tails, both dtypes and both head dimensions.

Tolerances are those of the unsplit path: O <= 1e-4 (float32 inputs) or
<= 2e-2 (bfloat16), L <= 1e-3, all max-abs.  Partials O_s are float32 in
both cases and carry the same bound.
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


def block_ranges(N, S, causal):
    """Key ranges of the documented split, per 256-row block of queries.

    Returns a list over blocks rb of (row_lo, row_hi, [(kv_lo, kv_hi)] * S):
    the keys visible to the block (all N, or causal: the first
    min(N, 256 (rb + 1))) cut on 64-key boundaries into S ranges.
    """
    out = []
    for r0 in range(0, N, 256):
        visible = min(N, r0 + 256) if causal else N
        T = (visible + 63) // 64
        rng = [((s * T // S) * 64, min(visible, ((s + 1) * T // S) * 64)) for s in range(S)]
        out.append((r0, min(N, r0 + 256), rng))
    return out


def check_partials(fa, ws, S, q, k, v, scale, causal, dtype):
    B, H, N, d = q.shape
    Os, Ls = fa.split_partials(ws, S, B, H, N, d)
    Os = Os.double().cpu().numpy()
    Ls = Ls.double().cpu().numpy()
    qn, kn, vn = to_f64_numpy(q), to_f64_numpy(k), to_f64_numpy(v)
    for r0, r1, ranges in block_ranges(N, S, causal):
        for s, (lo, hi) in enumerate(ranges):
            m, l, acc = oracle.attention_partial(qn, kn, vn, scale, causal, lo, hi)
            m, l, acc = m[:, :, r0:r1], l[:, :, r0:r1], acc[:, :, r0:r1]
            live = l > 0
            O_ref = np.where(live[..., None], acc / np.where(live, l, 1.0)[..., None], 0.0)
            L_ref = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
            Og, Lg = Os[s][:, :, r0:r1], Ls[s][:, :, r0:r1]
            where = f"rows [{r0},{r1}) range {s} keys [{lo},{hi})"
            assert np.array_equal(np.isneginf(Lg), ~live), f"{where}: empty rows differ"
            assert np.isfinite(Og).all()
            eo = np.abs(Og - O_ref).max()
            el = np.abs(np.where(live, Lg, 0.0) - np.where(live, L_ref, 0.0)).max()
            assert eo <= TOL_O[dtype], f"{where}: max |O_s - ref| = {eo}"
            assert el <= TOL_L, f"{where}: max |L_s - ref| = {el}"


SMALL = [
    # (B, H, N, d, dtype, causal, splits)
    (1, 1, 1, 64, "bf16", False, 1),
    (1, 1, 1, 128, "bf16", True, 3),      # more ranges than key tiles
    (1, 2, 300, 64, "bf16", True, 2),
    (2, 1, 640, 128, "bf16", False, 3),
    (1, 1, 1000, 128, "bf16", True, 5),
    (1, 2, 257, 64, "bf16", False, 8),    # ragged tail, empty ranges
    (1, 1, 129, 128, "bf16", True, 4),
    (1, 3, 2048, 64, "bf16", True, 16),   # many causal ranges past the diagonal
    (1, 1, 100, 64, "fp32", False, 2),
    (1, 2, 333, 128, "fp32", True, 3),
    (1, 1, 65, 64, "fp32", False, 5),
    (2, 1, 700, 64, "fp32", True, 7),
    (1, 2, 513, 128, "fp16", True, 3),
    (2, 1, 300, 64, "fp16", False, 4),
    (1, 2, 700, 32, "bf16", True, 3),
    (1, 1, 300, 32, "fp32", False, 2),
    (1, 2, 600, 256, "bf16", True, 3),
    (1, 1, 200, 256, "fp32", False, 2),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b{}h{}n{}d{}-{}-{}-s{}".format(
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full", c[6]))
def test_split_small(gpu_lib, case):
    B, H, N, d, dt, causal, S = case
    _say(f"[splitkv] small {case}")
    q, k, v = make_qkv(B, H, N, d, TORCH_DTYPE[dt], seed=N + d + S)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    O, L, ws = gpu_lib.fwd_splitkv(qd, kd, vd, S, scale=scale, causal=causal)
    torch.cuda.synchronize()
    Or, Lr = oracle.attention(to_f64_numpy(q), to_f64_numpy(k), to_f64_numpy(v), scale, causal)
    eo = np.abs(to_f64_numpy(O) - Or).max()
    el = np.abs(L.cpu().double().numpy() - Lr).max()
    assert torch.isfinite(O.float()).all() and torch.isfinite(L).all()
    assert eo <= TOL_O[dt], f"max |O - O_ref| = {eo}"
    assert el <= TOL_L, f"max |L - L_ref| = {el}"
    check_partials(gpu_lib, ws, S, q, k, v, scale, causal, dt)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [False, True])
def test_one_split_equals_fwd(gpu_lib, dt, causal):
    """With one range the merge weight is exactly 1: the result is fa_fwd's, bit for bit."""
    _say(f"[splitkv] S=1 vs fwd {dt} causal={causal}")
    q, k, v = make_qkv(2, 2, 513, 128, dt, seed=12, device="cuda")
    O1, L1 = gpu_lib.fwd(q, k, v, causal=causal)
    O2, L2, _ = gpu_lib.fwd_splitkv(q, k, v, 1, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_stress_logits_split(gpu_lib):
    """Ranges whose maxima differ by hundreds: the merge weights underflow safely."""
    _say("[splitkv] stress logits")
    q, k, v = make_qkv(2, 2, 777, 64, torch.bfloat16, seed=5, stress=True)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    O, L, ws = gpu_lib.fwd_splitkv(qd, kd, vd, 6, scale=0.125, causal=False)
    torch.cuda.synchronize()
    Or, Lr = oracle.attention(to_f64_numpy(q), to_f64_numpy(k), to_f64_numpy(v), 0.125, False)
    assert np.abs(to_f64_numpy(O) - Or).max() <= TOL_O["bf16"]
    assert np.abs(L.cpu().double().numpy() - Lr).max() <= TOL_L
    check_partials(gpu_lib, ws, 6, q, k, v, 0.125, False, "bf16")


def _sampled_check(fa, w, S, seed):
    q, k, v = make_inputs(w, seed)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    O, L, _ = fa.fwd_splitkv(qd, kd, vd, S, scale=w.scale, causal=w.causal)
    O_ref_gpu, L_ref_gpu = fa.fwd(qd, kd, vd, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    assert torch.isfinite(O.float()).all() and torch.isfinite(L).all()
    # Against the unsplit kernel on every row (both within the oracle's bound).
    assert (O.float() - O_ref_gpu.float()).abs().max().item() <= 2 * TOL_O[w.dtype]
    assert (L - L_ref_gpu).abs().max().item() <= 2 * TOL_L
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(w.B):
        for h in range(w.H):
            picks = {0, 63, 64, 255, 256, w.N // 2, w.N - 1}
            picks |= set(int(i) for i in rng.integers(0, w.N, size=24))
            rows += [(b, h, i) for i in sorted(picks) if i < w.N]
    idx = torch.tensor(rows, dtype=torch.long)
    Og = O[idx[:, 0], idx[:, 1], idx[:, 2]].double().cpu().numpy()
    Lg = L[idx[:, 0], idx[:, 1], idx[:, 2]].double().cpu().numpy()
    Or, Lr = oracle.attention_rows(to_f64_numpy(q), to_f64_numpy(k), to_f64_numpy(v),
                                   w.scale, w.causal, rows)
    eo, el = np.abs(Og - Or).max(), np.abs(Lg - Lr).max()
    _say(f"[splitkv]   rows={len(rows)} max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= TOL_O[w.dtype]
    assert el <= TOL_L


@pytest.mark.parametrize("ws", workloads.SPLIT, ids=lambda x: f"{x[0].name}-s{x[1]}")
def test_split_workload(gpu_lib, ws):
    w, S = ws
    _say(f"[splitkv] {w.describe()} splits={S}")
    _sampled_check(gpu_lib, w, S, seed=1)


def test_split_large_logits_every_row(gpu_lib):
    """The large-logits workload through four key ranges, every row against the
    oracle: each range's partial output is normalised by the sum of its own
    rounded probabilities and the merge weighs the ranges by their float32 L_s,
    which must keep the rows dominated by one key inside the bound."""
    w, S = workloads.STRESS, 4
    _say(f"[splitkv] every row: {w.describe()} splits={S}")
    q, k, v = workloads.make_inputs(w, 1)
    O, L, _ = gpu_lib.fwd_splitkv(q.cuda(), k.cuda(), v.cuda(), S, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    Og, Lg = to_f64_numpy(O), L.cpu().double().numpy()
    qn, kn, vn = to_f64_numpy(q), to_f64_numpy(k), to_f64_numpy(v)
    eo = el = 0.0
    for b in range(w.B):
        Or, Lr = oracle.attention(qn[b:b + 1], kn[b:b + 1], vn[b:b + 1], w.scale, w.causal)
        eo = max(eo, float(np.abs(Og[b:b + 1] - Or).max()))
        el = max(el, float(np.abs(Lg[b:b + 1] - Lr).max()))
    _say(f"[splitkv]   all {w.B * w.H * w.N} rows: max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= TOL_O[w.dtype]
    assert el <= TOL_L


def test_split_long_sequence_eight_ranges(gpu_lib):
    """N = 16384 cut into 8 key ranges (one GPU's share of an 8-way key split)."""
    w = workloads.LONG_16K
    _say(f"[splitkv] {w.describe()} splits=8")
    _sampled_check(gpu_lib, w, 8, seed=2)


def test_workspace_reuse_and_coverage(gpu_lib):
    """Every partial is written (no stale values), nothing past the workspace size is.

    Two calls share one NaN-filled workspace, the second with a smaller shape.
    """
    _say("[splitkv] workspace reuse")
    big = (2, 2, 700, 128, 5)
    small = (1, 3, 190, 64, 3)
    need_big = gpu_lib.fa_fwd_splitkv_workspace(*big)
    pad = 1 << 16
    buf = torch.full((need_big + pad,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN bytes
    ws = buf[:need_big]
    for (B, H, N, d, S), causal in ((big, True), (small, False)):
        q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=B + H + N, device="cuda")
        O, L, _ = gpu_lib.fwd_splitkv(q, k, v, S, causal=causal, workspace=ws)
        Or, Lr = gpu_lib.fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        need = gpu_lib.fa_fwd_splitkv_workspace(B, H, N, d, S)
        f = ws[:need].view(torch.float32)
        assert not torch.isnan(f).any(), "a partial was left unwritten"
        assert (O.float() - Or.float()).abs().max().item() <= 2 * TOL_O["bf16"]
        assert (L - Lr).abs().max().item() <= 2 * TOL_L
    assert (buf[need_big:] == 0xFF).all(), "write past the workspace"


def test_split_deterministic(gpu_lib):
    _say("[splitkv] determinism")
    q, k, v = make_qkv(1, 4, 1500, 128, torch.bfloat16, seed=4, device="cuda")
    O1, L1, _ = gpu_lib.fwd_splitkv(q, k, v, 6, causal=True)
    O2, L2, _ = gpu_lib.fwd_splitkv(q, k, v, 6, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_split_guard_bands(gpu_lib):
    """Writes stay inside O and L, and every element of both is written."""
    _say("[splitkv] guard bands")
    B, H, N, d, S = 2, 3, 201, 64, 4
    for dt in (torch.bfloat16, torch.float32):
        q, k, v = make_qkv(B, H, N, d, dt, seed=6, device="cuda")
        n_o, n_l, pad = B * H * N * d, B * H * N, 4096
        o_buf = torch.full((n_o + 2 * pad,), float("nan"), dtype=dt, device="cuda")
        l_buf = torch.full((n_l + 2 * pad,), float("nan"), dtype=torch.float32, device="cuda")
        O = o_buf[pad:pad + n_o].view(B, H, N, d)
        L = l_buf[pad:pad + n_l].view(B, H, N)
        gpu_lib.fwd_splitkv(q, k, v, S, causal=True, out=O, lse=L)
        torch.cuda.synchronize()
        assert torch.isnan(o_buf[:pad].float()).all() and torch.isnan(o_buf[-pad:].float()).all()
        assert torch.isnan(l_buf[:pad]).all() and torch.isnan(l_buf[-pad:]).all()
        assert torch.isfinite(O.float()).all() and torch.isfinite(L).all()


def test_split_error_status_raises(gpu_lib):
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.FaError) as ei:
        gpu_lib.fwd_splitkv(q, q.clone(), q.clone(), 0)
    assert ei.value.status == gpu_lib.FA_ERR_SPLITS
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu_lib.FaError) as ei:
        gpu_lib.fwd_splitkv(q, q.clone(), q.clone(), 2, workspace=small)
    assert ei.value.status == gpu_lib.FA_ERR_WORKSPACE
