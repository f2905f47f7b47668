"""The C ABI on the host (no GPU): exports and argument checks.

Every call here fails a host-side check, which the library performs before
any HIP runtime call, so nothing is launched and no device is needed.
"""

import glob
import math
import os
import re

import pytest

import io_aware_softmax_06_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa355.so is not built; run __graft_entry__.build()")
    return fa.load()


def test_header_declares_entry_points():
    assert {"fa_fwd", "fa_strerror", "fa_version"} <= set(declared_functions())


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version(lib):
    assert fa.fa_version() >= 100


def test_strerror_covers_every_code(lib):
    codes = [fa.FA_OK, fa.FA_ERR_NULL, fa.FA_ERR_SHAPE, fa.FA_ERR_UNSUPPORTED_D,
             fa.FA_ERR_DTYPE, fa.FA_ERR_SCALE, fa.FA_ERR_ALIGN, fa.FA_ERR_ALIAS,
             fa.FA_ERR_HIP, fa.FA_ERR_ARG]
    msgs = [fa.fa_strerror(c) for c in codes]
    assert len(set(msgs)) == len(codes)
    assert fa.fa_strerror(12345) == "unknown status code"


# Fake, well-separated, 256-byte aligned addresses; never dereferenced.
GB = 1 << 30
Q, K, V, O, L = 1 * GB, 3 * GB, 5 * GB, 7 * GB, 9 * GB
GOOD = dict(Q=Q, K=K, V=V, O=O, L=L, B=2, H=3, N=100, d=64, scale=0.125, causal=0,
            stream=None, dtype=fa.FA_BF16)


def call(**over):
    a = dict(GOOD, **over)
    return fa.fa_fwd(a["Q"], a["K"], a["V"], a["O"], a["L"], a["B"], a["H"], a["N"], a["d"],
                     a["scale"], a["causal"], a["stream"], a["dtype"])


@pytest.mark.parametrize("field", ["Q", "K", "V", "O", "L"])
def test_null_pointer(lib, field):
    assert call(**{field: None}) == fa.FA_ERR_NULL


@pytest.mark.parametrize("over", [dict(B=0), dict(H=0), dict(N=0), dict(N=-5), dict(B=-1),
                                  dict(N=2**31), dict(B=2**31, H=2**31)])
def test_bad_shape(lib, over):
    assert call(**over) == fa.FA_ERR_SHAPE


@pytest.mark.parametrize("d", [0, 1, 32, 63, 65, 96, 127, 129, 256])
def test_unsupported_head_dim(lib, d):
    assert call(d=d) == fa.FA_ERR_UNSUPPORTED_D


@pytest.mark.parametrize("dtype", [-1, 2, 7])
def test_bad_dtype(lib, dtype):
    assert call(dtype=dtype) == fa.FA_ERR_DTYPE


@pytest.mark.parametrize("scale", [0.0, -0.5, math.inf, -math.inf, math.nan])
def test_bad_scale(lib, scale):
    assert call(scale=scale) == fa.FA_ERR_SCALE


@pytest.mark.parametrize("causal", [-1, 2, 100])
def test_bad_causal(lib, causal):
    assert call(causal=causal) == fa.FA_ERR_ARG


@pytest.mark.parametrize("over", [dict(Q=Q + 8), dict(K=K + 2), dict(V=V + 4), dict(O=O + 1),
                                  dict(L=L + 2)])
def test_misaligned(lib, over):
    assert call(**over) == fa.FA_ERR_ALIGN


@pytest.mark.parametrize("over", [dict(O=Q), dict(O=K + 16), dict(O=V - 16), dict(L=Q + 64),
                                  dict(L=O + 1024), dict(O=L - 16)])
def test_aliasing(lib, over):
    assert call(**over) == fa.FA_ERR_ALIAS


def test_fp32_shares_the_checks(lib):
    assert call(dtype=fa.FA_F32, d=96) == fa.FA_ERR_UNSUPPORTED_D
    assert call(dtype=fa.FA_F32, O=V) == fa.FA_ERR_ALIAS
