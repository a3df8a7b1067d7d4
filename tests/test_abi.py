"""The C ABI library on the host: it loads, exports what include/lora.h
declares, and rejects every invalid argument before any HIP call.

No call here reaches a kernel launch: each one either fails validation or is
an empty-shape no-op, so these tests run without a GPU.
"""
import os
import re

import pytest

import rank_gemm_amd as rg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora.h")

# Fake, never dereferenced device addresses (16-byte aligned, far apart).
PX, PW, PA, PB, PY = (0x10000000 * (i + 1) for i in range(5))


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(lora_\w+)\s*\(", src))


def test_header_exports_match_library():
    declared = _declared()
    assert declared == set(rg.EXPORTS)
    out = os.popen(f"nm -D --defined-only {rg.LIB_PATH}").read()
    exported = set(re.findall(r"\bT\s+(lora_\w+)", out))
    assert declared <= exported, declared - exported


def test_version_and_status_strings():
    assert rg.abi_version() == 17
    for s in range(11):
        assert rg.status_str(s).startswith("LORA_")
    assert "unknown" in rg.status_str(99)


def test_variant_pick():
    assert rg.fwd_pick(rg.LORA_BF16, 1, 4096, 4096, 16) == 2
    assert rg.fwd_pick(rg.LORA_BF16, 16, 4096, 4096, 16) == 2
    assert rg.fwd_pick(rg.LORA_BF16, 17, 4096, 4096, 16) == 1      # tall tiles beyond 16 tokens
    assert rg.fwd_pick(rg.LORA_BF16, 64, 4096, 4096, 16) == 1
    assert rg.fwd_pick(rg.LORA_BF16, 65, 4096, 4096, 16) == 1
    assert rg.fwd_pick(rg.LORA_BF16, 8, 4096, 4096, 64) == 1      # rank above the decode kernel's
    assert rg.fwd_pick(rg.LORA_F32, 8, 512, 512, 16) == 1


def _fwd(**kw):
    a = dict(variant=0, dtype=rg.LORA_BF16, M=64, N=64, K=64, r=16, X=PX, ldx=64, W=PW, ldw=64,
             A=PA, lda=64, B=PB, ldb=16, scale=2.0, Y=PY, ldy=64)
    a.update(kw)
    return rg.fwd_raw(a["variant"], a["dtype"], a["M"], a["N"], a["K"], a["r"], a["X"], a["ldx"],
                      a["W"], a["ldw"], a["A"], a["lda"], a["B"], a["ldb"], a["scale"], a["Y"],
                      a["ldy"])


def _merge(**kw):
    a = dict(dtype=rg.LORA_BF16, N=64, K=64, r=16, W0=PW, ldw0=64, B=PB, ldb=16, A=PA, lda=64,
             scale=2.0, Wi=PY, ldwi=64)
    a.update(kw)
    return rg.merge_raw(a["dtype"], a["N"], a["K"], a["r"], a["W0"], a["ldw0"], a["B"], a["ldb"],
                        a["A"], a["lda"], a["scale"], a["Wi"], a["ldwi"])


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=7), rg.LORA_ERR_DTYPE),
    (dict(M=-1), rg.LORA_ERR_SHAPE),
    (dict(K=-8), rg.LORA_ERR_SHAPE),
    (dict(r=0), rg.LORA_ERR_SHAPE),
    (dict(r=257, ldb=257), rg.LORA_ERR_UNSUPPORTED),
    (dict(variant=9), rg.LORA_ERR_UNSUPPORTED),
    (dict(variant=2, M=65), rg.LORA_ERR_UNSUPPORTED),
    (dict(variant=2, dtype=rg.LORA_F32), rg.LORA_ERR_UNSUPPORTED),
    (dict(variant=2, r=33, ldb=33), rg.LORA_ERR_UNSUPPORTED),
    (dict(ldx=1 << 22), rg.LORA_ERR_UNSUPPORTED),
    (dict(ldw=1 << 22), rg.LORA_ERR_UNSUPPORTED),
    (dict(lda=1 << 22), rg.LORA_ERR_UNSUPPORTED),
    # fp32 A as one signed 32-bit byte range: r * lda * 4 > 2^31 - 1
    (dict(dtype=rg.LORA_F32, r=129, ldb=129, lda=(1 << 22) - 8), rg.LORA_ERR_UNSUPPORTED),
    (dict(dtype=rg.LORA_F32, r=256, ldb=256, lda=(1 << 21)), rg.LORA_ERR_UNSUPPORTED),
    (dict(M=1 << 30), rg.LORA_ERR_UNSUPPORTED),
    (dict(X=0), rg.LORA_ERR_NULL),
    (dict(W=0), rg.LORA_ERR_NULL),
    (dict(A=0), rg.LORA_ERR_NULL),
    (dict(B=0), rg.LORA_ERR_NULL),
    (dict(Y=0), rg.LORA_ERR_NULL),
    (dict(ldx=56), rg.LORA_ERR_STRIDE),
    (dict(ldw=8), rg.LORA_ERR_STRIDE),
    (dict(lda=63), rg.LORA_ERR_STRIDE),
    (dict(ldb=15), rg.LORA_ERR_STRIDE),
    (dict(ldy=63), rg.LORA_ERR_STRIDE),
    (dict(K=60, ldx=64, ldw=64, lda=64), rg.LORA_ERR_ALIGN),        # bf16 needs K % 8 == 0
    (dict(ldx=68), rg.LORA_ERR_ALIGN),
    (dict(X=PX + 2), rg.LORA_ERR_ALIGN),
    (dict(W=PW + 8), rg.LORA_ERR_ALIGN),
    (dict(Y=PY + 1), rg.LORA_ERR_ALIGN),
    (dict(dtype=rg.LORA_F32, K=62, ldx=64, ldw=64, lda=64), rg.LORA_ERR_ALIGN),
    (dict(Y=PX), rg.LORA_ERR_ALIAS),
    (dict(Y=PW + 64 * 63 * 2), rg.LORA_ERR_ALIAS),                 # overlaps W's last row
    (dict(Y=PB - 64 * 63 * 2), rg.LORA_ERR_ALIAS),                 # Y's tail runs into B
])
def test_fwd_rejects_before_any_hip_call(kw, want):
    assert _fwd(**kw) == want
    if kw.get("variant", 0) == 0:
        # the same arguments through the lora_fwd symbol itself
        assert _fwd_auto(**kw) == want


def _fwd_auto(**kw):
    a = dict(dtype=rg.LORA_BF16, M=64, N=64, K=64, r=16, X=PX, ldx=64, W=PW, ldw=64, A=PA,
             lda=64, B=PB, ldb=16, scale=2.0, Y=PY, ldy=64)
    a.update({k: v for k, v in kw.items() if k != "variant"})
    return rg.fwd_auto_raw(a["dtype"], a["M"], a["N"], a["K"], a["r"], a["X"], a["ldx"], a["W"],
                           a["ldw"], a["A"], a["lda"], a["B"], a["ldb"], a["scale"], a["Y"],
                           a["ldy"])


@pytest.mark.parametrize("kw", [dict(M=0), dict(N=0), dict(M=0, X=0, Y=0), dict(N=0, W=0, B=0)])
def test_fwd_empty_is_noop(kw):
    assert _fwd(**kw) == rg.LORA_OK
    assert _fwd_auto(**kw) == rg.LORA_OK


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=3), rg.LORA_ERR_DTYPE),
    (dict(N=-1), rg.LORA_ERR_SHAPE),
    (dict(r=0), rg.LORA_ERR_SHAPE),
    (dict(r=300, ldb=300), rg.LORA_ERR_UNSUPPORTED),
    (dict(W0=0), rg.LORA_ERR_NULL),
    (dict(Wi=0), rg.LORA_ERR_NULL),
    (dict(ldw0=32), rg.LORA_ERR_STRIDE),
    (dict(ldwi=32), rg.LORA_ERR_STRIDE),
    (dict(ldb=8), rg.LORA_ERR_STRIDE),
    (dict(W0=PW + 2), rg.LORA_ERR_ALIGN),
    (dict(Wi=PY + 4), rg.LORA_ERR_ALIGN),
    (dict(K=12, ldw0=64, lda=64, ldwi=64), rg.LORA_ERR_ALIGN),
    (dict(Wi=PW), rg.LORA_ERR_ALIAS),                                # in-place merge refused
    (dict(Wi=PA + 64), rg.LORA_ERR_ALIAS),
    (dict(Wi=PB - 96), rg.LORA_ERR_ALIAS),
])
def test_merge_rejects_before_any_hip_call(kw, want):
    assert _merge(**kw) == want


@pytest.mark.parametrize("kw", [dict(N=0), dict(K=0)])
def test_merge_empty_is_noop(kw):
    assert _merge(**kw) == rg.LORA_OK


def _desc(**kw):
    a = dict(N=64, K=64, r=16, W0=PW, ldw0=64, B=PB, ldb=16, A=PA, lda=64, scale=2.0, W_inf=PY,
             ldwi=64)
    a.update(kw)
    return rg.MergeDesc(a["N"], a["K"], a["r"], a["W0"], a["ldw0"], a["B"], a["ldb"], a["A"],
                        a["lda"], a["scale"], a["W_inf"], a["ldwi"])


# A second target, far from the first one's buffers.
SECOND = dict(W0=PX, B=PX + 0x100000, A=PX + 0x200000, W_inf=PX + 0x300000)


@pytest.mark.parametrize("descs,want", [
    ([_desc(r=0)], rg.LORA_ERR_SHAPE),
    ([_desc(), _desc(**SECOND, ldwi=8)], rg.LORA_ERR_STRIDE),        # second one invalid
    ([_desc(), _desc(**{**SECOND, "W0": PX + 2})], rg.LORA_ERR_ALIGN),
    ([_desc(W_inf=PW)], rg.LORA_ERR_ALIAS),                         # own input
    ([_desc(), _desc(**{**SECOND, "W0": PY})], rg.LORA_ERR_ALIAS),   # W_inf of 0 is W0 of 1
    ([_desc(), _desc(**{**SECOND, "W_inf": PY + 128})], rg.LORA_ERR_ALIAS),  # outputs overlap
    ([_desc(), _desc(**{**SECOND, "A": PY + 64})], rg.LORA_ERR_ALIAS),
])
def test_merge_batch_rejects_before_any_hip_call(descs, want):
    assert rg.merge_batch_raw(rg.LORA_BF16, descs) == want


def test_merge_batch_argument_checks():
    assert rg.merge_batch_raw(rg.LORA_BF16, []) == rg.LORA_OK
    assert rg.merge_batch_raw(5, [_desc()]) == rg.LORA_ERR_DTYPE
    L = rg.lib()
    assert L.lora_merge_batch(rg.LORA_BF16, -1, None, None) == rg.LORA_ERR_SHAPE
    assert L.lora_merge_batch(rg.LORA_BF16, 2, None, None) == rg.LORA_ERR_NULL
    # empty targets are skipped (no launch), whatever their pointers
    assert rg.merge_batch_raw(rg.LORA_BF16, [_desc(N=0, W0=0), _desc(K=0, W_inf=0)]) == rg.LORA_OK


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=3), rg.LORA_ERR_DTYPE),
    (dict(N=-1), rg.LORA_ERR_SHAPE),
    (dict(r=0), rg.LORA_ERR_SHAPE),
    (dict(W=0), rg.LORA_ERR_NULL),
    (dict(ldw=32), rg.LORA_ERR_STRIDE),
    (dict(W=PW + 2), rg.LORA_ERR_ALIGN),
    (dict(W=PA), rg.LORA_ERR_ALIAS),
    (dict(W=PB - 96), rg.LORA_ERR_ALIAS),
    (dict(N=0, W=0), rg.LORA_OK),
])
def test_merge_inplace_rejects_before_any_hip_call(kw, want):
    a = dict(dtype=rg.LORA_BF16, N=64, K=64, r=16, W=PW, ldw=64, B=PB, ldb=16, A=PA, lda=64,
             scale=2.0)
    a.update(kw)
    assert rg.merge_inplace_raw(a["dtype"], a["N"], a["K"], a["r"], a["W"], a["ldw"], a["B"],
                                a["ldb"], a["A"], a["lda"], a["scale"]) == want


def test_torch_wrapper_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    X = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rg.fwd(X, torch.zeros(8, 8, dtype=torch.bfloat16), torch.zeros(2, 8, dtype=torch.bfloat16),
               torch.zeros(8, 2, dtype=torch.bfloat16), 1.0)
    with pytest.raises(TypeError):
        rg.fwd(X.half(), torch.zeros(8, 8).half(), torch.zeros(2, 8).half(),
               torch.zeros(8, 2).half(), 1.0)


# Backward: a consistent argument set and single-field variations.  Every case
# fails validation, so nothing is launched.
PDX, PDA, PDB, PWS = (0x60000000 + 0x10000000 * i for i in range(4))


def _bwd(**kw):
    a = dict(dtype=rg.LORA_BF16, M=64, N=64, K=64, r=16, X=PX, ldx=64, W=PW, ldw=64, A=PA, lda=64,
             B=PB, ldb=16, dY=PY, lddy=64, scale=2.0, dX=PDX, lddx=64, dA=PDA, ldda=64, dB=PDB,
             lddb=16, ws=PWS, ws_bytes=1 << 24)
    a.update(kw)
    return rg.bwd_raw(a["dtype"], a["M"], a["N"], a["K"], a["r"], a["X"], a["ldx"], a["W"],
                      a["ldw"], a["A"], a["lda"], a["B"], a["ldb"], a["dY"], a["lddy"], a["scale"],
                      a["dX"], a["lddx"], a["dA"], a["ldda"], a["dB"], a["lddb"], a["ws"],
                      a["ws_bytes"])


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=rg.LORA_F32), rg.LORA_ERR_UNSUPPORTED),
    (dict(dtype=4), rg.LORA_ERR_DTYPE),
    (dict(M=-1), rg.LORA_ERR_SHAPE),
    (dict(r=0), rg.LORA_ERR_SHAPE),
    (dict(r=257, ldb=257, lddb=257), rg.LORA_ERR_UNSUPPORTED),
    (dict(M=1 << 24, r=128, ldb=128, lddb=128), rg.LORA_ERR_UNSUPPORTED),  # r * M past 2^30
    (dict(M=1 << 23, r=128, ldb=128, lddb=128), rg.LORA_ERR_UNSUPPORTED),  # exactly 2^30
    (dict(X=0), rg.LORA_ERR_NULL),
    (dict(A=0), rg.LORA_ERR_NULL),
    (dict(B=0), rg.LORA_ERR_NULL),
    (dict(dY=0), rg.LORA_ERR_NULL),
    (dict(W=0), rg.LORA_ERR_NULL),                      # W needed for dX
    (dict(dA=0), rg.LORA_ERR_NULL),
    (dict(dB=0), rg.LORA_ERR_NULL),
    (dict(ldx=56), rg.LORA_ERR_STRIDE),
    (dict(lddy=32), rg.LORA_ERR_STRIDE),
    (dict(lddx=8), rg.LORA_ERR_STRIDE),
    (dict(lddb=15), rg.LORA_ERR_STRIDE),
    (dict(ldda=63), rg.LORA_ERR_STRIDE),
    (dict(ldx=1 << 22), rg.LORA_ERR_UNSUPPORTED),
    (dict(K=60, ldx=64, ldw=64, lda=64, ldda=64, lddx=64), rg.LORA_ERR_ALIGN),   # K % 8
    (dict(N=60, lddy=64), rg.LORA_ERR_ALIGN),                                    # N % 8
    (dict(lddy=68), rg.LORA_ERR_ALIGN),
    (dict(X=PX + 2), rg.LORA_ERR_ALIGN),
    (dict(dA=PDA + 8), rg.LORA_ERR_ALIGN),
    (dict(dB=PDB + 1), rg.LORA_ERR_ALIGN),
    (dict(ws=0), rg.LORA_ERR_WORKSPACE),
    (dict(ws=PWS + 16), rg.LORA_ERR_WORKSPACE),          # not 256-B aligned
    (dict(ws_bytes=100), rg.LORA_ERR_WORKSPACE),
    (dict(dX=PX), rg.LORA_ERR_ALIAS),                    # dX over X
    (dict(dA=PA), rg.LORA_ERR_ALIAS),                    # dA over A
    (dict(dB=PDA + 64), rg.LORA_ERR_ALIAS),              # dB inside dA
    (dict(ws=PY), rg.LORA_ERR_ALIAS),                    # workspace over dY
])
def test_bwd_rejects_before_any_hip_call(kw, want):
    assert _bwd(**kw) == want


def test_bwd_workspace_size():
    assert rg.bwd_workspace_size(rg.LORA_F32, 64, 64, 64, 16) == -1
    assert rg.bwd_workspace_size(rg.LORA_BF16, 64, 64, 64, 0) == -1
    n = rg.bwd_workspace_size(rg.LORA_BF16, 4096, 1024, 1024, 16)
    assert n > 0 and n % 256 == 0
    # grows with the tokens only through T, G and the token ranges: bounded
    assert rg.bwd_workspace_size(rg.LORA_BF16, 1 << 20, 1024, 1024, 16) < (1 << 30)
    # a workspace one byte short is refused
    assert _bwd(M=4096, N=1024, K=1024, ldx=1024, ldw=1024, lda=1024, lddy=1024, lddx=1024,
                ldda=1024, ws_bytes=n - 1) == rg.LORA_ERR_WORKSPACE


@pytest.mark.parametrize("kw,want", [
    (dict(tile=20), rg.LORA_ERR_UNSUPPORTED),
    (dict(tile=19, r=32, ldb=32), rg.LORA_ERR_UNSUPPORTED),   # T-prologue 256 x 256: 32 < r
    (dict(tile=19, r=200, ldb=200), rg.LORA_ERR_UNSUPPORTED), # ... r <= 128
    (dict(tile=15, r=100, ldb=100), rg.LORA_ERR_UNSUPPORTED), # ping-pong 256 x 256: r <= 64
    (dict(tile=5), rg.LORA_ERR_UNSUPPORTED),                    # retired id
    (dict(tile=14, r=32, ldb=32), rg.LORA_ERR_UNSUPPORTED),   # T-keeping 128 x 256: 32 < r
    (dict(tile=14, r=200, ldb=200), rg.LORA_ERR_UNSUPPORTED), # ... r <= 128
    (dict(tile=10, r=100, ldb=100), rg.LORA_ERR_UNSUPPORTED),  # 64 x 64 loader tile: r <= 64
    (dict(tile=9, r=40, ldb=40), rg.LORA_ERR_UNSUPPORTED),     # 128 x 256 loader tile: r <= 32
    (dict(tile=13, r=40, ldb=40), rg.LORA_ERR_UNSUPPORTED),    # 256 x 160 loader tile: r <= 32
    (dict(tile=8, r=200, ldb=200), rg.LORA_ERR_UNSUPPORTED),   # loader tile: r <= 128
    (dict(tile=7, r=100, ldb=100), rg.LORA_ERR_UNSUPPORTED),   # k-split tile: r <= 64
    (dict(tile=6, r=200, ldb=200), rg.LORA_ERR_UNSUPPORTED),
    (dict(tile=-1), rg.LORA_ERR_UNSUPPORTED),
    (dict(tile=0, r=64, ldb=64), rg.LORA_ERR_UNSUPPORTED),     # 64 x 32 tile: r <= 32
    (dict(tile=4, r=100, ldb=100), rg.LORA_ERR_UNSUPPORTED),   # 256 x 256 tile: r <= 64
    (dict(dtype=rg.LORA_F32), rg.LORA_ERR_UNSUPPORTED),
    (dict(X=0), rg.LORA_ERR_NULL),
    (dict(ldx=56), rg.LORA_ERR_STRIDE),
    (dict(Y=PX), rg.LORA_ERR_ALIAS),
    (dict(M=0), rg.LORA_OK),
])
def test_fwd_tile_rejects_before_any_hip_call(kw, want):
    a = dict(tile=1, dtype=rg.LORA_BF16, M=64, N=64, K=64, r=16, X=PX, ldx=64, W=PW, ldw=64,
             A=PA, lda=64, B=PB, ldb=16, scale=2.0, Y=PY, ldy=64)
    a.update(kw)
    assert rg.fwd_tile_raw(a["tile"], a["dtype"], a["M"], a["N"], a["K"], a["r"], a["X"], a["ldx"],
                           a["W"], a["ldw"], a["A"], a["lda"], a["B"], a["ldb"], a["scale"],
                           a["Y"], a["ldy"]) == want


def _fdesc(**kw):
    a = dict(M=1, N=64, K=64, r=16, X=PX, ldx=64, W=PW, ldw=64, A=PA, lda=64, B=PB, ldb=16,
             scale=2.0, Y=PY, ldy=64)
    a.update(kw)
    return rg.FwdDesc(a["M"], a["N"], a["K"], a["r"], a["X"], a["ldx"], a["W"], a["ldw"], a["A"],
                      a["lda"], a["B"], a["ldb"], a["scale"], a["Y"], a["ldy"])


# A second forward sharing X (as q and k do), with its own W, A, B, Y.
SECOND_FWD = dict(W=PX + 0x100000, A=PX + 0x200000, B=PX + 0x300000, Y=PX + 0x400000)


@pytest.mark.parametrize("descs,want", [
    ([_fdesc(r=0)], rg.LORA_ERR_SHAPE),
    ([_fdesc(), _fdesc(**SECOND_FWD, ldy=8)], rg.LORA_ERR_STRIDE),
    ([_fdesc(), _fdesc(**{**SECOND_FWD, "W": PX + 0x100002})], rg.LORA_ERR_ALIGN),
    ([_fdesc(Y=PX)], rg.LORA_ERR_ALIAS),                                   # own input
    ([_fdesc(), _fdesc(**{**SECOND_FWD, "W": PY})], rg.LORA_ERR_ALIAS),    # Y of 0 is W of 1
    ([_fdesc(), _fdesc(**{**SECOND_FWD, "Y": PY + 64})], rg.LORA_ERR_ALIAS),  # outputs overlap
    ([_fdesc(), _fdesc(**{**SECOND_FWD, "X": PY})], rg.LORA_ERR_ALIAS),    # Y of 0 is X of 1
])
def test_fwd_batch_rejects_before_any_hip_call(descs, want):
    assert rg.fwd_batch_raw(rg.LORA_BF16, descs) == want


def test_fwd_batch_argument_checks():
    assert rg.fwd_batch_raw(rg.LORA_BF16, []) == rg.LORA_OK
    assert rg.fwd_batch_raw(9, [_fdesc()]) == rg.LORA_ERR_DTYPE
    L = rg.lib()
    assert L.lora_fwd_batch(rg.LORA_BF16, -1, None, None, 0, None) == rg.LORA_ERR_SHAPE
    assert L.lora_fwd_batch(rg.LORA_BF16, 3, None, None, 0, None) == rg.LORA_ERR_NULL
    n = rg.fwd_batch_workspace_size(2)
    assert n == 2 * rg.fwd_batch_workspace_size(1) > 0 and rg.fwd_batch_workspace_size(-1) == -1
    two = [_fdesc(), _fdesc(**SECOND_FWD)]
    WS = 0x70000000
    assert rg.fwd_batch_raw(rg.LORA_BF16, two, 0, WS, n - 1) == rg.LORA_ERR_WORKSPACE
    assert rg.fwd_batch_raw(rg.LORA_BF16, two, 0, WS + 16, n) == rg.LORA_ERR_WORKSPACE
    assert rg.fwd_batch_raw(rg.LORA_BF16, two, 0, PW, n) == rg.LORA_ERR_ALIAS
    # empty forwards are skipped, whatever their pointers
    assert rg.fwd_batch_raw(rg.LORA_BF16, [_fdesc(M=0, X=0, Y=0), _fdesc(N=0, W=0, B=0)]) == \
        rg.LORA_OK


def test_torch_wrapper_rejects_overlapping_rows():
    """A row stride shorter than the row (expand()ed or overlapping views)
    is refused before anything reaches the library: the kernels would
    otherwise read or write rows the tensor does not hold."""
    torch = pytest.importorskip("torch")
    row = torch.zeros(1, 64, dtype=torch.bfloat16)
    X = row.expand(32, 64)                                  # stride (0, 1)
    assert X.stride(0) == 0
    with pytest.raises(ValueError, match="row stride"):
        rg._mat(X, "X")
    flat = torch.zeros(200, dtype=torch.bfloat16)
    Y = flat.as_strided((10, 64), (8, 1))                   # rows overlap
    with pytest.raises(ValueError, match="row stride"):
        rg._mat(Y, "out")
    # one row, or rows padded past their length, are fine (then the device check)
    with pytest.raises(ValueError, match="HIP device"):
        rg._mat(row, "X")
    with pytest.raises(ValueError, match="HIP device"):
        rg._mat(flat.as_strided((2, 64), (72, 1)), "X")


def test_one_hip_runtime_per_process():
    """Loading the library before torch must not put a second HIP runtime in
    the process (torch ships its own libamdhip64 with the same soname): with
    two, the first GPU calls fail and later ones crash.  Checked in a fresh
    interpreter that loads the library first and torch afterwards."""
    import subprocess
    import sys
    code = ("import re, sys; sys.path.insert(0, %r); import rank_gemm_amd as rg; rg.lib(); "
            "import torch; maps = open('/proc/self/maps').read(); "
            "print(len(set(re.findall(r'/\\S*libamdhip64\\S*', maps))))" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1", out.stdout


def test_fwd_batch_noalloc_rejects_before_any_hip_call():
    """The no-allocation batch entry point validates like lora_fwd_batch and
    refuses more forwards than its static scratch holds."""
    d = _fdesc()
    assert rg.fwd_batch_noalloc_raw(rg.LORA_BF16, [d] * (rg.NOALLOC_MAX_FORWARDS + 1)) == \
        rg.LORA_ERR_SCRATCH
    assert rg.fwd_batch_noalloc_raw(7, [d]) == rg.LORA_ERR_DTYPE
    assert rg.fwd_batch_noalloc_raw(rg.LORA_BF16, []) == rg.LORA_OK
    assert rg.lib().lora_fwd_batch_noalloc(rg.LORA_BF16, -1, None, None) == rg.LORA_ERR_SHAPE
    assert rg.lib().lora_fwd_batch_noalloc(rg.LORA_BF16, 2, None, None) == rg.LORA_ERR_NULL
    assert rg.fwd_batch_noalloc_raw(rg.LORA_BF16, [_fdesc(r=0)]) == rg.LORA_ERR_SHAPE
    assert rg.fwd_batch_noalloc_raw(rg.LORA_BF16, [_fdesc(Y=PX)]) == rg.LORA_ERR_ALIAS
    assert rg.fwd_batch_noalloc_raw(rg.LORA_BF16, [_fdesc(M=0)]) == rg.LORA_OK


def test_ceilings_library_exports_its_header():
    """libceilings.so (the benchmark's machine-ceiling kernels, not part of
    the LoRA path) exports every function include/ceilings.h declares."""
    from rank_gemm_amd import build as b
    if not os.path.exists(b.CEIL_LIB):
        pytest.skip("libceilings.so not built")
    src = open(os.path.join(ROOT, "include", "ceilings.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    declared = set(re.findall(r"\b(ceil_\w+)\s*\(", src))
    assert {"ceil_mfma", "ceil_copy", "ceil_read"} <= declared
    out = os.popen(f"nm -D --defined-only {b.CEIL_LIB}").read()
    exported = set(re.findall(r"\bT\s+(ceil_\w+)", out))
    assert declared <= exported, declared - exported
