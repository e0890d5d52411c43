"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/kata.h, and rejects bad arguments before launching."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "kata.h")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
FAKE = 0x10000            # aligned, never dereferenced: every call below fails first
MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def L():
    from kernelized_linear_attention_phi_amd import lib
    return lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kata_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"kata_chunked_fwd", "kata_scan_states", "kata_decode_step"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in kata.h but not exported"
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_helpers(L):
    assert L.kata_phi_dim(16) == 136 and L.kata_phi_dim(32) == 528 and L.kata_phi_dim(-1) == -1
    for s, txt in [(0, b"ok"), (1, b"invalid argument"), (2, b"unsupported shape"),
                   (3, b"workspace too small"), (4, b"HIP launch error")]:
        assert L.kata_status_string(s) == txt
    assert re.fullmatch(rb"\d+\.\d+\.\d+", L.kata_version())


def fwd(L, B=1, H=1, T=64, dk=16, dv=64, C=64, causal=1, dtype=BF16, q=FAKE, S0=None, z0=None,
        S_out=None, z_out=None, ws=FAKE, ws_bytes=1 << 40, o=FAKE):
    return L.kata_chunked_fwd(q, FAKE, FAKE, o, B, H, T, dk, dv, C, causal, dtype, S0, z0,
                              S_out, z_out, ws, ws_bytes, None)


def test_fwd_rejects_before_launch(L):
    assert fwd(L, dk=24) == EUNSUPPORTED
    assert fwd(L, dv=48) == EUNSUPPORTED
    assert fwd(L, C=48) == EUNSUPPORTED
    assert fwd(L, C=0) == EINVAL
    assert fwd(L, T=-1) == EINVAL
    assert fwd(L, B=-2) == EINVAL
    assert fwd(L, dtype=7) == EINVAL
    assert fwd(L, q=None) == EINVAL
    assert fwd(L, q=MISALIGNED) == EINVAL
    assert fwd(L, S0=FAKE) == EINVAL              # S0 without z0
    assert fwd(L, S_out=FAKE) == EINVAL           # S_out without z_out
    assert fwd(L, ws_bytes=16) == EWORKSPACE
    assert fwd(L, ws=None) == EWORKSPACE
    # empty problems launch nothing
    assert fwd(L, T=0, q=None, o=None, ws=None, ws_bytes=0) == OK
    assert fwd(L, B=0, q=None, o=None, ws=None, ws_bytes=0) == OK


PSD, IDENTITY = 0, 1
SCAN, SEQUENTIAL = 0, 1


def fwd_ex(L, feature=IDENTITY, prefix=SCAN, B=1, H=1, T=64, dk=16, dv=64, C=64, causal=1,
           dtype=BF16, q=FAKE, ws=FAKE, ws_bytes=1 << 40, o=FAKE, S0=None, z0=None, G=0):
    return L.kata_chunked_fwd_ex(q, FAKE, FAKE, o, B, H, T, dk, dv, C, causal, dtype, feature,
                                 prefix, G, S0, z0, None, None, ws, ws_bytes, None)


def test_fwd_ex_rejects_before_launch(L):
    assert fwd_ex(L, feature=2) == EINVAL
    assert fwd_ex(L, prefix=5) == EINVAL
    # identity feature: fp32 inputs and chunk 16 take the VALU path, scan prefix only
    assert fwd_ex(L, dtype=F32, prefix=SEQUENTIAL) == EUNSUPPORTED
    assert fwd_ex(L, C=16, prefix=SEQUENTIAL) == EUNSUPPORTED
    assert fwd_ex(L, dtype=F32, ws_bytes=16) == EWORKSPACE
    assert fwd_ex(L, dk=24) == EUNSUPPORTED
    assert fwd_ex(L, feature=PSD, prefix=SEQUENTIAL, dtype=F32) == EUNSUPPORTED
    assert fwd_ex(L, feature=PSD, prefix=SEQUENTIAL, C=128) == EUNSUPPORTED   # d_k=16: C 32 or 64
    assert fwd_ex(L, prefix=SEQUENTIAL, ws_bytes=16) == EWORKSPACE
    assert fwd_ex(L, q=MISALIGNED) == EINVAL
    assert fwd_ex(L, S0=FAKE) == EINVAL
    assert fwd_ex(L, T=0, q=None, o=None, ws=None, ws_bytes=0) == OK           # empty: no launch
    assert fwd_ex(L, feature=PSD, prefix=SEQUENTIAL, B=0, q=None, o=None, ws=None, ws_bytes=0) == OK
    assert fwd_ex(L, feature=PSD, G=-1) == EINVAL                                # segment length


def test_segment_chunks_sets_the_plan(L):
    """G chunks per segment is an explicit argument (0 = automatic): it sets
    the number of segment records, so the workspace follows it."""
    ws = L.kata_chunked_fwd_ex_workspace
    rec16 = 9 * 4 * 256 + 256
    auto = ws(1, 8, 131072, 16, 64, 64, BF16, 1, PSD, SCAN, 0)
    assert auto == L.kata_chunked_fwd_workspace(1, 8, 131072, 16, 64, 64, BF16, 1)
    assert auto == ws(1, 8, 131072, 16, 64, 64, BF16, 1, PSD, SCAN, 16)     # automatic G = 16
    # G = 4: 512 segments per head, plus the initial and the final record
    assert ws(1, 8, 131072, 16, 64, 64, BF16, 1, PSD, SCAN, 4) == (512 + 2) * 8 * rec16 * 4
    assert ws(1, 8, 131072, 16, 64, 64, BF16, 1, PSD, SCAN, -1) == 0
    wsx = L.kata_chunked_fwd_decay_ex_workspace
    assert wsx(1, 8, 131072, 16, 64, 64, BF16, PSD, SCAN, 4) > wsx(1, 8, 131072, 16, 64, 64, BF16, PSD, SCAN, 0)
    assert wsx(1, 8, 131072, 16, 64, 64, BF16, PSD, SCAN, -2) == 0


def test_feature_dim_and_ex_workspace(L):
    assert L.kata_feature_dim(16, PSD) == 136 and L.kata_feature_dim(32, PSD) == 528
    assert L.kata_feature_dim(16, IDENTITY) == 16 and L.kata_feature_dim(32, IDENTITY) == 32
    assert L.kata_feature_dim(16, 7) == -1 and L.kata_feature_dim(-1, PSD) == -1
    ws = L.kata_chunked_fwd_ex_workspace
    # PSD with the scan: the same plan as kata_chunked_fwd
    assert ws(1, 8, 131072, 16, 64, 64, BF16, 1, PSD, SCAN, 0) == \
        L.kata_chunked_fwd_workspace(1, 8, 131072, 16, 64, 64, BF16, 1)
    # sequential: one record per head for the segment, the initial and the final state
    rec16 = 9 * 4 * 256 + 256            # d_k = 16, d_v = 64: nine feature tiles + Gram tile
    assert ws(1, 8, 131072, 16, 64, 64, BF16, 1, PSD, SEQUENTIAL, 0) == 3 * 8 * rec16 * 4
    rec1 = 1 * 5 * 256                   # identity, d_k = 16, d_v = 64: four value tiles + z
    assert ws(1, 8, 131072, 16, 64, 64, BF16, 1, IDENTITY, SEQUENTIAL, 0) == 3 * 8 * rec1 * 4
    assert ws(1, 8, 131072, 16, 64, 64, BF16, 1, IDENTITY, SCAN, 0) > 3 * 8 * rec1 * 4
    # identity on the VALU path: one S record (d_k x d_v) and one z record per chunk
    assert ws(1, 1, 64, 16, 64, 64, F32, 1, IDENTITY, SCAN, 0) == 16 * 64 * 4 + 256
    assert ws(1, 1, 64, 16, 64, 64, F32, 1, IDENTITY, SEQUENTIAL, 0) == 0
    assert ws(1, 1, 64, 16, 64, 64, BF16, 1, 9, SCAN, 0) == 0


def fwd_decay(L, B=1, H=2, T=64, dk=16, dv=64, C=64, dtype=BF16, prefix=SCAN, g=FAKE, q=FAKE,
              ws=FAKE, ws_bytes=1 << 40, o=FAKE):
    return L.kata_chunked_fwd_decay(q, FAKE, FAKE, g, o, B, H, T, dk, dv, C, dtype, prefix,
                                    None, None, None, None, ws, ws_bytes, None)


def test_decay_rejects_before_launch(L):
    assert fwd_decay(L, g=None) == EINVAL
    assert fwd_decay(L, g=MISALIGNED) == EINVAL
    assert fwd_decay(L, prefix=4) == EINVAL
    # shapes without a matrix-core path take the VALU path, scan prefix only
    assert fwd_decay(L, dtype=F32, prefix=SEQUENTIAL) == EUNSUPPORTED
    assert fwd_decay(L, dk=32, C=32, prefix=SEQUENTIAL) == EUNSUPPORTED
    assert fwd_decay(L, C=128, prefix=SEQUENTIAL) == EUNSUPPORTED
    assert fwd_decay(L, dtype=F32, ws_bytes=16) == EWORKSPACE
    assert fwd_decay(L, dk=12) == EUNSUPPORTED
    # several heads with T % 4 != 0: the VALU path, scan prefix only
    assert fwd_decay(L, T=66, prefix=SEQUENTIAL) == EUNSUPPORTED
    assert fwd_decay(L, dk=32, C=128, T=66, prefix=SEQUENTIAL) == EUNSUPPORTED
    assert fwd_decay(L, ws_bytes=16) == EWORKSPACE
    assert fwd_decay(L, T=0, q=None, o=None, g=None, ws=None, ws_bytes=0) == OK   # empty
    ws = L.kata_chunked_fwd_decay_workspace
    assert ws(1, 8, 131072, 16, 64, 64, BF16, SCAN) > ws(1, 8, 131072, 16, 64, 64, BF16, SEQUENTIAL) > 0
    # VALU path: per-chunk S and z records and one decay factor per chunk
    nrec = 8 * 128
    assert ws(1, 8, 4096, 32, 64, 32, BF16, SCAN) == nrec * 528 * 64 * 4 + nrec * 528 * 4 + nrec * 4
    assert ws(1, 8, 4096, 32, 64, 32, BF16, SEQUENTIAL) == 0
    # d_k = 32 on the matrix cores: segment records, initial and final state
    rec32 = 33 * 4 * 256 + 4 * 256
    assert ws(1, 8, 4096, 32, 64, 128, BF16, SEQUENTIAL) == 3 * 8 * rec32 * 4
    assert ws(1, 8, 4096, 32, 64, 128, BF16, SCAN) > 3 * 8 * rec32 * 4
    assert ws(2, 4, 4098, 32, 64, 128, BF16, SEQUENTIAL) == 0      # T % 4 != 0, several heads
    assert ws(1, 8, 4096, 16, 64, 64, F32, SCAN) == 8 * 64 * (136 * 64 * 4 + 136 * 4 + 4)
    dex = L.kata_chunked_fwd_decay_ex
    dex_args = lambda f, pf, wsb, dt=BF16, T=64, C=64: (FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, T, 16, 64, C,
                                                         dt, f, pf, 0, None, None, None, None, FAKE, wsb,
                                                         None)
    # identity: matrix cores for bf16 with chunk 32 or 64, else VALU with the scan only
    assert dex(*dex_args(IDENTITY, SEQUENTIAL, 1 << 40, dt=F32)) == EUNSUPPORTED
    assert dex(*dex_args(IDENTITY, SEQUENTIAL, 1 << 40, C=128)) == EUNSUPPORTED
    assert dex(*dex_args(IDENTITY, SEQUENTIAL, 1 << 40, T=66)) == EUNSUPPORTED   # VALU: scan only
    assert dex(*dex_args(IDENTITY, SCAN, 16)) == EWORKSPACE
    assert dex(*dex_args(IDENTITY, SCAN, 16, dt=F32)) == EWORKSPACE
    assert dex(*dex_args(5, SCAN, 1 << 40)) == EINVAL
    wsx = L.kata_chunked_fwd_decay_ex_workspace
    assert wsx(1, 8, 131072, 16, 64, 64, BF16, PSD, SCAN, 0) == ws(1, 8, 131072, 16, 64, 64, BF16, SCAN)
    assert wsx(1, 2, 64, 16, 64, 64, F32, IDENTITY, SCAN, 0) == 2 * 16 * 64 * 4 + 256 + 256
    rec1 = 1 * 5 * 256                   # identity, d_k = 16, d_v = 64: four value tiles + z
    assert wsx(1, 8, 131072, 16, 64, 64, BF16, IDENTITY, SEQUENTIAL, 0) == 3 * 8 * rec1 * 4
    assert wsx(1, 8, 131072, 16, 64, 64, BF16, IDENTITY, SCAN, 0) > 3 * 8 * rec1 * 4
    dec = L.kata_decode_step_decay
    assert dec(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 4, 16, 64, BF16, None) == EINVAL
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 12, 64, BF16, None) == EUNSUPPORTED
    assert dec(None, None, None, None, None, None, None, 0, 16, 64, BF16, None) == OK


def test_profiled_needs_five_events(L):
    prof = L.kata_chunked_fwd_profiled
    evs = (ctypes.c_void_p * 5)(*([FAKE] * 5))
    base = (FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 16, 64, 64, 1, BF16, None, None, None, None,
            FAKE, 1 << 40, None)
    assert prof(*base, None, 5) == EINVAL
    assert prof(*base, evs, 4) == EINVAL
    assert prof(*base[:4], 1, 1, 64, 24, *base[8:], evs, 5) == EUNSUPPORTED


def test_workspace_query(L):
    for args in [(1, 8, 131072, 16, 64, 64, BF16, 1), (1, 16, 32768, 32, 64, 128, BF16, 1),
                 (1, 1, 256, 16, 16, 64, F32, 1), (2, 3, 100, 16, 64, 32, BF16, 0)]:
        n = L.kata_chunked_fwd_workspace(*args)
        assert n > 0 and n % 256 == 0
    assert L.kata_chunked_fwd_workspace(1, 1, 0, 16, 64, 64, BF16, 1) == 0
    assert L.kata_chunked_fwd_workspace(1, 1, 64, 17, 64, 64, BF16, 1) == 0


def test_scan_and_decode_reject(L):
    sc = L.kata_scan_states
    assert sc(FAKE, FAKE, 1, 1, 64, 16, 64, 64, BF16, None, None, None, FAKE, None, None,
              None, 0, None) == EINVAL                       # S_prefix missing
    assert sc(FAKE, FAKE, 1, 1, 64, 20, 64, 64, BF16, None, None, FAKE, FAKE, None, None,
              None, 0, None) == EUNSUPPORTED
    assert sc(None, None, 1, 1, 0, 16, 64, 64, BF16, None, None, None, None, None, None,
              None, 0, None) == OK
    dec = L.kata_decode_step
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 12, 64, BF16, None) == EUNSUPPORTED
    assert dec(FAKE, FAKE, FAKE, None, FAKE, FAKE, 4, 16, 64, BF16, None) == EINVAL
    assert dec(FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE, 4, 16, 64, BF16, None) == EINVAL
    assert dec(None, None, None, None, None, None, 0, 16, 64, BF16, None) == OK
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 16, 64, BF16, None) == EINVAL


def test_flash_rejects_before_launch(L):
    fl = L.kata_flash_fwd
    assert fl(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 16, 64, 1, F32, None) == EUNSUPPORTED
    assert fl(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 24, 64, 1, BF16, None) == EUNSUPPORTED
    assert fl(FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 16, 48, 1, BF16, None) == EUNSUPPORTED
    assert fl(MISALIGNED, FAKE, FAKE, FAKE, 1, 1, 64, 16, 64, 1, BF16, None) == EINVAL
    assert fl(None, FAKE, FAKE, FAKE, 1, 1, 64, 16, 64, 1, BF16, None) == EINVAL
    assert fl(FAKE, FAKE, FAKE, FAKE, 1, 1, -3, 16, 64, 1, BF16, None) == EINVAL
    assert fl(None, None, None, None, 1, 1, 0, 16, 64, 1, BF16, None) == OK     # empty: no launch
    assert fl(None, None, None, None, 0, 4, 64, 32, 64, 0, BF16, None) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import kernelized_linear_attention_phi_amd._binding as b
    monkeypatch.setattr(b, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(b, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        b.lib()


def test_prefix_depth(L):
    """kata_prefix_depth: the sequential walk takes one combine per chunk; the
    blocked scan grows with the number of 128-record tiles; the tree takes
    ceil(log2 n) levels per tile pass plus one per level of tiles, within
    ceil(log2 n) + 2 ceil(log128 n) (no GPU is touched)."""
    import math
    TREE = 2
    dep = L.kata_prefix_depth
    # the fp32 path scans one state per chunk: depth = scan levels over NC
    for nc in [1, 2, 3, 100, 128, 129, 300, 2048, 16385, 100000]:
        d = dep(1, 1, nc * 16, 16, 16, 16, F32, PSD, TREE, 0)
        lg = math.ceil(math.log2(nc)) if nc > 1 else 0
        tl = 0
        n = nc
        while n > 1:
            n = -(-n // 128)
            tl += 1
        assert d <= lg + 2 * max(tl, 1), (nc, d)
        assert d >= lg                        # no scan beats log2 n levels
        # blocked scan: a walk below 33 records, else runs of 16, 8 groups and
        # the carry across 128-record tiles
        want = nc if nc <= 32 else 16 + 8 + -(-nc // 128)
        assert dep(1, 1, nc * 16, 16, 16, 16, F32, PSD, SCAN, 0) == want
    assert dep(1, 1, 128 * 16, 16, 16, 16, F32, PSD, TREE, 0) == 7 + 1
    assert dep(1, 1, 2048 * 16, 16, 16, 16, F32, PSD, TREE, 0) == 7 + (4 + 1) + 1
    # matrix cores: a segment's chunks in order, then the scan over segments
    assert dep(1, 8, 131072, 16, 64, 64, BF16, PSD, SEQUENTIAL, 0) == 2048
    assert dep(1, 8, 131072, 16, 64, 64, BF16, PSD, TREE, 0) == 16 + 7 + 1      # G 16, 128 segments
    assert dep(1, 8, 131072, 16, 64, 64, BF16, PSD, TREE, 1) == 1 + 7 + 5 + 1  # G 1, 2048 segments
    assert dep(1, 8, 131072, 16, 64, 64, BF16, PSD, SCAN, 0) == 16 + 16 + 8 + 1
    assert dep(1, 1, 64, 24, 64, 64, BF16, PSD, TREE, 0) == -1
    assert dep(1, 1, 64, 16, 64, 64, F32, PSD, SEQUENTIAL, 0) == -1
    assert dep(1, 1, 64, 16, 64, 64, BF16, PSD, 7, 0) == -1
    assert dep(0, 1, 64, 16, 64, 64, BF16, PSD, TREE, 0) == 0


def test_delta_rejects_before_launch(L):
    dfw = L.kata_delta_fwd
    args = lambda **kw: (kw.get("q", FAKE), FAKE, FAKE, kw.get("beta", FAKE), FAKE, 1, 2,
                         kw.get("T", 64), kw.get("dk", 16), kw.get("dv", 64), kw.get("C", 64),
                         kw.get("dtype", BF16), kw.get("S0", None), None, None, None,
                         kw.get("ws", FAKE), kw.get("nws", 1 << 40), None)
    assert dfw(*args(C=128)) == EUNSUPPORTED
    assert dfw(*args(dk=24)) == EUNSUPPORTED
    assert dfw(*args(dv=48)) == EUNSUPPORTED
    assert dfw(*args(beta=None)) == EINVAL
    assert dfw(*args(q=MISALIGNED)) == EINVAL
    assert dfw(*args(S0=FAKE)) == EINVAL             # S0 without z0
    assert dfw(*args(dtype=5)) == EINVAL
    assert dfw(*args(T=0, q=None, beta=None, ws=None, nws=0)) == OK   # empty: nothing launched
    need = L.kata_delta_fwd_workspace(1, 2, 64, 16, 64, 64, BF16)
    assert need == 2 * 1 * 2 * 64 * 64 * 4                      # 2 C^2 floats per head and chunk
    assert L.kata_delta_fwd_workspace(1, 2, 65, 16, 64, 64, BF16) == 2 * need   # ragged: 2 chunks
    assert L.kata_delta_fwd_workspace(1, 2, 64, 16, 64, 128, BF16) == 0          # unsupported
    assert dfw(*args(nws=need - 1)) == EWORKSPACE
    assert dfw(*args(ws=None)) == EWORKSPACE
    assert dfw(*args(ws=MISALIGNED)) == EINVAL
    dec = L.kata_decode_step_delta
    assert dec(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 4, 16, 64, BF16, None) == EINVAL
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 12, 64, BF16, None) == EUNSUPPORTED
    assert dec(None, None, None, None, None, None, None, 0, 16, 64, BF16, None) == OK


def test_factored_dim_and_workspace(L):
    MULTI, SUMMED = 0, 1
    assert L.kata_factored_dim(16, 2, MULTI) == 72 and L.kata_factored_dim(16, 2, SUMMED) == 36
    assert L.kata_factored_dim(16, 4, MULTI) == 40 and L.kata_factored_dim(16, 4, SUMMED) == 10
    assert L.kata_factored_dim(32, 4, MULTI) == 144 and L.kata_factored_dim(32, 2, SUMMED) == 136
    assert L.kata_factored_dim(16, 1, MULTI) == 136 == L.kata_factored_dim(16, 1, SUMMED)
    assert L.kata_factored_dim(16, 3, MULTI) == -1 and L.kata_factored_dim(16, 0, MULTI) == -1
    assert L.kata_factored_dim(16, 2, 7) == -1 and L.kata_factored_dim(-1, 1, MULTI) == -1
    ws = L.kata_factored_fwd_workspace
    # g = 1 is the plain forward's workspace
    assert ws(1, 8, 4096, 16, 64, 64, BF16, 1, 1, MULTI) == L.kata_chunked_fwd_workspace(
        1, 8, 4096, 16, 64, 64, BF16, 1)
    # segment records + initial + total record per head: 512 segments of
    # 5 tiles x 5 units x 256 floats for d_k 16, g 2, multi (72 features)
    B, H, T = 1, 8, 131072
    rec = 5 * 5 * 256 * 4
    assert ws(B, H, T, 16, 64, 64, BF16, 1, 2, MULTI) >= (512 + 2 * B * H) * rec
    assert ws(B, H, T, 16, 64, 64, F32, 1, 2, MULTI) == 0          # bf16 only
    assert ws(B, H, T, 16, 64, 32, BF16, 1, 2, MULTI) == 0         # chunk 64 only
    assert ws(B, H, T, 32, 64, 64, BF16, 1, 2, MULTI) == 0         # 272 features: not built
    assert ws(B, H, T, 16, 64, 64, BF16, 1, 3, MULTI) == 0         # 3 does not divide 16


def test_factored_rejects_before_launch(L):
    MULTI, SUMMED = 0, 1
    fw = L.kata_factored_fwd
    args = lambda **kw: (kw.get("q", FAKE), FAKE, FAKE, FAKE, 1, 2, kw.get("T", 256),
                         kw.get("dk", 16), kw.get("dv", 64), kw.get("C", 64), 1,
                         kw.get("dtype", BF16), kw.get("g", 2), kw.get("kind", MULTI),
                         kw.get("S0", None), None, None, None, kw.get("ws", FAKE),
                         kw.get("wsb", 1 << 30), None)
    assert fw(*args(g=3)) == EINVAL
    assert fw(*args(g=0)) == EINVAL
    assert fw(*args(kind=5)) == EINVAL
    assert fw(*args(dtype=F32)) == EUNSUPPORTED
    assert fw(*args(C=32)) == EUNSUPPORTED
    assert fw(*args(dv=16)) == EUNSUPPORTED
    assert fw(*args(dk=32, g=2, kind=MULTI)) == EUNSUPPORTED
    assert fw(*args(dk=24)) == EUNSUPPORTED
    assert fw(*args(q=MISALIGNED)) == EINVAL
    assert fw(*args(S0=FAKE)) == EINVAL                            # S0 without z0
    assert fw(*args(wsb=16)) == EWORKSPACE
    assert fw(*args(ws=None)) == EWORKSPACE
    assert fw(*args(T=0, q=None, ws=None, wsb=0)) == OK              # empty: nothing launched
    assert fw(*args(g=1, C=48)) == EUNSUPPORTED                     # g = 1: kata_chunked_fwd
    dec = L.kata_decode_step_factored
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 64, 3, MULTI, BF16, None) == EINVAL
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 64, 2, MULTI, BF16, None) == EUNSUPPORTED
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 48, 2, SUMMED, BF16, None) == EUNSUPPORTED
    assert dec(MISALIGNED, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 64, 2, SUMMED, F32, None) == EINVAL
    assert dec(None, None, None, None, None, None, 0, 16, 64, 2, SUMMED, BF16, None) == OK
