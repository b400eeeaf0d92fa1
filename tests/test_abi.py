"""C ABI checks that need no GPU: the library loads, exports every function
that include/kda.h declares, and rejects bad arguments with the documented
status codes before making any HIP call (so these run on a CPU-only host)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_40_amd import libkda as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.LIB_PATH):
        from gated_delta_rule_40_amd import build
        build.build()
    return K.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("kda_prefill", "kda_decode_step", "kda_status_string"):
        assert required in names
    assert set(names) == set(K.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.kda_version() >= 100
    for code in range(5):
        s = lib.kda_status_string(code)
        assert s and s.decode().startswith(("KDA_OK", "KDA_ERR"))
    assert lib.kda_status_string(99) is not None


# fake but 16-byte aligned, non-null device pointers: never dereferenced,
# because every call below fails validation before any HIP call
P = ctypes.c_void_p(0x10000)
NULL = None


def prefill(lib, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, init=NULL, cu=P, N=1, T=16, H=1, dk=128, dv=128,
             dtype=K.KDA_BF16, out=P, fin=NULL, chunk=0, dvb=0)
    a.update(kw)
    return lib.kda_prefill_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], a["init"], a["cu"], a["N"],
                              a["T"], a["H"], a["dk"], a["dv"], a["dtype"], a["out"], a["fin"],
                              a["chunk"], a["dvb"], None)


def decode(lib, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, state=P, N=1, H=1, dk=128, dv=128, dtype=K.KDA_BF16, out=P)
    a.update(kw)
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"], a["N"], a["H"],
                               a["dk"], a["dv"], a["dtype"], a["out"], None)


@pytest.mark.parametrize("field", ["q", "k", "v", "g", "beta", "cu", "out"])
def test_prefill_null_pointer(lib, field):
    assert prefill(lib, dk=64, **{field: NULL}) == K.KDA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), K.KDA_ERR_INVALID_ARG),
    (dict(T=-5), K.KDA_ERR_INVALID_ARG),
    (dict(H=0), K.KDA_ERR_INVALID_ARG),
    (dict(dk=0), K.KDA_ERR_INVALID_ARG),
    (dict(dtype=7), K.KDA_ERR_INVALID_ARG),
    (dict(q=ctypes.c_void_p(0x10008)), K.KDA_ERR_INVALID_ARG),   # misaligned
    (dict(dk=64), K.KDA_ERR_UNSUPPORTED),
    (dict(dv=256), K.KDA_ERR_UNSUPPORTED),
    (dict(chunk=48), K.KDA_ERR_UNSUPPORTED),
    (dict(chunk=16), K.KDA_ERR_UNSUPPORTED),                    # bf16 supports 32 / 64
    (dict(dtype=K.KDA_F32, chunk=64), K.KDA_ERR_UNSUPPORTED),   # fp32 supports 16 / 32
    (dict(dvb=24), K.KDA_ERR_UNSUPPORTED),
    (dict(chunk=64, dvb=16), K.KDA_ERR_UNSUPPORTED),             # 64-token bf16 chunks need >= 2 waves
])
def test_prefill_rejects(lib, kw, code):
    assert prefill(lib, **kw) == code


def test_prefill_empty_batch_is_a_no_op(lib):
    # no sequences: nothing to launch, success without touching the device
    assert prefill(lib, N=0, T=0) == K.KDA_OK


@pytest.mark.parametrize("field", ["q", "k", "v", "g", "beta", "state", "out"])
def test_decode_null_pointer(lib, field):
    assert decode(lib, **{field: NULL}) == K.KDA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(N=-2), K.KDA_ERR_INVALID_ARG),
    (dict(H=-1), K.KDA_ERR_INVALID_ARG),
    (dict(dtype=3), K.KDA_ERR_INVALID_ARG),
    (dict(state=ctypes.c_void_p(0x10004)), K.KDA_ERR_INVALID_ARG),
    (dict(dk=96), K.KDA_ERR_UNSUPPORTED),
])
def test_decode_rejects(lib, kw, code):
    assert decode(lib, **kw) == code


def test_decode_empty_batch_is_a_no_op(lib):
    assert decode(lib, N=0) == K.KDA_OK


def test_binding_raises_without_library(tmp_path):
    with pytest.raises(FileNotFoundError):
        K.load(str(tmp_path / "missing.so"))


def prefill_cp(lib, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, init=NULL, cu=P, N=1, T=4096, H=1, dk=128, dv=128,
             dtype=K.KDA_BF16, out=P, fin=NULL, seg=1024, ws=ctypes.c_void_p(0x100000), wsb=1 << 40)
    a.update(kw)
    return lib.kda_prefill_cp(a["q"], a["k"], a["v"], a["g"], a["beta"], a["init"], a["cu"], a["N"], a["T"],
                              a["H"], a["dk"], a["dv"], a["dtype"], a["out"], a["fin"], a["seg"], a["ws"],
                              a["wsb"], None)


def test_cp_workspace_size(lib):
    ws = lib.kda_prefill_cp_workspace_size
    B = K.KDA_BF16
    small = ws(1, 4096, 1, 128, 128, B, 1024)
    # at least: summaries (dk x (dv + dk)) and entering states (dk x dv) per
    # segment, and one chunk-operand image (> 24 KiB in bf16) per 32-token chunk
    assert small >= 5 * 128 * (256 + 128) * 4 + 128 * 24 * 1024
    assert ws(1, 4096, 1, 128, 128, K.KDA_F32, 1024) > small   # fp32 operand images are larger
    assert ws(1, 8192, 1, 128, 128, B, 1024) > small           # more segments and chunks
    assert ws(1, 4096, 4, 128, 128, B, 1024) > small           # more heads
    assert ws(1, 4096, 1, 128, 128, B, 0) > 0                  # automatic segment length
    assert ws(1, 4096, 1, 64, 128, B, 1024) == 0               # unsupported head size
    assert ws(1, 4096, 1, 128, 128, B, 48) == 0                # not a multiple of 32
    assert ws(3, 4096, 1, 128, 128, B, -1024) > 0              # pieces of 1,024 tokens
    assert ws(3, 4096, 1, 128, 128, B, -48) == 0
    assert ws(257, 4096, 1, 128, 128, B, -1024) > 0            # pieces with more than 256 sequences


def test_cp_automatic_cut(lib):
    # The automatic cut of a long bf16 batch (T H / 256 above 32,768 tokens,
    # at most 256 sequences) is 512 / H pieces per head: for 2^20 tokens in 8
    # sequences, 32 pieces at 16 heads and 8 at 64 heads (segments at most
    # pieces + 8), the layouts of explicit pieces of 1,025 and 4,097 chunks;
    # at 64 heads the per-sequence cut would take 32 + 8 segments.  fp32
    # inputs, more than 256 sequences and short batches keep the per-sequence
    # cut (segments of T H / 256 tokens, at most 32,768).
    ws = lib.kda_prefill_cp_workspace_size
    B, F = K.KDA_BF16, K.KDA_F32
    T = 1 << 20
    assert ws(8, T, 16, 128, 128, B, 0) == ws(8, T, 16, 128, 128, B, -1025 * 32)
    assert ws(8, T, 64, 128, 128, B, 0) == ws(8, T, 64, 128, 128, B, -4097 * 32)
    assert ws(8, T, 64, 128, 128, B, 0) < ws(8, T, 64, 128, 128, B, 32768)
    assert ws(8, T, 64, 128, 128, F, 0) == ws(8, T, 64, 128, 128, F, 32768)
    assert ws(257, T, 16, 128, 128, B, 0) == ws(257, T, 16, 128, 128, B, 32768)
    assert ws(4, 65536, 32, 128, 128, B, 0) == ws(4, 65536, 32, 128, 128, B, 8192)
    assert ws(1, 4096, 1, 128, 128, 7, 1024) == 0              # bad dtype
    assert ws(-1, 4096, 1, 128, 128, B, 1024) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(ws=NULL), K.KDA_ERR_INVALID_ARG),
    (dict(ws=ctypes.c_void_p(0x100010)), K.KDA_ERR_INVALID_ARG),   # workspace not 256-byte aligned
    (dict(wsb=1024), K.KDA_ERR_INVALID_ARG),                       # workspace too small
    (dict(seg=-48), K.KDA_ERR_UNSUPPORTED),                       # pieces: not a multiple of 32
    (dict(cu=NULL), K.KDA_ERR_INVALID_ARG),
    (dict(q=NULL), K.KDA_ERR_INVALID_ARG),
    (dict(seg=48), K.KDA_ERR_UNSUPPORTED),
    (dict(seg=16), K.KDA_ERR_UNSUPPORTED),
    (dict(dk=64), K.KDA_ERR_UNSUPPORTED),
])
def test_prefill_cp_rejects(lib, kw, code):
    assert prefill_cp(lib, **kw) == code


def test_prefill_cp_empty_batch_is_a_no_op(lib):
    assert prefill_cp(lib, N=0, T=0) == K.KDA_OK


def decode_tokens(lib, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, cu=P, nt=NULL, sin=P, sout=NULL, N=1, T=4, H=1, dk=128, dv=128,
             dtype=K.KDA_BF16, out=NULL)
    a.update(kw)
    return lib.kda_decode_tokens(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["nt"], a["sin"], a["sout"],
                                 a["N"], a["T"], a["H"], a["dk"], a["dv"], a["dtype"], a["out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), K.KDA_ERR_INVALID_ARG),
    (dict(cu=NULL), K.KDA_ERR_INVALID_ARG),
    (dict(sin=NULL), K.KDA_ERR_INVALID_ARG),
    (dict(sin=ctypes.c_void_p(0x10004)), K.KDA_ERR_INVALID_ARG),
    (dict(sout=ctypes.c_void_p(0x10008)), K.KDA_ERR_INVALID_ARG),
    (dict(out=ctypes.c_void_p(0x10002)), K.KDA_ERR_INVALID_ARG),
    (dict(N=-1), K.KDA_ERR_INVALID_ARG),
    (dict(dtype=5), K.KDA_ERR_INVALID_ARG),
    (dict(dk=64), K.KDA_ERR_UNSUPPORTED),
])
def test_decode_tokens_rejects(lib, kw, code):
    assert decode_tokens(lib, **kw) == code


def test_decode_tokens_empty_batch_is_a_no_op(lib):
    assert decode_tokens(lib, N=0, T=0) == K.KDA_OK


def prefill_snap(lib, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, init=NULL, cu=P, N=1, T=64, H=1, dk=128, dv=128,
             dtype=K.KDA_BF16, out=P, fin=NULL, every=64, maxs=2, snaps=P)
    a.update(kw)
    return lib.kda_prefill_snapshots(a["q"], a["k"], a["v"], a["g"], a["beta"], a["init"], a["cu"], a["N"], a["T"],
                                     a["H"], a["dk"], a["dv"], a["dtype"], a["out"], a["fin"], a["every"],
                                     a["maxs"], a["snaps"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(snaps=NULL), K.KDA_ERR_INVALID_ARG),
    (dict(every=0), K.KDA_ERR_INVALID_ARG),
    (dict(maxs=0), K.KDA_ERR_INVALID_ARG),
    (dict(every=48), K.KDA_ERR_UNSUPPORTED),
    (dict(every=48, N=0, T=0), K.KDA_ERR_UNSUPPORTED),          # checked before the empty-batch exit
    (dict(dk=64), K.KDA_ERR_UNSUPPORTED),
])
def test_prefill_snapshots_rejects(lib, kw, code):
    assert prefill_snap(lib, **kw) == code


def test_prefill_snapshots_empty_batch_is_a_no_op(lib):
    assert prefill_snap(lib, N=0, T=0) == K.KDA_OK


def backward(lib, **kw):
    a = dict(q=P, k=P, v=P, g=P, beta=P, init=NULL, cu=P, N=1, T=64, H=1, dk=128, dv=128, dtype=K.KDA_BF16,
             dout=P, dfin=NULL, dq=P, dk_=P, dv_=P, dg=P, db=P, dinit=NULL, ws=ctypes.c_void_p(0x100000),
             wsb=1 << 40)
    a.update(kw)
    return lib.kda_backward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["init"], a["cu"], a["N"], a["T"], a["H"],
                            a["dk"], a["dv"], a["dtype"], a["dout"], a["dfin"], a["dq"], a["dk_"], a["dv_"], a["dg"],
                            a["db"], a["dinit"], a["ws"], a["wsb"], None)


def test_backward_workspace_size(lib):
    ws = lib.kda_backward_workspace_size
    small = ws(1, 4096, 2, 128, 128, K.KDA_BF16)
    # at least the chunk-start states: (4096 / 32 + 2) chunks x 2 heads x 64 KiB
    assert small >= 130 * 2 * 65536
    assert ws(1, 8192, 2, 128, 128, K.KDA_BF16) > small and ws(2, 4096, 2, 128, 128, K.KDA_BF16) > small
    assert ws(1, 4096, 2, 128, 128, K.KDA_F32) > small      # fp32 chunk images are larger
    assert ws(1, 4096, 2, 64, 128, K.KDA_BF16) == 0 and ws(-1, 4096, 2, 128, 128, K.KDA_BF16) == 0
    assert ws(1, 4096, 2, 128, 128, 7) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dout=NULL), K.KDA_ERR_INVALID_ARG),
    (dict(dq=NULL), K.KDA_ERR_INVALID_ARG),
    (dict(db=NULL), K.KDA_ERR_INVALID_ARG),
    (dict(dg=ctypes.c_void_p(0x10004)), K.KDA_ERR_INVALID_ARG),
    (dict(dinit=ctypes.c_void_p(0x10008)), K.KDA_ERR_INVALID_ARG),
    (dict(ws=NULL), K.KDA_ERR_INVALID_ARG),
    (dict(wsb=4096), K.KDA_ERR_INVALID_ARG),
    (dict(cu=NULL), K.KDA_ERR_INVALID_ARG),
    (dict(dk=64), K.KDA_ERR_UNSUPPORTED),
])
def test_backward_rejects(lib, kw, code):
    assert backward(lib, **kw) == code


def test_backward_empty_batch_is_a_no_op(lib):
    assert backward(lib, N=0, T=0) == K.KDA_OK
