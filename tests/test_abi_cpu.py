"""The C-ABI library on a machine without a GPU: it loads, exports every symbol
include/flp.h declares, and its fail-closed gates reject bad arguments before
any HIP call.  Pointers here are fake addresses: validation never dereferences
them and every case returns before the device is touched."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flp.h")

abi = pytest.importorskip("lm_head_selected_bf16_amd._abi")
if not os.path.exists(abi.LIB_PATH):
    pytest.skip("libflp.so not built (run __graft_entry__.build())", allow_module_level=True)

lib = abi.load()
S = {v: k for k, v in abi.STATUS_NAMES.items()}
BF16, F32, I64, I32 = abi.FLP_BF16, abi.FLP_F32, abi.FLP_I64, abi.FLP_I32


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flp_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = header_functions()
    assert set(names) == set(abi.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_build_info():
    for code, name in abi.STATUS_NAMES.items():
        assert abi.flp_status_string(code).startswith(name)
    info = abi.flp_build_info()
    assert "gfx950" in info and "vocab_tile=256" in info
    # provenance: the library has no fallback path and says so
    assert "fallback=none" in info
    assert abi.flp_status_string(99) == "FLP_UNKNOWN_STATUS"


# fake, 16-byte aligned, non-overlapping device addresses
H, W, B, T, TMP, LP, LS, WS = (0x10000000 * (k + 1) for k in range(8))
N, D, V = 40, 64, 1000


def fwd(**kw):
    a = dict(N=N, D=D, V=V, x=BF16, hidden=H, weight=W, bias=B, targets=T, t=I64, temp=TMP,
             logp=LP, lse=LS, ws=WS, wsb=abi.flp_forward_workspace_bytes(N, D, V), stream=0)
    a.update(kw)
    return abi.flp_forward(a["N"], a["D"], a["V"], a["x"], a["hidden"], a["weight"], a["bias"],
                           a["targets"], a["t"], a["temp"], a["logp"], a["lse"], a["ws"], a["wsb"],
                           a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(N=-1), "FLP_INVALID_ARGUMENT"),
    (dict(D=0), "FLP_INVALID_ARGUMENT"),
    (dict(V=0), "FLP_INVALID_ARGUMENT"),
    (dict(x=I64), "FLP_UNSUPPORTED_DTYPE"),
    (dict(x=9), "FLP_UNSUPPORTED_DTYPE"),
    (dict(t=BF16), "FLP_UNSUPPORTED_DTYPE"),
    (dict(D=48), "FLP_UNSUPPORTED_SHAPE"),
    (dict(N=2 ** 60), "FLP_UNSUPPORTED_SHAPE"),
    (dict(hidden=0), "FLP_INVALID_ARGUMENT"),
    (dict(weight=0), "FLP_INVALID_ARGUMENT"),
    (dict(targets=0), "FLP_INVALID_ARGUMENT"),
    (dict(logp=0), "FLP_INVALID_ARGUMENT"),
    (dict(ws=0), "FLP_INVALID_ARGUMENT"),
    (dict(hidden=H + 8), "FLP_MISALIGNED"),
    (dict(weight=W + 4), "FLP_MISALIGNED"),
    (dict(logp=LP + 2), "FLP_MISALIGNED"),
    (dict(targets=T + 4), "FLP_MISALIGNED"),
    (dict(ws=WS + 8), "FLP_MISALIGNED"),
    (dict(logp=H + 64), "FLP_INVALID_ARGUMENT"),          # output inside hidden
    (dict(lse=LP + 16), "FLP_INVALID_ARGUMENT"),          # two outputs overlap
    (dict(ws=W + 1024), "FLP_INVALID_ARGUMENT"),          # workspace inside weight
    (dict(wsb=100), "FLP_WORKSPACE_TOO_SMALL"),
    (dict(N=0, hidden=0, targets=0, logp=0, ws=0), "FLP_OK"),   # empty batch: no-op
])
def test_forward_gates(kw, expect):
    assert abi.STATUS_NAMES[fwd(**kw)] == expect


@pytest.mark.parametrize("x,esize", [(BF16, 2), (abi.FLP_F16, 2), (F32, 4)])
def test_hidden_row_offsets_stay_within_32_bits(x, esize):
    """A logit tile addresses its up to 256 rows with 32-bit offsets r * D * size: the
    largest D whose 256 rows stay below 2^31 bytes passes the shape gate (the call then
    stops at the later workspace gate, before any device work), the next multiple of 32
    is rejected (for the forward, the shard forward and the backward)."""
    d_max = ((1 << 31) - 1) // (256 * esize) // 32 * 32
    for D_, expect in ((d_max, "FLP_WORKSPACE_TOO_SMALL"), (d_max + 32, "FLP_UNSUPPORTED_SHAPE")):
        assert abi.STATUS_NAMES[fwd(N=1, V=1, D=D_, x=x, wsb=16)] == expect, D_
    assert abi.STATUS_NAMES[fpart(N=1, D=d_max + 32, x=x, VL=256, vs=0, VT=256)] == \
        "FLP_UNSUPPORTED_SHAPE"
    # the backward rejects the same D before sizing its workspace
    assert abi.STATUS_NAMES[bwd(N=1, V=1, D=d_max + 32, x=x, dwt=x, wsb=1 << 40)] == \
        "FLP_UNSUPPORTED_SHAPE"


def fwd_noalloc(**kw):
    a = dict(N=N, D=D, V=V, x=BF16, hidden=H, weight=W, bias=B, targets=T, t=I64, temp=TMP,
             logp=LP, lse=LS, stream=0)
    a.update(kw)
    return abi.flp_forward_noalloc(a["N"], a["D"], a["V"], a["x"], a["hidden"], a["weight"],
                                   a["bias"], a["targets"], a["t"], a["temp"], a["logp"], a["lse"],
                                   a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(N=-1), "FLP_INVALID_ARGUMENT"),
    (dict(x=I64), "FLP_UNSUPPORTED_DTYPE"),
    (dict(D=48), "FLP_UNSUPPORTED_SHAPE"),
    (dict(hidden=0), "FLP_INVALID_ARGUMENT"),
    (dict(logp=0), "FLP_INVALID_ARGUMENT"),
    (dict(weight=W + 4), "FLP_MISALIGNED"),
    (dict(logp=H + 64), "FLP_INVALID_ARGUMENT"),          # output inside hidden
    (dict(lse=LP + 16), "FLP_INVALID_ARGUMENT"),          # two outputs overlap
    # the workspace of 8440 rows at V = 131072 exceeds the fixed 33 MiB array
    (dict(N=8440, D=64, V=131072), "FLP_WORKSPACE_TOO_SMALL"),
    (dict(N=0, hidden=0, targets=0, logp=0), "FLP_OK"),   # empty batch: no-op
])
def test_forward_noalloc_gates(kw, expect):
    assert abi.STATUS_NAMES[fwd_noalloc(**kw)] == expect


def test_forward_noalloc_limit():
    """The fixed array holds the forward workspace of up to 8439 rows at V = 131072 (the
    rollout batch of 8192 rows fits); one row more does not."""
    cap = abi.FLP_FORWARD_NOALLOC_MAX_BYTES
    assert cap == 33 << 20
    assert abi.flp_forward_workspace_bytes(8439, 2688, 131072) <= cap
    assert abi.flp_forward_workspace_bytes(8440, 2688, 131072) > cap
    assert abi.flp_forward_workspace_bytes(8192, 2688, 131072) <= cap


def fpart(**kw):
    a = dict(N=N, D=D, VL=512, vs=256, VT=1000, x=BF16, hidden=H, weight=W, bias=B, targets=T,
             t=I64, temp=TMP, part=LP, zt=LS, stream=0)
    a.update(kw)
    return abi.flp_forward_partial(a["N"], a["D"], a["VL"], a["vs"], a["VT"], a["x"], a["hidden"],
                                   a["weight"], a["bias"], a["targets"], a["t"], a["temp"],
                                   a["part"], a["zt"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(vs=128), "FLP_UNSUPPORTED_SHAPE"),            # shard start off a 256-column tile
    (dict(VL=300), "FLP_UNSUPPORTED_SHAPE"),            # ragged shard that does not end V
    (dict(vs=768, VL=512), "FLP_INVALID_ARGUMENT"),     # runs past the vocabulary
    (dict(vs=-256), "FLP_INVALID_ARGUMENT"),
    (dict(VL=0), "FLP_INVALID_ARGUMENT"),
    (dict(D=40), "FLP_UNSUPPORTED_SHAPE"),
    (dict(x=I32), "FLP_UNSUPPORTED_DTYPE"),
    (dict(part=0), "FLP_INVALID_ARGUMENT"),
    (dict(zt=0), "FLP_INVALID_ARGUMENT"),
    (dict(part=LP + 8), "FLP_MISALIGNED"),
    (dict(zt=LS + 2), "FLP_MISALIGNED"),
    (dict(zt=H + 32), "FLP_INVALID_ARGUMENT"),          # zt inside hidden
    (dict(part=LS - 64), "FLP_INVALID_ARGUMENT"),       # partials run into zt
    (dict(N=0, hidden=0, targets=0, part=0, zt=0), "FLP_OK"),
])
def test_forward_partial_gates(kw, expect):
    assert abi.STATUS_NAMES[fpart(**kw)] == expect


def mrg(**kw):
    a = dict(N=N, VT=V, part=WS, zt=TMP, targets=T, t=I32, logp=LP, lse=LS, stream=0)
    a.update(kw)
    return abi.flp_merge(a["N"], a["VT"], a["part"], a["zt"], a["targets"], a["t"], a["logp"],
                         a["lse"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(N=-1), "FLP_INVALID_ARGUMENT"),
    (dict(VT=0), "FLP_INVALID_ARGUMENT"),
    (dict(t=F32), "FLP_UNSUPPORTED_DTYPE"),
    (dict(part=0), "FLP_INVALID_ARGUMENT"),
    (dict(logp=0), "FLP_INVALID_ARGUMENT"),
    (dict(part=WS + 8), "FLP_MISALIGNED"),
    (dict(logp=WS + 256), "FLP_INVALID_ARGUMENT"),      # output inside the partials
    (dict(lse=LP), "FLP_INVALID_ARGUMENT"),             # the two outputs coincide
    (dict(N=0, part=0, zt=0, targets=0, logp=0), "FLP_OK"),
])
def test_merge_gates(kw, expect):
    assert abi.STATUS_NAMES[mrg(**kw)] == expect


def test_partial_bytes():
    assert abi.flp_forward_partial_bytes(N, 512) == 2 * N * 8
    assert abi.flp_forward_partial_bytes(N, 513) == 3 * N * 8
    assert abi.flp_forward_partial_bytes(N, 0) == 0


def bwd(**kw):
    a = dict(N=N, D=D, V=V, x=BF16, g=TMP, lse=LS, hidden=H, weight=W, bias=B, targets=T, t=I64,
             temp=0, dh=0x90000000, dw=0xA0000000, dwt=BF16, db=0xB0000000, ws=WS,
             wsb=abi.flp_backward_workspace_bytes(N, D, V, BF16, BF16, 0), stream=0)
    a.update(kw)
    return abi.flp_backward(a["N"], a["D"], a["V"], a["x"], a["g"], a["lse"], a["hidden"],
                            a["weight"], a["bias"], a["targets"], a["t"], a["temp"], a["dh"],
                            a["dw"], a["dwt"], a["db"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(N=-3), "FLP_INVALID_ARGUMENT"),
    (dict(x=F32, dwt=BF16), "FLP_UNSUPPORTED_DTYPE"),   # d_weight dtype must be x or f32
    (dict(dwt=I32), "FLP_UNSUPPORTED_DTYPE"),
    (dict(D=100), "FLP_UNSUPPORTED_SHAPE"),
    (dict(g=0), "FLP_INVALID_ARGUMENT"),
    (dict(lse=0), "FLP_INVALID_ARGUMENT"),
    (dict(ws=0), "FLP_INVALID_ARGUMENT"),
    (dict(dh=0x90000002), "FLP_MISALIGNED"),
    (dict(db=0xB0000002), "FLP_MISALIGNED"),
    (dict(dh=H), "FLP_INVALID_ARGUMENT"),               # d_hidden aliases hidden
    (dict(db=0xA0000000 + 64), "FLP_INVALID_ARGUMENT"), # d_bias inside d_weight
    (dict(wsb=1000), "FLP_WORKSPACE_TOO_SMALL"),
    (dict(dh=0, dw=0, db=0, ws=0), "FLP_OK"),           # nothing requested: no-op
    # empty batch: only d_weight / d_bias would be written (zeros), so they are checked
    (dict(N=0, g=0, lse=0, hidden=0, targets=0, ws=0, dw=0, db=0), "FLP_OK"),
    (dict(N=0, g=0, lse=0, hidden=0, targets=0, ws=0, dw=0xA0000008), "FLP_MISALIGNED"),
    (dict(N=0, g=0, lse=0, hidden=0, targets=0, ws=0, db=0xB0000002), "FLP_MISALIGNED"),
    (dict(N=0, g=0, lse=0, hidden=0, targets=0, ws=0, db=0xA0000000 + 64), "FLP_INVALID_ARGUMENT"),
    (dict(N=0, g=0, lse=0, hidden=0, targets=0, ws=0, dw=W), "FLP_INVALID_ARGUMENT"),
])
def test_backward_gates(kw, expect):
    assert abi.STATUS_NAMES[bwd(**kw)] == expect


def test_workspace_sizes():
    # forward: one (max, sum) pair per row and 256-column vocabulary tile + the target logits
    n_vt = -(-V // 256)
    fb = abi.flp_forward_workspace_bytes(N, D, V)
    assert fb >= n_vt * N * 8 + N * 4 and fb % 256 == 0
    assert abi.flp_forward_workspace_bytes(-1, D, V) == 0
    # backward: the minimum is a 256-row chunk; bigger chunks cost more
    lo = abi.flp_backward_workspace_bytes(5000, 2688, 131072, BF16, BF16, 0)
    hi = abi.flp_backward_workspace_bytes(5000, 2688, 131072, BF16, BF16, 5000)
    assert 0 < lo < hi
    # a single chunk needs no fp32 d_weight accumulator
    one = abi.flp_backward_workspace_bytes(256, 2688, 131072, BF16, BF16, 256)
    assert one < 131072 * 2688 * 4
    # several chunks with a bf16 d_weight need the fp32 accumulator
    assert lo > 131072 * 2688 * 4
    # chunk rows round up to multiples of 256 and are capped at N
    assert (abi.flp_backward_workspace_bytes(600, 64, 1000, BF16, BF16, 300) ==
            abi.flp_backward_workspace_bytes(600, 64, 1000, BF16, BF16, 512))
    assert (abi.flp_backward_workspace_bytes(600, 64, 1000, BF16, BF16, 10 ** 6) ==
            abi.flp_backward_workspace_bytes(600, 64, 1000, BF16, BF16, 768))


def test_workspace_below_minimum_rejected():
    lo = abi.flp_backward_workspace_bytes(N, D, V, BF16, BF16, 0)
    for short in (1, 255, 4096, lo - 1):
        assert abi.STATUS_NAMES[bwd(wsb=short)] == "FLP_WORKSPACE_TOO_SMALL"


def lfwd(**kw):
    a = dict(N=N, V=1024, x=BF16, z=WS, targets=T, t=I64, logp=LP, lse=LS, stream=0)
    a.update(kw)
    return abi.flp_logits_forward(a["N"], a["V"], a["x"], a["z"], a["targets"], a["t"], a["logp"],
                                  a["lse"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(N=-1), "FLP_INVALID_ARGUMENT"),
    (dict(V=0), "FLP_INVALID_ARGUMENT"),
    (dict(V=1001), "FLP_UNSUPPORTED_SHAPE"),            # rows must be whole 16-byte chunks
    (dict(x=F32, V=1022), "FLP_UNSUPPORTED_SHAPE"),
    (dict(x=I64), "FLP_UNSUPPORTED_DTYPE"),
    (dict(t=BF16), "FLP_UNSUPPORTED_DTYPE"),
    (dict(z=0), "FLP_INVALID_ARGUMENT"),
    (dict(logp=0), "FLP_INVALID_ARGUMENT"),
    (dict(z=WS + 8), "FLP_MISALIGNED"),
    (dict(logp=WS + 64), "FLP_INVALID_ARGUMENT"),       # output inside the logits
    (dict(N=0, z=0, targets=0, logp=0), "FLP_OK"),
])
def test_logits_forward_gates(kw, expect):
    assert abi.STATUS_NAMES[lfwd(**kw)] == expect


def lbwd(**kw):
    a = dict(N=N, V=1024, x=BF16, g=TMP, lse=LS, z=WS, targets=T, t=I32, d=0x90000000, stream=0)
    a.update(kw)
    return abi.flp_logits_backward(a["N"], a["V"], a["x"], a["g"], a["lse"], a["z"], a["targets"],
                                   a["t"], a["d"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(V=12), "FLP_UNSUPPORTED_SHAPE"),
    (dict(g=0), "FLP_INVALID_ARGUMENT"),
    (dict(d=0), "FLP_INVALID_ARGUMENT"),
    (dict(d=0x90000008), "FLP_MISALIGNED"),
    (dict(d=WS + 1024), "FLP_INVALID_ARGUMENT"),        # d_logits overlaps the logits
    (dict(N=0, g=0, lse=0, z=0, targets=0, d=0), "FLP_OK"),
])
def test_logits_backward_gates(kw, expect):
    assert abi.STATUS_NAMES[lbwd(**kw)] == expect


# ---- indexed variants ----
RW = 0xC0000000  # row ids


def ifwd(**kw):
    a = dict(N=N, D=D, V=V, x=BF16, hidden=H, weight=W, bias=B, targets=T, t=I64, temp=TMP,
             rows=RW, r=I64, n=17, logp=LP, lse=LS, ws=WS,
             wsb=abi.flp_forward_indexed_workspace_bytes(N, D, V, BF16, 17), stream=0)
    a.update(kw)
    return abi.flp_forward_indexed(a["N"], a["D"], a["V"], a["x"], a["hidden"], a["weight"],
                                   a["bias"], a["targets"], a["t"], a["temp"], a["rows"], a["r"],
                                   a["n"], a["logp"], a["lse"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(n=-1), "FLP_INVALID_ARGUMENT"),
    (dict(r=BF16), "FLP_UNSUPPORTED_DTYPE"),
    (dict(rows=0), "FLP_INVALID_ARGUMENT"),             # ids required when n_rows > 0
    (dict(rows=RW + 4), "FLP_MISALIGNED"),              # int64 ids 8-byte aligned
    (dict(rows=LP), "FLP_INVALID_ARGUMENT"),            # ids overlap an output
    (dict(rows=WS + 256), "FLP_INVALID_ARGUMENT"),      # ids inside the workspace
    (dict(N=1 << 31), "FLP_UNSUPPORTED_SHAPE"),         # compact positions are int32
    (dict(D=48), "FLP_UNSUPPORTED_SHAPE"),
    (dict(wsb=1024), "FLP_WORKSPACE_TOO_SMALL"),
    (dict(ws=0), "FLP_INVALID_ARGUMENT"),
    (dict(N=0, hidden=0, targets=0, logp=0, ws=0), "FLP_OK"),
])
def test_forward_indexed_gates(kw, expect):
    assert abi.STATUS_NAMES[ifwd(**kw)] == expect


def ibwd(**kw):
    a = dict(N=N, D=D, V=V, x=BF16, g=TMP, lse=LS, hidden=H, weight=W, bias=B, targets=T, t=I64,
             temp=0, rows=RW, r=I32, n=9, dh=0x90000000, dw=0xA0000000, dwt=BF16, db=0xB0000000,
             ws=WS, wsb=abi.flp_backward_indexed_workspace_bytes(N, D, V, BF16, BF16, 9, 0),
             stream=0)
    a.update(kw)
    return abi.flp_backward_indexed(a["N"], a["D"], a["V"], a["x"], a["g"], a["lse"], a["hidden"],
                                    a["weight"], a["bias"], a["targets"], a["t"], a["temp"],
                                    a["rows"], a["r"], a["n"], a["dh"], a["dw"], a["dwt"], a["db"],
                                    a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(n=-2), "FLP_INVALID_ARGUMENT"),
    (dict(r=F32), "FLP_UNSUPPORTED_DTYPE"),
    (dict(rows=RW + 2), "FLP_MISALIGNED"),              # int32 ids 4-byte aligned
    (dict(rows=0xA0000000 + 4096), "FLP_INVALID_ARGUMENT"),  # ids inside d_weight
    (dict(x=F32, dwt=BF16), "FLP_UNSUPPORTED_DTYPE"),
    (dict(g=0), "FLP_INVALID_ARGUMENT"),
    (dict(wsb=4096), "FLP_WORKSPACE_TOO_SMALL"),
    (dict(dh=0, dw=0, db=0, ws=0), "FLP_OK"),           # nothing requested: no-op
    (dict(N=0, g=0, lse=0, hidden=0, targets=0, ws=0, dw=0, db=0), "FLP_OK"),
    (dict(N=0, g=0, lse=0, hidden=0, targets=0, ws=0, dw=0xA0000008), "FLP_MISALIGNED"),
    (dict(N=0, g=0, lse=0, hidden=0, targets=0, ws=0, dw=0, db=B), "FLP_INVALID_ARGUMENT"),
])
def test_backward_indexed_gates(kw, expect):
    assert abi.STATUS_NAMES[ibwd(**kw)] == expect


def test_indexed_workspace_sizes():
    # the prefix (mask, positions, ids, gathered rows) plus the dense workspace of min(n, N) rows
    f = abi.flp_forward_indexed_workspace_bytes(1000, 2688, 131072, BF16, 300)
    assert f > abi.flp_forward_workspace_bytes(300, 2688, 131072) + 300 * 2688 * 2
    assert (abi.flp_forward_indexed_workspace_bytes(1000, 2688, 131072, BF16, 5000) ==
            abi.flp_forward_indexed_workspace_bytes(1000, 2688, 131072, BF16, 1000))
    assert abi.flp_forward_indexed_workspace_bytes(1000, 2688, 131072, BF16, 0) < 8192
    b = abi.flp_backward_indexed_workspace_bytes(1000, 2688, 131072, BF16, BF16, 300, 300)
    assert b > abi.flp_backward_workspace_bytes(300, 2688, 131072, BF16, BF16, 300)
    assert abi.flp_logits_indexed_workspace_bytes(1000) == 1024
    assert abi.flp_logits_indexed_workspace_bytes(0) == 0


def lifwd(**kw):
    a = dict(N=N, V=1024, x=BF16, z=WS, targets=T, t=I64, rows=RW, r=I64, n=5, logp=LP, lse=LS,
             ws=0x90000000, wsb=256, stream=0)
    a.update(kw)
    return abi.flp_logits_forward_indexed(a["N"], a["V"], a["x"], a["z"], a["targets"], a["t"],
                                          a["rows"], a["r"], a["n"], a["logp"], a["lse"], a["ws"],
                                          a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(n=-1), "FLP_INVALID_ARGUMENT"),
    (dict(r=F32), "FLP_UNSUPPORTED_DTYPE"),
    (dict(rows=0), "FLP_INVALID_ARGUMENT"),
    (dict(ws=0), "FLP_INVALID_ARGUMENT"),
    (dict(wsb=16), "FLP_WORKSPACE_TOO_SMALL"),          # one mask byte per row, 256-rounded
    (dict(ws=LP), "FLP_INVALID_ARGUMENT"),              # workspace overlaps logp
    (dict(V=1001), "FLP_UNSUPPORTED_SHAPE"),
    (dict(N=0, z=0, targets=0, logp=0, ws=0), "FLP_OK"),
])
def test_logits_forward_indexed_gates(kw, expect):
    assert abi.STATUS_NAMES[lifwd(**kw)] == expect


def libwd(**kw):
    a = dict(N=N, V=1024, x=BF16, g=TMP, lse=LS, z=WS, targets=T, t=I32, rows=RW, r=I32, n=5,
             d=0x90000000, ws=0xB0000000, wsb=256, stream=0)
    a.update(kw)
    return abi.flp_logits_backward_indexed(a["N"], a["V"], a["x"], a["g"], a["lse"], a["z"],
                                           a["targets"], a["t"], a["rows"], a["r"], a["n"], a["d"],
                                           a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(g=0), "FLP_INVALID_ARGUMENT"),
    (dict(lse=0), "FLP_INVALID_ARGUMENT"),
    (dict(d=0x90000008), "FLP_MISALIGNED"),
    (dict(rows=0x90000000 + 64), "FLP_INVALID_ARGUMENT"),  # ids inside d_logits
    (dict(wsb=0), "FLP_WORKSPACE_TOO_SMALL"),
    (dict(N=0, g=0, lse=0, z=0, targets=0, d=0, ws=0), "FLP_OK"),
])
def test_logits_backward_indexed_gates(kw, expect):
    assert abi.STATUS_NAMES[libwd(**kw)] == expect


# ---- untied embedding lookup ----

def efwd(**kw):
    a = dict(N=N, D=64, V=V, x=BF16, w=W, ids=T, t=I64, out=0x90000000, stream=0)
    a.update(kw)
    return abi.flp_embedding_forward(a["N"], a["D"], a["V"], a["x"], a["w"], a["ids"], a["t"],
                                     a["out"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(N=-1), "FLP_INVALID_ARGUMENT"),
    (dict(V=0), "FLP_INVALID_ARGUMENT"),
    (dict(x=I32), "FLP_UNSUPPORTED_DTYPE"),
    (dict(t=F32), "FLP_UNSUPPORTED_DTYPE"),
    (dict(D=4), "FLP_UNSUPPORTED_SHAPE"),               # rows move in 16-byte chunks
    (dict(x=F32, D=6), "FLP_UNSUPPORTED_SHAPE"),
    (dict(V=(1 << 31) - 1), "FLP_UNSUPPORTED_SHAPE"),   # id V must fit the 32-bit sort key
    (dict(w=0), "FLP_INVALID_ARGUMENT"),
    (dict(out=0x90000008), "FLP_MISALIGNED"),
    (dict(ids=T + 4), "FLP_MISALIGNED"),
    (dict(out=W + 64), "FLP_INVALID_ARGUMENT"),         # output inside the table
    (dict(N=0, w=0, ids=0, out=0), "FLP_OK"),
])
def test_embedding_forward_gates(kw, expect):
    assert abi.STATUS_NAMES[efwd(**kw)] == expect


def ebwd(**kw):
    a = dict(N=N, D=64, V=V, x=BF16, g=H, ids=T, t=I32, dw=0x90000000, dwt=BF16, ws=WS,
             wsb=abi.flp_embedding_backward_workspace_bytes(N, 64, V), stream=0)
    a.update(kw)
    return abi.flp_embedding_backward(a["N"], a["D"], a["V"], a["x"], a["g"], a["ids"], a["t"],
                                      a["dw"], a["dwt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(dwt=I64), "FLP_UNSUPPORTED_DTYPE"),
    (dict(x=F32, dwt=BF16), "FLP_UNSUPPORTED_DTYPE"),   # d_weight dtype must be x or f32
    (dict(g=0), "FLP_INVALID_ARGUMENT"),
    (dict(dw=0), "FLP_INVALID_ARGUMENT"),
    (dict(ws=0), "FLP_INVALID_ARGUMENT"),
    (dict(wsb=1024), "FLP_WORKSPACE_TOO_SMALL"),
    (dict(dw=0x90000004), "FLP_MISALIGNED"),
    (dict(dw=H), "FLP_INVALID_ARGUMENT"),               # d_weight overlaps grad
    (dict(ws=0x90000000 + 1024), "FLP_INVALID_ARGUMENT"),  # workspace inside d_weight
    # empty batch: d_weight is still written (zeros), so it is required and checked
    (dict(N=0, g=0, ids=0, dw=0, ws=0), "FLP_INVALID_ARGUMENT"),
    (dict(N=0, g=0, ids=0, dw=0x90000004, ws=0), "FLP_MISALIGNED"),
])
def test_embedding_backward_gates(kw, expect):
    assert abi.STATUS_NAMES[ebwd(**kw)] == expect


def test_embedding_workspace_bytes():
    # two (key, value) sort buffers of N, the per-block digit counts, two [V] bounds, and
    # two fp32 [N / 32, D] slots for segments that span groups
    b = abi.flp_embedding_backward_workspace_bytes(16384, 2688, 131072)
    assert b >= 4 * 16384 * 4 + 256 * 64 * 4 + 2 * 131072 * 4 + 2 * 512 * 2688 * 4
    assert abi.flp_embedding_backward_workspace_bytes(-1, 64, 10) == 0


# ---- measurement probes (gates only: every case is rejected before the device is used) ----

def test_probe_gates():
    sb = abi.flp_probe_scratch_bytes()
    assert sb >= 2048 * 4
    bad = [
        (dict(iters=0), "FLP_INVALID_ARGUMENT"),
        (dict(iters=10 ** 7), "FLP_INVALID_ARGUMENT"),
        (dict(scratch=0), "FLP_INVALID_ARGUMENT"),
        (dict(scratch=WS + 8), "FLP_MISALIGNED"),
        (dict(sbytes=sb - 1), "FLP_WORKSPACE_TOO_SMALL"),
    ]
    for kw, expect in bad:
        a = dict(iters=10, scratch=WS, sbytes=sb)
        a.update(kw)
        st, _, _ = abi.flp_probe_mfma(False, a["iters"], a["scratch"], a["sbytes"], 0)
        assert abi.STATUS_NAMES[st] == expect, kw
    bad = [
        (dict(buf=0), "FLP_INVALID_ARGUMENT"),
        (dict(nbytes=8), "FLP_INVALID_ARGUMENT"),
        (dict(nbytes=1000), "FLP_INVALID_ARGUMENT"),          # not a multiple of 16
        (dict(buf=H + 4), "FLP_MISALIGNED"),
        (dict(sbytes=16), "FLP_WORKSPACE_TOO_SMALL"),
        (dict(buf=WS - 1024, nbytes=4096), "FLP_INVALID_ARGUMENT"),  # buffer overlaps scratch
    ]
    for kw, expect in bad:
        a = dict(buf=H, nbytes=1 << 20, scratch=WS, sbytes=sb)
        a.update(kw)
        st, _ = abi.flp_probe_read(a["buf"], a["nbytes"], a["scratch"], a["sbytes"], 0)
        assert abi.STATUS_NAMES[st] == expect, kw


# ---- the backward's chunk planner (pure host arithmetic) ----

from hypothesis import given, settings, strategies as st  # noqa: E402

_DT = [(BF16, BF16), (BF16, F32), (F32, F32), (abi.FLP_F16, abi.FLP_F16)]


@settings(max_examples=300, deadline=None)
@given(N=st.integers(1, 200000), D=st.integers(1, 160).map(lambda k: 32 * k),
       V=st.integers(1, 300000), dt=st.sampled_from(_DT), chunk=st.integers(0, 70000),
       needs=st.sampled_from([(1, 1, 1), (1, 0, 0), (0, 1, 0), (0, 0, 1), (1, 1, 0)]))
def test_chunk_planner_properties(N, D, V, dt, chunk, needs):
    """The workspace asked for a chunk size is accepted and yields at least that chunk
    (capped at N rounded up to 256); the minimum yields a chunk; a chunk is a multiple of
    256; one byte less than the minimum yields none; more bytes never give a smaller chunk."""
    x, dw = dt
    q = 256
    full = -(-N // q) * q
    lo = abi.flp_backward_workspace_bytes(N, D, V, x, dw, 0)
    c_lo = abi.flp_backward_chunk_rows(N, D, V, x, dw, lo, *needs)
    assert c_lo >= q and c_lo % q == 0 and c_lo <= full
    if all(needs):
        assert abi.flp_backward_chunk_rows(N, D, V, x, dw, lo - 1, *needs) == 0
    want = min(-(-max(chunk, 1) // q) * q, full)
    b = abi.flp_backward_workspace_bytes(N, D, V, x, dw, max(chunk, 1))
    c = abi.flp_backward_chunk_rows(N, D, V, x, dw, b, *needs)
    assert c >= q and c % q == 0 and c <= full
    if all(needs) and want == full:
        assert c == full  # a workspace sized for the whole batch runs it as one chunk
    assert abi.flp_backward_chunk_rows(N, D, V, x, dw, b + (1 << 30), *needs) >= c


def test_chunk_planner_examples():
    # the long sequence in 16 GiB: chunks of 16384 rows (whole d_hidden waves)
    assert abi.flp_backward_chunk_rows(65600, 2688, 131072, BF16, BF16, 16 << 30) == 16384
    # the training batch in one chunk when it fits
    one = abi.flp_backward_workspace_bytes(16384, 2688, 131072, BF16, BF16, 16384)
    assert abi.flp_backward_chunk_rows(16384, 2688, 131072, BF16, BF16, one) == 16384
    # the minimum for 630 rows (accepted exactly; once rejected by an off-by-slack search)
    lo = abi.flp_backward_workspace_bytes(630, 128, 1000, BF16, BF16, 0)
    assert abi.flp_backward_chunk_rows(630, 128, 1000, BF16, BF16, lo) == 256
    assert abi.flp_backward_chunk_rows(0, 128, 1000, BF16, BF16, lo) == 0
    # a small vocabulary: one 512-row chunk (no fp32 accumulator) needs less than two of 256
    lo = abi.flp_backward_workspace_bytes(257, 1344, 177, BF16, BF16, 0)
    assert lo == abi.flp_backward_workspace_bytes(257, 1344, 177, BF16, BF16, 512)
    assert abi.flp_backward_chunk_rows(257, 1344, 177, BF16, BF16, lo) == 512
    assert abi.flp_backward_chunk_rows(257, 1344, 177, BF16, BF16, lo - 1) == 0
