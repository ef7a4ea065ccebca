"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/kda.h declares, sizes workspaces, and rejects invalid
arguments on the host before touching any pointer or calling HIP."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_55_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
BF16, F32 = kda.KDA_BF16, kda.KDA_F32
FAKE = 0x10000000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:kda|gdn)_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_55_amd import build
        build.build()
    return kda.load()


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert {"kda_chunk_fwd", "kda_decode_step", "kda_chunk_fwd_workspace_size",
            "kda_status_string", "kda_last_error", "kda_version",
            "gdn_chunk_fwd", "gdn_decode_step", "kda_layer_chunk_fwd",
            "kda_layer_decode_step", "kda_chunk_bwd", "kda_chunk_bwd_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in kda.h but not exported"


def test_version_and_status_strings(lib):
    assert lib.kda_version() == 150
    for code, name in [(0, b"KDA_OK"), (1, b"KDA_ERR_INVALID_ARG"), (2, b"KDA_ERR_UNSUPPORTED"),
                       (3, b"KDA_ERR_WORKSPACE"), (4, b"KDA_ERR_HIP")]:
        assert lib.kda_status_string(code) == name


def test_workspace_size(lib):
    ws = lib.kda_chunk_fwd_workspace_size
    # one package per (chunk, head); 4096 tokens, 64-token chunks, 32 heads
    per = ws(1, 4096, 32, 128, 128, 0, BF16, 64) // (64 * 32)
    assert per * 64 * 32 == ws(1, 4096, 32, 128, 128, 0, BF16, 64)
    assert per >= 2 * 64 * 128 * 2 + 128 * 64 * 2 + 2 * 64 * 128 * 4 + 128 * 4
    assert ws(1, 4096, 32, 128, 128, 0, BF16, 0) == ws(1, 4096, 32, 128, 128, 0, BF16, 64)
    # a partial chunk still takes a slot; varlen reserves one extra slot per sequence
    assert ws(1, 4097, 1, 16, 16, 0, F32, 16) == ws(1, 4112, 1, 16, 16, 0, F32, 16)
    assert ws(1, 1000, 2, 64, 64, 5, BF16, 64) > ws(1, 1000, 2, 64, 64, 0, BF16, 64)
    assert ws(3, 100, 2, 32, 32, 0, BF16, 32) == 3 * ws(1, 100, 2, 32, 32, 0, BF16, 32)
    # d_k and d_v are independent: the package grows with each
    assert ws(1, 64, 1, 16, 32, 0, BF16, 16) > ws(1, 64, 1, 16, 16, 0, BF16, 16)
    assert ws(1, 64, 1, 32, 16, 0, BF16, 16) > ws(1, 64, 1, 16, 16, 0, BF16, 16)
    for bad in [(1, 64, 1, 16, 16, 0, BF16, 48), (1, 64, 1, 24, 24, 0, BF16, 16),
                (1, 64, 1, 16, 24, 0, BF16, 16), (0, 64, 1, 16, 16, 0, BF16, 16),
                (1, -1, 1, 16, 16, 0, BF16, 16), (1, 64, 1, 16, 16, 0, 7, 16)]:
        assert ws(*bad) == 0, bad


def _chunk(lib, fn="kda_chunk_fwd", **kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, log_alpha=FAKE + 0x3000000,
             beta=FAKE + 0x4000000, init_state=None, cu_seqlens=None, B=1, T=64, H=1, Dk=16,
             Dv=16, n_seqs=0, dtype=BF16, chunk=16, o=FAKE + 0x5000000, final_state=None,
             ws=FAKE + 0x6000000, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return getattr(lib, fn)(p(a["q"]), p(a["k"]), p(a["v"]), p(a["log_alpha"]), p(a["beta"]),
                            p(a["init_state"]), p(a["cu_seqlens"]), a["B"], a["T"], a["H"],
                            a["Dk"], a["Dv"], a["n_seqs"], a["dtype"], a["chunk"], p(a["o"]),
                            p(a["final_state"]), p(a["ws"]), a["ws_bytes"], a["stream"])


def test_unit_count_beyond_the_state_grid(lib):
    """The state passes run Dv / 16 workgroups per (sequence, head) unit on a
    one-dimensional grid: more units than it takes are refused before any launch."""
    big = dict(B=1 << 20, T=1, H=1 << 10, Dk=128, Dv=128, chunk=64)  # 2^30 units x 8 slabs
    assert _chunk(lib, **big) == INVALID and b"units" in lib.kda_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), UNSUPPORTED),
    (dict(Dk=24, Dv=24), UNSUPPORTED),
    (dict(Dk=16, Dv=24), UNSUPPORTED),
    (dict(chunk=48), UNSUPPORTED),
    (dict(B=0), INVALID),
    (dict(T=-1), INVALID),
    (dict(H=0), INVALID),
    (dict(q=None), INVALID),
    (dict(o=None), INVALID),
    (dict(k=FAKE + 8), INVALID),                       # misaligned
    (dict(init_state=FAKE + 0x7000004), INVALID),      # misaligned
    (dict(ws=None), WORKSPACE),
    (dict(ws_bytes=16), WORKSPACE),
    (dict(ws=FAKE + 0x6000010), INVALID),              # workspace not 256-byte aligned
    (dict(o=FAKE), INVALID),                           # o aliases q
    (dict(ws=FAKE + 0x4000000), INVALID),              # workspace overlaps beta
    (dict(cu_seqlens=FAKE + 0x8000000, B=2), INVALID),
    (dict(cu_seqlens=FAKE + 0x8000000, n_seqs=0), INVALID),
    (dict(n_seqs=3), INVALID),                         # n_seqs without cu_seqlens
    (dict(final_state=FAKE + 0x5000000), INVALID),     # final_state aliases o
])
@pytest.mark.parametrize("fn", ["kda_chunk_fwd", "gdn_chunk_fwd"])
def test_chunk_fwd_rejects(lib, fn, kw, code):
    assert _chunk(lib, fn, **kw) == code
    assert lib.kda_last_error()  # a detail message is set


def test_chunk_fwd_partial_alias_of_init_state_rejected(lib):
    assert _chunk(lib, init_state=FAKE + 0x7000000, final_state=FAKE + 0x7000100) == INVALID


def _decode(lib, fn="kda_decode_step", **kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, log_alpha=FAKE + 0x3000000,
             beta=FAKE + 0x4000000, state=FAKE + 0x5000000, N=4, H=2, Dk=128, Dv=128,
             dtype=BF16, o=FAKE + 0x6000000, stream=None)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return getattr(lib, fn)(p(a["q"]), p(a["k"]), p(a["v"]), p(a["log_alpha"]), p(a["beta"]),
                            p(a["state"]), a["N"], a["H"], a["Dk"], a["Dv"], a["dtype"],
                            p(a["o"]), a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=9), UNSUPPORTED),
    (dict(Dk=8), UNSUPPORTED),
    (dict(Dv=256), UNSUPPORTED),
    (dict(N=-1), INVALID),
    (dict(H=0), INVALID),
    (dict(state=None), INVALID),
    (dict(beta=FAKE + 0x4000002), INVALID),   # beta needs 4-byte alignment only
    (dict(q=FAKE + 4), INVALID),
    (dict(o=FAKE + 0x5000000), INVALID),   # o aliases the state
    (dict(state=FAKE + 0x1000000), INVALID),  # state aliases k
])
@pytest.mark.parametrize("fn", ["kda_decode_step", "gdn_decode_step"])
def test_decode_rejects(lib, fn, kw, code):
    assert _decode(lib, fn, **kw) == code


def test_beta_and_cu_seqlens_need_only_natural_alignment(lib):
    # both still fail later validation on purpose (workspace missing), which
    # shows the alignment checks accepted them
    assert _chunk(lib, beta=FAKE + 0x4000004, ws=None) == WORKSPACE
    assert _chunk(lib, cu_seqlens=FAKE + 0x8000004, n_seqs=2, ws=None) == WORKSPACE
    assert _chunk(lib, beta=FAKE + 0x4000002) == INVALID


def test_empty_decode_is_a_no_op(lib):
    # N = 0: nothing to do, no pointer is touched and no HIP call is made
    assert _decode(lib, N=0, q=None, k=None, v=None, state=None, o=None) == OK


def test_gdn_gate_layout_and_alignment(lib):
    """GDN gates are [B, T, H] / [N, H] fp32 read one by one: 4-byte alignment
    suffices (the calls below then fail a later check on purpose, so no kernel
    is launched), 2-byte does not, and the gate's extent is T*H (or N*H)
    elements, not T*H*Dk."""
    assert _chunk(lib, "gdn_chunk_fwd", log_alpha=FAKE + 0x3000004, ws=None) == WORKSPACE
    assert _chunk(lib, "gdn_chunk_fwd", log_alpha=FAKE + 0x3000002) == INVALID
    assert _chunk(lib, "kda_chunk_fwd", log_alpha=FAKE + 0x3000004) == INVALID
    # o right after a [64, 1] gate: overlaps a KDA gate [64, 1, 16], not a GDN one
    assert _chunk(lib, "kda_chunk_fwd", o=FAKE + 0x3000000 + 256, ws=None) == WORKSPACE
    assert _chunk(lib, "kda_chunk_fwd", o=FAKE + 0x3000000 + 256) == INVALID
    assert b"o overlaps log_alpha" in lib.kda_last_error()
    # decode: accepted alignment, then the o/state alias is what is reported
    assert _decode(lib, "gdn_decode_step", log_alpha=FAKE + 0x3000004, o=FAKE + 0x5000000) == INVALID
    assert b"o overlaps state" in lib.kda_last_error()
    assert _decode(lib, "kda_decode_step", log_alpha=FAKE + 0x3000004) == INVALID
    assert b"log_alpha is not 16-byte aligned" in lib.kda_last_error()
    # gdn decode: state right after an [N, H] gate (4 x 2 floats) is no overlap,
    # so the o/state alias is reported instead
    assert _decode(lib, "gdn_decode_step", state=FAKE + 0x3000000 + 32, o=FAKE + 0x3000000 + 32) == INVALID
    assert b"o overlaps state" in lib.kda_last_error()
    assert _decode(lib, "kda_decode_step", state=FAKE + 0x3000000 + 32) == INVALID
    assert b"state overlaps log_alpha" in lib.kda_last_error()


def _layer_chunk(lib, **kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, xa=FAKE + 0x3000000, xb=FAKE + 0x4000000,
             g=FAKE + 0x5000000, w=FAKE + 0x6000000, l2=1e-6, ne=1e-5, init_state=None, cu_seqlens=None,
             B=1, T=64, H=1, Dk=128, Dv=128, n_seqs=0, o=FAKE + 0x7000000, final_state=None,
             ws=FAKE + 0x8000000, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.kda_layer_chunk_fwd(p(a["q"]), p(a["k"]), p(a["v"]), p(a["xa"]), p(a["xb"]), p(a["g"]),
                                   p(a["w"]), ctypes.c_float(a["l2"]), ctypes.c_float(a["ne"]),
                                   p(a["init_state"]), p(a["cu_seqlens"]), a["B"], a["T"], a["H"], a["Dk"],
                                   a["Dv"], a["n_seqs"], p(a["o"]), p(a["final_state"]), p(a["ws"]),
                                   a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(Dk=64, Dv=64), UNSUPPORTED, b"128"),
    (dict(l2=-1.0), INVALID, b"eps"),
    (dict(ne=float("nan")), INVALID, b"eps"),
    (dict(ne=float("inf")), INVALID, b"eps"),
    (dict(xa=None), INVALID, b"x_alpha is NULL"),
    (dict(w=None), INVALID, b"norm_weight is NULL"),
    (dict(xa=FAKE + 0x3000008), INVALID, b"x_alpha is not 16-byte aligned"),
    (dict(xb=FAKE + 0x4000001), INVALID, b"x_beta is not 2-byte aligned"),
    (dict(g=FAKE + 0x5000004), INVALID, b"out_gate is not 16-byte aligned"),
    (dict(o=FAKE + 0x5000000), INVALID, b"o overlaps out_gate"),
    (dict(ws=None), WORKSPACE, b"workspace"),
    (dict(xb=FAKE + 0x4000002, ws=None), WORKSPACE, b"workspace"),  # x_beta: 2-byte alignment suffices
])
def test_layer_chunk_rejects(lib, kw, code, msg):
    assert _layer_chunk(lib, **kw) == code
    assert msg in lib.kda_last_error()


def test_layer_workspace_size(lib):
    """The layer's workspace is the prefill's plus its row-norm exchange: 4 KiB
    per (chunk slot, head); a prefill-sized workspace is refused."""
    lws, ws = lib.kda_layer_chunk_fwd_workspace_size, lib.kda_chunk_fwd_workspace_size
    for B, T, H, n in [(1, 4096, 32, 0), (1, 157, 3, 0), (2, 100, 4, 0), (1, 1000, 2, 5)]:
        slots = (T + 63) // 64 * B + (n if n else 0)
        assert lws(B, T, H, n) == ws(B, T, H, 128, 128, n, BF16, 64) + slots * H * 4096, (B, T, H, n)
    assert lws(0, 64, 1, 0) == 0 and lws(1, -1, 1, 0) == 0 and lws(1, 64, 0, 0) == 0
    small = ws(1, 64, 1, 128, 128, 0, BF16, 64)
    assert _layer_chunk(lib, ws_bytes=small) == WORKSPACE


def test_layer_decode_rejects(lib):
    p = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(N=4, Dk=128, l2=1e-6, xb=FAKE + 0x4000000, o=FAKE + 0x7000000):
        return lib.kda_layer_decode_step(p(FAKE), p(FAKE + 0x1000000), p(FAKE + 0x2000000),
                                         p(FAKE + 0x3000000), p(xb), p(FAKE + 0x5000000),
                                         p(FAKE + 0x6000000), ctypes.c_float(l2), ctypes.c_float(1e-5),
                                         p(FAKE + 0x8000000), N, 2, Dk, 128, p(o), None)
    assert call(Dk=8) == UNSUPPORTED
    assert call(l2=-0.5) == INVALID
    assert call(xb=FAKE + 0x4000001) == INVALID and b"x_beta" in lib.kda_last_error()
    assert call(o=FAKE + 0x8000000) == INVALID and b"o overlaps state" in lib.kda_last_error()
    assert call(N=0) == OK


def test_bwd_workspace_size(lib):
    fws, bws = lib.kda_chunk_fwd_workspace_size, lib.kda_chunk_bwd_workspace_size
    st = 32 * 128 * 128 * 4  # one fp32 state per head, H = 32, d = 128
    # within one segment (16384 (chunk, head) items: 512 chunks at H = 32) the
    # workspace holds every chunk's package and two fp32 states per (chunk, head)
    a = bws(1, 4096, 32, 128, 128, 0, BF16, 64)
    b = bws(1, 8192, 32, 128, 128, 0, BF16, 64)
    assert b - a == (fws(1, 8192, 32, 128, 128, 0, BF16, 64) - fws(1, 4096, 32, 128, 128, 0, BF16, 64)) + 2 * 64 * st
    assert a > fws(1, 4096, 32, 128, 128, 0, BF16, 64) + 2 * 64 * st
    # past one segment it holds one segment's packages and states, one
    # checkpoint per further segment and two carries: 1M tokens are 32
    # segments of 512 chunks, 2M tokens 64
    seg = bws(1, 512 * 64, 32, 128, 128, 0, BF16, 64)
    m1 = bws(1, 1 << 20, 32, 128, 128, 0, BF16, 64)
    m2 = bws(1, 1 << 21, 32, 128, 128, 0, BF16, 64)
    assert m1 == seg + 31 * st + 2 * st
    assert m2 - m1 == 32 * st
    assert m1 < 5 * 2**30 < fws(1, 1 << 20, 32, 128, 128, 0, BF16, 64)
    # the segment is 16384 items at any H: H = 64 takes 256 chunks per segment
    assert bws(1, 1 << 20, 64, 128, 128, 0, BF16, 64) == bws(1, 256 * 64, 64, 128, 128, 0, BF16, 64) + 65 * 2 * st
    for bad in [(1, 64, 1, 16, 32, 0, BF16, 16), (1, 64, 1, 24, 24, 0, BF16, 16), (1, 64, 1, 16, 16, 0, BF16, 48),
                (0, 64, 1, 16, 16, 0, BF16, 16), (1, 64, 1, 16, 16, 0, 7, 16)]:
        assert bws(*bad) == 0, bad


def _bwd(lib, **kw):
    base = FAKE
    a = dict(q=base, k=base + 0x1000000, v=base + 0x2000000, log_alpha=base + 0x3000000,
             beta=base + 0x4000000, init_state=None, cu_seqlens=None, B=1, T=64, H=1, Dk=16, Dv=16,
             n_seqs=0, dtype=BF16, chunk=16, d_o=base + 0x5000000, d_final=None, dq=base + 0x6000000,
             dk=base + 0x7000000, dv=base + 0x8000000, dla=base + 0x9000000, dbeta=base + 0xa000000,
             ds0=None, ws=base + 0x10000000, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.kda_chunk_bwd(p(a["q"]), p(a["k"]), p(a["v"]), p(a["log_alpha"]), p(a["beta"]),
                             p(a["init_state"]), p(a["cu_seqlens"]), a["B"], a["T"], a["H"], a["Dk"], a["Dv"],
                             a["n_seqs"], a["dtype"], a["chunk"], p(a["d_o"]), p(a["d_final"]), p(a["dq"]),
                             p(a["dk"]), p(a["dv"]), p(a["dla"]), p(a["dbeta"]), p(a["ds0"]), p(a["ws"]),
                             a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(Dk=16, Dv=32), UNSUPPORTED, b"Dk = Dv"),
    (dict(Dk=24, Dv=24), UNSUPPORTED, b"Dk = Dv"),
    (dict(dtype=5), UNSUPPORTED, b"in_dtype"),
    (dict(chunk=48), UNSUPPORTED, b"chunk_size"),
    (dict(H=0), INVALID, b"H=0"),
    (dict(d_o=None), INVALID, b"d_o is NULL"),
    (dict(dq=None), INVALID, b"dq is NULL"),
    (dict(dbeta=FAKE + 0xa000002), INVALID, b"dbeta is not 4-byte aligned"),
    (dict(dk=FAKE + 0x7000008), INVALID, b"dk is not 16-byte aligned"),
    (dict(dq=FAKE + 0x5000000), INVALID, b"dq overlaps d_o"),
    (dict(dv=FAKE + 0x6000000), INVALID, b"dv overlaps dq"),
    (dict(ds0=FAKE + 0x3000000), INVALID, b"d_init_state overlaps log_alpha"),
    (dict(ws=FAKE + 0x9000000), INVALID, b"overlaps the workspace"),
    (dict(ws=None), WORKSPACE, b"workspace"),
    (dict(ws_bytes=1024), WORKSPACE, b"workspace"),
    (dict(ws=FAKE + 0x10000010), INVALID, b"256-byte"),
])
def test_chunk_bwd_rejects(lib, kw, code, msg):
    assert _bwd(lib, **kw) == code
    assert msg in lib.kda_last_error()


def test_dplr_workspace_size(lib):
    ws = lib.kda_dplr_chunk_fwd_workspace_size
    kda_ws = lib.kda_chunk_fwd_workspace_size
    per = ws(1, 4096, 32, 128, 0, BF16, 64) // (64 * 32)
    assert per * 64 * 32 == ws(1, 4096, 32, 128, 0, BF16, 64)
    # W and Q' (fp16), [A-tilde; K-tilde] (fp16, 2 x 64 tokens), U', O_intra, Gamma_last
    assert per >= 2 * 64 * 128 * 2 + 128 * 128 * 2 + 2 * 64 * 128 * 4 + 128 * 4
    # ... and V's rows for the state pass, kept in bf16 as given: 144 KiB in all
    assert per == 2 * 64 * 128 * 2 + 128 * 128 * 2 + 2 * 64 * 128 * 4 + 512 + 64 * 128 * 2
    assert ws(1, 4096, 32, 128, 0, BF16, 64) > kda_ws(1, 4096, 32, 128, 128, 0, BF16, 64)
    assert ws(1, 4096, 32, 128, 0, BF16, 0) == ws(1, 4096, 32, 128, 0, BF16, 64)
    assert ws(1, 1000, 2, 64, 5, BF16, 64) > ws(1, 1000, 2, 64, 0, BF16, 64)
    for bad in [(1, 64, 1, 16, 0, BF16, 48), (1, 64, 1, 24, 0, BF16, 16), (0, 64, 1, 16, 0, BF16, 16),
                (1, -1, 1, 16, 0, BF16, 16), (1, 64, 1, 16, 0, 7, 16)]:
        assert ws(*bad) == 0, bad


def _dplr(lib, **kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, a=FAKE + 0x3000000, b=FAKE + 0x4000000,
             log_alpha=FAKE + 0x5000000, init_state=None, cu_seqlens=None, B=1, T=64, H=1, D=16, n_seqs=0,
             dtype=BF16, chunk=16, o=FAKE + 0x6000000, final_state=None, ws=FAKE + 0x8000000,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.kda_dplr_chunk_fwd(p(a["q"]), p(a["k"]), p(a["v"]), p(a["a"]), p(a["b"]), p(a["log_alpha"]),
                                  p(a["init_state"]), p(a["cu_seqlens"]), a["B"], a["T"], a["H"], a["D"],
                                  a["n_seqs"], a["dtype"], a["chunk"], p(a["o"]), p(a["final_state"]),
                                  p(a["ws"]), a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(D=24), UNSUPPORTED, b"Dk=24"),
    (dict(dtype=5), UNSUPPORTED, b"in_dtype"),
    (dict(chunk=48), UNSUPPORTED, b"chunk_size"),
    (dict(H=0), INVALID, b"H=0"),
    (dict(a=None), INVALID, b"a is NULL"),
    (dict(b=None), INVALID, b"b is NULL"),
    (dict(log_alpha=None), INVALID, b"log_alpha is NULL"),
    (dict(b=FAKE + 0x4000008), INVALID, b"b is not 16-byte aligned"),
    (dict(o=FAKE + 0x3000000), INVALID, b"o overlaps a"),
    (dict(ws=FAKE + 0x4000000), INVALID, b"workspace overlaps b"),
    (dict(ws=None), WORKSPACE, b"workspace"),
    (dict(ws_bytes=1024), WORKSPACE, b"workspace"),
])
def test_dplr_chunk_fwd_rejects(lib, kw, code, msg):
    assert _dplr(lib, **kw) == code
    assert msg in lib.kda_last_error()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(D=24), UNSUPPORTED, b"Dk=24"),
    (dict(dtype=5), UNSUPPORTED, b"in_dtype"),
    (dict(H=0), INVALID, b"H=0"),
    (dict(a=None), INVALID, b"a is NULL"),
    (dict(b=FAKE + 0x4000008), INVALID, b"b is not 16-byte aligned"),
    (dict(log_alpha=None), INVALID, b"log_alpha is NULL"),
    (dict(o=FAKE + 0x3000000), INVALID, b"overlaps"),
])
def test_dplr_decode_rejects(lib, kw, code, msg):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, a=FAKE + 0x3000000, b=FAKE + 0x4000000,
             log_alpha=FAKE + 0x5000000, state=FAKE + 0x6000000, N=4, H=2, D=16, dtype=BF16,
             o=FAKE + 0x8000000, stream=None)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    rc = lib.kda_dplr_decode_step(p(a["q"]), p(a["k"]), p(a["v"]), p(a["a"]), p(a["b"]), p(a["log_alpha"]),
                                  p(a["state"]), a["N"], a["H"], a["D"], a["dtype"], p(a["o"]), a["stream"])
    assert rc == code
    assert msg in lib.kda_last_error()


@pytest.mark.parametrize("fn", ["kda_chunk_fwd", "gdn_chunk_fwd", "kda_dplr_chunk_fwd"])
def test_empty_varlen_needs_no_workspace(lib, fn):
    """T = 0 with cu_seqlens: every sequence is empty, so the call only copies
    init_state to final_state and never touches the workspace (which may be
    NULL or small).  Validation passes; with no GPU here the launch itself then
    reports KDA_ERR_HIP, never KDA_ERR_WORKSPACE or an argument error."""
    kw = dict(T=0, cu_seqlens=FAKE + 0x8000000, n_seqs=3, final_state=FAKE + 0x9000000, ws=None, ws_bytes=0)
    rc = _dplr(lib, **kw) if fn == "kda_dplr_chunk_fwd" else _chunk(lib, fn, **kw)
    assert rc in (OK, 4), lib.kda_last_error()
    # a small workspace placed right below final_state is not taken to overlap it at T = 0
    kw.update(ws=FAKE + 0x9000000 - 256, ws_bytes=256)
    rc = _dplr(lib, **kw) if fn == "kda_dplr_chunk_fwd" else _chunk(lib, fn, **kw)
    assert rc in (OK, 4), lib.kda_last_error()
    # with tokens the workspace is required again
    kw.update(T=64, ws=None, ws_bytes=0)
    rc = _dplr(lib, **kw) if fn == "kda_dplr_chunk_fwd" else _chunk(lib, fn, **kw)
    assert rc == WORKSPACE


def _noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, log_alpha=FAKE + 0x3000000,
             beta=FAKE + 0x4000000, init_state=None, cu_seqlens=None, B=1, T=64, H=1, Dk=16,
             Dv=16, n_seqs=0, dtype=BF16, chunk=16, o=FAKE + 0x5000000, final_state=None, stream=None)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.kda_chunk_fwd_noalloc(p(a["q"]), p(a["k"]), p(a["v"]), p(a["log_alpha"]), p(a["beta"]),
                                     p(a["init_state"]), p(a["cu_seqlens"]), a["B"], a["T"], a["H"],
                                     a["Dk"], a["Dv"], a["n_seqs"], a["dtype"], a["chunk"], p(a["o"]),
                                     p(a["final_state"]), a["stream"])


def test_noalloc_entry_limits_and_validation(lib):
    """kda_chunk_fwd_noalloc: sizes whose workspace exceeds the static scratch
    are refused on the host (KDA_ERR_WORKSPACE, before any HIP call); other
    argument errors are the ones kda_chunk_fwd reports."""
    cap = lib.kda_chunk_fwd_noalloc_max_workspace()
    assert cap == 256 << 20
    ws = lib.kda_chunk_fwd_workspace_size
    assert ws(1, 4096, 32, 128, 128, 0, BF16, 64) <= cap < ws(1, 8192, 32, 128, 128, 0, BF16, 64)
    assert _noalloc(lib, T=8192, H=32, Dk=128, Dv=128, chunk=64) == WORKSPACE
    assert b"static scratch" in lib.kda_last_error()
    assert _noalloc(lib, q=None) == INVALID
    assert _noalloc(lib, Dk=24) == UNSUPPORTED
    assert _noalloc(lib, o=FAKE) == INVALID  # o aliases q
    # a valid call passes validation; with no GPU here the scratch lookup then fails
    assert _noalloc(lib) == 4
    assert b"static scratch" in lib.kda_last_error()
