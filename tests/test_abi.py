"""Host-only checks of the C ABI (no GPU needed).

Every error path of titans_mem_forward / titans_mem_retrieve is detected on
the host before anything is enqueued, so each case below passes fake
(aligned, never dereferenced) device addresses with exactly one defect.
"""
import ctypes
import re

import pytest

from test_learned_neural_amd import titans_mem as tmm

HEADER = __import__("os").path.join(__import__("os").path.dirname(__file__), "..", "include", "titans_mem.h")

BASE = 0x7f0000000000  # fake device addresses: never dereferenced


@pytest.fixture(scope="module")
def lib():
    return tmm.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(titans_mem_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == sorted(tmm.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.titans_mem_abi_version() == tmm.ABI_VERSION


def test_param_count_and_paths(lib):
    d3 = tmm.make_desc(8, 16, 16384, 64, 256, 2, "bf16")
    assert tmm.param_count(d3) == 2 * 64 * 256
    d5 = tmm.make_desc(4, 8, 32768, 128, 512, 4, "bf16")
    assert tmm.param_count(d5) == 128 * 512 + 2 * 512 * 512 + 512 * 128
    d1 = tmm.make_desc(1, 1, 1024, 64, 0, 1, "f32")
    assert tmm.param_count(d1) == 64 * 64
    assert tmm.select_path(d1, 16) == tmm.PATH_GENERIC_F32
    # the deep-memory matrix-core path: bf16 MLPs with widths a multiple of 64, chunks 1..256, N >= 1
    assert tmm.select_path(d5, 128) == tmm.PATH_DEEP_BF16
    assert tmm.select_path(d5, 256) == tmm.PATH_DEEP_BF16
    assert tmm.select_path(d5, 257) == tmm.PATH_GENERIC_F32
    assert tmm.select_path(tmm.make_desc(4, 8, 32768, 128, 512, 4, "f32"), 128) == tmm.PATH_GENERIC_F32
    assert tmm.select_path(tmm.make_desc(4, 8, 32768, 128, 500, 4, "bf16"), 128) == tmm.PATH_GENERIC_F32
    assert tmm.select_path(tmm.make_desc(4, 8, 0, 128, 512, 4, "bf16"), 128) == tmm.PATH_GENERIC_F32
    assert tmm.select_path(tmm.make_desc(4, 8, 32768, 128, 512, 4, "bf16", flags=tmm.FLAG_FORCE_GENERIC),
                           128) == tmm.PATH_GENERIC_F32
    # its workspace: the same bytes per stream whatever the stream count, at least the fp32 state's
    # three rotating (W, S) slots, and a single short chunk needs no more than a full one
    w5 = tmm.workspace_bytes(d5, 128)
    assert w5 > 0 and w5 % 32 == 0
    assert tmm.workspace_bytes(tmm.make_desc(2, 8, 32768, 128, 512, 4, "bf16"), 128) * 2 == w5
    assert w5 // 32 >= 3 * 2 * 4 * tmm.param_count(d5)
    assert tmm.workspace_bytes(tmm.make_desc(4, 8, 100, 128, 512, 4, "bf16"), 128) <= w5
    assert tmm.select_path(d3, 0) == tmm.ERR_INVALID
    forced = tmm.make_desc(8, 16, 16384, 64, 256, 2, "bf16", flags=tmm.FLAG_FORCE_GENERIC)
    assert tmm.select_path(forced, 64) == tmm.PATH_GENERIC_F32
    # the MFMA kernel serves both read modes of the 2-layer d=64 h=256 bf16 memory, chunks 1..64
    for rm in (0, 1):
        d = tmm.make_desc(8, 16, 16384, 64, 256, 2, "bf16", read_mode=rm)
        assert tmm.select_path(d, 64) == tmm.PATH_MLP2_D64_H256
        assert tmm.select_path(d, 1) == tmm.PATH_MLP2_D64_H256
        assert tmm.select_path(d, 65) == tmm.PATH_DEEP_BF16
    assert tmm.select_path(tmm.make_desc(8, 16, 16384, 64, 256, 2, "f32"), 64) == tmm.PATH_GENERIC_F32
    assert tmm.workspace_bytes(d1, 16) > 0


@pytest.mark.parametrize("field,value", [("abi_version", 2), ("B", 0), ("H", -1), ("N", -1), ("d", 0),
                                         ("n_layers", 0), ("activation", 3), ("io_dtype", 7),
                                         ("read_mode", 5), ("flags", 0x80)])
def test_invalid_descriptor(lib, field, value):
    d = tmm.make_desc(2, 2, 64, 16, 32, 2, "f32")
    setattr(d, field, value)
    assert tmm.param_count(d) == tmm.ERR_INVALID
    assert tmm.select_path(d, 16) == tmm.ERR_INVALID
    assert tmm.workspace_bytes(d, 16) == tmm.ERR_INVALID


def test_hidden_required_for_mlp(lib):
    d = tmm.make_desc(1, 1, 8, 16, 32, 2, "f32")
    d.hidden = 0
    assert tmm.param_count(d) == tmm.ERR_INVALID
    d = tmm.make_desc(1, 1, 8, 16, 0, 1, "f32")
    assert tmm.param_count(d) == 256  # hidden ignored for the matrix memory


def test_too_many_layers_is_unsupported(lib):
    d = tmm.make_desc(1, 1, 8, 16, 32, 9, "f32")
    assert tmm.param_count(d) == tmm.ERR_UNSUPPORTED


class Buffers:
    """Disjoint fake device ranges laid out for one descriptor."""

    def __init__(self, desc, chunk):
        esz = 2 if desc.io_dtype == tmm.IO_BF16 else 4
        S = desc.B * desc.H
        P = tmm.param_count(desc)
        sizes = dict(k=S * desc.N * desc.d * esz, v=S * desc.N * desc.d * esz, q=S * desc.N * desc.d * esz,
                     alpha=S * desc.N * 4, eta=S * desc.N * 4, theta=S * desc.N * 4,
                     W_in=S * P * 4, S_in=S * P * 4, y=S * desc.N * desc.d * esz, W_out=S * P * 4,
                     S_out=S * P * 4, ws=max(tmm.workspace_bytes(desc, chunk), 16))
        self.ptr = {}
        cur = BASE
        for name, n in sizes.items():
            self.ptr[name] = cur
            cur += (n + 4095) // 4096 * 4096 + 4096
        self.ws_bytes = tmm.workspace_bytes(desc, chunk)

    def call(self, desc, chunk, **over):
        p = dict(self.ptr)
        ws_bytes = over.pop("ws_bytes", self.ws_bytes)
        p.update(over)
        return tmm.raw_forward(desc, p["k"], p["v"], p["q"], p["alpha"], p["eta"], p["theta"],
                               p["W_in"], p["S_in"], chunk, p["y"], p["W_out"], p["S_out"], p["ws"],
                               ws_bytes, 0)


@pytest.fixture
def setup(lib):
    desc = tmm.make_desc(2, 3, 100, 16, 32, 2, "f32")
    return desc, Buffers(desc, 8)


@pytest.mark.parametrize("name", ["k", "v", "q", "alpha", "eta", "theta", "W_in", "S_in", "y", "W_out", "S_out"])
def test_null_pointer(setup, name):
    desc, b = setup
    assert b.call(desc, 8, **{name: 0}) == tmm.ERR_INVALID


@pytest.mark.parametrize("name", ["k", "alpha", "W_in", "y", "W_out", "ws"])
def test_misaligned_pointer(setup, name):
    desc, b = setup
    assert b.call(desc, 8, **{name: b.ptr[name] + 4}) == tmm.ERR_INVALID


def test_chunk_must_be_positive(setup):
    desc, b = setup
    assert b.call(desc, 0) == tmm.ERR_INVALID
    assert b.call(desc, -3) == tmm.ERR_INVALID


def test_workspace_too_small(setup):
    desc, b = setup
    assert b.call(desc, 8, ws_bytes=b.ws_bytes - 16) == tmm.ERR_WORKSPACE
    assert b.call(desc, 8, ws=0, ws_bytes=0) == tmm.ERR_WORKSPACE


@pytest.mark.parametrize("a,b_,shift", [("y", "k", 0), ("W_out", "S_in", 0), ("W_out", "W_in", 16),
                                        ("S_out", "W_out", 0), ("ws", "y", 64), ("y", "alpha", 32),
                                        ("S_out", "S_in", 16)])
def test_illegal_aliasing(setup, a, b_, shift):
    desc, b = setup
    assert b.call(desc, 8, **{a: b.ptr[b_] + shift}) == tmm.ERR_ALIAS


def test_chunk_gates_flag(lib):
    """One gate value per chunk is a valid descriptor flag, served by the same paths."""
    d = tmm.make_desc(8, 16, 16384, 64, 256, 2, "bf16", flags=tmm.FLAG_CHUNK_GATES)
    assert tmm.param_count(d) == 2 * 64 * 256
    assert tmm.select_path(d, 64) == tmm.PATH_MLP2_D64_H256
    g = tmm.make_desc(2, 3, 100, 16, 32, 2, "f32", flags=tmm.FLAG_CHUNK_GATES | tmm.FLAG_FORCE_GENERIC)
    assert tmm.select_path(g, 8) == tmm.PATH_GENERIC_F32


def test_chunk_gates_alias_range(lib):
    """With per-chunk gates a gate array spans B*H*ceil(N/chunk) floats: an
    output inside that span is still rejected."""
    desc = tmm.make_desc(2, 3, 100, 16, 32, 2, "f32", flags=tmm.FLAG_CHUNK_GATES)
    b = Buffers(desc, 8)
    span = 2 * 3 * 13 * 4              # 13 chunks of 8 cover 100 tokens (312 bytes)
    assert b.call(desc, 8, y=b.ptr["theta"] + span - 24) == tmm.ERR_ALIAS
    assert b.call(desc, 8, W_out=b.ptr["eta"] + span - 40) == tmm.ERR_ALIAS


def test_empty_sequence_allows_null_token_buffers(lib):
    desc = tmm.make_desc(1, 2, 0, 16, 32, 2, "bf16")
    P = tmm.param_count(desc)
    # a misaligned state pointer still fails: the only defect, detected before launch
    rc = tmm.raw_forward(desc, 0, 0, 0, 0, 0, 0, BASE + 4, BASE + 8192, 4, 0, BASE + 2 * 8192,
                         BASE + 3 * 8192, 0, 0, 0)
    assert rc == tmm.ERR_INVALID
    assert P == 2 * 16 * 32


def test_retrieve_validation(lib):
    import ctypes
    desc = tmm.make_desc(1, 2, 10, 16, 32, 2, "f32")
    f = lib.titans_mem_retrieve
    assert f(ctypes.byref(desc), BASE, 0, BASE + 8192, 0) == tmm.ERR_INVALID
    assert f(ctypes.byref(desc), 0, BASE + 8192, BASE + 16384, 0) == tmm.ERR_INVALID
    assert f(ctypes.byref(desc), BASE, BASE + 65536, BASE + 64, 0) == tmm.ERR_ALIAS
    wide = tmm.make_desc(1, 1, 10, 16, 2048, 2, "f32")
    assert f(ctypes.byref(wide), BASE, BASE + (1 << 24), BASE + (2 << 24), 0) == tmm.ERR_UNSUPPORTED


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, 17):
        assert isinstance(tmm.status_string(code), str) and tmm.status_string(code)
    assert tmm.status_string(tmm.ERR_GAVE_UP) != tmm.status_string(17)


def test_workspace_status_argument_errors(lib):
    """titans_mem_workspace_status checks its arguments on the host before
    touching the device: a bad descriptor, a missing, short or misaligned
    workspace for the MFMA path."""
    f = lib.titans_mem_workspace_status
    d3 = tmm.make_desc(8, 16, 16384, 64, 256, 2, "bf16")
    need = tmm.workspace_bytes(d3, 64)
    assert need > 0
    bad = tmm.make_desc(8, 16, 16384, 64, 256, 2, "bf16")
    bad.abi_version = 2
    assert f(ctypes.byref(bad), 64, BASE, need, 0) == tmm.ERR_INVALID
    assert f(ctypes.byref(d3), 0, BASE, need, 0) == tmm.ERR_INVALID
    assert f(ctypes.byref(d3), 64, BASE, need - 1, 0) == tmm.ERR_WORKSPACE
    assert f(ctypes.byref(d3), 64, BASE + 8, need, 0) == tmm.ERR_INVALID
    # the no-wait test hook is a valid flag; other unknown bits are not
    nw = tmm.make_desc(8, 16, 16384, 64, 256, 2, "bf16", flags=tmm.FLAG_NO_WAIT)
    assert tmm.select_path(nw, 64) == tmm.PATH_MLP2_D64_H256
    assert tmm.select_path(tmm.make_desc(8, 16, 16384, 64, 256, 2, "bf16", flags=8), 64) == tmm.ERR_INVALID


def test_forward_noalloc_argument_errors(lib):
    """The allocation-free forward validates like titans_mem_forward (on
    the host, nothing enqueued) and serves only the MFMA path's shapes."""
    f = lib.titans_mem_forward_noalloc
    d3 = tmm.make_desc(2, 2, 128, 64, 256, 2, "bf16")
    tok, gate, state = 2 * 2 * 128 * 64 * 2, 2 * 2 * 128 * 4, 2 * 2 * 32768 * 4
    ptrs = []
    cur = BASE
    for n in (tok, tok, tok, gate, gate, gate, state, state, tok, state, state):
        ptrs.append(cur)
        cur += (n + 4095) // 4096 * 4096
    k, v, q, a, e, t, Wi, Si, y, Wo, So = ptrs
    call = lambda desc, chunk=64, **kw: f(ctypes.byref(desc), kw.get("k", k), v, q, a, e, t, Wi, Si, chunk, y,
                                          kw.get("Wo", Wo), So, 0)
    assert call(d3, chunk=0) == tmm.ERR_INVALID
    assert call(d3, k=0) == tmm.ERR_INVALID
    assert call(d3, k=k + 8) == tmm.ERR_INVALID
    assert call(d3, Wo=Si) == tmm.ERR_ALIAS
    assert call(tmm.make_desc(2, 2, 128, 64, 256, 2, "bf16"), chunk=65) == tmm.ERR_UNSUPPORTED
    assert call(tmm.make_desc(2, 2, 128, 64, 256, 2, "bf16", flags=tmm.FLAG_FORCE_GENERIC)) == tmm.ERR_UNSUPPORTED
    assert call(tmm.make_desc(2, 2, 128, 64, 0, 1, "f32")) in (tmm.ERR_UNSUPPORTED, tmm.ERR_ALIAS)


# ----------------------------------------------------------------------------
# titans_mem_input (x -> k, v, q and the gates)
# ----------------------------------------------------------------------------
class InputBuffers:
    """Disjoint fake device ranges for one input-side descriptor."""

    def __init__(self, desc):
        R, C = desc.B * desc.N, desc.H * desc.d
        sizes = dict(x=R * desc.D * 2, w_proj=3 * C * desc.D * 2, conv_w=3 * C * desc.conv_width * 4,
                     w_gate=3 * desc.H * desc.D * 2, b_gate=3 * desc.H * 4, k=R * C * 2, v=R * C * 2, q=R * C * 2,
                     alpha=R * desc.H * 4, eta=R * desc.H * 4, theta=R * desc.H * 4)
        self.ptr = {}
        cur = BASE
        for name, n in sizes.items():
            self.ptr[name] = cur
            cur += (n + 4095) // 4096 * 4096 + 4096

    def call(self, desc, **over):
        p = dict(self.ptr)
        p.update(over)
        return tmm.raw_input(desc, p["x"], p["w_proj"], p["conv_w"], p["w_gate"], p["b_gate"], (0.1, 1.0, 0.1),
                             p["k"], p["v"], p["q"], p["alpha"], p["eta"], p["theta"], 0)


@pytest.mark.parametrize("field,value,code", [("abi_version", 3, -1), ("B", 0, -1), ("N", -1, -1), ("D", 0, -1),
                                              ("H", 0, -1), ("d", 0, -1), ("conv_width", 0, -1), ("flags", 1, -1),
                                              ("D", 48, -2), ("d", 48, -2), ("d", 8, -2), ("conv_width", 5, -2),
                                              ("H", 3, -2)])
def test_input_invalid_descriptor(lib, field, value, code):
    desc = tmm.make_input_desc(2, 100, 256, 4, 64, 4)
    b = InputBuffers(desc)
    setattr(desc, field, value)
    assert b.call(desc) == code


@pytest.mark.parametrize("name", ["x", "w_proj", "conv_w", "w_gate", "b_gate", "k", "v", "q", "alpha", "eta",
                                  "theta"])
def test_input_null_and_misaligned(lib, name):
    desc = tmm.make_input_desc(2, 100, 256, 4, 64, 4)
    b = InputBuffers(desc)
    assert b.call(desc, **{name: 0}) == tmm.ERR_INVALID
    assert b.call(desc, **{name: b.ptr[name] + 4}) == tmm.ERR_INVALID


@pytest.mark.parametrize("a,b_,shift", [("k", "x", 0), ("v", "k", 256), ("alpha", "w_gate", 16), ("theta", "eta", 0),
                                        ("q", "conv_w", 32), ("eta", "b_gate", 0)])
def test_input_aliasing(lib, a, b_, shift):
    desc = tmm.make_input_desc(2, 100, 256, 4, 64, 4)
    b = InputBuffers(desc)
    assert b.call(desc, **{a: b.ptr[b_] + shift}) == tmm.ERR_ALIAS


def test_input_empty_sequences(lib):
    desc = tmm.make_input_desc(3, 0, 256, 4, 64, 4)
    assert InputBuffers(desc).call(desc) == tmm.OK


# ----------------------------------------------------------------------------
# titans_mem_backward (gradients through the memory)
# ----------------------------------------------------------------------------
class BackwardBuffers:
    """Disjoint fake device ranges for one backward call."""

    def __init__(self, desc, chunk):
        esz = 2 if desc.io_dtype == tmm.IO_BF16 else 4
        S = desc.B * desc.H
        P = tmm.param_count(desc)
        tok, gates, state = S * desc.N * desc.d, S * desc.N * 4, S * P * 4
        self.ws_bytes = tmm.backward_workspace_bytes(desc, chunk)
        sizes = dict(k=tok * esz, v=tok * esz, q=tok * esz, alpha=gates, eta=gates, theta=gates, W_in=state,
                     S_in=state, dy=tok * 4, dW_out=state, dS_out=state, dk=tok * 4, dv=tok * 4, dq=tok * 4,
                     dalpha=gates, deta=gates, dtheta=gates, dW_in=state, dS_in=state, ws=max(self.ws_bytes, 16))
        self.ptr = {}
        cur = BASE
        for name, n in sizes.items():
            self.ptr[name] = cur
            cur += (n + 4095) // 4096 * 4096 + 4096

    def call(self, desc, chunk, **over):
        p = dict(self.ptr)
        ws_bytes = over.pop("ws_bytes", self.ws_bytes)
        p.update(over)
        names = ("k", "v", "q", "alpha", "eta", "theta", "W_in", "S_in")
        outs = ("dy", "dW_out", "dS_out", "dk", "dv", "dq", "dalpha", "deta", "dtheta", "dW_in", "dS_in")
        return tmm.raw_backward(desc, *[p[n] for n in names], chunk, *[p[n] for n in outs], p["ws"], ws_bytes, 0)


@pytest.fixture
def bsetup(lib):
    desc = tmm.make_desc(2, 3, 50, 16, 32, 2, "f32")
    return desc, BackwardBuffers(desc, 8)


def test_backward_workspace_query(lib):
    d = tmm.make_desc(2, 3, 50, 16, 32, 2, "f32")
    P = tmm.param_count(d)
    nb = tmm.backward_workspace_bytes(d, 8)
    assert nb >= 2 * 3 * 7 * 2 * P * 4      # (W, S) at each of the 7 chunk starts, per stream
    assert tmm.backward_workspace_bytes(d, 0) == tmm.ERR_INVALID
    assert tmm.backward_workspace_bytes(tmm.make_desc(1, 1, 8, 6, 10, 2, "f32"), 4) == tmm.ERR_UNSUPPORTED
    assert tmm.backward_workspace_bytes(tmm.make_desc(1, 1, 8, 16, 2048, 2, "f32"), 4) == tmm.ERR_UNSUPPORTED
    assert tmm.backward_workspace_bytes(tmm.make_desc(1, 1, 8000, 16, 32, 2, "f32"), 4097) == tmm.ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["k", "v", "q", "alpha", "eta", "theta", "W_in", "S_in", "dk", "dv", "dq",
                                  "dalpha", "deta", "dtheta", "dW_in", "dS_in"])
def test_backward_required_pointers(bsetup, name):
    desc, b = bsetup
    assert b.call(desc, 8, **{name: 0}) == tmm.ERR_INVALID
    assert b.call(desc, 8, **{name: b.ptr[name] + 4}) == tmm.ERR_INVALID


@pytest.mark.parametrize("name", ["dy", "dW_out", "dS_out"])
def test_backward_optional_adjoints_must_be_aligned(bsetup, name):
    desc, b = bsetup
    assert b.call(desc, 8, **{name: b.ptr[name] + 8}) == tmm.ERR_INVALID


def test_backward_workspace_and_chunk(bsetup):
    desc, b = bsetup
    assert b.call(desc, 8, ws_bytes=b.ws_bytes - 16) == tmm.ERR_WORKSPACE
    assert b.call(desc, 8, ws=0, ws_bytes=0) == tmm.ERR_WORKSPACE
    assert b.call(desc, 0) == tmm.ERR_INVALID


@pytest.mark.parametrize("a,b_,shift", [("dk", "k", 0), ("dW_in", "W_in", 0), ("dS_in", "dW_in", 16),
                                        ("dalpha", "deta", 0), ("ws", "dq", 64), ("dq", "dy", 32)])
def test_backward_aliasing(bsetup, a, b_, shift):
    desc, b = bsetup
    assert b.call(desc, 8, **{a: b.ptr[b_] + shift}) == tmm.ERR_ALIAS
