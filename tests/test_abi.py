"""The C ABI on the CPU: the library loads, exports what include/kda.h declares,
and every invalid argument is rejected by host-only validation with its own
status code.  Pointers here are fake, 16-byte aligned addresses: validation must
never dereference them or call into the HIP runtime."""
import ctypes

import pytest

import gated_delta_rule_80_amd as kda
from gated_delta_rule_80_amd import _lib

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, UNSUP, WS, HIP, VALUE = range(10)


@pytest.fixture(scope="module")
def lib():
    return kda.load()


def test_exports_every_declared_symbol(lib):
    names = kda.declared_functions()
    assert {"kda_prefill", "kda_decode_step", "kda_conv_norm", "kda_prefill_stage",
            "kda_prefill_workspace_bytes", "kda_validate_prefill", "kda_validate_decode",
            "kda_validate_conv_norm", "kda_status_str", "kda_abi_version",
            "kda_prefill_walk_segments", "kda_prefill_state_map",
            "kda_prefill_state_map_workspace_bytes", "kda_training_workspace_bytes",
            "kda_prefill_forward_saved", "kda_prefill_backward_saved"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.kda_abi_version() == 7
    for s in range(11):
        assert kda.kda_status_str(s) and kda.kda_status_str(s) != "unknown status"


class Fake:
    """Disjoint fake device buffers (never dereferenced)."""

    def __init__(self):
        self.next = 0x7F0000000000

    def __call__(self, nbytes=1 << 32):
        p = self.next
        self.next += ((nbytes + 4095) // 4096 + 1) * 4096
        return p


def prefill(**kw):
    f = Fake()
    a = _lib.PrefillArgs()
    a.B, a.T, a.H, a.D, a.chunk, a.conv_k = 2, 100, 4, 128, 64, 4
    a.flags, a.l2_eps, a.scale, a.io = 1, 1e-6, 1.0, _lib.KDA_BF16
    for n in ("q", "k", "v", "g", "beta", "conv_w", "conv_state_in", "S0", "o", "S_T",
              "conv_state_out"):
        setattr(a, n, f())
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def decode(**kw):
    f = Fake()
    a = _lib.DecodeArgs()
    a.B, a.H, a.D, a.conv_k, a.flags, a.l2_eps, a.scale, a.io = 8, 4, 128, 4, 1, 1e-6, 1.0, 0
    for n in ("q", "k", "v", "g", "beta", "conv_w", "conv_state", "S", "o"):
        setattr(a, n, f())
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def conv_norm(**kw):
    f = Fake()
    a = _lib.ConvNormArgs()
    a.B, a.T, a.H, a.D, a.conv_k, a.flags, a.l2_eps, a.io = 2, 50, 4, 64, 4, 1, 1e-6, 0
    for n in ("q", "k", "v", "conv_w", "conv_state_in", "q_out", "k_out", "v_out",
              "conv_state_out"):
        setattr(a, n, f())
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def vp(a):
    return kda.kda_validate_prefill(a)


def test_prefill_valid_and_workspace(lib):
    a = prefill()
    assert vp(a) == OK
    ws = kda.kda_prefill_workspace_bytes(a)
    # 2 x 4 heads x 2 chunks x one 256-byte-aligned record per chunk
    assert ws > 0 and ws % 256 == 0 and ws % (2 * 4 * 2) == 0
    a.io = _lib.KDA_FP32
    a.chunk = 32
    assert vp(a) == OK
    assert kda.kda_prefill_workspace_bytes(prefill(B=0)) == 0


def test_walk_segments_plan(lib):
    """Host-only plan of the split state walk: few long walks are cut into
    segments, walks that fill the GPU are not; the workspace grows by the
    segments' maps and start states."""
    def segs(**kw):
        return lib.kda_prefill_walk_segments(ctypes.byref(prefill(**kw)))
    # 12 heads x 2 value blocks = 24 walks of 1,024 chunks: 10 segments of 103
    assert segs(B=1, T=65536, H=12) == 10
    assert segs(B=1, T=4096, H=12) == 4      # segments of at least 16 chunks
    assert segs(B=1, T=65536, H=96) == 1     # 192 walks
    assert segs(B=1, T=4096, H=96) == 1
    assert segs(B=1, T=1000, H=2) == 1       # 16 chunks
    assert segs(B=1, T=65536, H=2, D=64) == 32
    assert segs(B=1, T=0, H=12) == 1
    assert segs(B=0) == 0
    # packed sequences, and a walk that applies the output stage itself, never split
    f = Fake()
    assert segs(B=1, T=65536, H=12, cu_seqlens=f(), n_seqs=1) == 1
    assert segs(B=1, T=65536, H=2, D=64, o_norm_w=f()) == 1
    nrec = 12 * 1024
    rec = 74240  # one chunk record at C = 64, D = 128, bf16
    head = (256 + 4 * nrec + 255) // 256 * 256
    assert kda.kda_prefill_workspace_bytes(prefill(B=1, T=65536, H=12)) == \
        head + nrec * rec + 12 * (4 * 10 - 3) * 128 * 128 * 4


@pytest.mark.parametrize("field,value,code", [
    ("io", 7, DTYPE),
    ("B", 0, SHAPE), ("H", 0, SHAPE), ("T", -1, SHAPE), ("D", 0, SHAPE), ("chunk", 0, SHAPE),
    ("D", 96, UNSUP), ("D", 256, UNSUP), ("chunk", 48, UNSUP), ("chunk", 128, UNSUP),
    ("conv_k", 3, UNSUP), ("flags", 4, VALUE), ("flags", 1 << 31, VALUE), ("l2_eps", -1.0, VALUE),
    ("l2_eps", float("nan"), VALUE), ("scale", float("inf"), VALUE),
    ("q", None, NULL), ("k", None, NULL), ("v", None, NULL), ("g", None, NULL),
    ("beta", None, NULL), ("o", None, NULL), ("S_T", None, NULL), ("conv_w", None, NULL),
])
def test_prefill_rejects(lib, field, value, code):
    assert vp(prefill(**{field: value})) == code


def test_prefill_fp32_d128_c64_unsupported(lib):
    assert vp(prefill(io=_lib.KDA_FP32, D=128, chunk=64)) == UNSUP


def test_prefill_conv_k0_rules(lib):
    assert vp(prefill(conv_k=0)) == NULL  # filters given without a conv
    assert vp(prefill(conv_k=0, conv_w=None, conv_state_in=None, conv_state_out=None)) == OK


def test_prefill_optional_pointers(lib):
    assert vp(prefill(S0=None)) == OK
    assert vp(prefill(conv_state_in=None, conv_state_out=None)) == OK
    # empty sequences need no input pointers, only the state output
    assert vp(prefill(T=0, q=None, k=None, v=None, g=None, beta=None, o=None)) == OK
    assert kda.kda_prefill_workspace_bytes(prefill(T=0)) == 0


@pytest.mark.parametrize("field", ["q", "k", "v", "g", "beta", "conv_w", "conv_state_in", "S0",
                                   "o", "S_T", "conv_state_out"])
def test_prefill_alignment(lib, field):
    a = prefill()
    setattr(a, field, getattr(a, field) + 8)
    assert vp(a) == ALIGN


def test_prefill_aliasing(lib):
    a = prefill()
    a.o = a.q
    assert vp(a) == ALIAS
    a = prefill()
    a.o = a.S_T
    assert vp(a) == ALIAS
    a = prefill()
    a.S_T = a.S0  # in place is allowed
    assert vp(a) == OK
    a = prefill()
    a.S_T = a.S0 + 256  # partial overlap is not
    assert vp(a) == ALIAS
    a = prefill()
    a.conv_state_out = a.conv_state_in
    assert vp(a) == OK
    a = prefill()
    a.conv_state_out = a.conv_state_in + 1024
    assert vp(a) == ALIAS
    a = prefill()
    a.S_T = a.k + 4096
    assert vp(a) == ALIAS
    a = prefill()
    a.o = a.g + 16  # overlap inside the range
    assert vp(a) == ALIAS


def test_prefill_workspace_errors(lib):
    a = prefill()
    need = kda.kda_prefill_workspace_bytes(a)
    # NULL workspace / too small / misaligned: refused before any launch
    assert lib.kda_prefill(ctypes.byref(a), None, need, None) == WS
    assert lib.kda_prefill(ctypes.byref(a), ctypes.c_void_p(0x100000000000), need - 1, None) == WS
    assert lib.kda_prefill(ctypes.byref(a), ctypes.c_void_p(0x100000000010), need, None) == WS
    # workspace overlapping an output
    assert lib.kda_prefill(ctypes.byref(a), ctypes.c_void_p(a.o), need, None) == ALIAS
    # invalid stage number
    assert lib.kda_prefill_stage(ctypes.byref(a), ctypes.c_void_p(0x100000000000), need, 5,
                                 None) == VALUE
    assert lib.kda_prefill_stage(ctypes.byref(a), ctypes.c_void_p(0x100000000000), need, -1,
                                 None) == VALUE
    # invalid args are reported before the workspace
    b = prefill(io=9)
    assert lib.kda_prefill(ctypes.byref(b), None, 0, None) == DTYPE


def test_prefill_size_overflow(lib):
    assert vp(prefill(B=1 << 30, T=1 << 30)) == SHAPE


@pytest.mark.parametrize("field,value,code", [
    ("io", -1, DTYPE), ("B", 0, SHAPE), ("H", -2, SHAPE), ("D", 48, UNSUP), ("conv_k", 2, UNSUP),
    ("flags", 4, VALUE), ("l2_eps", float("inf"), VALUE), ("scale", float("nan"), VALUE),
    ("q", None, NULL), ("S", None, NULL), ("o", None, NULL), ("conv_state", None, NULL),
    ("conv_w", None, NULL),
])
def test_decode_rejects(lib, field, value, code):
    assert kda.kda_validate_decode(decode(**{field: value})) == code


def test_decode_valid_and_alias(lib):
    assert kda.kda_validate_decode(decode()) == OK
    assert kda.kda_validate_decode(decode(conv_k=0, conv_w=None, conv_state=None)) == OK
    a = decode()
    a.o = a.S + 64
    assert kda.kda_validate_decode(a) == ALIAS
    a = decode()
    a.S = a.q
    assert kda.kda_validate_decode(a) == ALIAS
    a = decode()
    a.conv_state = a.v
    assert kda.kda_validate_decode(a) == ALIAS
    a = decode()
    a.beta += 4
    assert kda.kda_validate_decode(a) == ALIGN


def test_conv_norm_validation(lib):
    assert kda.kda_validate_conv_norm(conv_norm()) == OK
    assert kda.kda_validate_conv_norm(conv_norm(conv_k=0)) == UNSUP
    assert kda.kda_validate_conv_norm(conv_norm(D=24)) == UNSUP
    assert kda.kda_validate_conv_norm(conv_norm(io=3)) == DTYPE
    assert kda.kda_validate_conv_norm(conv_norm(q_out=None)) == NULL
    a = conv_norm()
    a.k_out = a.q_out
    assert kda.kda_validate_conv_norm(a) == ALIAS
    a = conv_norm()
    a.v_out = a.v
    assert kda.kda_validate_conv_norm(a) == ALIAS
    a = conv_norm()
    a.conv_state_out = a.conv_state_in
    assert kda.kda_validate_conv_norm(a) == OK


def test_errors_before_launch_never_touch_hip(lib):
    """A rejected call returns its code from the entry point itself (no device)."""
    a = prefill(D=96)
    assert lib.kda_prefill(ctypes.byref(a), None, 0, None) == UNSUP
    d = decode(B=0)
    assert lib.kda_decode_step(ctypes.byref(d), None) == SHAPE
    c = conv_norm(conv_k=0)
    assert lib.kda_conv_norm(ctypes.byref(c), None) == UNSUP


def test_binding_raises_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load(str(tmp_path / "nope.so"))


# ------------------------------------------------------------ optional stages
def stages(make, **kw):
    """Valid args with every optional stage on (fake, disjoint buffers)."""
    f = Fake()
    f.next = 0x7E0000000000
    a = make()
    a.flags = 1 | 2  # L2 norm + beta logits
    a.A_log, a.dt_bias, a.o_norm_w, a.o_gate = f(), f(), f(), f()
    a.o_norm_eps = 1e-6
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("make,validate", [(prefill, kda.kda_validate_prefill),
                                           (decode, kda.kda_validate_decode)])
def test_stage_arguments(lib, make, validate):
    assert validate(stages(make)) == OK
    # each stage alone
    assert validate(stages(make, A_log=None, dt_bias=None)) == OK
    assert validate(stages(make, o_norm_w=None)) == OK
    assert validate(stages(make, o_gate=None)) == OK
    assert validate(stages(make, flags=1)) == OK
    # A_log and dt_bias come together
    assert validate(stages(make, A_log=None)) == NULL
    assert validate(stages(make, dt_bias=None)) == NULL
    # eps of the output norm is checked only when the norm is on
    assert validate(stages(make, o_norm_eps=float("nan"))) == VALUE
    assert validate(stages(make, o_norm_eps=-1.0)) == VALUE
    assert validate(stages(make, o_norm_eps=float("nan"), o_norm_w=None)) == OK
    for field in ("A_log", "dt_bias", "o_norm_w", "o_gate"):
        a = stages(make)
        setattr(a, field, getattr(a, field) + 4)
        assert validate(a) == ALIGN, field
    # the output may not overlap a stage input, nor may the state
    for field in ("A_log", "dt_bias", "o_norm_w", "o_gate"):
        a = stages(make)
        setattr(a, field, a.o)
        assert validate(a) == ALIAS, field
    a = stages(make)
    a.o_gate = a.S_T if make is prefill else a.S
    assert validate(a) == ALIAS


def test_stage_struct_layout_matches_header():
    """The ctypes structs end with the optional-stage fields in header order."""
    text = open(_lib.HEADER_PATH).read()
    for struct, cls in (("kda_prefill_args", _lib.PrefillArgs), ("kda_decode_args", _lib.DecodeArgs)):
        body = text[text.index("typedef struct " + struct):]
        body = body[:body.index("} " + struct)]
        import re
        body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
        names = re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*[,;]", body)
        assert [n for n, _ in cls._fields_] == names, struct


# ------------------------------------------------------------ packed sequences
def test_packed_arguments(lib):
    f = Fake()
    f.next = 0x7D0000000000
    cu = f()
    a = prefill(B=1, cu_seqlens=cu, n_seqs=5)
    assert vp(a) == OK
    assert vp(prefill(B=2, cu_seqlens=cu, n_seqs=5)) == SHAPE  # packed rows share B = 1
    assert vp(prefill(B=1, cu_seqlens=cu, n_seqs=0)) == SHAPE
    assert vp(prefill(B=1, n_seqs=3)) == SHAPE                 # n_seqs without offsets
    assert vp(prefill(B=1, cu_seqlens=cu + 4, n_seqs=5)) == ALIGN
    b = prefill(B=1, cu_seqlens=cu, n_seqs=5)
    b.cu_seqlens = b.o
    assert vp(b) == ALIAS
    # the workspace holds a head's chunk slots, one more per sequence, and the tables
    w1 = kda.kda_prefill_workspace_bytes(prefill(B=1, cu_seqlens=cu, n_seqs=1))
    w9 = kda.kda_prefill_workspace_bytes(prefill(B=1, cu_seqlens=cu, n_seqs=9))
    plain = kda.kda_prefill_workspace_bytes(prefill(B=1))
    assert plain < w1 < w9
    # T = 0 needs no workspace, packed or not
    assert kda.kda_prefill_workspace_bytes(prefill(B=1, T=0, cu_seqlens=cu, n_seqs=4)) == 0


def test_packed_state_sizes_follow_n_seqs(lib):
    """S_T of a packed call spans n_seqs states: an S_T placed right after S0's
    n_seqs states is fine, one starting inside them overlaps."""
    f = Fake()
    f.next = 0x7C0000000000
    a = prefill(B=1, cu_seqlens=f(), n_seqs=3)
    state = 3 * a.H * a.D * a.D * 4
    a.S_T = a.S0 + state
    assert vp(a) == OK
    a.S_T = a.S0 + state - 256
    assert vp(a) == ALIAS


# -------------------------------------------------------------------- backward
def backward(**kw):
    f = Fake()
    f.next = 0x7B0000000000
    a = _lib.BackwardArgs()
    a.fwd = prefill()
    for n in ("dO", "dS_T", "dq", "dk", "dv", "dg", "dbeta", "dS0", "dconv_w", "dconv_state"):
        setattr(a, n, f())
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_state_map_arguments(lib):
    """The state map's host-side checks: nothing is launched for any of these."""
    f = Fake()
    f.next = 0x7D0000000000  # clear of the argument buffers
    a = prefill(B=1, T=65536, H=12)
    need = kda.kda_prefill_state_map_workspace_bytes(a)
    assert need >= kda.kda_prefill_workspace_bytes(a) > 0
    M, N, ws = f(12 * 128 * 128 * 4), f(12 * 128 * 128 * 4), f(need)

    def sm(args, m=M, n=N, w=ws, nbytes=need):
        return lib.kda_prefill_state_map(ctypes.byref(args), ctypes.c_void_p(w), nbytes,
                                         ctypes.c_void_p(m), ctypes.c_void_p(n), None)
    assert sm(a, m=None) == NULL and sm(a, n=None) == NULL
    assert sm(a, m=M + 4) == ALIGN
    assert sm(a, n=M) == ALIAS and sm(a, m=a.q) == ALIAS and sm(a, n=a.S0) == ALIAS
    assert sm(a, w=M - 256) == ALIAS
    # the workspace against the call's own buffers, over all of its bytes
    assert sm(a, w=a.q) == ALIAS
    tail = (a.S0 - need + 256) // 256 * 256  # only its last bytes reach S0
    assert sm(a, w=tail) == ALIAS
    assert sm(a, nbytes=need - 1) == WS and sm(a, w=ws + 16) == WS and sm(a, w=None) == WS
    assert sm(prefill(B=1, T=64, H=2, cu_seqlens=f(), n_seqs=1)) == UNSUP
    assert sm(prefill(B=0)) == SHAPE
    assert kda.kda_prefill_state_map_workspace_bytes(prefill(B=1, T=0, H=2)) == 0


def test_saved_forward_arguments(lib):
    """Host-side checks of the training pair (nothing is launched)."""
    a = prefill(B=1, T=4096, H=8)
    need = kda.kda_training_workspace_bytes(a)
    assert need >= kda.kda_backward_workspace_bytes(backward(fwd=prefill(B=1, T=4096, H=8))) > 0
    f = Fake()
    f.next = 0x7D0000000000
    ws = f(need)

    def fs(args, w=ws, nbytes=need):
        return lib.kda_prefill_forward_saved(ctypes.byref(args), ctypes.c_void_p(w), nbytes, None)
    assert fs(a, nbytes=need - 1) == WS and fs(a, w=ws + 64) == WS and fs(a, w=None) == WS
    assert fs(a, w=a.q) == ALIAS
    same = prefill(B=1, T=4096, H=8)
    same.conv_state_out = same.conv_state_in
    assert fs(same) == ALIAS
    b = backward(fwd=prefill(B=1, T=4096, H=8))
    b.fwd.conv_state_out = b.fwd.conv_state_in
    assert lib.kda_prefill_backward_saved(ctypes.byref(b), ctypes.c_void_p(ws), need, None) == ALIAS
    # the output stage adds the mixer's output to the workspace
    g = f()
    assert kda.kda_training_workspace_bytes(prefill(B=1, T=4096, H=8, o_gate=g)) > need


def test_backward_workspace_holds_the_forward(lib):
    """The backward's workspace starts with its forward's (records and, when the
    walk splits, the segment maps that the reverse walk reuses) and stays within
    a bounded multiple of it."""
    for kw in (dict(B=1, T=100, H=4), dict(B=1, T=65536, H=12), dict(B=2, T=4096, H=96)):
        fwd = kda.kda_prefill_workspace_bytes(prefill(**kw))
        bwd = kda.kda_backward_workspace_bytes(backward(fwd=prefill(**kw)))
        assert fwd > 0 and fwd < bwd < 40 * fwd, (kw, fwd, bwd)


def test_backward_validation(lib):
    vb = kda.kda_validate_backward
    assert vb(backward()) == OK
    assert kda.kda_backward_workspace_bytes(backward()) > kda.kda_prefill_workspace_bytes(prefill())
    for n in ("dO", "dq", "dk", "dv", "dg", "dbeta", "dconv_w"):
        assert vb(backward(**{n: None})) == NULL, n
    assert vb(backward(dS_T=None, dS0=None, dconv_state=None)) == OK  # optional ones
    a = backward()
    a.dk = a.dq  # outputs may not overlap each other
    assert vb(a) == ALIAS
    a = backward()
    a.dg = a.fwd.g  # nor an input
    assert vb(a) == ALIAS
    a = backward()
    a.dq = a.fwd.o  # nor a forward output
    assert vb(a) == ALIAS
    a = backward()
    a.dbeta += 4
    assert vb(a) == ALIGN
    # the optional stages: their parameters' gradients only with the stage on
    f = Fake()
    f.next = 0x7A0000000000
    a = backward()
    a.fwd.A_log, a.fwd.dt_bias = f(), f()
    assert vb(a) == OK
    a.dA_log, a.ddt_bias = f(), f()
    assert vb(a) == OK
    a.ddt_bias = a.fwd.dt_bias  # may not overlap its parameter
    assert vb(a) == ALIAS
    a = backward()
    a.fwd.o_gate, a.fwd.o_norm_w = f(), f()
    a.do_gate, a.do_norm_w = f(), f()
    assert vb(a) == OK
    a.do_gate = a.dq  # nor another gradient
    assert vb(a) == ALIAS
    a = backward()
    a.fwd.flags = 3
    assert vb(a) == OK
    for n in ("dA_log", "ddt_bias", "do_norm_w", "do_gate"):
        assert vb(backward(**{n: f()})) == NULL, n  # stage off
    a = backward()
    a.fwd.o_gate = f()
    a.do_gate = f() + 4
    assert vb(a) == ALIGN
    # packed sequences: B = 1 and per-sequence states (the forward's rules)
    a = backward()
    a.fwd.B, a.fwd.cu_seqlens, a.fwd.n_seqs = 1, f(), 2
    assert vb(a) == OK
    assert kda.kda_backward_workspace_bytes(a) > 0
    a.fwd.B = 2
    assert vb(a) == SHAPE
    # unsupported modes
    a = backward()
    a.fwd.io, a.fwd.chunk = _lib.KDA_FP32, 32
    assert vb(a) == OK  # fp32 with D = 128 takes C <= 32
    a.fwd.chunk = 64
    assert vb(a) == UNSUP  # as in the forward
    a.fwd.D = 64
    assert vb(a) == OK
    # the forward's own rules still apply
    a = backward()
    a.fwd.D = 96
    assert vb(a) == UNSUP
    # conv_k = 0: no filter or history gradients
    a = backward(dconv_w=None, dconv_state=None)
    a.fwd.conv_k, a.fwd.conv_w, a.fwd.conv_state_in, a.fwd.conv_state_out = 0, None, None, None
    assert vb(a) == OK
    a.dconv_w = f()
    assert vb(a) == NULL
