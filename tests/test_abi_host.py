"""Host-side checks of the C ABI (no GPU needed, no compute call made).

* libpdn.so builds/loads and exports every function include/pdn.h declares;
* the ctypes mirrors have the exact size and field offsets of the C structs
  (a tiny C program compiled with gcc against pdn.h reports them);
* argument validation returns the documented codes before any launch.
"""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_77_amd as pdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pdn.h")
FAKE = 0x10000  # never dereferenced: only *_check entry points see it


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pdn.LIB_PATH):
        from gated_delta_rule_77_amd import build
        build.build()
    return pdn.load_library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pdn_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(pdn.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", pdn.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pdn_[a-z_0-9]+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_abi_version_and_strerror(lib):
    assert pdn.pdn_abi_version() == 5
    # the binding's struct mirrors follow the header's version
    m = re.search(r"#define PDN_ABI_VERSION (\d+)", open(HEADER).read())
    assert int(m.group(1)) == pdn.PDN_ABI_VERSION == pdn.pdn_abi_version()
    for code in (0, -1, -2, -3, -4, -5):
        assert pdn.pdn_strerror(code) and "unknown" not in pdn.pdn_strerror(code)
    assert "unknown" in pdn.pdn_strerror(-99)


def test_struct_layout_matches_header(tmp_path):
    prog = tmp_path / "layout.c"
    fields_c = [f for f, _ in pdn.ChunkFwdArgs._fields_]
    fields_d = [f for f, _ in pdn.DecodeArgs._fields_]
    fields_b = [f for f, _ in pdn.ChunkBwdArgs._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "pdn.h"', 'int main(void){']
    lines.append('printf("bwd %zu\\n", sizeof(pdn_chunk_bwd_args));')
    for f in fields_b:
        lines.append('printf("b.%s %%zu\\n", offsetof(pdn_chunk_bwd_args, %s));' % (f, f))
    lines.append('printf("chunk %zu\\n", sizeof(pdn_chunk_fwd_args));')
    for f in fields_c:
        lines.append('printf("c.%s %%zu\\n", offsetof(pdn_chunk_fwd_args, %s));' % (f, f))
    lines.append('printf("decode %zu\\n", sizeof(pdn_decode_args));')
    for f in fields_d:
        lines.append('printf("d.%s %%zu\\n", offsetof(pdn_decode_args, %s));' % (f, f))
    lines.append("return 0;}")
    prog.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"),
                           str(prog), "-o", str(exe)])
    got = dict(l.split() for l in subprocess.check_output([str(exe)], text=True).splitlines())
    assert int(got["chunk"]) == ctypes.sizeof(pdn.ChunkFwdArgs)
    assert int(got["decode"]) == ctypes.sizeof(pdn.DecodeArgs)
    for f in fields_c:
        assert int(got["c." + f]) == getattr(pdn.ChunkFwdArgs, f).offset, f
    for f in fields_d:
        assert int(got["d." + f]) == getattr(pdn.DecodeArgs, f).offset, f
    assert int(got["bwd"]) == ctypes.sizeof(pdn.ChunkBwdArgs)
    for f in fields_b:
        assert int(got["b." + f]) == getattr(pdn.ChunkBwdArgs, f).offset, f


def _chunk_ok():
    a = pdn.ChunkFwdArgs()
    a.B, a.H, a.T, a.dk, a.dv = 2, 3, 100, 128, 128
    a.qkv_dtype, a.o_dtype = pdn.PDN_BF16, pdn.PDN_F32
    a.q = a.k = a.v = a.o = FAKE
    a.alpha_mode, a.log_alpha = pdn.PDN_ALPHA_VEC, FAKE
    a.beta_mode, a.beta = pdn.PDN_GATE_VEC, FAKE
    a.gamma_mode, a.gamma = pdn.PDN_GATE_VEC, FAKE
    a.precond_eps = -1.0
    a.workspace, a.workspace_bytes = FAKE, 1 << 40  # at least what the call needs
    return a


def _decode_ok():
    a = pdn.DecodeArgs()
    a.B, a.H, a.dk, a.dv = 4, 2, 128, 64
    a.qkv_dtype, a.o_dtype = pdn.PDN_BF16, pdn.PDN_F32
    a.q = a.k = a.v = a.o = a.S = FAKE
    a.alpha_mode, a.log_alpha = pdn.PDN_ALPHA_SCALAR, FAKE
    a.beta_mode, a.beta = pdn.PDN_GATE_SCALAR, FAKE
    a.gamma_mode, a.gamma = pdn.PDN_GAMMA_SAME_AS_BETA, None
    a.precond_eps = -1.0
    return a


def _ccheck(lib, a):
    return lib.pdn_chunk_fwd_check(ctypes.byref(a))


def _dcheck(lib, a):
    return lib.pdn_decode_check(ctypes.byref(a))


def test_valid_arguments_pass_validation(lib):
    assert _ccheck(lib, _chunk_ok()) == pdn.PDN_OK
    assert _dcheck(lib, _decode_ok()) == pdn.PDN_OK


def _ws_size(lib, a):
    n = ctypes.c_size_t(123)
    assert lib.pdn_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(n)) == pdn.PDN_OK
    return n.value


def test_workspace_size_and_check(lib):
    # bf16, dk = 128, per-channel gates: one record of whole KiB per 32-token
    # chunk and (b, h); scalar gates and fp32 inputs need none
    a = _chunk_ok()
    n = _ws_size(lib, a)
    nchunk = a.B * a.H * ((a.T + 31) // 32)
    assert n > 0 and n % (nchunk * 1024) == 0
    a.precond_eps = 1e-6  # adds the per-chunk k.k sums
    assert _ws_size(lib, a) == n + nchunk * 128 * 4
    a.precond_eps = -1.0
    a.T = 33  # ragged tail: two chunks
    assert _ws_size(lib, a) == 2 * a.B * a.H * (n // nchunk)
    a.T = 0
    assert _ws_size(lib, a) == 0
    s = _chunk_ok()
    s.alpha_mode, s.beta_mode, s.gamma_mode = pdn.PDN_ALPHA_SCALAR, pdn.PDN_GATE_SCALAR, pdn.PDN_GATE_SCALAR
    assert _ws_size(lib, s) == 0
    f = _chunk_ok()
    f.qkv_dtype = pdn.PDN_F32
    assert _ws_size(lib, f) == 0
    # asymmetric keys run on the record-based kernels even with scalar gates
    for km in (pdn.PDN_KEY_ERASE_GATE, pdn.PDN_KEY_WRITE_GATE):
        s.key_mode = km
        assert _ws_size(lib, s) == n
    # too small or missing: PDN_EWORKSPACE, before any launch
    a = _chunk_ok()
    a.workspace_bytes = n - 1
    assert _ccheck(lib, a) == pdn.PDN_EWORKSPACE
    assert lib.pdn_chunk_fwd(ctypes.byref(a), None) == pdn.PDN_EWORKSPACE
    a.workspace, a.workspace_bytes = None, 0
    assert _ccheck(lib, a) == pdn.PDN_EWORKSPACE
    a.workspace_bytes = n
    assert _ccheck(lib, a) == pdn.PDN_EWORKSPACE


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "B", 0), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "H", -1), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "T", -5), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "q", None), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "o", None), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "qkv_dtype", 7), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "o_dtype", -1), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "alpha_mode", 9), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "log_alpha", None), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "beta_mode", pdn.PDN_GAMMA_SAME_AS_BETA), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "beta", None), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "gamma", None), pdn.PDN_EINVAL),
    (lambda a: (setattr(a, "gamma_mode", pdn.PDN_GAMMA_SAME_AS_BETA), setattr(a, "dv", 64)),
     pdn.PDN_EINVAL),
    (lambda a: setattr(a, "precond_eps", float("nan")), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "dk", 96), pdn.PDN_EUNSUPPORTED),
    (lambda a: setattr(a, "dv", 40), pdn.PDN_EUNSUPPORTED),
    (lambda a: setattr(a, "dv", 512), pdn.PDN_EUNSUPPORTED),
    (lambda a: (setattr(a, "B", 1 << 20), setattr(a, "H", 1 << 10)), pdn.PDN_EUNSUPPORTED),
    (lambda a: (setattr(a, "B", 1 << 12), setattr(a, "H", 1 << 10), setattr(a, "T", 1 << 15)),
     pdn.PDN_EUNSUPPORTED),  # 2^37 tokens: more than the launch grids can index
    (lambda a: (setattr(a, "S0", FAKE), setattr(a, "ST", FAKE + 64)), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "key_mode", 3), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "key_mode", -1), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "precond_mode", 2), pdn.PDN_EINVAL),
    # stabilised preconditioner: 1 < x <= 2, bf16 with dk = 128 in the prefill
    (lambda a: (setattr(a, "precond_eps", 1e-6), setattr(a, "precond_mode", pdn.PDN_PRECOND_STABILISED),
                setattr(a, "precond_x", 1.0)), pdn.PDN_EINVAL),
    (lambda a: (setattr(a, "precond_eps", 1e-6), setattr(a, "precond_mode", pdn.PDN_PRECOND_STABILISED),
                setattr(a, "precond_x", 2.5)), pdn.PDN_EINVAL),
    (lambda a: (setattr(a, "precond_eps", 1e-6), setattr(a, "precond_mode", pdn.PDN_PRECOND_STABILISED),
                setattr(a, "precond_x", float("nan"))), pdn.PDN_EINVAL),
    (lambda a: (setattr(a, "precond_eps", 1e-6), setattr(a, "precond_mode", pdn.PDN_PRECOND_STABILISED),
                setattr(a, "precond_x", 1.5), setattr(a, "qkv_dtype", pdn.PDN_F32)), pdn.PDN_EUNSUPPORTED),
    # asymmetric keys: bf16 inputs with dk = 128 only
    (lambda a: (setattr(a, "key_mode", pdn.PDN_KEY_ERASE_GATE), setattr(a, "qkv_dtype", pdn.PDN_F32)),
     pdn.PDN_EUNSUPPORTED),
    (lambda a: (setattr(a, "key_mode", pdn.PDN_KEY_WRITE_GATE), setattr(a, "dk", 64),
                setattr(a, "gamma_mode", pdn.PDN_GATE_SCALAR)), pdn.PDN_EUNSUPPORTED),
])
def test_chunk_validation_codes(lib, mutate, code):
    a = _chunk_ok()
    mutate(a)
    assert _ccheck(lib, a) == code
    # the launching entry point returns the same code before touching the GPU
    assert lib.pdn_chunk_fwd(ctypes.byref(a), None) == code


@pytest.mark.parametrize("km", [pdn.PDN_KEY_ERASE_GATE, pdn.PDN_KEY_WRITE_GATE])
def test_chunk_asymmetric_keys_accepted(lib, km):
    a = _chunk_ok()
    a.key_mode = km
    assert _ccheck(lib, a) == pdn.PDN_OK
    a.alpha_mode, a.beta_mode, a.gamma_mode = (pdn.PDN_ALPHA_SCALAR, pdn.PDN_GATE_SCALAR,
                                               pdn.PDN_GAMMA_SAME_AS_BETA)
    assert _ccheck(lib, a) == pdn.PDN_OK
    a.T = 0
    a.q = a.k = a.v = a.o = None
    assert _ccheck(lib, a) == pdn.PDN_OK
    a.qkv_dtype = pdn.PDN_F32  # the shape rule holds for empty sequences too
    assert _ccheck(lib, a) == pdn.PDN_EUNSUPPORTED


def test_chunk_allows_in_place_state(lib):
    a = _chunk_ok()
    a.S0 = a.ST = FAKE
    assert _ccheck(lib, a) == pdn.PDN_OK


def test_chunk_empty_sequence_needs_no_tensors(lib):
    a = _chunk_ok()
    a.T = 0
    a.q = a.k = a.v = a.o = None
    assert _ccheck(lib, a) == pdn.PDN_OK


@pytest.mark.parametrize("mutate,code", [
    (lambda a: setattr(a, "B", 0), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "S", None), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "k", None), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "qkv_dtype", 3), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "alpha_mode", 5), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "log_alpha", None), pdn.PDN_EINVAL),
    (lambda a: (setattr(a, "beta_mode", pdn.PDN_GATE_VEC), setattr(a, "dv", 64)),
     pdn.PDN_EINVAL),
    (lambda a: setattr(a, "precond_eps", 1e-6), pdn.PDN_EINVAL),  # no precond_A
    (lambda a: setattr(a, "dk", 32), pdn.PDN_EUNSUPPORTED),
    (lambda a: setattr(a, "dv", 256), pdn.PDN_EUNSUPPORTED),
    (lambda a: setattr(a, "key_mode", 3), pdn.PDN_EINVAL),
    (lambda a: (setattr(a, "precond_eps", 1e-6), setattr(a, "precond_A", FAKE),
                setattr(a, "precond_mode", pdn.PDN_PRECOND_STABILISED), setattr(a, "precond_x", 0.5)),
     pdn.PDN_EINVAL),
])
def test_decode_validation_codes(lib, mutate, code):
    a = _decode_ok()
    mutate(a)
    assert _dcheck(lib, a) == code
    assert lib.pdn_decode_step(ctypes.byref(a), None) == code


@pytest.mark.parametrize("km", [pdn.PDN_KEY_ERASE_GATE, pdn.PDN_KEY_WRITE_GATE])
def test_decode_asymmetric_keys_any_shape(lib, km):
    a = _decode_ok()
    a.key_mode = km
    assert _dcheck(lib, a) == pdn.PDN_OK
    a.dk, a.qkv_dtype = 64, pdn.PDN_F32
    assert _dcheck(lib, a) == pdn.PDN_OK


def test_stabilised_preconditioner_accepted(lib):
    a = _chunk_ok()
    a.precond_eps, a.precond_mode, a.precond_x = 1e-6, pdn.PDN_PRECOND_STABILISED, 1.5
    assert _ccheck(lib, a) == pdn.PDN_OK
    a.precond_x = 2.0
    assert _ccheck(lib, a) == pdn.PDN_OK
    # x is not read when the preconditioner is off or in the inverse mode
    a.precond_eps, a.precond_x = -1.0, 0.0
    assert _ccheck(lib, a) == pdn.PDN_OK
    d = _decode_ok()
    d.precond_eps, d.precond_A = 1e-6, FAKE
    d.precond_mode, d.precond_x = pdn.PDN_PRECOND_STABILISED, 1.5
    d.dk, d.qkv_dtype = 64, pdn.PDN_F32  # decode takes every shape
    assert _dcheck(lib, d) == pdn.PDN_OK


def test_null_args_pointer(lib):
    assert lib.pdn_chunk_fwd_check(None) == pdn.PDN_EINVAL
    assert lib.pdn_decode_check(None) == pdn.PDN_EINVAL
    assert lib.pdn_chunk_fwd(None, None) == pdn.PDN_EINVAL
    assert lib.pdn_decode_step(None, None) == pdn.PDN_EINVAL
    assert lib.pdn_chunk_fwd_workspace_size(None, None) == pdn.PDN_EINVAL


def test_c_abi_program_builds_and_links(tmp_path, lib):
    # the C test program compiles warning-free against include/pdn.h and links
    # against libpdn.so (it runs in the GPU tests)
    from cabi import build_c_abi_check
    import os
    assert os.access(build_c_abi_check(tmp_path), os.X_OK)


def test_binding_refuses_a_library_of_another_abi_version(tmp_path):
    # a library built from another header version would read the argument
    # structs at other offsets: load_library must refuse it before any call
    stub = tmp_path / "stub.c"
    stub.write_text("\n".join(
        ["int pdn_abi_version(void) { return %d; }" % (pdn.PDN_ABI_VERSION - 1),
         "const char *pdn_strerror(int c) { (void)c; return \"stub\"; }"] +
        ["int %s(void *a, void *b) { (void)a; (void)b; return -1; }" % n
         for n in pdn.EXPORTED if n not in ("pdn_abi_version", "pdn_strerror")]))
    so = tmp_path / "libstub.so"
    subprocess.check_call(["gcc", "-shared", "-fPIC", str(stub), "-o", str(so)])
    with pytest.raises(RuntimeError, match="ABI version"):
        pdn.load_library(str(so))


def test_workspace_for_sequence_segments(lib):
    # two heads, 1000 tokens, fp32 output: four segments, which add the
    # identity-column outputs [B,H,T,dk] and three [B,H,segments,dk,dv|dk]
    # state arrays (fp32); bf16 output keeps one pass and no extra
    a = _chunk_ok()
    a.B, a.H, a.T = 1, 2, 1000
    a.o_dtype = pdn.PDN_BF16
    one = _ws_size(lib, a)
    a.o_dtype = pdn.PDN_F32
    seg = _ws_size(lib, a)
    assert seg - one == 2 * 1000 * 128 * 4 + 3 * 2 * 4 * 128 * 128 * 4


def _bwd_ok():
    a = pdn.ChunkBwdArgs()
    a.fwd = _chunk_ok()
    a.fwd.o = None
    a.dO = a.dST = a.dq = a.dk = a.dv = FAKE
    a.dlog_alpha = a.dbeta = a.dgamma = a.dS0 = FAKE
    a.workspace, a.workspace_bytes = FAKE, 1 << 40
    return a


def _bcheck(lib, a):
    return lib.pdn_chunk_bwd_check(ctypes.byref(a))


def _bws(lib, a):
    n = ctypes.c_size_t(123)
    rc = lib.pdn_chunk_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return rc, n.value


BWD_BAD = [
    (lambda a: setattr(a, "dq", None), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "dO", None), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "dlog_alpha", None), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "dbeta", None), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "dgamma", None), pdn.PDN_EINVAL),
    (lambda a: setattr(a, "dv", FAKE + 4), pdn.PDN_EINVAL),          # misaligned
    (lambda a: setattr(a.fwd, "key_mode", 3), pdn.PDN_EINVAL),
    (lambda a: setattr(a.fwd, "dk", 96), pdn.PDN_EUNSUPPORTED),
    (lambda a: setattr(a.fwd, "dv", 48), pdn.PDN_EUNSUPPORTED),       # dv % 32
    (lambda a: setattr(a.fwd, "dv", 288), pdn.PDN_EUNSUPPORTED),
    (lambda a: (setattr(a.fwd, "precond_eps", 1e-6),
                setattr(a.fwd, "precond_mode", pdn.PDN_PRECOND_STABILISED),
                setattr(a.fwd, "precond_x", 2.5)), pdn.PDN_EINVAL),              # x out of (1, 2]
    (lambda a: setattr(a, "workspace_bytes", 1000), pdn.PDN_EWORKSPACE),
    (lambda a: setattr(a, "workspace", None), pdn.PDN_EWORKSPACE),
    (lambda a: setattr(a.fwd, "T", -1), pdn.PDN_EINVAL),
]


def test_bwd_valid_arguments(lib):
    assert _bcheck(lib, _bwd_ok()) == pdn.PDN_OK
    a = _bwd_ok()
    # fp32 inputs, dk = 64, scalar gates, every key mode, the inverse preconditioner
    a.fwd.qkv_dtype, a.fwd.dk, a.fwd.dv = pdn.PDN_F32, 64, 64
    a.fwd.alpha_mode, a.fwd.beta_mode = pdn.PDN_ALPHA_SCALAR, pdn.PDN_GATE_SCALAR
    a.fwd.gamma_mode, a.fwd.gamma, a.dgamma = pdn.PDN_GAMMA_SAME_AS_BETA, None, None
    a.fwd.precond_eps = 1e-6
    for km in (0, 1, 2):
        a.fwd.key_mode = km
        assert _bcheck(lib, a) == pdn.PDN_OK
    # the stabilised preconditioner
    a.fwd.precond_mode, a.fwd.precond_x = pdn.PDN_PRECOND_STABILISED, 1.5
    assert _bcheck(lib, a) == pdn.PDN_OK
    a.fwd.precond_mode = pdn.PDN_PRECOND_INVERSE
    # no decay: no d log alpha needed
    a.fwd.alpha_mode, a.fwd.log_alpha, a.dlog_alpha = pdn.PDN_ALPHA_NONE, None, None
    assert _bcheck(lib, a) == pdn.PDN_OK
    assert lib.pdn_chunk_bwd_check(None) == pdn.PDN_EINVAL
    assert lib.pdn_chunk_bwd(None, None) == pdn.PDN_EINVAL


@pytest.mark.parametrize("mutate,code", BWD_BAD)
def test_bwd_validation(lib, mutate, code):
    a = _bwd_ok()
    mutate(a)
    assert _bcheck(lib, a) == code
    # the launching entry point returns the same code without touching memory
    assert lib.pdn_chunk_bwd(ctypes.byref(a), None) == code


def test_bwd_workspace_size(lib):
    # per (b, h) and 32-token chunk, fp32: the record (3 32 x dk operand blocks,
    # 32 x dv values, two 32 x 32 blocks, dk), the chunk start state (one more
    # for S_T), the end-state gradient, U and Z (32 x dv each) and the gradient
    # record (3 32 x dk, two 32 x 32, dk); each array 256-byte aligned
    a = _bwd_ok()
    a.fwd.B, a.fwd.H, a.fwd.T, a.fwd.dk, a.fwd.dv = 1, 2, 100, 128, 64
    rc, n = _bws(lib, a)
    assert rc == pdn.PDN_OK
    nbh, nc, dk, dv = 2, 4, 128, 64
    al = lambda x: (x + 255) // 256 * 256
    want = (al(nbh * nc * (3 * 32 * dk + 32 * dv + 2 * 32 * 32 + dk) * 4)
            + al(nbh * (nc + 1) * dk * dv * 4) + al(nbh * nc * dk * dv * 4)
            + 2 * al(nbh * nc * 32 * dv * 4) + al(nbh * nc * (3 * 32 * dk + dk) * 4))
    assert n == want
    # the preconditioner adds four [B,H,chunks,dk] arrays and one [B,H,chunks*32,dk]
    a.fwd.precond_eps = 1e-6
    rc, n2 = _bws(lib, a)
    assert rc == pdn.PDN_OK
    assert n2 - n == 4 * al(nbh * nc * dk * 4) + al(nbh * nc * 32 * dk * 4)
    # the stabilised preconditioner adds the per-token channel means [B,H,chunks*32]
    a.fwd.precond_mode, a.fwd.precond_x = pdn.PDN_PRECOND_STABILISED, 1.5
    rc, n3 = _bws(lib, a)
    assert rc == pdn.PDN_OK and n3 - n2 == al(nbh * nc * 32 * 4)
    # T = 0 needs none
    a.fwd.T = 0
    assert _bws(lib, a) == (pdn.PDN_OK, 0)


def test_misaligned_workspace_is_rejected(lib):
    # the per-channel-gate kernels and the backward move their records with
    # 16-byte vector and buffer accesses: an offset workspace is refused
    a = _chunk_ok()
    a.workspace = FAKE + 8
    assert _ccheck(lib, a) == pdn.PDN_EINVAL
    assert lib.pdn_chunk_fwd(ctypes.byref(a), None) == pdn.PDN_EINVAL
    a.workspace = FAKE + 16
    assert _ccheck(lib, a) == pdn.PDN_OK
    b = _bwd_ok()
    b.workspace = FAKE + 4
    assert _bcheck(lib, b) == pdn.PDN_EINVAL
    assert lib.pdn_chunk_bwd(ctypes.byref(b), None) == pdn.PDN_EINVAL


# ---------------------------------------------------------------------------
# the Python binding checks every tensor's shape and device before it takes a
# pointer (the C ABI cannot know a tensor's extent).  Meta tensors carry a
# shape and no memory, so these run without a GPU: a shape error is reported
# by name before the binding would refuse the tensor for not being on a GPU.
# ---------------------------------------------------------------------------

def _meta(*shape):
    import torch
    return torch.empty(shape, device="meta", dtype=torch.float32)


def _meta_bf16(*shape):
    import torch
    return torch.empty(shape, device="meta", dtype=torch.bfloat16)


B_, H_, T_, DK_, DV_ = 2, 3, 10, 128, 64


def _fwd_kwargs():
    return dict(q=_meta_bf16(B_, H_, T_, DK_), k=_meta_bf16(B_, H_, T_, DK_),
                v=_meta_bf16(B_, H_, T_, DV_), o=_meta(B_, H_, T_, DV_),
                log_alpha=_meta(B_, H_, T_, DK_), beta=_meta(B_, H_, T_, DK_),
                gamma=_meta(B_, H_, T_, DV_), precond_eps=1e-6,
                precond_A0=_meta(B_, H_, DK_), precond_AT=_meta(B_, H_, DK_),
                S0=_meta(B_, H_, DK_, DV_), ST=_meta(B_, H_, DK_, DV_))


@pytest.mark.parametrize("name,bad", [
    ("o", (B_, H_, T_, DK_)),
    ("log_alpha", (B_, H_, T_, DV_)),          # per value channel: wrong axis
    ("log_alpha", (B_, H_)),
    ("beta", (B_, H_, T_, DV_)),               # a [B,H,T,dv] vector beta with dv < dk
    ("beta", (B_, H_, T_ + 1)),
    ("gamma", (B_, H_, T_, DK_)),
    ("precond_A0", (B_, H_, DV_)),
    ("precond_AT", (H_, DK_)),
    ("S0", (B_, H_, DV_, DK_)),
    ("ST", (H_, DK_, DV_)),                    # [H,dk,dv]: would be written past its end
])
def test_binding_rejects_misshaped_chunk_tensors(name, bad):
    kw = _fwd_kwargs()
    kw[name] = _meta(*bad)
    with pytest.raises(ValueError, match=name):
        pdn.pdn_chunk_fwd(**kw)
    with pytest.raises(ValueError, match=name):
        pdn.pdn_chunk_fwd_workspace_size(**kw)


def test_binding_requires_beta():
    kw = _fwd_kwargs()
    kw["beta"] = None
    with pytest.raises(ValueError, match="beta"):
        pdn.pdn_chunk_fwd(**kw)


def test_binding_shape_check_accepts_every_gate_rank():
    # well-shaped meta tensors pass the shape checks and stop only at the
    # device check (they live in no device memory)
    for la, be, ga in (((B_, H_, T_), (B_, H_, T_), (B_, H_, T_)),
                       ((B_, H_, T_, DK_), (B_, H_, T_, DK_), None),
                       (None, (B_, H_, T_), (B_, H_, T_, DV_))):
        kw = _fwd_kwargs()
        kw["log_alpha"] = None if la is None else _meta(*la)
        kw["beta"] = _meta(*be)
        kw["gamma"] = None if ga is None else _meta(*ga)
        with pytest.raises(ValueError, match="device memory"):
            pdn.pdn_chunk_fwd(**kw)


def test_binding_rejects_tensors_on_another_device():
    import torch
    kw = _fwd_kwargs()
    kw["S0"] = torch.zeros((B_, H_, DK_, DV_), dtype=torch.float32)   # host memory
    with pytest.raises(ValueError, match="S0 is on cpu"):
        pdn.pdn_chunk_fwd(**kw)


@pytest.mark.parametrize("name,bad", [
    ("log_alpha", (B_, H_, DV_)),
    ("beta", (B_, H_, DV_)),
    ("gamma", (B_, H_, DK_)),
    ("precond_A", (B_, H_, DV_)),
])
def test_binding_rejects_misshaped_decode_tensors(name, bad):
    kw = dict(q=_meta_bf16(B_, H_, DK_), k=_meta_bf16(B_, H_, DK_), v=_meta_bf16(B_, H_, DV_),
              o=_meta(B_, H_, DV_), S=_meta(B_, H_, DK_, DV_), log_alpha=_meta(B_, H_, DK_),
              beta=_meta(B_, H_, DK_), gamma=_meta(B_, H_, DV_), precond_eps=1e-6,
              precond_A=_meta(B_, H_, DK_))
    kw[name] = _meta(*bad)
    with pytest.raises(ValueError, match=name):
        pdn.pdn_decode_step(**kw)


@pytest.mark.parametrize("name,bad", [
    ("dST", (B_, H_, DV_, DK_)),
    ("dS0", (B_, H_, DK_)),
    ("dA0", (B_, H_, DK_, 1)),
    ("dO", (B_, H_, T_, DK_)),
])
def test_binding_rejects_misshaped_bwd_tensors(name, bad):
    f = _fwd_kwargs()
    kw = dict(q=f["q"], k=f["k"], v=f["v"], dO=_meta(B_, H_, T_, DV_),
              dq=_meta(B_, H_, T_, DK_), dk=_meta(B_, H_, T_, DK_), dv=_meta(B_, H_, T_, DV_),
              dlog_alpha=_meta(B_, H_, T_, DK_), dbeta=_meta(B_, H_, T_, DK_),
              dgamma=_meta(B_, H_, T_, DV_), dS0=_meta(B_, H_, DK_, DV_), dA0=_meta(B_, H_, DK_),
              log_alpha=f["log_alpha"], beta=f["beta"], gamma=f["gamma"], precond_eps=1e-6,
              precond_A0=f["precond_A0"], S0=f["S0"], dST=_meta(B_, H_, DK_, DV_))
    kw[name] = _meta(*bad)
    with pytest.raises(ValueError, match=name if name != "dO" else "o must"):
        pdn.pdn_chunk_bwd(**kw)


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    # the static scratch of pdn_chunk_fwd_noalloc holds PDN_NOALLOC_SCRATCH_BYTES;
    # a call that needs more returns PDN_ESCRATCH before touching the GPU
    m = re.search(r"#define PDN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    assert int(m.group(1)) << int(m.group(2)) == pdn.PDN_NOALLOC_SCRATCH_BYTES
    a = _chunk_ok()
    a.workspace, a.workspace_bytes = None, 0      # ignored by the no-allocation call
    a.B, a.H, a.T = 2, 32, 8192                   # per-channel gates: 0.94 GB of records
    assert _ws_size(lib, a) > pdn.PDN_NOALLOC_SCRATCH_BYTES
    assert lib.pdn_chunk_fwd_noalloc(ctypes.byref(a), None) == pdn.PDN_ESCRATCH
    # invalid arguments keep their own codes
    a.dk = 96
    assert lib.pdn_chunk_fwd_noalloc(ctypes.byref(a), None) == pdn.PDN_EUNSUPPORTED
    a.dk, a.B = 128, 0
    assert lib.pdn_chunk_fwd_noalloc(ctypes.byref(a), None) == pdn.PDN_EINVAL
    assert lib.pdn_chunk_fwd_noalloc(None, None) == pdn.PDN_EINVAL
