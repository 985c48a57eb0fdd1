"""Host-side checks of the C ABI (CPU only: no kernel is launched).

The library must load, export every function include/gdn.h declares, and reject
every bad argument on the host before any launch.  Pointers passed here are
never dereferenced: each call fails validation first.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from gated_deltanet_chunked_gdn_amd import _native as nat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    return nat.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_header_declares_what_the_binding_lists():
    assert declared_functions() == sorted(nat.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {nat.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_version_and_status_strings(lib):
    assert lib.gdn_abi_version() == 6
    for s in range(11):
        assert lib.gdn_status_str(s).decode() not in ("", "unknown status")
    assert lib.gdn_status_str(99).decode() == "unknown status"


def problem(**kw):
    p = nat.Problem()
    d = dict(B=2, T=100, H=3, Dk=128, Dv=128, num_seqs=2, io_dtype=nat.GDN_BF16, scale=1.0,
             chunk=64, num_segments=1)
    d.update(kw)
    for k, v in d.items():
        setattr(p, k, v)
    return p


def ws(p, pass_=nat.GDN_PASS_CHUNK_FWD):
    n = ctypes.c_size_t(12345)
    st = nat.load().gdn_workspace_size(ctypes.byref(p), pass_, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(io_dtype=7), nat.GDN_ERR_DTYPE),
    (dict(H=0), nat.GDN_ERR_SHAPE),
    (dict(T=-1), nat.GDN_ERR_SHAPE),
    (dict(Dk=96), nat.GDN_ERR_UNSUPPORTED),
    (dict(Dv=40), nat.GDN_ERR_UNSUPPORTED),
    (dict(Dv=512), nat.GDN_ERR_UNSUPPORTED),
    (dict(chunk=32), nat.GDN_ERR_UNSUPPORTED),
    (dict(num_segments=3), nat.GDN_ERR_UNSUPPORTED),
    (dict(num_segments=0), nat.GDN_ERR_UNSUPPORTED),
    (dict(num_segments=32), nat.GDN_ERR_UNSUPPORTED),
    (dict(num_seqs=3), nat.GDN_ERR_SHAPE),
    (dict(precision=2), nat.GDN_ERR_UNSUPPORTED),
    (dict(precision=-1), nat.GDN_ERR_UNSUPPORTED),
])
def test_problem_validation(kw, status):
    assert ws(problem(**kw))[0] == status


def test_precision_policy_scope():
    """IEEE fp32 products: the forward at both head sizes and io dtypes; the
    backward with fp32 io at both head sizes; not the per-channel-decay passes
    with bf16 io."""
    fp32 = nat.GDN_PRECISION_FP32
    assert ws(problem(io_dtype=nat.GDN_FP32, Dk=128))[0] == nat.GDN_OK
    assert ws(problem(precision=fp32))[0] == nat.GDN_OK
    assert ws(problem(precision=fp32, Dk=64))[0] == nat.GDN_OK
    assert ws(problem(precision=fp32), nat.GDN_PASS_CHUNK_BWD)[0] == nat.GDN_ERR_UNSUPPORTED
    assert ws(problem(io_dtype=nat.GDN_FP32, Dk=128), nat.GDN_PASS_CHUNK_BWD)[0] == nat.GDN_OK
    assert ws(problem(io_dtype=nat.GDN_FP32, Dk=64, precision=fp32), nat.GDN_PASS_CHUNK_BWD)[0] == nat.GDN_OK
    assert ws(problem(precision=fp32), nat.GDN_PASS_KDA_FWD)[0] == nat.GDN_ERR_UNSUPPORTED
    assert ws(problem(precision=fp32), nat.GDN_PASS_KDA_BWD)[0] == nat.GDN_ERR_UNSUPPORTED
    assert ws(problem(precision=fp32), nat.GDN_PASS_RECURRENT_FWD)[0] == nat.GDN_OK


def test_workspace_sizes():
    # forward: per (chunk slot, head) a T diag(beta) record of 3072 io elements
    # (six bf16 operand fragments, or the 2560 entries of its lower 16x16 blocks
    # for fp32), P (4096 io elements) and 128 fp32 decays, each array rounded up
    # to 256 bytes; slots = rows // 64 + N + 1
    slots = 200 // 64 + 2 + 1
    up = lambda b: (b + 255) // 256 * 256
    gates = up(slots * 3 * 128 * 4)
    recs = up(slots * 3 * 3072 * 2) + up(slots * 3 * 4096 * 2) + gates
    assert ws(problem()) == (nat.GDN_OK, recs)
    assert ws(problem(io_dtype=nat.GDN_FP32, Dk=64)) == (
        nat.GDN_OK, up(slots * 3 * 3072 * 4) + up(slots * 3 * 4096 * 4) + gates)
    # fp32 products on bf16 inputs keep fp32 records
    assert ws(problem(precision=nat.GDN_PRECISION_FP32)) == (
        nat.GDN_OK, up(slots * 3 * 3072 * 4) + up(slots * 3 * 4096 * 4) + gates)
    # segment split: then fp32 end and start states [G][N][H][Dk][Dv] and maps [G][N][H][Dk][Dk]
    for G in (2, 4, 16):
        seg = (2 * G * 2 * 3 * 128 * 96 + G * 2 * 3 * 128 * 128) * 4
        assert ws(problem(num_segments=G, Dv=96)) == (nat.GDN_OK, recs + seg)
    assert ws(problem(), nat.GDN_PASS_RECURRENT_FWD) == (nat.GDN_OK, 0)
    st, n = ws(problem(Dk=64), nat.GDN_PASS_RECURRENT_BWD)
    assert st == nat.GDN_OK and n > 0
    assert ws(problem(), 17)[0] == nat.GDN_ERR_UNSUPPORTED
    assert nat.load().gdn_workspace_size(ctypes.byref(problem()), 0, None) == nat.GDN_ERR_NULL
    assert nat.load().gdn_workspace_size(None, 0, ctypes.byref(ctypes.c_size_t())) == nat.GDN_ERR_NULL


def test_recurrent_backward_lds_limit():
    assert ws(problem(Dk=128, Dv=256), nat.GDN_PASS_RECURRENT_BWD)[0] == nat.GDN_ERR_UNSUPPORTED
    assert ws(problem(Dk=128, Dv=128), nat.GDN_PASS_RECURRENT_BWD)[0] == nat.GDN_OK


def test_cu_seqlens_validation():
    keep = []

    def packed(cu, T=None, **kw):
        host = np.asarray(cu, dtype=np.int32)
        keep.append(host)
        args = dict(B=1, T=int(host[-1]) if T is None else T, num_seqs=len(cu) - 1,
                    cu_seqlens_host=host.ctypes.data, cu_seqlens_dev=0x1000)
        args.update(kw)
        return problem(**args)

    assert ws(packed([0, 5, 5, 9]))[0] == nat.GDN_OK
    assert ws(packed([0, 5, 3, 9]))[0] == nat.GDN_ERR_SEQLENS
    assert ws(packed([1, 5, 9]))[0] == nat.GDN_ERR_SEQLENS
    assert ws(packed([0, 5, 9], T=10))[0] == nat.GDN_ERR_SEQLENS
    assert ws(packed([0, 5, 9], B=2))[0] == nat.GDN_ERR_SHAPE
    p = packed([0, 5, 9])
    p.cu_seqlens_dev = None
    assert ws(p)[0] == nat.GDN_ERR_NULL


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation


def fwd_call(p, q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30),
             beta=FAKE + (4 << 30), S0=None, o=FAKE + (5 << 30), Sf=None):
    P = ctypes.c_void_p
    return nat.load().gdn_chunk_fwd(ctypes.byref(p), P(q), P(k), P(v), P(g), P(beta), P(S0), P(o),
                                    P(Sf), None, 0, None)


def test_forward_pointer_checks():
    p = problem()
    assert fwd_call(p) == nat.GDN_ERR_WORKSPACE
    assert fwd_call(p, q=None) == nat.GDN_ERR_NULL
    assert fwd_call(p, o=None) == nat.GDN_ERR_NULL
    assert fwd_call(p, q=FAKE + 8) == nat.GDN_ERR_ALIGN
    assert fwd_call(p, g=FAKE + (3 << 30) + 2) == nat.GDN_ERR_ALIGN
    assert fwd_call(p, o=FAKE + 4096) == nat.GDN_ERR_ALIAS          # o inside q
    assert fwd_call(p, Sf=FAKE + (5 << 30) + 64) == nat.GDN_ERR_ALIAS  # S_final inside o
    assert fwd_call(problem(Dk=80)) == nat.GDN_ERR_UNSUPPORTED


def test_backward_entry_validates():
    P = ctypes.c_void_p
    lib = nat.load()
    z = [P(None)] * 15
    assert lib.gdn_chunk_bwd(ctypes.byref(problem(chunk=16)), *z, 0, None) == nat.GDN_ERR_UNSUPPORTED
    # the segment split is a forward-only option
    assert lib.gdn_chunk_bwd(ctypes.byref(problem(num_segments=2)), *z, 0, None) == nat.GDN_ERR_UNSUPPORTED
    assert lib.gdn_chunk_bwd(ctypes.byref(problem()), *z, 0, None) == nat.GDN_ERR_NULL
    # q k v g beta S0 dO dS_final dq dk dv dg dbeta dS0 ws
    ptrs = [P(FAKE + (i << 30)) for i in range(14)]
    for i in (5, 7, 13):  # S0, dS_final, dS0 optional
        ptrs[i] = P(None)
    assert lib.gdn_chunk_bwd(ctypes.byref(problem()), *ptrs, P(None), 0, None) == nat.GDN_ERR_WORKSPACE
    bad = list(ptrs)
    bad[8] = P(FAKE + (6 << 30) + 64)  # dq inside dO
    assert lib.gdn_chunk_bwd(ctypes.byref(problem()), *bad, P(None), 0, None) == nat.GDN_ERR_ALIAS
    bad = list(ptrs)
    bad[11] = P(FAKE + (11 << 30) + 2)  # misaligned dg
    assert lib.gdn_chunk_bwd(ctypes.byref(problem()), *bad, P(None), 0, None) == nat.GDN_ERR_ALIGN


def test_backward_workspace_size():
    # T (64 x 64), the T diag(beta) record (3072 io elements), the decays and P (64 x 64),
    # each rounded up to 256 bytes, then the states before and state gradients after
    # every chunk slot in the products' operand type (bf16 here, fp32 for fp32 io);
    # slots = rows // 64 + N + 1
    slots = 200 // 64 + 2 + 1
    up = lambda b: (b + 255) // 256 * 256
    st, n = ws(problem(Dv=96), nat.GDN_PASS_CHUNK_BWD)
    assert st == nat.GDN_OK
    assert n == (2 * up(slots * 3 * 4096 * 2) + up(slots * 3 * 3072 * 2) + up(slots * 3 * 128 * 4)
                 + 2 * slots * 3 * 128 * 96 * 2)
    st, n = ws(problem(io_dtype=nat.GDN_FP32, Dk=64, Dv=96), nat.GDN_PASS_CHUNK_BWD)
    assert st == nat.GDN_OK
    assert n == (2 * up(slots * 3 * 4096 * 4) + up(slots * 3 * 3072 * 4) + up(slots * 3 * 128 * 4)
                 + 2 * slots * 3 * 64 * 96 * 4)
    assert ws(problem(num_segments=4), nat.GDN_PASS_CHUNK_BWD)[0] == nat.GDN_ERR_UNSUPPORTED
    assert ws(problem(io_dtype=nat.GDN_FP32, Dk=128), nat.GDN_PASS_CHUNK_BWD)[0] == nat.GDN_OK


def test_saved_buffer_size_and_validation():
    # the backward workspace plus P in the forward's operand order (64 x 64 io elements per slot)
    slots = 200 // 64 + 2 + 1
    up = lambda b: (b + 255) // 256 * 256
    st, nb = ws(problem(Dv=96), nat.GDN_PASS_CHUNK_BWD)
    st2, ns = ws(problem(Dv=96), nat.GDN_PASS_CHUNK_SAVED)
    assert st == st2 == nat.GDN_OK and ns == nb + up(slots * 3 * 4096 * 2)
    assert ws(problem(num_segments=2), nat.GDN_PASS_CHUNK_SAVED)[0] == nat.GDN_ERR_UNSUPPORTED
    assert ws(problem(precision=nat.GDN_PRECISION_FP32), nat.GDN_PASS_CHUNK_SAVED)[0] == nat.GDN_ERR_UNSUPPORTED
    P = ctypes.c_void_p
    lib = nat.load()
    # gdn_chunk_fwd_save: q k v g beta S0 o S_final saved
    f = [P(FAKE + (i << 30)) for i in range(9)]
    f[5] = P(None)
    assert lib.gdn_chunk_fwd_save(ctypes.byref(problem()), *f[:8], P(None), 0, None) == nat.GDN_ERR_WORKSPACE
    assert lib.gdn_chunk_fwd_save(ctypes.byref(problem()), *f, 64, None) == nat.GDN_ERR_WORKSPACE
    assert lib.gdn_chunk_fwd_save(ctypes.byref(problem(num_segments=4)), *f, 1 << 30, None) == nat.GDN_ERR_UNSUPPORTED
    bad = list(f)
    bad[8] = P(FAKE + (2 << 30) + 4096)  # saved inside v
    assert lib.gdn_chunk_fwd_save(ctypes.byref(problem()), *bad, 1 << 30, None) == nat.GDN_ERR_ALIAS
    z = [P(None)] * 9
    assert lib.gdn_chunk_fwd_save(ctypes.byref(problem()), *z, 0, None) == nat.GDN_ERR_NULL
    # gdn_chunk_bwd_saved: q k v g beta dO dS_final dq dk dv dg dbeta dS0 saved
    b = [P(FAKE + (i << 30)) for i in range(14)]
    b[6] = P(None)
    b[12] = P(None)
    assert lib.gdn_chunk_bwd_saved(ctypes.byref(problem()), *b[:13], P(None), 0, None) == nat.GDN_ERR_WORKSPACE
    bad = list(b)
    bad[9] = P(FAKE + (5 << 30) + 64)  # dv inside dO
    assert lib.gdn_chunk_bwd_saved(ctypes.byref(problem()), *bad, 1 << 30, None) == nat.GDN_ERR_ALIAS
    assert lib.gdn_chunk_bwd_saved(ctypes.byref(problem(chunk=32)), *b, 1 << 30, None) == nat.GDN_ERR_UNSUPPORTED


def test_recurrent_backward_needs_workspace():
    p = problem(Dk=64)
    P = ctypes.c_void_p
    ptrs = [P(FAKE + (i << 30)) for i in range(16)]
    ptrs[5] = P(None)   # S0
    ptrs[9] = P(None)   # dS_final
    ptrs[15] = P(None)  # dS0
    st = nat.load().gdn_recurrent_ref(ctypes.byref(p), *ptrs, None, 0, None)
    assert st == nat.GDN_ERR_WORKSPACE


def prologue_call(p, gate=nat.GDN_GATE_GDN, **kw):
    """gdn_prologue with fake, well-separated pointers (overridable by name)."""
    names = ("q", "k", "a", "b", "A_log", "dt_bias", "q_out", "k_out", "g", "beta")
    ptr = {n: FAKE + (i << 30) for i, n in enumerate(names)}
    ptr.update(kw)
    P = ctypes.c_void_p
    return nat.load().gdn_prologue(ctypes.byref(p), P(ptr["q"]), P(ptr["k"]), P(ptr["a"]), P(ptr["b"]),
                                   P(ptr["A_log"]), P(ptr["dt_bias"]), gate, 0, P(ptr["q_out"]),
                                   P(ptr["k_out"]), P(ptr["g"]), P(ptr["beta"]), None)


def test_prologue_checks():
    p = problem()
    assert prologue_call(p, q=None) == nat.GDN_ERR_NULL
    assert prologue_call(p, beta=None) == nat.GDN_ERR_NULL
    assert prologue_call(p, A_log=None) == nat.GDN_ERR_NULL         # required by the GDN gate
    assert prologue_call(p, gate=7) == nat.GDN_ERR_UNSUPPORTED
    assert prologue_call(p, k=FAKE + (1 << 30) + 8) == nat.GDN_ERR_ALIGN
    assert prologue_call(p, q_out=FAKE + 4096) == nat.GDN_ERR_ALIAS  # q_out inside q
    assert prologue_call(problem(Dk=96)) == nat.GDN_ERR_UNSUPPORTED
    assert prologue_call(problem(io_dtype=5)) == nat.GDN_ERR_DTYPE
    # per-channel gates: dt_bias required, a, g and dt_bias 16-byte aligned, g spans B T H Dk floats
    ch = nat.GDN_GATE_GDN_CHANNEL
    assert prologue_call(p, gate=ch, dt_bias=None) == nat.GDN_ERR_NULL
    assert prologue_call(p, gate=ch, a=FAKE + (2 << 30) + 4) == nat.GDN_ERR_ALIGN
    assert prologue_call(p, gate=nat.GDN_GATE_GDN, a=FAKE + (2 << 30) + 4) != nat.GDN_ERR_ALIGN
    assert prologue_call(p, gate=ch, beta=FAKE + (8 << 30) + 2 * 100 * 3 * 4 * 8) == nat.GDN_ERR_ALIAS
    assert prologue_call(p, gate=3) == nat.GDN_ERR_UNSUPPORTED


def test_epilogue_checks():
    P = ctypes.c_void_p
    lib = nat.load()

    def call(p, o=FAKE, z=FAKE + (1 << 30), w=FAKE + (2 << 30), y=FAKE + (3 << 30)):
        return lib.gdn_epilogue(ctypes.byref(p), P(o), P(z), P(w), 1e-6, P(y), None)

    assert call(problem(), o=None) == nat.GDN_ERR_NULL
    assert call(problem(), y=None) == nat.GDN_ERR_NULL
    assert call(problem(Dv=96)) == nat.GDN_ERR_UNSUPPORTED          # not a power of two
    assert call(problem(), y=FAKE + 4096) == nat.GDN_ERR_ALIAS       # y inside o
    assert call(problem(), z=FAKE + (1 << 30) + 8) == nat.GDN_ERR_ALIGN


def test_kda_workspace_and_checks():
    # one record per (chunk slot, head): T diag(beta) and P (64 x 64 each), K o Gamma,
    # Q o Gamma and the decayed keys (64 x Dk each) in the io element type, then
    # Gamma_n (Dk fp32)
    slots = 200 // 64 + 2 + 1
    for Dk in (64, 128):
        for io, size in ((nat.GDN_BF16, 2), (nat.GDN_FP32, 4)):
            rec = (8192 + 3 * 64 * Dk) * size + 4 * Dk
            assert ws(problem(Dk=Dk, io_dtype=io), nat.GDN_PASS_KDA_FWD) == (nat.GDN_OK, slots * 3 * rec)
    # segment split: the fp32 end states, start states (G N H Dk Dv each) and maps (G N H Dk Dk)
    # after the records
    for G in (2, 16):
        rec = slots * 3 * ((8192 + 3 * 64 * 128) * 2 + 4 * 128)
        seg = (2 * G * 2 * 3 * 128 * 128 + G * 2 * 3 * 128 * 128) * 4
        assert ws(problem(num_segments=G), nat.GDN_PASS_KDA_FWD) == (nat.GDN_OK, rec + seg)
    assert ws(problem(num_segments=3), nat.GDN_PASS_KDA_FWD)[0] == nat.GDN_ERR_UNSUPPORTED
    assert ws(problem(Dk=96), nat.GDN_PASS_KDA_FWD)[0] == nat.GDN_ERR_UNSUPPORTED
    P = ctypes.c_void_p
    lib = nat.load()

    def call(p, q=FAKE, g=FAKE + (3 << 30), o=FAKE + (5 << 30), wsp=None, nws=0):
        return lib.gdn_kda_chunk_fwd(ctypes.byref(p), P(q), P(FAKE + (1 << 30)), P(FAKE + (2 << 30)), P(g),
                                     P(FAKE + (4 << 30)), None, P(o), None, P(wsp), nws, None)

    assert call(problem()) == nat.GDN_ERR_WORKSPACE
    assert call(problem(), q=None) == nat.GDN_ERR_NULL
    assert call(problem(), g=None) == nat.GDN_ERR_NULL
    assert call(problem(), g=FAKE + (3 << 30) + 2) == nat.GDN_ERR_ALIGN
    assert call(problem(), o=FAKE + 4096) == nat.GDN_ERR_ALIAS
    # g spans B T H Dk floats: an output starting inside that range aliases it
    assert call(problem(), o=FAKE + (3 << 30) + 2 * 100 * 3 * 128 * 4 - 16) == nat.GDN_ERR_ALIAS
    assert call(problem(num_segments=4)) == nat.GDN_ERR_WORKSPACE    # segments need the larger workspace
    assert call(problem(num_segments=5)) == nat.GDN_ERR_UNSUPPORTED
    assert call(problem(B=0, T=0, num_seqs=0)) == nat.GDN_OK   # nothing to do, nothing launched


def test_kda_bwd_workspace_and_checks():
    # the forward's records, then per (chunk slot, head) T, Ab and P in fp32 (3 x 64 x 64
    # floats), then the state before and the state gradient after every chunk (Dk Dv values
    # each, in the io element type)
    slots = 200 // 64 + 2 + 1
    for Dk in (64, 128):
        for io, size in ((nat.GDN_BF16, 2), (nat.GDN_FP32, 4)):
            rec = (8192 + 3 * 64 * Dk) * size + 4 * Dk
            aux = 3 * 4096 * 4
            st = Dk * 128 * size
            want = slots * 3 * (rec + aux + 2 * st)
            assert ws(problem(Dk=Dk, io_dtype=io), nat.GDN_PASS_KDA_BWD) == (nat.GDN_OK, want)
    # the retained-state pair uses the same buffer
    assert ws(problem(), nat.GDN_PASS_KDA_SAVED) == ws(problem(), nat.GDN_PASS_KDA_BWD)
    assert ws(problem(num_segments=2), nat.GDN_PASS_KDA_BWD)[0] == nat.GDN_ERR_UNSUPPORTED
    assert ws(problem(Dk=96), nat.GDN_PASS_KDA_BWD)[0] == nat.GDN_ERR_UNSUPPORTED
    assert ws(problem(Dv=24), nat.GDN_PASS_KDA_BWD)[0] == nat.GDN_ERR_UNSUPPORTED
    P = ctypes.c_void_p
    lib = nat.load()
    # inputs q k v g beta dO at FAKE + 0..5 GiB; outputs dq dk dv dg dbeta at 8..12 GiB
    GB = 1 << 30

    def call(p, q=FAKE, g=FAKE + 3 * GB, dq=FAKE + 8 * GB, dg=FAKE + 11 * GB, wsp=None, nws=0):
        return lib.gdn_kda_chunk_bwd(ctypes.byref(p), P(q), P(FAKE + GB), P(FAKE + 2 * GB), P(g),
                                     P(FAKE + 4 * GB), None, P(FAKE + 5 * GB), None, P(dq), P(FAKE + 9 * GB),
                                     P(FAKE + 10 * GB), P(dg), P(FAKE + 12 * GB), None, P(wsp), nws, None)

    assert call(problem()) == nat.GDN_ERR_WORKSPACE
    assert call(problem(), q=None) == nat.GDN_ERR_NULL
    assert call(problem(), dg=None) == nat.GDN_ERR_NULL
    assert call(problem(), g=FAKE + 3 * GB + 2) == nat.GDN_ERR_ALIGN
    assert call(problem(), dq=FAKE + 4096) == nat.GDN_ERR_ALIAS
    # dg spans B T H Dk floats: dq starting inside it aliases it
    assert call(problem(), dq=FAKE + 11 * GB + 2 * 100 * 3 * 128 * 4 - 16) == nat.GDN_ERR_ALIAS
    assert call(problem(num_segments=2)) == nat.GDN_ERR_UNSUPPORTED
    assert call(problem(precision=nat.GDN_PRECISION_FP32)) == nat.GDN_ERR_UNSUPPORTED
    assert call(problem(B=0, T=0, num_seqs=0)) == nat.GDN_OK   # nothing to do, nothing launched
    # the retained-state pair: the same checks; a short buffer is refused
    n = ws(problem(), nat.GDN_PASS_KDA_SAVED)[1]
    assert lib.gdn_kda_chunk_fwd_save(ctypes.byref(problem()), P(FAKE), P(FAKE + GB), P(FAKE + 2 * GB),
                                      P(FAKE + 3 * GB), P(FAKE + 4 * GB), None, P(FAKE + 8 * GB), None,
                                      P(FAKE + 13 * GB), n - 16, None) == nat.GDN_ERR_WORKSPACE
    assert lib.gdn_kda_chunk_fwd_save(ctypes.byref(problem(num_segments=4)), P(FAKE), P(FAKE + GB),
                                      P(FAKE + 2 * GB), P(FAKE + 3 * GB), P(FAKE + 4 * GB), None,
                                      P(FAKE + 8 * GB), None, P(FAKE + 13 * GB), n, None) == nat.GDN_ERR_UNSUPPORTED
    assert lib.gdn_kda_chunk_bwd_saved(ctypes.byref(problem()), P(FAKE), P(FAKE + GB), P(FAKE + 2 * GB),
                                       P(FAKE + 3 * GB), P(FAKE + 4 * GB), P(FAKE + 5 * GB), None,
                                       P(FAKE + 8 * GB), P(FAKE + 9 * GB), P(FAKE + 10 * GB), P(FAKE + 11 * GB),
                                       P(FAKE + 12 * GB), None, P(FAKE + 13 * GB), n - 16, None) == nat.GDN_ERR_WORKSPACE
    # the saved buffer may not overlap an output
    assert lib.gdn_kda_chunk_bwd_saved(ctypes.byref(problem()), P(FAKE), P(FAKE + GB), P(FAKE + 2 * GB),
                                       P(FAKE + 3 * GB), P(FAKE + 4 * GB), P(FAKE + 5 * GB), None,
                                       P(FAKE + 8 * GB), P(FAKE + 9 * GB), P(FAKE + 10 * GB), P(FAKE + 11 * GB),
                                       P(FAKE + 12 * GB), None, P(FAKE + 8 * GB + 4096), n, None) == nat.GDN_ERR_ALIAS


def test_noalloc_entry_checks_before_any_launch():
    """gdn_chunk_fwd_noalloc validates like gdn_chunk_fwd and rejects problems whose
    workspace exceeds its fixed device array, all before touching a device."""
    P = ctypes.c_void_p
    lib = nat.load()

    def call(p, q=FAKE, o=FAKE + (5 << 30)):
        return lib.gdn_chunk_fwd_noalloc(ctypes.byref(p), P(q), P(FAKE + (1 << 30)), P(FAKE + (2 << 30)),
                                         P(FAKE + (3 << 30)), P(FAKE + (4 << 30)), None, P(o), None, None)

    # 32 x 1024 tokens x 16 heads at Dk = 64, Dv = 128 needs ~126 MiB of workspace
    big = problem(B=32, T=1024, H=16, Dk=64, Dv=128, num_seqs=32)
    st, n = ws(big)
    assert st == nat.GDN_OK and n > nat.GDN_NOALLOC_SCRATCH_BYTES
    assert call(big) == nat.GDN_ERR_SCRATCH
    assert "no-allocation" in lib.gdn_status_str(nat.GDN_ERR_SCRATCH).decode()
    # the training shape fits
    st, n = ws(problem(B=4, T=4096, H=8, num_seqs=4))
    assert st == nat.GDN_OK and 0 < n <= nat.GDN_NOALLOC_SCRATCH_BYTES
    # ordinary validation comes first
    assert call(problem(Dk=96)) == nat.GDN_ERR_UNSUPPORTED
    assert call(problem(), q=None) == nat.GDN_ERR_NULL
    assert call(problem(num_segments=3)) == nat.GDN_ERR_UNSUPPORTED
    assert call(problem(B=0, T=0, num_seqs=0)) == nat.GDN_OK   # nothing to do, nothing launched


def test_device_copy_checks():
    P = ctypes.c_void_p
    lib = nat.load()
    assert lib.gdn_device_copy(None, P(FAKE), 64, None) == nat.GDN_ERR_NULL
    assert lib.gdn_device_copy(P(FAKE + (1 << 30)), P(FAKE), 60, None) == nat.GDN_ERR_ALIGN
    assert lib.gdn_device_copy(P(FAKE + 8), P(FAKE + (1 << 30)), 64, None) == nat.GDN_ERR_ALIGN
    assert lib.gdn_device_copy(P(FAKE + 32), P(FAKE), 64, None) == nat.GDN_ERR_ALIAS
    assert lib.gdn_device_copy(P(FAKE), P(FAKE), 0, None) == nat.GDN_OK   # nothing to do
