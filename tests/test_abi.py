"""C ABI checks that need no GPU: the library loads, exports every function
include/smla.h declares, and rejects malformed arguments on the host with the
documented status before any kernel is queued."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "smla.h")


@pytest.fixture(scope="module")
def b():
    from sparse_mla_decode_fp8_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_mla_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(b):
    decl = declared_functions()
    assert len(decl) >= 8
    lib = b.lib()
    for name in decl:
        assert hasattr(lib, name), f"{name} declared in smla.h but not exported"
    assert sorted(b.EXPORTED) == decl


def test_supported_range(b):
    assert not b.supported(0)
    assert b.supported(1) and b.supported(16) and b.supported(64) and b.supported(128)
    assert not b.supported(129)
    assert b.lib().sparse_mla_supported(16, 576, 512) == 1
    assert b.lib().sparse_mla_supported(16, 512, 512) == 0   # the record's QK dim is 576
    assert b.lib().sparse_mla_supported(16, 576, 576) == 0   # V is the 512 latent values


def test_workspace_bytes(b):
    assert b.workspace_bytes(0, 16, 0) >= 0
    small = b.workspace_bytes(4096, 64, 4096 * 2048)   # many rows: no split partials
    assert small < 1 << 20
    with pytest.raises(b.SmlaError) as e:
        b.workspace_bytes(1, 129, 10)
    assert e.value.status == b.SMLA_EUNSUPPORTED
    with pytest.raises(b.SmlaError) as e:
        b.workspace_bytes(-1, 16, 10)
    assert e.value.status == b.SMLA_EINVAL


FAKE = 0x10000  # a 256-aligned non-null address; never dereferenced by the failing calls


def call(b, **over):
    a = dict(q=FAKE, qst=576 * 16, qsh=576, kv=FAKE, n_kv=10, indptr=FAKE, indices=FAKE, nnz=4,
             T=1, H=16, scale=0.04, inv=0, out=FAKE, ost=512 * 16, osh=512, lse=None,
             ws=FAKE, wsb=1 << 40, stream=None)
    a.update(over)
    return b.lib().sparse_mla_fwd(a["q"], a["qst"], a["qsh"], a["kv"], a["n_kv"], a["indptr"],
                                  a["indices"], a["nnz"], a["T"], a["H"], a["scale"], a["inv"],
                                  a["out"], a["ost"], a["osh"], a["lse"], a["ws"], a["wsb"],
                                  a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(H=0), -2), (dict(H=129), -2), (dict(T=-1), -1), (dict(nnz=-1), -1),
    (dict(nnz=(1 << 30) - 4095), -1), (dict(n_kv=-1), -1), (dict(scale=float("inf")), -1),
    (dict(q=None), -1), (dict(kv=None), -1), (dict(indptr=None), -1), (dict(out=None), -1),
    (dict(ws=None), -1), (dict(indices=None), -1), (dict(q=FAKE + 8), -1),
    (dict(out=FAKE + 4), -1), (dict(kv=FAKE + 2), -1), (dict(ws=FAKE + 16), -1),
    (dict(qsh=577), -1), (dict(ost=-512), -1), (dict(wsb=100), -3),
    (dict(T=(1 << 31) - 1), -1), (dict(T=1 << 24, H=128), -1),
])
def test_host_validation(b, over, status):
    assert call(b, **over) == status
    assert b.lib().sparse_mla_last_error()  # a message for the failing call


def test_zero_rows_is_a_noop(b):
    assert call(b, T=0, q=None, out=None, ws=None) == 0


def test_options(b):
    assert b.lib().sparse_mla_set_option(b"split", 4) == 0
    assert b.lib().sparse_mla_set_option(b"split", 0) == 0
    assert b.lib().sparse_mla_set_option(b"split", 33) == -1
    assert b.lib().sparse_mla_set_option(b"nope", 1) == -1
    for v in (1, 2, 0):
        assert b.lib().sparse_mla_set_option(b"plan", v) == 0
    assert b.lib().sparse_mla_set_option(b"plan", 3) == -1
    for v in (1, 0):
        assert b.lib().sparse_mla_set_option(b"persist", v) == 0
    assert b.lib().sparse_mla_set_option(b"persist", 2) == -1


def test_decode_rows_validation(b):
    lib = b.lib()
    assert lib.sparse_mla_decode_rows(FAKE, 10, FAKE, -1, FAKE, None) == -1
    assert lib.sparse_mla_decode_rows(None, 10, FAKE, 3, FAKE, None) == -1
    assert lib.sparse_mla_decode_rows(FAKE + 4, 10, FAKE, 3, FAKE, None) == -1
    assert lib.sparse_mla_decode_rows(FAKE, 10, FAKE, 0, FAKE, None) == 0


def test_cache_write_validation(b):
    lib = b.lib()
    ok = dict(latent=FAKE, lst=512, rope=FAKE, rst=64, slots=FAKE, n=3, kv=FAKE, n_kv=10)

    def cw(**over):
        a = dict(ok)
        a.update(over)
        return lib.sparse_mla_cache_write(a["latent"], a["lst"], a["rope"], a["rst"], a["slots"],
                                          a["n"], a["kv"], a["n_kv"], None)
    for over in (dict(n=-1), dict(n_kv=-1), dict(latent=None), dict(rope=None), dict(slots=None),
                 dict(kv=None), dict(latent=FAKE + 8), dict(kv=FAKE + 4), dict(rope=FAKE + 4),
                 dict(slots=FAKE + 4), dict(lst=511), dict(lst=516), dict(rst=62), dict(rst=66)):
        assert cw(**over) == -1, over
        assert lib.sparse_mla_last_error()
    assert cw(n=0, latent=None, rope=None, slots=None, kv=None) == 0


def test_fwd_paged_validation(b):
    """Pool descriptors are checked on the host: page_records a power of two in
    [1, 2^30], base 16-byte aligned, page_stride a multiple of 16 and at least
    page_records * 656; a NULL base is an absent pool (accepted)."""
    lib = b.lib()

    def paged(pools, **over):
        a = dict(q=FAKE, qst=576 * 16, qsh=576, indptr=FAKE, indices=FAKE, nnz=4, T=1, H=16,
                 scale=0.04, inv=0, sink=None, out=FAKE, ost=512 * 16, osh=512, lse=None,
                 ws=FAKE, wsb=1 << 40)
        a.update(over)
        desc = None
        if pools is not None:
            desc = (b.KvPool * 2)(*[b.KvPool(*pl) for pl in pools])
        return lib.sparse_mla_fwd_paged(a["q"], a["qst"], a["qsh"], desc, a["indptr"], a["indices"],
                                        a["nnz"], a["T"], a["H"], a["scale"], a["inv"], a["sink"],
                                        a["out"], a["ost"], a["osh"], a["lse"], a["ws"], a["wsb"],
                                        None)
    good = (FAKE, 64 * 656, 64)
    bad_pools = [
        (FAKE, 3 * 656 + 16, 3),           # page_records not a power of two
        (FAKE, 0, 0),                      # page_records 0
        (FAKE, 656 * 2 ** 31, 2 ** 31),    # page_records above 2^30
        (FAKE + 8, 64 * 656, 64),          # misaligned base
        (FAKE, 64 * 656 - 16, 64),         # stride below a page of records
        (FAKE, 64 * 656 + 8, 64),          # stride not a multiple of 16
        (FAKE, 1 << 40, 1),                # stride so large that slot offsets overflow
    ]
    for bad in bad_pools:
        for pools in ([bad, good], [good, bad]):
            assert paged(pools) == -1, (bad, pools)
            assert lib.sparse_mla_last_error()
    assert paged(None) == -1
    assert paged([good, good], sink=FAKE + 2) == -1       # misaligned sink
    assert paged([good, good], H=129) == -2
    assert paged([good, good], wsb=100) == -3
    # absent pools and T = 0 are accepted without touching the device
    assert paged([(None, 0, 0), (None, 0, 0)], T=0, q=None, out=None, ws=None) == 0
    assert paged([good, (None, 0, 0)], T=0) == 0


def test_v41_validation(b):
    """V4.1 entry points reject malformed arguments on the host: heads above
    16, pools whose page stride cannot hold R x 584 bytes, missing pos /
    cos_sin / outputs, n_pos < 1, misaligned y_out; the MXFP8 hook needs n a
    multiple of 64."""
    lib = b.lib()
    good = (FAKE, 64 * 584, 64)

    def v41(pools=(good, good), **over):
        a = dict(q=FAKE, qst=512 * 16, qsh=512, indptr=FAKE, indices=FAKE, nnz=4, T=1, H=16,
                 scale=0.04, inv=0, sink=None, pos=FAKE, cs=FAKE, npos=8, xo=FAKE, xos=FAKE,
                 lse=None, y=None, ws=FAKE, wsb=1 << 40)
        a.update(over)
        desc = None if pools is None else (b.KvPool * 2)(*[b.KvPool(*pl) for pl in pools])
        return lib.sparse_mla_fwd_v41(a["q"], a["qst"], a["qsh"], desc, a["indptr"], a["indices"], a["nnz"],
                                      a["T"], a["H"], a["scale"], a["inv"], a["sink"], a["pos"], a["cs"],
                                      a["npos"], a["xo"], a["xos"], a["lse"], a["y"], a["ws"], a["wsb"], None)
    assert v41(H=17) == -2 and v41(H=0) == -2
    assert v41(pools=((FAKE, 64 * 584 - 16, 64), good)) == -1      # stride below R x 584
    assert v41(pools=((FAKE, 64 * 656, 3), good)) == -1            # R not a power of two
    assert v41(pools=None) == -1
    for over in (dict(pos=None), dict(cs=None), dict(xo=None), dict(xos=None), dict(npos=0),
                 dict(y=FAKE + 4), dict(xo=FAKE + 2), dict(q=FAKE + 8)):
        assert v41(**over) == -1, over
        assert lib.sparse_mla_last_error()
    assert v41(wsb=100) == -3
    assert v41(T=0, q=None, pos=None, cs=None, xo=None, xos=None, ws=None) == 0
    assert lib.sparse_mla_v41_workspace_bytes(4, 17, 10) == -2
    assert lib.sparse_mla_v41_workspace_bytes(4, 16, 10) > 0
    assert lib.sparse_mla_mxfp8(FAKE, 63, FAKE, FAKE, None) == -1
    assert lib.sparse_mla_mxfp8(FAKE, 64, FAKE + 4, FAKE, None) == -1
    assert lib.sparse_mla_mxfp8(None, 0, None, None, None) == 0


def test_profile_state_machine(b):
    lib = b.lib()
    ms = (ctypes.c_double * 4)()
    n = (ctypes.c_int64 * 4)()
    assert lib.sparse_mla_profile_end(ms, n) == -1      # not active
    assert lib.sparse_mla_profile_begin(0) == -1
