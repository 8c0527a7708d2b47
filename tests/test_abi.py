"""The C-ABI library loads without a GPU, exports every symbol include/pkv.h declares, and rejects bad
arguments on the host before any launch."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

from paged_kv_cache_416_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", src)))


def test_header_declarations_match_binding():
    assert _declared() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (pkv_\w+)", out))
    assert exported == set(_declared())


def test_header_compiles_as_c_and_cpp(tmp_path):
    for lang, comp in (("c", "gcc"), ("c++", "g++")):
        src = tmp_path / f"t.{'c' if lang == 'c' else 'cpp'}"
        src.write_text('#include "pkv.h"\nint main(void){ return pkv_version() == 0; }\n')
        r = subprocess.run([comp, "-x", lang, "-I", os.path.join(ROOT, "include"), "-c", str(src), "-o",
                            str(tmp_path / "t.o")], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_version_and_error_text():
    lib = _lib.load()
    assert b"gfx950" in lib.pkv_version()
    rc = lib.pkv_pool_create(0, 16, None, ctypes.byref(ctypes.c_void_p()))
    assert rc == _lib.PKV_EINVAL
    assert b"num_blocks" in lib.pkv_last_error()


NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every case below fails host validation


def _attn(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, num_blocks=10, tables=FAKE, max_blocks=4, ctx=FAKE, max_ctx=64,
             S=2, hq=4, hkv=4, d=128, B=16, scale=0.1, P=0, ws=NULL, ws_bytes=0, dtype=1, flags=0)
    a.update(kw)
    return _lib.load().pkv_paged_attention_decode(a["out"], a["q"], a["k"], a["v"], a["num_blocks"], a["tables"],
                                                  a["max_blocks"], a["ctx"], a["max_ctx"], a["S"], a["hq"], a["hkv"],
                                                  a["d"], a["B"], a["scale"], a["P"], a["ws"], a["ws_bytes"],
                                                  a["dtype"], a["flags"], NULL, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _lib.PKV_EINVAL),
    (dict(d=96), _lib.PKV_EUNSUPPORTED),
    (dict(B=12), _lib.PKV_EUNSUPPORTED),
    (dict(hq=6, hkv=4), _lib.PKV_EINVAL),
    (dict(hkv=0), _lib.PKV_EINVAL),
    (dict(S=-1), _lib.PKV_EINVAL),
    (dict(S=70000), _lib.PKV_EINVAL),
    (dict(P=24), _lib.PKV_EINVAL),            # not a multiple of block_size
    (dict(P=-2), _lib.PKV_EINVAL),            # negative, and not the balanced mode
    (dict(flags=8), _lib.PKV_EINVAL),         # unknown flag bit
    (dict(P=32), _lib.PKV_EINVAL),            # split mode without workspace
    (dict(P=32, ws=FAKE, ws_bytes=100), _lib.PKV_EINVAL),  # workspace too small
    (dict(scale=float("nan")), _lib.PKV_EINVAL),
    (dict(q=NULL), _lib.PKV_EINVAL),
    (dict(q=ctypes.c_void_p((1 << 20) + 8)), _lib.PKV_EINVAL),  # misaligned
    (dict(tables=NULL), _lib.PKV_EINVAL),
    (dict(max_blocks=0), _lib.PKV_EINVAL),
    (dict(max_ctx=-1), _lib.PKV_EINVAL),
])
def test_attention_rejects_bad_arguments(kw, code):
    assert _attn(**kw) == code
    assert _lib.load().pkv_last_error()


def _step(**kw):
    a = dict(out=FAKE, q=FAKE, nk=FAKE, nv=FAKE, slots=FAKE, k=FAKE, v=FAKE, num_blocks=10, tables=FAKE,
             max_blocks=4, ctx=FAKE, max_ctx=64, S=2, hq=4, hkv=4, d=128, B=16, scale=0.1, P=0, ws=NULL, ws_bytes=0,
             dtype=1, flags=0)
    a.update(kw)
    return _lib.load().pkv_paged_attention_decode_step(
        a["out"], a["q"], a["nk"], a["nv"], a["slots"], a["k"], a["v"], a["num_blocks"], a["tables"], a["max_blocks"],
        a["ctx"], a["max_ctx"], a["S"], a["hq"], a["hkv"], a["d"], a["B"], a["scale"], a["P"], a["ws"], a["ws_bytes"],
        a["dtype"], a["flags"], NULL, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(nk=NULL), _lib.PKV_EINVAL),
    (dict(nv=NULL), _lib.PKV_EINVAL),
    (dict(slots=NULL), _lib.PKV_EINVAL),
    (dict(nk=ctypes.c_void_p((1 << 20) + 8)), _lib.PKV_EINVAL),  # misaligned new rows
    (dict(B=12), _lib.PKV_EUNSUPPORTED),                            # the decode call's checks apply
    (dict(P=24), _lib.PKV_EINVAL),
])
def test_step_rejects_bad_arguments(kw, code):
    assert _step(**kw) == code
    assert _lib.load().pkv_last_error()


def test_step_with_no_sequences_is_a_no_op():
    assert _step(S=0, out=NULL, q=NULL, nk=NULL, nv=NULL, slots=NULL) == _lib.PKV_OK


def test_attention_with_no_sequences_is_a_no_op():
    assert _attn(S=0, out=NULL, q=NULL) == _lib.PKV_OK


def test_workspace_size_formula():
    lib = _lib.load()
    rows = 256 * 32 * 18
    got = lib.pkv_decode_workspace_bytes(256, 32, 128, 9216, 512)
    if torch.cuda.is_available():
        # the partition rows, padded to 16 bytes, then one slot per (wave, head of a group of up
        # to 16) for 8 waves per compute unit, then the 4097 prefix sums
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        assert got == ((rows * 130 + 3) // 4 * 4 + cus * 8 * 16 * 130 + 4097) * 4
    else:  # no device to size the persistent schedule for: the partition rows alone
        assert got == rows * 130 * 4
    assert lib.pkv_decode_workspace_bytes(30, 40, 128, 2048, 0) == 0
    assert lib.pkv_decode_workspace_bytes(3, 2, 64, 1, 16) == 3 * 2 * 1 * 66 * 4


def test_reshape_and_cache_rejects_bad_arguments():
    lib = _lib.load()
    f = lib.pkv_reshape_and_cache
    ok = dict(key=FAKE, value=FAKE, ks=512, vs=512, kc=FAKE, vc=FAKE, nb=4, slots=FAKE, T=3, hkv=4, d=128, B=16,
              dtype=1)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["key"], a["value"], a["ks"], a["vs"], a["kc"], a["vc"], a["nb"], a["slots"], a["T"], a["hkv"],
                 a["d"], a["B"], a["dtype"], NULL)

    assert call(dtype=5) == _lib.PKV_EINVAL
    assert call(ks=100) == _lib.PKV_EINVAL          # stride < Hkv * d
    assert call(ks=513) == _lib.PKV_EINVAL          # stride * elt not a multiple of 16
    assert call(key=NULL) == _lib.PKV_EINVAL
    assert call(d=4) == _lib.PKV_EINVAL             # row of 8 bytes
    assert call(T=0, key=NULL) == _lib.PKV_OK       # nothing to do


def test_copy_blocks_host_validation():
    lib = _lib.load()
    kp = (ctypes.c_void_p * 1)(1 << 20)
    vp = (ctypes.c_void_p * 1)(1 << 21)

    def call(pairs, nb=8, bb=4096):
        a = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1)
        return lib.pkv_copy_blocks(kp, vp, 1, nb, bb, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   len(a) // 2, NULL)

    assert call([0, 8]) == _lib.PKV_EINVAL           # out of range
    assert call([0, 3, 1, 3]) == _lib.PKV_EINVAL     # destination twice
    assert call([0, 3, 3, 4]) == _lib.PKV_EINVAL     # destination is also a source
    assert call([0, 3], bb=4100) == _lib.PKV_EINVAL  # block bytes not a multiple of 16
    assert call(np.zeros((0, 2))) == _lib.PKV_OK


def test_gpu_calls_fail_loudly_without_a_device():
    """No CPU fallback: a valid launch on a machine with no GPU reports a HIP error."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lib = _lib.load()
    slots = np.zeros(1, np.int64)
    rc = lib.pkv_reshape_and_cache(FAKE, FAKE, 512, 512, FAKE, FAKE, 4, slots.ctypes.data_as(ctypes.c_void_p), 1, 4,
                                   128, 16, 1, NULL)
    assert rc == _lib.PKV_EHIP


def test_read_probe_rejects_bad_arguments():
    lib = _lib.load()
    assert lib.pkv_read_probe(NULL, 1024, FAKE, NULL) == _lib.PKV_EINVAL
    assert lib.pkv_read_probe(FAKE, 1000, FAKE, NULL) == _lib.PKV_EINVAL  # not a multiple of 16
    assert lib.pkv_read_probe(ctypes.c_void_p((1 << 20) + 8), 1024, FAKE, NULL) == _lib.PKV_EINVAL
    assert lib.pkv_read_probe(FAKE, 0, FAKE, NULL) == _lib.PKV_OK


def test_balanced_split_refuses_more_than_4096_sequences():
    assert _attn(S=4097, P=-1) == _lib.PKV_EUNSUPPORTED
    assert "4096" in _lib.load().pkv_last_error().decode()


def test_swap_blocks_host_validation():
    lib = _lib.load()
    caches = (ctypes.c_void_p * 2)(FAKE, ctypes.c_void_p((1 << 30)))

    def call(pairs, bb=4096, ns=8, nd=4, src=caches, dst=None):
        pr = np.ascontiguousarray(np.asarray(pairs, np.int32).reshape(-1))
        d = dst if dst is not None else (ctypes.c_void_p * 2)(ctypes.c_void_p(1 << 31), ctypes.c_void_p(3 << 30))
        return lib.pkv_swap_blocks(src, d, 2, ns, nd, bb, pr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   len(pr) // 2, NULL)

    assert call([0, 4]) == _lib.PKV_EINVAL             # destination outside its pool
    assert call([8, 0]) == _lib.PKV_EINVAL             # source outside its pool
    assert call([0, 1, 2, 1]) == _lib.PKV_EINVAL       # a destination twice
    assert call([0, 1], bb=4100) == _lib.PKV_EINVAL    # block bytes not a multiple of 16
    assert call(np.zeros((0, 2))) == _lib.PKV_OK
    same = (ctypes.c_void_p * 2)(FAKE, ctypes.c_void_p(1 << 30))
    assert call([0, 1], src=same, dst=same) == _lib.PKV_EINVAL  # source overlaps destination
    # fake addresses are neither device nor pinned host memory: refused before any launch
    assert call([0, 1]) == _lib.PKV_EINVAL
    assert b"pinned" in lib.pkv_last_error()


def _prefill(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, num_blocks=10, tables=FAKE, max_blocks=4, ctx=FAKE, qs=FAKE, T=8,
             max_q=4, max_ctx=64, S=2, hq=8, hkv=2, d=128, B=16, scale=0.1, dtype=2, flags=0)
    a.update(kw)
    return _lib.load().pkv_paged_attention_prefill(a["out"], a["q"], a["k"], a["v"], a["num_blocks"], a["tables"],
                                                   a["max_blocks"], a["ctx"], a["qs"], a["T"], a["max_q"],
                                                   a["max_ctx"], a["S"], a["hq"], a["hkv"], a["d"], a["B"],
                                                   a["scale"], a["dtype"], a["flags"], NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), _lib.PKV_EINVAL),              # rows of q and out
    (dict(dtype=0), _lib.PKV_EUNSUPPORTED),     # fp32 has no matrix-core build
    (dict(d=64), _lib.PKV_EUNSUPPORTED),
    (dict(B=8), _lib.PKV_EUNSUPPORTED),
    (dict(hq=6, hkv=4), _lib.PKV_EINVAL),
    (dict(flags=1), _lib.PKV_EINVAL),
    (dict(qs=NULL), _lib.PKV_EINVAL),
    (dict(q=ctypes.c_void_p((1 << 20) + 8)), _lib.PKV_EINVAL),
    (dict(scale=float("inf")), _lib.PKV_EINVAL),
    (dict(max_blocks=0), _lib.PKV_EINVAL),
])
def test_prefill_rejects_bad_arguments(kw, code):
    assert _prefill(**kw) == code
    assert _lib.load().pkv_last_error()


def test_prefill_with_no_rows_is_a_no_op():
    assert _prefill(T=0, out=NULL, q=NULL) == _lib.PKV_OK
    assert _prefill(S=0, out=NULL, q=NULL) == _lib.PKV_OK


def test_prefill_wrapper_checks_the_table_shape():
    """The binding rejects a block table whose rows do not match the sequences before anything
    reaches the library (CPU tensors: the shape check comes first)."""
    torch = pytest.importorskip("torch")
    from paged_kv_cache_416_amd import kernels
    q = torch.zeros(6, 8, 128, dtype=torch.bfloat16)
    k = torch.zeros(4, 2, 16, 128, dtype=torch.bfloat16)
    ctx = torch.tensor([3, 3], dtype=torch.int32)
    qs = torch.tensor([0, 3, 6], dtype=torch.int32)
    for bad in (torch.zeros(3, 2, dtype=torch.int32), torch.zeros(4, dtype=torch.int32)):
        with pytest.raises(ValueError, match="block_tables"):
            kernels.paged_attention_prefill(torch.empty_like(q), q, k, k, bad, ctx, qs, 3, 3, 0.1)


def test_noalloc_decode_refuses_a_split_beyond_its_static_scratch():
    """The no-allocation decode call checks the split's workspace need against its static array
    before touching the device: 256 x 32 heads in 16-token parts of 9,216 tokens need 2.45 GB."""
    lib = _lib.load()
    rc = lib.pkv_paged_attention_decode_noalloc(FAKE, FAKE, FAKE, FAKE, 10, FAKE, 576, FAKE, 9216, 256, 32, 8, 128,
                                                16, 0.1, 16, 2, 0, NULL, NULL)
    assert rc == _lib.PKV_EINVAL
    assert b"static scratch" in lib.pkv_last_error()
    # the ordinary argument checks apply too
    assert lib.pkv_paged_attention_decode_noalloc(FAKE, FAKE, FAKE, FAKE, 10, FAKE, 4, FAKE, 64, 2, 4, 4, 96, 16,
                                                  0.1, 0, 1, 0, NULL, NULL) == _lib.PKV_EUNSUPPORTED
