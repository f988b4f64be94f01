"""C-ABI contract of liboctopus.so, on the host only (no kernel launch).

Checks that the library loads, exports every function include/octopus.h
declares, reports the record sizes of the bit splits (OCTOPUS paper Sec. 3.3:
B_tri = 2 b_dir + b_nrm bits per triplet, 43 triplets at d = 128), and that
every host-checkable error is reported before anything is launched.
"""
import ctypes

import numpy as np
import os
import re

import pytest

from quantized_decode_attention_octo_amd import binding as ob

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "octopus.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ob.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return ob.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(octo_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_function(L):
    names = header_functions()
    assert {"octo_encode", "octo_attend_decode", "octo_attend_chunk"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.octo_abi_version() == ob.ABI_VERSION
    for i, name in enumerate(ob.STATUS):
        assert L.octo_status_string(i).decode() == name
    assert L.octo_status_string(99).decode() == "OCTO_ERR_UNKNOWN"


_TABLE = np.linspace(-0.9, 0.9, 32).astype(np.float32)     # ascending, finite


def desc(bits=3, b_dir=0, b_nrm=0, qjl=0, head_dim=128, version=ob.ABI_VERSION, tables=True,
         rounding=0, table=_TABLE):
    p = table.ctypes.data if tables else 0
    return ob.CodecDesc(version, head_dim, bits, b_dir, b_nrm, rounding, qjl, 0, 0, p, p)


# words per token of the index stream (43 fields of 2 b_dir + b_nrm bits,
# padded to whole words) and of the QJL sketch of d = 128 bits
@pytest.mark.parametrize("bits,bd,bn,idx_w", [
    (4, 5, 3, 18), (3, 4, 2, 14), (2, 3, 1, 10),
    (4, 4, 4, 17), (3, 3, 3, 13), (2, 2, 2, 9)])
def test_record_sizes(L, bits, bd, bn, idx_w):
    explicit = (bd, bn) != (bits + 1, bits - 1)
    d = desc(bits, bd if explicit else 0, bn if explicit else 0, qjl=1, tables=False)
    s = ob.octo_record_sizes(d)
    assert (s.b_dir, s.b_nrm, s.n_triplets) == (bd, bn, 43)
    assert s.idx_words == idx_w == -(-(43 * (2 * bd + bn)) // 32)
    assert s.qjl_words == 4


def test_record_bytes_of_default_splits(L):
    # K record = index stream + gamma: 76 / 60 / 44 bytes at b = 4 / 3 / 2
    for bits, nbytes in ((4, 76), (3, 60), (2, 44)):
        s = ob.octo_record_sizes(desc(bits, tables=False))
        assert 4 * (s.idx_words + 1) == nbytes


def test_codec_errors(L):
    out = ob.StreamSizes()
    assert L.octo_record_sizes(None, ctypes.byref(out)) == 1
    assert L.octo_record_sizes(ctypes.byref(desc(version=7)), ctypes.byref(out)) == 6
    assert b"abi_version" in L.octo_last_error()
    assert L.octo_record_sizes(ctypes.byref(desc(head_dim=96)), ctypes.byref(out)) == 1
    assert L.octo_record_sizes(ctypes.byref(desc(head_dim=64)), ctypes.byref(out)) == 2
    assert L.octo_record_sizes(ctypes.byref(desc(bits=6)), ctypes.byref(out)) == 2
    # (1, 1) is no split of any kernel; (5, 1), a split of the (b + delta,
    # b - delta) sweep, only has its layout and the encoder
    assert L.octo_record_sizes(ctypes.byref(desc(b_dir=1, b_nrm=1)), ctypes.byref(out)) == 2
    assert L.octo_record_sizes(ctypes.byref(desc(b_dir=5, b_nrm=1)), ctypes.byref(out)) == 0
    assert L.octo_record_sizes(ctypes.byref(desc(rounding=5)), ctypes.byref(out)) == 1
    assert L.octo_record_sizes(ctypes.byref(desc(qjl=2)), ctypes.byref(out)) == 1
    assert L.octo_record_sizes(ctypes.byref(desc()), ctypes.byref(out)) == 0
    assert L.octo_last_error() == b""


def view(B=1, H=1, cap=128, ptr=4096, layout=0, qjl=False):
    q = ptr if qjl else None
    return ob.CacheView(ptr, ptr, q, q, B, H, cap, layout)


def enc(L, d, x, B, H, T, v, off, strides=(128 * 256, 128 * 256, 128, 1), dt=1):
    s = (ctypes.c_int64 * 4)(*strides)
    return L.octo_encode(ctypes.byref(d), x, dt, B, H, T, s, ctypes.byref(v) if v else None,
                         off, None)


def test_encode_errors(L):
    d = desc()
    x = ctypes.c_void_p(8192)
    assert enc(L, desc(tables=False), x, 1, 1, 64, view(), 0) == 1
    assert enc(L, d, x, 1, 1, 64, None, 0) == 1
    assert enc(L, d, x, 1, 1, 64, view(cap=100), 0) == 1
    assert enc(L, d, x, 1, 1, 64, view(layout=3), 0) == 1
    assert enc(L, d, x, 1, 1, 64, view(ptr=4100), 0) == 3
    assert enc(L, d, x, 2, 1, 64, view(), 0) == 1          # batch mismatch
    assert enc(L, d, x, 1, 1, 64, view(cap=128), 100) == 4  # beyond capacity
    assert enc(L, d, x, 1, 1, 64, view(), -1) == 1
    assert enc(L, d, x, 1, 1, 64, view(), 0, dt=5) == 1
    assert enc(L, d, x, 1, 1, 64, view(), 0, strides=(0, 0, 128, 2)) == 1
    assert enc(L, d, ctypes.c_void_p(8193), 1, 1, 64, view(), 0) == 3
    assert enc(L, desc(qjl=1), x, 1, 1, 64, view(), 0) == 1  # QJL needs its streams
    assert enc(L, d, x, 1, 1, 0, view(), 0) == 0            # T = 0: nothing to do


def test_codebook_values_are_checked(L):
    """The codebooks are host arrays read at each call: finite and ascending."""
    x = ctypes.c_void_p(8192)
    bad = _TABLE.copy()
    bad[3], bad[4] = bad[4], bad[3]                          # not ascending
    assert enc(L, desc(table=bad), x, 1, 1, 64, view(), 0) == 1
    assert b"ascending" in L.octo_last_error()
    bad = _TABLE.copy()
    bad[0] = np.nan
    assert enc(L, desc(table=bad), x, 1, 1, 64, view(), 0) == 1
    # only the 2^b_dir (2^b_nrm) leading values are read: a table whose tail is
    # not ascending is accepted for a smaller split
    tail = _TABLE.copy()
    tail[20] = -5.0
    assert enc(L, desc(table=tail), x, 1, 1, 0, view(), 0) == 0


def dec(L, kd, vd, kv, vv, Hq=4, lens=4096, max_len=128, out=4096, ws=4096, ws_bytes=1 << 20,
        q=4096, qdt=0):
    return L.octo_attend_decode(ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(kv),
                                ctypes.byref(vv), q, qdt, Hq, lens, max_len, 0.0, out, ws,
                                ws_bytes, None)


def test_sweep_splits_only_for_the_encoder(L):
    """A split of the (b + delta, b - delta) sweep beyond delta = 0, +1 has a
    record layout and the encoder, but no attention kernel."""
    sw = desc(bits=3, b_dir=5, b_nrm=1)
    assert dec(L, sw, sw, view(H=1), view(H=1), Hq=1) == 2
    assert b"not compiled" in L.octo_last_error()


def test_decode_errors(L):
    kd, vd = desc(), desc()
    kv, vv = view(H=2), view(H=2)
    assert dec(L, kd, vd, kv, vv, ws_bytes=0) == 5
    assert dec(L, kd, vd, kv, vv, ws=4097) == 3
    assert dec(L, kd, vd, kv, vv, Hq=3) == 1                 # not a multiple of kv_heads
    assert dec(L, kd, vd, kv, vv, Hq=34) == 2                # G = 17 > 16 MFMA columns
    assert dec(L, kd, vd, kv, vv, max_len=256) == 4          # beyond capacity
    assert dec(L, kd, desc(qjl=1), kv, view(H=2, qjl=True)) == 2   # QJL values
    assert dec(L, kd, desc(bits=2), kv, vv) == 2             # K/V split differ
    assert dec(L, kd, vd, kv, view(H=3)) == 1                # K/V shapes differ
    assert dec(L, kd, vd, kv, vv, q=None) == 1
    assert dec(L, kd, vd, kv, vv, qdt=7) == 1
    assert dec(L, kd, vd, kv, vv, lens=4098) == 3
    n = ctypes.c_size_t()
    assert L.octo_decode_workspace_bytes(ctypes.byref(kd), 1, 28, 4, 32768, ctypes.byref(n)) == 0
    assert n.value >= 28 * 130 * 4
    assert L.octo_decode_workspace_bytes(ctypes.byref(kd), 0, 28, 4, 32768, ctypes.byref(n)) == 1


def test_step_errors(L):
    """Host-side checks of octo_decode_step; no call here reaches a launch."""
    kd, vd = desc(), desc()
    kv, vv = view(H=2), view(H=2)
    n0, n1 = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.octo_decode_workspace_bytes(ctypes.byref(kd), 2, 4, 2, 128, ctypes.byref(n0)) == 0
    assert L.octo_decode_step_workspace_bytes(ctypes.byref(kd), 2, 4, 2, 128, ctypes.byref(n1)) == 0
    # 2 x 4 rows of one split: (m, l) pairs padded to 256 bytes, 128 sums per
    # partial; a step adds each sequence's (P, n), padded to 256 bytes
    assert n0.value == 256 + 2 * 4 * 1 * 128 * 4
    assert n1.value == n0.value + 256
    # the views below have batch 1: their workspace
    assert L.octo_decode_step_workspace_bytes(ctypes.byref(kd), 1, 4, 2, 128, ctypes.byref(n1)) == 0
    assert n1.value == 256 + 4 * 128 * 4 + 256
    p = ctypes.c_void_p(4096)

    def st(window=32, k_new=p, ring=p, lens=p, wlens=p, ws_bytes=n1.value, max_len=128):
        return L.octo_decode_step(ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(kv),
                                  ctypes.byref(vv), p, 0, 4, k_new, p, ring, p, window, lens,
                                  wlens, max_len, 0.0, p, p, ws_bytes, None)
    assert st(window=0) == 2
    assert st(window=257) == 2
    assert st(k_new=None) == 1
    assert st(wlens=None) == 1
    assert st(lens=None) == 1
    assert st(ring=ctypes.c_void_p(4097)) == 3
    assert st(ring=ctypes.c_void_p(4104)) == 3               # rows are read 16 bytes at a time
    assert st(k_new=ctypes.c_void_p(4104)) == 3
    assert st(wlens=ctypes.c_void_p(4098)) == 3
    assert st(ws_bytes=n1.value - 1) == 5
    assert st(max_len=129) == 4
    assert b"octo_decode_step" in L.octo_last_error()


def test_decode_tokens_errors(L):
    """Host-side checks of octo_decode_tokens; no call here reaches a launch."""
    kd = desc()
    kv = view(H=2)
    p = ctypes.c_void_p(4096)
    assert L.octo_decode_tokens(ctypes.byref(kd), ctypes.byref(kv), 0, 0, p, None) == 0   # nothing to do
    assert L.octo_decode_tokens(ctypes.byref(kd), ctypes.byref(kv), -1, 4, p, None) == 1
    assert L.octo_decode_tokens(ctypes.byref(kd), ctypes.byref(kv), 100, 29, p, None) == 4  # past 128
    assert L.octo_decode_tokens(ctypes.byref(kd), ctypes.byref(kv), 0, 4, None, None) == 1
    assert L.octo_decode_tokens(ctypes.byref(kd), ctypes.byref(kv), 0, 4, ctypes.c_void_p(4098), None) == 3
    assert L.octo_decode_tokens(ctypes.byref(desc(tables=False)), ctypes.byref(kv), 0, 4, p, None) == 1
    assert L.octo_decode_tokens(ctypes.byref(kd), None, 0, 4, p, None) == 1


def test_chunk_errors(L):
    kd, vd = desc(bits=2), desc(bits=2)
    kv, vv = view(H=2, cap=256), view(H=2, cap=256)
    n = ctypes.c_size_t()
    assert L.octo_chunk_workspace_bytes(ctypes.byref(kd), 1, 2, 2, 64, 128, 64, 0, ctypes.byref(n)) == 0
    need = n.value
    # the current chunk's rotated key rows [1, 2, 64, 128] and value rows
    # [1, 2, 64, 128]; the queries are rotated and the cached window decoded
    # inside the kernel
    assert need == 2 * 64 * 256 + 2 * 64 * 256
    # the same with 128 cached tokens more: nothing of the window is staged
    assert L.octo_chunk_workspace_bytes(ctypes.byref(kd), 1, 2, 2, 64, 256, 64, 0, ctypes.byref(n)) == 0
    assert n.value == need
    # the correction's query and key features are formed in the kernel
    assert L.octo_chunk_workspace_bytes(ctypes.byref(kd), 1, 2, 2, 64, 128, 64, 1, ctypes.byref(n)) == 0
    assert n.value == need
    assert L.octo_chunk_workspace_bytes(ctypes.byref(kd), 1, 2, 2, 64, 128, 64, 2, ctypes.byref(n)) == 1

    def ch(kd=kd, vd=vd, kv=kv, vv=vv, cached=128, Hq=2, Tq=64, Tc=64, ws=4096, ws_bytes=need,
           flags=0, qp=4096):
        p = ctypes.c_void_p(4096)
        return L.octo_attend_chunk(ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(kv),
                                   ctypes.byref(vv), cached, ctypes.c_void_p(qp), p, p, Hq, Tq, Tc,
                                   0.0, flags, p, ws, ws_bytes, None)
    assert ch(ws_bytes=need - 1) == 5
    assert ch(ws=4352 + 1) == 3
    assert ch(qp=4096 + 8) == 3                              # rows are read 16 bytes a lane
    assert ch(cached=300) == 4
    assert ch(Hq=3) == 1
    assert ch(Tq=-1) == 1
    assert ch(kd=desc(bits=2, qjl=1), kv=view(H=2, cap=256, qjl=True)) == 2
    assert ch(Tq=0) == 0                                     # nothing to do
    assert ch(flags=4) == 1                                  # unknown flag
    assert ch(flags=1) == 2                                  # correction with OCTOPUS keys
    # a plane's current value rows beyond 2 GiB (2^23 keys x 288 B): unsupported
    assert ch(Tc=1 << 23, ws_bytes=1 << 62) == 2
    # a plane's packed stream beyond 2 GiB (2^26 tokens x 9 words x 4 B): unsupported
    big = view(H=2, cap=1 << 26)
    assert ch(kv=big, vv=big, cached=1 << 20, Tc=64, ws_bytes=1 << 62) == 2


def gdesc(bits=2, group=32, b_dir=0, b_nrm=0, qjl=0):
    """Descriptor of the group-wise value codec (no codebooks)."""
    return ob.CodecDesc(ob.ABI_VERSION, 128, bits, b_dir, b_nrm, 0, qjl, group, 0, None, None)


@pytest.mark.parametrize("bits,group,words", [(2, 32, 11), (2, 16, 14), (3, 32, 15), (3, 16, 18),
                                              (4, 32, 19), (4, 16, 22)])
def test_group_record_sizes(L, bits, group, words):
    # 128 codes of b bits, 128/g E4M3 scales and 128/g BF16 zero-points:
    # b + 24/g bits per coordinate ("Quantized Keys Steal Attention", Sec. 4.3)
    out = ob.StreamSizes()
    assert L.octo_record_sizes(ctypes.byref(gdesc(bits, group)), ctypes.byref(out)) == 0
    assert out.idx_words == words == (128 * bits + 24 * 128 // group) // 32
    assert (out.qjl_words, out.n_triplets, out.b_dir, out.b_nrm) == (0, 0, 0, 0)


def test_group_codec_errors(L):
    out = ob.StreamSizes()

    def rs(d):
        return L.octo_record_sizes(ctypes.byref(d), ctypes.byref(out))
    assert rs(gdesc(group=24)) == 2
    assert rs(gdesc(group=-16)) == 1
    assert rs(gdesc(bits=5)) == 2
    assert rs(gdesc(bits=9)) == 1
    assert rs(gdesc(b_dir=3, b_nrm=1)) == 1
    assert rs(gdesc(qjl=1)) == 2
    # a group cache needs no gamma stream
    gv = view(H=2)
    gv.gamma = None
    p = ctypes.c_void_p(4096)
    kd = desc(bits=2)
    # keys need the OCTOPUS codec; values need the same b with a (b+1, b-1) key split
    assert dec(L, gdesc(), gdesc(), gv, gv) == 2
    assert dec(L, kd, gdesc(bits=3), view(H=2), gv) == 2
    assert dec(L, desc(bits=2, b_dir=2, b_nrm=2), gdesc(bits=2), view(H=2), gv) == 2
    assert dec(L, kd, gdesc(bits=2), view(H=2), gv, ws_bytes=0) == 5        # accepted up to here
    n = ctypes.c_size_t()
    assert L.octo_decode_workspace_bytes(ctypes.byref(gdesc()), 1, 4, 2, 128, ctypes.byref(n)) == 2
    # the chunk path takes group keys (and the correction needs them)
    assert L.octo_chunk_workspace_bytes(ctypes.byref(gdesc()), 1, 2, 2, 64, 128, 64, 1,
                                        ctypes.byref(n)) == 0
    assert L.octo_attend_chunk(ctypes.byref(gdesc()), ctypes.byref(gdesc()), ctypes.byref(gv),
                               ctypes.byref(gv), 64, p, p, p, 2, 64, 64, 0.0, 1, p, p, 16,
                               None) == 5
    assert L.octo_decode_tokens(ctypes.byref(gdesc()), ctypes.byref(gv), 100, 29, p, None) == 4
    assert L.octo_decode_tokens(ctypes.byref(gdesc()), ctypes.byref(gv), 0, 4, None, None) == 1


def test_noalloc_refuses_oversized_shapes_on_the_host(L):
    """octo_attend_decode_noalloc checks that the call's partials fit its
    static scratch before touching any device."""
    d = desc(bits=3)
    cache = ob.CacheView(None, None, None, None, 2500, 4, 64, 0)
    st = L.octo_attend_decode_noalloc(ctypes.byref(d), ctypes.byref(d), ctypes.byref(cache),
                                      ctypes.byref(cache), None, 1, 16, None, 64,
                                      ctypes.c_float(0.0), None, None)
    assert ob.STATUS[st] == "OCTO_ERR_CAPACITY"
    assert b"static" in L.octo_last_error()
