"""The binding's argument checks, on the host only.

The C ABI sees plain pointers, so the tensor shapes, dtypes, layouts and
devices that the kernels assume (d = 128 columns, one row per (batch, head),
the cache's batch and KV heads) can only be checked in the binding.  Each
case below hands one wrong tensor to an entry point and expects ValueError
before anything reaches the library or a device: the caches are allocated
in host memory here, so a check that let a call through would fail on the
device check instead, and the message would say so.
"""
import pytest
import torch

import quantized_decode_attention_octo_amd as octo
from quantized_decode_attention_octo_amd import binding as ob


@pytest.fixture(scope="module")
def setup():
    if not __import__("os").path.exists(ob.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    kc = octo.Codec(bits=4, device="cpu")
    vc = octo.Codec(bits=4, device="cpu")
    B, Hkv, cap = 2, 2, 128
    kcache = octo.PackedCache(kc, B, Hkv, cap, device="cpu")
    vcache = octo.PackedCache(vc, B, Hkv, cap, device="cpu")
    return kc, vc, kcache, vcache


def _raises(fn, *a, match=None, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_encode_shapes(setup):
    kc, _, kcache, _ = setup
    bf = torch.bfloat16
    _raises(ob.octo_encode, kc, torch.zeros(2, 2, 5, 64, dtype=bf), kcache, match="shape")
    _raises(ob.octo_encode, kc, torch.zeros(3, 2, 5, 128, dtype=bf), kcache, match="shape")
    _raises(ob.octo_encode, kc, torch.zeros(2, 1, 5, 128, dtype=bf), kcache, match="shape")
    _raises(ob.octo_encode, kc, torch.zeros(2, 2, 5, 128, dtype=torch.float16), kcache,
            match="dtype")
    _raises(ob.octo_encode, kc, torch.zeros(2, 2, 128, 5, dtype=bf).transpose(2, 3), kcache,
            match="device|stride")
    # the right shape in host memory: rejected as not on a device
    _raises(ob.octo_encode, kc, torch.zeros(2, 2, 5, 128, dtype=bf), kcache, match="device")
    # a cache allocated for another codec
    other = octo.Codec(bits=3, device="cpu")
    _raises(ob.octo_encode, other, torch.zeros(2, 2, 5, 128, dtype=bf), kcache, match="codec|device")


def test_decode_shapes(setup):
    kc, vc, kcache, vcache = setup
    bf, i32 = torch.bfloat16, torch.int32
    seq = torch.zeros(2, dtype=i32)
    q = torch.zeros(2, 4, 128, dtype=bf)
    for bad, m in ((torch.zeros(2, 4, 64, dtype=bf), "shape"),      # d = 64
                   (torch.zeros(3, 4, 128, dtype=bf), "shape"),     # batch 3 on a batch-2 cache
                   (torch.zeros(2, 3, 128, dtype=bf), "multiple"),  # 3 heads on 2 KV heads
                   (torch.zeros(2, 4, 128, dtype=torch.float16), "dtype"),
                   (torch.zeros(2, 128, 4, dtype=bf).transpose(1, 2), "shape|contiguous")):
        _raises(ob.octo_attend_decode, kc, vc, kcache, vcache, bad, seq, match=m)
    _raises(ob.octo_attend_decode, kc, vc, kcache, vcache, q, torch.zeros(3, dtype=i32),
            match="shape")
    _raises(ob.octo_attend_decode, kc, vc, kcache, vcache, q, torch.zeros(2, dtype=torch.int64),
            match="dtype")
    _raises(ob.octo_attend_decode, kc, vc, kcache, vcache, q, seq,
            out=torch.zeros(2, 4, 64), match="shape|device")
    _raises(ob.octo_attend_decode, kc, vc, kcache, vcache, q, seq, match="device")
    small = octo.PackedCache(vc, 2, 2, 64, device="cpu")
    _raises(ob.octo_attend_decode, kc, vc, kcache, small, q, seq, match="differ")
    v3 = octo.Codec(bits=3, device="cpu")
    _raises(ob.octo_attend_decode, kc, v3, kcache, vcache, q, seq, match="codec")


def test_step_shapes(setup):
    kc, vc, kcache, vcache = setup
    bf, i32 = torch.bfloat16, torch.int32
    q = torch.zeros(2, 4, 128, dtype=bf)
    new = torch.zeros(2, 2, 128, dtype=bf)
    ring = torch.zeros(2, 2, 8, 128, dtype=bf)
    lens = torch.zeros(2, dtype=i32)
    good = dict(q=q, k_new=new, v_new=new, k_window=ring, v_window=ring, packed_lens=lens,
                window_lens=lens)

    def call(**over):
        a = dict(good, **over)
        return ob.octo_decode_step(kc, vc, kcache, vcache, a["q"], a["k_new"], a["v_new"],
                                   a["k_window"], a["v_window"], a["packed_lens"],
                                   a["window_lens"])
    for over, m in ((dict(k_new=torch.zeros(2, 2, 64, dtype=bf)), "shape"),
                    (dict(v_new=torch.zeros(2, 3, 128, dtype=bf)), "shape"),
                    (dict(k_window=torch.zeros(2, 2, 8, 64, dtype=bf)), "shape"),
                    (dict(v_window=torch.zeros(2, 2, 4, 128, dtype=bf)), "shape"),
                    (dict(k_new=torch.zeros(2, 2, 128)), "dtype"),
                    (dict(packed_lens=torch.zeros(1, dtype=i32)), "shape"),
                    (dict(window_lens=torch.zeros(2, dtype=torch.int64)), "dtype"),
                    (dict(q=torch.zeros(1, 4, 128, dtype=bf)), "shape"),
                    ({}, "device")):
        with pytest.raises(ValueError, match=m):
            call(**over)


def test_chunk_shapes(setup):
    kc, vc, kcache, vcache = setup
    bf = torch.bfloat16
    q = torch.zeros(2, 4, 16, 128, dtype=bf)
    cur = torch.zeros(2, 2, 8, 128, dtype=bf)
    f = ob.octo_attend_chunk
    _raises(f, kc, vc, kcache, vcache, 64, torch.zeros(2, 4, 16, 64, dtype=bf), cur, cur, match="shape")
    _raises(f, kc, vc, kcache, vcache, 64, torch.zeros(2, 3, 16, 128, dtype=bf), cur, cur,
            match="multiple")
    _raises(f, kc, vc, kcache, vcache, 64, q, torch.zeros(2, 1, 8, 128, dtype=bf), cur, match="shape")
    _raises(f, kc, vc, kcache, vcache, 64, q, cur, torch.zeros(2, 2, 9, 128, dtype=bf), match="shape")
    _raises(f, kc, vc, kcache, vcache, 64, q, cur, torch.zeros(2, 2, 8, 128), match="dtype")
    _raises(f, kc, vc, kcache, vcache, 64, q.float(), cur, cur, match="dtype")
    _raises(f, kc, vc, kcache, vcache, 64, q, cur, cur, match="device")


def test_decode_tokens_shapes(setup):
    kc, _, kcache, _ = setup
    _raises(ob.octo_decode_tokens, kc, kcache, 0, 4, out=torch.zeros(2, 2, 4, 64), match="shape")
    _raises(ob.octo_decode_tokens, kc, kcache, 0, 4, out=torch.zeros(2, 2, 4, 128), match="device")
