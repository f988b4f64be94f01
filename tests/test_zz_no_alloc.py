"""octo_attend_decode_noalloc (the workspace-free variant for callers that
cannot allocate) against octo_attend_decode, through the C ABI.

Two calls in a row, the second with a smaller input, so that the second
reads nothing the first left in the shared static scratch: each call's
outputs must equal octo_attend_decode's on the same inputs bit for bit (the
same kernels and split plan), and stay within the 2e-3 bar of the float64
oracle.  Shapes whose partials exceed the scratch are refused before any
launch.
"""
import numpy as np
import pytest
import torch

from gpu_parity import ATOL, codecs, encode_gpu, make_inputs, oatt, octo, say, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(key, T, B=None):
    w = workload(key) if B is None else workload(key, B=B)
    inp = make_inputs(w, scale_T=T)
    kc, hk = codecs(w.bits, qjl=w.qjl)
    vc, hv = codecs(w.bits)
    kcache = encode_gpu(inp["K"], kc)
    vcache = encode_gpu(inp["V"], vc)
    return inp, kc, vc, hk, hv, kcache, vcache


def test_noalloc_matches_workspace_entry_point():
    # the larger call first (batch 3, 2500 tokens), then a smaller one
    # (batch 1, 700 tokens, another bit split and QJL keys)
    for key, T, B in (("batch16", 2500, 3), ("long128k", 700, 1)):
        inp, kc, vc, hk, hv, kcache, vcache = _case(key, T, B)
        q, seq = inp["q"].cuda(), inp["seq_lens"].cuda()
        a = octo.octo_attend_decode_noalloc(kc, vc, kcache, vcache, q, seq)
        torch.cuda.synchronize()
        b = octo.octo_attend_decode(kc, vc, kcache, vcache, q, seq)
        torch.cuda.synchronize()
        say(f"noalloc {key} B={B} T={T}: equal {torch.equal(a, b)}")
        assert torch.equal(a, b)
        ref = oatt.decode_attention(inp["q"].double().numpy(), kcache.to_host(), vcache.to_host(),
                                    hk, hv, inp["seq_lens"].numpy())
        assert np.abs(a.cpu().double().numpy() - ref).max() <= ATOL


def test_noalloc_refuses_shapes_beyond_the_scratch():
    # 40000 (batch, query-head) rows of partials need more than 16 MiB
    kc, _ = codecs(3)
    vc, _ = codecs(3)
    B, Hkv, G = 2500, 4, 4
    kcache = octo.PackedCache(kc, B, Hkv, 64)
    vcache = octo.PackedCache(vc, B, Hkv, 64)
    q = torch.zeros(B, Hkv * G, 128, dtype=torch.bfloat16, device="cuda")
    seq = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(octo.OctoError, match="static"):
        octo.octo_attend_decode_noalloc(kc, vc, kcache, vcache, q, seq)
