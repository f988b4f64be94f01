"""GPU parity of octo_decode_step (the decode step with a native-precision
residual window) against the oracle's step, oracle/step.py.

Each step compares:
  * the attention output with the oracle's float64 step on the same packed
    cache and ring (max-abs 2e-3);
  * the lengths (packed P_b and ring n_b) exactly;
  * the ring rows of the live tokens exactly (bf16);
  * the token that left the window: its packed slot, written by the step's
    one-wavefront encoder, against the oracle's encoding of the ring row
    (bit-exact indices outside the 1e-6 margins, gamma within 4 ulps).
After each step the oracle continues from the GPU-written cache, so every
step is judged on identical inputs.  Small cases span several splits, W = 1
(every token compressed after its step), W = 5 and 8, QJL keys, sequences of
different packed lengths and partly filled rings, and values in the
group-wise codec (its evicted records compared as octo_encode's are); the
full-size cases are the 32k-context GQA shape with a 32-token window.
"""
import numpy as np
import pytest
import torch

from gpu_parity import (ATOL, assert_encode_ok, assert_group_encode_ok, codecs, compare_encode,
                        compare_group_encode, encode_gpu, group_codecs, octo, say)
from oracle import step as ostep

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bf16(g, *shape, scale=1.0):
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


def run_steps(bits, qjl, W, G, Hkv, P0, n0, steps, cap, seed=0, q_f32=False, check_every=1,
              v_group=0):
    B = len(P0)
    Hq = G * Hkv
    kc, hk = codecs(bits, qjl=qjl, seed=seed)
    vc, hv = group_codecs(bits, v_group, seed=seed) if v_group else codecs(bits, seed=seed)
    g = torch.Generator().manual_seed(100 + seed)
    Tpre = max(p + n for p, n in zip(P0, n0))
    K0, V0 = bf16(g, B, Hkv, Tpre, 128), bf16(g, B, Hkv, Tpre, 128)
    kcache = encode_gpu(K0, kc, capacity=cap)
    vcache = encode_gpu(V0, vc, capacity=cap)
    kring = torch.zeros(B, Hkv, W, 128, dtype=torch.bfloat16)
    vring = torch.zeros(B, Hkv, W, 128, dtype=torch.bfloat16)
    for b in range(B):
        for j in range(n0[b]):
            kring[b, :, (P0[b] + j) % W] = K0[b, :, P0[b] + j]
            vring[b, :, (P0[b] + j) % W] = V0[b, :, P0[b] + j]
    st = ostep.new_state(hk, hv, B, Hkv, cap, W)
    st["k"], st["v"] = kcache.to_host(), vcache.to_host()
    st["k_ring"], st["v_ring"] = kring.double().numpy(), vring.double().numpy()
    st["P"], st["n"] = np.array(P0), np.array(n0)
    kr, vr = kring.cuda(), vring.cuda()
    plens = torch.tensor(P0, dtype=torch.int32).cuda()
    wlens = torch.tensor(n0, dtype=torch.int32).cuda()
    worst = 0.0
    for s in range(steps):
        q = bf16(g, B, Hq, 128)
        kn, vn = bf16(g, B, Hkv, 128), bf16(g, B, Hkv, 128)
        Pb = st["P"].copy()
        out = octo.octo_decode_step(kc, vc, kcache, vcache, (q.float() if q_f32 else q).cuda(),
                                    kn.cuda(), vn.cuda(), kr, vr, plens, wlens, cap)
        torch.cuda.synchronize()
        ref = ostep.decode_step(st, q.double().numpy(), kn.double().numpy(), vn.double().numpy(),
                                hk, hv)
        err = float(np.abs(out.cpu().double().numpy() - ref).max())
        worst = max(worst, err)
        assert err <= ATOL, (s, err)
        assert plens.cpu().tolist() == st["P"].tolist()
        assert wlens.cpu().tolist() == st["n"].tolist()
        if s % check_every == 0 or s == steps - 1:
            ring_k = kr.cpu().double().numpy()
            ring_v = vr.cpu().double().numpy()
            for b in range(B):
                for j in range(int(st["n"][b])):
                    slot = (int(st["P"][b]) + j) % W
                    assert np.array_equal(ring_k[b, :, slot], st["k_ring"][b, :, slot])
                    assert np.array_equal(ring_v[b, :, slot], st["v_ring"][b, :, slot])
        hk_now, hv_now = kcache.to_host(), vcache.to_host()
        for b in range(B):
            if st["P"][b] == Pb[b]:
                continue
            P = int(Pb[b])
            xk = torch.zeros(B, Hkv, 1, 128, dtype=torch.float64)
            xv = torch.zeros(B, Hkv, 1, 128, dtype=torch.float64)
            # the evicted rows, as the oracle saw them before its step
            xk[b, :, 0] = torch.tensor(st["k_ring"][b, :, P % W]) if W > 1 else kn[b].double()
            xv[b, :, 0] = torch.tensor(st["v_ring"][b, :, P % W]) if W > 1 else vn[b].double()
            planes = [(b, h) for h in range(Hkv)]
            assert_encode_ok(compare_encode(hk_now, hk, xk, P, planes=planes), f"step K b={b}")
            if v_group:
                assert_group_encode_ok(compare_group_encode(hv_now, hv, xv, P, planes=planes),
                                       f"step V b={b}")
            else:
                assert_encode_ok(compare_encode(hv_now, hv, xv, P, planes=planes), f"step V b={b}")
        # continue from the GPU-written cache
        st["k"], st["v"] = hk_now, hv_now
    say(f"[step bits={bits} qjl={qjl} W={W} G={G}] {steps} steps, max-abs err {worst:.2e}")
    return worst


@pytest.mark.parametrize("bits,qjl,W,G,P0,n0", [
    (3, False, 8, 4, [300, 61], [0, 5]),
    (2, True, 5, 7, [130, 1], [4, 2]),
    (4, False, 1, 2, [64, 200], [0, 0]),
    (4, True, 8, 1, [0, 9], [0, 7]),
])
def test_step_small(bits, qjl, W, G, P0, n0):
    run_steps(bits, qjl, W, G, Hkv=2, P0=P0, n0=n0, steps=2 * W + 3, cap=512)


def test_step_fp32_queries_and_uniform_split():
    run_steps(3, False, 4, 3, Hkv=1, P0=[100], n0=[3], steps=6, cap=256, q_f32=True)


def test_step_fills_an_empty_state():
    # no packed token at all: the first W steps are attention over the ring only
    run_steps(3, False, 6, 2, Hkv=2, P0=[0, 0], n0=[0, 0], steps=9, cap=128)


def test_step_full_size_gqa32k():
    # the 32k-context GQA shape (28/4 heads, b = 4) with a full 32-token window
    run_steps(4, False, 32, 7, Hkv=4, P0=[32768 - 64], n0=[31], steps=3, cap=32768,
              check_every=3)


@pytest.mark.parametrize("bits,qjl,W,G,P0,n0,group", [
    (3, False, 8, 4, [300, 61], [0, 5], 32),
    (2, True, 5, 7, [130, 1], [4, 2], 16),
    (4, False, 1, 2, [64, 200], [0, 0], 16),
])
def test_step_group_values(bits, qjl, W, G, P0, n0, group):
    run_steps(bits, qjl, W, G, Hkv=2, P0=P0, n0=n0, steps=2 * W + 3, cap=512, v_group=group)


def test_step_full_size_gqa32k_group_values():
    run_steps(4, False, 32, 7, Hkv=4, P0=[32768 - 64], n0=[31], steps=3, cap=32768,
              check_every=3, v_group=32)
