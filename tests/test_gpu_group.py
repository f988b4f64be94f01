"""GPU parity of the group-wise value codec (codec.group = 16 or 32).

The codec is the value codec shared by the OCTOPUS experiments (Sec. 4, group
size 16 or 32), read from "Quantized Keys Steal Attention" (Sec. 3, Sec. 4.3,
Sec. 5): rotated values, per-group E4M3 step size and BF16 zero-point,
round-to-nearest codes.  Checked against the oracle (oracle/group.py):
  * octo_encode: scales, zero-points and codes bit-exact up to decision
    margins below 1e-6 (ragged tails, appends, fp32 inputs, zero, constant,
    tiny and huge vectors, the full-size workload on sampled tokens);
  * octo_decode_tokens: relative error <= 1e-5 on the GPU-written cache;
  * octo_attend_decode and octo_attend_chunk with OCTOPUS keys and group
    values: max-abs 2e-3 against the oracle's float64 attention on the
    GPU-written caches, at small ragged sizes, the full 32k-context size,
    empty and clipped lengths and several GQA group sizes;
  * octo_attend_chunk with group keys, with and without the Jensen-bias
    correction of cached logits (QKSA Sec. 4.2, Eq. 15), the same bar, and
    the correction's own effect well above the error.
"""
import numpy as np
import pytest
import torch

from gpu_parity import (ATOL, assert_group_encode_ok, codecs, compare_group_encode, encode_gpu,
                        group_codecs, make_inputs, oatt, octo, plane_of, say, workload)

pytestmark = pytest.mark.gpu

SPLITS = [(2, 32), (2, 16), (3, 32), (3, 16), (4, 32), (4, 16)]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("bits,group", SPLITS)
def test_group_encode_small(bits, group):
    w = workload("gqa32k")
    say(f"group encode b={bits} g={group}")
    x = make_inputs(w, scale_T=333)["V"]
    gc, hc = group_codecs(bits, group, seed=5)
    cache = encode_gpu(x, gc)
    assert_group_encode_ok(compare_group_encode(cache.to_host(), hc, x), f"b{bits} g{group}")


def test_group_encode_appends_and_fp32():
    w = workload("batch16", B=2)
    x = make_inputs(w, scale_T=200)["V"].float()
    gc, hc = group_codecs(3, 16)
    cache = encode_gpu(x[:, :, :37], gc, capacity=256)
    for lo, hi in ((37, 100), (100, 101), (101, 200)):
        encode_gpu(x[:, :, lo:hi], gc, token_offset=lo, cache=cache)
    assert_group_encode_ok(compare_group_encode(cache.to_host(), hc, x), "append fp32")


def test_group_encode_degenerate_vectors():
    """Zero and constant vectors (step 0: all codes 0), values small enough
    for subnormal E4M3 steps, values large enough to saturate the step at
    448, and single large entries."""
    g = torch.Generator().manual_seed(11)
    x = torch.randn(1, 1, 64, 128, generator=g)
    x[0, 0, 0] = 0.0
    x[0, 0, 1] = 2.5
    x[0, 0, 2:10] *= 1e-3
    x[0, 0, 10:14] *= 3e-5
    x[0, 0, 14:20] *= 3e3
    x[0, 0, 20:24] = 0.0
    x[0, 0, 20:24, 7] = 100.0
    for bits, group in SPLITS:
        gc, hc = group_codecs(bits, group)
        cache = encode_gpu(x, gc)
        st = compare_group_encode(cache.to_host(), hc, x)
        assert_group_encode_ok(st, f"degenerate b{bits} g{group}")
        rec = octo.octo_decode_tokens(gc, cache, 0, 64).cpu()
        assert torch.all(rec[0, 0, 0] == 0.0)                    # the zero vector decodes to zero


def test_group_encode_full_size_sampled():
    """The full-size 32k-context values (the benchmark's group-codec
    configuration) on a seeded sample of tokens in two planes."""
    w = workload("gqa32k_g32")
    x = make_inputs(w)["V"]
    gc, hc = group_codecs(w.bits, w.v_group)
    cache = encode_gpu(x, gc, capacity=w.capacity)
    T = x.shape[2]
    rng = np.random.default_rng(2)
    tokens = np.sort(rng.choice(T, size=384, replace=False))
    tokens[-1] = T - 1
    st = compare_group_encode(cache.to_host(), hc, x, planes=[(0, 0), (0, w.Hkv - 1)], tokens=tokens)
    assert_group_encode_ok(st, "full size")


@pytest.mark.parametrize("bits,group", SPLITS)
def test_group_decode_tokens(bits, group):
    gc, hc = group_codecs(bits, group, seed=3)
    g = torch.Generator().manual_seed(bits * group)
    x = torch.randn(2, 2, 150, 128, generator=g).to(torch.bfloat16)
    cache = encode_gpu(x, gc, capacity=192, token_offset=10)
    rec = octo.octo_decode_tokens(gc, cache, 10, 150).cpu().double().numpy()
    host = cache.to_host()
    worst = 0.0
    for b in range(2):
        for h in range(2):
            ref, _ = oatt.reconstruct(host, hc, b, h, 10, 150)
            err = np.linalg.norm(rec[b, h] - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
            worst = max(worst, float(err.max()))
    say(f"[group decode_tokens b={bits} g={group}] max relative error {worst:.2e}")
    assert worst <= 1e-5


def run_decode(w, group, T=None, seq_override=None, max_len=None, planes=None, q_f32=False):
    inp = make_inputs(w, scale_T=T)
    kc, hk = codecs(w.bits, qjl=w.qjl)
    vc, hv = group_codecs(w.bits, group)
    K, V, q = inp["K"], inp["V"], inp["q"]
    seq = inp["seq_lens"].clone() if seq_override is None else torch.tensor(seq_override, dtype=torch.int32)
    cap = -(-K.shape[2] // 64) * 64
    kcache = encode_gpu(K, kc, capacity=cap)
    vcache = encode_gpu(V, vc, capacity=cap)
    qd = q.float() if q_f32 else q
    out = octo.octo_attend_decode(kc, vc, kcache, vcache, qd.cuda(), seq.cuda(), max_len)
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()
    hkc, hvc = kcache.to_host(), vcache.to_host()
    lens = seq.numpy().copy()
    if max_len is not None:
        lens = np.minimum(lens, max_len)
    lens = np.clip(lens, 0, cap)
    qn = qd.double().numpy()
    G = w.Hq // w.Hkv
    planes = planes or [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    err = 0.0
    for b, g in planes:
        ref = oatt.decode_attention(qn[b:b + 1, g * G:(g + 1) * G], plane_of(hkc, b, g),
                                    plane_of(hvc, b, g), hk, hv, lens[b:b + 1])
        err = max(err, np.abs(out[b, g * G:(g + 1) * G] - ref[0]).max())
    return err, out, lens


@pytest.mark.parametrize("key,T,group", [("gqa32k", 1000, 32), ("gqa32k", 700, 16),
                                         ("batch16", 777, 32), ("batch16", 500, 16),
                                         ("long128k", 1500, 32), ("long128k", 900, 16),
                                         ("tiny", None, 16)])
def test_group_decode_small(key, T, group):
    w = workload(key)
    if key == "batch16":
        w = workload(key, B=5, len_lo=1, len_hi=T)
    say(f"group decode {key} T={T} g={group}")
    err, _, lens = run_decode(w, group, T)
    say(f"  lens {lens.tolist()} max-abs err {err:.3e}")
    assert err <= ATOL


def test_group_decode_full_size():
    """The 32k-context GQA workload with group-32 values (all outputs)."""
    w = workload("gqa32k_g32")
    say("group decode full gqa32k_g32")
    err, _, _ = run_decode(w, w.v_group)
    say(f"  max-abs err {err:.3e}")
    assert err <= ATOL


def test_group_decode_edges():
    """Empty sequence -> zero row; clipped lengths; fp32 queries; GQA groups."""
    w = workload("gqa32k", B=4)
    err, out, lens = run_decode(w, 32, T=600, seq_override=[0, 1, 599, 600], max_len=590)
    say(f"  edge lens {lens.tolist()} err {err:.3e}")
    assert err <= ATOL and np.all(out[0] == 0.0)
    err, _, _ = run_decode(workload("gqa32k"), 16, T=300, q_f32=True)
    assert err <= ATOL
    for Hq, Hkv in ((1, 1), (6, 2), (16, 1)):
        err, _, _ = run_decode(workload("gqa32k", Hq=Hq, Hkv=Hkv, outliers=False), 32, T=260)
        assert err <= ATOL, (Hq, Hkv)


@pytest.mark.parametrize("group,cached,tc", [(32, None, None), (16, 57, None), (32, None, 0)])
def test_group_chunk(group, cached, tc):
    w = workload("chunk", Hq=4, Hkv=2, T=300, chunk_q=150)
    inp = make_inputs(w)
    kc, hk = codecs(w.bits)
    vc, hv = group_codecs(w.bits, group)
    K, V = inp["K"], inp["V"]
    cached = K.shape[2] if cached is None else cached
    cap = -(-K.shape[2] // 64) * 64
    kcache = encode_gpu(K, kc, capacity=cap)
    vcache = encode_gpu(V, vc, capacity=cap)
    q, kcur, vcur = inp["q"], inp["K_cur"], inp["V_cur"]
    if tc is not None:
        kcur, vcur = kcur[:, :, :tc].contiguous(), vcur[:, :, :tc].contiguous()
    out = octo.octo_attend_chunk(kc, vc, kcache, vcache, cached, q.cuda(), kcur.cuda(), vcur.cuda())
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()
    hkc, hvc = kcache.to_host(), vcache.to_host()
    G = w.Hq // w.Hkv
    err = 0.0
    for h in range(w.Hq):
        g = h // G
        ref = oatt.chunk_attention(q[:, h:h + 1].double().numpy(), plane_of(hkc, 0, g),
                                   plane_of(hvc, 0, g), hk, hv, cached,
                                   kcur[:, g:g + 1].double().numpy(), vcur[:, g:g + 1].double().numpy())
        err = max(err, np.abs(out[0, h] - ref[0, 0]).max())
    say(f"group chunk g={group} cached={cached} tc={tc} err {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("kbits,kgroup,vbits,vgroup,correction,cached,tc,hq,hkv,tq", [
    (2, 32, 2, 32, False, None, None, 4, 2, 150),
    (2, 32, 2, 32, True, None, None, 4, 2, 150),
    (3, 16, 3, 16, True, 57, None, 4, 2, 150),
    (4, 32, 2, 16, True, None, 0, 4, 2, 150),
    (2, 16, 2, 32, True, 0, None, 4, 2, 150),
    # split tails with the correction: r = 2 and 1 leftover blocks a plane
    # (taken in the first pass, their query features in their own rows) and
    # r = 3 (a second pass)
    (2, 32, 2, 32, True, None, None, 4, 2, 280),
    (2, 32, 2, 32, True, None, None, 2, 2, 544),
    (2, 32, 2, 32, True, None, None, 2, 2, 608),
])
def test_group_keys_chunk_and_jensen_correction(kbits, kgroup, vbits, vgroup, correction, cached, tc,
                                                hq, hkv, tq):
    """Group-codec keys in the chunk path ("Quantized Keys Steal Attention"
    setting: group-wise round-to-nearest keys and values), with and without
    the Jensen-bias correction of cached logits (Eq. 15, its appendix on the
    rotation), against the oracle on the GPU-written caches."""
    w = workload("chunk", Hq=hq, Hkv=hkv, T=300, chunk_q=tq)
    inp = make_inputs(w)
    kc, hk = group_codecs(kbits, kgroup, seed=3)
    vc, hv = group_codecs(vbits, vgroup, seed=4)
    K, V = inp["K"], inp["V"]
    cached = K.shape[2] if cached is None else cached
    cap = -(-K.shape[2] // 64) * 64
    kcache = encode_gpu(K, kc, capacity=cap)
    vcache = encode_gpu(V, vc, capacity=cap)
    q, kcur, vcur = inp["q"], inp["K_cur"], inp["V_cur"]
    if tc is not None:
        kcur, vcur = kcur[:, :, :tc].contiguous(), vcur[:, :, :tc].contiguous()
    out = octo.octo_attend_chunk(kc, vc, kcache, vcache, cached, q.cuda(), kcur.cuda(), vcur.cuda(),
                                 correction=correction)
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()
    hkc, hvc = kcache.to_host(), vcache.to_host()
    G = w.Hq // w.Hkv
    err = moved = 0.0
    for h in range(w.Hq):
        g = h // G
        args = (q[:, h:h + 1].double().numpy(), plane_of(hkc, 0, g), plane_of(hvc, 0, g), hk, hv,
                cached, kcur[:, g:g + 1].double().numpy(), vcur[:, g:g + 1].double().numpy())
        ref = oatt.chunk_attention(*args, correction=correction)
        err = max(err, np.abs(out[0, h] - ref[0, 0]).max())
        if correction and cached and kcur.shape[2]:
            moved = max(moved, np.abs(ref - oatt.chunk_attention(*args)).max())
    say(f"group-key chunk K b{kbits} g{kgroup} V b{vbits} g{vgroup} corr={correction} "
        f"cached={cached} tc={tc}: err {err:.3e} (correction moves the output by {moved:.3e})")
    assert err <= ATOL
    if correction and cached and kcur.shape[2]:
        assert moved > 10 * err                     # the test sees the correction itself
