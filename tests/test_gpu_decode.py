"""GPU parity of octo_attend_decode against the oracle's float64 attention on
the GPU-written packed cache (max-abs 2e-3).

Small cases span several 64-token tiles, several splits and ragged tails;
the full-size cases are the benchmark's configurations (all outputs for the
32k-context and batched workloads, sampled planes at 128k context).  Edge
cases: empty sequences, lengths clipped by max_seq_len, fp32 queries, every
GQA group size from 1 to 16, determinism, repeated calls on one workspace.
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


def run_case(w, T=None, seq_override=None, max_len=None, q_f32=False, planes=None,
             split=(None, None), v_own_tables=False):
    inp = make_inputs(w, scale_T=T)
    kc, hk = codecs(w.bits, qjl=w.qjl, b_dir=split[0], b_nrm=split[1])
    vc, hv = codecs(w.bits, b_dir=split[0], b_nrm=split[1])
    if v_own_tables:
        # same values at other addresses: the kernels cannot share one table
        vc = octo.Codec(bits=w.bits, b_dir=split[0], b_nrm=split[1],
                        tables=octo.binding.load_codebooks(128))
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
    if planes is None:
        ref = oatt.decode_attention(qn, hkc, hvc, hk, hv, lens)
        err = np.abs(out - ref).max()
    else:
        # only the query heads of the sampled (batch, kv head) planes
        G = w.Hq // w.Hkv
        err = 0.0
        for b, g in planes:
            ref = oatt.decode_attention(qn[b:b + 1, g * G:(g + 1) * G], _plane(hkc, b, g),
                                        _plane(hvc, b, g), hk, hv, lens[b:b + 1])
            err = max(err, np.abs(out[b, g * G:(g + 1) * G] - ref[0]).max())
    return err, out, lens


def _plane(h, b, g):
    """The host cache of plane (b, g) alone (same layout with B = H = 1)."""
    n = h["B"] * h["H"]
    p = b * h["H"] + g
    out = {"B": 1, "H": 1, "capacity": h["capacity"],
           "idx": h["idx"].reshape(n, -1)[p],
           "gamma": h["gamma"][b:b + 1, g:g + 1]}
    if "qjl" in h:
        out["qjl"] = h["qjl"].reshape(n, -1)[p]
        out["gamma_r"] = h["gamma_r"][b:b + 1, g:g + 1]
    return out


@pytest.mark.parametrize("key,T", [("tiny", None), ("gqa32k", 1000), ("batch16", 777),
                                   ("long128k", 1500)])
def test_decode_small(key, T):
    w = workload(key)
    if key == "batch16":
        w = workload(key, B=5, len_lo=1, len_hi=T)
    say(f"decode {key} T={T}")
    err, _, lens = run_case(w, T)
    say(f"  lens {lens.tolist()} max-abs err {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("split", [(5, 3), (4, 4), (4, 2), (3, 3), (3, 1), (2, 2)])
@pytest.mark.parametrize("own", [False, True])
def test_decode_table_modes(split, own):
    """Every bit split, with K and V sharing their codebook tables (one
    pre-split LDS table, the one-workgroup-per-CU mode for the big splits) and
    with V's tables at other addresses (separate tables; the fp32 table for
    the big splits)."""
    bits = (split[0] + split[1]) // 2
    w = workload("gqa32k", bits=bits)
    say(f"decode split {split} own V tables {own}")
    err, _, _ = run_case(w, T=1100, split=split, v_own_tables=own)
    say(f"  max-abs err {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("key", ["gqa32k", "batch16"])
def test_decode_full_size(key):
    w = workload(key)
    say(f"decode full {key}")
    err, _, lens = run_case(w)
    say(f"  lens {lens.tolist()} max-abs err {err:.3e}")
    assert err <= ATOL


def test_decode_full_size_long_context_sampled():
    w = workload("long128k")
    say("decode full long128k (planes (0,0) and (3,3))")
    err, _, _ = run_case(w, planes=[(0, 0), (3, 3)])
    say(f"  max-abs err {err:.3e}")
    assert err <= ATOL


def test_decode_edge_lengths():
    """Empty sequence -> zero row; max_seq_len clips the context; lengths that
    end inside a tile and inside a split."""
    w = workload("gqa32k", B=4)
    err, out, lens = run_case(w, T=600, seq_override=[0, 1, 599, 600], max_len=590)
    say(f"  edge lens {lens.tolist()} err {err:.3e}")
    assert err <= ATOL
    assert np.all(out[0] == 0.0)


def test_decode_fp32_queries():
    err, _, _ = run_case(workload("gqa32k"), T=300, q_f32=True)
    assert err <= ATOL


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (6, 2), (8, 2), (16, 2), (7, 1), (32, 2)])
def test_decode_group_sizes(Hq, Hkv):
    w = workload("gqa32k", Hq=Hq, Hkv=Hkv, outliers=False)
    err, _, _ = run_case(w, T=260)
    assert err <= ATOL


def test_decode_many_splits():
    """One KV head over a long context: more splits than the merge takes in
    one round (its running-maximum rescale across rounds), big-table mode."""
    w = workload("gqa32k", Hq=7, Hkv=1)
    say("decode 7/1 heads, 40000 tokens")
    err, _, _ = run_case(w, T=40000)
    say(f"  max-abs err {err:.3e}")
    assert err <= ATOL


def test_decode_deterministic():
    w = workload("gqa32k")
    inp = make_inputs(w, scale_T=2000)
    kc, _ = codecs(4)
    vc, _ = codecs(4)
    kcache = encode_gpu(inp["K"], kc)
    vcache = encode_gpu(inp["V"], vc)
    q, seq = inp["q"].cuda(), inp["seq_lens"].cuda()
    a = octo.octo_attend_decode(kc, vc, kcache, vcache, q, seq).cpu()
    b = octo.octo_attend_decode(kc, vc, kcache, vcache, q, seq).cpu()
    assert torch.equal(a, b)


def test_decode_reuses_workspace():
    """The workspace holds no state between calls: back-to-back calls on one
    workspace, with different shapes, keep matching the oracle."""
    ws = octo.workspace(1 << 22, "cuda")
    for T, key in ((700, "gqa32k"), (300, "long128k"), (700, "gqa32k")):
        w = workload(key)
        inp = make_inputs(w, scale_T=T)
        kc, hk = codecs(w.bits, qjl=w.qjl)
        vc, hv = codecs(w.bits)
        kcache = encode_gpu(inp["K"], kc)
        vcache = encode_gpu(inp["V"], vc)
        out = octo.octo_attend_decode(kc, vc, kcache, vcache, inp["q"].cuda(),
                                      inp["seq_lens"].cuda(), ws=ws)
        ref = oatt.decode_attention(inp["q"].double().numpy(), kcache.to_host(),
                                    vcache.to_host(), hk, hv, inp["seq_lens"].numpy())
        assert np.abs(out.cpu().double().numpy() - ref).max() <= ATOL


@pytest.mark.parametrize("key,B,T", [("gqa32k", 1, 1000), ("batch16", 32, 8192)])
def test_decode_graph_replays(key, B, T):
    """One call (scan and merge launches) captured in a HIP graph and
    replayed four times, with an eager call on the same workspace between
    replays: every replay matches the eager result bit for bit.  The 32k GQA
    shape (b = 4: one eight-wave workgroup a CU) and 32 sequences of up to
    8192 tokens (b = 3: two four-wave workgroups a CU)."""
    w = workload(key, B=B)
    inp = make_inputs(w, scale_T=T)
    kc, _ = codecs(w.bits)
    vc, _ = codecs(w.bits)
    kcache = encode_gpu(inp["K"], kc)
    vcache = encode_gpu(inp["V"], vc)
    q, seq = inp["q"].cuda(), inp["seq_lens"].cuda()
    max_len = int(inp["seq_lens"].max())
    ws = octo.workspace(octo.octo_decode_workspace_bytes(kc, w.B, w.Hq, w.Hkv, max_len), "cuda")
    out = torch.empty(w.B, w.Hq, 128, dtype=torch.float32, device="cuda")
    ref = octo.octo_attend_decode(kc, vc, kcache, vcache, q, seq, max_len, ws=ws).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        octo.octo_attend_decode(kc, vc, kcache, vcache, q, seq, max_len, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        octo.octo_attend_decode(kc, vc, kcache, vcache, q, seq, max_len, out=out, ws=ws)
    torch.cuda.synchronize()
    for i in range(4):
        say(f"decode graph replay {i}")
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        eager = octo.octo_attend_decode(kc, vc, kcache, vcache, q, seq, max_len, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(eager, ref), f"eager call after replay {i}"


def test_decode_max_len_zero():
    """max_seq_len = 0: every row is zero (the scan's speculative first-block
    loads read a zeroed device block instead of the cache)."""
    w = workload("gqa32k", B=2)
    err, out, lens = run_case(w, T=128, seq_override=[5, 128], max_len=0)
    assert err <= ATOL
    assert np.all(out == 0.0)


@pytest.mark.parametrize("vscale", [300.0, 3000.0])
def test_decode_large_value_norms(vscale):
    """Value norms of about 1e3 to 1e5 (values scaled by vscale on alternate
    runs of 37 tokens, so that one scan mixes norms near 20 with large ones)
    behind peaked scores (outlier channels): the value-side weight p gamma_v
    must stay inside the fp16 range of the MFMA operands.  Outputs scale with
    the values, so the 2e-3 bar is applied at unit value scale."""
    w = workload("gqa32k")
    inp = make_inputs(w, scale_T=1500)
    T = inp["V"].shape[2]
    s = torch.where((torch.arange(T) // 37) % 2 == 0, vscale, 1.0).view(1, 1, T, 1)
    V = (inp["V"].float() * s).to(torch.bfloat16)
    kc, hk = codecs(w.bits)
    vc, hv = codecs(w.bits)
    kcache = encode_gpu(inp["K"], kc)
    vcache = encode_gpu(V, vc)
    out = octo.octo_attend_decode(kc, vc, kcache, vcache, inp["q"].cuda(), inp["seq_lens"].cuda())
    torch.cuda.synchronize()
    hv_cache = vcache.to_host()
    say(f"  value norms up to {float(hv_cache['gamma'].max()):.3e}")
    ref = oatt.decode_attention(inp["q"].double().numpy(), kcache.to_host(), hv_cache, hk, hv,
                                inp["seq_lens"].numpy())
    err = np.abs(out.cpu().double().numpy() - ref).max()
    say(f"  vscale {vscale} max-abs err {err:.3e} (bar {ATOL * vscale:.3e})")
    assert np.isfinite(out.cpu().numpy()).all()
    assert err <= ATOL * vscale
