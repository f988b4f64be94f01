"""GPU parity of octo_attend_chunk against the oracle's float64 chunk attention
(cached packed window + full-precision current chunk, one unmasked softmax)
evaluated on the GPU-written cache (max-abs 2e-3).
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


def run_chunk(w, rows=None, heads=None, cached=None, tc=None):
    inp = make_inputs(w)
    kc, hk = codecs(w.bits)
    vc, hv = codecs(w.bits)
    K, V = inp["K"], inp["V"]
    cached = K.shape[2] if cached is None else cached
    cap = max(64, -(-K.shape[2] // 64) * 64)
    kcache = encode_gpu(K, kc, capacity=cap)
    vcache = encode_gpu(V, vc, capacity=cap)
    q, kcur, vcur = inp["q"], inp["K_cur"], inp["V_cur"]
    if tc is not None:
        kcur, vcur = kcur[:, :, :tc].contiguous(), vcur[:, :, :tc].contiguous()
    out = octo.octo_attend_chunk(kc, vc, kcache, vcache, cached, q.cuda(), kcur.cuda(), vcur.cuda())
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()
    hkc, hvc = kcache.to_host(), vcache.to_host()
    heads = heads or list(range(w.Hq))
    G = w.Hq // w.Hkv
    err = 0.0
    for b in range(w.B):
        for h in heads:
            g = h // G
            sub_k, sub_v = _plane(hkc, b, g), _plane(hvc, b, g)
            ref = oatt.chunk_attention(q[b:b + 1, h:h + 1].double().numpy(), sub_k, sub_v, hk, hv,
                                       cached, kcur[b:b + 1, g:g + 1].double().numpy(),
                                       vcur[b:b + 1, g:g + 1].double().numpy(), q_rows=rows)
            r = np.arange(w.chunk_q) if rows is None else np.asarray(rows)
            err = max(err, np.abs(out[b, h][r] - ref[0, 0][r]).max())
    return err, out


def _plane(h, b, g):
    n = h["B"] * h["H"]
    p = b * h["H"] + g
    return {"B": 1, "H": 1, "capacity": h["capacity"],
            "idx": h["idx"].reshape(n, -1)[p],
            "gamma": h["gamma"][b:b + 1, g:g + 1]}


def test_chunk_small():
    w = workload("chunk", Hq=4, Hkv=4, T=300, chunk_q=200)
    err, _ = run_chunk(w)
    say(f"chunk small err {err:.3e}")
    assert err <= ATOL


def test_chunk_gqa_and_ragged():
    w = workload("chunk", Hq=6, Hkv=2, T=130, chunk_q=77)
    err, _ = run_chunk(w)
    assert err <= ATOL


def test_chunk_no_current_tokens_and_no_cache():
    w = workload("chunk", Hq=2, Hkv=2, T=100, chunk_q=40)
    err, _ = run_chunk(w, cached=0)                 # current chunk only
    assert err <= ATOL
    err, _ = run_chunk(w, cached=57)                # part of the window
    assert err <= ATOL
    err, _ = run_chunk(w, tc=0)                     # cached window only
    assert err <= ATOL
    err, out = run_chunk(w, cached=0, tc=0)         # nothing to attend to: zero rows
    assert err <= ATOL and np.all(out == 0.0)


@pytest.mark.parametrize("bits", [3, 4])
def test_chunk_other_bit_widths(bits):
    w = workload("chunk", Hq=2, Hkv=2, T=200, chunk_q=64, bits=bits)
    err, _ = run_chunk(w)
    assert err <= ATOL


def test_chunk_full_size_sampled():
    """The full video-chunk shape: 40 heads, 1560 queries, 9360 cached + 1560
    current tokens; the oracle checks sampled query rows (the first and last
    among them) of every head."""
    w = workload("chunk")
    rng = np.random.default_rng(2)
    rows = np.sort(rng.choice(np.arange(1, w.chunk_q - 1), size=14, replace=False))
    rows = np.concatenate([[0], rows, [w.chunk_q - 1]])
    err, _ = run_chunk(w, rows=rows)
    say(f"chunk full err {err:.3e}")
    assert err <= ATOL


# leftover blocks a plane r = bpp mod 8: 1, 2, 1 (one tile in all, so that
# shares and their halves are empty), 1, 2 (taken in the first pass), then 3
# and 4 (a second pass over each workgroup's share)
@pytest.mark.parametrize("B,Hq,Hkv,Tq,cached,tc", [(1, 2, 2, 544, 300, 544), (1, 4, 2, 280, 200, 280),
                                                    (1, 2, 2, 544, 0, 32), (1, 1, 1, 1300, 700, 1300),
                                                    (2, 4, 2, 280, 150, 200), (1, 2, 2, 608, 300, 300),
                                                    (1, 2, 2, 640, 250, 100)])
def test_chunk_split_tails(B, Hq, Hkv, Tq, cached, tc):
    """Planes of 8 upp + r query blocks with upp >= 2 and r = 1..4 leftover
    blocks: each of a plane's upp workgroups takes 8 whole blocks and a share
    of the tiles for the leftover ones, whose partials a second launch
    merges.  17 blocks a plane (r = 1), 2 x 9 blocks of a GQA plane (r = 2,
    the last block ragged), one tile for two workgroups (the second's share
    empty), 41 blocks (upp = 5) over a ragged window, two sequences of GQA
    planes (the planes' blocks and partials indexed across the batch), and 19
    and 20 blocks a plane (r = 3 and 4, which take a second pass)."""
    w = workload("chunk", B=B, Hq=Hq, Hkv=Hkv, T=max(cached, 64), chunk_q=Tq)
    err, _ = run_chunk(w, cached=cached, tc=tc)
    say(f"chunk split tails B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} cached {cached} current {tc} err {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("cached,tc", [(0, 1), (5, 20), (20, 12), (31, 1), (32, 32), (40, 40), (64, 32),
                                       (40, 57)])
def test_chunk_tile_counts(cached, tc):
    """Windows of one, two and three 32-key tiles, full and ragged, so that
    both buffers of the tile pipeline serve as the last one and a single
    partial tile is the whole key range."""
    w = workload("chunk", Hq=2, Hkv=2, T=64, chunk_q=max(tc, 1))
    err, _ = run_chunk(w, cached=cached, tc=tc)
    say(f"chunk cached {cached} current {tc} err {err:.3e}")
    assert err <= ATOL
