"""Benchmark of the OCTOPUS hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa32k]
                    [--extras batch16,long128k,chunk,step32k | none]

A step is one pass of the whole hot path over one batch of synthetic input
with everything already resident in HBM:
  decode workloads  encode the full context (K and V) into the packed cache,
                    then single-query decode attention over it;
  chunk workload    encode the current chunk (K and V) into the cache slots
                    after the cached window, then chunk attention of its
                    queries over the window and the chunk;
  step workload     one decode step with a residual window (append, attend,
                    evict).
The timed region brackets exactly K steps with torch.cuda.synchronize();
HIP events recorded on the stream the kernels run on give the per-call
durations.  One JSON line is printed: the headline workload (--workload) at
the top level and every workload of --extras under "configs", each with the
same keys.

value      cached KV-tokens/s of the attention call: tokens attended per
           step (sum of the sequence lengths; for the chunk workload the
           window plus the chunk) divided by its mean duration.
roofline   for the attention call: algorithmic bytes (packed cache of the
           attended tokens, K and V) per launch over the mean duration,
           against 8 TB/s (decode), or algorithmic MFMA flops against the
           fp16 dense peak (chunk).
cpu_baseline  the float64 oracle on bounded samples in the same units:
           attention (one KV-head plane at a time of the decode workloads; a
           few query rows of the chunk workload) and the encoder (token
           positions/s), each with every available core and with one thread
           (single_core, encode_single_core).
parity     by-product of the oracle legs: the encoder's indices on the
           sampled tokens against the GPU-written records (triplets,
           mismatches, forgiven near-threshold ones, bad ones) and the
           largest difference between the oracle's and the GPU's attention
           outputs on the sampled rows.
cold       (decode) the same call over cache replicas spanning 600 MB, taken in
           turn, so each call reads from HBM rather than the 256 MB
           Infinity Cache; achieved GB/s and fraction of 8 TB/s beside it.
           stream_copy_ceiling_GBps: read + write rate of a 1 GiB device copy.
traffic    memory-side bytes per attention call, from rocprofv3 FETCH_SIZE and
           WRITE_SIZE counters (one --pmc run each) scaled by what the same
           counters read for a plain copy of known size; read from
           profiles/traffic_<workload>.json and reported only while the
           library sources hash to the value recorded there (else null).

Counter helpers (run under rocprofv3 --pmc, then summarized here):
    python bench.py --copy-calibration          # a 512 MiB device copy
    python bench.py --pmc-summary WORKLOAD FETCH.csv WRITE.csv COPY_FETCH.csv COPY_WRITE.csv
"""
import argparse
import csv
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import quantized_decode_attention_octo_amd as octo  # noqa: E402
from quantized_decode_attention_octo_amd.workloads import WORKLOADS, make_inputs  # noqa: E402

METRIC = "decode-attn cached KV-tokens/s + % of HBM peak on packed cache; encode tokens/s"
HBM_PEAK_GBS = 8000.0
COPY_MIB = 512                     # size of the counter calibration copy
MFMA_FP16_PEAK_TFLOPS = 2500.0
# decode: both contractions on MFMA with fp16 operands split into hi + lo
# pairs (about 2^-20 relative per product), fp32 accumulation and softmax
DECODE_DTYPE = "f16-hi/lo-mfma/f32-acc"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash():
    """Hash of the library sources: recorded counters apply to these kernels only."""
    h = hashlib.sha256()
    src = os.path.join(ROOT, "quantized_decode_attention_octo_amd", "csrc")
    for f in sorted(os.listdir(src)):
        with open(os.path.join(src, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    with open(os.path.join(ROOT, "include", "octopus.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def recorded_traffic(workload):
    """Memory-side bytes per attention call from the recorded counters, or None."""
    try:
        with open(traffic_file(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    return rec["attention_bytes_per_call"]


def copy_calibration(mib):
    """A plain device copy of known size, for scaling the memory counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "copies": 3}), flush=True)


COLD_BYTES = 600 * (1 << 20)        # replicas span this, beyond the 256 MB MALL


def stream_ceiling_gbs():
    """Read + write GB/s of a plain 1 GiB device copy: a practical ceiling,
    reported beside (never instead of) the 8 TB/s peak."""
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / 5
    del src, dst
    return 2 * n * 4 / t / 1e9


def cold_decode(w, kc, vc, kcache, vcache, q, seq, max_len, ws, out, steps):
    """Attention over replicas of the packed cache taken in turn, spanning
    COLD_BYTES, so that each call reads a cache the previous calls have
    pushed out of the Infinity Cache.  Returns (replicas, mean us, percentiles)."""
    per = kcache.nbytes() + vcache.nbytes()
    n = max(2, -(-COLD_BYTES // per))
    reps = []
    for _ in range(n):
        kr = octo.PackedCache(kc, w.B, w.Hkv, w.capacity)
        vr = octo.PackedCache(vc, w.B, w.Hkv, w.capacity)
        for a, b in ((kr, kcache), (vr, vcache)):
            for f in ("idx", "gamma", "qjl", "gamma_r"):
                if getattr(a, f) is not None:
                    getattr(a, f).copy_(getattr(b, f))
        reps.append((kr, vr))
    t = Timer()
    for i in range(steps + n):
        kr, vr = reps[i % n]
        e0 = t.start() if i >= n else None
        octo.octo_attend_decode(kc, vc, kr, vr, q, seq, max_len, out=out, ws=ws)
        if i >= n:
            t.stop(e0)
    torch.cuda.synchronize()
    res = (n, t.mean_ms() * 1e3, t.percentiles_us())
    del reps
    torch.cuda.empty_cache()
    return res


def _pmc_per_kernel(path, counter):
    """Mean counter value per dispatch, by kernel name, from a rocprofv3 csv."""
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def pmc_summary(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """Writes profiles/traffic_<workload>.json from the four counter runs."""
    fetch = _pmc_per_kernel(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_kernel(write_csv, "WRITE_SIZE")
    cf = _pmc_per_kernel(copy_fetch_csv, "FETCH_SIZE")
    cw = _pmc_per_kernel(copy_write_csv, "WRITE_SIZE")
    # the copy kernel is the largest dispatch of the calibration run
    ck = max(cf, key=cf.get)
    copy_bytes = float(COPY_MIB * (1 << 20))
    f_scale = copy_bytes / (cf[ck] * 1024.0)
    w_scale = copy_bytes / (cw[ck] * 1024.0)
    att = [k for k in fetch if ("decode_kernel" in k or "merge_kernel" in k or "chunk" in k
                                or "rotate_rows" in k or "decode_rows" in k)]
    kernels = {k: {"fetch_kib": fetch[k], "write_kib": write.get(k, 0.0),
                   "bytes": fetch[k] * 1024.0 * f_scale + write.get(k, 0.0) * 1024.0 * w_scale}
               for k in att}
    rec = {"source_hash": source_hash(), "workload": workload,
           "copy_kernel": ck, "copy_bytes": copy_bytes,
           "copy_fetch_kib": cf[ck], "copy_write_kib": cw[ck],
           "fetch_scale": f_scale, "write_scale": w_scale,
           "kernels": kernels,
           "attention_bytes_per_call": sum(v["bytes"] for v in kernels.values())}
    with open(traffic_file(workload), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def packed_bytes_per_token(codec):
    s = codec.sizes()
    if codec.group:
        return 4 * s.idx_words                        # codes, scales and zero-points
    b = 4 * s.idx_words + 4                           # index stream + gamma
    if codec.qjl:
        b += 4 * s.qjl_words + 2                      # sigma + fp16 gamma_r
    return b


class Timer:
    """HIP events on the current stream around each call of one kind."""

    def __init__(self):
        self.pairs = []

    def start(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, e0):
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.append((e0, e1))

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(1, len(self.pairs))

    def percentiles_us(self):
        d = sorted(a.elapsed_time(b) * 1e3 for a, b in self.pairs)
        if not d:
            return None
        pick = lambda q: d[min(len(d) - 1, int(q * (len(d) - 1) + 0.5))]
        return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def value_codec(w):
    """The workload's value codec: OCTOPUS, or the group-wise codec."""
    return octo.Codec(bits=w.bits, group=w.v_group) if w.v_group else octo.Codec(bits=w.bits)


def run_decode(w, steps, warmup):
    inp = make_inputs(w)
    kc = octo.Codec(bits=w.bits, qjl=w.qjl)
    vc = value_codec(w)
    K, V = inp["K"].cuda(), inp["V"].cuda()
    q, seq = inp["q"].cuda(), inp["seq_lens"].cuda()
    cap = w.capacity
    kcache = octo.PackedCache(kc, w.B, w.Hkv, cap)
    vcache = octo.PackedCache(vc, w.B, w.Hkv, cap)
    max_len = int(inp["seq_lens"].max())
    ws = octo.workspace(octo.octo_decode_workspace_bytes(kc, w.B, w.Hq, w.Hkv, max_len), "cuda")
    out = torch.empty(w.B, w.Hq, 128, dtype=torch.float32, device="cuda")
    t_enc, t_att = Timer(), Timer()

    def step(timed):
        e0 = t_enc.start() if timed else None
        octo.octo_encode(kc, K, kcache)
        octo.octo_encode(vc, V, vcache)
        if timed:
            t_enc.stop(e0)
            e0 = t_att.start()
        octo.octo_attend_decode(kc, vc, kcache, vcache, q, seq, max_len, out=out, ws=ws)
        if timed:
            t_att.stop(e0)

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tokens = int(inp["seq_lens"].sum())
    att_ms, enc_ms = t_att.mean_ms(), t_enc.mean_ms()
    kv_bytes = tokens * w.Hkv * (packed_bytes_per_token(kc) + packed_bytes_per_token(vc))
    achieved = kv_bytes / (att_ms * 1e-3) / 1e9
    enc_tokens = w.B * w.T
    n_rep, cold_us, cold_pct = cold_decode(w, kc, vc, kcache, vcache, q, seq, max_len, ws, out,
                                           steps)
    ceiling = stream_ceiling_gbs()
    res = {
        "value": tokens / (att_ms * 1e-3),
        "unit": "cached KV-tokens/s",
        "ms_per_step": wall / steps * 1e3,
        "dtype": DECODE_DTYPE,
        "attention_us": att_ms * 1e3,
        "attention_us_percentiles": t_att.percentiles_us(),
        "cold": {"attention_us": cold_us, "percentiles_us": cold_pct, "replicas": n_rep,
                 "achieved_GBps": kv_bytes / (cold_us * 1e-6) / 1e9,
                 "frac": kv_bytes / (cold_us * 1e-6) / 1e9 / HBM_PEAK_GBS},
        "encode_us": enc_ms * 1e3,
        "encode_tokens_per_s": enc_tokens / (enc_ms * 1e-3),
        "token_kv_heads_per_s": tokens * w.Hkv / (att_ms * 1e-3),
        "_out": out,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(w.key),
                     "kernel": "octo_attend_decode (split-K scan + merge)",
                     "algorithmic_bytes_per_launch": kv_bytes,
                     "stream_copy_ceiling_GBps": ceiling},
    }
    return res, (inp, kc, vc, kcache, vcache)


def run_step(w, steps, warmup):
    """Decode steps with a residual window of W tokens over a context of up to
    T tokens: the packed prefix starts with P0 = T - W - 63 tokens and the
    rings with the next W - 1, and step s appends a token from the pool,
    attends over P0 + W + s tokens (at most T over 64 steps) and encodes the
    token leaving the window.  The split plan is sized by the last step's
    packed length, T - W."""
    if warmup + steps > 64:
        raise SystemExit("the decode-step workload runs at most 64 steps (warmup included)")
    inp = make_inputs(w)
    kc = octo.Codec(bits=w.bits, qjl=w.qjl)
    vc = octo.Codec(bits=w.bits)
    W, T = w.window, w.T
    P0 = T - W - 63
    max_packed = T - W
    K, V = inp["K"].cuda(), inp["V"].cuda()
    cap = w.capacity
    kcache = octo.PackedCache(kc, w.B, w.Hkv, cap)
    vcache = octo.PackedCache(vc, w.B, w.Hkv, cap)
    octo.octo_encode(kc, K[:, :, :P0].contiguous(), kcache)
    octo.octo_encode(vc, V[:, :, :P0].contiguous(), vcache)
    kr = torch.zeros(w.B, w.Hkv, W, w.d, dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    for j in range(P0, P0 + W - 1):
        kr[:, :, j % W] = K[:, :, j]
        vr[:, :, j % W] = V[:, :, j]
    plens = torch.full((w.B,), P0, dtype=torch.int32, device="cuda")
    wlens = torch.full((w.B,), W - 1, dtype=torch.int32, device="cuda")
    q = inp["q"].cuda()
    kn, vn = inp["K_new"].cuda(), inp["V_new"].cuda()
    new = [(kn[:, :, i].contiguous(), vn[:, :, i].contiguous()) for i in range(kn.shape[2])]
    ws = octo.workspace(octo.octo_decode_step_workspace_bytes(kc, w.B, w.Hq, w.Hkv, max_packed), "cuda")
    out = torch.empty(w.B, w.Hq, 128, dtype=torch.float32, device="cuda")
    t_att = Timer()
    count = [0]

    def step(timed):
        k1, v1 = new[count[0] % len(new)]
        e0 = t_att.start() if timed else None
        octo.octo_decode_step(kc, vc, kcache, vcache, q, k1, v1, kr, vr, plens, wlens,
                              max_packed, out=out, ws=ws)
        if timed:
            t_att.stop(e0)
        count[0] += 1

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    att_ms = t_att.mean_ms()
    # tokens attended per step: P + W = P0 + W + s at step s (every step evicts)
    tokens = w.B * (P0 + W + warmup + (steps - 1) / 2.0)
    packed = w.B * w.Hkv * (tokens / w.B - W) * (packed_bytes_per_token(kc) + packed_bytes_per_token(vc))
    native = w.B * w.Hkv * (W * 2 * w.d * 2 + 2 * w.d * 2)      # window rows read, new rows written
    enc = w.B * w.Hkv * (2 * w.d * 2 + packed_bytes_per_token(kc) + packed_bytes_per_token(vc))
    step_bytes = packed + native + enc
    achieved = step_bytes / (att_ms * 1e-3) / 1e9
    res = {
        "value": tokens / (att_ms * 1e-3),
        "unit": "cached KV-tokens/s",
        "ms_per_step": wall / steps * 1e3,
        "dtype": DECODE_DTYPE,
        "attention_us": att_ms * 1e3,
        "attention_us_percentiles": t_att.percentiles_us(),
        "encode_us": None,
        "encode_tokens_per_s": None,
        "token_kv_heads_per_s": tokens * w.Hkv / (att_ms * 1e-3),
        "_out": out,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(w.key),
                     "kernel": "octo_decode_step (split-K scan with the window workgroup + merge)",
                     "algorithmic_bytes_per_launch": step_bytes},
    }
    state = (inp, kc, vc, kcache, vcache, kr, vr, plens, wlens, new)
    return res, state


def run_chunk(w, steps, warmup):
    inp = make_inputs(w)
    kc = octo.Codec(bits=w.bits, group=w.k_group) if w.k_group else octo.Codec(bits=w.bits)
    vc = value_codec(w)
    cached, Tq = w.T, w.chunk_q
    kcache = octo.PackedCache(kc, w.B, w.Hkv, w.capacity)
    vcache = octo.PackedCache(vc, w.B, w.Hkv, w.capacity)
    octo.octo_encode(kc, inp["K"].cuda(), kcache)
    octo.octo_encode(vc, inp["V"].cuda(), vcache)
    q, kcur, vcur = inp["q"].cuda(), inp["K_cur"].cuda(), inp["V_cur"].cuda()
    flags = octo.binding.CHUNK_JENSEN_CORRECTION if w.jensen else 0
    ws = octo.workspace(octo.octo_chunk_workspace_bytes(kc, w.B, w.Hq, w.Hkv, Tq, cached, Tq, flags),
                        "cuda")
    out = torch.empty(w.B, w.Hq, Tq, 128, dtype=torch.float32, device="cuda")
    t_enc, t_att = Timer(), Timer()

    def step(timed):
        e0 = t_enc.start() if timed else None
        octo.octo_encode(kc, kcur, kcache, token_offset=cached)
        octo.octo_encode(vc, vcur, vcache, token_offset=cached)
        if timed:
            t_enc.stop(e0)
            e0 = t_att.start()
        octo.octo_attend_chunk(kc, vc, kcache, vcache, cached, q, kcur, vcur, out=out, ws=ws,
                               correction=w.jensen)
        if timed:
            t_att.stop(e0)

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    att_ms, enc_ms = t_att.mean_ms(), t_enc.mean_ms()
    keys = cached + Tq
    flops = 4.0 * w.B * w.Hq * Tq * keys * 128
    achieved = flops / (att_ms * 1e-3) / 1e12
    res = {
        "value": w.B * keys / (att_ms * 1e-3),
        "unit": "cached KV-tokens/s",
        "ms_per_step": wall / steps * 1e3,
        "dtype": "f16-mfma/f32-acc",
        "attention_us": att_ms * 1e3,
        "attention_us_percentiles": t_att.percentiles_us(),
        "encode_us": enc_ms * 1e3,
        "encode_tokens_per_s": w.B * Tq / (enc_ms * 1e-3),
        "_out": out,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_FP16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_FP16_PEAK_TFLOPS,
                     "traffic": recorded_traffic(w.key),
                     "kernel": "octo_attend_chunk (current-row pre-pass, MFMA attention decoding "
                               "the window tile by tile, leftover-block merge)",
                     "algorithmic_flops_per_launch": flops},
    }
    return res, (inp, kc, vc, kcache, vcache)


CPU_SECONDS = 8.0                  # oracle attention work per leg (bounded sample)
ENC_SECONDS = 4.0                  # oracle encoder work per leg


def _host_plane(h, b, g):
    """Host cache of plane (b, g) alone, in the same layout with B = H = 1."""
    n = h["B"] * h["H"]
    p = b * h["H"] + g
    out = {"B": 1, "H": 1, "capacity": h["capacity"], "idx": h["idx"].reshape(n, -1)[p]}
    if "gamma" in h:
        out["gamma"] = h["gamma"][b:b + 1, g:g + 1]
    if "qjl" in h:
        out["qjl"] = h["qjl"].reshape(n, -1)[p]
        out["gamma_r"] = h["gamma_r"][b:b + 1, g:g + 1]
    return out


def _attention_leg(w, state, out_gpu, hk, hv, hkc, hvc, seconds):
    """The oracle's attention on a bounded sample of the workload, timed,
    and the largest difference to the GPU outputs of the same rows."""
    import numpy as np
    from oracle import attention as oatt
    inp = state[0]
    G = w.Hq // w.Hkv
    lens = inp["seq_lens"].numpy()
    done, dt, units, err = 0.0, 0.0, 0, 0.0
    if w.window:
        # one oracle decode step per (batch, KV head) plane, in order and
        # repeated, from the state the GPU steps left; a plane-step counts
        # (P + n + 1) / Hkv of a step's cached KV-tokens
        from oracle import step as ostep
        _, _, _, _, _, kr, vr, plens, wlens, new = state
        kr_h, vr_h = kr.double().cpu().numpy(), vr.double().cpu().numpy()
        P, n = plens.cpu().numpy(), wlens.cpu().numpy()
        planes = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
        while dt < seconds:
            b, g = planes[units % len(planes)]
            st = {"k": _host_plane(hkc, b, g), "v": _host_plane(hvc, b, g),
                  "k_ring": kr_h[b:b + 1, g:g + 1].copy(), "v_ring": vr_h[b:b + 1, g:g + 1].copy(),
                  "P": P[b:b + 1].astype(np.int64), "n": n[b:b + 1].astype(np.int64),
                  "W": w.window}
            k1, v1 = new[units % len(new)]
            qn = inp["q"][b:b + 1, g * G:(g + 1) * G].double().numpy()
            t0 = time.perf_counter()
            ostep.decode_step(st, qn, k1[b:b + 1, g:g + 1].double().cpu().numpy(),
                              v1[b:b + 1, g:g + 1].double().cpu().numpy(), hk, hv)
            dt += time.perf_counter() - t0
            done += (int(P[b]) + int(n[b]) + 1) / w.Hkv
            units += 1
        sample = (f"{units} oracle decode steps, one (batch, KV head) plane each ({len(planes)} "
                  f"in all, in order and repeated), {G} query heads over the packed prefix and "
                  f"the window; each counts (P + n + 1) / {w.Hkv} cached KV-tokens")
        return done / dt, dt, sample, None
    if not w.chunk_q:
        # (batch, KV head) planes in order, repeated if the workload is
        # smaller than the budget; a plane of sequence b is len_b / Hkv of
        # the step's cached KV-tokens
        planes = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
        ref_o = out_gpu.double().cpu().numpy()
        while dt < seconds:
            b, g = planes[units % len(planes)]
            qn = inp["q"][b:b + 1, g * G:(g + 1) * G].double().numpy()
            t0 = time.perf_counter()
            o = oatt.decode_attention(qn, _host_plane(hkc, b, g), _host_plane(hvc, b, g), hk, hv,
                                      lens[b:b + 1])
            dt += time.perf_counter() - t0
            err = max(err, float(np.abs(o[0] - ref_o[b, g * G:(g + 1) * G]).max()))
            done += lens[b] / w.Hkv
            units += 1
        sample = (f"oracle decode attention over {units} (batch, KV head) planes of the workload "
                  f"({len(planes)} in all, taken in order and repeated), "
                  f"{G} query heads each; each plane counts len_b / {w.Hkv} cached KV-tokens")
        return done / dt, dt, sample, err
    # 8-row groups of head 0's queries; one row attends the whole window and
    # chunk, 1 / (Hq Tq) of the step
    pk, pv = _host_plane(hkc, 0, 0), _host_plane(hvc, 0, 0)
    keys = w.T + w.chunk_q
    ref_o = out_gpu[0, 0].double().cpu().numpy()
    while dt < seconds and units * 8 < w.chunk_q:
        rows = np.arange(units * 8, min(units * 8 + 8, w.chunk_q))
        t0 = time.perf_counter()
        o = oatt.chunk_attention(inp["q"][:, :1].double().numpy(), pk, pv, hk, hv, w.T,
                                 inp["K_cur"][:, :1].double().numpy(),
                                 inp["V_cur"][:, :1].double().numpy(), q_rows=rows,
                                 correction=w.jensen)
        dt += time.perf_counter() - t0
        err = max(err, float(np.abs(o[0, 0][rows] - ref_o[rows]).max()))
        done += len(rows)
        units += 1
    sample = (f"oracle chunk attention of head 0, {int(done)} query rows over {keys} keys, "
              f"scaled to {w.Hq} heads x {w.chunk_q} rows")
    return keys * done / (dt * w.Hq * w.chunk_q), dt, sample, err


def _encode_leg(w, state, hk, hv, hkc, hvc, seconds):
    """The oracle encoder on a bounded sample (K and V vectors of plane (0, 0),
    64 tokens at a time, from the first token of the step's encode), timed,
    and its indices compared with the GPU-written records of the same tokens:
    (token positions / s, seconds, sample, counts)."""
    import numpy as np
    from oracle import cache as ocache
    from oracle import encode as oenc
    from oracle import group as ogroup
    inp = state[0]
    off = w.T if w.chunk_q else 0
    src = {"K": inp["K_cur"] if w.chunk_q else inp["K"], "V": inp["V_cur"] if w.chunk_q else inp["V"]}
    T = src["K"].shape[2]
    st = dict(vectors=0, triplets=0, mismatch=0, forgiven=0, bad=0, codes=0)
    dt, t = 0.0, 0
    while dt < seconds and t < T:
        ts = np.arange(t, min(t + 64, T))
        for name, hc, host in (("K", hk, hkc), ("V", hv, hvc)):
            xv = src[name][0, 0].double().numpy()[ts]
            t0 = time.perf_counter()
            if hc.get("group"):
                e = ogroup.encode(xv, hc["bits"], hc["group"], hc["seed"])
            else:
                e = oenc.encode(xv, hc["c_xi"], hc["c_rho"], hc["seed"], rounding=hc["rounding"],
                                qjl=hc["qjl"])
            dt += time.perf_counter() - t0
            rec = ocache.read_tokens(host, hc, 0, 0, off + ts[0], len(ts))
            st["vectors"] += len(ts)
            if hc.get("group"):
                cm = rec["codes"] != e["codes"]
                st["codes"] += cm.size
                st["mismatch"] += int(cm.sum())
            else:
                mism = ((rec["i_xi"] != e["i_xi"]) | (rec["i_eta"] != e["i_eta"]) |
                        (rec["i_rho"] != e["i_rho"]))
                bad = mism & (e["margin"] >= 1e-6)
                st["triplets"] += mism.size
                st["mismatch"] += int(mism.sum())
                st["bad"] += int(bad.sum())
                st["forgiven"] += int((mism & ~bad).sum())
        t += len(ts)
    # a token position of the step encodes 2 Hkv B vectors
    rate = st["vectors"] / 2 / dt / (w.Hkv * w.B)
    sample = (f"oracle encode of tokens 0..{t - 1} of plane (0, 0), K and V, scaled to "
              f"{w.B} x {w.Hkv} planes")
    return rate, dt, sample, st


def cpu_baseline(w, state, out_gpu, seconds=CPU_SECONDS, enc_seconds=ENC_SECONDS):
    """The oracle on the host over bounded samples, in the units of the GPU
    figures: attention (cached KV-tokens/s) and encode (token positions/s),
    each with BLAS and torch limited to one thread and with every available
    core.  Its by-products are the parity record of the sample: the index
    comparison of the encoded tokens and the largest output difference."""
    from threadpoolctl import threadpool_limits
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle_codecs import codec as oracle_codec
    from oracle_codecs import group_codec as oracle_group_codec
    inp, kc, vc, kcache, vcache = state[:5]
    hk = (oracle_group_codec(bits=w.bits, group=w.k_group) if w.k_group
          else oracle_codec(bits=w.bits, qjl=w.qjl))
    hv = oracle_group_codec(bits=w.bits, group=w.v_group) if w.v_group else oracle_codec(bits=w.bits)
    hkc, hvc = kcache.to_host(), vcache.to_host()
    cores = len(os.sched_getaffinity(0))
    legs, parity = {}, {}
    default_threads = torch.get_num_threads()
    for label, n in (("single_core", 1), ("all_cores", cores)):
        with threadpool_limits(limits=n):
            torch.set_num_threads(n)
            v, dt, sample, err = _attention_leg(w, state, out_gpu, hk, hv, hkc, hvc, seconds)
            legs[label] = {"value": v, "unit": "cached KV-tokens/s", "cores": n, "kind": "oracle",
                           "sample": sample, "seconds": dt}
            if err is not None:
                parity["attention_max_abs_err"] = max(err, parity.get("attention_max_abs_err", 0.0))
            if not w.window:
                ev, edt, esample, est = _encode_leg(w, state, hk, hv, hkc, hvc, enc_seconds)
                legs["encode_" + label] = {"value": ev, "unit": "token positions/s", "cores": n,
                                           "kind": "oracle", "sample": esample, "seconds": edt}
                parity["encode"] = est
    torch.set_num_threads(default_threads)
    main = dict(legs["all_cores"])
    main.update({"single_core": legs["single_core"], "encode": legs.get("encode_all_cores"),
                 "encode_single_core": legs.get("encode_single_core"),
                 "cpu_model": _cpu_model(), "host_cores_available": cores})
    if parity:
        parity["rule"] = ("indices bit-exact except where the oracle's decision margin is below "
                          "1e-6 (forgiven); attention max-abs 2e-3 against the float64 oracle on "
                          "the GPU-written cache")
        parity["attention_atol"] = 2e-3
    return main, (parity or None)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


EXTRAS = ("batch16", "long128k", "chunk", "step32k")


def _config(key, w):
    return {"workload": f"{key}: {w.name}", "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
            "head_dim": w.d, "context": w.T, "bits": w.bits, "qjl": w.qjl,
            "chunk_queries": w.chunk_q, "window": w.window, "value_group": w.v_group,
            "key_group": w.k_group, "jensen_correction": w.jensen}


def run_one(key, steps, warmup, cpu, cpu_seconds, enc_seconds):
    """Times one workload and runs its oracle legs; returns the JSON entry."""
    w = WORKLOADS[key]
    if w.window:
        # the decode-step workload runs at most 64 steps, warmup included
        warmup = min(warmup, 16)
        steps = min(steps, 64 - warmup)
    log(f"bench {key}: {w.name}; warmup {warmup}, steps {steps}")
    if w.chunk_q:
        res, state = run_chunk(w, steps, warmup)
    elif w.window:
        res, state = run_step(w, steps, warmup)
    else:
        res, state = run_decode(w, steps, warmup)
    out_gpu = res.pop("_out")
    enc = "" if res["encode_us"] is None else f", encode {res['encode_us']:.1f} us"
    log(f"  attention {res['attention_us']:.1f} us{enc}, roofline frac {res['roofline']['frac']:.3f}")
    base, parity = None, None
    if cpu:
        base, parity = cpu_baseline(w, state, out_gpu, cpu_seconds, enc_seconds)
        log(f"  cpu baseline {base['value']:.3g} {base['unit']} ({base['cores']} cores), "
            f"parity {json.dumps(parity)}")
    entry = {"value": res["value"], "unit": res["unit"], "steps": steps, "warmup": warmup,
             "ms_per_step": res["ms_per_step"], "dtype": res["dtype"],
             "config": _config(key, w), "roofline": res["roofline"], "cpu_baseline": base,
             "parity": parity, "attention_us": res["attention_us"],
             "attention_us_percentiles": res.get("attention_us_percentiles"),
             "encode_us": res["encode_us"], "encode_tokens_per_s": res["encode_tokens_per_s"]}
    for k in ("token_kv_heads_per_s", "cold"):
        if k in res:
            entry[k] = res[k]
    del state, out_gpu
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return entry


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa32k", choices=sorted(WORKLOADS),
                    help="the headline workload (value, roofline, cpu_baseline)")
    ap.add_argument("--extras", default=",".join(EXTRAS),
                    help="comma-separated workloads reported beside it under 'configs' "
                         "('none' for the headline alone)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pmc-summary", nargs=5,
                    metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"))
    a = ap.parse_args()
    if a.pmc_summary:
        pmc_summary(*a.pmc_summary)
        return
    if a.copy_calibration:
        copy_calibration(COPY_MIB)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the workloads fit one MI355X and no multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)
    extras = [] if a.extras in ("", "none") else [e for e in a.extras.split(",") if e != a.workload]
    for e in extras:
        if e not in WORKLOADS:
            raise SystemExit(f"unknown workload {e}")
    octo.lib()
    cpu = not a.no_cpu_baseline
    head = run_one(a.workload, a.steps, a.warmup, cpu, CPU_SECONDS, ENC_SECONDS)
    line = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"], "data": "synthetic (seeded Gaussian, see workloads.py)",
        "config": head["config"], "roofline": head["roofline"], "cpu_baseline": head["cpu_baseline"],
        "parity": head["parity"], "attention_us": head["attention_us"],
        "encode_us": head["encode_us"], "attention_us_percentiles": head["attention_us_percentiles"],
        "encode_tokens_per_s": head["encode_tokens_per_s"],
    }
    for k in ("token_kv_heads_per_s", "cold"):
        if k in head:
            line[k] = head[k]
    # the other configurations, each with its own roofline, oracle legs and
    # parity record (shorter oracle legs)
    line["configs"] = {e: run_one(e, a.steps, a.warmup, cpu, CPU_SECONDS / 2, ENC_SECONDS / 2)
                       for e in extras}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
