"""Seeded synthetic workloads (inputs only; none of the codec's arithmetic).

The shapes stand in for the OCTOPUS paper's evaluation settings: a single
head for correctness, the Qwen2.5-7B-Instruct-1M attention shape (28 query
heads, 4 KV heads, head dim 128; Sec. 4.2) at several context lengths and
batch sizes, and chunk-wise video-diffusion attention (Sec. 4.3, CausVid with
3-frame chunks; the cached-window / current-chunk structure of "Quantized Keys
Steal Attention", Sec. 3).  No dataset, prompt or model weight is used:
everything is Gaussian noise from one torch CPU generator per workload.

Draw order per workload (one torch.Generator("cpu").manual_seed(seed)):
  K, V (fp32 N(0,1), [B, H_kv, T, d]), q (fp32 N(0,1)), then, when outliers
  are on, one randperm(d)[:4] per KV head whose channels are scaled by 10 in
  K, V and in every query head of that KV head's group, then the sequence
  lengths (uniform integers in [len_lo, len_hi]) when they vary.
  Chunk workloads draw K, V of the cached window, q, then K_cur, V_cur.
  Decode-step workloads (window > 0) then draw a pool of new-token rows
  K_new, V_new [B, H_kv, 64, d], with the same outlier channels scaled.
bf16 workloads are cast from fp32 with round-to-nearest-even.
"""
import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    T: int                 # tokens generated per (b, h) plane (= capacity)
    bits: int
    dtype: str             # "fp32" | "bf16"
    outliers: bool = False
    qjl: bool = False
    len_lo: int = 0        # > 0: per-sequence lengths ~ U[len_lo, len_hi]
    len_hi: int = 0
    chunk_q: int = 0       # > 0: chunk workload with this many queries / current tokens
    window: int = 0        # > 0: decode-step workload with a residual window of this size
    v_group: int = 0       # > 0: values in the group-wise codec with this group size
    k_group: int = 0       # > 0: keys in the group-wise codec (chunk workloads)
    jensen: bool = False   # chunk workloads: the Jensen-bias correction of cached logits
    seed: int = 0

    @property
    def capacity(self):
        total = self.T + self.chunk_q
        return -(-total // 64) * 64


WORKLOADS = {
    "tiny": Workload("tiny", "1 head, d=128, 256 tokens, 1 query, fp32, b=3",
                     B=1, Hq=1, Hkv=1, d=128, T=256, bits=3, dtype="fp32"),
    "gqa32k": Workload("gqa32k", "GQA 28/4 heads, d=128, batch 1, context 32768, bf16 + outliers, b=4",
                       B=1, Hq=28, Hkv=4, d=128, T=32768, bits=4, dtype="bf16", outliers=True),
    "gqa32k_g32": Workload("gqa32k_g32", "GQA 28/4 heads, d=128, batch 1, context 32768, bf16 + outliers, "
                           "b=4 keys, values in the group-32 codec at b=4",
                           B=1, Hq=28, Hkv=4, d=128, T=32768, bits=4, dtype="bf16", outliers=True,
                           v_group=32),
    "batch16": Workload("batch16", "GQA 28/4, batch 16, context U[4096, 8192] (capacity 8192), bf16 + outliers, b=3",
                        B=16, Hq=28, Hkv=4, d=128, T=8192, bits=3, dtype="bf16", outliers=True,
                        len_lo=4096, len_hi=8192),
    "long128k": Workload("long128k", "GQA 28/4, batch 4, context 131072, bf16, b=2 + QJL keys",
                         B=4, Hq=28, Hkv=4, d=128, T=131072, bits=2, dtype="bf16", qjl=True),
    "step32k": Workload("step32k", "decode step, GQA 28/4, batch 1, context up to 32768 (last 32 tokens native), bf16 + outliers, b=4",
                        B=1, Hq=28, Hkv=4, d=128, T=32768, bits=4, dtype="bf16", outliers=True,
                        window=32),
    "chunk_qksa": Workload("chunk_qksa", "MHA 40 heads, d=128, 1560 queries over 9360 cached + 1560 current "
                           "tokens, bf16, group-32 INT2 keys and values, Jensen-bias correction",
                           B=1, Hq=40, Hkv=40, d=128, T=9360, bits=2, dtype="bf16", chunk_q=1560,
                           k_group=32, v_group=32, jensen=True),
    "chunk": Workload("chunk", "MHA 40 heads, d=128, 1560 queries over 9360 cached + 1560 current tokens, bf16, b=2",
                      B=1, Hq=40, Hkv=40, d=128, T=9360, bits=2, dtype="bf16", chunk_q=1560),
}


def _cast(x, dtype):
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def make_inputs(w: Workload, scale_T=None):
    """CPU tensors for workload w.

    scale_T: optional smaller token count (same recipe, same seed) for tests
    that need the shape family at a size the oracle finishes quickly.
    Returns a dict with K, V [B,Hkv,T,d], q ([B,Hq,d], or [B,Hq,Tq,d] for
    chunk workloads), seq_lens (int32 [B]), and for chunk workloads K_cur,
    V_cur [B,Hkv,Tq,d]."""
    T = w.T if scale_T is None else scale_T
    g = torch.Generator("cpu").manual_seed(w.seed)
    K = torch.randn(w.B, w.Hkv, T, w.d, generator=g)
    V = torch.randn(w.B, w.Hkv, T, w.d, generator=g)
    if w.chunk_q:
        q = torch.randn(w.B, w.Hq, w.chunk_q, w.d, generator=g)
        K_cur = torch.randn(w.B, w.Hkv, w.chunk_q, w.d, generator=g)
        V_cur = torch.randn(w.B, w.Hkv, w.chunk_q, w.d, generator=g)
    else:
        q = torch.randn(w.B, w.Hq, w.d, generator=g)
    chans = []
    if w.outliers:
        G = w.Hq // w.Hkv
        for h in range(w.Hkv):
            ch = torch.randperm(w.d, generator=g)[:4]
            chans.append(ch)
            K[:, h, :, ch] *= 10.0
            V[:, h, :, ch] *= 10.0
            q[:, h * G:(h + 1) * G, ..., ch] *= 10.0
    if w.len_lo:
        lo = min(w.len_lo, T)
        hi = min(w.len_hi, T)
        seq = torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int32)
    else:
        seq = torch.full((w.B,), T, dtype=torch.int32)
    out = {"K": _cast(K, w.dtype), "V": _cast(V, w.dtype), "q": _cast(q, w.dtype), "seq_lens": seq}
    if w.chunk_q:
        out["K_cur"] = _cast(K_cur, w.dtype)
        out["V_cur"] = _cast(V_cur, w.dtype)
    if w.window:
        K_new = torch.randn(w.B, w.Hkv, 64, w.d, generator=g)
        V_new = torch.randn(w.B, w.Hkv, 64, w.d, generator=g)
        for h, ch in enumerate(chans):
            K_new[:, h, :, ch] *= 10.0
            V_new[:, h, :, ch] *= 10.0
        out["K_new"] = _cast(K_new, w.dtype)
        out["V_new"] = _cast(V_new, w.dtype)
    return out
