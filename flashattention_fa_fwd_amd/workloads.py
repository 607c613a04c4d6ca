"""Seeded synthetic inputs for guarded BF16 attention.

This module only draws random numbers and plants structure; it computes no
part of attention (no scores, no softmax, no products with V).  Both the HIP
path's tests/benchmark and the CPU oracle receive exactly these arrays.

Workloads (shapes taken from the pages' models; the data is synthetic):
  * ``tiny``      B=1, H=1, N=128, d=64, causal.  Q, K ~ N(0,1); V features
                  0..31 ~ N(-0.5,1) (negative-dominated), 32..63 ~ N(0,1);
                  10% of query rows get a planted exact repeated maximum
                  (seed 1014: of the seeds 1001..1040 with a tie rate near 10%, the one
                  whose bf16 Ō has the fewest elements the oracle cannot
                  certify).
  * ``gpt2s``     GPT-2 Small attention layer: B=16, H=12, N=1024, d=64,
                  causal.  Q, K ~ N(0, 1.5^2); V = mu[b,h,f] + N(0,1) with
                  mu ~ U(-1,1); key 0 is an attention sink (+4 logits); 5% of
                  rows get planted exact ties.
  * ``gpt2m``     GPT-2 Medium attention layer: B=8, H=16, N=1024, d=64,
                  causal, as gpt2s with 20% planted tie rows.
  * ``llama8b``   Llama-3.1-8B-shaped GQA: B=1, Hq=32, Hkv=8, N=8192, d=128,
                  causal.  Q, K ~ N(0,1); V ~ N(-0.3,1); sink +6 logits; 2% of
                  rows get ties planted in the shared KV head (all 4 query
                  heads of the group).
  * ``stress``    Large logits: B=4, H=8, N=4096, d=128, non-causal.  Q, K ~
                  N(0, 4^2) so row maxima reach 30-60; V ~ N(0,1); 30% of rows
                  get exact ties or near ties (gap in [1e-5, 5e-4]).
In every workload dO ~ N(0,1).

The sink: feature f_s = d-1 is reserved; Q[:, f_s] = 1, K[0, f_s] = bf16(c/alpha)
and K[j>0, f_s] = 0, so key 0 gets +c (exactly, when c/alpha is a bf16 value)
on every query's scaled logit.

A planted tie for query row i: pick two distinct visible keys a and b (not
the sink), copy K[a] into K[b] bit for bit, and add lambda*K[a] to Q[i]
(lambda = plant_logit / (alpha * d * var_q_k)), which lifts both keys about
plant_logit above the row's typical logit.  The named configurations use a
lift of 3.5-4 standard deviations of the row's logits (tiny 3.5, GPT-2 8,
stress 56), where a natural row maximum falls, or 2 above the sink where the
sink is the larger (Llama: sink 6, lift 8), so the pair is the row maximum
in most planted rows without dominating the row.  ``gpt2s_dup``
duplicates the keys without lifting the rows (the recipe as stated, where a
pair is a row's maximum only by chance).  The ``_sink``
study workloads lift the pair 16-20 logits, the attention-sink regime in
which the pages locate the biased rounding (P̄ = 1 exactly at the repeated
maximum and a small same-sign residual from the rest).  The two keys have
identical scores in any arithmetic.  A near tie additionally moves one
feature of K[b] by one bf16 step, in a feature where that changes the
scaled logit by 1e-5..5e-4.  Duplicated keys also touch other rows, so the
achieved tie rate is whatever the oracle's flags report, not the planted
fraction.  This module never computes a score: which key is a row's
maximum is left to the lift.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make", "make_custom", "to_bf16_bits", "bits_to_f32"]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even (torch CPU)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    head_dim: int
    causal: bool
    q_std: float
    k_std: float
    v_mode: str              # "split" | "mu_uniform" | "const"
    v_mean: float = 0.0
    sink_logit: float = 0.0  # 0: no sink
    tie_frac: float = 0.0
    near_tie_frac: float = 0.0  # fraction of the planted ties made near ties
    plant_logit: float = 8.0
    seed: int = 1000
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def alpha(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.head_dim)))

    def flops_fwd(self) -> float:
        """Counted work: 4*B*Hq*N^2*d, halved for causal (the usual FA count)."""
        f = 4.0 * self.batch * self.heads_q * self.seqlen ** 2 * self.head_dim
        return f / 2 if self.causal else f

    def flops_fwd_bwd(self) -> float:
        return 3.5 * self.flops_fwd()


WORKLOADS = {
    # the configurations as stated: the planted pair sits about 3.5-4 standard
    # deviations of the row's logits above the typical logit, i.e. where a
    # natural maximum of the row falls, so it is the row maximum without
    # dominating the row
    "tiny": Workload("tiny", 1, 1, 1, 128, 64, True, 1.0, 1.0, "split", -0.5,
                     0.0, 0.10, 0.0, 3.5, 1014,
                     "single head, causal, N=128, d=64"),
    "gpt2s": Workload("gpt2s", 16, 12, 12, 1024, 64, True, 1.5, 1.5, "mu_uniform", 0.0,
                      4.0, 0.05, 0.0, 8.0, 1002,
                      "GPT-2 Small attention layer B=16 H=12 N=1024 d=64 causal"),
    "gpt2m": Workload("gpt2m", 8, 16, 16, 1024, 64, True, 1.5, 1.5, "mu_uniform", 0.0,
                      4.0, 0.20, 0.0, 8.0, 1003,
                      "GPT-2 Medium attention layer B=8 H=16 N=1024 d=64 causal"),
    "llama8b": Workload("llama8b", 1, 32, 8, 8192, 128, True, 1.0, 1.0, "const", -0.3,
                        6.0, 0.02, 0.0, 8.0, 1004,
                        "Llama-3.1-8B GQA attention B=1 Hq=32 Hkv=8 N=8192 d=128 causal"),
    "stress": Workload("stress", 4, 8, 8, 4096, 128, False, 4.0, 4.0, "const", 0.0,
                       0.0, 0.30, 0.5, 56.0, 1005,
                       "large-logit stress B=4 H=8 N=4096 d=128 non-causal"),
    # study variant: keys duplicated as the configurations state, with no
    # lift of the query rows (a pair is a row's maximum only where the
    # duplicated key happens to be one)
    "gpt2s_dup": Workload("gpt2s_dup", 16, 12, 12, 1024, 64, True, 1.5, 1.5, "mu_uniform", 0.0,
                          4.0, 0.05, 0.0, 0.0, 1002,
                          "GPT-2 Small attention layer B=16 H=12 N=1024 d=64 causal, keys duplicated, no lift"),
    # study variants in the attention-sink regime where the pages locate the
    # biased rounding: the planted pair 16-20 logits above the row, so every
    # other P̄ of a tie row is tiny (same shapes and distributions otherwise)
    "tiny_sink": Workload("tiny_sink", 1, 1, 1, 128, 64, True, 1.0, 1.0, "split", -0.5,
                          0.0, 0.10, 0.0, 16.0, 1001,
                          "single head, causal, N=128, d=64, ties lifted 16 logits"),
    "gpt2s_sink": Workload("gpt2s_sink", 16, 12, 12, 1024, 64, True, 1.5, 1.5, "mu_uniform", 0.0,
                           4.0, 0.05, 0.0, 20.0, 1002,
                           "GPT-2 Small attention layer B=16 H=12 N=1024 d=64 causal, ties lifted 20 logits"),
    "gpt2m_sink": Workload("gpt2m_sink", 8, 16, 16, 1024, 64, True, 1.5, 1.5, "mu_uniform", 0.0,
                           4.0, 0.20, 0.0, 20.0, 1003,
                           "GPT-2 Medium attention layer B=8 H=16 N=1024 d=64 causal, ties lifted 20 logits"),
}


def _plant_ties(rng, wl: Workload, q: np.ndarray, kb: np.ndarray, nrows: int):
    """Plant exact/near ties.  q: fp32 [B,Hq,N,d] (rounded later);
    kb: bf16 bits [B,Hkv,N,d] (edited in place).  Returns planted (b,hk,i) rows."""
    B, Hq, N, d = q.shape
    Hkv = kb.shape[1]
    g = Hq // Hkv
    first_key = 1 if wl.sink_logit else 0
    lam = wl.plant_logit / (wl.alpha * d * wl.q_std * wl.k_std)
    planted = []
    n_target = int(round(wl.tie_frac * nrows))
    if n_target == 0:
        return planted
    lo_row = first_key + 1 if wl.causal else 0
    for b in range(B):
        for hk in range(Hkv):
            rows = rng.choice(np.arange(lo_row, N), size=min(n_target, N - lo_row), replace=False)
            for i in np.sort(rows):
                hi_key = i + 1 if wl.causal else N
                cand = np.arange(first_key, hi_key)
                a, bb = rng.choice(cand, size=2, replace=False)
                kb[b, hk, bb] = kb[b, hk, a]
                kf = bits_to_f32(kb[b, hk, a])
                for h in range(hk * g, (hk + 1) * g):
                    q[b, h, i] += lam * kf
                planted.append((b, hk, int(i), int(a), int(bb)))
    return planted


def _near_ties(rng, wl: Workload, qb: np.ndarray, kb: np.ndarray, planted):
    """Turn a fraction of the planted ties into near ties by moving one
    feature of K[b] by one bf16 step (gap alpha*|q|*step in [1e-5, 5e-4])."""
    Hq, Hkv = qb.shape[1], kb.shape[1]
    g = Hq // Hkv
    n_near = int(round(wl.near_tie_frac * len(planted)))
    idx = rng.choice(len(planted), size=n_near, replace=False) if n_near else []
    done = 0
    for t in idx:
        b, hk, i, a, bb = planted[t]
        qrow = np.abs(bits_to_f32(qb[b, hk * g, i])).astype(np.float64)
        kbits = kb[b, hk, bb].astype(np.int32)
        kval = bits_to_f32(kb[b, hk, bb]).astype(np.float64)
        # one bf16 step of |k| away from zero: the step is 2^(exponent-7)
        e = np.floor(np.log2(np.maximum(np.abs(kval), 1e-30)))
        step = np.exp2(e - 7)
        gap = wl.alpha * qrow * step
        ok = np.where((gap >= 1e-5) & (gap <= 5e-4) & (np.abs(kval) > 0))[0]
        ok = ok[ok != qb.shape[-1] - 1] if wl.sink_logit else ok
        if ok.size == 0:
            continue
        f = int(rng.choice(ok))
        kbits[f] += 1  # next bf16 value away from zero (same sign)
        kb[b, hk, bb] = kbits.astype(np.uint16)
        done += 1
    return done


def make_custom(wl: Workload, seed: int | None = None, seqlen: int | None = None,
                batch: int | None = None):
    """Generate one workload (optionally at another seed / seqlen / batch).

    Returns a dict of uint16 bf16 bit arrays q, k, v, do ([B,H,N,d]) and
    metadata: the Workload, the seed and the planted tie rows.
    """
    if seqlen is not None or batch is not None:
        wl = Workload(**{**wl.__dict__, "seqlen": seqlen or wl.seqlen, "batch": batch or wl.batch})
    s = wl.seed if seed is None else seed
    rng = np.random.default_rng(s)
    B, Hq, Hkv, N, d = wl.batch, wl.heads_q, wl.heads_kv, wl.seqlen, wl.head_dim
    q = rng.standard_normal((B, Hq, N, d), dtype=np.float32) * np.float32(wl.q_std)
    k = rng.standard_normal((B, Hkv, N, d), dtype=np.float32) * np.float32(wl.k_std)
    v = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    if wl.v_mode == "split":
        v[..., : d // 2] += np.float32(wl.v_mean)
    elif wl.v_mode == "mu_uniform":
        mu = rng.uniform(-1.0, 1.0, size=(B, Hkv, 1, d)).astype(np.float32)
        v += mu
    else:
        v += np.float32(wl.v_mean)
    do = rng.standard_normal((B, Hq, N, d), dtype=np.float32)
    if wl.sink_logit:
        fs = d - 1
        q[..., fs] = 1.0
        k[..., fs] = 0.0
        k[:, :, 0, fs] = wl.sink_logit / wl.alpha
    kb = to_bf16_bits(k)
    planted = _plant_ties(rng, wl, q, kb, N)
    qb = to_bf16_bits(q)
    if wl.sink_logit:
        one = to_bf16_bits(np.ones(1, np.float32))[0]
        qb[..., d - 1] = one  # the plant never touches the sink feature
    n_near = _near_ties(rng, wl, qb, kb, planted) if wl.near_tie_frac else 0
    return dict(q=qb, k=kb, v=to_bf16_bits(v), do=to_bf16_bits(do), workload=wl,
                seed=s, planted=planted, n_near=n_near)


def make(name: str, seed: int | None = None, **kw):
    return make_custom(WORKLOADS[name], seed=seed, **kw)
