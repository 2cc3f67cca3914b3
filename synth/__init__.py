"""Seeded synthetic inputs shared by the tests, the bench and the oracle's
callers.  This module holds none of the method's arithmetic: it only draws
token ids, separator id sets and normal tensors, and rounds floats to bf16
bit patterns (round to nearest even) so both sides see identical bits.

Recipes (stand-ins for the pages' workloads, which need datasets and weights
that are not available):

* separator ids: ``n_sep`` distinct ids uniform without replacement from
  ``[0, vocab)``, sorted;
* i.i.d. token ids: each position is a separator with probability ``p_sep``
  (its id uniform over the separator set), otherwise an id uniform over the
  rest of the vocabulary;
* bursty token ids: alternating runs -- a non-separator run of length
  ~ Geometric(1/mean_seg) (support >= 1) then a separator run of length
  ~ Geometric(1/2);
* tensors: ``standard_normal`` float32, rounded to bf16 when asked.

Every draw comes from ``numpy.random.default_rng(seed)`` in a fixed order.
"""

import numpy as np

# The benchmark configurations (shapes and distributions).  Names say what the
# workload is; the sizes are the ones the throughput figures are quoted on.
CONFIGS = {
    "tiny_fp32": dict(seed=1, B=1, Hq=1, Hkv=1, S=512, d=64, dtype="f32", vocab=50_000,
                      p_sep=0.08, bursty=False, a=4, n=64, bwd=False),
    "pythia160m": dict(seed=2, B=8, Hq=12, Hkv=12, S=2048, d=64, dtype="bf16", vocab=50_000,
                       p_sep=0.08, bursty=False, a=4, n=64, bwd=True),
    "llama3_8b_prefill": dict(seed=3, B=1, Hq=32, Hkv=8, S=8192, d=128, dtype="bf16",
                              vocab=128_000, p_sep=0.08, bursty=False, a=4, n=256, bwd=False),
    "long_context_32k": dict(seed=4, B=1, Hq=32, Hkv=8, S=32768, d=128, dtype="bf16",
                             vocab=128_000, p_sep=None, bursty=True, a=4, n=256, bwd=True),
    "sepcache_decode": dict(seed=5, B=64, Hq=32, Hkv=8, d=128, dtype="bf16", vocab=128_000,
                            p_sep=0.08, a=4, s=64, w=256, c=800, theta=500000.0, steps=4096),
}


def rng(seed):
    return np.random.default_rng(seed)


def separator_ids(r, vocab, n_sep=9):
    return np.sort(r.choice(vocab, size=n_sep, replace=False)).astype(np.int32)


def token_ids_iid(r, shape, vocab, sep_ids, p_sep):
    sep_ids = np.asarray(sep_ids)
    is_sep = r.random(shape) < p_sep
    sep_pick = sep_ids[r.integers(0, len(sep_ids), size=shape)]
    # non-separator ids: uniform over the vocabulary minus the separator set
    others = np.setdiff1d(np.arange(vocab), sep_ids)
    other_pick = others[r.integers(0, len(others), size=shape)]
    return np.where(is_sep, sep_pick, other_pick).astype(np.int32)


def token_ids_bursty(r, B, S, vocab, sep_ids, mean_seg=15):
    sep_ids = np.asarray(sep_ids)
    others = np.setdiff1d(np.arange(vocab), sep_ids)
    out = np.empty((B, S), dtype=np.int32)
    for b in range(B):
        flags = np.zeros(S, dtype=bool)
        x = 0
        while x < S:
            x += int(r.geometric(1.0 / mean_seg))      # non-separator run
            run = int(r.geometric(0.5))                  # separator run
            flags[x:x + run] = True
            x += run
        out[b] = np.where(flags, sep_ids[r.integers(0, len(sep_ids), size=S)],
                          others[r.integers(0, len(others), size=S)])
    return out


def bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def normal(r, shape, dtype):
    """standard_normal tensor; returns (payload, values_f64).  For "bf16" the
    payload is the uint16 bit array, for "f32" the float32 array."""
    x = r.standard_normal(shape, dtype=np.float32)
    if dtype == "bf16":
        bits = bf16_bits(x)
        return bits, bf16_to_f64(bits)
    return x, x.astype(np.float64)


def prefill_inputs(cfg, S=None, B=None, Hq=None, Hkv=None, seed=None, with_grad=None):
    """Inputs of a prefill/training configuration (a dict from CONFIGS, or any
    dict with the same keys).  Optional overrides shrink it for tests."""
    c = dict(cfg)
    for key, val in (("S", S), ("B", B), ("Hq", Hq), ("Hkv", Hkv), ("seed", seed)):
        if val is not None:
            c[key] = val
    r = rng(c["seed"])
    sep = separator_ids(r, c["vocab"])
    if c.get("bursty"):
        tok = token_ids_bursty(r, c["B"], c["S"], c["vocab"], sep)
    else:
        tok = token_ids_iid(r, (c["B"], c["S"]), c["vocab"], sep, c["p_sep"])
    B_, Hq_, Hkv_, S_, d = c["B"], c["Hq"], c["Hkv"], c["S"], c["d"]
    q, qf = normal(r, (B_, Hq_, S_, d), c["dtype"])
    k, kf = normal(r, (B_, Hkv_, S_, d), c["dtype"])
    v, vf = normal(r, (B_, Hkv_, S_, d), c["dtype"])
    out = dict(cfg=c, sep=sep, tok=tok, q=q, k=k, v=v, qf=qf, kf=kf, vf=vf,
               scale=1.0 / np.sqrt(d))
    if with_grad if with_grad is not None else c.get("bwd"):
        do, dof = normal(r, (B_, Hq_, S_, d), c["dtype"])
        out.update(do=do, dof=dof)
    return out


class DecodeStream:
    """Per-step inputs of the streaming-decode workload: for each step a token
    id per sequence (separator with probability ``p_sep``) and new q/k/v rows,
    bf16, drawn in a fixed order from one generator."""

    def __init__(self, cfg, B=None, seed=None):
        self.c = dict(cfg)
        if B is not None:
            self.c["B"] = B
        self.r = rng(self.c["seed"] if seed is None else seed)
        self.sep = separator_ids(self.r, self.c["vocab"])

    def step(self):
        c = self.c
        tok = token_ids_iid(self.r, (c["B"],), c["vocab"], self.sep, c["p_sep"])
        q, qf = normal(self.r, (c["B"], c["Hq"], c["d"]), "bf16")
        k, kf = normal(self.r, (c["B"], c["Hkv"], c["d"]), "bf16")
        v, vf = normal(self.r, (c["B"], c["Hkv"], c["d"]), "bf16")
        return dict(tok=tok, q=q, k=k, v=v, qf=qf, kf=kf, vf=vf)
