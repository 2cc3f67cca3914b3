"""GPU parity of the prefill -> SepCache hand-off: one sepcache_prefill call
over a prompt leaves every cache bit-exact equal to the oracle's list
simulation after streaming the same prompt token by token (K/V rows of the
occupied slots, positions, ids, counters), whatever the cache held before;
streaming on from there stays bit-exact."""

import numpy as np
import pytest
import torch

import synth
from oracle import sepcache as osc
from tests.gpu_util import dev_tensor, require_gpu, say
from tests.test_gpu_sepcache import _compare_cache

pytestmark = pytest.mark.gpu


def _prompt(B, Hkv, d, P, p_sep, seed, vocab=5000):
    r = synth.rng(seed)
    sep = synth.separator_ids(r, vocab)
    tok = synth.token_ids_iid(r, (B, P), vocab, sep, p_sep)
    kb, _ = synth.normal(r, (B, Hkv, P, d), "bf16")
    vb, _ = synth.normal(r, (B, Hkv, P, d), "bf16")
    return sep, tok, kb, vb


def _sims(sep, tok, kb, vb, a, s, w, c):
    B, P = tok.shape
    sims = []
    for b in range(B):
        sim = osc.SepCacheSim(a, s, w, c, sep)
        for t in range(P):
            sim.append(tok[b, t], kb[b, :, t, :], vb[b, :, t, :])
        sims.append(sim)
    return sims


def _dirty(cache, B, Hkv, d, steps=25):
    g = torch.Generator(device="cuda").manual_seed(1)
    for t in range(steps):
        k = torch.randn((B, Hkv, d), device="cuda", generator=g).to(torch.bfloat16)
        cache.update(k, k, torch.full((B,), t % 3, dtype=torch.int32, device="cuda"), [1])


CASES = [
    # B, Hkv, d, P, a, s, w, c, p_sep
    (3, 2, 64, 1, 4, 2, 3, 12, 0.3),
    (3, 2, 64, 3, 4, 2, 3, 12, 0.3),
    (2, 2, 64, 11, 4, 2, 3, 12, 0.3),
    (2, 2, 64, 12, 4, 2, 3, 12, 0.3),
    (4, 2, 128, 1000, 4, 8, 32, 60, 0.2),
    (2, 1, 64, 3000, 0, 0, 5, 9, 0.5),
    (2, 2, 64, 500, 3, 40, 16, 64, 1.0),
    (3, 2, 64, 777, 2, 6, 10, 30, 0.0),
    (16, 8, 128, 2048, 4, 64, 256, 800, 0.08),
]


@pytest.mark.parametrize("case", CASES)
def test_prefill_handoff_bit_exact(case):
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    B, Hkv, d, P, a, s, w, c, p = case
    say(f"prefill hand-off {case}")
    sep, tok, kb, vb = _prompt(B, Hkv, d, P, p, seed=P + c)
    cache = sa.SepCache(B, Hkv, d, c, a, s, w)
    _dirty(cache, B, Hkv, d)
    tok_d = torch.from_numpy(tok).cuda()
    idx = sa.build_index(tok_d, sep, a, 64)
    cache.prefill(dev_tensor(kb, "bf16"), dev_tensor(vb, "bf16"), tok_d, idx)
    torch.cuda.synchronize()
    _compare_cache(cache, _sims(sep, tok, kb, vb, a, s, w, c), Hkv, d, c, where=f"P={P}")


def test_prefill_then_stream():
    """Streaming on after the hand-off equals streaming the whole sequence."""
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    B, Hkv, d, P, a, s, w, c = 3, 2, 64, 400, 4, 6, 12, 40
    sep, tok, kb, vb = _prompt(B, Hkv, d, P + 200, 0.25, seed=9)
    cache = sa.SepCache(B, Hkv, d, c, a, s, w)
    tok_d = torch.from_numpy(tok[:, :P].copy()).cuda()
    idx = sa.build_index(tok_d, sep, a, 64)
    cache.prefill(dev_tensor(kb[:, :, :P].copy(), "bf16"), dev_tensor(vb[:, :, :P].copy(), "bf16"), tok_d, idx)
    sims = _sims(sep, tok[:, :P], kb[:, :, :P], vb[:, :, :P], a, s, w, c)
    for t in range(P, P + 200):
        cache.update(dev_tensor(kb[:, :, t].copy(), "bf16"), dev_tensor(vb[:, :, t].copy(), "bf16"),
                     torch.from_numpy(tok[:, t].copy()).cuda(), sep)
        fired = False
        for b in range(B):
            fired |= sims[b].append(tok[b, t], kb[b, :, t], vb[b, :, t])
        if fired or t % 50 == 0 or t == P + 199:
            _compare_cache(cache, sims, Hkv, d, c, where=f"t={t}")
