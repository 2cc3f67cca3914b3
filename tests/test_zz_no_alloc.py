"""sepcache_decode_noalloc (the decode entry point that allocates nothing,
for callers that cannot allocate: graph capture, serving loops) against
sepcache_decode with a caller workspace, through the C ABI: the same kernels,
so the outputs must agree bit for bit, on two calls in a row -- the
streaming-decode shape (B64, 32 q / 8 kv heads, d128, c800) and then a
smaller one -- and after a larger call has left its partials in the fixed
scratch."""

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev_tensor, require_gpu, say

pytestmark = pytest.mark.gpu


def _filled_cache(B, Hq, Hkv, d, c, a, s, w, steps, seed):
    import sparse_attention_sepattn_amd as sa
    cache = sa.SepCache(B, Hkv, d, c, a, s, w)
    st = synth.DecodeStream(dict(seed=seed, B=B, Hq=Hq, Hkv=Hkv, d=d, vocab=128_000, p_sep=0.08))
    for _ in range(steps):
        x = st.step()
        cache.update(dev_tensor(x["k"], "bf16"), dev_tensor(x["v"], "bf16"), torch.from_numpy(x["tok"]).cuda(),
                     st.sep)
    return cache, dev_tensor(x["q"], "bf16")


def _compare(B, Hq, Hkv, d, c, a, s, w, steps, seed):
    import sparse_attention_sepattn_amd as sa
    say(f"no-alloc decode B={B} Hq={Hq} Hkv={Hkv} d={d} c={c} steps={steps}")
    cache, q = _filled_cache(B, Hq, Hkv, d, c, a, s, w, steps, seed)
    cos, sin = sa.rope_table(500000.0, c, d)
    cos, sin = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    ref = cache.decode(q, cos, sin)
    got = torch.full_like(ref, float("nan"))
    cache.decode_noalloc(q, cos, sin, o=got)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(ref.float()).all())
    assert torch.equal(got, ref)
    L = cache.state[:, :3].sum(1).cpu().numpy()
    say(f"  cached slots min={L.min()} max={L.max()}: identical")
    return L


def test_noalloc_matches_workspace_decode_twice():
    require_gpu()
    cfg = synth.CONFIGS["sepcache_decode"]
    # first call: the streaming-decode shape, past its first compression
    L1 = _compare(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["c"], cfg["a"], cfg["s"], cfg["w"], 900, 5)
    assert L1.max() > 256
    # second call, smaller: fewer sequences, heads and slots (the scratch
    # still holds the first call's partials past this call's extent)
    L2 = _compare(3, 4, 2, 64, 150, 2, 8, 32, 170, 6)
    assert L2.max() < L1.min()


def test_noalloc_rejects_inputs_beyond_the_scratch():
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    L = sa.load_library()
    B, Hq, Hkv, d, c = 600, 32, 8, 128, 800
    assert L.sepcache_decode_workspace(__import__("ctypes").byref(
        sa._Cache(B, Hkv, d, c, 4, 64, 256, 1, 1, 1, 1, 1)), Hq) > (16 << 20)
    cache = sa.SepCache(B, Hkv, d, c, 4, 64, 256)
    cos, sin = sa.rope_table(500000.0, c, d)
    cos, sin = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sa.SepattnError, match="scratch"):
        cache.decode_noalloc(q, cos, sin)
