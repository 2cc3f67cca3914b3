"""The Python binding refuses mis-shaped, mistyped, strided or host buffers
before anything reaches the library (GPU tensors needed to get past the
device check), and decode over an empty cache returns zeros."""

import ctypes

import pytest
import torch

from tests.gpu_util import require_gpu

pytestmark = pytest.mark.gpu


class _Spy:
    """Counts calls of one library entry point (wraps the ctypes function)."""

    def __init__(self, monkeypatch, lib, name):
        self.n = 0
        fn = getattr(lib, name)

        def wrapped(*a):
            self.n += 1
            return fn(*a)
        monkeypatch.setattr(lib, name, wrapped)


def test_bwd_refuses_bad_output_buffers(monkeypatch):
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    B, Hq, Hkv, S, d = 1, 4, 2, 100, 64
    q = torch.randn((B, Hq, S, d), device="cuda").to(torch.bfloat16)
    k = torch.randn((B, Hkv, S, d), device="cuda").to(torch.bfloat16)
    tok = torch.zeros((B, S), dtype=torch.int32, device="cuda")
    idx = sa.build_index(tok, [5], 4, 16)
    o, lse = sa.fwd(q, k, k, idx)
    spy = _Spy(monkeypatch, sa.load_library(), "sepattn_bwd")
    bad = [
        dict(dq=torch.empty((B, Hq, S, d + 1), dtype=torch.bfloat16, device="cuda")),     # shape
        dict(dk=torch.empty((B, Hq, S, d), dtype=torch.bfloat16, device="cuda")),         # q's shape, not k's
        dict(dv=torch.empty((B, Hkv, S, d), dtype=torch.float32, device="cuda")),         # dtype
        dict(dq=torch.empty((B, Hq, d, S), dtype=torch.bfloat16, device="cuda").transpose(2, 3)),  # strided
        dict(dk=torch.empty((B, Hkv, S, d), dtype=torch.bfloat16)),                       # host
        dict(ws=torch.empty(1 << 20, dtype=torch.float32, device="cuda")),                # ws dtype
        dict(ws=torch.empty(1 << 20, dtype=torch.uint8)),                                 # ws on the host
    ]
    for kw in bad:
        with pytest.raises((TypeError, ValueError)):
            sa.bwd(q, k, k, o, lse, q, idx, **kw)
    assert spy.n == 0
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(sa.SepattnError, match="workspace"):
        sa.bwd(q, k, k, o, lse, q, idx, ws=small)
    assert spy.n == 1


def test_decode_refuses_bad_buffers_and_empty_cache_gives_zero(monkeypatch):
    require_gpu()
    import sparse_attention_sepattn_amd as sa
    B, Hkv, Hq, d, c = 2, 2, 4, 64, 40
    cache = sa.SepCache(B, Hkv, d, c, 2, 4, 8)
    cos, sin = sa.rope_table(500000.0, c, d)
    cos, sin = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    q = torch.randn((B, Hq, d), device="cuda").to(torch.bfloat16)
    spy = _Spy(monkeypatch, sa.load_library(), "sepcache_decode")
    bad = [
        dict(o=torch.empty((B, Hq, d + 2), dtype=torch.bfloat16, device="cuda")),
        dict(o=torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")),
        dict(o=torch.empty((B, Hq, d), dtype=torch.bfloat16)),
        dict(o=torch.empty((B, d, Hq), dtype=torch.bfloat16, device="cuda").transpose(1, 2)),
        dict(ws=torch.empty(4096, dtype=torch.int32, device="cuda")),
    ]
    for kw in bad:
        with pytest.raises((TypeError, ValueError)):
            cache.decode(q, cos, sin, **kw)
    assert spy.n == 0
    # nothing appended since init: L = 0 for every sequence, the output is zero
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    cache.decode(q, cos, sin, o=o)
    torch.cuda.synchronize()
    assert spy.n == 1
    assert bool((o == 0).all())
