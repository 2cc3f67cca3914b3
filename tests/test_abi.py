"""The C-ABI library loads, exports every symbol include/sepattn.h declares,
and rejects bad arguments on the host before anything is launched (CPU only:
no call here reaches a kernel)."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch  # noqa: F401  (loads torch's HIP runtime before the library)

import sparse_attention_sepattn_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sepattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sep\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = sa.load_library()
    names = declared_functions()
    assert set(names) == set(sa.EXPORTS)
    for name in names:
        assert hasattr(L, name), name


def test_strerror_and_sizes():
    L = sa.load_library()
    for st in range(6):
        assert L.sepattn_strerror(st)
    assert L.sepattn_index_bytes(0, 10) == 0
    n = L.sepattn_index_bytes(2, 1000)
    assert n >= 2 * 1000 * (1 + 4 + 4) and n % 256 == 0


def test_index_bind_carves_buffer_without_touching_it():
    L = sa.load_library()
    B, S = 3, 300
    n = L.sepattn_index_bytes(B, S)
    st = sa._Index()
    base = 1 << 40  # never dereferenced: bind only computes addresses
    assert L.sepattn_index_bind(ctypes.c_void_p(base), n, B, S, ctypes.byref(st)) == 0
    ptrs = [st.is_sep, st.sep_prefix, st.anchor_pos, st.anchor_count, st.qtile, st.tile_class]
    assert ptrs == sorted(ptrs) and all(p % 256 == 0 for p in ptrs)
    assert st.tile_class + B * 3 * 5 <= base + n
    assert L.sepattn_index_bind(ctypes.c_void_p(base), n - 1, B, S, ctypes.byref(st)) == 4
    assert L.sepattn_index_bind(ctypes.c_void_p(base + 8), n, B, S, ctypes.byref(st)) == 1


def test_argument_errors_are_host_side():
    L = sa.load_library()
    fake = ctypes.c_void_p(1 << 40)
    st = sa._Index()
    L.sepattn_index_bind(fake, L.sepattn_index_bytes(1, 64), 1, 64, ctypes.byref(st))
    st.n = 4
    z = ctypes.c_void_p(0)
    # unsupported head dim, bad GQA ratio, null pointers
    assert L.sepattn_fwd(fake, fake, fake, 1, 2, 1, 64, 96, 1, 0.1, ctypes.byref(st), fake, fake, z) == 2
    assert L.sepattn_fwd(fake, fake, fake, 1, 3, 2, 64, 64, 1, 0.1, ctypes.byref(st), fake, fake, z) == 1
    assert L.sepattn_fwd(z, fake, fake, 1, 2, 1, 64, 64, 1, 0.1, ctypes.byref(st), fake, fake, z) == 1
    # index bound for another shape
    assert L.sepattn_fwd(fake, fake, fake, 1, 2, 1, 128, 64, 1, 0.1, ctypes.byref(st), fake, fake, z) == 1
    # a (sequence, head) slice of 2^31 bytes or more (32-bit buffer offsets)
    assert L.sepattn_fwd(fake, fake, fake, 1, 2, 1, 1 << 23, 128, 1, 0.1, ctypes.byref(st), fake, fake, z) == 2
    assert L.sepattn_bwd_workspace(1, 2, 1, 1 << 23, 128, 1) == 0
    assert L.sepattn_bwd_workspace(1, 2, 1, (1 << 23) - 1, 128, 0) == 0  # fp32: 2^31 bytes at 2^22 rows
    assert L.sepattn_bwd_workspace(1, 2, 1, 65535 * 128, 128, 1) > 0
    # launch grid dimensions: query tiles, batch x kv heads, batch of the index
    assert L.sepattn_bwd_workspace(1, 2, 1, 65535 * 128 + 1, 64, 1) == 0
    assert L.sepattn_bwd_workspace(65536, 2, 1, 64, 64, 1) == 0
    assert L.sepattn_bwd_workspace(32768, 4, 2, 64, 64, 1) == 0
    # build_index: n < 1, a < 0, too many separator ids
    ids = (ctypes.c_int32 * 65)(*range(65))
    assert L.sepattn_build_index(fake, 1, 64, ids, 3, 4, 0, ctypes.byref(st), z) == 1
    assert L.sepattn_build_index(fake, 1, 64, ids, 3, -1, 4, ctypes.byref(st), z) == 1
    assert L.sepattn_build_index(fake, 1, 64, ids, 65, 4, 4, ctypes.byref(st), z) == 1
    assert L.sepattn_build_index(fake, 65536, 64, ids, 3, 4, 4, ctypes.byref(st), z) == 2  # grid dimension
    # fixed-interval index: interval < 1, index bound for another shape
    assert L.sepattn_build_index_interval(1, 64, 0, 4, 4, ctypes.byref(st), z) == 1
    assert L.sepattn_build_index_interval(1, 128, 12, 4, 4, ctypes.byref(st), z) == 1
    # bwd workspace too small
    need = L.sepattn_bwd_workspace(1, 2, 1, 64, 64, 1)
    assert need > 0
    assert L.sepattn_bwd(fake, fake, fake, fake, fake, fake, 1, 2, 1, 64, 64, 1, 0.1, ctypes.byref(st),
                         fake, fake, fake, fake, need - 1, z) == 4
    # profiled variant: the event array is required and holds 4 entries (NULL entries are allowed)
    ev4 = (ctypes.c_void_p * 4)()
    assert L.sepattn_bwd_profiled(fake, fake, fake, fake, fake, fake, 1, 2, 1, 64, 64, 1, 0.1, ctypes.byref(st),
                                  fake, fake, fake, fake, need, z, None, 4) == 1
    assert L.sepattn_bwd_profiled(fake, fake, fake, fake, fake, fake, 1, 2, 1, 64, 64, 1, 0.1, ctypes.byref(st),
                                  fake, fake, fake, fake, need, z, ev4, 3) == 1
    assert L.sepattn_bwd_profiled(fake, fake, fake, fake, fake, fake, 1, 2, 1, 64, 64, 1, 0.1, ctypes.byref(st),
                                  fake, fake, fake, fake, need - 1, z, ev4, 4) == 4


def test_cache_capacity_errors():
    L = sa.load_library()
    fake = 1 << 40
    c = sa._Cache(2, 8, 128, 324, 4, 64, 256, fake, fake, fake, fake, fake)
    z = ctypes.c_void_p(0)
    assert L.sepcache_init(ctypes.byref(c), z) == 3          # c <= a + s + w
    c.c, c.w = 800, 0
    assert L.sepcache_init(ctypes.byref(c), z) == 3          # w < 1
    c.w, c.d = 256, 96
    assert L.sepcache_init(ctypes.byref(c), z) == 2          # head dim
    c.d, c.B = 128, 65536
    assert L.sepcache_init(ctypes.byref(c), z) == 2          # batch beyond a grid dimension
    c.B = 2
    # prefill hand-off: index of another shape or another `a`, P < 1 (all
    # rejected on the host before any launch)
    c.d = 128
    st = sa._Index()
    L.sepattn_index_bind(ctypes.c_void_p(fake), L.sepattn_index_bytes(2, 64), 2, 64, ctypes.byref(st))
    st.a, st.n = 4, 64
    f = ctypes.c_void_p(fake)
    assert L.sepcache_prefill(ctypes.byref(c), f, f, f, 32, ctypes.byref(st), z) == 1       # P != idx.S
    st.a = 3
    assert L.sepcache_prefill(ctypes.byref(c), f, f, f, 64, ctypes.byref(st), z) == 1       # a mismatch
    st.a = 4
    assert L.sepcache_prefill(ctypes.byref(c), f, f, f, 0, ctypes.byref(st), z) == 1        # P < 1
    c.d = 128
    assert L.sepcache_decode_workspace(ctypes.byref(c), 32) > 0
    assert L.sepcache_decode_workspace(ctypes.byref(c), 30) == 0   # Hq % Hkv
    fp = ctypes.c_void_p(fake)
    assert L.sepcache_decode(ctypes.byref(c), fp, 96, fp, fp, 0.1, fp, fp, 1 << 30, z) == 2  # group of 12


def test_cache_hard_limits():
    """The hard limits stated in sepattn.h: capacity c <= 8192 (ECAPACITY),
    at most 128 kv heads (EUNSUPPORTED), a decode group Hq/Hkv of 1, 2, 4 or
    8 (EUNSUPPORTED), decode workspace size and alignment (EWORKSPACE,
    EINVAL) -- all on the host, before any launch."""
    L = sa.load_library()
    fake = 1 << 40
    fp = ctypes.c_void_p(fake)
    z = ctypes.c_void_p(0)
    c = sa._Cache(2, 8, 128, 8192, 4, 64, 256, fake, fake, fake, fake, fake)
    assert L.sepcache_decode_workspace(ctypes.byref(c), 32) > 0       # c = 8192 is accepted
    c.c = 8193
    assert L.sepcache_init(ctypes.byref(c), z) == 3
    assert L.sepcache_update(ctypes.byref(c), fp, fp, fp, None, 0, z) == 3
    assert L.sepcache_decode_workspace(ctypes.byref(c), 32) == 0
    c.c, c.Hkv = 800, 128
    assert L.sepcache_decode_workspace(ctypes.byref(c), 128) > 0      # Hkv = 128 is accepted
    c.Hkv = 129
    assert L.sepcache_init(ctypes.byref(c), z) == 2
    assert L.sepcache_update(ctypes.byref(c), fp, fp, fp, None, 0, z) == 2
    c.Hkv = 8
    need = L.sepcache_decode_workspace(ctypes.byref(c), 32)
    for Hq in (24, 48, 128):  # groups of 3, 6 and 16
        assert L.sepcache_decode(ctypes.byref(c), fp, Hq, fp, fp, 0.1, fp, fp, 1 << 30, z) == 2, Hq
    assert L.sepcache_decode(ctypes.byref(c), fp, 32, fp, fp, 0.1, fp, fp, need - 1, z) == 4
    assert L.sepcache_decode(ctypes.byref(c), ctypes.c_void_p(fake + 16), 32, fp, fp, 0.1, fp,
                             ctypes.c_void_p(fake + 16), need, z) == 1      # ws not 256-byte aligned
    assert L.sepcache_decode(ctypes.byref(c), fp, 32, fp, fp, 0.0, fp, fp, need, z) == 1   # scale <= 0
    for st in (2, 3):
        text = L.sepattn_strerror(st).decode()
        assert ("128" in text) if st == 2 else ("8192" in text), text


def test_noalloc_decode_host_checks():
    """sepcache_decode_noalloc refuses, on the host, an input whose partials
    would not fit the fixed scratch (ESCRATCH) and the usual bad arguments."""
    L = sa.load_library()
    fake = 1 << 40
    fp = ctypes.c_void_p(fake)
    z = ctypes.c_void_p(0)
    c = sa._Cache(600, 8, 128, 800, 4, 64, 256, fake, fake, fake, fake, fake)
    assert L.sepcache_decode_workspace(ctypes.byref(c), 32) > (16 << 20)
    assert L.sepcache_decode_noalloc(ctypes.byref(c), fp, 32, fp, fp, 0.1, fp, z) == 6
    assert "scratch" in L.sepattn_strerror(6).decode()
    c.B = 64
    assert L.sepcache_decode_workspace(ctypes.byref(c), 32) <= (16 << 20)
    assert L.sepcache_decode_noalloc(ctypes.byref(c), z, 32, fp, fp, 0.1, fp, z) == 1    # null q
    assert L.sepcache_decode_noalloc(ctypes.byref(c), fp, 24, fp, fp, 0.1, fp, z) == 2   # group of 3
    assert L.sepcache_decode_noalloc(ctypes.byref(c), fp, 32, fp, fp, -1.0, fp, z) == 1  # scale


def test_rope_table_host_matches_double_precision():
    c, d, theta = 800, 128, 500000.0
    cos, sin = sa.rope_table(theta, c, d)
    p = np.arange(c)[:, None].astype(np.float64)
    f = theta ** (-2.0 * np.arange(d // 2) / d)
    assert np.array_equal(cos, np.cos(p * f).astype(np.float32))
    assert np.array_equal(sin, np.sin(p * f).astype(np.float32))


def test_binding_refuses_host_tensors():
    """No CPU path: every entry point of the binding raises on host tensors
    before anything reaches the library."""
    import torch
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16)
    k = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    tok = torch.zeros((1, 64), dtype=torch.int32)
    with pytest.raises(TypeError, match="CUDA"):
        sa.build_index(tok, [1, 2], 4, 8)
    with pytest.raises(TypeError, match="CUDA"):
        sa.fwd(q, k, k, None)
    with pytest.raises(TypeError, match="CUDA"):
        sa.bwd(q, k, k, q, torch.zeros((1, 2, 64)), q, None)


def _anchor_chunks(B, Hq, Hkv, S, d):
    """Anchor chunks of a bf16 backward, read off its workspace size: the
    per-row (LSE, D) block plus, with several chunks, one fp32 dK and one dV
    partial slot of [B, Hkv, S, d] per chunk."""
    L = sa.load_library()
    a256 = lambda x: (x + 255) // 256 * 256
    ws = L.sepattn_bwd_workspace(B, Hq, Hkv, S, d, 1)
    rest = ws - a256(B * Hq * ((S + 63) // 64) * 128 * 4)
    slot = B * Hkv * S * d * 4
    assert rest % (2 * slot) == 0, (ws, rest, slot)
    return max(1, rest // (2 * slot))


@pytest.mark.parametrize("B,Hq,Hkv,S,d,chunks", [
    (8, 12, 12, 2048, 64, 1),     # Pythia-shaped: no split
    (1, 32, 8, 8192, 128, 13),    # Llama-shaped 8k: 13 chunks of 5 query tiles
    (1, 32, 8, 32768, 128, 7),    # 32k tokens: 4 by the item target, 7 once chunks stop at 40 tiles
    (1, 12, 12, 12288, 64, 3),    # 2 by the target, 3 by the 40-tile bound
    (1, 2, 1, 2304, 128, 9),      # 256 by the target: 16 at most, so chunks of 2 tiles
])
def test_anchor_chunk_split(B, Hq, Hkv, S, d, chunks):
    """The backward's anchor chunking: the item target, chunks of at most 40
    query tiles once the anchor rows are split, at most 16 chunks (host
    logic; the GPU tests run these splits against the oracle)."""
    assert _anchor_chunks(B, Hq, Hkv, S, d) == chunks


def test_anchor_chunks_never_more_than_16():
    for S in (4096, 16384, 65536, 131072, 262144):
        for B, Hkv in ((1, 1), (1, 8), (4, 8)):
            assert 1 <= _anchor_chunks(B, Hkv, Hkv, S, 128) <= 16
