"""Pins of the oracle's attention forward and backward (CPU only).

* reductions to library routines: torch SDPA on the CPU in fp64 with
  ``is_causal`` (n >= S) and with a sink + sliding-window mask built from
  triangular matrices (no separators);
* closed forms: a=0, no separators, n=1 gives O = V and zero dQ/dK; Q = 0
  gives the mean of the visible values and LSE = log(visible count);
* gradients: torch autograd in fp64 on an independent formulation (masked
  fill + softmax with repeated kv heads), and central finite differences;
* internal consistency of the row-blocked and sampled variants.
"""

import numpy as np
import pytest
import torch

from oracle import attention, sepmask


def _rand(seed, B, Hq, Hkv, S, d, p_sep=0.2):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, S, d))
    k = r.standard_normal((B, Hkv, S, d))
    v = r.standard_normal((B, Hkv, S, d))
    do = r.standard_normal((B, Hq, S, d))
    sep_ids = [3, 9]
    tok = np.where(r.random((B, S)) < p_sep, 3, 20 + r.integers(0, 50, (B, S)))
    return q, k, v, do, tok, sep_ids


def _torch_ref(q, k, v, mask, scale):
    """Independent torch formulation: kv heads repeated to the query heads,
    masked_fill(-inf), softmax, matmul.  mask: bool [B,S,S]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    kk = k.repeat_interleave(Hq // Hkv, dim=1)
    vv = v.repeat_interleave(Hq // Hkv, dim=1)
    z = scale * torch.matmul(q, kk.transpose(-1, -2).contiguous())
    z = z.masked_fill(~mask[:, None], float("-inf"))
    lse = torch.logsumexp(z, dim=-1)
    return torch.matmul(torch.softmax(z, dim=-1), vv), lse


def _masks(tok, sep_ids, a, n):
    return torch.tensor(np.stack([sepmask.sep_mask(t, sep_ids, a, n) for t in tok]))


def test_dense_reduction_matches_sdpa():
    q, k, v, do, tok, sep = _rand(0, 2, 2, 2, 40, 8)
    o, lse = attention.attention_forward(q, k, v, tok, sep, a=3, n=40)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k), torch.tensor(v), is_causal=True)
    assert np.abs(o - ref.numpy()).max() < 1e-12


def test_streaming_reduction_matches_sdpa_band():
    q, k, v, do, tok, sep = _rand(1, 1, 3, 3, 64, 8)
    tok = np.full_like(tok, 50)  # no separators
    a, n = 4, 9
    o, _ = attention.attention_forward(q, k, v, tok, sep, a=a, n=n)
    S = 64
    ones = torch.ones(S, S, dtype=torch.bool)
    allowed = (torch.tril(ones) & torch.triu(ones, -(n - 1))) | (torch.tril(ones) & (torch.arange(S)[None] < a))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k), torch.tensor(v), attn_mask=allowed)
    assert np.abs(o - ref.numpy()).max() < 1e-12


def test_closed_form_identity_window():
    """a=0, no separators, n=1: each query sees only itself."""
    q, k, v, do, tok, sep = _rand(2, 2, 4, 2, 23, 6)
    tok = np.full_like(tok, 50)
    o, lse = attention.attention_forward(q, k, v, tok, sep, a=0, n=1)
    grp = 2
    for h in range(4):
        assert np.array_equal(o[:, h], v[:, h // grp])
        scale = 1 / np.sqrt(6)
        assert np.allclose(lse[:, h], scale * (q[:, h] * k[:, h // grp]).sum(-1), atol=1e-13)
    dq, dk, dv = attention.attention_backward(q, k, v, do, tok, sep, a=0, n=1)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    assert np.allclose(dv[:, 0], do[:, 0] + do[:, 1], atol=1e-13)
    assert np.allclose(dv[:, 1], do[:, 2] + do[:, 3], atol=1e-13)


def test_closed_form_zero_query():
    """Q = 0: uniform weights over the visible keys."""
    q, k, v, do, tok, sep = _rand(3, 1, 2, 1, 70, 5)
    q[:] = 0
    a, n = 2, 7
    o, lse = attention.attention_forward(q, k, v, tok, sep, a=a, n=n)
    M = sepmask.sep_mask(tok[0], sep, a, n)
    cnt = M.sum(1)
    want = (M.astype(float) @ v[0, 0]) / cnt[:, None]
    assert np.abs(o[0, 0] - want).max() < 1e-13
    assert np.abs(lse[0, 1] - np.log(cnt)).max() < 1e-13


@pytest.mark.parametrize("Hq,Hkv,a,n", [(4, 2, 2, 5), (3, 3, 0, 1), (2, 1, 4, 64), (4, 1, 1, 3)])
def test_forward_backward_match_autograd(Hq, Hkv, a, n):
    q, k, v, do, tok, sep = _rand(4 + n, 2, Hq, Hkv, 33, 8, p_sep=0.25)
    scale = 0.37
    o, lse = attention.attention_forward(q, k, v, tok, sep, a, n, scale=scale)
    dq, dk, dv = attention.attention_backward(q, k, v, do, tok, sep, a, n, scale=scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ref, ref_lse = _torch_ref(tq, tk, tv, _masks(tok, sep, a, n), scale)
    (ref * torch.tensor(do)).sum().backward()
    assert np.abs(o - ref.detach().numpy()).max() < 1e-12
    assert np.abs(lse - ref_lse.detach().numpy()).max() < 1e-12
    for mine, theirs in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        t = theirs.numpy()
        assert np.abs(mine - t).max() <= 1e-10 * max(1.0, np.abs(t).max())


def test_backward_finite_differences():
    q, k, v, do, tok, sep = _rand(9, 1, 2, 1, 10, 3, p_sep=0.3)
    a, n, scale = 1, 3, 0.8
    dq, dk, dv = attention.attention_backward(q, k, v, do, tok, sep, a, n, scale=scale)

    def loss(qq, kk, vv):
        o, _ = attention.attention_forward(qq, kk, vv, tok, sep, a, n, scale=scale)
        return (o * do).sum()

    eps = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][ix] += eps
            args_m[which][ix] -= eps
            num[ix] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        rel = np.abs(num - grad).max() / max(1e-3, np.abs(grad).max())
        assert rel < 1e-6, (which, rel)


def test_row_blocking_and_sampled_variants_agree():
    q, k, v, do, tok, sep = _rand(11, 1, 4, 2, 90, 8, p_sep=0.15)
    a, n = 3, 11
    scale = 1 / np.sqrt(8)
    o1, l1 = attention.attention_forward(q, k, v, tok, sep, a, n)
    o2, l2 = attention.attention_forward(q, k, v, tok, sep, a, n, row_block=7)
    assert np.abs(o1 - o2).max() < 1e-13 and np.abs(l1 - l2).max() < 1e-13
    g1 = attention.attention_backward(q, k, v, do, tok, sep, a, n)
    g2 = attention.attention_backward(q, k, v, do, tok, sep, a, n, row_block=13)
    for x, y in zip(g1, g2):
        assert np.abs(x - y).max() < 1e-12
    sepf = np.isin(tok[0], sep)
    rows = np.array([0, 5, 44, 89])
    orow, lrow = attention.attention_rows(q[0, 3], k[0, 1], v[0, 1], sepf, a, n, scale, rows)
    assert np.abs(orow - o1[0, 3, rows]).max() < 1e-13
    assert np.abs(lrow - l1[0, 3, rows]).max() < 1e-13
    dqr = attention.grad_q_rows(q[0, 2], k[0, 1], v[0, 1], do[0, 2], sepf, a, n, scale, rows)
    assert np.abs(dqr - g1[0][0, 2, rows]).max() < 1e-12
    cols = np.array([0, 2, 3, 40, 88, 89])
    dkc, dvc = attention.grad_kv_cols([q[0, 2], q[0, 3]], k[0, 1], v[0, 1], [do[0, 2], do[0, 3]],
                                      sepf, a, n, scale, cols, row_block=16)
    assert np.abs(dkc - g1[1][0, 1, cols]).max() < 1e-12
    assert np.abs(dvc - g1[2][0, 1, cols]).max() < 1e-12
