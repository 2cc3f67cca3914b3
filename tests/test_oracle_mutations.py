"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case swaps one oracle function for a copy with a deliberate mistake of
the kind the pins are meant to catch -- a dropped term, an off-by-one, a
wrong sign, a term taken from the wrong operand -- and runs the pins that
should notice; at least one of them must fail.  A control case runs the
same harness with no mistake planted, and every pin must then pass, so a
failure can only come from the mistake.  The copies live here, in the test;
the oracle itself is never edited.
"""

import numpy as np
import pytest

import tests.test_oracle_attention as pa
import tests.test_oracle_mask as pm
import tests.test_oracle_sepcache as pc
from oracle import attention, sepcache, sepmask


def _failures(calls):
    """Names of the pins (callables with their arguments) that fail."""
    out = []
    for fn, args in calls:
        try:
            fn(*args)
        except AssertionError:
            out.append(fn.__name__)
    return out


# --- the mask -----------------------------------------------------------------

def _mask_rows(kind):
    def mask_rows(sep, a, n, rows):
        S = sep.shape[0]
        i = np.asarray(rows, dtype=np.int64)[:, None]
        j = np.arange(S, dtype=np.int64)[None, :]
        causal = j <= i
        initial = j < a
        separator = sep[None, :]
        window = (i - j) < n
        if kind == "window_off_by_one":
            window = (i - j) <= n
        elif kind == "no_initial_term":
            initial = np.zeros_like(initial)
        elif kind == "no_causal_bound":
            causal = np.ones_like(causal)
        elif kind == "query_is_separator":
            separator = sep[np.asarray(rows)][:, None]
        return causal & (initial | separator | window)
    return mask_rows


@pytest.mark.parametrize("kind", ["none", "window_off_by_one", "no_initial_term", "no_causal_bound",
                                  "query_is_separator"])
def test_mask_pins_catch_planted_mistakes(kind, monkeypatch, golden):
    monkeypatch.setattr(sepmask, "mask_rows", _mask_rows(kind))
    failed = _failures([(pm.test_golden_mask_example, (golden,)), (pm.test_brute_force_all_patterns, (5,)),
                        (pm.test_brute_force_random_longer, ()), (pm.test_dense_reduction, ()),
                        (pm.test_streaming_reduction, ())])
    if kind == "none":
        assert failed == []
    else:
        assert failed, kind


def _row_nnz(kind):
    def row_nnz(sep, a, n, row_block=1024):
        S = sep.shape[0]
        out = np.zeros(S, dtype=np.int64)
        for r0 in range(0, S, row_block):
            hi = min(S, r0 + row_block)
            if kind == "last_row_of_block_dropped":
                hi = max(r0, hi - 1)
            rows = np.arange(r0, hi)
            if kind == "causal_count_only":
                out[rows] = rows + 1
            else:
                out[rows] = sepmask.mask_rows(sep, a, n, rows).sum(axis=1)
        return out
    return row_nnz


@pytest.mark.parametrize("kind", ["none", "last_row_of_block_dropped", "causal_count_only"])
def test_row_nnz_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(sepmask, "row_nnz", _row_nnz(kind))
    failed = _failures([(pm.test_row_nnz_brute_force_all_patterns, (6,)), (pm.test_row_nnz_random_longer_blocked, ()),
                        (pm.test_row_nnz_special_cases, ())])
    if kind == "none":
        assert failed == []
    else:
        assert failed, kind


# --- attention forward / backward ----------------------------------------------

def _masked_softmax(kind):
    def masked_softmax(Z, M):
        Zm = np.where(M, Z, -np.inf)
        m = Zm.max(axis=1)
        E = np.where(M, np.exp(Zm - m[:, None]), 0.0)
        ssum = E.sum(axis=1)
        if kind == "normaliser_over_masked_keys":
            ssum = np.exp(Z - m[:, None]).sum(axis=1)
        P = E / ssum[:, None]
        return P, m + np.log(ssum)
    return masked_softmax


def _backward(kind):
    """A dense fp64 backward (one materialised mask per sequence) with the
    mistake `kind` planted."""
    def backward(q, k, v, do, tok, sep_ids, a, n, scale=None, row_block=1024):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        B, Hq, S, d = q.shape
        grp = Hq // k.shape[1]
        scale = 1.0 / np.sqrt(d) if scale is None else scale
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            M = sepmask.sep_mask(tok[b], sep_ids, a, n)
            for h in range(Hq):
                g = h // grp
                Zm = np.where(M, scale * (q[b, h] @ k[b, g].T), -np.inf)
                P = np.exp(Zm - Zm.max(axis=1, keepdims=True))
                P /= P.sum(axis=1, keepdims=True)
                dP = do[b, h] @ v[b, g].T
                D = (P * dP).sum(axis=1, keepdims=True)
                dS = P * dP if kind == "dropped_D" else P * (dP - D)
                dq[b, h] = scale * (dS @ k[b, g])
                dk[b, g] += (1.0 if kind == "dk_without_scale" else scale) * (dS.T @ q[b, h])
                dv[b, g] += (P @ do[b, h]) if kind == "dv_untransposed_P" else (P.T @ do[b, h])
        return dq, dk, dv
    return backward


@pytest.mark.parametrize("kind", ["none", "normaliser_over_masked_keys"])
def test_forward_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(attention, "_masked_softmax", _masked_softmax(kind))
    failed = _failures([(pa.test_streaming_reduction_matches_sdpa_band, ()), (pa.test_closed_form_zero_query, ()),
                        (pa.test_forward_backward_match_autograd, (2, 1, 4, 64))])
    if kind == "none":
        assert failed == []
    else:
        assert failed, kind


@pytest.mark.parametrize("kind", ["none", "dropped_D", "dk_without_scale", "dv_untransposed_P"])
def test_backward_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(attention, "attention_backward", _backward(kind))
    failed = _failures([(pa.test_backward_finite_differences, ()),
                        (pa.test_forward_backward_match_autograd, (4, 2, 2, 5))])
    if kind == "none":
        assert failed == []
    else:
        assert failed, kind


# --- SepCache --------------------------------------------------------------------

def _append(kind):
    """SepCacheSim.append with the mistake `kind` planted."""
    def append(self, tok, k=None, v=None):
        e = sepcache.Entry(self.t, int(tok), k, v)
        if len(self.I) < self.a:
            self.I.append(e)
        else:
            self.W.append(e)
        self.t += 1
        fire = self.usage() == self.c if self.trigger == "capacity" else len(self.W) > self.w
        if not fire:
            return False
        cut = len(self.W) - self.w
        if kind == "window_keeps_oldest":
            past, self.W = self.W[self.w:], self.W[:self.w]
        else:
            past, self.W = self.W[:cut], self.W[cut:]
        self.Sp = self.Sp + [x for x in past if self.is_sep(x.tok)]
        if self.s is not None and len(self.Sp) > self.s:
            self.Sp = self.Sp[:self.s] if kind == "separators_keep_oldest" else self.Sp[len(self.Sp) - self.s:]
        self.compressions += 1
        return True
    return append


def _rope(kind):
    def rope_rotate(x, p, theta):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        h = d // 2
        f = theta ** (-2.0 * np.arange(h, dtype=np.float64) / d)
        ang = np.asarray(p, dtype=np.float64)[..., None] * f
        c, s = np.cos(ang), np.sin(ang)
        if kind == "sign_flipped":
            s = -s
        lo, hi = x[..., :h], x[..., h:]
        return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)
    return rope_rotate


def _decode(kind):
    def decode_attention(q, kslots, vslots, scale, theta):
        q, K, V = (np.asarray(x, dtype=np.float64) for x in (q, kslots, vslots))
        L, Hkv, d = K.shape
        grp = q.shape[0] // Hkv
        qr = sepcache.rope_rotate(q, L if kind == "query_at_slot_L" else L - 1, theta)
        kr = sepcache.rope_rotate(K, np.arange(L)[:, None], theta)
        o = np.zeros((q.shape[0], d))
        for h in range(q.shape[0]):
            z = scale * (kr[:, h // grp, :] @ qr[h])
            p = np.exp(z - z.max())
            o[h] = (p / p.sum()) @ V[:, h // grp, :]
        return o
    return decode_attention


@pytest.mark.parametrize("kind", ["none", "window_keeps_oldest", "separators_keep_oldest"])
def test_cache_update_pins_catch_planted_mistakes(kind, monkeypatch, golden):
    monkeypatch.setattr(sepcache.SepCacheSim, "append", _append(kind))
    failed = _failures([(pc.test_golden_trace, (golden,)), (pc.test_invariants, (2, 2, 3, 8, 0.4)),
                        (pc.test_cache_equals_mask_row_when_compressing_every_overflow, (2, 5, 0.3))])
    if kind == "none":
        assert failed == []
    else:
        assert failed, kind


def _cache_arrays(kind):
    def cache_arrays(sim, c, Hkv, d):
        slots = sim.I + sim.W + sim.Sp if kind == "window_before_separators" else sim.slots()
        L = len(slots)
        k = np.zeros((Hkv, c, d), dtype=np.uint16)
        v = np.zeros((Hkv, c, d), dtype=np.uint16)
        fill = 0 if kind == "zero_past_length" else -1
        pos = np.full(c, fill, dtype=np.int32)
        tok = np.full(c, fill, dtype=np.int32)
        for i, e in enumerate(slots):
            k[:, i, :] = e.k
            v[:, i, :] = e.k if kind == "value_from_key" else e.v
            pos[i] = e.pos
            tok[i] = e.tok
        n_init, n_sep, n_win, t = sim.state()
        if kind == "counters_swapped":
            n_sep, n_win = n_win, n_sep
        return k[:, :L], v[:, :L], pos, tok, np.array([n_init, n_sep, n_win, t], dtype=np.int32)
    return cache_arrays


@pytest.mark.parametrize("kind", ["none", "window_before_separators", "zero_past_length", "value_from_key",
                                  "counters_swapped"])
def test_cache_arrays_pins_catch_planted_mistakes(kind, monkeypatch, golden):
    monkeypatch.setattr(sepcache, "cache_arrays", _cache_arrays(kind))
    failed = _failures([(pc.test_cache_arrays_golden_trace, (golden,))])
    if kind == "none":
        assert failed == []
    else:
        assert failed, kind


@pytest.mark.parametrize("kind", ["none", "sign_flipped"])
def test_rope_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(sepcache, "rope_rotate", _rope(kind))
    failed = _failures([(pc.test_rope_forms_and_properties, ()),
                        (pc.test_decode_before_compression_is_causal_attention, ())])
    if kind == "none":
        assert failed == []
    else:
        assert failed, kind


@pytest.mark.parametrize("kind", ["none", "query_at_slot_L"])
def test_decode_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(sepcache, "decode_attention", _decode(kind))
    failed = _failures([(pc.test_decode_before_compression_is_causal_attention, ()),
                        (pc.test_decode_closed_forms, ())])
    if kind == "none":
        assert failed == []
    else:
        assert failed, kind
