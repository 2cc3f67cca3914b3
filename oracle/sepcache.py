"""SepCache: the streaming four-block KV cache, positional shifting and decode
attention over it (oracle; test infrastructure only -- see ``oracle/__init__.py``).

Sources
-------
* "How SepLLM Reorchestrates the Language Model for Speed and Efficiency"
  (beiduofen.top), "SepLLM's Architecture: Composing Efficiency": four blocks --
  an Initial Cache of the first few tokens, a Local Window Cache of capacity
  ``w``, a Past Window Cache that holds older tokens until total usage reaches
  ``c``, and a Separator Cache that keeps only the separators of the Past
  Window; when usage reaches ``c`` the separators move to the Separator Cache
  and the other Past-Window tokens are dropped.
* atlas.scime.ai, "Measured effects reported in the paper": Separator Cache
  capacity ``s`` (32 or 64); removing positional-encoding shifting in the
  streaming setting ruins perplexity.  Project card (sourcepulse.org),
  "Limitations & Caveats": the streaming variant needs positional-encoding
  shifting.
* atlas.scime.ai, "Key results": a streaming run at total capacity c = 800.

Readings (the pages leave these open)
-------------------------------------
* the cache starts empty and the first ``a`` streamed tokens form the Initial
  Cache; every later token enters the window;
* compression fires right after an append brings usage ``|I|+|Sp|+|W|`` to
  ``c``: the Past Window is everything in the window but its ``w`` most recent
  tokens; its separators join the Separator Cache in stream order, the rest are
  dropped; attention then runs on the compressed cache (so it sees at most
  ``c - 1`` slots);
* Separator Cache overflow: first in, first out -- only the ``s`` most recent
  separators are kept;
* positional shifting: slot ``k`` of the cache (order I, Sp, W) has position
  ``k``; the current token's query sits at the last slot;
* rotary embedding: rotate-half form with frequencies ``theta^(-2m/d)``,
  ``m < d/2``; keys and values are stored without it and rotated by slot at
  attention time;
* grouped-query heads: query head ``h`` reads kv head ``h // (Hq // Hkv)``.
"""

import numpy as np


class Entry:
    """One cached token: stream position, token id and an opaque payload
    (the key and value rows, carried bit for bit)."""

    __slots__ = ("pos", "tok", "k", "v")

    def __init__(self, pos, tok, k, v):
        self.pos = pos
        self.tok = tok
        self.k = k
        self.v = v


class SepCacheSim:
    """List simulation of one sequence's SepCache.

    ``trigger="capacity"`` is the policy of the pages (compress when usage
    reaches ``c``).  ``trigger="window"`` compresses as soon as the window
    holds more than ``w`` tokens; with ``s=None`` (unbounded) its cache equals
    the set of keys the SepLLM mask lets the newest token see with ``n = w``
    -- a tie between the two definitions used as a pin.
    """

    def __init__(self, a, s, w, c, sep_ids, trigger="capacity"):
        if trigger == "capacity" and not (c > a + (s or 0) + w):
            raise ValueError("capacity must exceed a + s + w")
        if w < 1:
            raise ValueError("window capacity must be >= 1")
        self.a, self.s, self.w, self.c = a, s, w, c
        self.sep_ids = set(int(x) for x in np.asarray(sep_ids).reshape(-1))
        self.trigger = trigger
        self.I, self.Sp, self.W = [], [], []
        self.t = 0
        self.compressions = 0

    def is_sep(self, tok):
        return int(tok) in self.sep_ids

    def usage(self):
        return len(self.I) + len(self.Sp) + len(self.W)

    def append(self, tok, k=None, v=None):
        """Stream one token in; returns True when a compression happened."""
        e = Entry(self.t, int(tok), k, v)
        if len(self.I) < self.a:
            self.I.append(e)
        else:
            self.W.append(e)
        self.t += 1
        if self.trigger == "capacity":
            fire = self.usage() == self.c
        else:
            fire = len(self.W) > self.w
        if fire:
            cut = len(self.W) - self.w
            past = self.W[:cut]
            self.W = self.W[cut:]
            self.Sp = self.Sp + [e for e in past if self.is_sep(e.tok)]
            if self.s is not None and len(self.Sp) > self.s:
                self.Sp = self.Sp[len(self.Sp) - self.s:]
            self.compressions += 1
            return True
        return False

    def slots(self):
        """Cache contents in slot order: Initial, Separator, Window."""
        return self.I + self.Sp + self.W

    def positions(self):
        return [e.pos for e in self.slots()]

    def state(self):
        """(n_init, n_sep, n_win, tokens seen)."""
        return (len(self.I), len(self.Sp), len(self.W), self.t)


def rope_rotate(x, p, theta):
    """Rotate-half rotary embedding of ``x`` [..., d] at position(s) ``p``
    (broadcast against x[..., 0]), fp64:

      x'_m       = x_m cos(p f_m) - x_{m+d/2} sin(p f_m)
      x'_{m+d/2} = x_{m+d/2} cos(p f_m) + x_m sin(p f_m),   f_m = theta^(-2m/d).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    m = np.arange(h, dtype=np.float64)
    f = theta ** (-2.0 * m / d)
    ang = np.asarray(p, dtype=np.float64)[..., None] * f
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def decode_attention(q, kslots, vslots, scale, theta):
    """Decode attention of the newest token over a compressed cache.

    q [Hq,d] (pre-rotation), kslots/vslots [L,Hkv,d] in slot order
    (pre-rotation keys).  The query is rotated at slot ``L-1`` and key ``k`` at
    slot ``k``; softmax over all ``L`` slots; returns o [Hq,d] fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(kslots, dtype=np.float64)
    V = np.asarray(vslots, dtype=np.float64)
    L, Hkv, d = K.shape
    Hq = q.shape[0]
    grp = Hq // Hkv
    qr = rope_rotate(q, L - 1, theta)
    kr = rope_rotate(K, np.arange(L)[:, None], theta)
    o = np.zeros((Hq, d))
    for h in range(Hq):
        g = h // grp
        z = scale * (kr[:, g, :] @ qr[h])
        z = z - z.max()
        p = np.exp(z)
        p /= p.sum()
        o[h] = p @ V[:, g, :]
    return o


def cache_arrays(sim, c, Hkv, d):
    """The cache of one sequence laid out as the GPU keeps it: slots
    ``[0, L)`` hold I, Sp, W in order; ``pos``/``tok`` are -1 past ``L``;
    K/V rows are the payloads (uint16 bf16 bit patterns [Hkv,d]); returns
    (k [Hkv,L,d] uint16, v [Hkv,L,d], pos [c] int32, tok [c] int32,
    state [4] int32) -- only the ``L`` occupied slots of k and v."""
    slots = sim.slots()
    L = len(slots)
    k = np.zeros((Hkv, c, d), dtype=np.uint16)
    v = np.zeros((Hkv, c, d), dtype=np.uint16)
    pos = np.full(c, -1, dtype=np.int32)
    tok = np.full(c, -1, dtype=np.int32)
    for i, e in enumerate(slots):
        k[:, i, :] = e.k
        v[:, i, :] = e.v
        pos[i] = e.pos
        tok[i] = e.tok
    st = np.array(sim.state(), dtype=np.int32)
    return k[:, :L], v[:, :L], pos, tok, st
