"""Stand-in target models for the greedy-identity check of the oracle's decode loop.

Neither is the method: they only play the main model's part (logits and hiddens
for every fed position, a cache that can be cut, a recurrent state that must be
copied and restored)."""
import hashlib

import numpy as np


def _rms(x):
    return x / np.sqrt(np.mean(x * x) + 1e-6)


class HashTarget:
    """Stateless random LM: logits and hidden at a position are a seeded function of the prefix."""

    def __init__(self, vocab, hidden, scale=1.0):
        self.V, self.H, self.scale = vocab, hidden, scale

    def new_state(self):
        return {"toks": []}

    def _out(self, toks):
        seed = int.from_bytes(hashlib.blake2b(np.asarray(toks, np.int64).tobytes(), digest_size=8).digest(), "little")
        g = np.random.default_rng(seed)
        return g.standard_normal(self.V) * self.scale, g.standard_normal(self.H)

    def forward(self, st, tokens):
        L, Hs = [], []
        for t in tokens:
            st["toks"].append(int(t))
            l, h = self._out(st["toks"])
            L.append(l)
            Hs.append(h)
        return np.array(L), np.array(Hs)

    def length(self, st):
        return len(st["toks"])

    def crop(self, st, n):
        del st["toks"][n:]

    def recurrent(self, st):
        return np.zeros((1, 0), np.uint8)

    def set_recurrent(self, st, b):
        pass


class TinyHybridTarget:
    """Two causal attention layers and one toy recurrent layer (S <- 0.9 S + k v^T over a
    width-4 causal convolution of its inputs), final RMSNorm and lm_head.  The
    recurrent layer only exercises the snapshot / restore mechanism."""

    def __init__(self, embed, seed=0, heads=2, hd=8):
        g = np.random.default_rng(seed)
        self.E = np.asarray(embed, float)
        self.V, self.H = self.E.shape
        H = self.H
        self.heads, self.hd = heads, hd
        self.att = [dict(q=g.standard_normal((heads * hd, H)) * 0.3, k=g.standard_normal((heads * hd, H)) * 0.3,
                         v=g.standard_normal((heads * hd, H)) * 0.3, o=g.standard_normal((H, heads * hd)) * 0.2)
                    for _ in range(2)]
        self.conv_w = g.standard_normal(4) * 0.5
        self.rk = g.standard_normal((8, H)) * 0.3
        self.rv = g.standard_normal((8, H)) * 0.3
        self.rq = g.standard_normal((8, H)) * 0.3
        self.ro = g.standard_normal((H, 8)) * 0.3
        self.lm = g.standard_normal((self.V, H)) * 1.5

    def new_state(self):
        return {"k": [[], []], "v": [[], []], "S": np.zeros((8, 8)), "conv": np.zeros((3, self.H)), "pos": 0}

    def _rot(self, x, pos):
        half = self.hd // 2
        ang = pos * 1e4 ** (-np.arange(half) * 2.0 / self.hd)
        a, b = x[..., :half], x[..., half:]
        return np.concatenate([a * np.cos(ang) - b * np.sin(ang), b * np.cos(ang) + a * np.sin(ang)], -1)

    def forward(self, st, tokens):
        L, Hs = [], []
        for t in tokens:
            x = self.E[int(t)].copy()
            pos = st["pos"]
            for li, w in enumerate(self.att):
                a = _rms(x)
                q = self._rot((w["q"] @ a).reshape(self.heads, self.hd), pos)
                k = self._rot((w["k"] @ a).reshape(self.heads, self.hd), pos)
                v = (w["v"] @ a).reshape(self.heads, self.hd)
                st["k"][li].append(k)
                st["v"][li].append(v)
                K, Vv = np.array(st["k"][li]), np.array(st["v"][li])
                o = []
                for h in range(self.heads):
                    s = K[:, h] @ q[h] / np.sqrt(self.hd)
                    p = np.exp(s - s.max())
                    o.append((p / p.sum()) @ Vv[:, h])
                x = x + w["o"] @ np.concatenate(o)
            a = _rms(x)
            win = np.concatenate([st["conv"], a[None]], 0)
            c = self.conv_w @ win
            st["conv"] = win[1:]
            st["S"] = 0.9 * st["S"] + np.outer(self.rk @ c, self.rv @ c)
            x = x + self.ro @ (st["S"].T @ (self.rq @ c))
            h = _rms(x)
            L.append(self.lm @ h)
            Hs.append(h)
            st["pos"] += 1
        return np.array(L), np.array(Hs)

    def length(self, st):
        return st["pos"]

    def crop(self, st, n):
        for li in range(2):
            del st["k"][li][n:]
            del st["v"][li][n:]
        st["pos"] = n

    def recurrent(self, st):
        return np.concatenate([st["S"].ravel(), st["conv"].ravel()]).view(np.uint8)[None].copy()

    def set_recurrent(self, st, b):
        f = np.ascontiguousarray(b[0]).view(np.float64)
        st["S"] = f[:64].reshape(8, 8).copy()
        st["conv"] = f[64:].reshape(3, self.H).copy()


def plain_greedy(target, prompt, max_new):
    """One target forward per token, argmax (first maximum) each time."""
    st = target.new_state()
    logits, _ = target.forward(st, list(prompt))
    x = int(np.argmax(logits[-1]))
    out = [x]
    while len(out) < max_new:
        logits, _ = target.forward(st, [x])
        x = int(np.argmax(logits[-1]))
        out.append(x)
    return out
