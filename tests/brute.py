"""Brute-force attention with scalar Python loops, for pinning the oracle on tiny inputs.

Written independently of ``oracle``: visible keys come from closed-form index
ranges (not from boolean predicates over an index grid), every sum is
``math.fsum`` and every exponential is ``math.exp``.  Only for inputs of a few
dozen elements.

A mask spec is a dict with any of:
    causal: True               keys 0 .. p
    window: (left, right)      keys p-left .. p+right (negative = unbounded)
    docs: [len, ...]           keys of the document holding p
    block: bs                  keys 0 .. (p // bs + 1) * bs - 1
    tiles: (tile_map, T, inner_spec)   BlockMask over raw query index q; tile_map is
                               [q tile][k tile], or [Bm][Hm][q tile][k tile] with a
                               size-1 batch or head level shared
    key_range: (lo, hi)        keys lo .. hi - 1
with p = q + (Nk - Nq).
"""
import math


def _range_keys(spec, q, Nq, Nk, b=0, h=0):
    p = q + (Nk - Nq)
    keys = set(range(Nk))
    if spec.get("causal"):
        keys &= set(range(0, min(Nk, p + 1)))
    if "window" in spec:
        left, right = spec["window"]
        lo = 0 if left < 0 else max(0, p - left)
        hi = Nk - 1 if right < 0 else min(Nk - 1, p + right)
        keys &= set(range(lo, hi + 1))
    if "docs" in spec:
        start = 0
        doc = set()
        for ln in spec["docs"]:
            if start <= p < start + ln:
                doc = set(range(start, start + ln))
            start += ln
        keys &= doc
    if "block" in spec:
        bs = spec["block"]
        keys &= set(range(0, min(Nk, (p // bs + 1) * bs)))
    if "key_range" in spec:
        lo, hi = spec["key_range"]
        keys &= set(range(lo, hi))
    if "tiles" in spec:
        tmap, T, inner = spec["tiles"]
        if isinstance(tmap[0][0], (list, tuple)):  # one map per (batch, head)
            tmap = tmap[b if len(tmap) > 1 else 0]
            tmap = tmap[h if len(tmap) > 1 else 0]
        inner_keys = set(_range_keys(inner, q, Nq, Nk, b, h))
        allowed = set()
        for kt in range(len(tmap[0])):
            state = int(tmap[q // T][kt])
            tile_keys = set(range(kt * T, min(Nk, (kt + 1) * T)))
            if state == 2:
                allowed |= tile_keys
            elif state == 1:
                allowed |= tile_keys & inner_keys
        keys &= allowed
    return sorted(keys)


def _bias(score_spec, h, j, p):
    """Additive score change for query head h, key j, query position p."""
    if not score_spec:
        return 0.0
    add = 0.0
    if "alibi" in score_spec:
        add += score_spec["alibi"][h] * (j - p)
    if "alibi_sym" in score_spec:
        add -= score_spec["alibi_sym"][h] * abs(j - p)
    if "rel" in score_spec:
        table, R = score_spec["rel"]
        d = j - p
        if d < -R:
            d = -R
        if d > R:
            d = R
        add += table[h][d + R]
    return add


def _cap(score_spec, x):
    """Tanh capping of the scaled score, applied before the additive terms."""
    if not score_spec or "softcap" not in score_spec:
        return x
    c = score_spec["softcap"]
    return c * math.tanh(x / c)


def attention(q, k, v, scale, spec, score_spec=None):
    """q: nested lists [B][Hq][Nq][D]; k, v: [B][Hkv][Nk][D].  Returns (O, LSE) nested lists.

    score_spec (optional) adds to each scaled score: "alibi": slopes per head
    (+ slope (j - p)), "alibi_sym": slopes (- slope |j - p|), "rel": (table, R)
    (+ table[h][clamp(j - p, -R, R) + R]), "softcap": cap (the scaled score becomes
    cap * tanh(score / cap) before the additive terms)."""
    B, Hq = len(q), len(q[0])
    Hkv = len(k[0])
    Nq, Nk = len(q[0][0]), len(k[0][0])
    G = Hq // Hkv
    O, L = [], []
    for b in range(B):
        Ob, Lb = [], []
        for h in range(Hq):
            kv = h // G
            Oh, Lh = [], []
            for i in range(Nq):
                keys = _range_keys(spec, i, Nq, Nk, b, h)
                dv = len(v[b][kv][0]) if Nk else len(q[b][h][i])
                if not keys:
                    Oh.append([0.0] * dv)
                    Lh.append(-math.inf)
                    continue
                pos = i + (Nk - Nq)
                s = {j: _cap(score_spec, scale * math.fsum(a * c for a, c in zip(q[b][h][i], k[b][kv][j])))
                     + _bias(score_spec, h, j, pos) for j in keys}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in keys}
                tot = math.fsum(e.values())
                Oh.append([math.fsum(e[j] * v[b][kv][j][d] for j in keys) / tot for d in range(dv)])
                Lh.append(m + math.log(tot))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        L.append(Lb)
    return O, L
