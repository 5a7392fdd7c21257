"""Pure-Python brute-force attention for tiny shapes (TEST INFRASTRUCTURE ONLY).

A second, independent statement of softmax(scale * Q K^T) V ("FlashInfer
kernel library ...", zyxy.net/archives/24491, section 1) on nested lists, with
math.exp / math.log and exactly-rounded sums (math.fsum).  It exists to
cross-check the C oracle on shapes of a handful of elements; it does not share
code with it.
"""
import math


def attention_row(q, keys, values, scale, allowed=None):
    """One query row against lists of key and value rows.

    ``allowed[j]`` False masks key j.  Returns (o, lse); a row with no allowed
    key gives ([0]*d, -inf).
    """
    n = len(keys)
    d = len(values[0]) if values else len(q)
    s = []
    for j in range(n):
        if allowed is not None and not allowed[j]:
            s.append(None)
        else:
            s.append(scale * math.fsum(q[c] * keys[j][c] for c in range(len(q))))
    live = [x for x in s if x is not None]
    if not live:
        return [0.0] * d, -math.inf
    m = max(live)
    w = [0.0 if x is None else math.exp(x - m) for x in s]
    total = math.fsum(w)
    o = [math.fsum(w[j] * values[j][c] for j in range(n)) / total for c in range(d)]
    return o, m + math.log(total)


def attention(q, k, v, causal, scale):
    """q [B][Hq][Tq][D], k/v [B][Hkv][Tk][D] as nested lists of floats."""
    B, Hq, Hkv = len(q), len(q[0]), len(k[0])
    group = Hq // Hkv
    o = []
    lse = []
    for b in range(B):
        ob, lb = [], []
        for h in range(Hq):
            keys, vals = k[b][h // group], v[b][h // group]
            tq, tk = len(q[b][h]), len(keys)
            oh, lh = [], []
            for i in range(tq):
                allowed = [(not causal) or j <= i + (tk - tq) for j in range(tk)]
                r, l = attention_row(q[b][h][i], keys, vals, scale, allowed)
                oh.append(r)
                lh.append(l)
            ob.append(oh)
            lb.append(lh)
        o.append(ob)
        lse.append(lb)
    return o, lse


def unified_fallback_count(q, keys, lengths, scale, split_tokens, phi, window=60.0):
    """Fallback pairs of the unified-max softmax, by brute force.

    q[b][h] is a query row, keys[b][kvh][t] the t-th key of sequence b (no
    paging), lengths[b] the number of keys; head h reads kv head
    h // (len(q[b]) // len(keys[b])).  A (row, chunk of split_tokens keys) pair
    counts when its largest scaled score is more than window away from phi.
    """
    count = 0
    for b in range(len(q)):
        group = len(q[b]) // len(keys[b])
        for h in range(len(q[b])):
            ks = keys[b][h // group]
            for c0 in range(0, lengths[b], split_tokens):
                s = [scale * math.fsum(x * y for x, y in zip(q[b][h], ks[t]))
                     for t in range(c0, min(lengths[b], c0 + split_tokens))]
                if abs(max(s) - phi) > window:
                    count += 1
    return count
