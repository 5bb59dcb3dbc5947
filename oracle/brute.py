"""Pure-Python scalar MLA decode for tiny inputs.

TEST INFRASTRUCTURE ONLY (same import rule as ``oracle.mla_ref``). A second,
loop-by-loop statement of the same attention, written without NumPy, used to
pin ``oracle.mla_ref.attend_sequence`` on inputs small enough for scalar loops.

Per query j of Q (position p = L - Q + j) and head h, for every cached token
t <= p: the content key is W_UK[h] c_t, the positional key is the RoPE key of
token t rotated by t, the positional query is q_rope rotated by p; the score is
scale times the sum of both dot products ("Beyond the Attention Bottleneck",
"Down-Projection and Up-Projection Mechanics" and "The RoPE Compatibility
Problem"). Softmax over t, then the weighted sum of V_t = W_UV[h] c_t.

With a drafted tree (``parents``, "The Architecture of Memory", "Tree
Attention Verification"), query j sees every prefix token and the drafted
tokens met by following parent links up from j; a drafted token's position,
for its key and its query, is L - Q plus the number of parent links from it
to the prefix.
"""
import math


def _rotate(vec, pos, base):
    d = len(vec)
    out = [0.0] * d
    for i in range(d // 2):
        ang = pos * base ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        a, b = vec[2 * i], vec[2 * i + 1]
        out[2 * i] = a * c - b * s
        out[2 * i + 1] = a * s + b * c
    return out


def _dot(a, b):
    acc = 0.0
    for x, y in zip(a, b):
        acc += x * y
    return acc


def _matvec(m, v):
    return [_dot(row, v) for row in m]


def _links_to_prefix(parents, i):
    n = 0
    while parents[i] != -1:
        i = parents[i]
        n += 1
    return n


def _on_branch(parents, j, i):
    k = j
    while k != -1:
        if k == i:
            return True
        k = parents[k]
    return False


def brute_sequence(c, k_rope, q_nope, q_rope, w_uk, w_uv, scale, base=10000.0, parents=None,
                   selected=None):
    """Nested lists in, nested lists out: (o [Q][H][d_v], o_lat [Q][H][d_c], lse [Q][H]).

    ``selected``: per query, the cached tokens it reads (a sparse read); each
    keeps its own position."""
    L = len(c)
    Q = len(q_nope)
    H = len(w_uk)
    pre = L - Q

    def key_pos(t):
        if parents is None or t < pre:
            return t
        return pre + _links_to_prefix(parents, t - pre)

    def sees(j, t):
        if selected is not None:
            assert parents is None
            return t in selected[j] and t <= pre + j
        if parents is None:
            return t <= pre + j
        return t < pre or _on_branch(parents, j, t - pre)

    o, o_lat, lse = [], [], []
    for j in range(Q):
        p = pre + j if parents is None else pre + _links_to_prefix(parents, j)
        vis = [t for t in range(L) if sees(j, t)]
        oj, olj, lj = [], [], []
        for h in range(H):
            q_pe = _rotate(q_rope[j][h], p, base)
            scores = []
            for t in vis:
                k_c = _matvec(w_uk[h], c[t])
                k_r = _rotate(k_rope[t], key_pos(t), base)
                scores.append(scale * (_dot(q_nope[j][h], k_c) + _dot(q_pe, k_r)))
            m = max(scores)
            ex = [math.exp(s - m) for s in scores]
            z = sum(ex)
            dv = len(w_uv[h])
            acc = [0.0] * dv
            acc_lat = [0.0] * len(c[0])
            for k, t in enumerate(vis):
                w = ex[k] / z
                v_t = _matvec(w_uv[h], c[t])
                for i in range(dv):
                    acc[i] += w * v_t[i]
                for i in range(len(c[0])):
                    acc_lat[i] += w * c[t][i]
            oj.append(acc)
            olj.append(acc_lat)
            lj.append(m + math.log(z))
        o.append(oj)
        o_lat.append(olj)
        lse.append(lj)
    return o, o_lat, lse


def brute_index_scores(q_idx, w_idx, k_idx):
    """Scalar loops: score[j][t] = sum over scorer heads h of
    w[j][h] * max(0, q[j][h] . k[t]) ("DeepSeek's Config Says 16 KV Heads",
    section 6, "Sparse attention"; the weighted-ReLU form is a reading)."""
    out = []
    for qj, wj in zip(q_idx, w_idx):
        row = []
        for kt in k_idx:
            acc = 0.0
            for qh, wh in zip(qj, wj):
                d = _dot(qh, kt)
                if d > 0.0:
                    acc += wh * d
            row.append(acc)
        out.append(row)
    return out
