"""Float64 CPU oracle of exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Sources (web pages on IO-aware exact attention; cited by title and section):
  [FAQ-short] "Walk through what FlashAttention does differently from standard
              attention, and what changes between v1, v2, and v3" (zenaique.com,
              attn-flashattention-family-shortans-hard): answer paragraphs 1-2.
  [Card]      "FlashAttention Kernel & Online Softmax" (talentme.airsota.com
              mind-map card): definition paragraph, history paragraph, prompts.
  [Blog]      "FlashAttention" (akshathtiwari.co.in/blog/flashattention): the
              explainer paragraph (online softmax with m, ell and O; recompute
              in the backward pass).
  [FAQ-mcq]   "What does FlashAttention v1 actually change vs standard
              attention?" (zenaique.com, attn-flashattention-family-mcq-hard):
              answer, the online-softmax code figure, the version table.

What is computed. All pages agree that the tiled method returns the result of
the textbook formula Attn(Q,K,V) = softmax(Q K^T / sqrt(d)) V exactly, with
only floating-point rounding differing ([FAQ-short] answer paragraphs 1-2,
[Blog], [FAQ-mcq] answer). So this oracle is that formula written out: it
materialises the full score matrix in float64 and never tiles, fuses or
reorders anything.

Readings where the pages are silent (each also listed in the design notes):
  * scale: passed explicitly (the configurations use 1/sqrt(d)); the float64
    value of the float32 scale argument multiplies Q K^T.
  * causal: key j is visible to query i iff j <= i (lower-triangular mask).
  * logsumexp: lse_i = m_i + ln(l_i) over the *scaled* scores, natural log --
    the pages save the running max m and denominator l for the backward pass
    ([FAQ-short] answer paragraph 2; [FAQ-mcq] answer "tile + save m,l");
    their log-sum is one number per row carrying both.
  * backward: the pages only say that the backward pass recomputes the score
    blocks from Q, K, V and the saved statistics ([FAQ-short] paragraph 2,
    [Card] history paragraph, [Blog]); the gradients themselves are the
    textbook softmax Jacobian of <O, dO>, written out in `backward`.
  * fp8 inputs: the path multiplies E4M3 codes by per-tensor float32 scales;
    the oracle works on the dequantised values code * scale, which float64
    holds exactly.
  * grouped-query heads: [Blog] (lineage paragraph) pairs the method with
    grouped-query attention without defining it. Reading: H query heads and
    Hkv key/value heads, H a multiple of Hkv; query head h uses key/value
    head floor(h / G) with G = H / Hkv (G consecutive query heads per group).
    Hkv = H is ordinary multi-head attention, Hkv = 1 multi-query attention.
  * decode: [Card] (prompts) names the decode step, a few new query rows
    against a long key/value cache. Reading: the Nq query rows are the last
    Nq positions of a sequence of Nk keys, so with the causal mask query row
    i (0-based) sees keys j <= Nk - Nq + i (bottom-right alignment; for
    Nq = Nk this is the ordinary mask).
"""
import math

import numpy as np

__all__ = [
    "scores", "probabilities", "forward", "forward_quantized", "backward",
    "backward_rows", "backward_causal_tail",
    "forward_gqa", "backward_gqa", "forward_decode", "backward_quantized",
    "softmax_by_chunks", "brute_force_forward", "brute_force_backward",
    "decode_e4m3fn", "decode_e5m2",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def scores(q, k, scale, causal, rows=None):
    """Scaled scores S = c * Q K^T for one head, masked.

    q: [Nq, d] (all rows, or the rows listed in `rows`), k: [Nk, d].
    rows: optional 1-D index array; the query positions the rows of `q`
          stand for (needed for the causal mask when only a sample of rows
          is computed). Default: 0..Nq-1.
    Masked entries are -inf. Definition: [FAQ-short] answer paragraph 1
    (the softmax argument Q K^T / sqrt(d_k)); [Card] definition paragraph
    (S = Q K^T / sqrt(d)).
    """
    q = _f64(q)
    k = _f64(k)
    c = float(np.float32(scale))
    s = c * (q @ k.T)
    if causal:
        qi = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
        kj = np.arange(k.shape[0])
        s = np.where(kj[None, :] <= qi[:, None], s, -np.inf)
    return s


def _softmax_rows(s):
    """Row softmax with the max subtracted; returns (P, m, l)."""
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    return e / l, m[:, 0], l[:, 0]


def probabilities(q, k, scale, causal):
    """Full attention matrix P = softmax(S) of one head (rows sum to 1)."""
    p, _, _ = _softmax_rows(scores(q, k, scale, causal))
    return p


def forward(q, k, v, scale, causal, rows=None):
    """O = softmax(c Q K^T) V and lse for tensors laid out [B, H, N, d].

    rows: None for every query row, or an int array [B, H, R] of query
          positions (each row is computed against all keys and masked
          causally by its own position).
    Returns (O [B,H,R,d], lse [B,H,R]) in float64, lse = m + ln(l) with
    m = max_j S_ij and l = sum_j exp(S_ij - m).
    Definition: [FAQ-short] answer paragraph 1, [Card] definition paragraph.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, H, N, d = q.shape
    R = N if rows is None else np.asarray(rows).shape[-1]
    out = np.empty((B, H, R, v.shape[-1]))
    lse = np.empty((B, H, R))
    for b in range(B):
        for h in range(H):
            idx = None if rows is None else np.asarray(rows)[b, h]
            qh = q[b, h] if idx is None else q[b, h][idx]
            p, m, l = _softmax_rows(scores(qh, k[b, h], scale, causal, idx))
            out[b, h] = p @ v[b, h]
            lse[b, h] = m + np.log(l)
    return out, lse


def decode_e4m3fn(codes):
    """Decode OCP FP8 E4M3 ("fn": no infinities) bytes to float64.

    Format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 is subnormal (mantissa * 2^-9); S.1111.111 is NaN;
    largest finite magnitude 448. This is the E4M3 format the pages name for
    the FP8 path ([FAQ-short] answer paragraph 2; [FAQ-mcq] version table).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    mant = c & 0x7
    normal = sign * (1.0 + mant / 8.0) * np.exp2(e - 7.0)
    sub = sign * mant * 2.0 ** -9
    val = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def decode_e5m2(codes):
    """Decode OCP FP8 E5M2 bytes to float64.

    Format: 1 sign bit, 5 exponent bits with bias 15, 2 mantissa bits;
    exponent field 0 is subnormal (mantissa * 2^-16); exponent field 31 is
    infinity (mantissa 0) or NaN; largest finite magnitude 57344. This is
    the E5M2 format the pages name next to E4M3 for the FP8 path
    ([FAQ-short] answer paragraph 2; [FAQ-mcq] version table).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    mant = c & 0x3
    normal = sign * (1.0 + mant / 4.0) * np.exp2(e - 15.0)
    sub = sign * mant * 2.0 ** -16
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 31) & (mant == 0), sign * np.inf, val)
    return np.where((e == 31) & (mant != 0), np.nan, val)


def forward_quantized(qc, kc, vc, sq, sk, sv, scale, causal, rows=None, fmt="e4m3"):
    """Attention of per-tensor-scaled FP8 inputs.

    qc, kc, vc: uint8 codes [B,H,N,d] in the format `fmt` ("e4m3" or
    "e5m2"); sq, sk, sv: the float32 per-tensor scales. The inputs the path
    sees are code * scale, so the oracle is `forward` on exactly those values
    (float64 holds each product exactly: at most 4 significant bits times 24).
    """
    dec = decode_e4m3fn if fmt == "e4m3" else decode_e5m2
    q = dec(qc) * float(np.float32(sq))
    k = dec(kc) * float(np.float32(sk))
    v = dec(vc) * float(np.float32(sv))
    return forward(q, k, v, scale, causal, rows)


def backward(q, k, v, do, scale, causal, heads=None):
    """Gradients of <O, dO> with respect to Q, K, V ([B,H,N,d] tensors).

    The pages state only that the backward pass recomputes P from Q, K, V
    and the saved statistics instead of storing it ([FAQ-short] paragraph 2,
    [Card] history paragraph, [Blog]). The gradient formulas are the
    textbook chain rule through O = P V and the row softmax:
        dV = P^T dO
        dP = dO V^T
        D_i = sum_j P_ij dP_ij
        dS = P * (dP - D)          (softmax Jacobian, row by row)
        dQ = c dS K,  dK = c dS^T Q
    heads: optional list of (b, h) pairs; others are left as NaN.
    Returns (dQ, dK, dV) float64.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    c = float(np.float32(scale))
    B, H, N, d = q.shape
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        p = probabilities(q[b, h], k[b, h], scale, causal)
        dv[b, h] = p.T @ do[b, h]
        dp = do[b, h] @ v[b, h].T
        dd = np.sum(p * dp, axis=1, keepdims=True)
        ds = p * (dp - dd)
        dq[b, h] = c * (ds @ k[b, h])
        dk[b, h] = c * (ds.T @ q[b, h])
    return dq, dk, dv


def backward_rows(q, k, v, do, scale, causal, rows):
    """dQ at the listed query rows only, for sequences too long for `backward`.

    Everything the chain rule needs for dQ_i lives in row i: its softmax row
    P_i (all keys, masked by the row's own position), dP_i = dO_i V^T,
    D_i = sum_j P_ij dP_ij, dS_i = P_i * (dP_i - D_i), and dQ_i = c dS_i K --
    the formulas of `backward` restricted to those rows.
    rows: int array [B, H, R] of query positions. Returns float64 [B, H, R, d].
    """
    c = float(np.float32(scale))
    rows = np.asarray(rows)
    B, H = rows.shape[:2]
    out = np.empty((B, H, rows.shape[-1], q.shape[-1]))
    for b in range(B):
        for h in range(H):
            idx = rows[b, h]
            kh = _f64(k[b, h])
            p_rows, _, _ = _softmax_rows(scores(_f64(q[b, h][idx]), kh, scale, causal, idx))
            dp_rows = _f64(do[b, h][idx]) @ _f64(v[b, h]).T
            d_rows = np.sum(p_rows * dp_rows, axis=1, keepdims=True)
            ds_rows = p_rows * (dp_rows - d_rows)
            out[b, h] = c * (ds_rows @ kh)
    return out


def backward_causal_tail(q, k, v, do, scale, ntail):
    """dK and dV of the last `ntail` keys under the causal mask.

    With the mask, key j receives gradient only from query rows i >= j, so
    the last T keys are reached by the last T rows alone. Those rows' full
    softmax rows (every key they see) give P, dP, D and dS exactly as in
    `backward`; dK and dV of the tail keys are then the tail columns of
    c dS^T Q and P^T dO over those rows.
    Returns (dK, dV) float64 [B, H, T, d] for keys N - T .. N - 1.
    """
    c = float(np.float32(scale))
    B, H, N, _ = q.shape
    t0 = N - ntail
    idx = np.arange(t0, N)
    dk = np.empty((B, H, ntail, k.shape[-1]))
    dv = np.empty((B, H, ntail, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            qt, dot = _f64(q[b, h][t0:]), _f64(do[b, h][t0:])
            p_t, _, _ = _softmax_rows(scores(qt, _f64(k[b, h]), scale, True, idx))
            dp_t = dot @ _f64(v[b, h]).T
            d_t = np.sum(p_t * dp_t, axis=1, keepdims=True)
            ds_t = p_t * (dp_t - d_t)
            dk[b, h] = c * (ds_t[:, t0:].T @ qt)
            dv[b, h] = p_t[:, t0:].T @ dot
    return dk, dv


def _group(q, k):
    H, Hkv = q.shape[1], k.shape[1]
    assert Hkv >= 1 and H % Hkv == 0, "query heads must be a multiple of key/value heads"
    return H // Hkv


def forward_gqa(q, k, v, scale, causal, rows=None):
    """Grouped-query attention: q [B,H,N,d]; k, v [B,Hkv,N,d].

    Query head h attends with key/value head floor(h / G), G = H / Hkv (the
    grouped-query reading in the module notes; [Blog] lineage paragraph).
    Each query head's result is then ordinary attention, so this is
    `forward` with every key/value head repeated for the G query heads of
    its group. Returns (O [B,H,R,d], lse [B,H,R]).
    """
    k = _f64(k)
    v = _f64(v)
    G = _group(q, k)
    return forward(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), scale, causal, rows)


def backward_gqa(q, k, v, do, scale, causal):
    """Gradients of <O, dO> for grouped-query attention.

    A key/value head is an input of the G query heads of its group, so its
    gradient is the sum of the gradients those heads send it (chain rule for
    a shared input); dQ is per query head as in `backward`.
    Returns (dQ [B,H,N,d], dK [B,Hkv,N,d], dV [B,Hkv,N,d]).
    """
    k = _f64(k)
    v = _f64(v)
    G = _group(q, k)
    B, Hkv, N, d = k.shape
    dq, dke, dve = backward(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), do, scale, causal)
    return dq, dke.reshape(B, Hkv, G, N, d).sum(axis=2), dve.reshape(B, Hkv, G, N, d).sum(axis=2)


def forward_decode(q, k, v, scale, causal):
    """Decode step: q [B,H,Nq,d] against a key/value cache k, v [B,Hkv,Nk,d].

    Nq <= Nk new query rows sit at positions Nk - Nq .. Nk - 1 of the
    sequence (the decode reading in the module notes; [Card] prompts), so
    with the causal mask row i sees keys j <= Nk - Nq + i. Key/value heads
    are shared by groups of query heads as in `forward_gqa`. Each row is
    the full softmax over its visible keys.
    Returns (O [B,H,Nq,d], lse [B,H,Nq]).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    G = _group(q, k)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    assert 1 <= Nq <= Nk
    pos = np.arange(Nk - Nq, Nk)
    out = np.empty((B, H, Nq, v.shape[-1]))
    lse = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            p, m, l = _softmax_rows(scores(q[b, h], k[b, h // G], scale, causal, pos))
            out[b, h] = p @ v[b, h // G]
            lse[b, h] = m + np.log(l)
    return out, lse


def backward_quantized(qc, kc, vc, doc, sq, sk, sv, sdo, scale, causal, fmt_in="e4m3", fmt_do="e5m2"):
    """Gradients of <O, dO> for per-tensor-scaled FP8 inputs and gradient.

    qc, kc, vc: uint8 codes [B,H(kv),N,d] in `fmt_in`; doc: uint8 codes of dO
    in `fmt_do` (E5M2, the wider-range FP8 format the pages name next to
    E4M3, for the gradient); sq, sk, sv, sdo: float32 scales. The values are
    code * scale (exact in float64), and the gradients are those of
    `backward_gqa` on exactly those values.
    """
    dec_in = decode_e4m3fn if fmt_in == "e4m3" else decode_e5m2
    dec_do = decode_e4m3fn if fmt_do == "e4m3" else decode_e5m2
    q = dec_in(qc) * float(np.float32(sq))
    k = dec_in(kc) * float(np.float32(sk))
    v = dec_in(vc) * float(np.float32(sv))
    do = dec_do(doc) * float(np.float32(sdo))
    return backward_gqa(q, k, v, do, scale, causal)


def softmax_by_chunks(s_row, v_rows, bounds):
    """Softmax-weighted sum of one score row, assembled chunk by chunk.

    Each chunk of keys bounds[c] .. bounds[c+1]-1 is summarised on its own:
    its largest score M_c, its exponential sum L_c = sum_j exp(s_j - M_c) and
    its weighted values A_c = sum_j exp(s_j - M_c) v_j. Two summaries become
    the summary of their union once both are re-expressed against the larger
    of the two maxima M: L = L_a exp(M_a - M) + L_b exp(M_b - M), and A the
    same way. Folding the chunks in one after the other is the pages' running
    max / running denominator / rescaled output with its exp(m - m_new)
    correction ([Card] definition paragraph; [Blog] explainer paragraph; the
    code figure of [FAQ-mcq] keeps only m and l), and the final A / L is the
    softmax-weighted output ([Card]: normalise by 1/l at the end).
    A chunk whose scores are all -inf has the empty summary (M = -inf,
    L = 0, A = 0) and leaves the others unchanged: the reading that such a
    chunk holds no mass (the figure's exp(m - m_new) would form -inf + inf).

    s_row: [n] scores (may hold -inf for masked keys); v_rows: [n, d];
    bounds: chunk edges 0 = b0 < b1 < ... < bK = n.
    Returns (M, L, A / L) of the whole row.
    """
    s_row = _f64(s_row)
    v_rows = _f64(v_rows)
    width = v_rows.shape[1]

    def summary(lo, hi):
        part = s_row[lo:hi]
        top = float(np.max(part))
        if top == -math.inf:
            return -math.inf, 0.0, np.zeros(width)
        w = np.exp(part - top)
        return top, float(np.sum(w)), w @ v_rows[lo:hi]

    def union(a, b):
        (ma, la, xa), (mb, lb, xb) = a, b
        top = max(ma, mb)
        if top == -math.inf:
            return a
        fa, fb = math.exp(ma - top), math.exp(mb - top)
        return top, la * fa + lb * fb, xa * fa + xb * fb

    total = (-math.inf, 0.0, np.zeros(width))
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        total = union(total, summary(lo, hi))
    m, l, acc = total
    return m, l, acc / l


def _bf_scores(q, k, c, causal):
    n, nk = len(q), len(k)
    s = [[-math.inf] * nk for _ in range(n)]
    for i in range(n):
        for j in range(nk):
            if not causal or j <= i:
                s[i][j] = c * math.fsum(q[i][t] * k[j][t] for t in range(len(q[i])))
    return s


def _bf_softmax(s):
    p = []
    for row in s:
        m = max(row)
        e = [math.exp(x - m) for x in row]
        tot = math.fsum(e)
        p.append([x / tot for x in e])
    return p


def brute_force_forward(q, k, v, scale, causal):
    """Pure-Python single-head forward with math.fsum (tiny N only).

    q, k, v: nested lists / arrays [N, d]. Returns (O, lse) as lists.
    """
    c = float(np.float32(scale))
    q, k, v = [[float(x) for x in r] for r in q], [[float(x) for x in r] for r in k], [[float(x) for x in r] for r in v]
    s = _bf_scores(q, k, c, causal)
    p = _bf_softmax(s)
    o = [[math.fsum(p[i][j] * v[j][t] for j in range(len(v))) for t in range(len(v[0]))] for i in range(len(q))]
    lse = []
    for row in s:
        m = max(row)
        lse.append(m + math.log(math.fsum(math.exp(x - m) for x in row)))
    return o, lse


def brute_force_backward(q, k, v, do, scale, causal):
    """Pure-Python single-head backward with math.fsum (tiny N only).

    Written element by element from the chain rule:
      dV_jt = sum_i P_ij dO_it
      dS_ij = P_ij (sum_t dO_it V_jt - sum_j' P_ij' sum_t dO_it V_j't)
      dQ_it = c sum_j dS_ij K_jt ;  dK_jt = c sum_i dS_ij Q_it
    """
    c = float(np.float32(scale))
    q, k, v, do = ([[float(x) for x in r] for r in t] for t in (q, k, v, do))
    n, nk, d = len(q), len(k), len(q[0])
    p = _bf_softmax(_bf_scores(q, k, c, causal))
    dv = [[math.fsum(p[i][j] * do[i][t] for i in range(n)) for t in range(d)] for j in range(nk)]
    dp = [[math.fsum(do[i][t] * v[j][t] for t in range(d)) for j in range(nk)] for i in range(n)]
    ds = []
    for i in range(n):
        dd = math.fsum(p[i][j] * dp[i][j] for j in range(nk))
        ds.append([p[i][j] * (dp[i][j] - dd) for j in range(nk)])
    dq = [[c * math.fsum(ds[i][j] * k[j][t] for j in range(nk)) for t in range(d)] for i in range(n)]
    dk = [[c * math.fsum(ds[i][j] * q[i][t] for i in range(n)) for t in range(d)] for j in range(nk)]
    return dq, dk, dv
