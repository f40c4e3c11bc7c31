"""Checks that pin the float64 oracle to facts other than itself.

Each pin takes an implementation namespace `o` exposing the oracle's public
functions, so the same checks run against the real oracle (they must pass)
and against copies with planted mistakes (each must fail at least one).
The facts used: a hand-worked example, closed forms, invariants of the
softmax, a library special case (torch's float64 CPU attention and autograd),
finite differences, and pure-Python brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, B, H, N, d, nk=None):
    g = _rng(seed)
    nk = N if nk is None else nk
    return (g.standard_normal((B, H, N, d)), g.standard_normal((B, H, nk, d)),
            g.standard_normal((B, H, nk, d)), g.standard_normal((B, H, N, d)))


def pin_hand_example(o):
    """Hand-derived two-query example (tests/golden/hand_example.json)."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    q, k, v, do = (np.array(g[n])[None, None] for n in ("q", "k", "v", "do"))
    for causal, key in ((False, "noncausal"), (True, "causal")):
        out, lse = o.forward(q, k, v, g["scale"], causal)
        assert np.allclose(out[0, 0], g[key]["o"], atol=1e-12, rtol=0), (key, out)
        assert np.allclose(lse[0, 0], g[key]["lse"], atol=1e-12, rtol=0), (key, lse)
        dq, dk, dv = o.backward(q, k, v, do, g["scale"], causal)
        for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert np.allclose(got[0, 0], g[key][name], atol=1e-12, rtol=0), (key, name, got)


def pin_rows_sum_to_one(o):
    """I1: every row of P sums to 1 (normalisation by 1/l at the end)."""
    for (n, nk, d) in ((7, 7, 3), (33, 33, 16), (64, 64, 64)):
        q, k, _, _ = _qkv(1, 1, 1, n, d, nk)
        for causal in (False, True):
            p = o.probabilities(q[0, 0] * 3.0, k[0, 0], 1.0 / math.sqrt(d), causal)
            assert np.all(p >= 0)
            assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12
            if causal:
                assert np.all(np.triu(p, 1) == 0.0)


def pin_chunked_equals_full(o):
    """I2: the streaming softmax over chunks equals the one-shot softmax.

    The reference result is scipy's softmax (a library routine) times V.
    Chunkings: single elements (the element-wise update), four equal blocks
    (the four-block streaming example), ragged random splits, and rows with
    masked (-inf) entries at the front and back.
    """
    from scipy.special import softmax
    g = _rng(2)
    for n in (1, 2, 5, 16, 37, 64):
        for trial in range(3):
            s = g.standard_normal(n) * (1 + 4 * trial)
            v = g.standard_normal((n, 3))
            if trial == 2 and n > 3:
                s[: n // 4] = -np.inf if n > 8 else s[: n // 4]
                s[-1] = -np.inf
            ref_o = softmax(s) @ v
            finite = s[np.isfinite(s)]
            ref_m = np.max(finite)
            ref_l = np.sum(np.exp(finite - ref_m))
            splits = [list(range(n + 1))]
            if n % 4 == 0:
                splits.append([0, n // 4, n // 2, 3 * n // 4, n])
            cut = sorted(set(g.integers(1, n, size=min(3, max(n - 1, 0))).tolist())) if n > 1 else []
            splits.append([0] + cut + [n])
            splits.append([0, n])
            for b in splits:
                m, l, out = o.softmax_by_chunks(s, v, b)
                assert abs(m - ref_m) <= 1e-12, (n, b)
                assert abs(l - ref_l) <= 1e-12 * max(1.0, ref_l), (n, b, l, ref_l)
                assert np.max(np.abs(out - ref_o)) <= 1e-12, (n, b)


def pin_constant_column(o):
    """I3: a constant value column is reproduced exactly (convex weights)."""
    q, k, v, _ = _qkv(3, 2, 2, 40, 8)
    v[..., 5] = 2.75
    for causal in (False, True):
        out, _ = o.forward(q * 2, k, v, 0.35, causal)
        assert np.max(np.abs(out[..., 5] - 2.75)) <= 1e-12 * 2.75


def pin_uniform_scores(o):
    """I4: equal scores give the mean of V (prefix means when causal), and
    lse = s + ln(#visible keys)."""
    B, H, N, d = 1, 2, 23, 4
    g = _rng(4)
    v = g.standard_normal((B, H, N, d))
    q = np.zeros((B, H, N, d))
    k = g.standard_normal((B, H, N, d))
    out, lse = o.forward(q, k, v, 0.5, False)
    assert np.allclose(out, v.mean(axis=2, keepdims=True), atol=1e-12, rtol=0)
    assert np.allclose(lse, math.log(N), atol=1e-12, rtol=0)
    out, lse = o.forward(q, k, v, 0.5, True)
    prefix = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert np.allclose(out, prefix, atol=1e-12, rtol=0)
    assert np.allclose(lse, np.log(np.arange(1, N + 1))[None, None, :], atol=1e-12, rtol=0)
    # all keys equal: scores in a row are equal but nonzero
    q = g.standard_normal((B, H, N, d))
    k = np.broadcast_to(g.standard_normal((1, 1, 1, d)), (B, H, N, d)).copy()
    c = 0.3
    out, lse = o.forward(q, k, v, c, True)
    s = c * (q[..., :] @ k[0, 0, 0])
    assert np.allclose(out, prefix, atol=1e-12, rtol=0)
    assert np.allclose(lse, float(np.float32(c)) / c * s + np.log(np.arange(1, N + 1)), atol=1e-12, rtol=0)


def pin_brute_force(o):
    """I5: pure-Python fsum brute force agrees, forward and backward."""
    for (n, d, seed) in ((1, 1, 5), (2, 2, 6), (5, 8, 7), (16, 8, 8), (11, 2, 9)):
        q, k, v, do = _qkv(seed, 1, 1, n, d)
        for causal in (False, True):
            c = 1.0 / math.sqrt(d)
            out, lse = o.forward(q, k, v, c, causal)
            bo, bl = o.brute_force_forward(q[0, 0], k[0, 0], v[0, 0], c, causal)
            assert np.max(np.abs(out[0, 0] - np.array(bo))) <= 1e-12
            assert np.max(np.abs(lse[0, 0] - np.array(bl))) <= 1e-12
            dq, dk, dv = o.backward(q, k, v, do, c, causal)
            bq, bk, bv = o.brute_force_backward(q[0, 0], k[0, 0], v[0, 0], do[0, 0], c, causal)
            for a, b in ((dq, bq), (dk, bk), (dv, bv)):
                assert np.max(np.abs(a[0, 0] - np.array(b))) <= 1e-12


def pin_torch_sdpa(o):
    """X1: torch's float64 CPU attention and autograd give the same numbers."""
    import torch
    import torch.nn.functional as F
    for (B, H, N, d, seed) in ((2, 3, 17, 8, 10), (1, 2, 64, 32, 11)):
        q, k, v, do = _qkv(seed, B, H, N, d)
        c = float(np.float32(1.0 / math.sqrt(d)))
        for causal in (False, True):
            tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
            ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=c)
            ref.backward(torch.tensor(do))
            s = c * torch.matmul(tq.detach(), tk.detach().transpose(-1, -2))
            if causal:
                s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
            ref_lse = torch.logsumexp(s, dim=-1).numpy()
            out, lse = o.forward(q, k, v, c, causal)
            assert np.max(np.abs(out - ref.detach().numpy())) <= 1e-12
            assert np.max(np.abs(lse - ref_lse)) <= 1e-12
            dq, dk, dv = o.backward(q, k, v, do, c, causal)
            assert np.max(np.abs(dq - tq.grad.numpy())) <= 1e-10
            assert np.max(np.abs(dk - tk.grad.numpy())) <= 1e-10
            assert np.max(np.abs(dv - tv.grad.numpy())) <= 1e-10


def pin_finite_differences(o):
    """X2: central differences of <O, dO> match the analytic gradients."""
    B, H, N, d = 1, 1, 6, 3
    q, k, v, do = _qkv(12, B, H, N, d)
    c = 0.7
    h = 1e-6
    for causal in (False, True):
        dq, dk, dv = o.backward(q, k, v, do, c, causal)
        for which, grad in ((0, dq), (1, dk), (2, dv)):
            num = np.zeros_like(grad)
            for idx in np.ndindex(grad.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += h
                fp = np.sum(o.forward(*args, c, causal)[0] * do)
                args[which][idx] -= 2 * h
                fm = np.sum(o.forward(*args, c, causal)[0] * do)
                num[idx] = (fp - fm) / (2 * h)
            err = np.max(np.abs(num - grad)) / max(1.0, np.max(np.abs(grad)))
            assert err <= 1e-6, (causal, which, err)


def pin_single_key(o):
    """X3: N = 1 gives O = V and lse = c q.k; causal row 0 likewise."""
    q, k, v, _ = _qkv(13, 2, 2, 1, 5)
    c = 0.25
    for causal in (False, True):
        out, lse = o.forward(q, k, v, c, causal)
        assert np.allclose(out, v, atol=1e-15, rtol=0)
        assert np.allclose(lse[..., 0], c * np.sum(q[..., 0, :] * k[..., 0, :], axis=-1), atol=1e-14, rtol=0)
    q, k, v, _ = _qkv(14, 1, 1, 9, 5)
    out, lse = o.forward(q, k, v, c, True)
    assert np.allclose(out[0, 0, 0], v[0, 0, 0], atol=1e-15, rtol=0)
    assert abs(lse[0, 0, 0] - c * float(q[0, 0, 0] @ k[0, 0, 0])) <= 1e-14


def pin_two_keys(o):
    """X4: with two keys, O = sigmoid(s0-s1) v0 + sigmoid(s1-s0) v1."""
    q, k, v, _ = _qkv(15, 1, 3, 2, 4)
    c = 0.625  # exactly representable in float32, the scale argument's type
    out, _ = o.forward(q, k, v, c, False)
    for h in range(3):
        for i in range(2):
            s0 = c * float(q[0, h, i] @ k[0, h, 0])
            s1 = c * float(q[0, h, i] @ k[0, h, 1])
            sig = 1.0 / (1.0 + math.exp(s1 - s0))
            ref = sig * v[0, h, 0] + (1 - sig) * v[0, h, 1]
            assert np.max(np.abs(out[0, h, i] - ref)) <= 1e-13


def pin_permutations(o):
    """X5: non-causal O is invariant to a joint permutation of (K, V) rows and
    equivariant to a permutation of Q rows."""
    q, k, v, _ = _qkv(16, 1, 2, 19, 6)
    g = _rng(17)
    c = 0.4
    out, lse = o.forward(q, k, v, c, False)
    pk = g.permutation(19)
    out2, lse2 = o.forward(q, k[:, :, pk], v[:, :, pk], c, False)
    assert np.max(np.abs(out - out2)) <= 1e-12 and np.max(np.abs(lse - lse2)) <= 1e-12
    pq = g.permutation(19)
    out3, _ = o.forward(q[:, :, pq], k, v, c, False)
    assert np.max(np.abs(out3 - out[:, :, pq])) <= 1e-12


def pin_backward_invariants(o):
    """X6: sum_j dK_j = 0; sum_j dV_j = sum_i dO_i; equal keys give dQ = 0."""
    q, k, v, do = _qkv(18, 2, 2, 30, 8)
    for causal in (False, True):
        dq, dk, dv = o.backward(q, k, v, do, 0.3, causal)
        assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12
        assert np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) <= 1e-12
    k2 = np.broadcast_to(k[:, :, :1], k.shape).copy()
    dq, _, _ = o.backward(q, k2, v, do, 0.3, False)
    assert np.max(np.abs(dq)) <= 1e-12


def pin_masked_chunk(o):
    """X7: a chunk that is entirely masked leaves (m, l, O) unchanged."""
    g = _rng(19)
    s = g.standard_normal(12)
    v = g.standard_normal((12, 2))
    s_masked = np.concatenate([np.full(4, -np.inf), s, np.full(4, -np.inf)])
    v_masked = np.concatenate([g.standard_normal((4, 2)), v, g.standard_normal((4, 2))])
    m, l, out = o.softmax_by_chunks(s, v, [0, 6, 12])
    m2, l2, out2 = o.softmax_by_chunks(s_masked, v_masked, [0, 4, 10, 16, 20])
    assert m == m2 and abs(l - l2) <= 1e-13 * l and np.max(np.abs(out - out2)) <= 1e-13


def pin_sampled_rows(o):
    """A sample of query rows computed alone equals those rows of the full run."""
    q, k, v, _ = _qkv(20, 1, 2, 50, 8)
    rows = np.array([[[0, 3, 17, 49], [1, 2, 30, 48]]])
    for causal in (False, True):
        full_o, full_l = o.forward(q, k, v, 0.35, causal)
        so, sl = o.forward(q, k, v, 0.35, causal, rows=rows)
        for h in range(2):
            assert np.max(np.abs(so[0, h] - full_o[0, h][rows[0, h]])) <= 1e-13
            assert np.max(np.abs(sl[0, h] - full_l[0, h][rows[0, h]])) <= 1e-13


def pin_e4m3_decode(o):
    """OCP E4M3 ("fn") decoding: fixed points of the format and its range."""
    dec = o.decode_e4m3fn(np.arange(256, dtype=np.uint8))
    assert dec[0x00] == 0.0 and dec[0x38] == 1.0 and dec[0xB8] == -1.0
    assert dec[0x7E] == 448.0 and dec[0xFE] == -448.0
    assert dec[0x01] == 2.0 ** -9 and dec[0x08] == 2.0 ** -6 and dec[0x07] == 7 * 2.0 ** -9
    assert dec[0x40] == 2.0 and dec[0x3C] == 1.5 and dec[0x30] == 0.5
    assert math.isnan(dec[0x7F]) and math.isnan(dec[0xFF])
    pos = dec[:0x7F]
    assert np.all(np.diff(pos) > 0)


def pin_quantized_forward(o):
    """The FP8 entry computes attention of code * scale."""
    g = _rng(21)
    codes = [g.integers(0, 0x7E, size=(1, 1, 9, 4), dtype=np.uint8) | (g.integers(0, 2, size=(1, 1, 9, 4), dtype=np.uint8) << 7) for _ in range(3)]
    sc = (0.01, 0.02, 0.03)
    out, lse = o.forward_quantized(*codes, *sc, 0.5, True)
    # decode one code by hand: 0x38 | 0x05 = 1.625
    assert o.decode_e4m3fn(np.uint8(0x3D)) == 1.625
    vals = [o.decode_e4m3fn(cd) * float(np.float32(s)) for cd, s in zip(codes, sc)]
    ref, ref_lse = o.forward(*vals, 0.5, True)
    assert np.max(np.abs(out - ref)) == 0.0 and np.max(np.abs(lse - ref_lse)) == 0.0


def _gqa_inputs(seed, B, H, Hkv, Nq, Nk, d):
    g = _rng(seed)
    q = g.standard_normal((B, H, Nq, d))
    k = g.standard_normal((B, Hkv, Nk, d))
    v = g.standard_normal((B, Hkv, Nk, d))
    do = g.standard_normal((B, H, Nq, d))
    return q, k, v, do


def pin_gqa_torch(o):
    """Grouped-query heads: torch's float64 CPU attention with enable_gqa and
    its autograd (a library implementation of the same head sharing) agree."""
    import torch
    import torch.nn.functional as F
    for (B, H, Hkv, N, d, seed) in ((2, 6, 2, 19, 8, 30), (1, 4, 1, 33, 16, 31), (1, 4, 4, 12, 8, 32)):
        q, k, v, do = _gqa_inputs(seed, B, H, Hkv, N, N, d)
        c = float(np.float32(1.0 / math.sqrt(d)))
        for causal in (False, True):
            tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
            ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=c, enable_gqa=True)
            ref.backward(torch.tensor(do))
            out, lse = o.forward_gqa(q, k, v, c, causal)
            assert np.max(np.abs(out - ref.detach().numpy())) <= 1e-12
            dq, dk, dv = o.backward_gqa(q, k, v, do, c, causal)
            assert dk.shape == k.shape and dv.shape == v.shape
            assert np.max(np.abs(dq - tq.grad.numpy())) <= 1e-10
            assert np.max(np.abs(dk - tk.grad.numpy())) <= 1e-10
            assert np.max(np.abs(dv - tv.grad.numpy())) <= 1e-10


def pin_gqa_brute_force(o):
    """Grouped-query heads against the pure-Python brute force, head by head:
    query head h uses key/value head h // G; a shared head's gradient is the
    fsum of what each query head of its group sends it."""
    B, H, Hkv, N, d = 1, 6, 2, 7, 3
    G = H // Hkv
    q, k, v, do = _gqa_inputs(33, B, H, Hkv, N, N, d)
    for causal in (False, True):
        c = 0.5
        out, lse = o.forward_gqa(q, k, v, c, causal)
        dq, dk, dv = o.backward_gqa(q, k, v, do, c, causal)
        sk = [[[0.0] * d for _ in range(N)] for _ in range(Hkv)]
        parts_k = [[[[] for _ in range(d)] for _ in range(N)] for _ in range(Hkv)]
        parts_v = [[[[] for _ in range(d)] for _ in range(N)] for _ in range(Hkv)]
        for h in range(H):
            kv = h // G
            bo, bl = o.brute_force_forward(q[0, h], k[0, kv], v[0, kv], c, causal)
            assert np.max(np.abs(out[0, h] - np.array(bo))) <= 1e-12
            assert np.max(np.abs(lse[0, h] - np.array(bl))) <= 1e-12
            bq, bk, bv = o.brute_force_backward(q[0, h], k[0, kv], v[0, kv], do[0, h], c, causal)
            assert np.max(np.abs(dq[0, h] - np.array(bq))) <= 1e-12
            for j in range(N):
                for t in range(d):
                    parts_k[kv][j][t].append(bk[j][t])
                    parts_v[kv][j][t].append(bv[j][t])
        for kv in range(Hkv):
            for j in range(N):
                for t in range(d):
                    assert abs(dk[0, kv, j, t] - math.fsum(parts_k[kv][j][t])) <= 1e-12
                    assert abs(dv[0, kv, j, t] - math.fsum(parts_v[kv][j][t])) <= 1e-12


def pin_gqa_finite_differences(o):
    """Central differences of <O, dO> with respect to a shared K/V head."""
    B, H, Hkv, N, d = 1, 4, 2, 5, 3
    q, k, v, do = _gqa_inputs(34, B, H, Hkv, N, N, d)
    c, h = 0.7, 1e-6
    for causal in (False, True):
        _, dk, dv = o.backward_gqa(q, k, v, do, c, causal)
        f = lambda kk, vv: float(np.sum(o.forward_gqa(q, kk, vv, c, causal)[0] * do))
        for (kv, j, t) in ((0, 0, 0), (1, 3, 2), (0, 4, 1)):
            e = np.zeros_like(k)
            e[0, kv, j, t] = h
            gk = (f(k + e, v) - f(k - e, v)) / (2 * h)
            gv = (f(k, v + e) - f(k, v - e)) / (2 * h)
            assert abs(gk - dk[0, kv, j, t]) <= 1e-6 * max(1.0, abs(gk))
            assert abs(gv - dv[0, kv, j, t]) <= 1e-6 * max(1.0, abs(gv))


def pin_decode_torch(o):
    """Decode rows: torch's float64 CPU attention with an explicit
    bottom-right causal mask (row i sees keys j <= Nk - Nq + i) agrees."""
    import torch
    import torch.nn.functional as F
    for (B, H, Hkv, Nq, Nk, d, seed) in ((2, 4, 2, 1, 37, 8, 35), (1, 8, 1, 5, 64, 16, 36), (1, 2, 2, 9, 9, 4, 37)):
        q, k, v, _ = _gqa_inputs(seed, B, H, Hkv, Nq, Nk, d)
        c = float(np.float32(1.0 / math.sqrt(d)))
        for causal in (False, True):
            tq, tk, tv = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
            mask = None
            if causal:
                mask = torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=Nk - Nq)
            ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=c, enable_gqa=True)
            out, lse = o.forward_decode(q, k, v, c, causal)
            assert np.max(np.abs(out - ref.numpy())) <= 1e-12


def pin_decode_is_tail_of_full(o):
    """Decode rows are the last rows of the full causal forward; one causal
    decode row sees every key (so equals the non-causal row)."""
    B, H, Hkv, N, d = 1, 4, 2, 23, 8
    q, k, v, _ = _gqa_inputs(38, B, H, Hkv, N, N, d)
    c = 0.3
    full, full_lse = o.forward_gqa(q, k, v, c, True)
    for nq in (1, 4, N):
        out, lse = o.forward_decode(q[:, :, N - nq:], k, v, c, True)
        assert np.max(np.abs(out - full[:, :, N - nq:])) <= 1e-12
        assert np.max(np.abs(lse - full_lse[:, :, N - nq:])) <= 1e-12
    a, al = o.forward_decode(q[:, :, N - 1:], k, v, c, True)
    b, bl = o.forward_decode(q[:, :, N - 1:], k, v, c, False)
    assert np.max(np.abs(a - b)) == 0.0 and np.max(np.abs(al - bl)) == 0.0


def pin_e5m2_decode(o):
    """OCP E5M2 decoding: fixed points of the format, and torch's own
    float8_e5m2 conversion (a library implementation) on all 256 codes."""
    import torch
    dec = o.decode_e5m2(np.arange(256, dtype=np.uint8))
    assert dec[0x00] == 0.0 and dec[0x3C] == 1.0 and dec[0xBC] == -1.0
    assert dec[0x7B] == 57344.0 and dec[0x01] == 2.0 ** -16 and dec[0x04] == 2.0 ** -14
    assert dec[0x3D] == 1.25 and dec[0x40] == 2.0 and dec[0x38] == 0.5
    assert dec[0x7C] == np.inf and dec[0xFC] == -np.inf and math.isnan(dec[0x7D]) and math.isnan(dec[0xFF])
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    both_nan = np.isnan(dec) & np.isnan(ref)
    assert np.all(both_nan | (dec == ref))


def pin_quantized_forward_e5m2(o):
    """The E5M2 entry computes attention of code * scale."""
    g = _rng(22)
    codes = [g.integers(0, 0x7B, size=(1, 1, 9, 4), dtype=np.uint8) | (g.integers(0, 2, size=(1, 1, 9, 4), dtype=np.uint8) << 7) for _ in range(3)]
    sc = (0.001, 0.002, 0.003)
    out, lse = o.forward_quantized(*codes, *sc, 0.5, True, fmt="e5m2")
    assert o.decode_e5m2(np.uint8(0x3E)) == 1.5
    vals = [o.decode_e5m2(cd) * float(np.float32(s)) for cd, s in zip(codes, sc)]
    ref, ref_lse = o.forward(*vals, 0.5, True)
    assert np.max(np.abs(out - ref)) == 0.0 and np.max(np.abs(lse - ref_lse)) == 0.0


def pin_quantized_backward(o):
    """The FP8 backward entry is the backward of code * scale (E4M3 inputs,
    E5M2 gradient), including shared key/value heads."""
    g = _rng(23)
    rnd = lambda shape, top: g.integers(0, top, size=shape, dtype=np.uint8) | (g.integers(0, 2, size=shape, dtype=np.uint8) << 7)
    qc, kc, vc = rnd((1, 4, 7, 4), 0x7E), rnd((1, 2, 7, 4), 0x7E), rnd((1, 2, 7, 4), 0x7E)
    doc = rnd((1, 4, 7, 4), 0x7B)
    sc = (0.01, 0.02, 0.03, 0.0004)
    got = o.backward_quantized(qc, kc, vc, doc, *sc, 0.5, True)
    q = o.decode_e4m3fn(qc) * float(np.float32(sc[0]))
    k = o.decode_e4m3fn(kc) * float(np.float32(sc[1]))
    v = o.decode_e4m3fn(vc) * float(np.float32(sc[2]))
    do = o.decode_e5m2(doc) * float(np.float32(sc[3]))
    ref = o.backward_gqa(q, k, v, do, 0.5, True)
    for a, b in zip(got, ref):
        assert np.max(np.abs(a - b)) == 0.0
    assert o.decode_e5m2(np.uint8(0x3F)) == 1.75


def _torch_grads(q, k, v, do, c, causal):
    """torch's float64 CPU attention and autograd: (dQ, dK, dV) as numpy."""
    import torch
    import torch.nn.functional as F
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=c).backward(torch.tensor(do))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_backward_rows_torch(o):
    """X8: dQ at chosen rows equals those rows of torch's autograd dQ (rows
    out of order and with gaps, so a mask built from 0..R-1 would fail)."""
    B, H, N, d, seed = 1, 2, 37, 16, 40
    q, k, v, do = _qkv(seed, B, H, N, d)
    c = float(np.float32(1.0 / math.sqrt(d)))
    rows = np.array([[[36, 0, 17, 5, 30]], [[1, 2, 35, 20, 9]]]).reshape(B, H, 5)
    for causal in (False, True):
        ref = _torch_grads(q, k, v, do, c, causal)[0]
        got = o.backward_rows(q, k, v, do, c, causal, rows)
        for h in range(H):
            assert np.max(np.abs(got[0, h] - ref[0, h][rows[0, h]])) <= 1e-10, (causal, h)


def pin_causal_tail_torch(o):
    """X9: dK, dV of the last T keys under the causal mask equal the last T
    rows of torch's autograd dK, dV (T = 1, a few, and all keys)."""
    B, H, N, d, seed = 2, 1, 29, 8, 41
    q, k, v, do = _qkv(seed, B, H, N, d)
    c = float(np.float32(1.0 / math.sqrt(d)))
    _, rk, rv = _torch_grads(q, k, v, do, c, True)
    for t in (1, 6, N):
        dk, dv = o.backward_causal_tail(q, k, v, do, c, t)
        assert np.max(np.abs(dk - rk[:, :, N - t:])) <= 1e-10, t
        assert np.max(np.abs(dv - rv[:, :, N - t:])) <= 1e-10, t


ALL_PINS = [
    pin_hand_example, pin_rows_sum_to_one, pin_chunked_equals_full, pin_constant_column,
    pin_uniform_scores, pin_brute_force, pin_torch_sdpa, pin_finite_differences,
    pin_single_key, pin_two_keys, pin_permutations, pin_backward_invariants,
    pin_masked_chunk, pin_sampled_rows, pin_e4m3_decode, pin_quantized_forward,
    pin_gqa_torch, pin_gqa_brute_force, pin_gqa_finite_differences, pin_decode_torch,
    pin_decode_is_tail_of_full, pin_e5m2_decode, pin_quantized_forward_e5m2, pin_quantized_backward,
    pin_backward_rows_torch, pin_causal_tail_torch,
]
