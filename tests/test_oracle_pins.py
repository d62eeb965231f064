"""Pins: check the oracle against things other than itself.

Each test fixes part of the oracle by a closed form, an invariant, brute force
on a tiny input, a hand-worked example, or an independent library routine
(``scipy`` cosine distance, ``torch`` scaled-dot-product attention, ``heapq``,
complex-number rotation). ``test_oracle_mutations.py`` plants plausible
mistakes in the oracle and checks that these pins catch each one.

Sources cited: the MSA pages — [techblg] portal.techblg.uk IRMaD reading
(section M), [rainbus] paper.rainbus.top (method steps), [chooseai]
chooseai.io (sections 2.1–2.4), [zhichai] zhichai.net (关键技术细节).
"""
import cmath
import heapq
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20260323)


def bf16_randn(shape, std=1.0, rng=None):
    rng = RNG if rng is None else rng
    x = torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_of(values):
    """bf16 patterns of values that are exactly representable (asserted)."""
    v = np.asarray(values, dtype=np.float32)
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    assert np.all((v.view(np.uint32) & 0xFFFF) == 0)
    return bits


# ---------------------------------------------------------------------------
# constants printed by the pages
# ---------------------------------------------------------------------------
def test_constants_match_pages():
    c = json.load(open(os.path.join(GOLDEN, "paper_constants.json")))
    assert O.CHUNK == c["chunk_P"]["value"]
    assert O.TOP_K == c["top_k"]["value"]
    assert O.N_KV_HEADS == c["heads"]["value"] == O.N_ROUTER_HEADS
    assert O.HEAD_DIM == c["head_dim"]["value"]
    assert O.N_ROUTED_LAYERS == c["routed_layers"]["value"]


def test_footprint_within_3pct_of_pages():
    # [techblg] §M Memory Parallel bullet: ≈56 GB of router keys, ≈169 GB total.
    c = json.load(open(os.path.join(GOLDEN, "paper_constants.json")))
    one = O.store_bytes(c["memory_tokens"]["value"])
    assert one == 1_562_500 * 8 * 128 * 2 * 18 == 57_600_000_000
    assert abs(one / 1e9 - c["footprint_router_keys_GB"]["value"]) / 56 < 0.03
    assert abs(3 * one / 1e9 - c["footprint_all_GB"]["value"]) / 169 < 0.03


# ---------------------------------------------------------------------------
# bf16 coding
# ---------------------------------------------------------------------------
def test_bf16_decode_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x0000, 0x3E00, 0x0001, 0x7F80, 0x4049], np.uint16)
    exp = [1.0, -2.0, 0.0, 0.125, 2.0 ** -133, math.inf, 3.140625]
    assert list(O.bf16_to_f64(pats)) == exp


def test_bf16_encode_hand_ties():
    # 1+2^-8 lies halfway between 1 (0x3F80, even) and 1+2^-7 (0x3F81): even wins.
    # 1+3·2^-8 lies halfway between 0x3F81 and 0x3F82 (even): rounds up.
    # Just above a tie rounds away; just below rounds back.
    x = [1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30, 1 + 2 ** -8 - 2 ** -30, -1 - 2 ** -8]
    assert list(O.f64_to_bf16(x)) == [0x3F80, 0x3F82, 0x3F81, 0x3F80, 0xBF80]


def test_bf16_roundtrip_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vals = O.bf16_to_f64(bits)
    ok = ~np.isnan(vals)
    assert np.array_equal(O.f64_to_bf16(vals[ok]), bits[ok])


def test_bf16_ord_is_the_rank_of_the_value():
    """bf16_ord, which the 1-ulp pooled criterion counts in, orders all
    non-NaN patterns by value, ±0 share code 0, and neighbouring values differ
    by exactly one code (so a code distance is a count of representable
    values)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vals = O.bf16_to_f64(bits)
    ok = ~np.isnan(vals)
    b, v = bits[ok], vals[ok]
    code = O.bf16_ord(b).astype(np.int64)
    order = np.argsort(v, kind="stable")
    vs, cs = v[order], code[order]
    step = np.diff(cs)
    rises = np.diff(vs) > 0
    assert np.array_equal(step[rises], np.ones(int(rises.sum()), np.int64))
    assert np.array_equal(step[~rises], np.zeros(int((~rises).sum()), np.int64))
    assert int(O.bf16_ord(np.uint16(0x0000))) == 0 == int(O.bf16_ord(np.uint16(0x8000)))
    assert np.array_equal(np.sign(code), np.sign(v).astype(np.int64))
    # hand values: 1.0 and the next bf16 above it; -1.0 and the next below it
    assert int(O.bf16_ord(np.uint16(0x3F81)) - O.bf16_ord(np.uint16(0x3F80))) == 1
    assert int(O.bf16_ord(np.uint16(0xBF80)) - O.bf16_ord(np.uint16(0xBF81))) == 1
    assert int(O.bf16_ord(np.uint16(0x0001)) - O.bf16_ord(np.uint16(0x8001))) == 2


def test_bf16_encode_matches_torch_on_float32():
    # torch rounds float32 -> bf16 to nearest-even in one step (library routine).
    x = (RNG.standard_normal(200_000) * np.exp(RNG.uniform(-30, 30, 200_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_bf16(x.astype(np.float64)), ref)


# ---------------------------------------------------------------------------
# chunk plan ([chooseai] §2.1: each document cut into fixed-length chunks)
# ---------------------------------------------------------------------------
def test_plan_chunks_hand():
    offs = np.cumsum([0, 1, 64, 65, 128, 129, 512])
    assert list(O.plan_chunks(offs)) == [0, 1, 2, 4, 6, 9, 17]


def test_plan_chunks_rejects_empty_doc():
    with pytest.raises(ValueError):
        O.plan_chunks([0, 5, 5, 9])


# ---------------------------------------------------------------------------
# RoPE ([techblg] §M positional bullet; [zhichai] 关键技术细节 1)
# ---------------------------------------------------------------------------
def test_rope_hand_worked_D4():
    # D=4, θ=1e4: ω=(1, 0.01); pairs (x0,x2), (x1,x3); position t=1.
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    y = O.rope_rotate(x, np.array([1]), theta=1e4)[0, 0]
    c1, s1, c2, s2 = math.cos(1), math.sin(1), math.cos(0.01), math.sin(0.01)
    exp = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    assert np.allclose(y, exp, rtol=0, atol=1e-15)


def test_rope_equals_complex_multiplication():
    # Independent form: z_m = x_m + i·x_{m+64} turns into z_m·e^{i·t·ω_m}.
    x = RNG.standard_normal((5, 3, 128))
    pos = np.array([0, 1, 7, 1000, 8191])
    y = O.rope_rotate(x, pos, 1e6)
    for n in range(5):
        for m in range(64):
            w = 1e6 ** (-m / 64.0)
            z = complex(x[n, 1, m], x[n, 1, m + 64]) * cmath.exp(1j * pos[n] * w)
            assert abs(y[n, 1, m] - z.real) < 1e-9 and abs(y[n, 1, m + 64] - z.imag) < 1e-9


def test_rope_identity_norm_and_relative():
    x = RNG.standard_normal((4, 2, 128))
    assert np.array_equal(O.rope_rotate(x, np.zeros(4)), x)
    y = O.rope_rotate(x, np.array([3, 50, 700, 4000]))
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-12)
    q, k = RNG.standard_normal((1, 1, 128)), RNG.standard_normal((1, 1, 128))
    d1 = (O.rope_rotate(q, [37]) * O.rope_rotate(k, [5])).sum()
    d2 = (O.rope_rotate(q, [37 + 911]) * O.rope_rotate(k, [5 + 911])).sum()
    assert abs(d1 - d2) < 1e-10
    ab = O.rope_rotate(O.rope_rotate(x, np.full(4, 11)), np.full(4, 31))
    assert np.allclose(ab, O.rope_rotate(x, np.full(4, 42)), atol=1e-12)


# ---------------------------------------------------------------------------
# pooling with document RoPE ([techblg] §M routing bullet K̄=φ(K) etc.;
# [techblg] §M positional bullet: positions restart at 0 in each document)
# ---------------------------------------------------------------------------
def _constant_doc(lengths, vec_k, vec_v, vec_r):
    T = int(sum(lengths))
    K = np.tile(bf16_of(vec_k)[None, None, :], (T, 1, 1))
    V = np.tile(bf16_of(vec_v)[None, None, :], (T, 1, 1))
    R = np.tile(bf16_of(vec_r)[None, None, :], (T, 1, 1))
    return K, V, R, np.concatenate([[0], np.cumsum(lengths)])


def test_pool_constant_input_closed_form():
    # V and K^R constant -> the mean is the constant. K rotated per position:
    # mean_{t=a}^{b-1} e^{itω} = e^{iaω}(1 − e^{inω}) / (n(1 − e^{iω})).
    Dh = 8
    vk = np.array([1, 0, 0, 0, 0.5, 0, 0, 0], np.float32)
    vv = np.array([0.25, -3, 7, 1, 0, 2, 0.5, 1], np.float32)
    K, V, R, offs = _constant_doc([150, 64], vk, vv, vv)
    Kb, Vb, Rb, dco = O.pool(K, V, R, offs, chunk=64, theta=100.0)
    assert list(dco) == [0, 3, 4]
    assert np.all(Vb == bf16_of(vv)) and np.all(Rb == bf16_of(vv))
    chunks = [(0, 64), (64, 128), (128, 150), (0, 64)]   # doc-local ranges
    for row, (a, b) in enumerate(chunks):
        n = b - a
        for m in range(Dh // 2):
            w = 100.0 ** (-2.0 * m / Dh)
            z0 = complex(vk[m], vk[m + Dh // 2])
            mean = cmath.exp(1j * a * w) * (1 - cmath.exp(1j * n * w)) / (n * (1 - cmath.exp(1j * w)))
            z = z0 * mean
            exp = O.bf16_to_f64(O.f64_to_bf16(np.array([z.real, z.imag])))
            got = O.bf16_to_f64(Kb[row, 0, [m, m + Dh // 2]])
            assert got[0] == exp[0] and got[1] == exp[1]     # values (±0 alike)


def test_pool_ramp_and_partial_chunk():
    # V_t = global token index (exact in bf16 below 256): chunk mean is
    # start + (n-1)/2; the one-token tail chunk returns its token exactly.
    lengths = [65, 100]
    T = sum(lengths)
    V = np.tile(bf16_of(np.arange(T, dtype=np.float32))[:, None, None], (1, 2, 4))
    K = np.zeros_like(V)
    Kb, Vb, Rb, dco = O.pool(K, V, V, np.array([0, 65, 165]), chunk=64)
    # chunk means: 0..63 -> 31.5; 64 -> 64; 65..128 -> 96.5; 129..164 -> 146.5,
    # which is a bf16 tie between 146 (even) and 147 -> 146.
    got = O.bf16_to_f64(Vb[:, 0, 0])
    assert list(got) == [31.5, 64.0, 96.5, 146.0]
    assert list(dco) == [0, 2, 4]
    assert got[1] == 64.0


def test_pool_document_position_reset():
    # The same raw document placed first or after another gives identical K̄.
    rng = np.random.default_rng(5)
    doc = bf16_randn((130, 2, 128), rng=rng)
    other = bf16_randn((77, 2, 128), rng=rng)
    K1 = doc
    K2 = np.concatenate([other, doc])
    a = O.pool(K1, K1, K1, np.array([0, 130]))[0]
    b = O.pool(K2, K2, K2, np.array([0, 77, 207]))[0]
    assert np.array_equal(a, b[2:])
    # t = 0 is unrotated: a one-token doc pools to itself
    c = O.pool(doc[:1], doc[:1], doc[:1], np.array([0, 1]))[0]
    assert np.array_equal(c[0], doc[0])


def test_pool_chunk_rope_mode():
    # CHUNK mode: the mean of K is rotated at the chunk index c (closed form
    # with a constant input: R(c)·x), and differs from TOKEN mode.
    vk = np.array([1, 0.5, -2, 0.25, 0.75, 1, 0, 3], np.float32)
    K, V, R, offs = _constant_doc([200], vk, vk, vk)
    kc = O.pool(K, V, R, offs, chunk=64, theta=50.0, doc_rope_mode=O.DOC_ROPE_CHUNK)[0]
    kt = O.pool(K, V, R, offs, chunk=64, theta=50.0, doc_rope_mode=O.DOC_ROPE_TOKEN)[0]
    for c in range(4):
        for m in range(4):
            z = complex(vk[m], vk[m + 4]) * cmath.exp(1j * c * 50.0 ** (-2.0 * m / 8))
            exp = O.f64_to_bf16(np.array([z.real, z.imag]))
            assert kc[c, 0, m] == exp[0] and kc[c, 0, m + 4] == exp[1]
    assert not np.array_equal(kc, kt)


def test_pool_brute_force_tiny():
    # Pure-Python loops (complex rotation, running sums) on a 2-head, D=4 case.
    rng = np.random.default_rng(9)
    lengths = [5, 1, 9]
    T = sum(lengths)
    K, V, R = (bf16_randn((T, 2, 4), rng=rng) for _ in range(3))
    offs = [0, 5, 6, 15]
    Kb, Vb, Rb, dco = O.pool(K, V, R, np.array(offs), chunk=4, theta=10.0)
    row = 0
    for d in range(3):
        n = offs[d + 1] - offs[d]
        for c in range((n + 3) // 4):
            toks = list(range(c * 4, min(c * 4 + 4, n)))
            for h in range(2):
                for m in range(2):
                    acc_k = 0j
                    acc_v = [0.0, 0.0]
                    acc_r = [0.0, 0.0]
                    for t in toks:
                        g = offs[d] + t
                        kk = complex(float(O.bf16_to_f64(K[g, h, m])), float(O.bf16_to_f64(K[g, h, m + 2])))
                        acc_k += kk * cmath.exp(1j * t * 10.0 ** (-2.0 * m / 4))
                        for j, mm in enumerate((m, m + 2)):
                            acc_v[j] += float(O.bf16_to_f64(V[g, h, mm]))
                            acc_r[j] += float(O.bf16_to_f64(R[g, h, mm]))
                    L = len(toks)
                    ek = O.f64_to_bf16(np.array([acc_k.real / L, acc_k.imag / L]))
                    assert Kb[row, h, m] == ek[0] and Kb[row, h, m + 2] == ek[1]
                    for j, mm in enumerate((m, m + 2)):
                        assert Vb[row, h, mm] == O.f64_to_bf16(np.array([acc_v[j] / L]))[0]
                        assert Rb[row, h, mm] == O.f64_to_bf16(np.array([acc_r[j] / L]))[0]
            row += 1
    assert row == dco[-1] == 2 + 1 + 3


# ---------------------------------------------------------------------------
# routing score ([techblg] §M routing bullet: max_t mean_h cos)
# ---------------------------------------------------------------------------
def test_route_hand_worked():
    # 2 heads, D=2: cos(q0,k0) = (1·1+0·1)/√2, cos(q1,k1) = 2/2 → mean.
    q = bf16_of([[[1, 0], [0, 1]]])
    k = bf16_of([[[1, 1], [0, 2]]])
    s = O.token_chunk_scores(q.reshape(1, 2, 2), k.reshape(1, 2, 2))
    assert abs(s[0, 0] - (1 / math.sqrt(2) + 1) / 2) < 1e-15


def test_route_special_cases():
    k = bf16_randn((3, 8, 128))
    kf = O.bf16_to_f64(k)
    same = O.token_chunk_scores(k[:1], k)
    assert abs(same[0, 0] - 1) < 1e-12
    neg = O.token_chunk_scores(O.f64_to_bf16(-kf[:1]), k)
    assert abs(neg[0, 0] + 1) < 1e-12
    q = bf16_randn((4, 8, 128))
    s1 = O.token_chunk_scores(q, k)
    s2 = O.token_chunk_scores(O.f64_to_bf16(O.bf16_to_f64(q) * 4.0), O.f64_to_bf16(kf * 0.25))
    assert np.allclose(s1, s2, atol=1e-14) and np.all(np.abs(s1) <= 1 + 1e-12)
    # one aligned head, seven orthogonal heads -> 1/8
    q1 = np.zeros((1, 8, 128))
    k1 = np.zeros((1, 8, 128))
    q1[0, :, 0] = 1.0
    k1[0, 0, 0] = 2.0
    k1[0, 1:, 1] = 1.0
    assert abs(O.token_chunk_scores(O.f64_to_bf16(q1), O.f64_to_bf16(k1))[0, 0] - 1 / 8) < 1e-15
    # an all-zero key scores 0 (the norm clamp), not NaN
    assert O.token_chunk_scores(q[:1], np.zeros((1, 8, 128), np.uint16))[0, 0] == 0.0


def test_route_matches_scipy_cosine():
    from scipy.spatial.distance import cosine
    q = bf16_randn((3, 8, 128))
    k = bf16_randn((5, 8, 128), std=0.125)
    S = O.token_chunk_scores(q, k)
    qf, kf = O.bf16_to_f64(q), O.bf16_to_f64(k)
    for t in range(3):
        for c in range(5):
            ref = np.mean([1.0 - cosine(qf[t, h], kf[c, h]) for h in range(8)])
            assert abs(S[t, c] - ref) < 1e-12
    assert np.allclose(O.chunk_scores(q, k, O.TOKEN_REDUCE_MAX), S.max(axis=0), atol=0)
    assert np.allclose(O.chunk_scores(q, k, O.TOKEN_REDUCE_MEAN), S.mean(axis=0), atol=1e-15)


# ---------------------------------------------------------------------------
# doc reduce and top-k ([techblg] §M routing bullet: s_i = max_j S_ij, Top-k)
# ---------------------------------------------------------------------------
def test_route_topk_brute_force():
    rng = np.random.default_rng(11)
    counts = rng.integers(1, 5, size=40)
    dco = np.concatenate([[0], np.cumsum(counts)])
    C = int(dco[-1])
    k = bf16_randn((C, 2, 4), rng=rng)
    q = bf16_randn((3, 2, 4), rng=rng)
    s, ids, sc, mg = O.route_topk(q, k, dco, k=7)
    qf, kf = O.bf16_to_f64(q), O.bf16_to_f64(k)
    brute = []
    for i in range(40):
        best = -math.inf
        for c in range(dco[i], dco[i + 1]):
            for t in range(3):
                acc = 0.0
                for h in range(2):
                    dot = sum(qf[t, h, j] * kf[c, h, j] for j in range(4))
                    nq = math.sqrt(sum(qf[t, h, j] ** 2 for j in range(4)))
                    nk = math.sqrt(sum(kf[c, h, j] ** 2 for j in range(4)))
                    acc += dot / (nq * nk)
                best = max(best, acc / 2)
        brute.append(best)
    assert np.allclose(s, brute, atol=1e-12)
    top = heapq.nlargest(7, range(40), key=lambda i: (brute[i], -i))
    assert list(ids) == top
    assert np.allclose(mg[:-1], sc[:-1] - sc[1:], atol=0)


def test_topk_ties_small_n_nan():
    ids, sc, mg = O.topk(np.array([0.5, 0.9, 0.9, 0.1, 0.7]), 3)
    assert list(ids) == [1, 2, 4] and list(mg) == [0.0, pytest.approx(0.2), pytest.approx(0.2)]
    ids, sc, mg = O.topk(np.array([0.2, 0.3]), 16)
    assert list(ids) == [1, 0] and mg[-1] == math.inf
    ids, _, _ = O.topk(np.array([np.nan, -5.0, 1.0]), 3)
    assert list(ids) == [2, 1, 0]


def test_duplicate_documents_tie_to_lowest_id():
    k = bf16_randn((6, 8, 128))
    k[3:6] = k[0:3]                         # doc 1 is a byte copy of doc 0
    dco = np.array([0, 3, 6])
    q = bf16_randn((2, 8, 128))
    s, ids, _, mg = O.route_topk(q, k, dco, k=1)
    assert s[0] == s[1] and list(ids) == [0] and mg[0] == 0.0


def test_planted_recall_cfg1():
    import synth
    mem, q, _ = synth.cfg1_tiny("cpu")
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    Kb, Vb, Rb, dco = O.pool(u16(mem.K), u16(mem.V), u16(mem.KR), mem.doc_token_offsets)
    s, ids, sc, mg = O.route_topk(u16(q.QR[0]), Rb, dco)
    assert len(ids) == 16
    assert set(ids[:4]) == set(mem.planted.keys())
    assert mg[3] > 0.1                      # planted docs stand well clear


# ---------------------------------------------------------------------------
# sparse attention ([techblg] §M routing bullet: Output = Attention(Q, K_ctx, V_ctx);
# §M positional bullet: global RoPE offset from k)
# ---------------------------------------------------------------------------
def _dense_reference(Q, K_loc, V_loc, Kbar, Vbar, pos0, theta=O.ROPE_THETA, k_rotated=False):
    """Independent dense attention: every pooled chunk in document order plus
    the causal local context, via torch SDPA (fp64, CPU, boolean mask) and a
    complex-number rotary embedding."""
    def rot(x, pos):
        x = torch.from_numpy(x)
        half = x.shape[-1] // 2
        w = theta ** (-torch.arange(half, dtype=torch.float64) / half)
        z = torch.complex(x[..., :half], x[..., half:])
        z = z * torch.exp(1j * torch.as_tensor(pos, dtype=torch.float64)[:, None, None] * w)
        return torch.cat([z.real, z.imag], dim=-1)
    M, Hq, Dh = Q.shape
    M_loc, Hkv, _ = K_loc.shape
    q = rot(O.bf16_to_f64(Q), pos0 + np.arange(M_loc - M, M_loc))
    kl = torch.from_numpy(O.bf16_to_f64(K_loc)) if k_rotated else \
        rot(O.bf16_to_f64(K_loc), pos0 + np.arange(M_loc))
    keys = torch.cat([torch.from_numpy(O.bf16_to_f64(Kbar)), kl], 0)
    vals = torch.cat([torch.from_numpy(O.bf16_to_f64(Vbar)), torch.from_numpy(O.bf16_to_f64(V_loc))], 0)
    C = Kbar.shape[0]
    mask = torch.ones((M, C + M_loc), dtype=torch.bool)
    for u in range(M):
        mask[u, C + (M_loc - M + u) + 1:] = False
    g = Hq // Hkv
    kk = keys.permute(1, 0, 2).repeat_interleave(g, 0)        # [Hq, S, D]
    vv = vals.permute(1, 0, 2).repeat_interleave(g, 0)
    out = torch.nn.functional.scaled_dot_product_attention(
        q.permute(1, 0, 2), kk, vv, attn_mask=mask)
    return out.permute(1, 0, 2).numpy()


def test_attend_all_docs_equals_dense():
    rng = np.random.default_rng(21)
    counts = [3, 1, 5, 2]
    dco = np.concatenate([[0], np.cumsum(counts)])
    C = int(dco[-1])
    Kb, Vb = bf16_randn((C, 8, 128), 0.3, rng), bf16_randn((C, 8, 128), 0.3, rng)
    Q, Kl, Vl = bf16_randn((3, 32, 128), rng=rng), bf16_randn((5, 8, 128), rng=rng), bf16_randn((5, 8, 128), rng=rng)
    sel = [2, 0, 3, 1]                       # k >= N: every document, rank order
    out = O.sparse_attend(Q, Kl, Vl, Kb, Vb, dco, sel)
    ref = _dense_reference(Q, Kl, Vl, Kb, Vb, pos0=4)
    assert np.allclose(out, ref, atol=1e-10, rtol=1e-10)
    # order of the selected documents does not matter
    out2 = O.sparse_attend(Q, Kl, Vl, Kb, Vb, dco, [0, 1, 2, 3])
    assert np.allclose(out, out2, atol=1e-12)


def test_attend_prerotated_local_keys():
    # k_loc_rotated: keys the caller already turned are used as given.
    rng = np.random.default_rng(24)
    dco = np.array([0, 2, 3])
    Kb, Vb = bf16_randn((3, 8, 128), 0.3, rng), bf16_randn((3, 8, 128), 0.3, rng)
    Q, Kl, Vl = bf16_randn((2, 32, 128), rng=rng), bf16_randn((4, 8, 128), rng=rng), bf16_randn((4, 8, 128), rng=rng)
    out = O.sparse_attend(Q, Kl, Vl, Kb, Vb, dco, [1, 0], k_loc_rotated=True)
    ref = _dense_reference(Q, Kl, Vl, Kb, Vb, pos0=2, k_rotated=True)
    assert np.allclose(out, ref, atol=1e-10, rtol=1e-10)


def test_attend_special_cases():
    rng = np.random.default_rng(22)
    Q = bf16_randn((1, 32, 128), rng=rng)
    Kl, Vl = bf16_randn((1, 8, 128), rng=rng), bf16_randn((1, 8, 128), rng=rng)
    empty = np.zeros((0, 8, 128), np.uint16)
    out = O.sparse_attend(Q, Kl, Vl, empty, empty, np.array([0]), [])
    assert np.array_equal(out, np.repeat(O.bf16_to_f64(Vl), 4, axis=1))  # one visible key
    # identical memory keys and no local competition beyond them -> mean of V
    Vb = bf16_randn((4, 8, 128), rng=rng)
    Kl0 = np.zeros((1, 8, 128), np.uint16)   # zero keys everywhere: all logits 0
    Kb0 = np.zeros((4, 8, 128), np.uint16)
    out = O.sparse_attend(Q, Kl0, Vl, Kb0, Vb, np.array([0, 4]), [0])
    exp = (O.bf16_to_f64(Vb).sum(0) + O.bf16_to_f64(Vl)[0]) / 5
    assert np.allclose(out[0], np.repeat(exp, 4, axis=0), atol=1e-14)
    # GQA: q head h reads kv head h // 4
    Vg = np.stack([O.f64_to_bf16(np.full((8, 128), 0.0) + np.arange(8)[:, None])])
    out = O.sparse_attend(Q, Kl, Vg, empty, empty, np.array([0]), [])
    assert np.array_equal(out[0, :, 0], np.arange(32) // 4)


def test_attend_causal_and_pos0():
    rng = np.random.default_rng(23)
    Q = bf16_randn((4, 32, 128), rng=rng)
    Kl, Vl = bf16_randn((6, 8, 128), rng=rng), bf16_randn((6, 8, 128), rng=rng)
    empty = np.zeros((0, 8, 128), np.uint16)
    a = O.sparse_attend(Q, Kl, Vl, empty, empty, np.array([0]), [], pos0=0)
    # without memory, only relative positions matter: pos0 shifts nothing
    b = O.sparse_attend(Q, Kl, Vl, empty, empty, np.array([0]), [], pos0=1234)
    assert np.allclose(a, b, atol=1e-10)
    # a change to the last local token leaves the earlier queries unchanged
    Kl2, Vl2 = Kl.copy(), Vl.copy()
    Kl2[-1] = bf16_randn((8, 128), rng=rng)
    Vl2[-1] = bf16_randn((8, 128), rng=rng)
    c = O.sparse_attend(Q, Kl2, Vl2, empty, empty, np.array([0]), [], pos0=0)
    assert np.allclose(a[:3], c[:3], atol=0) and not np.allclose(a[3], c[3])
    # with memory present, pos0 matters (memory keys carry no global RoPE)
    Kb, Vb = bf16_randn((2, 8, 128), rng=rng), bf16_randn((2, 8, 128), rng=rng)
    d0 = O.sparse_attend(Q, Kl, Vl, Kb, Vb, np.array([0, 2]), [0], pos0=1)
    d1 = O.sparse_attend(Q, Kl, Vl, Kb, Vb, np.array([0, 2]), [0], pos0=16)
    assert not np.allclose(d0, d1)
    assert np.array_equal(O.sparse_attend(Q, Kl, Vl, Kb, Vb, np.array([0, 2]), [0]), d0)


# ---------------------------------------------------------------------------
# interleave ([techblg] §M Memory Interleave bullet; [chooseai] §2.4)
# ---------------------------------------------------------------------------
def test_interleave_incremental_equals_full_reroute():
    import synth
    mem, chains = synth.cfg5_memory("cpu", seed=7, n_tokens=60_000, n_queries=2, hops=3)
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    Kb, Vb, Rb, dco = O.pool(u16(mem.K), u16(mem.V), u16(mem.KR), mem.doc_token_offsets)
    for qi, chain in enumerate(chains):
        st = O.InterleaveState(len(dco) - 1)
        for r, doc in enumerate(chain):
            QR, Q, Kn, Vn = synth.cfg5_round(mem, doc, qi, r, seed=7, M_new=96, block=64)
            ids, sc, mg, out = O.interleave_step(st, u16(Q), u16(Kn), u16(Vn), u16(QR), Rb, Kb, Vb, dco, k=4)
            full = O.doc_scores(O.chunk_scores(st.QR_all, Rb), dco)
            assert np.array_equal(full, st.doc_scores)
            assert doc in set(ids)
            assert all(d in set(ids) for d in chain[:r + 1])
            assert out.shape == (96, 32, 128)


def test_interleave_attends_over_the_whole_active_context():
    """Each round's output is dense attention of the new tokens over every
    pooled chunk (k >= N selects all documents, pos0 = N) plus *all* local
    tokens appended so far, the new ones last and causal: checked against the
    independent torch SDPA + complex-rotation reference, round by round."""
    rng = np.random.default_rng(31)
    counts = [2, 1, 3]
    dco = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    C = int(dco[-1])
    Kb, Vb = bf16_randn((C, 8, 128), 0.3, rng), bf16_randn((C, 8, 128), 0.3, rng)
    Rb = bf16_randn((C, 8, 128), 0.125, rng)
    st = O.InterleaveState(len(counts))
    Ks, Vs = [], []
    for r, m_new in enumerate((5, 3, 4)):
        Q = bf16_randn((m_new, 32, 128), rng=rng)
        Kn, Vn = bf16_randn((m_new, 8, 128), rng=rng), bf16_randn((m_new, 8, 128), rng=rng)
        QR = bf16_randn((m_new, 8, 128), rng=rng)
        Ks.append(Kn)
        Vs.append(Vn)
        ids, sc, mg, out = O.interleave_step(st, Q, Kn, Vn, QR, Rb, Kb, Vb, dco, k=4)
        assert sorted(int(x) for x in ids) == [0, 1, 2]
        ref = _dense_reference(Q, np.concatenate(Ks), np.concatenate(Vs), Kb, Vb, pos0=3)
        assert np.allclose(out, ref, atol=1e-10, rtol=1e-10), f"round {r}"


# ---------------------------------------------------------------------------
# Router supervision: L_aux and its gradient ([techblg] §M training bullet)
# ---------------------------------------------------------------------------
def _aux_instance(seed, M=3, counts=(2, 3, 4), scale=1.0):
    rng = np.random.default_rng(seed)
    dco = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    q = rng.normal(size=(M, 8, 128)) * scale
    k = rng.normal(size=(int(dco[-1]), 8, 128))
    return q, k, dco


def test_aux_loss_gradient_matches_finite_differences():
    """Central differences on sampled coordinates of q and k (the maxima are
    attained with clear margins on random data, so the loss is smooth there)."""
    q, k, dco = _aux_instance(11)
    pos, tau = [1], 0.1
    loss, dq, dk, s, cs, ts, gaps = O.aux_loss_f64(q, k, dco, pos, tau)
    assert np.all(gaps > 1e-3)
    rng = np.random.default_rng(12)
    h = 1e-6
    for arr, grad in ((q, dq), (k, dk)):
        for _ in range(40):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            old = arr[idx]
            arr[idx] = old + h
            fp = O.aux_loss_f64(q, k, dco, pos, tau)[0]
            arr[idx] = old - h
            fm = O.aux_loss_f64(q, k, dco, pos, tau)[0]
            arr[idx] = old
            fd = (fp - fm) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (idx, fd, grad[idx])


def test_aux_loss_gradient_matches_torch_autograd():
    """An independent forward in torch (float64, CPU) differentiated by
    autograd, including a query token at the norm clamp (a zero vector)."""
    q, k, dco = _aux_instance(13, M=4, counts=(3, 1, 5, 2))
    q[2, 5] = 0.0                       # clamped norm: the gradient is k̂ / eps
    pos, tau = [0, 3], 0.05
    loss, dq, dk, *_ = O.aux_loss_f64(q, k, dco, pos, tau)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    qh = tq / tq.norm(dim=-1, keepdim=True).clamp_min(O.NORM_EPS)
    kh = tk / tk.norm(dim=-1, keepdim=True).clamp_min(O.NORM_EPS)
    S = torch.einsum("mhd,chd->mc", qh, kh) / 8
    s = torch.stack([S[:, int(dco[i]):int(dco[i + 1])].max() for i in range(len(dco) - 1)])
    neg = torch.ones(len(s), dtype=torch.bool)
    neg[pos] = False
    terms = []
    for i in pos:
        logits = torch.cat([(s[i] / tau).reshape(1), s[neg] / tau])
        terms.append(-(logits[0] - torch.logsumexp(logits, 0)))
    L = torch.stack(terms).mean()
    L.backward()
    assert abs(L.item() - loss) < 1e-12
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-9, atol=1e-12)


def test_aux_loss_invariants():
    q, k, dco = _aux_instance(14, M=2, counts=(4, 4, 4, 4))
    pos, tau = [2], 0.2
    loss, dq, dk, *_ = O.aux_loss_f64(q, k, dco, pos, tau)
    # cosines ignore scale: each row's gradient is orthogonal to the row
    assert np.abs((dq * q).sum(-1)).max() < 1e-12
    assert np.abs((dk * k).sum(-1)).max() < 1e-12
    # ... and scaling q by 3 keeps the loss and divides dq by 3
    l3, dq3, dk3, *_ = O.aux_loss_f64(3.0 * q, k, dco, pos, tau)
    assert abs(l3 - loss) < 1e-12
    np.testing.assert_allclose(dq3, dq / 3.0, rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(dk3, dk, rtol=1e-9, atol=1e-15)


def test_aux_loss_closed_forms():
    rng = np.random.default_rng(15)
    q = rng.normal(size=(2, 8, 128))
    row = rng.normal(size=(8, 128))
    k = np.repeat(row[None], 6, axis=0)            # every chunk the same key
    dco = np.array([0, 1, 3, 4, 6])
    # all document scores equal: each positive's share is 1 / (1 + n_neg)
    for pos in ([0], [1, 3]):
        loss = O.aux_loss_f64(q, k, dco, pos, 0.07)[0]
        assert abs(loss - math.log(4 - len(pos) + 1)) < 1e-12
    # no negatives: every positive has probability 1, loss and gradients 0
    loss, dq, dk, *_ = O.aux_loss_f64(q, k, dco, [0, 1, 2, 3], 0.07)
    assert abs(loss) < 1e-15 and not dq.any() and not dk.any()
    # very high temperature: the scores stop mattering
    q2, k2, dco2 = _aux_instance(16, counts=(2, 2, 2, 2, 2))
    assert abs(O.aux_loss_f64(q2, k2, dco2, [4], 1e12)[0] - math.log(5)) < 1e-9


def test_aux_loss_subgradient_rules():
    """Ties at the maxima go to the first chunk and the first token."""
    rng = np.random.default_rng(17)
    u = rng.normal(size=(8, 128))
    q = np.stack([u, u, rng.normal(size=(8, 128))])   # tokens 0 and 1 identical
    k = np.stack([rng.normal(size=(8, 128)), u, u, rng.normal(size=(8, 128))])
    dco = np.array([0, 3, 4])                           # doc 0: chunks 0-2 (1 and 2 tie)
    _, dq, dk, s, cs, ts, gaps = O.aux_loss_f64(q, k, dco, [1], 0.1)
    assert cs[0] == 1 and ts[0] == 0 and gaps[0] == 0.0
    assert not dk[2].any() and not dq[1].any()


def test_aux_batched_key_gradient_is_the_sum_over_queries():
    """route_aux_loss over B queries: loss[b] and dQR[b] are query b's, and
    dK̄ᴿ is the gradient of the summed loss — checked by central differences
    of Σ_b loss_b in the keys (decoded bf16 values, perturbed in float64)."""
    rng = np.random.default_rng(41)
    dco = np.array([0, 2, 5, 6, 9], dtype=np.int64)
    C = int(dco[-1])
    KR = bf16_randn((C, 8, 128), 0.125, rng)
    QR = bf16_randn((3, 2, 8, 128), rng=rng)
    positives = [[1], [0, 3], [2]]
    tau = 0.1
    loss, dQ, dK, s, cs, ts, gaps = O.route_aux_loss(QR, KR, dco, positives, tau)
    assert np.all(gaps > 1e-3)
    k = O.bf16_to_f64(KR)
    qs = [O.bf16_to_f64(QR[b]) for b in range(3)]
    for b in range(3):
        assert loss[b] == O.aux_loss_f64(qs[b], k, dco, positives[b], tau)[0]

    def total(kk):
        return sum(O.aux_loss_f64(qs[b], kk, dco, positives[b], tau)[0] for b in range(3))

    h = 1e-6
    # rows that carry gradient from more than one query are among those sampled
    rows = sorted(set(int(c) for c in cs.ravel()))
    for _ in range(30):
        idx = (int(rng.choice(rows)), int(rng.integers(0, 8)), int(rng.integers(0, 128)))
        old = k[idx]
        k[idx] = old + h
        fp = total(k)
        k[idx] = old - h
        fm = total(k)
        k[idx] = old
        fd = (fp - fm) / (2 * h)
        assert abs(fd - dK[idx]) <= 1e-6 * max(1.0, abs(fd)), (idx, fd, dK[idx])
    # each query's dQR is that query's own gradient
    for b in range(3):
        idx = (1, 4, 77)
        q = qs[b]
        old = q[idx]
        q[idx] = old + h
        fp = O.aux_loss_f64(q, k, dco, positives[b], tau)[0]
        q[idx] = old - h
        fm = O.aux_loss_f64(q, k, dco, positives[b], tau)[0]
        q[idx] = old
        assert abs((fp - fm) / (2 * h) - dQ[b][idx]) <= 1e-6


def test_aux_choice_evaluates_at_the_given_pairs():
    """``choice``: at the first maxima it reproduces the free call; at other
    (chunk, token) pairs, s_i is the head-mean cosine at that pair and the
    gradient is that of an independent torch forward that reads s_i there."""
    rng = np.random.default_rng(43)
    dco = np.array([0, 3, 4, 7], dtype=np.int64)
    C = int(dco[-1])
    KR = bf16_randn((C, 8, 128), 0.125, rng)
    QR = bf16_randn((2, 3, 8, 128), rng=rng)
    positives = [[2], [0]]
    tau = 0.2
    free = O.route_aux_loss(QR, KR, dco, positives, tau)
    same = O.route_aux_loss(QR, KR, dco, positives, tau, choice=(free[4], free[5]))
    for a, b in zip(free, same):
        assert np.array_equal(a, b)
    # other pairs: the last chunk of every document and token 2 (query 0),
    # the first chunk and token 1 (query 1)
    c_alt = np.stack([dco[1:] - 1, dco[:-1]])
    t_alt = np.stack([np.full(3, 2), np.full(3, 1)])
    loss, dQ, dK, s, cs, ts, _ = O.route_aux_loss(QR, KR, dco, positives, tau, choice=(c_alt, t_alt))
    assert np.array_equal(cs, c_alt) and np.array_equal(ts, t_alt)
    tk = torch.tensor(O.bf16_to_f64(KR), requires_grad=True)
    kh = tk / tk.norm(dim=-1, keepdim=True).clamp_min(O.NORM_EPS)
    total = 0.0
    tqs = []
    for b in range(2):
        tq = torch.tensor(O.bf16_to_f64(QR[b]), requires_grad=True)
        tqs.append(tq)
        qh = tq / tq.norm(dim=-1, keepdim=True).clamp_min(O.NORM_EPS)
        sb = torch.stack([(qh[int(t_alt[b, i])] * kh[int(c_alt[b, i])]).sum(-1).mean()
                          for i in range(3)])
        assert np.allclose(s[b], sb.detach().numpy(), rtol=0, atol=1e-15)
        neg = torch.ones(3, dtype=torch.bool)
        neg[positives[b]] = False
        terms = [-(sb[i] / tau - torch.logsumexp(torch.cat([(sb[i] / tau).reshape(1),
                                                            sb[neg] / tau]), 0))
                 for i in positives[b]]
        Lb = torch.stack(terms).mean()
        assert abs(Lb.item() - loss[b]) < 1e-12
        total = total + Lb
    total.backward()
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=1e-9, atol=1e-12)
    for b in range(2):
        np.testing.assert_allclose(dQ[b], tqs[b].grad.numpy(), rtol=1e-9, atol=1e-12)
