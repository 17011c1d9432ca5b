"""Pins of the multi-token decode oracle (oracle/kvc_multi_oracle.py), on the CPU.

Several new tokens per sequence ([ARCH] section 7's parallel verification of
gamma drafted tokens; section 6's chunked prefill).  The pins hold the oracle
to things other than itself:

* one token at a time: appending the n tokens one by one and running the
  single-token oracle after each gives the same rows ([KVC] step 1 and FAQ:
  cached decode equals recomputation under the causal mask);
* full causal recomputation of the whole sequence (the unwindowed oracle's
  causal_attention_full, with [BOOK] listing 2.4's mask): the last n rows;
* torch's scaled_dot_product_attention in float64 with an explicit
  causal-with-offset (and band) mask;
* n = 1 is the single-token step; a window is the windowed oracle row by row;
* paged == contiguous.

Planted mistakes in a copy of the module must each fail one of them.
"""
import types

import numpy as np
import pytest
import torch

import oracle.kvc_oracle as O
import oracle.kvc_multi_oracle as MO
import oracle.kvc_window_oracle as WO

SRC = open(MO.__file__).read()


def _inputs(rng, B, n, H_q, H_kv, d, T, cached, dtype="bf16"):
    mk = lambda *s: O.round_store(rng.standard_normal(s).astype(np.float32), dtype)
    k, v = mk(B, H_kv, T, d), mk(B, H_kv, T, d)
    return k, v, mk(B, n, H_q, d), mk(B, n, H_kv, d), mk(B, n, H_kv, d)


# --- checks (True when the module passes) ------------------------------------


def check_one_at_a_time(M) -> bool:
    rng = np.random.default_rng(41)
    B, n, H_q, H_kv, d, T = 3, 5, 6, 2, 16, 40
    cached = np.array([0, 7, 30])
    cos, sin = O.rope_table(T, d)
    k, v, q, kn, vn = _inputs(rng, B, n, H_q, H_kv, d, T, cached)
    ok = True
    for window in (0, 3, 9):
        k2, v2, q2 = M.append_multi(k, v, cached, kn, vn, cos, sin, "bf16", q=q)
        got = M.decode_attention_multi(q2, k2, v2, cached + n, "bf16", window)
        ks, vs = k.copy(), v.copy()
        for i in range(n):
            ks, vs, qi = O.append_contiguous(ks, vs, cached + i, kn[:, i], vn[:, i], cos, sin, "bf16", q=q[:, i])
            ok &= bool(np.array_equal(ks, k2) if i == n - 1 else True)
            ref = WO.decode_attention_window(qi, ks, vs, cached + i + 1, window, "bf16")
            ok &= bool(np.allclose(got[:, i], ref, rtol=0, atol=1e-12))
            ok &= bool(np.array_equal(q2[:, i], qi))
        ok &= bool(np.array_equal(vs, v2))
    return ok


def check_full_recompute(M) -> bool:
    """A sequence of N tokens: the first N - n appended one step at a time is
    the same cache as a prefix; the last n verified together must equal the
    last n rows of the whole sequence's causal recomputation."""
    rng = np.random.default_rng(42)
    N, n, H_q, H_kv, d = 12, 4, 4, 2, 16
    cos, sin = O.rope_table(N, d)
    mk = lambda *s: O.round_store(rng.standard_normal(s).astype(np.float32), "bf16")
    q_raw, k_raw, v_raw = mk(H_q, N, d), mk(H_kv, N, d), mk(H_kv, N, d)
    full = O.causal_attention_full(q_raw, k_raw, v_raw, cos, sin, "bf16")
    c = N - n
    k = np.zeros((1, H_kv, N, d), np.uint16)
    v = np.zeros_like(k)
    for t in range(c):
        k, v, _ = O.append_contiguous(k, v, [t], k_raw[None, :, t], v_raw[None, :, t], cos, sin, "bf16")
    k2, v2, q2 = M.append_multi(k, v, [c], k_raw[None, :, c:].transpose(0, 2, 1, 3),
                                v_raw[None, :, c:].transpose(0, 2, 1, 3), cos, sin, "bf16",
                                q=q_raw[None, :, c:].transpose(0, 2, 1, 3))
    got = M.decode_attention_multi(q2, k2, v2, [N], "bf16")[0]       # [n, H_q, d]
    return bool(np.allclose(got, full[:, c:].transpose(1, 0, 2), rtol=0, atol=1e-12))


def check_sdpa(M) -> bool:
    rng = np.random.default_rng(43)
    B, n, H_q, H_kv, d, T = 2, 6, 8, 2, 32, 30
    G = H_q // H_kv
    k, v, q, _, _ = _inputs(rng, B, n, H_q, H_kv, d, T, None)
    L = [30, 11]
    ok = True
    for window in (0, 5):
        got = M.decode_attention_multi(q, k, v, L, "bf16", window)
        for b in range(B):
            Lb = L[b]
            pos = np.arange(Lb - n, Lb)[:, None]
            t = np.arange(Lb)[None, :]
            mask = t <= pos
            if window:
                mask &= t > pos - window
            Q = torch.from_numpy(O.to_f64(q[b], "bf16").transpose(1, 0, 2))          # [H_q, n, d]
            K = torch.from_numpy(np.repeat(O.to_f64(k[b, :, :Lb], "bf16"), G, axis=0))
            V = torch.from_numpy(np.repeat(O.to_f64(v[b, :, :Lb], "bf16"), G, axis=0))
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=torch.from_numpy(mask))
            ok &= bool(np.allclose(got[b], ref.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12))
    return ok


def check_single_token(M) -> bool:
    rng = np.random.default_rng(44)
    B, H_q, H_kv, d, T = 3, 4, 4, 16, 20
    cached = np.array([3, 0, 19])
    cos, sin = O.rope_table(T, d)
    k, v, q, kn, vn = _inputs(rng, B, 1, H_q, H_kv, d, T, cached)
    k2, v2, q2 = M.append_multi(k, v, cached, kn, vn, cos, sin, "bf16", q=q)
    ka, va, qa = O.append_contiguous(k, v, cached, kn[:, 0], vn[:, 0], cos, sin, "bf16", q=q[:, 0])
    ok = bool(np.array_equal(k2, ka) and np.array_equal(v2, va) and np.array_equal(q2[:, 0], qa))
    ok &= bool(np.array_equal(M.decode_attention_multi(q2, k2, v2, cached + 1, "bf16")[:, 0],
                              O.decode_attention(qa, ka, va, cached + 1, "bf16")))
    return ok


def check_paged(M) -> bool:
    rng = np.random.default_rng(45)
    B, n, H_q, H_kv, d, bs = 2, 3, 4, 2, 16, 4
    T = 24
    nb = T // bs
    cached = np.array([13, 2])
    cos, sin = O.rope_table(T, d)
    k, v, q, kn, vn = _inputs(rng, B, n, H_q, H_kv, d, T, cached)
    table = rng.permutation(B * nb).reshape(B, nb)
    pk = np.zeros((B * nb, H_kv, bs, d), np.uint16)
    pv = np.zeros_like(pk)
    for b in range(B):
        for lb in range(nb):
            pk[table[b, lb]] = k[b, :, lb * bs:(lb + 1) * bs]
            pv[table[b, lb]] = v[b, :, lb * bs:(lb + 1) * bs]
    k2, v2, q2 = M.append_multi(k, v, cached, kn, vn, cos, sin, "bf16", q=q)
    pk2, pv2, pq2 = M.append_multi_paged(pk, pv, table, bs, cached, kn, vn, cos, sin, "bf16", q=q)
    ok = bool(np.array_equal(q2, pq2))
    for window in (0, 4):
        ok &= bool(np.array_equal(M.decode_attention_multi_paged(pq2, pk2, pv2, table, bs, cached + n, "bf16", window),
                                  M.decode_attention_multi(q2, k2, v2, cached + n, "bf16", window)))
    return ok


CHECKS = [check_one_at_a_time, check_full_recompute, check_sdpa, check_single_token, check_paged]


@pytest.mark.parametrize("chk", CHECKS, ids=lambda c: c.__name__)
def test_pin_holds(chk):
    assert chk(MO)


def test_verification_width_of_the_worked_example():
    """[ARCH] section 7's example drafts gamma = 5 tokens: the target checks
    gamma + 1 = 6 positions in one pass; the last one sees every token."""
    L, n = 8192 + 6, 6
    assert [MO.query_range(L, n, i) for i in (0, n - 1)] == [(0, 8193), (0, L)]


# --- planted mistakes -------------------------------------------------------

MUTATIONS = {
    "no causal mask among the new tokens": ("hi = L - n + i + 1", "hi = L"),
    "causal limit one short": ("hi = L - n + i + 1", "hi = L - n + i"),
    "window counted from the last token": ("lo = max(0, hi - window) if", "lo = max(0, L - window) if"),
    "all new keys rotated at the first position": (
        "k2[b, :, p, :] = O.rope_rotate(k_new[b, i], dtype, cos[p], sin[p], style)",
        "k2[b, :, p, :] = O.rope_rotate(k_new[b, i], dtype, cos[c], sin[c], style)"),
    "queries not rotated at their own position": (
        "q2[b, i] = O.rope_rotate(q[b, i], dtype, cos[p], sin[p], style)\n    return k2, v2, q2\n\n\ndef append_multi_paged",
        "q2[b, i] = O.rope_rotate(q[b, i], dtype, cos[c], sin[c], style)\n    return k2, v2, q2\n\n\ndef append_multi_paged"),
    "new tokens stored in reverse": ("            p = c + i\n            k2[b, :, p, :]", "            p = c + n - 1 - i\n            k2[b, :, p, :]"),
    "paged slot of the first token for all": ("lb, off = O.paged_location(p, block_size)",
                                              "lb, off = O.paged_location(c, block_size)"),
}


def _load(src: str) -> types.ModuleType:
    m = types.ModuleType("multi_oracle_mutant")
    src = src.replace("from . import kvc_oracle as O", "import oracle.kvc_oracle as O")
    exec(compile(src, "multi_oracle_mutant", "exec"), m.__dict__)
    return m


def _passes(chk, M) -> bool:
    try:
        return bool(chk(M))
    except Exception:
        return False


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, f"mutation anchor not found once: {old}"
    M = _load(SRC.replace(old, new))
    assert not all(_passes(c, M) for c in CHECKS), f"no pin catches: {name}"


def test_checks_pass_on_an_unedited_copy():
    M = _load(SRC)
    assert all(_passes(c, M) for c in CHECKS)
