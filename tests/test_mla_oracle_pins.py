"""Pins of the MLA oracle (oracle/kvc_mla_oracle.py), on the CPU.

The oracle follows the MultiHeadLatentAttention listing of "KV Cache 최적화
심층 분석: GQA·MLA·MHA 어텐션 메커니즘과 메모리 효율화 전략" (youngju.dev).  The
pins hold it to things other than itself:

* brute force on tiny inputs in plain Python (explicit sums for the
  up-projections and the softmax, the listing's view(S, n_heads, d_k) head
  split written out as index arithmetic);
* the absorbed form, an exact rewrite: q~ = W_uk,h^T q_h, scores q~ . c_t,
  output W_uv,h (sum_t p_t c_t) + b_uv,h;
* closed forms: one token gives W_uv,h c_0 + b_uv,h; the key bias shifts
  every score of a head by one constant, which the softmax removes;
* k_rope is stored but does not reach the attention (the listing as written);
* the append writes exactly one row, [c_kv | k_rope];
* the listing's cache-size comment.

Planted mistakes in a copy of the module must each fail one of them.
"""
import math
import types

import numpy as np
import pytest

import oracle.kvc_oracle as O
import oracle.kvc_mla_oracle as MLA

SRC = open(MLA.__file__).read()


def _case(rng, B=2, H=3, d_k=4, dl=8, rd=2, T=6, dtype="f32"):
    mk = lambda *s, scale=1.0: O.round_store((scale * rng.standard_normal(s)).astype(np.float32), dtype)
    cache = mk(B, T, dl + rd)
    q = mk(B, H, d_k)
    Wk, Wv = mk(H * d_k, dl, scale=dl ** -0.5), mk(H * d_k, dl, scale=dl ** -0.5)
    bk, bv = mk(H * d_k, scale=0.1), mk(H * d_k, scale=0.1)
    return cache, q, Wk, bk, Wv, bv


def _brute(q, cache, L, Wk, bk, Wv, bv, dl, dtype):
    """Plain Python: k[h][t][i] = sum_l Wk[h*d_k + i][l] c[t][l] + bk[h*d_k + i]."""
    f = lambda a: O.to_f64(a, dtype).tolist()
    qv, cv, Wkv, bkv, Wvv, bvv = f(q), f(cache), f(Wk), f(bk), f(Wv), f(bv)
    B, H, d_k = q.shape
    out = np.zeros((B, H, d_k))
    for b in range(B):
        c = [row[:dl] for row in cv[b][:L[b]]]
        for h in range(H):
            keys = [[sum(Wkv[h * d_k + i][l] * ct[l] for l in range(dl)) + bkv[h * d_k + i] for i in range(d_k)]
                    for ct in c]
            vals = [[sum(Wvv[h * d_k + i][l] * ct[l] for l in range(dl)) + bvv[h * d_k + i] for i in range(d_k)]
                    for ct in c]
            s = [sum(qv[b][h][i] * kt[i] for i in range(d_k)) / math.sqrt(d_k) for kt in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            for i in range(d_k):
                out[b, h, i] = sum(wt * vt[i] for wt, vt in zip(w, vals)) / z
    return out


# --- checks (True when the module passes) ------------------------------------


def check_brute_force(M) -> bool:
    rng = np.random.default_rng(51)
    ok = True
    for dtype in ("f32", "bf16"):
        cache, q, Wk, bk, Wv, bv = _case(rng, dtype=dtype)
        L = [6, 3]
        got = M.decode_attention_mla(q, cache, L, Wk, bk, Wv, bv, 8, dtype)
        ok &= bool(np.allclose(got, _brute(q, cache, L, Wk, bk, Wv, bv, 8, dtype), rtol=0, atol=1e-12))
    return ok


def check_absorbed(M) -> bool:
    rng = np.random.default_rng(52)
    B, H, d_k, dl, rd, T = 3, 4, 8, 16, 4, 20
    cache, q, Wk, bk, Wv, bv = _case(rng, B, H, d_k, dl, rd, T, "bf16")
    L = [20, 9, 1]
    got = M.decode_attention_mla(q, cache, L, Wk, bk, Wv, bv, dl, "bf16")
    f = lambda a: O.to_f64(a, "bf16")
    qf, Wkf, bkf, Wvf, bvf = f(q), f(Wk), f(bk), f(Wv), f(bv)
    ok = True
    for b in range(B):
        c = f(cache[b, :L[b], :dl])
        for h in range(H):
            rows = slice(h * d_k, (h + 1) * d_k)
            qt = Wkf[rows].T @ qf[b, h]                      # absorbed query, d_latent
            s = (c @ qt + qf[b, h] @ bkf[rows]) / math.sqrt(d_k)
            p = np.exp(s - s.max())
            p /= p.sum()
            ref = Wvf[rows] @ (p @ c) + bvf[rows]
            ok &= bool(np.allclose(got[b, h], ref, rtol=0, atol=1e-12))
    return ok


def check_closed_forms(M) -> bool:
    rng = np.random.default_rng(53)
    cache, q, Wk, bk, Wv, bv = _case(rng, B=2, H=3, d_k=4, dl=8, rd=2, T=5, dtype="bf16")
    f = lambda a: O.to_f64(a, "bf16")
    one = M.decode_attention_mla(q, cache, [1, 1], Wk, bk, Wv, bv, 8, "bf16")
    ok = True
    for b in range(2):
        for h in range(3):
            rows = slice(h * 4, (h + 1) * 4)
            ok &= bool(np.allclose(one[b, h], f(Wv)[rows] @ f(cache[b, 0, :8]) + f(bv)[rows], rtol=0, atol=1e-14))
    # the key bias cancels in the softmax; the value bias does not
    L = [5, 4]
    base = M.decode_attention_mla(q, cache, L, Wk, bk, Wv, bv, 8, "bf16")
    bk2 = O.round_store(rng.standard_normal(bk.shape).astype(np.float32), "bf16")
    ok &= bool(np.allclose(M.decode_attention_mla(q, cache, L, Wk, bk2, Wv, bv, 8, "bf16"), base, rtol=0, atol=1e-12))
    bv2 = O.round_store(rng.standard_normal(bv.shape).astype(np.float32), "bf16")
    ok &= not bool(np.allclose(M.decode_attention_mla(q, cache, L, Wk, bk, Wv, bv2, 8, "bf16"), base, atol=1e-3))
    return ok


def check_rope_part_unread(M) -> bool:
    rng = np.random.default_rng(54)
    cache, q, Wk, bk, Wv, bv = _case(rng, dtype="bf16")
    L = [6, 4]
    base = M.decode_attention_mla(q, cache, L, Wk, bk, Wv, bv, 8, "bf16")
    c2 = cache.copy()
    c2[..., 8:] = O.round_store(rng.standard_normal(c2[..., 8:].shape).astype(np.float32), "bf16")
    return bool(np.array_equal(M.decode_attention_mla(q, c2, L, Wk, bk, Wv, bv, 8, "bf16"), base))


def check_append(M) -> bool:
    rng = np.random.default_rng(55)
    B, T, dl, rd = 3, 7, 8, 2
    cache = O.round_store(rng.standard_normal((B, T, dl + rd)).astype(np.float32), "bf16")
    ckv = O.round_store(rng.standard_normal((B, dl)).astype(np.float32), "bf16")
    kr = O.round_store(rng.standard_normal((B, rd)).astype(np.float32), "bf16")
    cached = np.array([0, 4, 6])
    c2 = M.append_mla(cache, cached, ckv, kr)
    ok = True
    for b, p in enumerate(cached):
        ok &= bool(np.array_equal(c2[b, p], np.concatenate([ckv[b], kr[b]])))
        mask = np.ones(T, bool)
        mask[p] = False
        ok &= bool(np.array_equal(c2[b, mask], cache[b, mask]))
    return ok


def check_heads_subset(M) -> bool:
    rng = np.random.default_rng(56)
    cache, q, Wk, bk, Wv, bv = _case(rng, B=3, H=4, d_k=8, dl=16, rd=4, T=12, dtype="bf16")
    L = [12, 5, 1]
    full = M.decode_attention_mla(q, cache, L, Wk, bk, Wv, bv, 16, "bf16")
    pairs = [(0, 3), (1, 0), (2, 2), (0, 1)]
    sub = M.decode_attention_mla_heads(q, cache, L, Wk, bk, Wv, bv, 16, "bf16", pairs)
    return all(np.array_equal(sub[n], full[b, h]) for n, (b, h) in enumerate(pairs))


CHECKS = [check_heads_subset, check_brute_force, check_absorbed, check_closed_forms, check_rope_part_unread, check_append]


@pytest.mark.parametrize("chk", CHECKS, ids=lambda c: c.__name__)
def test_pin_holds(chk):
    assert chk(MLA)


def test_cache_size_comment_of_the_listing():
    """The listing's comment: B * S * (d_latent + rope_dim) elements, and
    d_latent / (2 * n_heads * d_k) of a full per-head cache.  For 32 heads of
    128 and a 512-wide latent with 64 rope values: 1152 bytes per token in
    bf16 against 16384, the latent part 1/16 of it."""
    assert MLA.mla_cache_bytes_per_token(512, 64, 2) == 1152
    assert O.kv_bytes_per_token(1, 32, 128, 2) == 16384
    assert 512 / (2 * 32 * 128) == 1 / 16


# --- planted mistakes -------------------------------------------------------

MUTATIONS = {
    "heads split d_k-major": ("y.reshape(c_kv.shape[0], n_heads, d_k).transpose(1, 0, 2)",
                              "y.reshape(c_kv.shape[0], d_k, n_heads).transpose(2, 0, 1)"),
    "value bias dropped": ("V = up_project(c, Wv, bv, H, d_k)", "V = up_project(c, Wv, 0.0 * bv, H, d_k)"),
    "scaled by the latent width": ("sc = 1.0 / math.sqrt(d_k) if", "sc = 1.0 / math.sqrt(d_latent) if"),
    "keys from the value projection": ("K = up_project(c, Wk, bk, H, d_k)", "K = up_project(c, Wv, bv, H, d_k)"),
    "latent read from the row's end": ("c = O.to_f64(cache[b, :L, :d_latent], dtype)",
                                       "c = O.to_f64(cache[b, :L, -d_latent:], dtype)"),
    "append one slot late": ("c2[b, p, :dl] = c_kv_new[b]", "c2[b, p + 1, :dl] = c_kv_new[b]"),
    "new token not attended": ("        L = int(seq_lens[b])\n        c = O.to_f64",
                               "        L = int(seq_lens[b]) - 1\n        c = O.to_f64"),
}


def _load(src: str) -> types.ModuleType:
    m = types.ModuleType("mla_oracle_mutant")
    src = src.replace("from . import kvc_oracle as O", "import oracle.kvc_oracle as O")
    exec(compile(src, "mla_oracle_mutant", "exec"), m.__dict__)
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
