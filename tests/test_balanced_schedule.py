"""The balanced schedule of the bf16 matrix-core decode kernel, modelled on
the host (no GPU).

The kernel's workgroups each read all sequence lengths, lay the units'
loop steps out as one list (unit u = b * H_kv + j holds n_b =
max(1, ceil(L_b / step)) steps), and take equal ranges of it: workgroup w of
N takes [w T / N, (w + 1) T / N) (N the planned count, or T if smaller, so
that no range is empty).  A range crossing units is run as one
segment per unit; a unit shared by several workgroups is merged by the last
to arrive from partial rows that each workgroup writes to one of two slots
of its own (slot 0: its first segment, slot 1: its last).

This model restates that integer arithmetic and checks, over many ragged
shapes, what the kernel relies on for correctness and memory safety:
every step of every unit is covered exactly once; a segment is at most
kBalMaxSteps steps long; each partial slot is written by at most one
segment, and the merge of each unit reads exactly the slots its own
segments wrote, in workgroup order; slot indices stay inside the N * 2 rows
the plan allocates; a unit inside one workgroup writes no partial.
"""

import random

import pytest

K_BAL_MAX_TOKENS = 15360   # kvc_internal.h: kBalMaxTokens


def steps_of(L, step):
    return (L + step - 1) // step if L > 0 else 1


def plan_workgroups(units, max_len, step, slots):
    """The plan's workgroup count: one round, more if a range would exceed
    kBalMaxTokens tokens (bound from the longest possible sequence)."""
    bound = units * ((max(max_len, 1) + step - 1) // step)
    max_steps = K_BAL_MAX_TOKENS // step
    return max(slots, (bound + max_steps - 1) // max_steps)


def schedule(lens, H_kv, N, step):
    """Every workgroup's segments, as the kernel derives them: a list per
    workgroup of dicts (unit, first/last step, t_begin, t_end, nsp, split,
    partial row slot, the unit's first workgroup and slot0)."""
    B = len(lens)
    n = [steps_of(L, step) for L in lens]
    pre = [0]
    for x in n:
        pre.append(pre[-1] + x)
    T = pre[B] * H_kv
    N = min(N, T)           # with fewer steps, the first T workgroups take one each

    def w_of(x):
        return ((x + 1) * N - 1) // T

    def unit_start(b, j):
        return H_kv * pre[b] + j * n[b], n[b]

    out = []
    for w in range(N):
        s0, s1 = w * T // N, (w + 1) * T // N
        segs = []
        assert s0 < s1, "every taking part workgroup has a step"
        if s0 < s1:
            # the one sequence holding step s0
            hits = [b for b in range(B) if pre[b] * H_kv <= s0 < pre[b + 1] * H_kv]
            assert len(hits) == 1
            b0 = hits[0]
            sb0, n0 = unit_start(b0, 0)
            u0 = b0 * H_kv + (s0 - sb0) // n0
            it = 0
            while True:
                u = u0 + it
                if u >= B * H_kv:
                    break
                bq, jj = divmod(u, H_kv)
                ub, nb = unit_start(bq, jj)
                if ub >= s1:
                    break
                ue = ub + nb
                sa, se = max(ub, s0), min(ue, s1)
                wf = w_of(ub)
                segs.append(dict(unit=u, b=bq, sa=sa, se=se, ub=ub, ue=ue,
                                 t_begin=(sa - ub) * step, t_end=min((se - ub) * step, lens[bq]),
                                 nsp=w_of(ue - 1) - wf + 1, split=w - wf, wf=wf,
                                 slot=0 if it == 0 else 1,
                                 slot0=1 if wf * T // N < ub else 0))
                it += 1
        out.append(segs)
    return out, T


def check(lens, H_kv, N, step):
    sched, T = schedule(lens, H_kv, N, step)
    N = min(N, T)
    B = len(lens)
    covered = {}
    written = {}
    units = {}
    for w, segs in enumerate(sched):
        assert len(segs) == 0 or segs[0]["sa"] == w * T // N
        for k, sg in enumerate(segs):
            assert (sg["se"] - sg["sa"]) * step <= K_BAL_MAX_TOKENS or N * (K_BAL_MAX_TOKENS // step) < T
            for x in range(sg["sa"], sg["se"]):
                assert x not in covered
                covered[x] = sg["unit"]
            assert 0 <= sg["t_begin"] <= sg["t_end"] <= lens[sg["b"]] or lens[sg["b"]] == 0
            assert 0 <= sg["split"] < sg["nsp"]
            units.setdefault(sg["unit"], []).append((w, sg))
            if sg["nsp"] > 1:
                row = 2 * w + sg["slot"]
                assert 0 <= row < 2 * N
                assert row not in written, "two segments share a partial slot"
                written[row] = sg["unit"]
            # only the first segment of a workgroup may start inside a unit,
            # only the last may end inside one
            if sg["sa"] > sg["ub"]:
                assert k == 0
            if sg["se"] < sg["ue"]:
                assert k == len(segs) - 1
    assert len(covered) == T and set(covered) == set(range(T))
    assert sorted(units) == list(range(B * H_kv))
    for u, lst in units.items():
        ws = [w for w, _ in lst]
        sg0 = lst[0][1]
        assert ws == list(range(sg0["wf"], sg0["wf"] + sg0["nsp"])), "a unit's workgroups are consecutive"
        # the first segment of the unit holds t = 0, the last its end
        assert lst[0][1]["t_begin"] == 0 and lst[-1][1]["t_end"] == lens[u // H_kv]
        if sg0["nsp"] > 1:
            # the merge's slots are exactly the ones its segments wrote
            reads = [2 * (sg0["wf"] + s) + (sg0["slot0"] if s == 0 else 0) for s in range(sg0["nsp"])]
            wrote = [2 * w + sg["slot"] for w, sg in lst]
            assert reads == wrote
            assert all(written[r] == u for r in reads)


@pytest.mark.parametrize("seed", range(40))
def test_random_ragged_shapes(seed):
    rng = random.Random(seed)
    B = rng.choice([1, 2, 3, 7, 16, 32, 64, 100])
    H_kv = rng.choice([1, 2, 8])
    step = rng.choice([64, 128])          # the bf16 and the quantized kernels' loop steps
    max_len = rng.choice([1, 63, 64, 65, 500, 4096, 16384])
    lens = [rng.choice([0, 1, rng.randint(0, max_len), max_len, (rng.randint(0, max_len) // 64) * 64])
            for _ in range(B)]
    lens = [min(max(x, 0), max_len) for x in lens]
    N = plan_workgroups(B * H_kv, max_len, step, rng.choice([4, 7, 256, 768]))
    check(lens, H_kv, N, step)


@pytest.mark.parametrize("lens,H_kv,N", [
    ([0], 1, 256),                       # one empty sequence: one step, one workgroup
    ([1], 1, 256),
    ([64, 64], 8, 3),                    # fewer workgroups than units
    ([4096] * 64, 1, 256),               # even split, ranges on unit boundaries
    ([100000], 8, 4000),                 # long sequence, many workgroups per unit
    ([5, 0, 70, 129, 0, 64], 2, 5),
])
def test_edge_shapes(lens, H_kv, N):
    check(lens, H_kv, N, 64)


def test_workload_shapes():
    """The ragged paged workload the schedule serves: 32 sequences of
    1024..16384 tokens under 8 KV heads, on 768 workgroups of 64-token steps
    (bf16) and 512 of 128-token steps (uint8); and a 64-sequence MQA batch."""
    rng = random.Random(7)
    lens = [rng.randint(1024, 16384) + 1 for _ in range(32)]
    check(lens, 8, 768, 64)
    check(lens, 8, 512, 128)
    check([rng.randint(512, 4096) + 1 for _ in range(64)], 1, 256, 64)


def test_plan_bounds_range_length():
    """The planned workgroup count keeps every range within kBalMaxTokens
    tokens (960 blocks of 16, inside the staged table of 1024 entries)
    whatever the lengths (at most max_len each), for both kernels' steps."""
    for step in (64, 128):
        for units, max_len in ((256, 16384), (8, 131072), (512, 1 << 20), (1, 64)):
            N = plan_workgroups(units, max_len, step, 256)
            T = units * steps_of(max_len, step)
            assert -(-T // N) * step <= K_BAL_MAX_TOKENS
            assert K_BAL_MAX_TOKENS // 16 + 2 <= 1024
