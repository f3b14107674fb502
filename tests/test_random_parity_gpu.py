"""Seeded random shapes through pa_prefill, pa_decode, pa_decode_append and
pa_decode_multi, each checked against the float64 oracle on the same bar as
the other parity tests (and, for the decode step, the cache bytes it writes): random batch sizes, context lengths drawn half from the tile and block
edges (1, 63..65, 127..129, 255..257, 511..513, 1023..1025) and half
uniformly, every supported head grouping, prefill rows with and without a
cached prefix (including 1..6-row short blocks), empty decode contexts, and
1..8 rows per sequence for the multi-row decode (at most 32 rows per kv head).
Case i draws from its own generator, so a failing case is reproduced alone."""

import numpy as np
import pytest

import workloads as wl
import test_decode_append_gpu as ta
import test_decode_gpu as td
import test_decode_multi_gpu as tm
import test_prefill_gpu as tp

pytestmark = pytest.mark.gpu

EDGES = [1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025]
GROUPS = [(1, 1), (2, 1), (4, 1), (8, 1), (8, 8), (16, 8), (32, 8), (64, 8), (4, 2), (8, 2)]
CASES = 60


def _ctx(rng, most):
    if rng.random() < 0.4:
        return int(rng.choice([e for e in EDGES if e <= most]))
    return int(rng.integers(1, most + 1))


@pytest.mark.parametrize("i", range(CASES))
def test_random_shape(i):
    rng = np.random.default_rng(7000 + i)
    hq, hkv = GROUPS[int(rng.integers(len(GROUPS)))]
    g = hq // hkv
    kind = ("prefill", "decode", "multi", "append")[i % 4]
    if kind == "prefill":
        b = int(rng.integers(1, 7))
        ctx = [_ctx(rng, 2000) for _ in range(b)]
        ql = []
        for c in ctx:
            r = rng.random()
            ql.append(c if r < 0.4 else (int(rng.integers(1, min(c, 6) + 1)) if r < 0.7
                                         else int(rng.integers(1, c + 1))))
        tp.check(wl.make_case(f"random_p{i}", "prefill", 7000 + i, ctx, hq, hkv, q_lens=ql))
    elif kind == "decode":
        b = int(rng.integers(1, 40))
        ctx = [0 if rng.random() < 0.05 else _ctx(rng, 9000) for _ in range(b)]
        ctx[0] = max(ctx[0], 1)
        td.check_full(wl.make_case(f"random_d{i}", "decode", 7000 + i, ctx, hq, hkv))
    elif kind == "append":
        b = int(rng.integers(1, 40))
        ctx = [0 if rng.random() < 0.05 else _ctx(rng, 9000) for _ in range(b)]
        ctx[0] = max(ctx[0], 1)
        ta.check_append(wl.make_case(f"random_a{i}", "decode", 7000 + i, ctx, hq, hkv))
    else:
        q = int(rng.integers(1, min(32 // g, 8) + 1))
        b = int(rng.integers(1, 12))
        ctx = [max(q, _ctx(rng, 6000)) for _ in range(b)]
        tm.check(wl.make_case(f"random_m{i}", "prefill", 7000 + i, ctx, hq, hkv, q_lens=[q] * b), q)
