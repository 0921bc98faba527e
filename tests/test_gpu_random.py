"""A seeded sweep of random layer configurations through the whole path, on the GPU.

Each case draws its hyper-parameters (widths, expert count, top-k, token count, top-p,
norm_topk, routed scale, bias, expert format and sometimes group-limited routing) from a
fixed seed and compares routing, union, expert rows and the layer output (fp32 and bf16)
with the oracle, as the hand-picked shapes of test_gpu_parity do.  The sizes keep the
oracle's work small; every selection, union and expert-FFN path is reached by some case
(T = 1, 2-4, 5-8, 9-16 and larger; 16- and 32-row items; partial K chunks and output
blocks).
"""
import numpy as np
import pytest

from routed_int4_expert_amd import synth as S

from test_gpu_parity import full_parity, say

pytestmark = pytest.mark.gpu

N_CASES = 160


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    while True:
        H = pick([64, 128, 192, 256, 320, 448, 512, 1024, 1344, 2048])
        F = pick([64, 128, 192, 256, 384, 512])
        Fs = pick([0, 64, 128, 256, 320])
        E = pick([4, 8, 12, 16, 24, 32, 48, 64, 96, 128, 200, 256])
        k = int(rng.integers(1, min(E, 16) + 1))
        T = pick([1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17, 24, 33, 40, 64, 65, 100, 129, 300, 513, 1000])
        if T * k * H * F <= 4e8:
            break
    fmt = pick([S.FMT_INT4, S.FMT_INT4, S.FMT_MXFP4, S.FMT_INT3])
    kw = dict(hidden=H, n_experts=E, ffn=F, shared_ffn=Fs, top_k=k, tokens=T,
              top_p=pick([0.0, 0.0, 0.5, 0.8, 0.95, 1.0]), norm_topk=pick([0, 1]),
              routed_scale=pick([1.0, 2.5]), bias_amp=pick([0.0, 0.05, 0.3]),
              router_std=pick([0.5, 1.0, 2.0]) / np.sqrt(H), expert_fmt=fmt)
    groups = None
    # group-limited routing where the expert count allows it: n_group | E, at least two
    # experts per group, n_group <= 64, topk_group groups holding at least k experts
    cands = [g for g in (2, 4, 8, 16) if E % g == 0 and E // g >= 2]
    if cands and rng.random() < 0.3:
        g = pick(cands)
        tg = int(rng.integers(1, g + 1))
        if tg * (E // g) >= k:
            groups = (g, tg)
    return kw, groups


CASES = [_draw(i) for i in range(N_CASES)]


def _name(i):
    kw, groups = CASES[i]
    g = f"_g{groups[0]}of{groups[1]}" if groups else ""
    return (f"r{i}_H{kw['hidden']}F{kw['ffn']}s{kw['shared_ffn']}E{kw['n_experts']}k{kw['top_k']}"
            f"T{kw['tokens']}_{S.FMT_NAMES[kw['expert_fmt']]}{g}")


@pytest.mark.parametrize("i", range(N_CASES), ids=[_name(i) for i in range(N_CASES)])
def test_random_configuration(i):
    kw, groups = CASES[i]
    sh = S.custom(_name(i), **kw)
    d = S.make_layer(sh, seed=i)
    if groups:
        d.update(n_group=groups[0], topk_group=groups[1])
    x = S.make_batch(sh, d, seed=i)
    say(f"random case {_name(i)}")
    full_parity(sh, d, x)
