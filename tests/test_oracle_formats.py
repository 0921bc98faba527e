"""Pins of the oracle's other expert formats: fp4 experts with UE8M0 block scales
(MXFP4, "colibri 开发演进实录" §五 and §六) and int3-g64 ("colibri 开发演进实录" §8.3).

Checked against the E2M1 table (tests/golden/e2m1.txt), hand-built int3 rows whose codes
follow from the bit layout by inspection, and exact identities with the int4-gs64 path
(itself pinned in test_oracle_pins.py): a matrix whose codes and scales are expressible
in both formats must give the same FFN output bit for bit.  CPU only.
"""
import math
import os

import numpy as np
import pytest

import oracle as R
from routed_int4_expert_amd import synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_table():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "e2m1.txt")) if ln.strip() and ln[0] != "#"]
    assert len(rows) == 16
    for code, val in rows:
        got = R.e2m1(int(code, 16))
        assert got == float(val) and math.copysign(1.0, got) == math.copysign(1.0, float(val)), code


def test_ue8m0():
    assert R.ue8m0(127) == 1.0 and R.ue8m0(128) == 2.0 and R.ue8m0(126) == 0.5
    assert R.ue8m0(0) == 2.0 ** -127 and R.ue8m0(254) == 2.0 ** 127
    assert math.isnan(R.ue8m0(255))


def _int3_row(low_bytes=None, sign_bytes=None, K=64):
    row = np.zeros(3 * K // 8, np.uint8)
    for i, v in (low_bytes or {}).items():
        row[i] = v
    for i, v in (sign_bytes or {}).items():
        row[K // 4 + i] = v
    return row


def test_int3_hand_rows():
    K = 64
    # nothing set: every code 0
    row = _int3_row()
    assert all(R.int3_code(row, K, k) == 0 for k in range(K))
    # all low bits set, no sign bit: every code 3
    row = _int3_row({i: 0xFF for i in range(16)})
    assert all(R.int3_code(row, K, k) == 3 for k in range(K))
    # only sign bits: every code -4
    row = _int3_row(sign_bytes={i: 0xFF for i in range(8)})
    assert all(R.int3_code(row, K, k) == -4 for k in range(K))
    # both: every code -1
    row = _int3_row({i: 0xFF for i in range(16)}, {i: 0xFF for i in range(8)})
    assert all(R.int3_code(row, K, k) == -1 for k in range(K))
    # low-plane byte 5 = word 1, byte 1; bits 2-3 = pair 1 = (a 0, o 1): element
    # 16*1 + 8*0 + 2*1 + 1 = 19, low bits 01 -> code 1
    row = _int3_row({5: 0b0100})
    assert [k for k in range(K) if R.int3_code(row, K, k) != 0] == [19]
    assert R.int3_code(row, K, 19) == 1
    # sign-plane byte 6 = word 1, byte 2; bit 5 = (m 2, o 1): element 32 + 16 + 4 + 1 = 53
    row = _int3_row(sign_bytes={6: 1 << 5})
    assert [k for k in range(K) if R.int3_code(row, K, k) != 0] == [53]
    assert R.int3_code(row, K, 53) == -4
    # second group (K = 128): low-plane byte 16 + 0 (word 0, byte 0), bits 0-1 = 10 -> element 64: 2;
    # its sign plane starts at K/4 + 8 = 40; byte 0 bit 0 -> element 64 as well: 2 - 4 = -2
    row = _int3_row({16: 0b10}, K=128)
    assert [k for k in range(128) if R.int3_code(row, 128, k) != 0] == [64]
    assert R.int3_code(row, 128, 64) == 2
    row[32 + 8] = 1
    assert R.int3_code(row, 128, 64) == -2


def _pack_int3(codes):
    """Test-side encoder of int3 codes [N][K] into the bit-plane rows (its own loops
    over the element index, from the layout the library states)."""
    N, K = codes.shape
    q = np.zeros((N, 3 * K // 8), np.uint8)
    for n in range(N):
        for k in range(K):
            G, i = divmod(k, 64)
            u = int(codes[n, k]) & 7
            low, sgn = u & 3, u >> 2
            d, r = divmod(i, 16)
            a, r = divmod(r, 8)
            b, o = divmod(r, 2)
            q[n, 16 * G + 4 * d + b] |= low << (2 * (2 * a + o))
            h, r = divmod(i, 32)
            m, r = divmod(r, 8)
            q[n, K // 4 + 8 * G + 4 * h + b] |= sgn << (2 * m + o)
    return q


def _pack_int4(codes):
    c = codes.astype(np.int64) & 15
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def _two_format_layer(fmt, H, F, E, seed):
    """A layer in `fmt` and the int4-gs64 layer with the same weights (exactly)."""
    rng = np.random.default_rng(seed)
    mats = {}
    for nm, (N, K) in (("gate", (F, H)), ("up", (F, H)), ("down", (H, F))):
        qa, sa, q4, s4 = [], [], [], []
        for _ in range(E + 1):  # E routed experts and the shared one
            if fmt == R.FMT_INT3:
                c = rng.integers(-4, 4, size=(N, K))
                sc = (rng.uniform(0.5, 1.5, size=(N, K // 64)) / 64).astype(np.float32)
                qa.append(_pack_int3(c)); sa.append(sc)
                q4.append(_pack_int4(c)); s4.append(sc)
            else:
                # E2M1 codes whose doubled value 2v is an int4 code: every code but +4 and +-6
                allowed = np.array([0, 1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13, 14], np.int64)
                cf = rng.choice(allowed, size=(N, K))
                two_v = np.array([int(2 * R.e2m1(int(x))) for x in range(16)])[cf]
                eg = rng.integers(118, 126, size=(N, K // 64))   # one exponent per 64-group
                e32 = np.repeat(eg, 2, axis=1).astype(np.uint8)  # both 32-blocks share it
                qa.append((cf[:, 0::2] | (cf[:, 1::2] << 4)).astype(np.uint8)); sa.append(e32)
                q4.append(_pack_int4(two_v)); s4.append((2.0 ** (eg - 128)).astype(np.float32))
        mats[nm] = (qa, sa, q4, s4)
    base = dict(hidden=H, n_experts=E, ffn=F, shared_ffn=F, top_k=2, top_p=0.0, norm_topk=1,
                routed_scale=1.5)
    rw = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
    rb = rng.uniform(-0.1, 0.1, size=E).astype(np.float32)
    da = dict(base, router_w=rw, router_bias=rb, expert_fmt=fmt)
    d4 = dict(base, router_w=rw, router_bias=rb, expert_fmt=R.FMT_INT4)
    for nm, (qa, sa, q4, s4) in mats.items():
        da[nm + "_q"], da[nm + "_s"] = np.stack(qa[:E]), np.stack(sa[:E])
        da["sh_" + nm + "_q"], da["sh_" + nm + "_s"] = qa[E], sa[E]
        d4[nm + "_q"], d4[nm + "_s"] = np.stack(q4[:E]), np.stack(s4[:E])
        d4["sh_" + nm + "_q"], d4["sh_" + nm + "_s"] = q4[E], s4[E]
    return da, d4


@pytest.mark.parametrize("fmt", [R.FMT_INT3, R.FMT_MXFP4])
def test_format_equals_int4_on_shared_values(fmt):
    """Weights representable in both formats: dequantised matrices, expert rows and the
    layer output equal the int4-gs64 oracle's exactly."""
    H, F, E, T = 128, 64, 4, 5
    da, d4 = _two_format_layer(fmt, H, F, E, seed=7 + fmt)
    for nm in ("gate", "up", "down"):
        K = H if nm != "down" else F
        for e in range(E):
            wa = R.dequantize(fmt, da[nm + "_q"][e], da[nm + "_s"][e], K)
            w4 = R.dequantize(R.FMT_INT4, d4[nm + "_q"][e], d4[nm + "_s"][e], K)
            np.testing.assert_array_equal(wa, w4)
    La, L4 = R.Layer(da), R.Layer(d4)
    x = np.random.default_rng(3).standard_normal((T, H)).astype(np.float32)
    np.testing.assert_array_equal(R.layer_forward(La, x), R.layer_forward(L4, x))
    ids, _, keff = R.route(La, x)
    u = R.union(E, ids, keff)
    np.testing.assert_array_equal(R.expert_ffn(La, x, u["off"], u["row_tok"]),
                                  R.expert_ffn(L4, x, u["off"], u["row_tok"]))


def test_mxfp4_block_scales_are_per_32():
    """Two 32-blocks of one 64-group with different exponents: element k uses block k//32."""
    K = 64
    q = np.full((1, K // 2), 0x22, np.uint8)  # every element E2M1 code 2 = 1.0
    e = np.array([[127 + 3, 127 - 2]], np.uint8)
    w = R.dequantize(R.FMT_MXFP4, q, e, K)
    np.testing.assert_array_equal(w[0, :32], np.full(32, 8.0))
    np.testing.assert_array_equal(w[0, 32:], np.full(32, 0.25))
    # nibble order: byte j holds element 2j low, 2j+1 high
    q = np.zeros((1, K // 2), np.uint8)
    q[0, 3] = 0x7 | (0xF << 4)  # element 6: +6, element 7: -6
    w = R.dequantize(R.FMT_MXFP4, q, np.full((1, 2), 127, np.uint8), K)
    assert w[0, 6] == 6.0 and w[0, 7] == -6.0 and np.count_nonzero(w) == 2
    # an exponent byte of 255 is NaN for its block only
    w = R.dequantize(R.FMT_MXFP4, np.full((1, K // 2), 0x22, np.uint8), np.array([[255, 127]], np.uint8), K)
    assert np.isnan(w[0, :32]).all() and (w[0, 32:] == 1.0).all()


@pytest.mark.parametrize("fmt", [S.FMT_INT3, S.FMT_MXFP4])
def test_generator_round_trip(fmt):
    """The synthetic quantisers and the oracle's decoders read the same layout: every
    decoded weight is within the format's rounding bound of the fp32 draw."""
    N, K, std = 16, 256, 0.02
    q, s = S.q_normal(fmt, 0, "fmt_round_trip", N, K, std)
    w = R.dequantize(fmt, q, s, K)
    ref = S.normal_f32(0, "fmt_round_trip", (N, K), std=std).astype(np.float64)
    if fmt == S.FMT_INT3:
        step = np.repeat(s.astype(np.float64), 64, axis=1)        # amax/3
        bound = 0.5 * step * (1 + 1e-6)
    else:
        blk = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
        # E2M1 spacing is at most 2 (between 4 and 6) in units of the block scale, and the
        # block's largest magnitude is below 8 units, so it saturates by at most 2 units
        bound = 2.0 * blk
    assert (np.abs(w - ref) <= bound).all()
    # and the codes carry information: the decoded matrix correlates with the draw
    assert np.corrcoef(w.ravel(), ref.ravel())[0, 1] > 0.9


def test_mxfp4_nan_scale_propagates_to_the_output():
    H, F, E = 64, 64, 2
    da, _ = _two_format_layer(R.FMT_MXFP4, H, F, E, seed=1)
    da["sh_gate_s"] = da["sh_gate_s"].copy()
    da["sh_gate_s"][0, 0] = 255
    x = np.ones((1, H), np.float32)
    out = R.layer_forward(R.Layer(da), x)
    assert np.isnan(out).all()  # h[0] is NaN and the down projection spreads it
