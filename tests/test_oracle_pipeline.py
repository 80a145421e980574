"""Pins for the whole oracle pipeline: pure-Python brute force on tiny
inputs, closed-form special cases, and the reduction to textbook softmax
attention (checked against torch's SDPA in float64 on the CPU)."""
import math
import struct

import numpy as np
import pytest
import torch

import oracle
import workloads

TAU = 1 / math.sqrt(128)
LOG2E = 1 / math.log(2)


def _dec(c):
    """E4M3 byte -> value, straight from the format (bias 7, 3 mantissa bits)."""
    s = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 0xF, c & 7
    return s * (m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8))


def _enc(y):
    """nearest E4M3 byte by exhaustive search over the 127 magnitudes
    (ties to the even code, saturating)."""
    a = abs(y)
    best, bestd = 0, math.inf
    for c in range(127):
        d = abs(_dec(c) - a)
        if d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best | (0x80 if math.copysign(1.0, y) < 0 else 0)


def _scales(amax):
    if amax < 2.0 ** -100:            # all-zero and tiny blocks: unit scale, every code 0
        return np.float32(1), np.float32(1)
    a = np.float32(amax)
    return np.float32(a / np.float32(448)), np.float32(np.float32(448) / a)


def _bf16(x):
    """fp32 value -> nearest bf16 value, ties to even, by its bit pattern"""
    u = struct.unpack("<I", struct.pack("<f", float(np.float32(x))))[0]
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def brute_force(q, k, v, tau=TAU, k_smooth=False, v_smooth=False):
    """ExpCast attention with explicit loops over tokens, channels and keys.
    k_smooth: subtract the mean key (exact sum by math.fsum, divided by S,
    rounded to fp32; fp32 subtraction) before the K blocks are quantized.
    v_smooth: quantize each value minus its 128-token block mean (bf16 of the
    fp32 mean) and add the means back weighted by each block's weight sum."""
    S, D = len(k), len(k[0])
    if k_smooth:
        kbar = [np.float32(math.fsum(k[i][c] for i in range(S)) / S) for c in range(D)]
        k = [[float(np.float32(k[i][c]) - kbar[c]) for c in range(D)] for i in range(S)]
    mu = None
    if v_smooth:
        mu = []
        for b0 in range(0, S, 128):
            blk = range(b0, min(S, b0 + 128))
            mu.append([_bf16(math.fsum(v[i][c] for i in blk) / len(blk)) for c in range(D)])
        v = [[float(np.float32(v[i][c]) - np.float32(mu[i // 128][c])) for c in range(D)] for i in range(S)]
    qc, kc, sq, sk = [None] * S, [None] * S, [0.0] * S, [0.0] * S
    for x, codes, sc in ((q, qc, sq), (k, kc, sk)):
        for b0 in range(0, S, 128):
            blk = range(b0, min(S, b0 + 128))
            s, inv = _scales(max(abs(x[i][c]) for i in blk for c in range(D)))
            for i in blk:
                codes[i] = [_enc(float(np.float32(x[i][c]) * inv)) for c in range(D)]
                sc[i] = float(s)
    sv, invv = _scales(max(abs(v[i][c]) for i in range(S) for c in range(D)))
    vd = [[float(sv) * _dec(_enc(float(np.float32(v[i][c]) * invv))) for c in range(D)] for i in range(S)]
    out, Ms, Ls = [], [], []
    for i in range(S):
        xs = []
        for j in range(S):
            dot = sum(_dec(qc[i][c]) * _dec(kc[j][c]) for c in range(D))
            xs.append(tau * LOG2E * dot * (sq[i] * sk[j]))
        M = math.ceil(max(xs))
        w = [_dec(min(126, max(0, round(8 * (xj - M) + 120 - 0.35)))) for xj in xs]
        L = sum(w)
        row = [sum(w[j] * vd[j][c] for j in range(S)) for c in range(D)]
        if mu is not None:
            for t in range(len(mu)):
                lt = sum(w[j] for j in range(128 * t, min(S, 128 * t + 128)))
                row = [row[c] + lt * mu[t][c] for c in range(D)]
        out.append([x / L for x in row])
        Ms.append(M)
        Ls.append(L)
    return np.array(out), np.array(Ms), np.array(Ls)


@pytest.mark.parametrize("S", [1, 2, 3, 17, 129, 130])
def test_brute_force_matches_vectorized(S):
    q, k, v = (t[0, :, 0].double().numpy() for t in workloads.random_qkv(1, S, 1, seed=S, scale=1.5))
    # give the blocks different ranges so per-block scales differ
    q = q * np.where(np.arange(S) < 128, 1.0, 3.0)[:, None]
    k = k * np.where(np.arange(S) < 128, 2.0, 0.5)[:, None]
    q, k = (torch.from_numpy(t).bfloat16().double().numpy() for t in (q, k))
    o_ref, M_ref, L_ref = brute_force(q.tolist(), k.tolist(), v.tolist())
    r = oracle.expcast_attention_head(q, k, v)
    assert np.array_equal(r["M"], M_ref)
    np.testing.assert_allclose(r["L"], L_ref, rtol=1e-14)
    np.testing.assert_allclose(r["out"], o_ref, rtol=1e-12, atol=1e-12)


def test_single_key_gives_its_dequantized_value():
    q, k, v = (t[0, :, 0].double().numpy() for t in workloads.random_qkv(1, 1, 1, seed=5))
    r = oracle.expcast_attention_head(q, k, v)
    ph = r["ph"]
    np.testing.assert_allclose(r["out"][0], float(ph.sv) * oracle.decode(ph.vc[0]), rtol=1e-15)


def test_identical_keys_give_mean_of_dequantized_values():
    S = 300
    q, k, v = (t[0, :, 0].double().numpy() for t in workloads.random_qkv(1, S, 1, seed=6))
    k[:] = k[0]
    r = oracle.expcast_attention_head(q, k, v, rows=[0, 150, 299])
    ph = r["ph"]
    mean = float(ph.sv) * oracle.decode(ph.vc).mean(axis=0)
    np.testing.assert_allclose(r["out"], np.tile(mean, (3, 1)), rtol=1e-12, atol=1e-14)


def test_dominant_key_gives_its_dequantized_value():
    """When one key's log2-logit exceeds all others by more than 15.1, every
    other weight underflows to byte 0."""
    S = 200
    rng = np.random.default_rng(2)
    q = np.zeros((S, 128))
    q[:, 0] = 12.0
    k = rng.normal(0, 0.05, (S, 128))
    k[77, 0] = 12.0
    v = rng.normal(0, 1, (S, 128))
    q, k, v = (torch.from_numpy(t).bfloat16().double().numpy() for t in (q, k, v))
    r = oracle.expcast_attention_head(q, k, v, rows=[0, 5, 199])
    ph = r["ph"]
    want = float(ph.sv) * oracle.decode(ph.vc[77])
    np.testing.assert_allclose(r["out"], np.tile(want, (3, 1)), rtol=1e-15)


def test_reduces_to_softmax_attention_without_codec_and_expcast():
    """Codec switched to identity and ExpCast to exact weights: the oracle's
    plumbing (row max, weights, row sum, value product) must be softmax
    attention, as torch's SDPA computes it in float64."""
    S = 333
    q, k, v = (t[0, :, 0].double().numpy() for t in workloads.random_qkv(1, S, 1, seed=9, scale=2.0))
    r = oracle.expcast_attention_head(q, k, v, quantize=False, weights="exp")
    t = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a)[None, None] for a in (q, k, v)), scale=TAU)[0, 0].numpy()
    np.testing.assert_allclose(r["out"], t, rtol=1e-10, atol=1e-12)
    ex = oracle.exact_attention_head(q, k, v)
    np.testing.assert_allclose(ex, t, rtol=1e-10, atol=1e-12)


def test_key_block_permutation_invariance():
    """Non-causal attention does not depend on the order of whole 128-key
    blocks (moved together with their values and scales)."""
    S = 512
    q, k, v = (t[0, :, 0].double().numpy() for t in workloads.random_qkv(1, S, 1, seed=10))
    perm = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in (2, 0, 3, 1)])
    rows = [0, 100, 511]
    a = oracle.expcast_attention_head(q, k, v, rows=rows)["out"]
    b = oracle.expcast_attention_head(q, k[perm], v[perm], rows=rows)["out"]
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_block_scales_are_per_128_tokens():
    S = 260
    x = np.ones((S, 128))
    x[:128] *= 2.0
    x[128:256] *= 0.25
    x[256:] *= 7.0
    codes, scales = oracle.quantize_blocks(x)
    np.testing.assert_array_equal(scales, np.float32([2 / 448, 0.25 / 448, 7 / 448]))
    assert np.all(codes == 0x7E)
    z, s = oracle.quantize_blocks(np.zeros((5, 128)))
    assert s[0] == 1.0 and np.all(z == 0)


def test_error_vs_exact_on_small_workload():
    """rel-L2 of the faithful method vs exact float64 attention on the
    i.i.d. N(0,1) workload (about 5.5%; a parity-unpinned level, checked for
    being in a sane range only)."""
    q, k, v = workloads.make_inputs("s1024_h2")
    errs = []
    for h in range(2):
        qh, kh, vh = (t[0, :, h].double().numpy() for t in (q, k, v))
        rows = np.arange(0, 1024, 8)
        o = oracle.expcast_attention_head(qh, kh, vh, rows=rows)["out"]
        ex = oracle.exact_attention_head(qh, kh, vh, rows=rows)
        errs.append(oracle.rel_l2(o, ex))
    assert all(0.04 < e < 0.07 for e in errs), errs


# ---- the single-pass (online) form --------------------------------------

def _pairwise(xs):
    """pairwise summation by recursive halving"""
    if len(xs) == 1:
        return xs[0]
    h = len(xs) // 2
    return _pairwise(xs[:h]) + _pairwise(xs[h:])


def brute_force_online(q, k, v, order, tau=TAU, weights="expcast", budget=0.0):
    """Online ExpCast attention with explicit loops: key tiles of 128 in the
    given order, running integer max raised before each tile's bytes, running
    sums multiplied by 2**(M_old - M_new). weights="exp_cast" takes each byte
    as the E4M3 cast of the fp32 weight 2**(x - M + 8) instead. With a budget,
    the ceil(budget*S) tokens whose fp32 residual v - sv*dec(v_hat) has the
    largest energy (sum of squares, pairwise; ties to the lower index) get
    their E4M3-quantized residual added to the value after the last tile,
    weighted by bytes against the final max, with the row sum unchanged."""
    S, D = len(k), len(k[0])
    qc, kc, sq, sk = [None] * S, [None] * S, [0.0] * S, [0.0] * S
    for x, codes, sc in ((q, qc, sq), (k, kc, sk)):
        for b0 in range(0, S, 128):
            blk = range(b0, min(S, b0 + 128))
            s, inv = _scales(max(abs(x[i][c]) for i in blk for c in range(D)))
            for i in blk:
                codes[i] = [_enc(float(np.float32(x[i][c]) * inv)) for c in range(D)]
                sc[i] = float(s)
    sv, invv = _scales(max(abs(v[i][c]) for i in range(S) for c in range(D)))
    vd = [[_dec(_enc(float(np.float32(v[i][c]) * invv))) for c in range(D)] for i in range(S)]
    sel, rd, sr = [], [], 0.0
    kk = math.ceil(budget * S - 1e-9) if budget > 0 else 0
    if kk:
        res = [[np.float32(np.float32(v[j][c]) - np.float32(sv) * np.float32(vd[j][c])) for c in range(D)]
               for j in range(S)]
        energy = [_pairwise([float(x) * float(x) for x in res[j]]) for j in range(S)]
        sel = sorted(sorted(range(S), key=lambda j: (-energy[j], j))[:kk])
        sr, invr = _scales(max(abs(float(res[j][c])) for j in sel for c in range(D)))
        rd = [[_dec(_enc(float(np.float32(res[j][c]) * invr))) for c in range(D)] for j in sel]
    out = []
    for i in range(S):
        M, L, O = None, 0.0, [0.0] * D
        for t in order:
            keys = range(128 * t, min(S, 128 * t + 128))
            xs = {}
            for j in keys:
                dot = sum(_dec(qc[i][c]) * _dec(kc[j][c]) for c in range(D))
                xs[j] = tau * LOG2E * dot * (sq[i] * sk[j])
            Mt = math.ceil(max(xs.values()))
            if M is None or Mt > M:
                f = 0.0 if M is None else 2.0 ** (M - Mt)
                L, O = L * f, [o * f for o in O]
                M = Mt
            for j in keys:
                if weights == "expcast":
                    w = _dec(min(126, max(0, round(8 * (xs[j] - M) + 120 - 0.35))))
                else:
                    w = _dec(_enc(float(np.float32(2.0 ** (xs[j] - M + 8)))))
                L += w
                for c in range(D):
                    O[c] += w * vd[j][c]
        O = [float(sv) * o for o in O]
        for n, j in enumerate(sel):
            dot = sum(_dec(qc[i][c]) * _dec(kc[j][c]) for c in range(D))
            xj = tau * LOG2E * dot * (sq[i] * sk[j])
            if weights == "expcast":
                w = _dec(min(126, max(0, round(8 * (xj - M) + 120 - 0.35))))
            else:
                w = _dec(_enc(float(np.float32(2.0 ** (xj - M + 8)))))
            for c in range(D):
                O[c] += float(sr) * w * rd[n][c]
        out.append([o / L for o in O])
    return np.array(out)


def test_key_tile_order_is_mid_window():
    assert oracle.key_tile_order(1) == [0]
    assert oracle.key_tile_order(2) == [0, 1]
    assert oracle.key_tile_order(5) == [2, 1, 3, 0, 4]
    assert oracle.key_tile_order(6) == [2, 1, 3, 0, 4, 5]
    for n in (1, 7, 64, 574):
        assert sorted(oracle.key_tile_order(n)) == list(range(n))


@pytest.mark.parametrize("S,budget", [(130, 0.0), (300, 0.0), (130, 0.05), (300, 0.3)])
def test_online_brute_force_matches_vectorized(S, budget):
    q, k, v = (t[0, :, 0].double().numpy() for t in workloads.random_qkv(1, S, 1, seed=S + 1, scale=2.0))
    # a strong key late in the order so the running max has to grow
    k[S - 1] = q[3] * 1.5
    k = torch.from_numpy(k).bfloat16().double().numpy()
    rows = [0, 3, 77, S - 1]
    nT = -(-S // 128)
    for order, name in ((oracle.key_tile_order(nT), "mid"), (list(range(nT)), "ascending")):
        want = brute_force_online(q.tolist(), k.tolist(), v.tolist(), order, budget=budget)[rows]
        got = oracle.expcast_attention_online(q, k, v, rows=rows, order=name, budget=budget)["out"]
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    if budget:
        # the repair term is resolved: it moves the output far above the tolerance used here
        plain = oracle.expcast_attention_online(q, k, v, rows=rows)["out"]
        assert np.abs(plain - got).max() > 1e-4


@pytest.mark.parametrize("S", [2, 17, 130])
def test_k_smoothing_brute_force_matches_vectorized(S):
    q, k, v = (t[0, :, 0].double().numpy() for t in workloads.random_qkv(1, S, 1, seed=S + 11, scale=2.0))
    k = torch.from_numpy(k + 5.0 * np.sin(np.arange(128))[None, :]).bfloat16().double().numpy()   # channel bias
    rows = [0, S - 1]
    want = brute_force(q.tolist(), k.tolist(), v.tolist(), k_smooth=True)[0][rows]
    got = oracle.expcast_attention_head(q, k, v, rows=rows, k_smooth=True)["out"]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("S", [2, 130])
def test_v_smoothing_brute_force_matches_vectorized(S):
    q, k, v = (t[0, :, 0].double().numpy() for t in workloads.random_qkv(1, S, 1, seed=S + 13, scale=2.0))
    v = torch.from_numpy(v + 4.0 * np.cos(np.arange(128))[None, :]).bfloat16().double().numpy()
    rows = [0, S - 1]
    want = brute_force(q.tolist(), k.tolist(), v.tolist(), v_smooth=True)[0][rows]
    got = oracle.expcast_attention_head(q, k, v, rows=rows, v_smooth=True)["out"]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    online = oracle.expcast_attention_online(q, k, v, rows=rows, v_smooth=True)["out"]
    np.testing.assert_allclose(online, want, rtol=1e-9, atol=1e-10)


def test_v_smoothing_is_exact_for_blockwise_constant_values():
    """When every token of a block has the same value vector, the block mean
    is that vector and the residuals are zero, so the value path is exact:
    the output is the ExpCast weights applied to the unquantized values."""
    rng = np.random.default_rng(8)
    S = 300
    blocks = rng.integers(-40, 40, size=(3, 128)) / 8.0          # bf16-exact
    v = blocks[np.arange(S) // 128]
    q = torch.from_numpy(rng.normal(size=(S, 128))).bfloat16().double().numpy()
    k = torch.from_numpy(rng.normal(size=(S, 128))).bfloat16().double().numpy()
    rows = np.arange(0, S, 7)
    r = oracle.expcast_attention_head(q, k, v, rows=rows, v_smooth=True)
    x = oracle.log2_logits(r["ph"], rows, TAU)
    P = oracle.VALUES[oracle.expcast_codes(x, oracle.bitaligned_row_max(x))]
    np.testing.assert_allclose(r["out"], (P @ v) / P.sum(axis=1, keepdims=True), rtol=1e-13, atol=1e-13)
    plain = oracle.expcast_attention_head(q, k, v, rows=rows)["out"]
    assert np.abs(plain - r["out"]).max() > 1e-3       # the plain path rounds V to E4M3


def test_v_smoothing_lowers_error_on_channel_biased_values():
    rng = np.random.default_rng(9)
    S = 1024
    q, k = rng.normal(size=(S, 128)), rng.normal(size=(S, 128))
    v = rng.normal(size=(S, 128)) + rng.normal(0, 5, size=128)
    q, k, v = (torch.from_numpy(t).bfloat16().double().numpy() for t in (q, k, v))
    rows = np.arange(0, S, 4)
    exact = oracle.exact_attention_head(q, k, v, rows=rows)
    plain = oracle.rel_l2(oracle.expcast_attention_head(q, k, v, rows=rows)["out"], exact)
    smooth = oracle.rel_l2(oracle.expcast_attention_head(q, k, v, rows=rows, v_smooth=True)["out"], exact)
    assert smooth < 0.8 * plain, (plain, smooth)


def test_v_smoothing_with_full_repair_restores_the_values():
    """Budget 1 repairs every residual: the value path error falls to the
    second-order quantization of the residual of the residual."""
    q, k, v = (t[0, :, 0].double().numpy() for t in workloads.random_qkv(1, 256, 1, seed=21, scale=2.0))
    rows = np.arange(0, 256, 5)
    ph = oracle.prepare_head(q, k, v, budget=1.0, v_smooth=True)
    x = oracle.log2_logits(ph, rows, TAU)
    P = oracle.VALUES[oracle.expcast_codes(x, oracle.bitaligned_row_max(x))]
    ideal = (P @ v) / P.sum(axis=1, keepdims=True)
    got = oracle.expcast_attention_head(q, k, v, rows=rows, ph=ph)["out"]
    assert oracle.rel_l2(got, ideal) < 2e-3


def test_k_smoothing_removes_a_shared_key_offset_exactly():
    """Keys with zero mean plus a per-channel offset: smoothing takes the
    offset off exactly, so codes and scales equal those of the offset-free
    keys, and the outputs agree to rounding (softmax ignores a per-row
    shift of the scores)."""
    rng = np.random.default_rng(5)
    S = 256
    u = rng.integers(1, 8, size=(S // 2, 128)) / 8.0
    k0 = np.empty((S, 128))
    k0[0::2], k0[1::2] = u, -u                        # every column sums to zero
    c = rng.integers(-9, 10, size=128).astype(np.float64)
    k = k0 + c                                        # exact in bf16 (at most 8 significant bits)
    assert np.array_equal(torch.from_numpy(k).bfloat16().double().numpy(), k)
    q = torch.from_numpy(rng.normal(size=(S, 128))).bfloat16().double().numpy()
    v = torch.from_numpy(rng.normal(size=(S, 128))).bfloat16().double().numpy()
    np.testing.assert_array_equal(oracle.key_mean(k), c.astype(np.float32))
    a = oracle.prepare_head(q, k, v, k_smooth=True)
    b = oracle.prepare_head(q, k0, v)
    np.testing.assert_array_equal(a.kc, b.kc)
    np.testing.assert_array_equal(a.sk, b.sk)
    # without smoothing the offset changes the K codes
    assert not np.array_equal(oracle.prepare_head(q, k, v).kc, b.kc)


def test_k_smoothing_lowers_error_on_biased_keys():
    """A large per-channel key bias wastes the FP8 range of every K block;
    removing the mean brings the error against exact attention down."""
    rng = np.random.default_rng(6)
    S = 1024
    q = rng.normal(size=(S, 128)) + rng.normal(0, math.sqrt(3), size=128)
    k = rng.normal(size=(S, 128)) + rng.normal(0, math.sqrt(3), size=128)
    v = rng.normal(size=(S, 128))
    q, k, v = (torch.from_numpy(t).bfloat16().double().numpy() for t in (q, k, v))
    rows = np.arange(0, S, 4)
    exact = oracle.exact_attention_head(q, k, v, rows=rows)
    plain = oracle.rel_l2(oracle.expcast_attention_head(q, k, v, rows=rows)["out"], exact)
    smooth = oracle.rel_l2(oracle.expcast_attention_head(q, k, v, rows=rows, k_smooth=True)["out"], exact)
    assert smooth < 0.8 * plain, (plain, smooth)


@pytest.mark.parametrize("S", [3, 130])
def test_online_exp_cast_brute_force_matches_vectorized(S):
    """The comparison path (exponential, fp32, then E4M3 cast) in the online
    form against explicit loops."""
    q, k, v = (t[0, :, 0].double().numpy() for t in workloads.random_qkv(1, S, 1, seed=S + 7, scale=2.0))
    k[S - 1] = q[1] * 1.5
    k = torch.from_numpy(k).bfloat16().double().numpy()
    rows = [0, 1, S - 1]
    nT = -(-S // 128)
    want = brute_force_online(q.tolist(), k.tolist(), v.tolist(), oracle.key_tile_order(nT), weights="exp_cast")[rows]
    got = oracle.expcast_attention_online(q, k, v, rows=rows, weights="exp_cast")["out"]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    # the two paths write different bytes, so the outputs differ
    other = oracle.expcast_attention_online(q, k, v, rows=rows)["out"]
    assert np.abs(other - got).max() > 1e-6


def test_exp_cast_path_tracks_exact_weights_closer_than_expcast():
    """Both byte paths approximate 256*2^(x - M); the exponential path is a
    plain rounding (ratio within 1 -+ 1/17), ExpCast a shifted one (ratio in
    [0.929, 1.075]), so the exp path's total variation is the smaller."""
    rng = np.random.default_rng(3)
    x = rng.normal(0.0, 2.0, size=(64, 512))
    M = np.ceil(x.max(axis=1))
    exact = np.exp2(x - M[:, None])
    exact /= exact.sum(axis=1, keepdims=True)
    for codes, bound in ((oracle.exp_cast_codes(x, M), 1 / 17), (oracle.expcast_codes(x, M), 0.0746)):
        w = oracle.VALUES[codes]
        normal = codes >= 8
        ratio = w[normal] / (256.0 * np.exp2(x - M[:, None])[normal])
        assert np.all(np.abs(ratio - 1) <= bound + 1e-12)
    tv = lambda c: 0.5 * np.abs(oracle.VALUES[c] / oracle.VALUES[c].sum(axis=1, keepdims=True) - exact).sum(axis=1)  # noqa: E731
    assert tv(oracle.exp_cast_codes(x, M)).mean() < tv(oracle.expcast_codes(x, M)).mean()


@pytest.mark.parametrize("budget", [0.0, 0.02, 0.3, 1.0])
def test_online_equals_two_pass_when_max_is_visited_first(budget):
    """If every row's largest logit lies in the first tile visited, all bytes
    are written against the final max and both forms coincide, the repair
    term of the single-pass form (bytes of the selected keys against the
    final max, unrepaired row sums) included."""
    S = 700
    rng = np.random.default_rng(4)
    q = rng.normal(0, 1, (S, 128))
    k = rng.normal(0, 1, (S, 128))
    c = oracle.key_tile_order(-(-S // 128))[0]
    q[:, 0] += 6.0
    k[c * 128 + 7, 0] = 30.0          # the dominant key sits in the middle tile
    v = rng.normal(0, 1, (S, 128))
    q, k, v = (torch.from_numpy(t).bfloat16().double().numpy() for t in (q, k, v))
    rows = np.arange(0, S, 5)
    a = oracle.expcast_attention_online(q, k, v, rows=rows, budget=budget)
    b = oracle.expcast_attention_head(q, k, v, rows=rows, budget=budget)
    np.testing.assert_array_equal(a["M"], b["M"])
    np.testing.assert_allclose(a["L"], b["L"], rtol=1e-13)
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-14)


def test_online_and_two_pass_differ_only_through_the_underflow_tail():
    """Relative to the final max, weights that land in the normal E4M3 range
    are identical in both forms; the forms differ by at most the tail."""
    q, k, v = workloads.make_inputs("s8192_h8", S=2048, H=1)
    qh, kh, vh = (t[0, :, 0].double().numpy() for t in (q, k, v))
    rows = np.arange(0, 2048, 64)
    a = oracle.expcast_attention_online(qh, kh, vh, rows=rows, order="ascending")
    b = oracle.expcast_attention_head(qh, kh, vh, rows=rows)
    np.testing.assert_array_equal(a["M"], b["M"])
    x = oracle.log2_logits(b["ph"], rows, TAU)
    tail = np.where(x - b["M"][:, None] < -14.0, np.exp2(x - b["M"][:, None] + 8), 0.0).sum(axis=1)
    vmax = float(b["ph"].sv) * np.abs(oracle.decode(b["ph"].vc)).max()
    bound = 2.0 * tail * vmax / b["L"]            # |dO| <= (tail mass difference) * max|v| / L, both forms
    dO = np.abs(a["out"] - b["out"]).max(axis=1)
    assert np.all(dO <= bound + 1e-12)


def test_online_replays_a_max_trace():
    """Feeding the single-pass form its own running-max sequence reproduces
    it exactly; raising every entry by one only moves weights that sit in the
    underflow tail (bytes shift by 8, normal values by exact factors of 2)."""
    q, k, v = workloads.make_inputs("s8192_h8", S=1500, H=1)
    qh, kh, vh = (t[0, :, 0].double().numpy() for t in (q, k, v))
    rows = np.arange(0, 1500, 37)
    a = oracle.expcast_attention_online(qh, kh, vh, rows=rows)
    b = oracle.expcast_attention_online(qh, kh, vh, rows=rows, m_trace=a["m_trace"])
    np.testing.assert_array_equal(a["out"], b["out"])
    c = oracle.expcast_attention_online(qh, kh, vh, rows=rows, m_trace=a["m_trace"] + 1)
    assert oracle.rel_l2(c["out"], a["out"]) < 0.05
    np.testing.assert_array_equal(c["M"], a["M"] + 1)


@pytest.mark.parametrize("weights", ["expcast", "exp_cast"])
def test_online_replays_bytes(weights):
    """code_trace / rcode_trace: all entries negative (or the form's own
    bytes) reproduce it exactly; replacing single bytes gives, on a one-tile
    sequence, the weighted mean written out directly with those bytes
    (O = sv * (sum_j dec(c_j) v_j + sr * sum_sel dec(r_j) r_j) / sum_j dec(c_j))."""
    S = 120
    q, k, v = workloads.make_inputs("s8192_h8", S=S, H=1)
    qh, kh, vh = (t[0, :, 0].double().numpy() for t in (q, k, v))
    rows = np.arange(0, S, 7)
    budget = 0.05
    a = oracle.expcast_attention_online(qh, kh, vh, rows=rows, weights=weights, budget=budget)
    ph = a["ph"]
    k_sel = ph.repair.k
    none = np.full((len(rows), S), -1)
    b = oracle.expcast_attention_online(qh, kh, vh, rows=rows, weights=weights, ph=ph, code_trace=none,
                                        rcode_trace=np.full((len(rows), k_sel), -1))
    np.testing.assert_array_equal(a["out"], b["out"])
    x = oracle.log2_logits(ph, rows, TAU)
    M = oracle.bitaligned_row_max(x)
    codes_of = oracle.expcast_codes if weights == "expcast" else oracle.exp_cast_codes
    own = codes_of(x, M).astype(np.int64)
    rown = codes_of(x[:, ph.repair.sel], M).astype(np.int64)
    c = oracle.expcast_attention_online(qh, kh, vh, rows=rows, weights=weights, ph=ph, code_trace=own,
                                        rcode_trace=rown)
    np.testing.assert_array_equal(a["out"], c["out"])
    # one byte per row moved by one code (the row's largest weight), and one repair byte
    mod = own.copy()
    j = np.argmax(x, axis=1)
    mod[np.arange(len(rows)), j] -= 1
    rmod = rown.copy()
    rmod[:, 0] = np.minimum(rmod[:, 0] + 1, 126)
    d = oracle.expcast_attention_online(qh, kh, vh, rows=rows, weights=weights, ph=ph,
                                        code_trace=np.where(np.arange(S)[None, :] == j[:, None], mod, -1),
                                        rcode_trace=np.where(np.arange(k_sel)[None, :] == 0, rmod, -1))
    dec = lambda c_: np.array([_dec(int(z)) for z in np.ravel(c_)]).reshape(np.shape(c_))  # noqa: E731
    vd = dec(ph.vc)
    rd = dec(ph.repair.rc)
    P, R = dec(mod), dec(rmod)
    want = (float(ph.sv) * (P @ vd) + float(ph.repair.sr) * (R @ rd)) / P.sum(axis=1)[:, None]
    np.testing.assert_allclose(d["out"], want, rtol=1e-12, atol=0)
    assert oracle.rel_l2(d["out"], a["out"]) > 1e-3
