"""Test-side helpers for the GPU parity tests: read the prepared tensors out
of a workspace (restating the pack layouts documented in include/oc_attn.h),
read the attention kernel's parity-aid dump, validate its running-max
decisions, and run the oracle on the same inputs."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def head64(t, b, h):
    """[S,128] float64 numpy slice of a [B,S,H,128] tensor (any device)."""
    return t[b, :, h].double().cpu().numpy()


def _key_col(j):
    j = np.asarray(j)
    return 32 * ((j >> 2) & 3) + 4 * (j >> 4) + (j & 3)


def _opidx(row, col):
    """byte offset of (row, col) in a 128x128 tile stored in MFMA operand
    order: chunk c = col // 16 of row r is 16-byte chunk
    (2*(r//16) + c%2)*64 + 16*(c//2) + r%16 of the tile"""
    row, col = np.asarray(row), np.asarray(col)
    c = col >> 4
    lane = ((c >> 1) << 4) | (row & 15)
    return ((((row >> 4) << 1) | (c & 1)) * 64 + lane) * 16 + (col & 15)


def unpack_k(tiles: np.ndarray, S: int) -> np.ndarray:
    """kpack bytes of one head [nT*16384] -> key codes [S, 128]."""
    nT = tiles.size // 16384
    t = tiles.reshape(nT, 16384)
    off = _opidx(np.arange(128)[:, None], np.arange(128)[None, :])   # [key, channel]
    return t[:, off].reshape(nT * 128, 128)[:S]


def unpack_v(tiles: np.ndarray, S: int) -> np.ndarray:
    """vpack bytes of one head [nT*16384] -> value codes [S, 128]."""
    nT = tiles.size // 16384
    t = tiles.reshape(nT, 16384)
    off = _opidx(np.arange(128)[None, :], _key_col(np.arange(128))[:, None])   # [key, d]
    return t[:, off].reshape(nT * 128, 128)[:S]


class WsView:
    """numpy views of one prepared workspace."""

    def __init__(self, prep):
        self.prep = prep
        self.L = prep.plan.layout
        self.B, self.S, self.H, _ = prep.shape
        self.raw = prep.ws.cpu().numpy()

    def _arr(self, off, dtype, count):
        nb = np.dtype(dtype).itemsize * count
        return self.raw[off:off + nb].view(dtype)

    def bh(self, b, h):
        return b * self.H + h

    def qcodes(self, b, h):
        n = self.L.s_pad_q * 128
        a = self._arr(self.L.qhat + self.bh(b, h) * n, np.uint8, n)
        return a.reshape(self.L.s_pad_q, 128)

    def sq(self, b, h):
        n = self.L.s_pad_q // 128
        return self._arr(self.L.sq + 4 * self.bh(b, h) * n, np.float32, n)

    def kcodes(self, b, h):
        n = self.L.n_ktiles * 16384
        return unpack_k(self._arr(self.L.kpack + self.bh(b, h) * n, np.uint8, n), self.S)

    def sk(self, b, h):
        n = self.L.n_ktiles
        return self._arr(self.L.sk + 4 * self.bh(b, h) * n, np.float32, n)

    def vcodes(self, b, h):
        n = self.L.n_ktiles * 16384
        return unpack_v(self._arr(self.L.vpack + self.bh(b, h) * n, np.uint8, n), self.S)

    def vraw(self, b, h):
        n = self.L.n_ktiles * 16384
        return self._arr(self.L.vpack + self.bh(b, h) * n, np.uint8, n)

    def sv(self, b, h):
        return self._arr(self.L.sv + 8 * self.bh(b, h), np.float32, 2)

    # repair set (packed with the actual count k)
    def sel(self, b, h, k):
        return self._arr(self.L.sel + 4 * self.bh(b, h) * k, np.int32, k)

    def rcodes(self, b, h, k):
        nts = math.ceil(k / 128)
        n = nts * 16384
        return unpack_v(self._arr(self.L.rpack + self.bh(b, h) * n, np.uint8, n), k)

    def kselcodes(self, b, h, k):
        nts = math.ceil(k / 128)
        n = nts * 16384
        return unpack_k(self._arr(self.L.kselpack + self.bh(b, h) * n, np.uint8, n), k)

    def sksel(self, b, h, k):
        n = math.ceil(k / 128) * 128
        return self._arr(self.L.sksel + 4 * self.bh(b, h) * n, np.float32, n)

    def sr(self, b, h):
        return self._arr(self.L.sr + 8 * self.bh(b, h), np.float32, 2)

    def vmu(self, b, h):
        n = self.L.n_ktiles * 128
        return self._arr(self.L.vmu + 2 * n * self.bh(b, h), np.uint16, n).reshape(self.L.n_ktiles, 128)

    def kmean(self, b, h):
        return self._arr(self.L.kmean + 4 * 128 * self.bh(b, h), np.float32, 128)

    def energy(self, b, h):
        return self._arr(self.L.energy + 8 * self.bh(b, h) * self.S, np.float64, self.S)


def oracle_rows(q, k, v, b, h, rows, budget=0.0, tau=None, order="mid", m_trace=None, weights="expcast",
                k_smooth=False, v_smooth=False, code_trace=None, rcode_trace=None):
    """oracle output rows for one (b, h), in the single-pass form the kernel
    computes (key tiles from the middle of the window outwards), plus the
    prepared head; m_trace replays given running-max decisions and
    code_trace / rcode_trace given byte decisions; weights "exp_cast" is the
    comparison byte path"""
    qh, kh, vh = head64(q, b, h), head64(k, b, h), head64(v, b, h)
    return oracle.expcast_attention_online(qh, kh, vh, tau=tau, rows=rows, budget=budget, order=order,
                                           m_trace=m_trace, weights=weights, k_smooth=k_smooth, v_smooth=v_smooth,
                                           code_trace=code_trace, rcode_trace=rcode_trace)


def out_rows(out, b, h, rows):
    return out[b, :, h].float().cpu().numpy()[np.asarray(rows)].astype(np.float64)


TOL = 5e-3
# With every floating-point decision replayed (validated running maxima and
# bytes), what is left between kernel and oracle is the kernel's arithmetic:
# the BF16 rounding of the output (at most 2^-8 relative per element, about
# 1.7e-3 rel-L2 on these outputs) and its fp32 accumulation of P V and the
# row sums (below 1e-4, test_error_decomposition). This bar sits above their
# sum with margin.
TOL_REPLAYED = 2.5e-3
# oracle byte path -> the kernel's name for it
KERNEL_WEIGHTS = {"expcast": "expcast", "exp_cast": "exp_fp8"}


def _oc():
    import bit_fp8_attention_block_amd as oc
    return oc


def logit_error_bound(ph, rows, tau):
    """Worst-case difference between the kernel's log2-logit and the exact one:
    the FP8 MFMA's summation error, bounded by 2^-10 of the largest possible
    product max|q| * max|k| (test_gpu_mfma_precision checks that bound on the
    hardware, on adversarial and workload data), plus fp32 rounding of the
    sum (128 * 2^-24 * sum |products|) and of the three scale products and
    the FMA (a few ulp of the logit)."""
    qd = np.abs(oracle.decode(ph.qc[np.asarray(rows)]))
    kd = np.abs(oracle.decode(ph.kc))
    sqr = ph.sq[np.asarray(rows) // 128].astype(np.float64)
    skk = ph.sk[np.arange(ph.S) // 128].astype(np.float64)
    scale = (tau / math.log(2)) * (sqr[:, None] * skk[None, :])
    mag = scale * (qd @ kd.T)
    top = scale * np.outer(qd.max(axis=1), kd.max(axis=1))
    return mag * (128 * 2.0 ** -24) + mag * 2.0 ** -20 + top * 2.0 ** -10


def check_max_trace(trace, x, bound, order="mid"):
    """Validate every running-max decision the kernel made for these rows.

    trace[i, t] is the max the kernel wrote tile t's bytes against (by tile
    number); x the exact log2-logits, bound their worst-case kernel error.
    Visiting the tiles in the kernel's order, each entry must be
    max(previous entry, ceil(m)) for some tile max m the kernel could have
    seen: m between the largest (x - bound) and the largest (x + bound) of
    the tile. So entries never decrease, equal the exact decision wherever
    the tile's largest logit is further than the bound from an integer, and
    elsewhere may differ only toward the side such a rounding reaches.
    Returns the number of rows with at least one such tie-broken entry."""
    n, nT = trace.shape
    S = x.shape[1]
    tiles = oracle.key_tile_order(nT) if order == "mid" else list(range(nT))
    prev = np.full(n, -np.inf)
    tie = np.zeros(n, dtype=bool)
    for t in tiles:
        sl = slice(t * 128, min(S, t * 128 + 128))
        lo = np.ceil((x[:, sl] - bound[:, sl]).max(axis=1))
        hi = np.ceil((x[:, sl] + bound[:, sl]).max(axis=1))
        exact = np.maximum(prev, np.ceil(x[:, sl].max(axis=1)))
        got = trace[:, t].astype(np.float64)
        ok = (got >= np.maximum(prev, lo)) & (got <= np.maximum(prev, hi))
        bad = np.nonzero(~ok)[0]
        assert len(bad) == 0, (f"tile {t}: row {bad[0]} kernel max {got[bad[0]]}, previous {prev[bad[0]]}, "
                               f"allowed [{max(prev[bad[0]], lo[bad[0]])}, {max(prev[bad[0]], hi[bad[0]])}]")
        tie |= got != exact
        prev = got
    return int(tie.sum())


# the kernel's own rounding beyond the logit error bound, in log2-logit
# units: its unorm16 conversion takes the FMA's operands divided by 65535
# (about 2^-24 relative of a byte value below 128), its comparison path a
# hardware exp2 (a few ulp); both far below this
CODE_EPS = 1e-5


def validated_codes(kc, x, M, bound, weights="expcast"):
    """Check the kernel's bytes kc for exact log2-logits x against running
    maxima M (all [rows, keys]): each must be a byte that some logit within
    the kernel's logit error bound (plus CODE_EPS) of the exact one gives,
    i.e. lie between the oracle's bytes for x - bound and x + bound (bytes
    rise with the logit on both byte paths). Where the bound is below the
    distance to a rounding boundary that is the oracle's own byte; near a
    boundary it is one of the two codes either side; for logits far from
    zero, whose fp32 value can be off by more than a binade, it is a wider
    range. Returns ([rows, keys] array holding the kernel's byte where it
    differs from the oracle's own and -1 elsewhere, their number)."""
    codes_of = oracle.expcast_codes if weights == "expcast" else oracle.exp_cast_codes
    own = codes_of(x, M).astype(np.int64)
    kc = np.asarray(kc).astype(np.int64)
    trace = np.full(kc.shape, -1, dtype=np.int64)
    idx = np.nonzero(kc != own)
    if len(idx[0]) == 0:
        return trace, 0
    a, xi, Mi, bi = kc[idx], x[idx], M[idx], bound[idx] + CODE_EPS
    lo = codes_of((xi - bi)[None, :], Mi[None, :])[0].astype(np.int64)
    hi = codes_of((xi + bi)[None, :], Mi[None, :])[0].astype(np.int64)
    ok = (lo <= a) & (a <= hi)
    if not ok.all():
        i = int(np.nonzero(~ok)[0][0])
        raise AssertionError(f"byte at (row {idx[0][i]}, key {idx[1][i]}): kernel {a[i]}, oracle {own[idx][i]}, "
                             f"logits within the bound {bi[i]:.3e} give bytes {lo[i]}..{hi[i]}")
    trace[idx] = a
    return trace, len(a)


def kernel_dump(prep, b, h, rows, out=None, weights="expcast", with_repair=False, **want):
    """The parity-aid dump for one (b, h) and the given rows, as numpy arrays.
    With `out` (the output of the production call on the same inputs), the
    dump variant's own output for that (b, h) must equal it bit for bit: it
    then took the same decisions as the kernel whose output is compared."""
    oc = _oc()
    d = oc.debug_pcodes(prep, b, h, rows=np.asarray(rows), weights=KERNEL_WEIGHTS.get(weights, weights),
                        with_repair=with_repair, **want)
    torch.cuda.synchronize()
    if out is not None:
        assert torch.equal(d.out[b, :, h], out[b, :, h]), "dump variant and production kernel disagree"
    for f in ("codes", "m_used", "scores", "rcodes", "out_f32"):
        t = getattr(d, f)
        if t is not None:
            setattr(d, f, t.cpu().numpy())
    return d


def validated_trace(q, k, v, prep, b, h, rows, out=None, budget=0.0, tau=None, order="mid", weights="expcast",
                    k_smooth=False, v_smooth=False):
    """The kernel's running-max decisions for `rows` of (b, h), after
    check_max_trace has accepted every one of them; (trace, tie rows)."""
    d = kernel_dump(prep, b, h, rows, out=out, weights=weights, with_repair=budget > 0, codes=False)
    own = oracle_rows(q, k, v, b, h, rows, budget=budget, tau=tau, order=order, weights=weights,
                      k_smooth=k_smooth, v_smooth=v_smooth)
    t = tau if tau else 1 / math.sqrt(128)
    x = oracle.log2_logits(own["ph"], rows, t)
    ties = check_max_trace(d.m_used, x, logit_error_bound(own["ph"], rows, t), order)
    return d.m_used, ties


def replayed_decisions(q, k, v, prep, b, h, rows, out=None, budget=0.0, tau=None, order="mid", weights="expcast",
                       k_smooth=False, v_smooth=False):
    """The kernel's running-max and byte decisions for `rows` of (b, h), read
    from the parity-aid dump and each validated (check_max_trace,
    validated_codes) before the oracle may replay it. Where floating point
    decides an integer (the bit-aligned max, a byte), the two sides then take
    the decision in the same precision, the kernel's, wherever the exact
    value is within the kernel's rounding of the boundary; everywhere else
    the oracle's exact decision must be the kernel's. (How many bytes differ
    is bounded by the byte-parity tests on the workloads, not here: on
    inputs whose logits sit far from zero, the fp32 logits of a whole row
    can lie within rounding of a boundary.)"""
    d = kernel_dump(prep, b, h, rows, out=out, weights=weights, with_repair=budget > 0, codes=True)
    own = oracle_rows(q, k, v, b, h, rows, budget=budget, tau=tau, order=order, weights=weights,
                      k_smooth=k_smooth, v_smooth=v_smooth)
    t = tau if tau else 1 / math.sqrt(128)
    ph = own["ph"]
    x = oracle.log2_logits(ph, rows, t)
    bound = logit_error_bound(ph, rows, t)
    ties = check_max_trace(d.m_used, x, bound, order)
    S = x.shape[1]
    Mk = d.m_used[:, np.arange(S) // 128].astype(np.float64)
    ct, nb = validated_codes(d.codes, x, Mk, bound, weights)
    n = ct.size
    rct = None
    if budget > 0 and ph.repair is not None and ph.repair.k > 0:
        sel = np.asarray(ph.repair.sel)
        Mf = np.repeat(d.m_used.max(axis=1).astype(np.float64)[:, None], len(sel), axis=1)
        rct, nr = validated_codes(d.rcodes, x[:, sel], Mf, bound[:, sel], weights)
        nb += nr
        n += rct.size
    return {"m_trace": d.m_used, "ties": ties, "code_trace": ct, "rcode_trace": rct, "nbytes": nb, "n": n,
            "own": own}


def compare(q, k, v, out, pairs, rows, budget=0.0, tol=TOL, label="", order="mid", prep=None, weights="expcast",
            k_smooth=False, v_smooth=False, tau=None):
    """rel-L2 of the kernel's rows against the single-pass oracle. With a
    prepared workspace (of the same inputs and options), the oracle replays
    the running-max and byte decisions the kernel made where the exact value
    is within the kernel's rounding of a boundary, each validated first
    (replayed_decisions), and the dump's output must equal `out` bit for
    bit. The error against the oracle's own decisions is reported beside it."""
    errs, two, own_errs = [], [], []
    nflip = nbyte = nall = 0
    kw = dict(budget=budget, tau=tau, order=order, weights=weights, k_smooth=k_smooth, v_smooth=v_smooth)
    for b, h in pairs:
        got = out_rows(out, b, h, rows)
        if prep is not None:
            rp = replayed_decisions(q, k, v, prep, b, h, rows, out=out, **kw)
            nflip += rp["ties"]
            nbyte += rp["nbytes"]
            nall += rp["n"]
            r = oracle_rows(q, k, v, b, h, rows, m_trace=rp["m_trace"], code_trace=rp["code_trace"],
                            rcode_trace=rp["rcode_trace"], **kw)
            own_errs.append(oracle.rel_l2(got, rp["own"]["out"]))
        else:
            r = oracle_rows(q, k, v, b, h, rows, **kw)
        e = oracle.rel_l2(got, r["out"])
        errs.append(e)
        if prep is not None:
            assert e <= TOL_REPLAYED, (label, b, h, e, "with every decision replayed")
        r2 = oracle.expcast_attention_head(head64(q, b, h), head64(k, b, h), head64(v, b, h), tau=tau, rows=rows,
                                           ph=r["ph"], weights=weights)
        two.append(oracle.rel_l2(got, r2["out"]))
        assert np.isfinite(got).all()
        assert e <= tol, (label, b, h, e)
    log(f"  {label}: rel-L2 vs oracle (single-pass form) max {max(errs):.2e}; vs two-pass form max {max(two):.2e}"
        + (f"; against the oracle's own decisions max {max(own_errs):.2e}; rows with a tie-broken max {nflip}; "
           f"bytes taken the kernel's way {nbyte} of {nall}" if prep is not None else ""))
    return errs
