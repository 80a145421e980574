"""ExpCast FP8 attention, step by step, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's CPU
baseline may import this module; the GPU library shares no code with it.

Sources (the pages this follows):
  * Open VC Attention product page (ailibri.com), API paragraph: multi-head
    forward attention, head dim 128, FP16/BF16 inputs [B,S,H,128], the call
    quantizes to FP8 itself and returns BF16.
  * same page, kernel paragraph: softmax weights are written to FP8 straight
    from the scores; Q and K carry per-block scales, V a per-head scale; keys
    are visited from the middle of the window.
  * VC-Attention write-up (Nunchux AI), section "ExpCast-FP8": an E4M3 byte
    read as an integer is about 8*log2(v)+56, so the byte is produced from the
    log-domain score with one fused multiply-add; beta = -0.35 centres the
    rounding error; the result equals the exp-then-cast byte on 79.6% of
    entries and is otherwise one code away; per-row total variation < 3.64%
    plus any underflow tail.
  * Open-VC news (aikraft.ru), section "Решение: ExpCast и отказ от экспонент",
    and the product page, repair paragraph: V-residual repair adds back the
    quantized residual of the worst-rounded value tokens, chosen by residual
    energy, with a token budget (0.005 in the example).

Readings where the pages leave a step open:
  * weights are stored as 256*p, p = 2^(x - M) relative to the row max, so the
    code is 8*(x - M) + 120 + beta; the largest weight lands on code 120.
  * the byte is the round-to-nearest-even of that affine value, clamped to the
    finite codes [0, 126]; keys beyond S get no code.
  * M is the bit-aligned row max: M = ceil(max_j x_j), an integer. The
    two-pass form (expcast_attention_head) uses the final M for every key;
    the single-pass form (expcast_attention_online) follows the kernel the
    pages describe: key tiles of 128 from the middle of the key window
    outwards, bytes relative to the running M, exact power-of-two rescales.
  * the row sum is over the decoded weights: L = sum_j dec(c_j).
  * Q/K scale blocks are 128 tokens x 128 channels; scale s = amax/448 in fp32,
    quantization multiplies by the fp32 reciprocal 448/amax; a block whose
    amax is below 2^-100 (an all-zero block included) gets s = 1 and so
    codes 0.
  * K-mean smoothing (an option, off by default; the VC-Attention write-up,
    section on why attention is the bottleneck, names Q/K smoothing as prior
    practice): before the K blocks are quantized, every key loses the mean key
    of its (batch, head), k' = fp32(k - kbar) with kbar = fp32(sum_j k_j / S)
    per channel. q.k' = q.k - q.kbar shifts each score row by a constant, which
    softmax ignores.
  * V-Smooth block means (an option, off by default; VC-Attention write-up,
    section "V-Smooth", without its k-means grouping): every 128-token block
    of V loses its mean, mu_t = bf16(fp32(sum_j v_j / n_t)) per channel over
    the block's n_t tokens (sum in float64); the residuals fp32(v - mu_t) are
    quantized with the per-head scale in place of v; the output adds the means
    back with each key tile's row sum: O_i = (sv * sum_j P_ij dec(r_j) +
    sum_t l_it mu_t) / L_i, l_it = sum over tile t of P_ij. With repair, the
    repaired residual is taken of fp32(v - mu_t) in place of v.
  * repair: residual r = v - sv*dec(v_hat) in fp32; energy = sum over the 128
    channels of r^2 in float64, added pairwise up a balanced binary tree in
    channel order (residual_energy); the top
    k = ceil(budget*S) tokens by energy (ties to the lower index) are repaired
    with an E4M3 residual carrying its own per-head scale; the row sums L are
    left unchanged. The budget is a float64 fraction of the tokens.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .e4m3 import VALUES, decode, encode

BETA = -0.35
CODE_OF_PMAX = 120.0     # E4M3 code of 256 = 2^8 (8*8 + 56): where a weight of 1 lands
QK_BLOCK = 128
LOG2E = 1.0 / math.log(2.0)
F32 = np.float32


# A block (or head, or repair set) whose amax lies below this is quantized with
# the unit scale, like an all-zero block: 448/amax would otherwise approach
# the top of the fp32 range (and overflow below about 1.3e-36), while every
# element rounds to code 0 under the unit scale anyway.
SCALE_FLOOR = 2.0 ** -100


def quant_scale(amax: float):
    """fp32 dequantization scale s = amax/448 and quantization multiplier
    inv = 448/amax, both correctly rounded fp32 divisions. amax below
    2^-100 (zero included) -> (1, 1)."""
    a = F32(amax)
    if a < F32(SCALE_FLOOR):
        return F32(1.0), F32(1.0)
    return F32(a / F32(448.0)), F32(F32(448.0) / a)


def quantize_with(x: np.ndarray, inv) -> np.ndarray:
    """E4M3 codes of fp32(x * inv) (x must be exact in fp32)."""
    y = x.astype(F32) * F32(inv)               # fp32 product, round to nearest even
    return encode(y.astype(np.float64))


def quantize_blocks(x: np.ndarray, block: int = QK_BLOCK):
    """Per-block quantization of one head's [S, 128] tensor: one scale per
    `block` consecutive tokens (over all 128 channels)."""
    S = x.shape[0]
    nblk = (S + block - 1) // block
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(nblk, dtype=F32)
    for i in range(nblk):
        sl = slice(i * block, min(S, (i + 1) * block))
        s, inv = quant_scale(np.abs(x[sl]).max())
        scales[i] = s
        codes[sl] = quantize_with(x[sl], inv)
    return codes, scales


def quantize_head(x: np.ndarray):
    """One scale for the whole head's [S, 128] tensor."""
    s, inv = quant_scale(np.abs(x).max())
    return quantize_with(x, inv), s


@dataclass
class RepairSet:
    k: int
    sel: np.ndarray          # selected token indices, ascending
    energy: np.ndarray       # float64 residual energy of every token
    rc: np.ndarray           # E4M3 codes of the selected residuals [k, 128]
    sr: np.float32           # residual dequantization scale


@dataclass
class PreparedHead:
    qc: np.ndarray
    sq: np.ndarray           # per 128-token block
    kc: np.ndarray
    sk: np.ndarray
    vc: np.ndarray
    sv: np.float32
    repair: RepairSet | None = field(default=None)
    vmean: np.ndarray | None = field(default=None)   # V-Smooth: [n_blocks, 128] block means (bf16 values)

    @property
    def S(self):
        return self.kc.shape[0]


def repair_count(budget: float, S: int) -> int:
    """k = ceil(budget * S) in float64, with a 1e-9 allowance so that a budget
    such as 0.05 of 600 tokens gives 30 despite binary rounding; capped at S."""
    b = float(budget)
    if not (0.0 <= b <= 1.0):
        raise ValueError("budget must lie in [0, 1]")
    return max(0, min(S, int(math.ceil(b * S - 1e-9))))


def residual_energy(r: np.ndarray) -> np.ndarray:
    """Per token, the sum over the 128 channels of r^2 in float64, added by
    pairwise summation in channel order: neighbouring channels first, then
    neighbouring pairs, and so on up a balanced binary tree (seven levels).
    Each square of an fp32 residual is exact in float64, so only the order of
    the additions decides the rounding, and this order fixes it."""
    e = r.astype(np.float64) ** 2
    if e.shape[1] & (e.shape[1] - 1):
        raise ValueError("the channel count must be a power of two")
    while e.shape[1] > 1:
        e = e[:, 0::2] + e[:, 1::2]
    return e[:, 0]


def repair_select(v: np.ndarray, vc: np.ndarray, sv, budget: float) -> RepairSet:
    """Rank value tokens by the energy of their quantization residual and
    quantize the residual of the top-k tokens."""
    S = v.shape[0]
    k = repair_count(budget, S)
    t = F32(sv) * decode(vc).astype(F32)       # fp32 product sv*dec(v_hat)
    r = v.astype(F32) - t                      # fp32 residual
    energy = residual_energy(r)
    order = np.lexsort((np.arange(S), -energy))  # energy descending, then index ascending
    sel = np.sort(order[:k])
    if k == 0:
        return RepairSet(0, sel, energy, np.zeros((0, v.shape[1]), np.uint8), F32(1.0))
    rs = r[sel]
    sr, inv = quant_scale(np.abs(rs).max())
    return RepairSet(k, sel, energy, quantize_with(rs, inv), sr)


def key_mean(k: np.ndarray) -> np.ndarray:
    """fp32 mean key over the S tokens, per channel: the float64 sum divided by
    S, rounded to fp32 (the sum of bf16/fp16 values is exact in float64 unless
    a channel spans more than about 28 binades)."""
    return (k.sum(axis=0) / k.shape[0]).astype(F32)


def smooth_keys(k: np.ndarray) -> np.ndarray:
    """K-mean smoothing: fp32(k - kbar), returned as float64."""
    return (k.astype(F32) - key_mean(k)).astype(np.float64)


def to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values -> nearest bf16 values (round to nearest even), as float64."""
    u = np.asarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(F32).astype(np.float64)


def value_block_means(v: np.ndarray, block: int = QK_BLOCK) -> np.ndarray:
    """V-Smooth block means [n_blocks, 128]: bf16(fp32(sum / n)) over each
    block's tokens, the sum in float64."""
    S = v.shape[0]
    n = (S + block - 1) // block
    mu = np.empty((n, v.shape[1]))
    for t in range(n):
        blk = v[t * block:min(S, (t + 1) * block)]
        mu[t] = to_bf16((blk.sum(axis=0) / blk.shape[0]).astype(F32))
    return mu


def smooth_values(v: np.ndarray, mu: np.ndarray, block: int = QK_BLOCK) -> np.ndarray:
    """fp32(v - mu of the token's block), as float64."""
    m = mu[np.arange(v.shape[0]) // block]
    return (v.astype(F32) - m.astype(F32)).astype(np.float64)


def prepare_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, budget: float = 0.0,
                 k_smooth: bool = False, v_smooth: bool = False) -> PreparedHead:
    """Quantize one (batch, head) slice; inputs are float64 [S, 128] holding
    bf16/fp16-exact values. k_smooth subtracts the mean key first; v_smooth
    quantizes V as block-mean residuals."""
    qc, sq = quantize_blocks(q)
    kc, sk = quantize_blocks(smooth_keys(k) if k_smooth else k)
    mu = value_block_means(v) if v_smooth else None
    vv = smooth_values(v, mu) if v_smooth else v
    vc, sv = quantize_head(vv)
    rep = repair_select(vv, vc, sv, budget) if budget > 0 else None
    return PreparedHead(qc, sq, kc, sk, vc, sv, rep, mu)


def log2_logits(ph: PreparedHead, rows, tau: float) -> np.ndarray:
    """x_ij = tau*log2(e) * sq(i)*sk(j) * <dec(q_hat_i), dec(k_hat_j)> for the
    given query rows against every key. The dot products of decoded E4M3
    values are exact in float64 (each product has at most 8 significant bits
    between 2^-18 and 2^18, so every partial sum of 128 fits in 53 bits)."""
    rows = np.asarray(rows)
    qd = decode(ph.qc[rows])
    kd = decode(ph.kc)
    dots = qd @ kd.T
    sqr = ph.sq[rows // QK_BLOCK].astype(np.float64)
    skk = ph.sk[np.arange(ph.S) // QK_BLOCK].astype(np.float64)
    return (tau * LOG2E) * dots * (sqr[:, None] * skk[None, :])


def bitaligned_row_max(x: np.ndarray) -> np.ndarray:
    """M_i = ceil(max_j x_ij) as an integer."""
    return np.ceil(x.max(axis=1)).astype(np.int64)


def expcast_codes(x: np.ndarray, M, beta: float = BETA) -> np.ndarray:
    """ExpCast byte: round-to-nearest-even of 8*(x - M) + 120 + beta, clamped
    to the finite E4M3 codes [0, 126]."""
    M = np.asarray(M, dtype=np.float64)
    if M.ndim == 1:
        M = M[:, None]
    y = 8.0 * (x - M) + CODE_OF_PMAX + beta
    return np.clip(np.rint(y), 0, 126).astype(np.uint8)


def exp_cast_codes(x: np.ndarray, M) -> np.ndarray:
    """The path ExpCast replaces: weight 256*2^(x-M) computed in fp32, then
    cast to E4M3 with round-to-nearest-even."""
    M = np.asarray(M, dtype=np.float64)
    if M.ndim == 1:
        M = M[:, None]
    w = np.exp2(x - M + 8.0).astype(F32).astype(np.float64)
    return encode(w)


def expcast_attention_head(q, k, v, tau=None, rows=None, budget=0.0, ph=None,
                           quantize=True, weights="expcast", chunk=512, k_smooth=False, v_smooth=False):
    """Output rows of ExpCast attention for one (batch, head) slice.

    q, k, v: float64 [S, 128]. Returns a dict with the float64 output rows
    `out`, the row maxima `M`, row sums `L` and the prepared head `ph`.

    quantize=False skips the FP8 codec (unit scales, raw values);
    weights="exp" uses the exact weights 2^(x - M) instead of ExpCast bytes,
    and weights="exp_cast" the E4M3 cast of the fp32 weight 256*2^(x - M)
    (the path ExpCast replaces, exp_cast_codes). With the codec and the
    weights both switched off the result is textbook softmax attention.
    """
    S, D = k.shape
    tau = 1.0 / math.sqrt(D) if tau is None else tau
    rows = np.arange(S) if rows is None else np.asarray(rows)
    if ph is None:
        if quantize:
            ph = prepare_head(q, k, v, budget, k_smooth=k_smooth, v_smooth=v_smooth)
        else:
            ones = lambda n: np.ones(n, dtype=F32)  # noqa: E731
            ph = PreparedHead(None, ones((S + QK_BLOCK - 1) // QK_BLOCK), None,
                              ones((S + QK_BLOCK - 1) // QK_BLOCK), None, F32(1.0))
    vd = decode(ph.vc) if quantize else v
    out = np.empty((len(rows), D))
    Ms = np.empty(len(rows), dtype=np.int64)
    Ls = np.empty(len(rows))
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        if quantize:
            x = log2_logits(ph, r, tau)
        else:
            x = (tau * LOG2E) * (q[r] @ k.T)
        M = bitaligned_row_max(x)
        if weights == "expcast":
            P = VALUES[expcast_codes(x, M)]
        elif weights == "exp_cast":
            P = VALUES[exp_cast_codes(x, M)]
        elif weights == "exp":
            P = np.exp2(x - M[:, None])
        else:
            raise ValueError(weights)
        L = P.sum(axis=1)
        acc = float(ph.sv) * (P @ vd)
        if quantize and ph.vmean is not None:
            acc += P @ ph.vmean[np.arange(S) // QK_BLOCK]     # the block means, weighted by the row sums
        if quantize and ph.repair is not None and ph.repair.k > 0:
            rp = ph.repair
            acc += float(rp.sr) * (P[:, rp.sel] @ decode(rp.rc))
        out[c0:c0 + len(r)] = acc / L[:, None]
        Ms[c0:c0 + len(r)] = M
        Ls[c0:c0 + len(r)] = L
    return {"out": out, "M": Ms, "L": Ls, "ph": ph}


def key_tile_order(n_tiles: int) -> list:
    """Order in which the online form visits the 128-key tiles: from the
    middle of the key window outwards, c, c-1, c+1, c-2, c+2, ... with
    c = (n_tiles-1)//2, continuing on the longer side once the shorter one
    is used up (Open VC Attention product page, kernel paragraph; Open-VC
    news, "Архитектурные оптимизации")."""
    c = (n_tiles - 1) // 2
    order = [c]
    for d in range(1, n_tiles):
        if c - d >= 0:
            order.append(c - d)
        if c + d < n_tiles:
            order.append(c + d)
    return order


def expcast_attention_online(q, k, v, tau=None, rows=None, budget=0.0, ph=None, order="mid", chunk=256,
                             m_trace=None, weights="expcast", k_smooth=False, v_smooth=False, code_trace=None,
                             rcode_trace=None):
    """Single-pass (flash) form of ExpCast attention, as the pages' kernel runs
    it: keys are consumed in 128-key tiles in `order` ("mid" = key_tile_order,
    "ascending" = 0, 1, 2, ...). Per row, a running bit-aligned max M is raised
    to ceil(max logit of the tile) before that tile's bytes are written, so
    bytes are relative to the running max. The partial sums O and L are
    carried across tiles and multiplied by the exact power of two
    2^(M_old - M_new) whenever M grows. The repair residuals use the final M.

    It equals expcast_attention_head except for keys whose byte relative to
    the final max would fall below the normal E4M3 range (the underflow tail):
    those are kept more precisely when they were visited before the max.

    m_trace, if given, is an integer array [len(rows), n_tiles] holding, by
    tile number, the running max to use for that tile's bytes instead of the
    one computed here (to replay another implementation's max decisions,
    which can differ where a tile's largest logit is within rounding of an
    integer). The rescale factors then follow from consecutive entries.

    code_trace, if given, is an integer array [len(rows), S]: where an entry
    is non-negative, that byte is used for (row, key) instead of the one
    computed here; rcode_trace [len(rows), k] does the same for the repair
    residuals' bytes. They replay another implementation's byte decisions at
    entries whose exact value lies within that implementation's rounding of
    a boundary between two codes (the caller checks that they do).

    weights="exp_cast" writes each tile's bytes by the path ExpCast replaces
    (exp_cast_codes against the same running max) instead; everything else
    is the same.
    """
    if weights not in ("expcast", "exp_cast"):
        raise ValueError(weights)
    codes_of = expcast_codes if weights == "expcast" else exp_cast_codes
    S, D = k.shape
    tau = 1.0 / math.sqrt(D) if tau is None else tau
    rows = np.arange(S) if rows is None else np.asarray(rows)
    if ph is None:
        ph = prepare_head(q, k, v, budget, k_smooth=k_smooth, v_smooth=v_smooth)
    nT = (S + QK_BLOCK - 1) // QK_BLOCK
    tiles = key_tile_order(nT) if order == "mid" else list(range(nT))
    vd = decode(ph.vc)
    out = np.empty((len(rows), D))
    Ms = np.empty(len(rows), dtype=np.int64)
    Ls = np.empty(len(rows))
    trace = np.zeros((len(rows), nT), dtype=np.int64)
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        x = log2_logits(ph, r, tau)
        M = np.full(len(r), -np.inf)
        O = np.zeros((len(r), D))
        Omu = np.zeros((len(r), D))        # V-Smooth: sum over tiles of (tile row sum) * (block mean)
        L = np.zeros(len(r))
        for t in tiles:
            ks = slice(t * QK_BLOCK, min(S, (t + 1) * QK_BLOCK))
            xt = x[:, ks]
            if m_trace is None:
                Mn = np.maximum(M, np.ceil(xt.max(axis=1)))
            else:
                Mn = np.asarray(m_trace[c0:c0 + len(r), t], dtype=np.float64)
            f = np.where(np.isinf(M), 0.0, np.exp2(M - Mn))     # exact powers of two
            codes = codes_of(xt, Mn)
            if code_trace is not None:
                ct = np.asarray(code_trace[c0:c0 + len(r), ks])
                codes = np.where(ct >= 0, ct, codes).astype(np.uint8)
            P = VALUES[codes]
            O = O * f[:, None] + P @ vd[ks]
            if ph.vmean is not None:
                Omu = Omu * f[:, None] + P.sum(axis=1)[:, None] * ph.vmean[t][None, :]
            L = L * f + P.sum(axis=1)
            M = Mn
            trace[c0:c0 + len(r), t] = Mn.astype(np.int64)
        O *= float(ph.sv)
        O += Omu
        if ph.repair is not None and ph.repair.k > 0:
            rp = ph.repair
            codes = codes_of(x[:, rp.sel], M)
            if rcode_trace is not None:
                ct = np.asarray(rcode_trace[c0:c0 + len(r)])
                codes = np.where(ct >= 0, ct, codes).astype(np.uint8)
            P = VALUES[codes]
            O += float(rp.sr) * (P @ decode(rp.rc))
        out[c0:c0 + len(r)] = O / L[:, None]
        Ms[c0:c0 + len(r)] = M.astype(np.int64)
        Ls[c0:c0 + len(r)] = L
    return {"out": out, "M": Ms, "L": Ls, "ph": ph, "m_trace": trace}


def exact_attention_head(q, k, v, tau=None, rows=None, chunk=512):
    """softmax(tau * q k^T) v in float64 on the unquantized inputs."""
    S, D = k.shape
    tau = 1.0 / math.sqrt(D) if tau is None else tau
    rows = np.arange(S) if rows is None else np.asarray(rows)
    out = np.empty((len(rows), D))
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        s = tau * (q[r] @ k.T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[c0:c0 + len(r)] = (p @ v) / p.sum(axis=1, keepdims=True)
    return out


def row_total_variation(codes: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Per row, half the L1 distance between the normalized decoded weights
    and the exact softmax of the same (quantized) logits."""
    P = VALUES[codes]
    P = P / P.sum(axis=1, keepdims=True)
    p = np.exp2(x - x.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    return 0.5 * np.abs(P - p).sum(axis=1)


def rel_l2(a, b) -> float:
    """Frobenius-norm relative error ||a - b|| / ||b||."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))
