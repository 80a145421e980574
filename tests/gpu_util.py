"""Test-side helpers for the GPU parity tests: read the prepared tensors out
of a workspace (restating the pack layouts documented in include/oc_attn.h)
and run the oracle on the same inputs."""
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
                k_smooth=False, v_smooth=False):
    """oracle output rows for one (b, h), in the single-pass form the kernel
    computes (key tiles from the middle of the window outwards), plus the
    prepared head; m_trace replays given running-max decisions; weights
    "exp_cast" is the comparison byte path"""
    qh, kh, vh = head64(q, b, h), head64(k, b, h), head64(v, b, h)
    return oracle.expcast_attention_online(qh, kh, vh, tau=tau, rows=rows, budget=budget, order=order,
                                           m_trace=m_trace, weights=weights, k_smooth=k_smooth, v_smooth=v_smooth)


def out_rows(out, b, h, rows):
    return out[b, :, h].float().cpu().numpy()[np.asarray(rows)].astype(np.float64)
