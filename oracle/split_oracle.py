"""Plain CPU oracle for the outlier-channel mixed bit-width variant of
TurboQuant (a few outlier channels at one bit more than the rest; 2.5 and
3.5 bits per coordinate when half of the channels are outliers).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It imports
nothing from the product; each channel group is the oracle's own TurboQuant
(``tq_oracle``).

Sources (pages cited by title and section):
  "TurboQuant压缩效果" (video transcript): the 2.5 / 3.5-bit figures are
      averages over the 128 channels of a head: a few outlier channels get 3
      bits and the great majority 2.
  [P5] "谷歌TurboQuant如何绕过内存墙？重新审视它的技术突破", 第一阶段 and
      第二阶段: each group is quantised by the two-stage method (rotation +
      Lloyd-Max on b-1 bits, then 1-bit QJL of the residual).

Readings (numbered; tests and comments refer to them):
  M1  the number of outlier channels n_out is a parameter (32, 64 or 96 of
      128 on the device).  The page names both "a few" outlier channels and
      averages of 2.5 / 3.5 bits; with b_out = b_rest + 1 the average is
      b_rest + n_out / d, so 2.5 needs n_out = d / 2 (the default), while a
      few outliers (n_out = 32) give b_rest + 1/4.
  M2  the split is made before the rotation (after it every coordinate has the
      same law and there are no outlier channels); each group is its own
      TurboQuant instance in prod mode of dimension d_g (n_out, then
      d - n_out) with m = d_g QJL rows, rotation seed seed_pi + g and JL seed
      seed_s + g (g = 0 for the outlier group, 1 for the rest).
  M3  the channel list is an input (a permutation of 0 .. d-1 whose first
      n_out entries are the outlier channels); ``outlier_channels`` picks the
      n_out channels of largest mean square of a sample, as a caller would
      from a prompt's keys.
  M4  the logit is the sum of the two groups' estimators,
      nu_g <Pi_g q_g, c_g[idx_g]> + sqrt(pi/2)/d_g ||r_g|| <S_g q_g, s_g>.
"""
from __future__ import annotations

import numpy as np

from oracle import tq_oracle as tqo


class SplitParams:
    def __init__(self, channels, b_out: int, b_rest: int, seed_pi: int = 2, seed_s: int = 3,
                 n_out: int | None = None):
        ch = np.asarray(channels, dtype=np.int64)
        self.d = ch.size
        assert sorted(ch.tolist()) == list(range(self.d))
        self.n_out = self.d // 2 if n_out is None else int(n_out)
        assert 0 < self.n_out < self.d
        self.channels = ch
        self.dims = (self.n_out, self.d - self.n_out)
        self.b_out, self.b_rest = int(b_out), int(b_rest)
        self.groups = [tqo.Params(self.dims[0], self.b_out, self.dims[0], tqo.MODE_PROD, seed_pi, seed_s),
                       tqo.Params(self.dims[1], self.b_rest, self.dims[1], tqo.MODE_PROD, seed_pi + 1, seed_s + 1)]

    def group_channels(self, g: int) -> np.ndarray:
        return self.channels[:self.n_out] if g == 0 else self.channels[self.n_out:]

    @property
    def bits_per_coordinate(self) -> float:
        return (self.dims[0] * self.b_out + self.dims[1] * self.b_rest) / self.d


def outlier_channels(x: np.ndarray, n_out: int) -> np.ndarray:
    """The n_out channels of largest mean square first (ascending channel
    order within each group), then the rest."""
    ms = np.mean(np.asarray(x, dtype=np.float64) ** 2, axis=0)
    order = np.argsort(-ms, kind="stable")
    out = np.sort(order[:n_out])
    rest = np.sort(order[n_out:])
    return np.concatenate([out, rest])


def encode(x: np.ndarray, p: SplitParams) -> list:
    x = np.asarray(x, dtype=np.float64)
    return [tqo.encode(x[:, p.group_channels(g)], p.groups[g]) for g in range(2)]


def score(q: np.ndarray, codes: list, p: SplitParams, n_kv: int, g: int, seq: int) -> np.ndarray:
    q = np.asarray(q, dtype=np.float64).reshape(n_kv * g, p.d)
    return sum(tqo.score(q[:, p.group_channels(k)], codes[k], p.groups[k], n_kv, g, seq) for k in range(2))


# ---------------------------------------------------------------------------
# Packed layout (a format, defined here and in include/tq.h), d = 128
# ---------------------------------------------------------------------------
# Per vector: uint32 words, group 0 then group 1; a group of dimension d_g
# and B Lloyd-Max bits holds B index planes then its sign plane, each plane
# d_g / 32 words.  Coordinate c = 16 t + 4 k + i of the group (t < d_g / 16,
# k, i < 4) is bit k d_g / 4 + 4 t + i of the plane's bit string, whose bit j
# is bit j % 32 of word j // 32 (for d_g = 64: word k // 2, bit
# 16 (k % 2) + 4 t + i).  float32 norms [n][4]: ||x_0||, ||r_0||, ||x_1||,
# ||r_1||.
def words_per_vector(p: SplitParams) -> int:
    return sum((p.groups[g].B + 1) * p.dims[g] // 32 for g in range(2))


def _plane_pos(dg: int, c: int) -> int:
    t, k, i = c // 16, (c // 4) % 4, c % 4
    return k * (dg // 4) + 4 * t + i


def _plane_bits(bits: np.ndarray) -> np.ndarray:
    """bool [n, d_g] -> uint32 [n, d_g / 32]."""
    n, dg = bits.shape
    w = np.zeros((n, dg // 32), dtype=np.uint64)
    for c in range(dg):
        j = _plane_pos(dg, c)
        w[:, j // 32] |= bits[:, c].astype(np.uint64) << np.uint64(j % 32)
    return w.astype(np.uint32)


def _plane_unbits(w: np.ndarray, dg: int) -> np.ndarray:
    w = w.astype(np.uint64)
    out = []
    for c in range(dg):
        j = _plane_pos(dg, c)
        out.append(((w[:, j // 32] >> np.uint64(j % 32)) & np.uint64(1)).astype(bool))
    return np.stack(out, axis=1)


def pack(codes: list, p: SplitParams) -> dict:
    assert p.d == 128 and all(dg % 32 == 0 for dg in p.dims)
    n = codes[0]["knorm"].shape[0]
    words, norms = [], np.zeros((n, 4), dtype=np.float32)
    for g in range(2):
        c = codes[g]
        for j in range(p.groups[g].B):
            words.append(_plane_bits(((c["idx"] >> j) & 1).astype(bool)))
        words.append(_plane_bits(c["sign"]))
        norms[:, 2 * g] = c["knorm"]
        norms[:, 2 * g + 1] = c["rnorm"]
    return {"words": np.concatenate(words, axis=1), "norms": norms}


def unpack(packed: dict, p: SplitParams) -> list:
    words = np.asarray(packed["words"]).astype(np.uint32)
    norms = np.asarray(packed["norms"], dtype=np.float32)
    out, at = [], 0
    for g in range(2):
        B, dg = p.groups[g].B, p.dims[g]
        nw = dg // 32
        idx = np.zeros((words.shape[0], dg), dtype=np.int64)
        for j in range(B):
            idx |= _plane_unbits(words[:, at:at + nw], dg).astype(np.int64) << j
            at += nw
        sign = _plane_unbits(words[:, at:at + nw], dg)
        at += nw
        out.append({"idx": idx, "sign": sign, "knorm": norms[:, 2 * g].copy(), "rnorm": norms[:, 2 * g + 1].copy()})
    return out
