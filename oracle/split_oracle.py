"""Plain CPU oracle for the outlier-channel mixed bit-width variant of
TurboQuant (2.5 and 3.5 bits per coordinate).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It imports
nothing from the product; each channel group is the oracle's own TurboQuant
(``tq_oracle``).

Sources (pages cited by title and section):
  "TurboQuant压缩效果" (video transcript): the 2.5 / 3.5-bit figures are
      averages over the 128 channels of a head: the outlier channels get 3
      bits and the ordinary ones 2.
  [P5] "谷歌TurboQuant如何绕过内存墙？重新审视它的技术突破", 第一阶段 and
      第二阶段: each group is quantised by the two-stage method (rotation +
      Lloyd-Max on b-1 bits, then 1-bit QJL of the residual).

Readings (numbered; tests and comments refer to them):
  M1  the average fixes the split: with b_out = b_rest + 1 bits, an average of
      b_rest + 1/2 bits needs half of the d channels in the outlier group
      (the page's "a few" outlier channels cannot give 2.5 with 3 / 2 bits).
  M2  the split is made before the rotation (after it every coordinate has the
      same law and there are no outlier channels); each group of 64 channels
      is its own TurboQuant instance of dimension 64 in prod mode, with m = 64
      QJL rows, rotation seed seed_pi + g and JL seed seed_s + g (g = 0 for
      the outlier group, 1 for the rest).
  M3  the channel list is an input (a permutation of 0 .. d-1 whose first d/2
      entries are the outlier channels); ``outlier_channels`` picks the d/2
      channels of largest mean square of a sample, as a caller would from a
      prompt's keys.
  M4  the logit is the sum of the two groups' estimators,
      nu_g <Pi_g q_g, c_g[idx_g]> + sqrt(pi/2)/64 ||r_g|| <S_g q_g, s_g>.
"""
from __future__ import annotations

import numpy as np

from oracle import tq_oracle as tqo


class SplitParams:
    def __init__(self, channels, b_out: int, b_rest: int, seed_pi: int = 2, seed_s: int = 3):
        ch = np.asarray(channels, dtype=np.int64)
        self.d = ch.size
        assert sorted(ch.tolist()) == list(range(self.d)) and self.d % 2 == 0
        self.channels = ch
        self.h = self.d // 2
        self.b_out, self.b_rest = int(b_out), int(b_rest)
        self.groups = [tqo.Params(self.h, self.b_out, self.h, tqo.MODE_PROD, seed_pi, seed_s),
                       tqo.Params(self.h, self.b_rest, self.h, tqo.MODE_PROD, seed_pi + 1, seed_s + 1)]

    def group_channels(self, g: int) -> np.ndarray:
        return self.channels[g * self.h:(g + 1) * self.h]

    @property
    def bits_per_coordinate(self) -> float:
        return (self.h * self.b_out + self.h * self.b_rest) / self.d


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
# Per vector: uint32 words, group 0 then group 1; a group of B Lloyd-Max bits
# holds B index planes then its sign plane, each plane two words: coordinate
# c = 16 t + 4 k + i of the group (t, k, i < 4) at word k // 2, bit
# 16 (k % 2) + 4 t + i.  float32 norms [n][4]: ||x_0||, ||r_0||, ||x_1||, ||r_1||.
def words_per_vector(p: SplitParams) -> int:
    return 2 * (p.groups[0].B + 1 + p.groups[1].B + 1)


def _word_bit(c: int):
    t, k, i = c // 16, (c // 4) % 4, c % 4
    return k // 2, 16 * (k % 2) + 4 * t + i


def _plane_bits(bits: np.ndarray) -> np.ndarray:
    """bool [n, 64] -> uint32 [n, 2]."""
    n = bits.shape[0]
    w = np.zeros((n, 2), dtype=np.uint64)
    for c in range(64):
        wi, b = _word_bit(c)
        w[:, wi] |= bits[:, c].astype(np.uint64) << np.uint64(b)
    return w.astype(np.uint32)


def _plane_unbits(w: np.ndarray) -> np.ndarray:
    w = w.astype(np.uint64)
    out = []
    for c in range(64):
        wi, b = _word_bit(c)
        out.append(((w[:, wi] >> np.uint64(b)) & np.uint64(1)).astype(bool))
    return np.stack(out, axis=1)


def pack(codes: list, p: SplitParams) -> dict:
    assert p.d == 128
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
        B = p.groups[g].B
        idx = np.zeros((words.shape[0], 64), dtype=np.int64)
        for j in range(B):
            idx |= _plane_unbits(words[:, at:at + 2]).astype(np.int64) << j
            at += 2
        sign = _plane_unbits(words[:, at:at + 2])
        at += 2
        out.append({"idx": idx, "sign": sign, "knorm": norms[:, 2 * g].copy(), "rnorm": norms[:, 2 * g + 1].copy()})
    return out
