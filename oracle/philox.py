"""Philox4x32-10 and the uniform token draw of the canvas (test infrastructure only).

Philox4x32-10 is the counter-based generator of J. Salmon, M. Moraes, R. Dror
and D. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).  One round
multiplies counter words 0 and 2 by two fixed 32-bit constants, keeps both
halves of each 64-bit product, and mixes the high halves with counter words 1
and 3 and the two key words; between rounds each key word is advanced by a
Weyl constant (the golden ratio and sqrt(3)-1, scaled to 32 bits).  Ten rounds.

Canvas draws: the pages describe a uniform-state canvas whose slots start as
random vocabulary tokens and whose unkept slots are re-randomised each pass
([P5] "When to use a diffusion LLM", section "How block diffusion works").  A
slot's token is
    U(seed, block, step, slot) = floor(word0 * V / 2^32),
    word0 = Philox4x32-10(key = (seed mod 2^32, seed div 2^32),
                          counter = (slot, step, block, 0))[0].
For V a power of two this is exactly uniform on [0, V).
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """counter: 4 arrays (or ints) of 32-bit words; key: 2 ints.  Returns 4 uint64 arrays of 32-bit words."""
    c = [np.asarray(w, dtype=np.uint64) & _MASK32 for w in counter]
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = m0 * c[0]          # < 2^64, exact in uint64
        p1 = m1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return c


def uniform_tokens(seed: int, block: int, step: int, slots, vocab: int) -> np.ndarray:
    """U(seed, block, step, slot) for each slot in ``slots``, as int64."""
    slots = np.asarray(slots, dtype=np.uint64)
    n = slots.shape
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    ctr = (slots, np.full(n, step, dtype=np.uint64), np.full(n, block, dtype=np.uint64),
           np.zeros(n, dtype=np.uint64))
    w0 = philox4x32_10(ctr, key)[0]
    return ((w0 * np.uint64(vocab)) >> np.uint64(32)).astype(np.int64)


def gumbel_noise(seed: int, block: int, step: int, slots, vocab: int) -> np.ndarray:
    """Standard Gumbel noise G[i, v] for slot ``slots[i]`` and token v, float64 [len(slots), vocab].

    The recommended sampler draws each slot's token from the softmax at the pass's
    temperature ([P2] "Architecture Details": the temperature falls linearly from 0.8
    to 0.4 over the passes; [P5] "Appendix: Methodology", "Decoding").  The draw uses the Gumbel-max identity
    (E. J. Gumbel, 1954; argmax_v (l_v + G_v) with i.i.d. standard Gumbel G_v is
    distributed as softmax(l)), which needs one uniform per (slot, token):
        w = word (v mod 4) of Philox4x32-10(key = (seed mod 2^32, seed div 2^32),
                                            counter = (v div 4, slot + 2^16 step, block, 1)),
        u = (2 floor(w / 2^9) + 1) / 2^24          (exact in fp32, never 0 or 1),
        G = -ln(-ln u).
    Counter word 3 is 1 here and 0 for the canvas draws, so the two streams never share
    a counter.  Slots and steps must stay below 2^16.
    """
    slots = np.asarray(slots, dtype=np.uint64)
    nq = (vocab + 3) // 4
    n = slots.shape[0]
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    c0 = np.broadcast_to(np.arange(nq, dtype=np.uint64)[None, :], (n, nq))
    c1 = np.broadcast_to((slots + (np.uint64(step) << np.uint64(16)))[:, None], (n, nq))
    c2 = np.full((n, nq), block, dtype=np.uint64)
    c3 = np.ones((n, nq), dtype=np.uint64)
    words = philox4x32_10((c0, c1, c2, c3), key)
    w = np.stack(words, axis=-1).reshape(n, 4 * nq)[:, :vocab]
    u = (2.0 * (w >> np.uint64(9)).astype(np.float64) + 1.0) / float(1 << 24)
    return -np.log(-np.log(u))
