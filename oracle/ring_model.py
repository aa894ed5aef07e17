"""Byte-exact model of the compact sliding-window ring cache.  TEST
INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline).

Pages cited (title; section):
  [SPYRE]  "Enable compact sliding-window attention for Gemma 3 and Gemma 4
           variants" (torch-spyre/hf-adapters pull request 496)
  [BONSAI] "Gemma3 Local Attention Cache" (jax-ml/bonsai issue 124)

What the pages fix, restated:
  - [SPYRE] Summary: the prompt-sized sliding cache is compacted at the first
    decode into a buffer of window + 64 rows anchored at a buffer origin,
    and every 64 decode tokens the compact cache is rolled with offset-aware
    device-to-device copies; left padding is preserved.
  - [SPYRE] Compilation behavior: decode position, buffer origin, unwritten
    rows, padding and window placement are tensor data, never host values.
  - [BONSAI] Steps 2 and 3: cache writes wrap around with a modulo and the
    window mask follows the wrap.

Readings taken where the pages are silent:
  - per sequence b the state is ring_meta[b] = (pos, anchor, start, lo):
    pos = position of the newest row, anchor = position held by logical
    ring row 0 (the buffer origin), start = physical row of the anchor,
    lo = number of left-pad positions (bit 31 is a sticky overflow flag);
  - position p lives at physical row slot(p) = (start + p - anchor) mod R
    for anchor <= p < anchor + R;
  - compaction of a prompt of length L sets anchor = L - W (may be negative
    for short prompts), start = anchor mod R, pos = L - 1, copies the
    prompt rows the ring can hold and zero-fills every other row;
  - append of position p = pos + 1 is refused (flag set, nothing written)
    when p - anchor >= R;
  - the roll fires for a sequence when pos + 1 - anchor >= R; it rotates the
    physical rows left by A = R - W (new[r] = old[(r + A) mod R]) and sets
    anchor += A, leaving start unchanged;
  - decode reads position a iff max(lo, pos - W + 1, 0) <= a <= pos.
"""
import numpy as np

ERR_BIT = np.int32(-2 ** 31)  # bit 31 of ring_meta[b, 3]


class RingModel:
    """Rings K/V [B, Hkv, R, D] of one element type plus ring_meta [B, 4]."""

    def __init__(self, batch, hkv, ring_rows, d, window, dtype=np.uint16):
        if window < 1 or ring_rows <= window:
            raise ValueError("ring needs window >= 1 and ring_rows > window")
        self.B, self.hkv, self.R, self.d, self.W = batch, hkv, ring_rows, d, window
        self.A = ring_rows - window
        self.k = np.zeros((batch, hkv, ring_rows, d), dtype=dtype)
        self.v = np.zeros((batch, hkv, ring_rows, d), dtype=dtype)
        self.meta = np.zeros((batch, 4), dtype=np.int32)

    # -- addressing ---------------------------------------------------------
    def slot(self, b, p):
        pos, anchor, start, _ = (int(x) for x in self.meta[b])
        if not (anchor <= p < anchor + self.R):
            raise IndexError("position %d outside the ring span of sequence %d" % (p, b))
        return (start + p - anchor) % self.R

    def lower(self, b):
        pos, _, _, lo = (int(x) for x in self.meta[b])
        lo &= 0x7FFFFFFF
        return max(lo, pos - self.W + 1, 0)

    def valid_rows(self, b):
        """(physical row, position) pairs decode reads, in position order."""
        pos, anchor, start, _ = (int(x) for x in self.meta[b])
        low = self.lower(b)
        out = []
        for r in range(self.R):
            a = anchor + (r - start) % self.R
            if low <= a <= pos:
                out.append((r, a))
        out.sort(key=lambda t: t[1])
        return out

    # -- the three cache operations ----------------------------------------
    def compact(self, k_src, v_src, cu_seqlens, prompt_lens=None, left_pad=None):
        """Fill every sequence's ring from packed prompt rows [T, Hkv, D].

        Sequence b's packed rows are the LAST n_b = cu[b+1]-cu[b] positions
        of its prompt of length L_b (prompt_lens[b], default n_b)."""
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        for b in range(self.B):
            n = int(cu[b + 1] - cu[b])
            L = n if prompt_lens is None else int(prompt_lens[b])
            lo = 0 if left_pad is None else int(left_pad[b])
            if L < 1 or n < 0 or n > L or lo < 0 or lo >= L:
                raise ValueError("sequence %d: bad prompt (L=%d, n=%d, lo=%d)" % (b, L, n, lo))
            anchor = L - self.W
            start = anchor % self.R
            self.meta[b] = (L - 1, anchor, start, lo)
            need = max(lo, L - self.W + 1, 0)
            if L - n > need:
                raise ValueError("sequence %d: prompt rows do not cover the window" % b)
            self.k[b] = 0
            self.v[b] = 0
            for p in range(max(anchor, 0, L - n), L):
                src = int(cu[b]) + (p - (L - n))
                r = self.slot(b, p)
                self.k[b, :, r, :] = k_src[src]
                self.v[b, :, r, :] = v_src[src]

    def append(self, k_new, v_new):
        """Write the token at position pos + 1 of every sequence."""
        for b in range(self.B):
            pos, anchor = int(self.meta[b, 0]), int(self.meta[b, 1])
            p = pos + 1
            if p - anchor >= self.R:
                self.meta[b, 3] |= ERR_BIT
                continue
            r = self.slot(b, p)
            self.k[b, :, r, :] = k_new[b]
            self.v[b, :, r, :] = v_new[b]
            self.meta[b, 0] = p

    def roll(self, copy=True):
        """Roll every full ring by A = R - W rows.

        copy=True moves the bytes (new[r] = old[(r + A) mod R]) and keeps
        start; copy=False is the metadata-only equivalent (start += A)."""
        for b in range(self.B):
            pos, anchor, start = (int(x) for x in self.meta[b, :3])
            if pos + 1 - anchor < self.R:
                continue
            if copy:
                idx = (np.arange(self.R) + self.A) % self.R
                self.k[b] = self.k[b][:, idx, :]
                self.v[b] = self.v[b][:, idx, :]
            else:
                self.meta[b, 2] = (start + self.A) % self.R
            self.meta[b, 1] = anchor + self.A

    # -- helpers for decode parity -----------------------------------------
    def gather_linear(self, b):
        """K/V rows decode reads for sequence b, ordered by position, with
        the first position: (k [n, Hkv, D], v [n, Hkv, D], first_pos)."""
        rows = self.valid_rows(b)
        if not rows:
            return (np.zeros((0, self.hkv, self.d), self.k.dtype),
                    np.zeros((0, self.hkv, self.d), self.v.dtype), int(self.meta[b, 0]) + 1)
        r_idx = [r for r, _ in rows]
        k = np.ascontiguousarray(self.k[b][:, r_idx, :].transpose(1, 0, 2))
        v = np.ascontiguousarray(self.v[b][:, r_idx, :].transpose(1, 0, 2))
        return k, v, rows[0][1]
