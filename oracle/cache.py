"""The four-region cache and its seal rule (oracle; test infrastructure only).

SJ-KVaRN, section 2.1 "The life of a token":
1. sink: the first 128 tokens stay at 16 bits for the whole run;
2. staging: a new token's key and value are rotated and written to a ring in
   tq6_0;
3. exact tail: the newest tokens stay in that ring;
4. seal: when the tail reaches its maximum, every full 128-token group older
   than the newest 4,096 tokens is compressed into body records in one batch.
Section 4.3 "Adaptive tail": the tail grows from 4,096 to 8,192 tokens, then
everything older than the newest 4,096 is sealed; an idle server also seals
back to 4,096 between requests.  Section 3: the staging ring is allocated at
full size up front, sized for 8,192 tokens plus margin (section 4.3).
Section 10: sealed records cannot be partly rewritten.

Readings:
* token t < 128 goes to the sink, every later token to the ring; body record
  r covers tokens [128 + 128 r, 256 + 128 r);
* "reaches its maximum" is ring_len >= tail_max; the seal then takes
  floor((ring_len - tail_min) / 128) groups, oldest first; the idle seal-back
  (mode TO_MIN) takes the same count without the tail_max test;
* ring capacity = round_up(tail_max + margin, 128) token slots; token t sits
  in slot (t - 128) mod capacity, so a 128-token group never wraps;
* appending more tokens than the ring can hold fails (the caller seals
  first); appending beyond the per-sequence context capacity fails.
The rotation, staging codec, balancing and rounding are the other oracle
modules; this one only moves tokens between regions and builds records.

Staging precision (SJ-KVaRN section 4.1: a 6-bit tail instead of 16-bit; KV
Cache Precision Tail, section 2: KVarN's exact tail is F16, its staging and
record path F16-based): with stage="f16" the ring holds each token's key and
value exactly as given, in the original domain like the sink (an exact tail:
unquantized floating point).  The seal then reads the group's fp16 rows and
rotates them, R x computed exactly and rounded once to fp32 -- the values the
6-bit staging would have quantised -- and balances and rounds them as usual.
Decode reads f16 ring tokens as they are, like the sink.
"""
from __future__ import annotations

import numpy as np

from . import attention, record, rotation, rounding, sinkhorn, tq6

SINK = 128
GROUP = 128

OK, ERR_INVALID, ERR_CAPACITY, ERR_RING_FULL, ERR_SEALED = 0, -1, -2, -3, -4
SEAL_IF_FULL, SEAL_TO_MIN = 0, 1
REGION_SINK, REGION_RING, REGION_BODY = 0, 1, 2


def ring_capacity(tail_max: int, margin: int) -> int:
    return -(-(tail_max + margin) // GROUP) * GROUP


def groups_to_seal(ring_len: int, tail_min: int, tail_max: int, mode: int) -> int:
    if mode == SEAL_IF_FULL and ring_len < tail_max:
        return 0
    return max(0, (ring_len - tail_min) // GROUP)


def max_records(max_ctx: int) -> int:
    return max(0, (max_ctx - SINK) // GROUP)


def encode_tile(x32, passes: int, bits: int):
    """Seal one 128 x sub tile of rotated fp32 values: balance, then round rows."""
    bal = sinkhorn.balance(np.asarray(x32, np.float64), passes)
    codes, S, Z = rounding.round_rows(x32, bal["C"], bits)
    return {"codes": codes, "C": bal["C"], "S": S, "Z": Z}


class OracleCache:
    """Host model of one cache: every (sequence, layer) has its own regions."""

    def __init__(self, n_layers, n_kv_heads, head_dim, n_q_heads, max_seqs, max_ctx,
                 tail_min, tail_max, margin=512, k_bits=4, v_bits=4, passes=16, signs=None, stage="tq6"):
        assert head_dim in (128, 256, 512) and stage in ("tq6", "f16")
        self.stage = stage
        assert tail_min % GROUP == 0 and tail_min <= tail_max
        self.L, self.H, self.D, self.Hq = n_layers, n_kv_heads, head_dim, n_q_heads
        self.max_seqs, self.max_ctx = max_seqs, max_ctx
        self.tail_min, self.tail_max, self.margin = tail_min, tail_max, margin
        self.k_bits, self.v_bits, self.passes = k_bits, v_bits, passes
        self.signs = signs
        self.cap = ring_capacity(tail_max, margin)
        self.nb = head_dim // tq6.BLOCK
        self.sub = record.sub_width(head_dim)
        self.nsub = record.n_sub(head_dim)
        self.st = {}

    # ------------------------------------------------------------ state
    def _state(self, seq, layer):
        key = (seq, layer)
        if key not in self.st:
            H, D, nb, cap = self.H, self.D, self.nb, self.cap
            self.st[key] = {
                "n_tok": 0, "n_rec": 0,
                "sink_k": np.zeros((SINK, H, D), np.float16), "sink_v": np.zeros((SINK, H, D), np.float16),
                "ring_d": np.zeros((2, cap, H, nb), np.float16),
                "ring_u": np.full((2, cap, H, nb, tq6.BLOCK), 32, np.uint8),
                "ring_x": np.zeros((2, cap, H, D), np.float16),   # f16 staging: tokens as given
                "records": [[] for _ in range(H)],
            }
        return self.st[key]

    def ring_len(self, seq, layer) -> int:
        s = self._state(seq, layer)
        return max(0, s["n_tok"] - SINK - GROUP * s["n_rec"])

    def info(self, seq, layer):
        s = self._state(seq, layer)
        return s["n_tok"], s["n_rec"], self.ring_len(seq, layer)

    # ------------------------------------------------------------ append
    def append(self, layer: int, seqs, k16, v16) -> int:
        """k16, v16: fp16 [n_seqs][n_tok][H][D].  All-or-nothing."""
        k16 = np.asarray(k16, np.float16)
        v16 = np.asarray(v16, np.float16)
        n = k16.shape[1]
        if not (0 <= layer < self.L) or len(set(seqs)) != len(seqs):
            return ERR_INVALID
        for seq in seqs:
            if not (0 <= seq < self.max_seqs):
                return ERR_INVALID
            s = self._state(seq, layer)
            if s["n_tok"] + n > self.max_ctx:
                return ERR_CAPACITY
            ring_after = max(0, s["n_tok"] + n - SINK - GROUP * s["n_rec"])
            if ring_after > self.cap:
                return ERR_RING_FULL
        for b, seq in enumerate(seqs):
            s = self._state(seq, layer)
            pos = np.arange(s["n_tok"], s["n_tok"] + n)
            to_sink = pos < SINK
            s["sink_k"][pos[to_sink]] = k16[b, to_sink]
            s["sink_v"][pos[to_sink]] = v16[b, to_sink]
            rest = ~to_sink
            if rest.any():
                slots = (pos[rest] - SINK) % self.cap
                for side, src in ((0, k16[b, rest]), (1, v16[b, rest])):
                    if self.stage == "f16":
                        s["ring_x"][side, slots] = src
                        continue
                    x = rotation.rotate(src, self.D, self.signs).reshape(-1, self.H, self.nb, tq6.BLOCK)
                    d, u = tq6.encode_blocks(x)
                    s["ring_d"][side, slots] = d
                    s["ring_u"][side, slots] = u
            s["n_tok"] += n
        return OK

    # ------------------------------------------------------------ seal
    def ring_tile(self, seq, layer, head, group_start_token, side) -> np.ndarray:
        """Dequantised rotated fp32 values of 128 ring tokens: (128, D)."""
        s = self._state(seq, layer)
        slots = [(group_start_token + i - SINK) % self.cap for i in range(GROUP)]
        if self.stage == "f16":
            return rotation.rotate(s["ring_x"][side, slots, head], self.D, self.signs)
        d = s["ring_d"][side, slots, head]
        u = s["ring_u"][side, slots, head]
        return tq6.decode_blocks(d, u).reshape(GROUP, self.D)

    def seal(self, layer: int, mode: int, seqs=None) -> int:
        """Seal eligible groups of one layer (or every layer if layer == -1)."""
        layers = range(self.L) if layer == -1 else [layer]
        total = 0
        for ly in layers:
            for (seq, l2) in sorted(self.st):
                if l2 != ly or (seqs is not None and seq not in seqs):
                    continue
                s = self.st[(seq, l2)]
                g = groups_to_seal(self.ring_len(seq, ly), self.tail_min, self.tail_max, mode)
                for _ in range(g):
                    t0 = SINK + GROUP * s["n_rec"]
                    for h in range(self.H):
                        xk = self.ring_tile(seq, ly, h, t0, 0)
                        xv = self.ring_tile(seq, ly, h, t0, 1)
                        parts = []
                        for i in range(self.nsub):
                            cs = slice(i * self.sub, (i + 1) * self.sub)
                            k = encode_tile(xk[:, cs], self.passes, self.k_bits)
                            v = encode_tile(xv[:, cs], self.passes, self.v_bits)
                            parts.append(record.build_sub(k, v, self.k_bits, self.v_bits))
                        s["records"][h].append(b"".join(parts))
                    s["n_rec"] += 1
                    total += 1
        return total

    # ------------------------------------------------------------ canonical bytes
    def export(self, seq, layer, head, region, index) -> bytes:
        """Canonical bytes of one sink token [K f16 D][V f16 D], one ring slot
        [K tq6 blocks][V tq6 blocks], or one body record."""
        s = self._state(seq, layer)
        if region == REGION_SINK:
            return s["sink_k"][index, head].tobytes() + s["sink_v"][index, head].tobytes()
        if region == REGION_RING and self.stage == "f16":
            return s["ring_x"][0, index, head].tobytes() + s["ring_x"][1, index, head].tobytes()
        if region == REGION_RING:
            out = b""
            for side in (0, 1):
                for b in range(self.nb):
                    out += tq6.block_bytes(s["ring_d"][side, index, head, b], s["ring_u"][side, index, head, b])
            return out
        if region == REGION_BODY:
            return s["records"][head][index]
        raise ValueError(region)

    def import_ring(self, seq, layer, head, slot, buf):
        """Canonical bytes of one ring slot (the export layout) into the ring: a
        test hook that places chosen staged tiles."""
        s = self._state(seq, layer)
        buf = bytes(buf)
        if self.stage == "f16":
            assert len(buf) == 4 * self.D
            x = np.frombuffer(buf, np.float16).reshape(2, self.D)
            s["ring_x"][:, slot, head] = x
            return
        assert len(buf) == 2 * self.nb * tq6.BLOCK_BYTES
        for side in (0, 1):
            for b in range(self.nb):
                o = (side * self.nb + b) * tq6.BLOCK_BYTES
                d, u = tq6.parse_block(buf[o:o + tq6.BLOCK_BYTES])
                s["ring_d"][side, slot, head, b] = d
                s["ring_u"][side, slot, head, b] = u

    def import_record(self, seq, layer, head, index, buf):
        s = self._state(seq, layer)
        recs = s["records"][head]
        if index == len(recs):
            recs.append(bytes(buf))
        else:
            recs[index] = bytes(buf)

    # ------------------------------------------------------------ attention
    def head_kv(self, seq, layer, head):
        """Original-domain float64 keys and values of every cached token, in
        token order: (n_tok, D) each."""
        s = self._state(seq, layer)
        n_tok, n_rec = s["n_tok"], s["n_rec"]
        ks, vs = [], []
        ns = min(n_tok, SINK)
        ks.append(s["sink_k"][:ns, head].astype(np.float64))
        vs.append(s["sink_v"][:ns, head].astype(np.float64))
        for r in range(n_rec):
            subs = record.parse_record(s["records"][head][r], self.D, self.k_bits, self.v_bits)
            kr = np.concatenate([rounding.dequant(k["codes"], k["C"], k["S"], k["Z"]) for k, _ in subs], axis=1)
            vr = np.concatenate([rounding.dequant(v["codes"], v["C"], v["S"], v["Z"]) for _, v in subs], axis=1)
            ks.append(rotation.inverse_exact(kr, self.D, self.signs))
            vs.append(rotation.inverse_exact(vr, self.D, self.signs))
        t0 = SINK + GROUP * n_rec
        if n_tok > t0:
            slots = [(t - SINK) % self.cap for t in range(t0, n_tok)]
            for side, lst in ((0, ks), (1, vs)):
                if self.stage == "f16":
                    lst.append(s["ring_x"][side, slots, head].astype(np.float64))
                    continue
                x = tq6.decode_blocks(s["ring_d"][side, slots, head], s["ring_u"][side, slots, head])
                lst.append(rotation.inverse_exact(x.reshape(len(slots), self.D), self.D, self.signs))
        return np.concatenate(ks), np.concatenate(vs)

    def attention(self, layer, seq, q16, scale: float) -> np.ndarray:
        """q16 (H_q, D) -> float64 (H_q, D)."""
        keys, vals = [], []
        for h in range(self.H):
            k, v = self.head_kv(seq, layer, h)
            keys.append(k)
            vals.append(v)
        return attention.attend_gqa(np.asarray(q16, np.float16).astype(np.float64), keys, vals, scale)

    def attention_block(self, layer, seq, q16, scale: float) -> np.ndarray:
        """Causal attention of the newest n_q cached tokens' queries.
        q16 (n_q, H_q, D): query t belongs to the token at position
        n_tok - n_q + t and sees every cached token up to that position,
        whichever region holds it.  -> float64 (n_q, H_q, D)."""
        q = np.asarray(q16, np.float16).astype(np.float64)
        n_q = q.shape[0]
        n_tok = self._state(seq, layer)["n_tok"]
        if not 1 <= n_q <= n_tok:
            raise ValueError("the query block must be among the cached tokens")
        keys, vals = [], []
        for h in range(self.H):
            k, v = self.head_kv(seq, layer, h)
            keys.append(k)
            vals.append(v)
        return attention.attend_causal_gqa(q, keys, vals, n_tok - n_q, scale)
