"""Builds the same cache twice, through the HIP library and through the oracle,
from the same seeded inputs and the same append/seal schedule, and compares
them with the parity rules:

* sink and ring bytes: bit-exact;
* records: column scales C within 1e-3 relative of the oracle's; given the
  GPU's own C, the codes, S and Z the oracle's rounding produces from the same
  tile must equal the GPU's bit for bit, except codes whose pre-rounding value
  lies within 1e-6 relative of a rounding midpoint (counted);
* attention: max |o_gpu - o_ref| / rms(o_ref) <= 2e-3 against float64 attention
  over the same cache.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import cache as ocache
from oracle import record, rotation, rounding, tq6
from quantized_kv_cache_seal_amd import inputs, kvq

ATTN_TOL = 2e-3
SCALE_TOL = 1e-3
BOUNDARY_REL = 1e-6


def seq_spec(w, s):
    return inputs.KVSpec(w.n_layers, w.n_kv_heads, w.head_dim, w.seed + 7919 * s, w.k_dist,
                         w.outliers, w.outlier_scale)


class Pair:
    def __init__(self, w, lens, signs=None, extra_ctx=0):
        """extra_ctx: room for that many more tokens per sequence after build()."""
        import torch
        self.w, self.lens, self.signs = w, list(lens), signs
        self.n = len(lens)
        words = inputs.signs_to_words(signs) if signs is not None else [0, 0, 0, 0]
        max_ctx = max(lens) + extra_ctx
        self.gpu = kvq.Cache(kvq.config_for(w, max_ctx=max_ctx, max_seqs=self.n, sign_words=words))
        self.ora = ocache.OracleCache(w.n_layers, w.n_kv_heads, w.head_dim, w.n_q_heads, self.n, max_ctx,
                                      w.tail_min, w.tail_max, w.margin, w.k_bits, w.v_bits, w.passes, signs,
                                      stage=w.stage)
        self.specs = [seq_spec(w, s) for s in range(self.n)]
        self.kv = {}   # (s, layer) -> (k, v) fp16 numpy [len][H][D]
        for s in range(self.n):
            for l in range(w.n_layers):
                self.kv[(s, l)] = (self.specs[s].tokens(l, "k", 0, lens[s]), self.specs[s].tokens(l, "v", 0, lens[s]))
        self.torch = torch

    def _append(self, layer, seqs, t0, n):
        t = self.torch
        k = np.stack([self.kv[(s, layer)][0][t0:t0 + n] for s in seqs])
        v = np.stack([self.kv[(s, layer)][1][t0:t0 + n] for s in seqs])
        self.gpu.append(layer, seqs, t.from_numpy(k).cuda(), t.from_numpy(v).cuda())
        assert self.ora.append(layer, seqs, k, v) == ocache.OK

    def build(self, chunk, seal_to_min=True, seal_every=True):
        """Append every sequence in chunks of `chunk` tokens (all sequences with a
        full chunk left in one call, then the ragged remainders one sequence at a
        time), checking the seal rule after each round."""
        pos = [0] * self.n
        while any(p < L for p, L in zip(pos, self.lens)):
            full = [s for s in range(self.n) if self.lens[s] - pos[s] >= chunk]
            if full:
                assert len({pos[s] for s in full}) == 1
                for l in range(self.w.n_layers):
                    self._append(l, full, pos[full[0]], chunk)
                for s in full:
                    pos[s] += chunk
            else:
                for s in range(self.n):
                    rest = self.lens[s] - pos[s]
                    if rest > 0:
                        for l in range(self.w.n_layers):
                            self._append(l, [s], pos[s], rest)
                        pos[s] += rest
            if seal_every:
                assert self.gpu.seal(-1, kvq.SEAL_IF_FULL) == self.ora.seal(-1, ocache.SEAL_IF_FULL)
        if seal_to_min:
            assert self.gpu.seal(-1, kvq.SEAL_TO_MIN) == self.ora.seal(-1, ocache.SEAL_TO_MIN)
        self.torch.cuda.synchronize()
        return self

    # ------------------------------------------------------------ byte parity
    def check_info(self):
        for s in range(self.n):
            for l in range(self.w.n_layers):
                assert self.gpu.info(s, l) == self.ora.info(s, l), (s, l)

    def check_sink_ring(self):
        n_units = 0
        for s in range(self.n):
            for l in range(self.w.n_layers):
                nt, nr, ring = self.ora.info(s, l)
                for h in range(self.w.n_kv_heads):
                    for t in range(min(nt, 128)):
                        assert self.gpu.export(s, l, h, kvq.REGION_SINK, t) == \
                            self.ora.export(s, l, h, ocache.REGION_SINK, t), ("sink", s, l, h, t)
                        n_units += 1
                    for t in range(128 + 128 * nr, nt):
                        slot = (t - 128) % self.ora.cap
                        g = self.gpu.export(s, l, h, kvq.REGION_RING, slot)
                        o = self.ora.export(s, l, h, ocache.REGION_RING, slot)
                        assert g == o, ("ring", s, l, h, t, slot)
                        n_units += 1
        return n_units

    def tile_inputs(self, s, l, h, r, side):
        """Rotated, tq6-staged fp32 tile of record r, recomputed from the inputs
        (f16 staging: the rotation alone)."""
        x16 = self.kv[(s, l)][side][128 + 128 * r:256 + 128 * r, h]
        if self.w.stage == "f16":
            return rotation.rotate(x16, self.w.head_dim, self.signs)
        x = rotation.rotate(x16, self.w.head_dim, self.signs).reshape(128, -1, 128)
        d, u = tq6.encode_blocks(x)
        return tq6.decode_blocks(d, u).reshape(128, self.w.head_dim)

    def check_records(self):
        stats = {"codes": 0, "boundary": 0, "uncond_mismatch": 0, "c_flips": 0, "scales": 0, "max_c_rel": 0.0}
        w = self.w
        sub = record.sub_width(w.head_dim)
        for s in range(self.n):
            for l in range(w.n_layers):
                nr = self.ora.info(s, l)[1]
                for h in range(w.n_kv_heads):
                    for r in range(nr):
                        gb = self.gpu.export(s, l, h, kvq.REGION_BODY, r)
                        ob = self.ora.export(s, l, h, ocache.REGION_BODY, r)
                        gsubs = record.parse_record(gb, w.head_dim, w.k_bits, w.v_bits)
                        osubs = record.parse_record(ob, w.head_dim, w.k_bits, w.v_bits)
                        for side, bits in ((0, w.k_bits), (1, w.v_bits)):
                            x = self.tile_inputs(s, l, h, r, side)
                            for i in range(len(gsubs)):
                                g, o = gsubs[i][side], osubs[i][side]
                                xs = x[:, i * sub:(i + 1) * sub]
                                rel = np.abs(g["C"].astype(np.float64) / o["C"].astype(np.float64) - 1)
                                stats["max_c_rel"] = max(stats["max_c_rel"], float(rel.max()))
                                assert rel.max() <= SCALE_TOL, ("C", s, l, h, r, side, i, rel.max())
                                codes, S, Z = rounding.round_rows(xs, g["C"], bits)
                                assert np.array_equal(S, g["S"]) and np.array_equal(Z, g["Z"]), ("SZ", s, l, h, r, side)
                                bad = codes != g["codes"]
                                if bad.any():
                                    t = rounding.pre_round_values(xs, g["C"], g["S"], g["Z"])
                                    k = np.floor(t[bad])
                                    mid = np.abs(t[bad] - (k + 0.5)) <= BOUNDARY_REL * np.abs(k + 0.5)
                                    assert mid.all(), ("codes", s, l, h, r, side, int(bad.sum()))
                                    stats["boundary"] += int(bad.sum())
                                stats["codes"] += codes.size
                                stats["scales"] += 1
                                # against the oracle's own codes: a code may differ only
                                # where the inputs of its rounding differ (its column's
                                # fp16 C, or its row's S or Z, which a flip of C moves)
                                # or where it is a counted boundary code
                                mism = g["codes"] != o["codes"]
                                why = ((g["C"] != o["C"])[None, :] | (g["S"] != o["S"])[:, None]
                                       | (g["Z"] != o["Z"])[:, None])
                                if bad.any():
                                    why = why | bad
                                assert not (mism & ~why).any(), ("unexplained code", s, l, h, r, side, i)
                                stats["uncond_mismatch"] += int(mism.sum())
                                stats["c_flips"] += int((g["C"] != o["C"]).sum())
        return stats

    def import_oracle_records(self, first=0):
        """Copy the oracle's records (from record index `first` on) into the GPU cache."""
        for s in range(self.n):
            for l in range(self.w.n_layers):
                for h in range(self.w.n_kv_heads):
                    for r in range(first, self.ora.info(s, l)[1]):
                        self.gpu.import_(s, l, h, kvq.REGION_BODY, r, self.ora.export(s, l, h, ocache.REGION_BODY, r))

    def own_record_errors(self, layer, q16, scale=1.0):
        """The decode criterion on a GPU-built cache (the GPU's exported records
        dequantised by the oracle): max |o_gpu - o_ref| / rms(o_ref) per sequence
        against float64 attention over the GPU's own records, and, for the
        record, the float64 difference the GPU's records make against the
        oracle's (fp16 flips of C).  The oracle's records are restored."""
        t = self.torch
        out = self.gpu.attn_decode(layer, list(range(self.n)), t.from_numpy(q16).cuda(), scale=scale)
        got = out.float().cpu().numpy().astype(np.float64)
        errs, cross = [], []
        for s in range(self.n):
            ref_o = self.ora.attention(layer, s, q16[s], scale)
            saved = {}
            for h in range(self.w.n_kv_heads):
                for r in range(self.ora.info(s, layer)[1]):
                    saved[(h, r)] = self.ora.export(s, layer, h, ocache.REGION_BODY, r)
                    self.ora.import_record(s, layer, h, r, self.gpu.export(s, layer, h, kvq.REGION_BODY, r))
            ref_g = self.ora.attention(layer, s, q16[s], scale)
            for (h, r), buf in saved.items():
                self.ora.import_record(s, layer, h, r, buf)
            rms = math.sqrt(np.mean(ref_g ** 2))
            errs.append(float(np.max(np.abs(got[s] - ref_g)) / rms))
            cross.append(float(np.max(np.abs(ref_g - ref_o)) / rms))
        return errs, cross

    # ------------------------------------------------------------ attention
    def queries(self, step, layer):
        return inputs.queries(self.w.seed, step, layer, self.n, self.w.n_q_heads, self.w.head_dim)

    def decode_errors(self, layer, q16, scale=1.0, path=kvq.PATH_AUTO, out_f16=False):
        t = self.torch
        self.gpu.set_decode_path(path)
        out = self.gpu.attn_decode(layer, list(range(self.n)), t.from_numpy(q16).cuda(), scale=scale,
                                   out_f16=out_f16)
        got = out.float().cpu().numpy().astype(np.float64)
        errs = []
        for s in range(self.n):
            ref = self.ora.attention(layer, s, q16[s], scale)
            errs.append(float(np.max(np.abs(got[s] - ref)) / math.sqrt(np.mean(ref ** 2))))
        return errs, got
