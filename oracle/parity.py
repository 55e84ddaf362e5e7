"""Comparison of GPU outputs with the oracle's, block by block -- TEST
INFRASTRUCTURE ONLY (used by the tests, the smoke check and the benchmark's
validation before timing; never by the product path).

Quant-only casts must match bit for bit.  The fused casts compute their
activation in fp32 with hardware exp2/reciprocal, so a value may land one
bf16 step away from the exact one; the bar (from "Add swiglu + MXFP8 fused
CuTe DSL kernel", Numerics and tests, which allows one-code differences in
backward data):
  - E4M3 codes within one step of the oracle's (signed ordinal distance,
    +0 and -0 equal), except in invalid (NaN/Inf) blocks, which must match
    exactly (scale 255, data 0x7F);
  - scales bit-exact, except in blocks whose exact amax lies within one
    bf16 step of a power-of-two scale boundary: there the GPU scale may be
    the neighbouring one, its data is then compared with the oracle's
    values quantized at the GPU's scale, and such blocks must be at most
    1e-4 of all blocks (at least one allowed in small cases).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np



def e4m3_ordinal(codes: np.ndarray) -> np.ndarray:
    """Signed position of an E4M3 code on the number line (+0 and -0 both 0)."""
    c = np.asarray(codes).astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


@dataclass
class Stats:
    blocks: int = 0
    scale_mismatch: int = 0
    code_off_by_one: int = 0
    elements: int = 0
    notes: list = field(default_factory=list)

    def merge(self, o: "Stats") -> "Stats":
        return Stats(self.blocks + o.blocks, self.scale_mismatch + o.scale_mismatch,
                     self.code_off_by_one + o.code_off_by_one, self.elements + o.elements, self.notes + o.notes)

    @property
    def scale_mismatch_rate(self) -> float:
        """Blocks whose scale differs from the oracle's, over all blocks."""
        return self.scale_mismatch / max(1, self.blocks)

    @property
    def one_code_rate(self) -> float:
        """Elements one E4M3 step from the oracle's code, over all elements."""
        return self.code_off_by_one / max(1, self.elements)

    def record(self) -> dict:
        return {"blocks": self.blocks, "scale_mismatch": self.scale_mismatch,
                "scale_mismatch_rate": self.scale_mismatch_rate, "elements": self.elements,
                "one_code": self.code_off_by_one, "one_code_rate": self.one_code_rate}


def assert_exact(name, got, want):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{name}: {len(bad)} mismatches, first at {bad[:5].tolist()}: got {got[tuple(bad[0])]:#x} want {want[tuple(bad[0])]:#x}"


def _near_boundary(oracle, amax_bits: np.ndarray) -> np.ndarray:
    """True where a one-step change of the bf16 amax changes the RCEIL byte."""
    out = np.zeros(amax_bits.shape, bool)
    for idx, a in np.ndenumerate(amax_bits):
        a = int(a)
        b = oracle.e8m0_rceil(oracle.bf16_decode(a))
        for nb in (a - 1, a + 1):
            if 0 <= nb < 0x7F80 and oracle.e8m0_rceil(oracle.bf16_decode(nb)) != b:
                out[idx] = True
    return out


def compare_blocks(oracle, name, q_gpu, s_gpu, q_orc, s_orc, values_bits) -> Stats:
    """Compare one layout.  All arrays are arranged as [rows, blocks, 32]
    (q and values) and [rows, blocks] (scales), in the same order."""
    q_gpu = np.asarray(q_gpu)
    q_orc = np.asarray(q_orc)
    assert q_gpu.shape == q_orc.shape and s_gpu.shape == s_orc.shape, name
    st = Stats(blocks=int(s_orc.size), elements=int(q_orc.size))
    invalid = s_orc == 255
    # invalid blocks: exact
    assert (s_gpu[invalid] == 255).all(), f"{name}: GPU missed a NaN/Inf block"
    assert (q_gpu[invalid] == 0x7F).all(), f"{name}: invalid block data must be 0x7F"
    assert not (s_gpu[~invalid] == 255).any(), f"{name}: GPU flagged a finite block as invalid"
    same = (s_gpu == s_orc) & ~invalid
    d = np.abs(e4m3_ordinal(q_gpu) - e4m3_ordinal(q_orc))
    dsame = d[same]
    assert dsame.max(initial=0) <= 1, f"{name}: code differs by {dsame.max()} steps"
    st.code_off_by_one += int((dsame == 1).sum())
    diff = ~same & ~invalid
    if diff.any():
        idx = np.argwhere(diff)
        st.scale_mismatch = len(idx)
        vals = np.asarray(values_bits)
        amax = (vals[diff] & 0x7FFF).max(axis=-1)
        assert (np.abs(s_gpu[diff].astype(int) - s_orc[diff].astype(int)) == 1).all(), f"{name}: scale off by >1"
        near = _near_boundary(oracle, amax)
        assert near.all(), f"{name}: scale mismatch away from a power-of-two boundary at {idx[~near][:5].tolist()}"
        for (r, b) in idx:
            y = (vals[r, b].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            q_at = oracle.quant_block_at(y, int(s_gpu[r, b]))
            dd = np.abs(e4m3_ordinal(q_gpu[r, b]) - e4m3_ordinal(q_at))
            assert dd.max() <= 1, f"{name}: block ({r},{b}) at the GPU scale differs by {dd.max()}"
            st.code_off_by_one += int((dd == 1).sum())
    allowed = max(1, int(1e-4 * st.blocks))
    assert st.scale_mismatch <= allowed, f"{name}: {st.scale_mismatch} scale mismatches of {st.blocks} blocks"
    return st


def rowwise_view(q, s, values):
    M, W = q.shape
    return q.reshape(M, W // 32, 32), s.reshape(M, W // 32), values.reshape(M, W // 32, 32)


def colwise_view(q, s, values):
    """q, s are [W, M], [W, M/32]; values is the [M, W] matrix."""
    W, M = q.shape
    vt = np.ascontiguousarray(values.T)
    return q.reshape(W, M // 32, 32), s.reshape(W, M // 32), vt.reshape(W, M // 32, 32)


def compare_fused(oracle, name, gpu, orc, values, layout) -> Stats:
    """gpu / orc: (q_row, s_row, q_col, s_col) numpy tuples; values: [M, W] bf16 bits.
    The returned Stats covers every enabled layout; ``.notes`` holds the
    per-layout Stats as ("row" | "col", Stats) pairs."""
    st = Stats()
    if layout & 1:
        part = compare_blocks(oracle, name + "/row", *rowwise_view(gpu[0], gpu[1], values)[:2],
                              *rowwise_view(orc[0], orc[1], values))
        st = st.merge(part)
        st.notes.append(("row", part))
    if layout & 2:
        part = compare_blocks(oracle, name + "/col", *colwise_view(gpu[2], gpu[3], values)[:2],
                              *colwise_view(orc[2], orc[3], values))
        st = st.merge(part)
        st.notes.append(("col", part))
    rate = st.code_off_by_one / max(1, st.elements)
    assert rate <= 1e-3, f"{name}: one-step code differences on {rate:.2e} of elements"
    return st


def layout_parts(st: Stats) -> dict:
    """{"row" | "col": Stats} of a compare_fused result (merged when the
    result itself merges several comparisons)."""
    out = {}
    for lay, part in st.notes:
        out[lay] = out[lay].merge(part) if lay in out else part
    return out
