"""GPU parity of the grouped (mixture-of-experts) consumers of the casts and
of the per-group padded colwise scale layout.

"[mxfp8 moe training] add compile support", Perf analysis: the casts feed
grouped GEMMs (forward and input gradient grouped along the token rows, the
weight gradient contracting over each expert's tokens); Summary and review
comments: per-group scale buffers sized by an upper bound, offsets left on
the device.  "[mxfp8 moe training] update 3d quant colwise scaling kernel to
use single input/output TMA descriptors", Summary: the 3D cast's column-
major-per-expert output is the input gradient's expert operand.

The GEMMs are held to the matrix-core error bound (tests/gemm_bounds.py);
the plain casts are bit-exact, so a pipeline that starts from bf16 inputs
gives the GEMM the same operands on both sides.
"""
import numpy as np
import pytest
import torch

import swiglu_activation_cast_amd as mx
from swiglu_activation_cast_amd import synth
from gemm_bounds import check
from helpers import torch_bf16_to_bits
from oracle.parity import assert_exact

pytestmark = pytest.mark.gpu

ROW, COL, BOTH = 1, 2, 3


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _np(t):
    return t.cpu().numpy()


def _t(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


# ------------------------------------------------- input gradient (dgrad)
@pytest.mark.parametrize("offs", [[130, 400, 400, 1000], [1000, 1000, 1000, 1000], [0, 0, 999, 1000]])
def test_dgrad_grouped_gemm_on_the_3d_cast(oracle_mod, offs):
    """dx = dy W_g per expert: A = rowwise cast of dy [M, N] (blocks along
    N), B_g = the 3D colwise cast of W (E, N, K), whose expert g is the
    [K, N] operand with blocks along N, consumed as it is written."""
    dev = _dev()
    E, N, K, M = 4, 512, 384, 1000
    print(f"case: dgrad grouped gemm on the 3D cast, offsets {offs}", flush=True)
    dy = synth.normal_bf16((M, N), 1.0, seed=90, device=dev)
    w = synth.expert_weights(E, N, K, seed=91, std=0.05, device=dev)
    qa, _, sa, _ = mx.mxfp8_quant_2d(dy, rowwise=True)
    q3, s3 = mx.mxfp8_quant_3d_colwise(w)
    offs_t = torch.tensor(offs, dtype=torch.int32, device=dev)
    c = mx.mxfp8_grouped_gemm(qa, sa, q3, s3, offs_t)
    # the oracle's own casts of the same bf16 inputs, then its grouped GEMM
    oq, osc, _, _ = oracle_mod.quant_2d(torch_bf16_to_bits(dy), ROW)
    o3q, o3s = oracle_mod.quant_3d_colwise(torch_bf16_to_bits(w))
    assert_exact("dy q", _np(qa), oq)
    assert_exact("dy s", _np(sa), osc)
    assert_exact("w q3", _np(q3), o3q)
    assert_exact("w s3", _np(s3), o3s)
    want, mag = oracle_mod.mx_grouped_gemm(oq, osc, o3q, o3s, np.array(offs, np.int32))
    got = _np(c)
    start = 0
    for g in range(E):
        end = int(min(max(offs[g], start), M))
        if end > start:
            worst = check(f"dgrad g{g}", got[start:end], want[start:end], mag[start:end], oq[start:end],
                          osc[start:end], o3q[g], o3s[g])
            print(f"  group {g}: rows {start}..{end}, worst {worst:.3f} of the bound")
        start = end


def test_dgrad_16640x5120x8192_g4_sampled(oracle_mod):
    """The pages' grouped shape as the input gradient: 16640 tokens over 4
    experts, dx [16640, 5120] = dy [16640, 8192] W_g [8192, 5120]; sampled
    rows of every group and sampled columns."""
    dev = _dev()
    M, N, K, E = 16640, 8192, 5120, 4
    print(f"case: dgrad grouped gemm {M}x{K}x{N} E={E}, sampled", flush=True)
    dy = synth.normal_bf16((M, N), 1.0, seed=92, device=dev)
    w = synth.expert_weights(E, N, K, seed=93, std=0.02, device=dev)
    qa, _, sa, _ = mx.mxfp8_quant_2d(dy, rowwise=True)
    q3, s3 = mx.mxfp8_quant_3d_colwise(w)
    offs = np.array([3000, 7100, 12000, 16640], np.int32)
    c = mx.mxfp8_grouped_gemm(qa, sa, q3, s3, _t(offs, dev))
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    cols = np.unique(np.concatenate([[0, K - 1], rng.integers(0, K, 14)]))
    start = 0
    for g in range(E):
        end = int(offs[g])
        rows = np.unique(np.concatenate([[start, end - 1], rng.integers(start, end, 6)]))
        ridx = _t(rows, dev)
        oq, osc, _, _ = oracle_mod.quant_2d(torch_bf16_to_bits(dy[ridx]), ROW)
        # expert g's [K, N] operand: the 3D oracle on the sampled K columns of W_g
        o3q, o3s = oracle_mod.quant_3d_colwise(torch_bf16_to_bits(w[g][:, _t(cols, dev)]).reshape(1, N, len(cols)))
        assert_exact(f"g{g} dy q", _np(qa[ridx]), oq)
        assert_exact(f"g{g} w q3", _np(q3[g][_t(cols, dev)]), o3q[0])
        want, mag = oracle_mod.mx_gemm(oq, osc, o3q[0], o3s[0])
        check(f"g{g}", _np(c[ridx][:, _t(cols, dev)]), want, mag, oq, osc, o3q[0], o3s[0])
        start = end
    del dy, w, qa, sa, q3, s3, c
    torch.cuda.empty_cache()


# ------------------------------------------- per-group padded colwise scales
def _expected_padded(oracle_mod, plain, M, offs, width):
    """The plain colwise scales [W, M/32] placed where the oracle's layout
    puts them; unused positions zero."""
    st, en = oracle_mod.group_bounds(offs, M)
    out = np.zeros((plain.shape[0], width), np.uint8)
    for g in range(len(offs) + 1):
        base = oracle_mod.group_scale_base(g, st[g])
        out[:, base:base + (en[g] - st[g]) // 32] = plain[:, st[g] // 32:en[g] // 32]
    return out


CAST_CASES = [
    (640, [64, 64, 320, 608]),          # an empty group and a tail
    (640, [100, 50, 2000]),             # unrounded, decreasing and past-the-end ends
    (512, [-5, 96, 96, 700]),
    (1024, [1024]),                     # one group: the plain layout
    (4096, "100 random"),               # more groups than a wavefront has lanes
    (32768, "1024 equal"),              # the most groups
]


def _offsets(M, spec, rng):
    if isinstance(spec, list):
        return spec
    n = int(spec.split()[0])
    if spec.endswith("equal"):
        return [(g + 1) * (M // n) for g in range(n)]
    return np.sort(rng.integers(0, M // 32 + 1, n) * 32).tolist()


@pytest.mark.parametrize("kind", ["quant", "fwd", "bwd"])
@pytest.mark.parametrize("M,spec", CAST_CASES)
def test_grouped_cast_padded_scales(oracle_mod, kind, M, spec):
    """Every output of a grouped cast equals the ungrouped cast's, except
    that the colwise scales sit in the per-group padded layout (the oracle's
    positions); positions no block maps to are left untouched."""
    dev = _dev()
    rng = np.random.default_rng(M)
    offs = _offsets(M, spec, rng)
    G = len(offs)
    N = 160 if M <= 4096 else 64
    print(f"case: grouped {kind} cast M={M} N={N} G={G}", flush=True)
    offs_t = torch.tensor(offs, dtype=torch.int32, device=dev)
    inp = synth.swiglu_inputs(M, N, seed=M + G, std=2.0, device=dev)
    if kind == "quant":
        grouped = mx.mxfp8_quant_2d_grouped(inp.gate, offs_t, rowwise=True, colwise=True)
        plain = mx.mxfp8_quant_2d(inp.gate, rowwise=True, colwise=True)
    elif kind == "fwd":
        grouped = mx.mxfp8_gated_fwd_grouped(inp.gate, inp.up, offs_t, rowwise=True, colwise=True)
        plain = mx.mxfp8_swiglu_fwd(inp.gate, inp.up, rowwise=True, colwise=True)
    else:
        grouped = mx.mxfp8_gated_bwd_grouped(inp.dh, inp.gate, inp.up, offs_t, rowwise=True, colwise=True)
        plain = mx.mxfp8_swiglu_bwd(inp.dh, inp.gate, inp.up, rowwise=True, colwise=True)
    for i, name in ((0, "q_row"), (1, "q_col"), (2, "s_row")):
        assert torch.equal(grouped[i], plain[i]), name
    s_pad = _np(grouped[3])
    assert s_pad.shape[1] == M // 32 + 16 * G
    want = _expected_padded(oracle_mod, _np(plain[3]), M, offs, s_pad.shape[1])
    assert_exact("s_col padded", s_pad, want)
    if kind == "quant":
        # exact cast: the oracle's own scales in the oracle's padded layout
        _, _, _, os_col = oracle_mod.quant_2d(torch_bf16_to_bits(inp.gate), COL)
        assert_exact("s_col vs oracle", s_pad, oracle_mod.pad_group_scales(os_col, M, offs, fill=0))


def test_grouped_cast_guard_bytes():
    """A padded scale buffer wider than needed, inside a larger 0xA5 buffer:
    only the used positions change."""
    dev = _dev()
    M, K, offs = 256, 96, [64, 200, 256]
    x = synth.normal_bf16((M, K), 1.0, seed=7, device=dev)
    width = M // 32 + 16 * len(offs)
    big = torch.full((K + 2, width + 24), 0xA5, dtype=torch.uint8, device=dev)
    s_view = big[1:K + 1, :width]
    q = torch.empty((K, M), dtype=torch.uint8, device=dev)
    empty = torch.empty(0, dtype=torch.uint8, device=dev)
    mx.mxfp8_quant_2d_grouped(x, torch.tensor(offs, dtype=torch.int32, device=dev), rowwise=False, colwise=True,
                              out=(empty, q, empty, s_view))
    plain = mx.mxfp8_quant_2d(x, rowwise=False, colwise=True)
    torch.cuda.synchronize()
    assert torch.equal(q, plain[1])
    assert (big[0] == 0xA5).all() and (big[K + 1] == 0xA5).all() and (big[:, width:] == 0xA5).all()
    used = torch.zeros(width, dtype=torch.bool)
    st = [0, 64, 192, 256]  # 200 rounds down to 192
    for g in range(4):
        base = 16 * (g + st[g] // 512)
        n = ((st[g + 1] if g < 3 else 256) - st[g]) // 32
        used[base:base + n] = True
    assert (s_view[:, ~used.to(dev)] == 0xA5).all()


# ------------------------------------------------ weight gradient (wgrad)
KGEMM_CASES = [(640, [64, 64, 320, 608]), (1024, [1024]), (512, [96, 50, 700]), (2048, [0, 512, 1536, 2048]),
               (320, [-3, 128, 128, 1000]), (5216, [1000, 2016, 5216])]


@pytest.mark.parametrize("T,offs", KGEMM_CASES)
def test_grouped_gemm_k_random(oracle_mod, T, offs):
    dev = _dev()
    print(f"case: K-grouped gemm T={T} offsets {offs}", flush=True)
    rng = np.random.default_rng(T + len(offs))
    M, N = 200, 300

    def operand(rows):
        codes = rng.integers(0, 256, (rows, T)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x3A  # no NaN codes
        plain = rng.integers(118, 137, (rows, T // 32)).astype(np.uint8)
        return codes, plain, oracle_mod.pad_group_scales(plain, T, offs, fill=127)

    a, sa, sap = operand(M)
    b, sb, sbp = operand(N)
    out = torch.full((len(offs), M, N), -3.0, dtype=torch.float32, device=dev)
    mx.mxfp8_grouped_gemm_k(_t(a, dev), _t(sap, dev), _t(b, dev), _t(sbp, dev),
                            torch.tensor(offs, dtype=torch.int32, device=dev), out=out)
    want, mag = oracle_mod.mx_grouped_gemm_k(a, sap, b, sbp, offs)
    got = _np(out)
    st, en = oracle_mod.group_bounds(offs, T)
    for g in range(len(offs)):
        if en[g] == st[g]:
            assert np.all(got[g] == 0), g
            continue
        sl, bl = slice(st[g], en[g]), slice(st[g] // 32, en[g] // 32)
        check(f"g{g}", got[g], want[g], mag[g], a[:, sl], sa[:, bl], b[:, sl], sb[:, bl])


def test_wgrad_pipeline_from_grouped_casts(oracle_mod):
    """dW_g = dy_g^T x_g: the colwise grouped casts of dy [T, N] and x [T, K]
    (codes [N, T] and [K, T], padded scales) feed the K-grouped GEMM as they
    are written; the oracle runs the same chain from the same bf16 inputs."""
    dev = _dev()
    T, N, K = 1024, 192, 160
    offs = [96, 96, 512, 1000]
    print(f"case: wgrad pipeline T={T} N={N} K={K} offsets {offs}", flush=True)
    dy = synth.normal_bf16((T, N), 1.0, seed=94, device=dev)
    x = synth.normal_bf16((T, K), 1.0, seed=95, device=dev)
    offs_t = torch.tensor(offs, dtype=torch.int32, device=dev)
    _, qa, _, sa = mx.mxfp8_quant_2d_grouped(dy, offs_t)
    _, qb, _, sb = mx.mxfp8_quant_2d_grouped(x, offs_t)
    c = mx.mxfp8_grouped_gemm_k(qa, sa, qb, sb, offs_t)
    _, _, oqa, osa = oracle_mod.quant_2d(torch_bf16_to_bits(dy), COL)
    _, _, oqb, osb = oracle_mod.quant_2d(torch_bf16_to_bits(x), COL)
    osa_p = oracle_mod.pad_group_scales(osa, T, offs, fill=0)
    osb_p = oracle_mod.pad_group_scales(osb, T, offs, fill=0)
    assert_exact("dy^T q", _np(qa), oqa)
    assert_exact("dy^T s", _np(sa), osa_p)
    assert_exact("x^T q", _np(qb), oqb)
    assert_exact("x^T s", _np(sb), osb_p)
    want, mag = oracle_mod.mx_grouped_gemm_k(oqa, osa_p, oqb, osb_p, offs)
    got = _np(c)
    st, en = oracle_mod.group_bounds(offs, T)
    for g in range(len(offs)):
        if en[g] == st[g]:
            assert np.all(got[g] == 0)
            continue
        sl, bl = slice(st[g], en[g]), slice(st[g] // 32, en[g] // 32)
        check(f"wgrad g{g}", got[g], want[g], mag[g], oqa[:, sl], osa[:, bl], oqb[:, sl], osb[:, bl])
    # and the result is close to the bf16 weight gradient of each group
    for g in range(len(offs)):
        if en[g] > st[g]:
            ref = dy[st[g]:en[g]].float().t() @ x[st[g]:en[g]].float()
            rel = ((c[g] - ref).norm() / ref.norm()).item()
            assert rel < 0.08, (g, rel)


def test_wgrad_16640x8192x5120_g4_sampled(oracle_mod):
    """The pages' grouped shape as the weight gradient: 16640 tokens over 4
    experts, dW_g [8192, 5120] = dy_g^T x_g; sampled rows and columns of
    every group's result, the oracle casting the sampled columns itself."""
    dev = _dev()
    T, N, K = 16640, 8192, 5120
    offs = np.array([3008, 7104, 12000, 16640], np.int32)
    print(f"case: wgrad K-grouped gemm {N}x{K}, T={T}, G=4, sampled", flush=True)
    dy = synth.normal_bf16((T, N), 1.0, seed=96, device=dev)
    x = synth.normal_bf16((T, K), 1.0, seed=97, device=dev)
    offs_t = _t(offs, dev)
    _, qa, _, sa = mx.mxfp8_quant_2d_grouped(dy, offs_t)
    _, qb, _, sb = mx.mxfp8_quant_2d_grouped(x, offs_t)
    c = mx.mxfp8_grouped_gemm_k(qa, sa, qb, sb, offs_t)
    torch.cuda.synchronize()
    rng = np.random.default_rng(14)
    rows = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 10)]))
    cols = np.unique(np.concatenate([[0, K - 1], rng.integers(0, K, 18)]))
    _, _, oqa, osa = oracle_mod.quant_2d(torch_bf16_to_bits(dy[:, _t(rows, dev)]), COL)
    _, _, oqb, osb = oracle_mod.quant_2d(torch_bf16_to_bits(x[:, _t(cols, dev)]), COL)
    osa_p = oracle_mod.pad_group_scales(osa, T, offs, fill=0)
    osb_p = oracle_mod.pad_group_scales(osb, T, offs, fill=0)
    assert_exact("dy^T q", _np(qa[_t(rows, dev)]), oqa)
    assert_exact("dy^T s", _np(sa[_t(rows, dev)]), osa_p)
    want, mag = oracle_mod.mx_grouped_gemm_k(oqa, osa_p, oqb, osb_p, offs)
    got = _np(c[:, _t(rows, dev)][:, :, _t(cols, dev)])
    st, en = oracle_mod.group_bounds(offs, T)
    for g in range(4):
        sl, bl = slice(st[g], en[g]), slice(st[g] // 32, en[g] // 32)
        check(f"wgrad g{g}", got[g], want[g], mag[g], oqa[:, sl], osa[:, bl], oqb[:, sl], osb[:, bl])
    del dy, x, qa, sa, qb, sb, c
    torch.cuda.empty_cache()
