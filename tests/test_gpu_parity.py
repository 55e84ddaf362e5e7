"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Quant-only casts (2D and 3D) must be bit-exact.  Fused SwiGLU casts follow
the tolerance in oracle/parity.py.  Inputs come from the seeded generators in
swiglu_activation_cast_amd.synth (or are built explicitly for edge cases);
the oracle reads back the exact device bytes.
"""
import numpy as np
import pytest
import torch

import swiglu_activation_cast_amd as mx
from swiglu_activation_cast_amd import synth
from concurrent.futures import ThreadPoolExecutor

from helpers import all_bf16_bits, bits_to_torch_bf16, record_rates, torch_bf16_to_bits
from oracle.parity import assert_exact, compare_fused

pytestmark = pytest.mark.gpu

ROW, COL, BOTH = 1, 2, 3
LAYOUTS = (ROW, COL, BOTH)
_LNAME = {ROW: "rowwise launch", COL: "colwise launch", BOTH: "both-layout launch"}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _np(t):
    return t.cpu().numpy()


def _gpu(outs):
    """Binding order (q_row, q_col, s_row, s_col) -> oracle order (q_row, s_row, q_col, s_col)."""
    q_row, q_col, s_row, s_col = outs
    return _np(q_row), _np(s_row), _np(q_col), _np(s_col)


def _flags(layout):
    return dict(rowwise=bool(layout & ROW), colwise=bool(layout & COL))


def _to_dev(bits, dev):
    return bits_to_torch_bf16(bits).to(dev)


def _exact(name, gpu, orc, layout):
    if layout & ROW:
        assert_exact(name + "/q_row", gpu[0], orc[0])
        assert_exact(name + "/s_row", gpu[1], orc[1])
    if layout & COL:
        assert_exact(name + "/q_col", gpu[2], orc[2])
        assert_exact(name + "/s_col", gpu[3], orc[3])


def _fwd_check(oracle_mod, name, g_bits, u_bits, layout, dev):
    g, u = _to_dev(g_bits, dev), _to_dev(u_bits, dev)
    gpu = _gpu(mx.mxfp8_swiglu_fwd(g, u, **_flags(layout)))
    orc = oracle_mod.swiglu_fwd(g_bits, u_bits, layout)
    vals = oracle_mod.swiglu_fwd_values(np.ascontiguousarray(g_bits), np.ascontiguousarray(u_bits))
    return compare_fused(oracle_mod, name, gpu, orc, vals, layout)


def _bwd_check(oracle_mod, name, dh_bits, g_bits, u_bits, layout, dev):
    dh, g, u = _to_dev(dh_bits, dev), _to_dev(g_bits, dev), _to_dev(u_bits, dev)
    gpu = _gpu(mx.mxfp8_swiglu_bwd(dh, g, u, **_flags(layout)))
    orc = oracle_mod.swiglu_bwd(dh_bits, g_bits, u_bits, layout)
    dg, du = oracle_mod.swiglu_bwd_values(*(np.ascontiguousarray(a) for a in (dh_bits, g_bits, u_bits)))
    vals = np.concatenate([dg, du], axis=1)
    return compare_fused(oracle_mod, name, gpu, orc, vals, layout)


# ------------------------------------------------------------ quant-only, exact
def test_quant_2d_all_bf16_patterns(oracle_mod):
    dev = _dev()
    print("case: quant_2d all bf16 patterns [2048, 32]", flush=True)
    rng = np.random.default_rng(0)
    x = rng.permutation(all_bf16_bits()).reshape(2048, 32)
    gpu = _gpu(mx.mxfp8_quant_2d(_to_dev(x, dev), rowwise=True, colwise=True))
    _exact("all_patterns", gpu, oracle_mod.quant_2d(x, BOTH), BOTH)


def test_quant_2d_every_value_under_many_scales(oracle_mod):
    """Each block: one driver element at 448 * 2^k (fixing the scale to byte
    127 + k) and 31 finite bf16 values of smaller magnitude, covering every
    such value once per chosen k."""
    dev = _dev()
    bits = all_bf16_bits()
    mag = bits & 0x7FFF
    rng = np.random.default_rng(1)
    for k in (-127, -126, -100, -8, 0, 5, 60, 119, 120):
        print(f"case: quant_2d value sweep at scale byte {127 + k}", flush=True)
        # 448 * 2^120 overflows bf16: the largest finite bf16 drives byte 247
        driver = oracle_mod.bf16_round(448.0 * 2.0**k) if k < 120 else 0x7F7F
        pool = bits[(mag < 0x7F80) & (mag <= (driver & 0x7FFF))]
        pool = rng.permutation(pool)
        nblk = -(-pool.size // 31)
        body = np.resize(pool, nblk * 31).reshape(nblk, 31)
        x = np.concatenate([np.full((nblk, 1), driver, np.uint16), body], axis=1)
        gpu = _gpu(mx.mxfp8_quant_2d(_to_dev(x, dev), rowwise=True, colwise=False))
        orc = oracle_mod.quant_2d(x, ROW)
        assert (orc[1][:, 0] == 127 + k).all()
        _exact(f"sweep{k}", gpu, orc, ROW)


@pytest.mark.parametrize("M,K,layout", [(37, 96, ROW), (96, 40, COL), (160, 224, BOTH), (128, 64, COL),
                                        (32, 8, COL), (1, 32, ROW), (224, 1056, BOTH)])
def test_quant_2d_shapes(oracle_mod, M, K, layout):
    dev = _dev()
    print(f"case: quant_2d M={M} K={K} layout={layout}", flush=True)
    x = torch_bf16_to_bits(synth.normal_bf16((M, K), 2.0, seed=M * 7 + K))
    gpu = _gpu(mx.mxfp8_quant_2d(_to_dev(x, dev), **_flags(layout)))
    _exact(f"shape{M}x{K}", gpu, oracle_mod.quant_2d(x, layout), layout)


def test_quant_2d_strided_input(oracle_mod):
    dev = _dev()
    big = torch_bf16_to_bits(synth.normal_bf16((96, 320), 1.0, seed=5))
    x_dev = _to_dev(big, dev)[:, 64:256]  # ld = 320
    gpu = _gpu(mx.mxfp8_quant_2d(x_dev, rowwise=True, colwise=True))
    _exact("strided", gpu, oracle_mod.quant_2d(big[:, 64:256], BOTH), BOTH)


def test_quant_2d_e4m3_boundary_amax(oracle_mod):
    """amax exactly 448 * 2^k and one bf16 step either side."""
    dev = _dev()
    rows = []
    rng = np.random.default_rng(2)
    for k in range(-127, 121, 3):
        b = oracle_mod.bf16_round(448.0 * 2.0**k)
        for a in (b - 1, b, b + 1):
            row = np.zeros(32, np.uint16)
            row[:] = rng.integers(0, max(1, a), 32)
            row[rng.integers(0, 32)] = a | (0x8000 if rng.random() < 0.5 else 0)
            rows.append(row)
    x = np.stack(rows)
    x = x[: len(x) // 32 * 32]
    gpu = _gpu(mx.mxfp8_quant_2d(_to_dev(x, dev), rowwise=True, colwise=True))
    _exact("boundary", gpu, oracle_mod.quant_2d(x, BOTH), BOTH)


# ---------------------------------------------------------------- fused, small
@pytest.mark.parametrize("layout", LAYOUTS)
def test_swiglu_fwd_128x128(oracle_mod, layout):
    dev = _dev()
    print(f"case: fwd 128x128 seed 0 layout={layout}", flush=True)
    inp = synth.workload("swiglu_128x128")
    st = _fwd_check(oracle_mod, f"fwd128/{layout}", torch_bf16_to_bits(inp.gate), torch_bf16_to_bits(inp.up), layout,
                    dev)
    record_rates(f"swiglu_128x128 [{_LNAME[layout]}]", "fwd", st)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_swiglu_bwd_128x128(oracle_mod, layout):
    dev = _dev()
    print(f"case: bwd 128x128 seed 0 layout={layout}", flush=True)
    inp = synth.workload("swiglu_128x128")
    st = _bwd_check(oracle_mod, f"bwd128/{layout}", torch_bf16_to_bits(inp.dh), torch_bf16_to_bits(inp.gate),
                    torch_bf16_to_bits(inp.up), layout, dev)
    record_rates(f"swiglu_128x128 [{_LNAME[layout]}]", "bwd", st)


@pytest.mark.parametrize("M,N,layout", [(37, 64, ROW), (96, 96, COL), (160, 224, BOTH), (64, 1056, BOTH)])
def test_swiglu_ragged_shapes(oracle_mod, M, N, layout):
    dev = _dev()
    print(f"case: fwd/bwd ragged M={M} N={N} layout={layout}", flush=True)
    inp = synth.swiglu_inputs(M, N, seed=M + N, std=2.0)
    g, u, dh = (torch_bf16_to_bits(t) for t in (inp.gate, inp.up, inp.dh))
    _fwd_check(oracle_mod, f"fwd{M}x{N}", g, u, layout, dev)
    _bwd_check(oracle_mod, f"bwd{M}x{N}", dh, g, u, layout, dev)


# ------------------------------------------------------ fused, 4096 x 2048 full
@pytest.fixture(scope="module")
def c2_inputs():
    inp = synth.workload("swiglu_4096x2048_outliers")
    return tuple(torch_bf16_to_bits(t) for t in (inp.gate, inp.up, inp.dh))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_swiglu_fwd_4096x2048_outliers(oracle_mod, c2_inputs, layout):
    dev = _dev()
    print(f"case: fwd 4096x2048 outliers layout={layout}", flush=True)
    g, u, _ = c2_inputs
    st = _fwd_check(oracle_mod, f"fwdC2/{layout}", g, u, layout, dev)
    record_rates(f"swiglu_4096x2048_outliers [{_LNAME[layout]}]", "fwd", st)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_swiglu_bwd_4096x2048_outliers(oracle_mod, c2_inputs, layout):
    dev = _dev()
    print(f"case: bwd 4096x2048 outliers layout={layout}", flush=True)
    g, u, dh = c2_inputs
    st = _bwd_check(oracle_mod, f"bwdC2/{layout}", dh, g, u, layout, dev)
    record_rates(f"swiglu_4096x2048_outliers [{_LNAME[layout]}]", "bwd", st)


def test_cross_mode_bitwise(c2_inputs):
    """Both-mode output equals the rowwise-only and colwise-only outputs."""
    dev = _dev()
    g, u, dh = (_to_dev(a, dev) for a in c2_inputs)
    for name, fn, args in (("quant", mx.mxfp8_quant_2d, (g,)), ("fwd", mx.mxfp8_swiglu_fwd, (g, u)),
                           ("bwd", mx.mxfp8_swiglu_bwd, (dh, g, u))):
        both = fn(*args, rowwise=True, colwise=True)
        row = fn(*args, rowwise=True, colwise=False)
        col = fn(*args, rowwise=False, colwise=True)
        assert torch.equal(both[0], row[0]) and torch.equal(both[2], row[2]), name
        assert torch.equal(both[1], col[1]) and torch.equal(both[3], col[3]), name


# -------------------------------------------------------------- edge values
def test_far_negative_gates(oracle_mod):
    """Whole blocks of gates in [-98, -80]: silu is a tiny (often subnormal)
    negative number, not -0."""
    dev = _dev()
    rng = np.random.default_rng(3)
    M, N = 64, 128
    g = torch.from_numpy(rng.uniform(-98, -80, (M, N))).to(torch.bfloat16)
    u = torch.from_numpy(rng.standard_normal((M, N))).to(torch.bfloat16)
    dh = torch.from_numpy(rng.standard_normal((M, N))).to(torch.bfloat16)
    g, u, dh = (torch_bf16_to_bits(t) for t in (g, u, dh))
    for layout in LAYOUTS:
        _fwd_check(oracle_mod, f"far_fwd/{layout}", g, u, layout, dev)
        _bwd_check(oracle_mod, f"far_bwd/{layout}", dh, g, u, layout, dev)


def test_special_values(oracle_mod):
    """NaN/Inf in any input, all-zero blocks, bf16 subnormals, huge gates."""
    dev = _dev()
    rng = np.random.default_rng(4)
    M, N = 96, 160
    g, u, dh = (torch_bf16_to_bits(torch.from_numpy(rng.standard_normal((M, N)) * 3).to(torch.bfloat16))
                for _ in range(3))
    g[0, 3] = 0x7FC0
    u[5, 40] = 0x7F80
    dh[9, 100] = 0xFF80
    g[40, 70] = 0xFF80          # -Inf gate
    g[41, 71] = 0x7F80          # +Inf gate
    g[64:96, 0:32] = 0          # all-zero blocks in both layouts
    u[64:96, 32:64] = rng.integers(1, 0x7F, (32, 32))  # subnormal up
    g[10:12, 128:160] = rng.integers(1, 0x7F, (2, 32)).astype(np.uint16) | 0x8000  # subnormal gates
    g[20, 130:140] = 0x4400     # 512
    g[21, 130:140] = 0xC400     # -512
    for layout in LAYOUTS:
        _fwd_check(oracle_mod, f"special_fwd/{layout}", g, u, layout, dev)
        _bwd_check(oracle_mod, f"special_bwd/{layout}", dh, g, u, layout, dev)


def test_exhaustive_gate_values(oracle_mod):
    """Every finite bf16 gate once (u = 1, dh = 1): the fp32 activation's
    distance from the exact one, over the whole gate range."""
    dev = _dev()
    bits = all_bf16_bits()
    fin = bits[(bits & 0x7FFF) < 0x7F80]
    fin = np.resize(fin, (fin.size // (32 * 64) + 1) * 32 * 64).reshape(-1, 64)
    one = np.full_like(fin, 0x3F80)
    st = _fwd_check(oracle_mod, "all_gates_fwd", fin, one, BOTH, dev)
    st2 = _bwd_check(oracle_mod, "all_gates_bwd", one, fin, one, BOTH, dev)
    record_rates("every finite bf16 gate, up = dh = 1 [both-layout launch]", "fwd", st)
    record_rates("every finite bf16 gate, up = dh = 1 [both-layout launch]", "bwd", st2)


def wide_bf16(shape, seed, emin, emax):
    """Random bf16 patterns with uniform sign and mantissa and an unbiased
    exponent uniform in [emin, emax]."""
    rng = np.random.default_rng(seed)
    e = rng.integers(emin + 127, emax + 128, shape, dtype=np.int64)
    m = rng.integers(0, 128, shape, dtype=np.int64)
    sgn = rng.integers(0, 2, shape, dtype=np.int64)
    return ((sgn << 15) | (e << 7) | m).astype(np.uint16)


def test_exhaustive_gates_wide_upstream(oracle_mod):
    """Every finite bf16 gate with up (2^-20 .. 2^20) and dh (2^-40 .. 2^24)
    drawn over wide exponent ranges, so that da = dh * up spans 2^-60 ..
    2^45: the far-negative backward must not overflow an intermediate where
    the exact dgate is finite (it once formed da (1 + g) first, which is inf
    for g near -2^127 once |da| > 2, and inf times the vanished exponential
    gave NaN).  The far forms hold their exponential at 2^64 times its value,
    which keeps every representable result exact to its last rounding for
    |da| < 2^49."""
    dev = _dev()
    bits = all_bf16_bits()
    fin = bits[(bits & 0x7FFF) < 0x7F80]
    fin = np.resize(fin, (fin.size // (32 * 64) + 1) * 32 * 64).reshape(-1, 64)
    u = wide_bf16(fin.shape, 11, -20, 20)
    dh = wide_bf16(fin.shape, 12, -40, 24)
    _fwd_check(oracle_mod, "all_gates_wide_fwd", fin, u, BOTH, dev)
    _bwd_check(oracle_mod, "all_gates_wide_bwd", dh, fin, u, BOTH, dev)


# ------------------------------------------------ full-size, sampled slabs
def _slabs(M, n, seed):
    rng = np.random.default_rng(seed)
    picks = {0, M // 32 - 1} | set(rng.integers(0, M // 32, n).tolist())
    return sorted(picks)


def _oracle_slabs(oracle_mod, inp, slabs, bwd):
    """Oracle outputs (both layouts) and values of each sampled 32-row slab,
    computed on the host cores (the oracle is single-threaded C, called from
    a thread pool; each call covers one slab)."""
    args = (inp.dh, inp.gate, inp.up) if bwd else (inp.gate, inp.up)
    host = {sb: [torch_bf16_to_bits(a[sb * 32:sb * 32 + 32]) for a in args] for sb in slabs}

    def one(sb):
        h = host[sb]
        if bwd:
            dg, du = oracle_mod.swiglu_bwd_values(*h)
            return sb, oracle_mod.swiglu_bwd(*h, BOTH), np.concatenate([dg, du], axis=1)
        return sb, oracle_mod.swiglu_fwd(*h, BOTH), oracle_mod.swiglu_fwd_values(*h)

    with ThreadPoolExecutor(max_workers=16) as pool:
        return {sb: (orc, vals) for sb, orc, vals in pool.map(one, slabs)}


def _compare_slabs(oracle_mod, name, outs, layout, ref):
    """Sampled slabs of one launch's outputs against the oracle; returns the
    merged Stats (per layout in .notes)."""
    q_row, q_col, s_row, s_col = outs
    total = None
    for sb, (orc, vals) in ref.items():
        r0, r1 = sb * 32, sb * 32 + 32
        gpu = (_np(q_row[r0:r1]) if layout & ROW else None, _np(s_row[r0:r1]) if layout & ROW else None,
               _np(q_col[:, r0:r1]) if layout & COL else None, _np(s_col[:, sb:sb + 1]) if layout & COL else None)
        st = compare_fused(oracle_mod, f"{name}/slab{sb}", gpu, orc, vals, layout)
        total = st if total is None else total.merge(st)
    return total


def _sampled_all_launches(oracle_mod, workload, inp, direction, n_slabs, seed):
    """Row-only, col-only and both-layout launches at full size: the
    both-layout outputs equal the single-layout ones bit for bit over the
    whole result, and each launch's outputs match the oracle on the sampled
    slabs; the rates are recorded per launch and layout and held to the bar
    (scale mismatches at most 1e-4 of blocks) over all slabs together."""
    bwd = direction == "bwd"
    M = inp.gate.shape[0]
    fn = mx.mxfp8_swiglu_bwd if bwd else mx.mxfp8_swiglu_fwd
    args = (inp.dh, inp.gate, inp.up) if bwd else (inp.gate, inp.up)
    slabs = _slabs(M, n_slabs, seed)
    ref = _oracle_slabs(oracle_mod, inp, slabs, bwd)
    both = fn(*args, rowwise=True, colwise=True)
    for lay in (ROW, COL):
        one = fn(*args, **_flags(lay))
        torch.cuda.synchronize()
        i, j = (0, 2) if lay == ROW else (1, 3)
        assert torch.equal(one[i], both[i]) and torch.equal(one[j], both[j]), f"{workload} {direction}: {lay}"
        st = _compare_slabs(oracle_mod, f"{workload}/{direction}/{lay}", one, lay, ref)
        record_rates(f"{workload} [{_LNAME[lay]}]", direction, st)
        assert st.scale_mismatch_rate <= 1e-4, (workload, direction, lay, st.record())
        del one
    st = _compare_slabs(oracle_mod, f"{workload}/{direction}/both", both, BOTH, ref)
    record_rates(f"{workload} [{_LNAME[BOTH]}]", direction, st)
    assert st.scale_mismatch_rate <= 1e-4, (workload, direction, "both", st.record())
    del both
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def c3_inputs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    inp = synth.workload("swiglu_16384x7168_w13", device=torch.device("cuda", 0))
    yield inp
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_swiglu_16384x7168_w13_sampled(oracle_mod, c3_inputs, direction):
    _dev()
    print(f"case: 16384x7168 w13 {direction}, all launches, 64 sampled slabs", flush=True)
    _sampled_all_launches(oracle_mod, "swiglu_16384x7168_w13", c3_inputs, direction, 64, 11)


@pytest.fixture(scope="module")
def c5_inputs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    inp = synth.workload("swiglu_131072x8192_w13", device=torch.device("cuda", 0))
    yield inp
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_swiglu_131072x8192_w13_sampled(oracle_mod, c5_inputs, direction):
    _dev()
    print(f"case: 131072x8192 w13 {direction}, all launches, 64 sampled slabs", flush=True)
    _sampled_all_launches(oracle_mod, "swiglu_131072x8192_w13", c5_inputs, direction, 64, 12)


# ------------------------------- large ragged both-layout launches, scale strides
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("N", [7200, 7680])
def test_both_layout_large_ragged_and_scale_strides(oracle_mod, N, direction):
    """Both-layout launches at 131072 rows with a partial last column tile
    (N = 7200: 56 whole tiles and one of 32 columns, scale rows of 225 or
    450 bytes) and with whole tiles (N = 7680).  The both-layout result
    equals the rowwise and colwise launches bit for bit over the whole
    output (the rowwise launch is a different kernel), and matches the
    oracle on sampled slabs.  Rowwise scales written through a padded
    stride and through an unaligned one equal the packed ones, and the
    padding bytes are untouched."""
    dev = _dev()
    M = 131072
    print(f"case: both-layout {M}x{N} {direction}", flush=True)
    inp = synth.swiglu_inputs(M, N, seed=31 + N, std=1.0, device=dev)
    bwd = direction == "bwd"
    fn = mx.mxfp8_swiglu_bwd if bwd else mx.mxfp8_swiglu_fwd
    args = (inp.dh, inp.gate, inp.up) if bwd else (inp.gate, inp.up)
    W = 2 * N if bwd else N
    both = fn(*args, rowwise=True, colwise=True)
    for lay in (ROW, COL):
        one = fn(*args, **_flags(lay))
        torch.cuda.synchronize()
        i, j = (0, 2) if lay == ROW else (1, 3)
        assert torch.equal(one[i], both[i]) and torch.equal(one[j], both[j]), (N, direction, lay)
        del one
    ref = _oracle_slabs(oracle_mod, inp, _slabs(M, 8, N), bwd)
    st = _compare_slabs(oracle_mod, f"ragged_{N}/{direction}", both, BOTH, ref)
    assert st.scale_mismatch_rate <= 1e-4, st.record()
    for extra in (16, 5):  # aligned padding, unaligned stride
        ld = W // 32 + extra
        buf = torch.full((M, ld), 0xA5, dtype=torch.uint8, device=dev)
        q_row, q_col = torch.empty_like(both[0]), torch.empty_like(both[1])
        s_col = torch.empty_like(both[3])
        fn(*args, rowwise=True, colwise=True, out=(q_row, q_col, buf[:, :W // 32], s_col))
        torch.cuda.synchronize()
        assert torch.equal(buf[:, :W // 32], both[2]), (N, direction, extra)
        assert (buf[:, W // 32:] == 0xA5).all(), (N, direction, extra)
        assert torch.equal(q_row, both[0]) and torch.equal(q_col, both[1]) and torch.equal(s_col, both[3])
        del buf, q_row, q_col, s_col
    del both, inp
    torch.cuda.empty_cache()


# ------------------------------------------------------------------- 3D
def test_quant_3d_small_shapes(oracle_mod):
    dev = _dev()
    for E, N, K in ((1, 32, 8), (3, 96, 40), (2, 160, 200), (5, 64, 64)):
        print(f"case: 3d E={E} N={N} K={K}", flush=True)
        w = torch_bf16_to_bits(synth.expert_weights(E, N, K, seed=E * N + K, std=0.5))
        q, s = mx.mxfp8_quant_3d_colwise(_to_dev(w.reshape(E * N, K), dev).reshape(E, N, K))
        qo, so = oracle_mod.quant_3d_colwise(w)
        assert_exact("q3d", _np(q), qo)
        assert_exact("s3d", _np(s), so)


def test_quant_3d_strided_experts(oracle_mod):
    dev = _dev()
    big = torch_bf16_to_bits(synth.expert_weights(3, 100, 72, seed=9, std=1.0))
    w_dev = _to_dev(big.reshape(300, 72), dev).reshape(3, 100, 72)[:, 4:68, 8:56]  # stride_e 7200, ld 72
    q, s = mx.mxfp8_quant_3d_colwise(w_dev)
    qo, so = oracle_mod.quant_3d_colwise(big[:, 4:68, 8:56])
    assert_exact("q3d_strided", _np(q), qo)
    assert_exact("s3d_strided", _np(s), so)


@pytest.mark.parametrize("E", [1, 4, 16, 64])
def test_quant_3d_experts_8192x5120(oracle_mod, E):
    """Full expert stacks (every expert count of the workload): every
    expert's output equals the plain 2D colwise cast of that expert, bit for
    bit over the whole (K, N) result; and the oracle checks 64-column slices
    of the first, the last and two random experts bit for bit."""
    dev = _dev()
    print(f"case: 3d E={E} 8192x5120", flush=True)
    w = synth.expert_workload(E, device=dev)
    q, s = mx.mxfp8_quant_3d_colwise(w)
    for e in range(E):
        _, q2, _, s2 = mx.mxfp8_quant_2d(w[e], rowwise=False, colwise=True)
        assert torch.equal(q[e], q2) and torch.equal(s[e], s2), e
        del q2, s2
    rng = np.random.default_rng(E)
    experts = sorted({0, E - 1} | set(rng.integers(0, E, 2).tolist()))
    for e in experts:
        k0 = int(rng.integers(0, 5120 // 64)) * 64
        host = torch_bf16_to_bits(w[e][:, k0:k0 + 64])
        qo, so = oracle_mod.quant_3d_colwise(host.reshape(1, 8192, 64))
        assert_exact(f"q3d_e{e}", _np(q[e, k0:k0 + 64]), qo[0])
        assert_exact(f"s3d_e{e}", _np(s[e, k0:k0 + 64]), so[0])
    del w, q, s
    torch.cuda.empty_cache()


# ----------------------------------------------------- bounds and contract
def test_guard_bytes_and_padding_untouched():
    """Outputs carved out of larger 0xA5-filled buffers with padded leading
    dimensions: only the result bytes change."""
    dev = _dev()
    M, N = 96, 160
    inp = synth.swiglu_inputs(M, N, seed=21, device=dev)
    pad = 4096
    for fn, args, W in ((mx.mxfp8_swiglu_fwd, (inp.gate, inp.up), N),
                        (mx.mxfp8_swiglu_bwd, (inp.dh, inp.gate, inp.up), 2 * N)):
        ldq_r, lds_r, ldq_c, lds_c = W + 32, W // 32 + 5, M + 48, M // 32 + 3
        shapes = ((M, ldq_r), (M, lds_r), (W, ldq_c), (W, lds_c))
        bufs = [torch.full((pad * 2 + r * c,), 0xA5, dtype=torch.uint8, device=dev) for r, c in shapes]
        views = [b[pad:pad + r * c].view(r, c) for b, (r, c) in zip(bufs, shapes)]
        outs = (views[0][:, :W], views[2][:, :M], views[1][:, :W // 32], views[3][:, :M // 32])
        ref = fn(*args, rowwise=True, colwise=True)
        fn(*args, rowwise=True, colwise=True, out=outs)
        for o, r in zip(outs, ref):
            assert torch.equal(o, r)
        for b, v, (r, c), used in zip(bufs, views, shapes, (W, W // 32, M, M // 32)):
            assert (b[:pad] == 0xA5).all() and (b[pad + r * c:] == 0xA5).all()
            assert (v[:, used:] == 0xA5).all()


def test_misaligned_and_bad_shapes_raise():
    dev = _dev()
    x = torch.zeros((64, 72), dtype=torch.bfloat16, device=dev)
    with pytest.raises(mx.Mxfp8Error) as ei:
        mx.mxfp8_quant_2d(x[:, 1:65], rowwise=True)  # pointer 2 bytes past a 16-byte boundary
    assert ei.value.status == 4
    with pytest.raises(mx.Mxfp8Error) as ei:
        mx.mxfp8_swiglu_fwd(x[:, :48], x[:, :48])  # width not a multiple of 32
    assert ei.value.status == 2
    with pytest.raises(mx.Mxfp8Error) as ei:
        mx.mxfp8_quant_2d(x[:40, :64], colwise=True, rowwise=False)  # rows not a multiple of 32
    assert ei.value.status == 2


def test_empty_inputs_are_noops():
    dev = _dev()
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    outs = mx.mxfp8_swiglu_fwd(x, x, rowwise=True, colwise=True)
    assert outs[0].shape == (0, 64) and outs[1].shape == (64, 0)
    q, s = mx.mxfp8_quant_3d_colwise(torch.zeros((0, 32, 8), dtype=torch.bfloat16, device=dev))
    assert q.numel() == 0 and s.numel() == 0


# -------------------------------------------------- unfused pipeline (bf16)
@pytest.mark.parametrize("M,N", [(128, 128), (96, 1056), (4096, 2048)])
def test_bf16_values_match_oracle_and_feed_the_plain_cast(oracle_mod, M, N):
    """The activation-only kernels agree with the oracle's values on nearly
    all elements, and the plain 2D cast of their output equals the fused
    cast bit for bit (same value code on the GPU).

    Bound: the fp32 silu may round to the bf16 neighbour of the exact s; a
    one-step change of s is 2^-8..2^-7 relative, which is up to two steps of
    h = bf16(s * u) (and of du = bf16(dh * s)) when s's mantissa is near 1
    and the product's near 2.  dg rounds one fp32 expression of exact bf16
    operands: at most one step.  (Two bf16 steps stay below one E4M3 step,
    which is what the fused casts are held to.)"""
    dev = _dev()
    print(f"case: bf16 values M={M} N={N}", flush=True)
    inp = synth.swiglu_inputs(M, N, seed=M + 3 * N, std=2.0, outlier_rate=1e-3, device=dev)
    h = mx.mxfp8_swiglu_fwd_bf16(inp.gate, inp.up)
    y = mx.mxfp8_swiglu_bwd_bf16(inp.dh, inp.gate, inp.up)
    g, u, dh = (torch_bf16_to_bits(t) for t in (inp.gate, inp.up, inp.dh))
    h_o = oracle_mod.swiglu_fwd_values(g, u)
    dg_o, du_o = oracle_mod.swiglu_bwd_values(dh, g, u)
    y_o = np.concatenate([dg_o, du_o], axis=1)
    yb = torch_bf16_to_bits(y)
    for name, got, want, bound in (("h", torch_bf16_to_bits(h), h_o, 2), ("dg", yb[:, :N], y_o[:, :N], 1),
                                   ("du", yb[:, N:], y_o[:, N:], 2)):
        steps = np.abs(got.astype(np.int32) - want.astype(np.int32))
        zero = ((got & 0x7FFF) == 0) & ((want & 0x7FFF) == 0)
        steps[zero] = 0  # +0 and -0
        assert steps.max() <= bound, (name, int(steps.max()))
        assert (steps > 0).mean() < 2e-3, name
    for fused, vals in ((mx.mxfp8_swiglu_fwd(inp.gate, inp.up, rowwise=True, colwise=True), h),
                        (mx.mxfp8_swiglu_bwd(inp.dh, inp.gate, inp.up, rowwise=True, colwise=True), y)):
        plain = mx.mxfp8_quant_2d(vals, rowwise=True, colwise=True)
        for a, b in zip(fused, plain):
            assert torch.equal(a, b)


def test_bf16_values_every_gate(oracle_mod):
    """The activation-only kernels over every finite bf16 gate (up = dh = 1,
    so h = du = bf16(silu(g)) and dg = bf16(silu'(g))): h and du equal the
    exact definition for every gate (the refined reciprocal keeps g = 5.9375,
    whose exact silu lies about an fp32 ulp below a bf16 rounding midpoint,
    on the right side); dg within one step, on at most two gates."""
    dev = _dev()
    bits = all_bf16_bits()
    g = np.ascontiguousarray(bits[(bits & 0x7FFF) < 0x7F80].reshape(-1, 32))
    one = np.full_like(g, 0x3F80)
    gd, od = _to_dev(g, dev), _to_dev(one, dev)
    h = torch_bf16_to_bits(mx.mxfp8_swiglu_fwd_bf16(gd, od))
    y = torch_bf16_to_bits(mx.mxfp8_swiglu_bwd_bf16(od, gd, od))
    dg_o, du_o = oracle_mod.swiglu_bwd_values(one, g, one)
    h_o = oracle_mod.swiglu_fwd_values(g, one)

    def steps(a, b):
        d = np.abs(a.astype(np.int32) - b.astype(np.int32))
        d[((a & 0x7FFF) == 0) & ((b & 0x7FFF) == 0)] = 0  # +0 and -0
        return d

    assert steps(h, h_o).max() == 0, int((steps(h, h_o) > 0).sum())
    assert steps(y[:, 32:], du_o).max() == 0
    d = steps(y[:, :32], dg_o)
    assert d.max() <= 1 and (d > 0).sum() <= 2, int((d > 0).sum())


def test_bf16_values_strided_output():
    dev = _dev()
    inp = synth.swiglu_inputs(64, 256, seed=77, device=dev, packed=True)
    big = torch.full((64, 600), 7.0, dtype=torch.bfloat16, device=dev)
    out = big[:, 8:520]
    y = mx.mxfp8_swiglu_bwd_bf16(inp.dh, inp.gate, inp.up, out=out)
    ref = mx.mxfp8_swiglu_bwd_bf16(inp.dh, inp.gate, inp.up)
    assert torch.equal(y, ref)
    assert (big[:, :8] == 7.0).all() and (big[:, 520:] == 7.0).all()

