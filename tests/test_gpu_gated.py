"""GPU parity of the other gated activations (GELU exact, GELU tanh, ReLU;
SiLU as the control) through mxfp8_gated_fwd / mxfp8_gated_bwd.

"Add swiglu + MXFP8 fused CuTe DSL kernel", API (the activation is a
compile-time policy of one kernel source) and Follow-ups (more gated
activations).  Same bar as the SwiGLU casts (oracle/parity.py): codes within
one E4M3 step, scales bit-exact except next to a power-of-two boundary,
invalid blocks exact.  The oracle evaluates each activation in double.
"""
import numpy as np
import pytest
import torch

import swiglu_activation_cast_amd as mx
from swiglu_activation_cast_amd import synth
from concurrent.futures import ThreadPoolExecutor

from helpers import all_bf16_bits, bits_to_torch_bf16, record_rates, torch_bf16_to_bits
from oracle.parity import compare_fused

pytestmark = pytest.mark.gpu

ROW, COL, BOTH = 1, 2, 3
LAYOUTS = (ROW, COL, BOTH)
ACTS = ("silu", "gelu_tanh", "gelu", "relu")
OTHER = ("gelu_tanh", "gelu", "relu")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _np(t):
    return t.cpu().numpy()


def _gpu(outs):
    q_row, q_col, s_row, s_col = outs
    return _np(q_row), _np(s_row), _np(q_col), _np(s_col)


def _flags(layout):
    return dict(rowwise=bool(layout & ROW), colwise=bool(layout & COL))


def _to_dev(bits, dev):
    return bits_to_torch_bf16(bits).to(dev)


def fwd_check(oracle_mod, name, act, g_bits, u_bits, layout, dev):
    oa = oracle_mod.ACTS[act]
    g, u = _to_dev(g_bits, dev), _to_dev(u_bits, dev)
    gpu = _gpu(mx.mxfp8_gated_fwd(g, u, act=act, **_flags(layout)))
    orc = oracle_mod.gated_fwd(g_bits, u_bits, layout, oa)
    vals = oracle_mod.gated_fwd_values(np.ascontiguousarray(g_bits), np.ascontiguousarray(u_bits), oa)
    return compare_fused(oracle_mod, f"{act}/{name}", gpu, orc, vals, layout)


def bwd_check(oracle_mod, name, act, dh_bits, g_bits, u_bits, layout, dev):
    oa = oracle_mod.ACTS[act]
    dh, g, u = _to_dev(dh_bits, dev), _to_dev(g_bits, dev), _to_dev(u_bits, dev)
    gpu = _gpu(mx.mxfp8_gated_bwd(dh, g, u, act=act, **_flags(layout)))
    orc = oracle_mod.gated_bwd(dh_bits, g_bits, u_bits, layout, oa)
    dg, du = oracle_mod.gated_bwd_values(*(np.ascontiguousarray(a) for a in (dh_bits, g_bits, u_bits)), oa)
    return compare_fused(oracle_mod, f"{act}/{name}", gpu, orc, np.concatenate([dg, du], axis=1), layout)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_gated_128x128(oracle_mod, act, layout):
    dev = _dev()
    print(f"case: gated {act} 128x128 std 2 layout={layout}", flush=True)
    inp = synth.swiglu_inputs(128, 128, seed=40, std=2.0)
    g, u, dh = (torch_bf16_to_bits(t) for t in (inp.gate, inp.up, inp.dh))
    fwd_check(oracle_mod, f"fwd128/{layout}", act, g, u, layout, dev)
    bwd_check(oracle_mod, f"bwd128/{layout}", act, dh, g, u, layout, dev)


@pytest.mark.parametrize("act", OTHER)
@pytest.mark.parametrize("M,N,layout", [(37, 64, ROW), (96, 96, COL), (64, 1056, BOTH)])
def test_gated_ragged_shapes(oracle_mod, act, M, N, layout):
    dev = _dev()
    print(f"case: gated {act} ragged M={M} N={N} layout={layout}", flush=True)
    inp = synth.swiglu_inputs(M, N, seed=M + 2 * N, std=3.0)
    g, u, dh = (torch_bf16_to_bits(t) for t in (inp.gate, inp.up, inp.dh))
    fwd_check(oracle_mod, f"fwd{M}x{N}", act, g, u, layout, dev)
    bwd_check(oracle_mod, f"bwd{M}x{N}", act, dh, g, u, layout, dev)


@pytest.fixture(scope="module")
def c2_inputs():
    inp = synth.workload("swiglu_4096x2048_outliers")
    return tuple(torch_bf16_to_bits(t) for t in (inp.gate, inp.up, inp.dh))


@pytest.mark.parametrize("act", OTHER)
def test_gated_4096x2048_outliers(oracle_mod, c2_inputs, act):
    dev = _dev()
    print(f"case: gated {act} 4096x2048 outliers, both layouts", flush=True)
    g, u, dh = c2_inputs
    st = fwd_check(oracle_mod, "fwdC2", act, g, u, BOTH, dev)
    st2 = bwd_check(oracle_mod, "bwdC2", act, dh, g, u, BOTH, dev)
    record_rates(f"{act}: swiglu_4096x2048_outliers inputs [both-layout launch]", "fwd", st)
    record_rates(f"{act}: swiglu_4096x2048_outliers inputs [both-layout launch]", "bwd", st2)


def test_gated_silu_is_swiglu(c2_inputs):
    """act = silu runs the very kernels of mxfp8_swiglu_*: identical bytes."""
    dev = _dev()
    g, u, dh = (_to_dev(a, dev) for a in c2_inputs)
    for layout in LAYOUTS:
        a = mx.mxfp8_gated_fwd(g, u, act="silu", **_flags(layout))
        b = mx.mxfp8_swiglu_fwd(g, u, **_flags(layout))
        assert all(torch.equal(x, y) for x, y in zip(a, b))
        a = mx.mxfp8_gated_bwd(dh, g, u, act="silu", **_flags(layout))
        b = mx.mxfp8_swiglu_bwd(dh, g, u, **_flags(layout))
        assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("act", OTHER)
def test_gated_cross_mode_bitwise(c2_inputs, act):
    dev = _dev()
    g, u, dh = (_to_dev(a, dev) for a in c2_inputs)
    for fn, args in ((mx.mxfp8_gated_fwd, (g, u)), (mx.mxfp8_gated_bwd, (dh, g, u))):
        both = fn(*args, act=act, rowwise=True, colwise=True)
        row = fn(*args, act=act, rowwise=True, colwise=False)
        col = fn(*args, act=act, rowwise=False, colwise=True)
        assert torch.equal(both[0], row[0]) and torch.equal(both[2], row[2])
        assert torch.equal(both[1], col[1]) and torch.equal(both[3], col[3])


@pytest.mark.parametrize("act", OTHER)
def test_gated_exhaustive_gate_values(oracle_mod, act):
    """Every finite bf16 gate once (u = 1, dh = 1): blocks hold 32
    consecutive patterns, so whole blocks sit in each activation's far
    tails and tiny-scale regimes."""
    dev = _dev()
    print(f"case: gated {act} every finite gate", flush=True)
    bits = all_bf16_bits()
    fin = bits[(bits & 0x7FFF) < 0x7F80]
    fin = np.resize(fin, (fin.size // (32 * 64) + 1) * 32 * 64).reshape(-1, 64)
    one = np.full_like(fin, 0x3F80)
    st = fwd_check(oracle_mod, "all_gates_fwd", act, fin, one, BOTH, dev)
    st2 = bwd_check(oracle_mod, "all_gates_bwd", act, one, fin, one, BOTH, dev)
    record_rates(f"{act}: every finite bf16 gate, up = dh = 1 [both-layout launch]", "fwd", st)
    record_rates(f"{act}: every finite bf16 gate, up = dh = 1 [both-layout launch]", "bwd", st2)


@pytest.mark.parametrize("act", OTHER)
def test_gated_exhaustive_gates_wide_upstream(oracle_mod, act):
    """Every finite bf16 gate with up (2^-20 .. 2^20) and dh (2^-40 .. 2^24)
    over wide exponent ranges (|da| up to 2^45): no far-negative form may
    overflow an intermediate for a large da where the exact dgate is
    finite."""
    from test_gpu_parity import wide_bf16
    dev = _dev()
    print(f"case: gated {act} every finite gate, wide upstream", flush=True)
    bits = all_bf16_bits()
    fin = bits[(bits & 0x7FFF) < 0x7F80]
    fin = np.resize(fin, (fin.size // (32 * 64) + 1) * 32 * 64).reshape(-1, 64)
    u = wide_bf16(fin.shape, 13, -20, 20)
    dh = wide_bf16(fin.shape, 14, -40, 24)
    fwd_check(oracle_mod, "all_gates_wide_fwd", act, fin, u, BOTH, dev)
    bwd_check(oracle_mod, "all_gates_wide_bwd", act, dh, fin, u, BOTH, dev)


# gate ranges where each activation's plain fp32 form would flush a
# representable result and the careful (2^64-scaled) form takes over
FAR = {"gelu_tanh": (-10.75, -9.25), "gelu": (-14.0, -7.5), "relu": (-5.0, -0.5)}


@pytest.mark.parametrize("act", OTHER)
def test_gated_far_negative_gates(oracle_mod, act):
    dev = _dev()
    print(f"case: gated {act} far-negative gates {FAR[act]}", flush=True)
    rng = np.random.default_rng(30)
    M, N = 64, 128
    lo, hi = FAR[act]
    g = torch_bf16_to_bits(torch.from_numpy(rng.uniform(lo, hi, (M, N))).to(torch.bfloat16))
    u = torch_bf16_to_bits(torch.from_numpy(rng.standard_normal((M, N))).to(torch.bfloat16))
    dh = torch_bf16_to_bits(torch.from_numpy(rng.standard_normal((M, N))).to(torch.bfloat16))
    for layout in LAYOUTS:
        fwd_check(oracle_mod, f"far_fwd/{layout}", act, g, u, layout, dev)
        bwd_check(oracle_mod, f"far_bwd/{layout}", act, dh, g, u, layout, dev)


@pytest.mark.parametrize("act", OTHER)
def test_gated_special_values(oracle_mod, act):
    """NaN/Inf in any input, +-Inf gates, all-zero blocks, subnormals,
    huge finite gates (whose squares overflow fp32)."""
    dev = _dev()
    print(f"case: gated {act} special values", flush=True)
    rng = np.random.default_rng(31)
    M, N = 96, 160
    g, u, dh = (torch_bf16_to_bits(torch.from_numpy(rng.standard_normal((M, N)) * 3).to(torch.bfloat16))
                for _ in range(3))
    g[0, 3] = 0x7FC0
    g[1, 4] = 0xFFC0            # negative NaN gate
    u[5, 40] = 0x7F80
    dh[9, 100] = 0xFF80
    g[40, 70] = 0xFF80          # -Inf gate
    g[41, 71] = 0x7F80          # +Inf gate
    g[64:96, 0:32] = 0          # all-zero blocks in both layouts
    g[64:96, 32:64] = 0x8000    # -0 gates
    u[64:96, 32:64] = rng.integers(1, 0x7F, (32, 32))  # subnormal up
    g[10:12, 128:160] = rng.integers(1, 0x7F, (2, 32)).astype(np.uint16) | 0x8000  # subnormal gates
    g[20, 130:140] = 0x4400     # 512
    g[21, 130:140] = 0xC400     # -512
    g[22, 130:140] = 0x7F00     # 1.7e38: g^2 overflows fp32
    g[23, 130:140] = 0xFF00     # -1.7e38
    g[24, 130:140] = 0x5F80     # 2^64
    g[25, 130:140] = 0xDF80     # -2^64
    for layout in LAYOUTS:
        fwd_check(oracle_mod, f"special_fwd/{layout}", act, g, u, layout, dev)
        bwd_check(oracle_mod, f"special_bwd/{layout}", act, dh, g, u, layout, dev)


def _sampled_both(oracle_mod, workload, act, n_slabs, seed):
    """One both-layout launch per direction on a full-size workload, random
    32-row slabs of it against the oracle (computed on the host cores); the
    rates are recorded and held to the bar over all slabs together."""
    dev = _dev()
    inp = synth.workload(workload, device=dev)
    oa = oracle_mod.ACTS[act]
    M = inp.gate.shape[0]
    rng = np.random.default_rng(seed)
    slabs = sorted({0, M // 32 - 1} | set(rng.integers(0, M // 32, n_slabs).tolist()))
    for bwd in (False, True):
        args = (inp.dh, inp.gate, inp.up) if bwd else (inp.gate, inp.up)
        fn = mx.mxfp8_gated_bwd if bwd else mx.mxfp8_gated_fwd
        q_row, q_col, s_row, s_col = fn(*args, act=act, rowwise=True, colwise=True)
        torch.cuda.synchronize()
        host = {sb: [torch_bf16_to_bits(a[sb * 32:sb * 32 + 32]) for a in args] for sb in slabs}

        def ref(sb):
            h = host[sb]
            if bwd:
                dg, du = oracle_mod.gated_bwd_values(*h, oa)
                return sb, oracle_mod.gated_bwd(*h, BOTH, oa), np.concatenate([dg, du], axis=1)
            return sb, oracle_mod.gated_fwd(*h, BOTH, oa), oracle_mod.gated_fwd_values(*h, oa)

        with ThreadPoolExecutor(max_workers=16) as pool:
            refs = list(pool.map(ref, slabs))
        total = None
        for sb, orc, vals in refs:
            r0, r1 = sb * 32, sb * 32 + 32
            gpu = (_np(q_row[r0:r1]), _np(s_row[r0:r1]), _np(q_col[:, r0:r1]), _np(s_col[:, sb:sb + 1]))
            st = compare_fused(oracle_mod, f"{act}/{'bwd' if bwd else 'fwd'}/{workload}/slab{sb}", gpu, orc, vals,
                               BOTH)
            total = st if total is None else total.merge(st)
        record_rates(f"{act}: {workload} [both-layout launch]", "bwd" if bwd else "fwd", total)
        assert total.scale_mismatch_rate <= 1e-4, (act, bwd, total.record())
        del q_row, q_col, s_row, s_col
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("act", OTHER)
def test_gated_16384x7168_w13_sampled(oracle_mod, act):
    """The 16384 x 7168 packed-w13 workload, both layouts in one launch,
    64 sampled 32-row slabs against the oracle."""
    print(f"case: gated {act} 16384x7168 w13, sampled slabs", flush=True)
    _sampled_both(oracle_mod, "swiglu_16384x7168_w13", act, 64, 32)


@pytest.mark.parametrize("act", OTHER)
def test_gated_131072x8192_w13_sampled(oracle_mod, act):
    """The 131072 x 8192 packed-w13 workload the benchmark times, both
    layouts in one launch, 64 sampled 32-row slabs against the oracle."""
    print(f"case: gated {act} 131072x8192 w13, sampled slabs", flush=True)
    _sampled_both(oracle_mod, "swiglu_131072x8192_w13", act, 64, 33)


def test_gated_pages_api_names(c2_inputs):
    """gated_act_mxfp8_forward/backward on the packed [M, 2N] input take the
    activation by name and equal the split-pointer calls."""
    dev = _dev()
    g, u, dh = (_to_dev(a, dev) for a in c2_inputs)
    w13 = torch.cat([g, u], dim=1)
    for act in ACTS:
        a = mx.gated_act_mxfp8_forward(w13, rowwise=True, colwise=True, activation=act)
        b = mx.mxfp8_gated_fwd(g, u, act=act, rowwise=True, colwise=True)
        assert all(torch.equal(x, y) for x, y in zip(a, b)), act
        a = mx.gated_act_mxfp8_backward(dh, w13, rowwise=True, colwise=False, activation=act)
        b = mx.mxfp8_gated_bwd(dh, g, u, act=act, rowwise=True, colwise=False)
        assert all(torch.equal(x, y) for x, y in zip(a, b)), act
