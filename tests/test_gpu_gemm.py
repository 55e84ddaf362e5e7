"""GPU parity of the MX GEMM consumer (mxfp8_gemm) against the oracle.

C = A B^T of MXFP8 operands stored K-contiguous, as the casts emit them
("[mxfp8 moe training] add compile support", Perf analysis: the cast
outputs feed a scaled grouped GEMM).

The bar is the error bound of the matrix core's arithmetic.  Every single
product is exact (checked for all 65536 code pairs), but inside one 64-term
block-scaled MFMA the products are aligned to the largest one and each is
truncated toward zero 13 bits below its leading bit (measured: a product
smaller than 2^-13 of the largest is dropped); the 64-term sum then enters
the fp32 accumulator.  So, per 64-element K step s with largest product
magnitude pmax_s:
    |C_gpu - C| <= sum_s 64 * 2^-13 * pmax_s + (K / 64) * 2^-24 * sum_k |a_k b_k|,
with C the oracle's exact-product double sum, and NaN exactly where the
oracle has NaN.
"""
import numpy as np
import pytest
import torch

import swiglu_activation_cast_amd as mx
from swiglu_activation_cast_amd import synth

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _rand_operands(rng, rows, K, lo=118, hi=137):
    codes = rng.integers(0, 256, (rows, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A  # no NaN codes
    return codes, rng.integers(lo, hi, (rows, K // 32)).astype(np.uint8)


def _values(q, s):
    """Element values, decoded independently of the oracle (torch's E4M3 cast)."""
    v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):
        return v * np.ldexp(1.0, np.repeat(s.astype(np.int64), 32, axis=1) - 127)


def _step_max_sum(a, sa, b, sb):
    """sum over 64-element K steps of the largest |product| in the step."""
    va, vb = _values(a, sa), _values(b, sb)
    out = np.zeros((a.shape[0], b.shape[0]))
    for k0 in range(0, a.shape[1], 64):
        with np.errstate(invalid="ignore"):
            p = np.abs(va[:, None, k0:k0 + 64] * vb[None, :, k0:k0 + 64])
        out += np.nan_to_num(p.max(-1), nan=0.0)
    return out


def _check(oracle_mod, name, a, sa, b, sb, got):
    want, mag = oracle_mod.mx_gemm(a, sa, b, sb)
    got = np.asarray(got, np.float64)
    K = a.shape[1]
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), f"{name}: NaN pattern differs"
    bound = 64 * 2.0 ** -13 * _step_max_sum(a, sa, b, sb) + (K / 64 + 1) * 2.0 ** -24 * mag
    err = np.abs(got[~nan] - want[~nan])
    worst = (err / np.maximum(bound[~nan], 1e-300)).max(initial=0)
    assert np.all(err <= bound[~nan]), f"{name}: error {worst:.2f}x the matrix-core bound"
    print(f"  {name}: worst error {worst:.3f} of the bound")
    return worst


def _to_dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (37, 45, 96), (128, 128, 64), (200, 130, 256), (256, 384, 1024),
                                   (64, 300, 4096), (300, 140, 1120)])
def test_gemm_random_codes(oracle_mod, M, N, K):
    dev = _dev()
    print(f"case: gemm random codes M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M * 1000 + N + K)
    a, sa = _rand_operands(rng, M, K)
    b, sb = _rand_operands(rng, N, K)
    c = mx.mxfp8_gemm(_to_dev(a, dev), _to_dev(sa, dev), _to_dev(b, dev), _to_dev(sb, dev))
    _check(oracle_mod, f"gemm{M}x{N}x{K}", a, sa, b, sb, c.cpu().numpy())


def test_gemm_half_tiles_match_whole_tiles(oracle_mod):
    """A last round of T tiles runs as 2 T 256 x 128 half tiles when T is at
    most half the CUs, as 4 T 256 x 64 quarter tiles when at most a quarter.
    Over the same A, 4352 x 4096 (272 tiles: 16 in the last round on 256
    CUs), 4352 x 4352 (289: 33) and 4352 x 5120 (340: 84) put different
    tiles in that round, run whole, halved or quartered, so their common
    columns come from different forms in different launches: they must agree
    bit for bit (each element is the same sum in the same order).  A's first
    4160 rows against 4096 columns (a last round of 64-row quarter tiles)
    must equal the same rows of the first result.  The last tile row is
    checked against the oracle on sampled rows and columns."""
    dev = _dev()
    M, K, N1, N2, N3 = 4352, 512, 4096, 4352, 5120
    print(f"case: gemm half and quarter tiles {M}x{N1}/{N2}/{N3}x{K}", flush=True)
    rng = np.random.default_rng(77)
    a, sa = _rand_operands(rng, M, K)
    b, sb = _rand_operands(rng, N3, K)
    A, SA, B, SB = _to_dev(a, dev), _to_dev(sa, dev), _to_dev(b, dev), _to_dev(sb, dev)
    c1 = mx.mxfp8_gemm(A, SA, B[:N1], SB[:N1])
    c2 = mx.mxfp8_gemm(A, SA, B[:N2], SB[:N2])
    c3 = mx.mxfp8_gemm(A, SA, B, SB)
    c4 = mx.mxfp8_gemm(A[:4160], SA[:4160], B[:N1], SB[:N1])
    torch.cuda.synchronize()
    assert torch.equal(c2[:, :N1], c1)
    assert torch.equal(c3[:, :N2], c2)
    assert torch.equal(c4, c1[:4160])
    rows = np.unique(np.concatenate([[0, 3071, 3072, 4095, 4096, 4223, 4224, M - 1], rng.integers(3072, M, 10),
                                     rng.integers(0, M, 6)]))
    cols = np.unique(np.concatenate([[0, 63, 64, 127, 128, 255, 256, N2 - 1, N2, N3 - 65, N3 - 64, N3 - 1],
                                     rng.integers(0, N3, 40)]))
    got = c3.cpu().numpy()[rows][:, cols]
    _check(oracle_mod, "half_tiles", a[rows], sa[rows], b[cols], sb[cols], got)
    cols1 = cols[cols < N1]
    _check(oracle_mod, "quarter_tiles", a[rows], sa[rows], b[cols1], sb[cols1], c1.cpu().numpy()[rows][:, cols1])


@pytest.mark.parametrize("tail", [1, 32, 64, 65, 128, 129])
def test_gemm_short_tiles_match_whole_tiles(oracle_mod, tail):
    """A last tile of at most 64 (128) rows runs in the form whose
    wavefronts compute one (two) row blocks each and load only those rows.
    Its rows must equal, bit for bit, the same rows computed inside whole
    tiles: A's first 1024 + tail rows against all 1280 rows (the tail rows
    at 1024.. fall in a short tile in the first launch and in a whole tile
    in the second; 160 tiles, so no half tiles in either).  Then the
    grouped form with two groups ending in short tiles (192 whole-width
    tiles) against the plain GEMM of each group's rows (96 tiles, all run
    as half tiles)."""
    dev = _dev()
    M, N, K = 1280, 8192, 640
    print(f"case: gemm short tiles, tail {tail}", flush=True)
    rng = np.random.default_rng(300 + tail)
    a, sa = _rand_operands(rng, M, K)
    b, sb = _rand_operands(rng, N, K)
    A, SA, B, SB = _to_dev(a, dev), _to_dev(sa, dev), _to_dev(b, dev), _to_dev(sb, dev)
    m = 1024 + tail
    c_short = mx.mxfp8_gemm(A[:m], SA[:m], B, SB)
    c_whole = mx.mxfp8_gemm(A, SA, B, SB)
    torch.cuda.synchronize()
    assert torch.equal(c_short, c_whole[:m])
    rows = np.unique(np.concatenate([[1024, m - 1], rng.integers(1024, m, 6)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 20)]))
    _check(oracle_mod, f"short_tail{tail}", a[rows], sa[rows], b[cols], sb[cols], c_short.cpu().numpy()[rows][:, cols])
    # two groups of 512 + tail rows, each against expert b (the same matrix twice)
    g1 = 512 + tail
    offs = torch.tensor([g1, 2 * g1], dtype=torch.int32, device=dev)
    Ag = torch.cat([A[:g1], A[:g1]])
    SAg = torch.cat([SA[:g1], SA[:g1]])
    Bg = torch.stack([B, B])
    SBg = torch.stack([SB, SB])
    cg = mx.mxfp8_grouped_gemm(Ag, SAg, Bg, SBg, offs)
    c_plain = mx.mxfp8_gemm(A[:g1], SA[:g1], B, SB)
    torch.cuda.synchronize()
    assert torch.equal(cg[:g1], c_plain) and torch.equal(cg[g1:], c_plain)


@pytest.mark.parametrize("K,shift", [(4160, 0), (1088, 1), (1600, 3), (1056, 2)])
def test_gemm_unaligned_scale_rows_match_aligned(oracle_mod, K, shift):
    """Scale rows that do not start 16-byte aligned (packed rows of K/32
    bytes, the table starting `shift` bytes into its buffer) are read as
    4-byte words, and a last group of fewer than 16 blocks byte by byte.
    The result must equal, bit for bit, the same GEMM with its scale rows
    padded to 16-byte aligned starts (read straight into shared memory)."""
    dev = _dev()
    M, N = 600, 520
    print(f"case: gemm unaligned scale rows K={K} shift={shift}", flush=True)
    rng = np.random.default_rng(K + shift)
    a, sa = _rand_operands(rng, M, K)
    b, sb = _rand_operands(rng, N, K)
    A, B = _to_dev(a, dev), _to_dev(b, dev)

    def placed(s, ld, off):
        rows, w = s.shape
        buf = torch.zeros(off + rows * ld + 16, dtype=torch.uint8, device=dev)
        view = buf[off:off + rows * ld].view(rows, ld)[:, :w]
        view.copy_(torch.from_numpy(s).to(dev))
        return view

    kb = K // 32
    pad = -(-kb // 16) * 16
    c_aligned = mx.mxfp8_gemm(A, placed(sa, pad, 0), B, placed(sb, pad, 0))
    c_packed = mx.mxfp8_gemm(A, placed(sa, kb, shift), B, placed(sb, kb, shift))
    torch.cuda.synchronize()
    assert torch.equal(c_packed, c_aligned)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 12)]))
    _check(oracle_mod, f"unaligned_scales_K{K}", a[rows], sa[rows], b[cols], sb[cols],
           c_packed.cpu().numpy()[rows][:, cols])


def test_gemm_repeated_launches_bit_identical():
    """Twelve launches of one GEMM (16 stages, an even count, and a last
    round of half tiles) give the same result bit for bit: a race between
    the pipeline's loads and its LDS reads shows up as a difference."""
    dev = _dev()
    M, N, K = 4352, 4352, 1024
    print(f"case: gemm repeated launches {M}x{N}x{K}", flush=True)
    rng = np.random.default_rng(78)
    a, sa = _rand_operands(rng, M, K)
    b, sb = _rand_operands(rng, N, K)
    A, SA, B, SB = _to_dev(a, dev), _to_dev(sa, dev), _to_dev(b, dev), _to_dev(sb, dev)
    first = mx.mxfp8_gemm(A, SA, B, SB)
    out = torch.empty_like(first)
    for _ in range(11):
        out.fill_(float("nan"))
        mx.mxfp8_gemm(A, SA, B, SB, out=out)
        assert torch.equal(out, first)


def test_gemm_on_cast_outputs(oracle_mod):
    """The pipeline the casts serve: A = rowwise cast of x [M, K]; B = the
    colwise cast of w [K, N] (q_col [N, K], s_col [N, K/32]) and, again, the
    rowwise cast of w^T [N, K]: both layouts give the same B."""
    dev = _dev()
    M, N, K = 192, 160, 512
    x = synth.normal_bf16((M, K), 1.0, seed=50, device=dev)
    w = synth.normal_bf16((K, N), 0.05, seed=51, device=dev)
    qa, _, sa, _ = mx.mxfp8_quant_2d(x, rowwise=True, colwise=False)
    _, qb, _, sbc = mx.mxfp8_quant_2d(w, rowwise=False, colwise=True)
    qb2, _, sb2, _ = mx.mxfp8_quant_2d(w.t().contiguous(), rowwise=True, colwise=False)
    assert torch.equal(qb, qb2) and torch.equal(sbc, sb2)
    c = mx.mxfp8_gemm(qa, sa, qb, sbc)
    _check(oracle_mod, "cast_pipeline", qa.cpu().numpy(), sa.cpu().numpy(), qb.cpu().numpy(), sbc.cpu().numpy(),
           c.cpu().numpy())
    # and the MX result is close to the bf16 product (quantization error only)
    ref = x.float() @ w.float()
    rel = ((c - ref).norm() / ref.norm()).item()
    assert rel < 0.08, rel


def test_gemm_nan_blocks(oracle_mod):
    dev = _dev()
    rng = np.random.default_rng(7)
    a, sa = _rand_operands(rng, 64, 128)
    b, sb = _rand_operands(rng, 64, 128)
    a[3, 70] = 0x7F
    sb[10, 2] = 255
    c = mx.mxfp8_gemm(_to_dev(a, dev), _to_dev(sa, dev), _to_dev(b, dev), _to_dev(sb, dev))
    _check(oracle_mod, "nan", a, sa, b, sb, c.cpu().numpy())


@pytest.mark.parametrize("K", [160, 1056])
def test_gemm_strided_and_guarded(oracle_mod, K):
    """Operands carved out of wider buffers (scale rows at odd byte
    offsets); C written into a padded buffer whose padding stays untouched."""
    dev = _dev()
    rng = np.random.default_rng(8 + K)
    M, N = 70, 90
    abig, sabig = _rand_operands(rng, M, K + 64)
    bbig, sbbig = _rand_operands(rng, N, K + 96)
    a, sa = abig[:, 32:32 + K], sabig[:, 1:1 + K // 32]
    b, sb = bbig[:, 64:64 + K], sbbig[:, 3:3 + K // 32]
    da, dsa = _to_dev(abig, dev)[:, 32:32 + K], _to_dev(sabig, dev)[:, 1:1 + K // 32]
    db, dsb = _to_dev(bbig, dev)[:, 64:64 + K], _to_dev(sbbig, dev)[:, 3:3 + K // 32]
    big = torch.full((M + 2, N + 7), 7.0, dtype=torch.float32, device=dev)
    out = big[1:M + 1, 2:N + 2]
    mx.mxfp8_gemm(da, dsa, db, dsb, out=out)
    _check(oracle_mod, "strided", a, sa, b, sb, out.cpu().numpy())
    assert (big[0] == 7).all() and (big[M + 1] == 7).all() and (big[:, :2] == 7).all() and (big[:, N + 2:] == 7).all()


def test_gemm_k_zero_gives_zeros():
    dev = _dev()
    a = torch.zeros((5, 0), dtype=torch.uint8, device=dev)
    sa = torch.zeros((5, 0), dtype=torch.uint8, device=dev)
    b = torch.zeros((3, 0), dtype=torch.uint8, device=dev)
    sb = torch.zeros((3, 0), dtype=torch.uint8, device=dev)
    out = torch.full((5, 3), 9.0, device=dev)
    # K = 0: an empty sum is 0 (tensors of zero width have no data pointer
    # requirement beyond being non-NULL; allocate 16 bytes to pass one)
    pad = torch.zeros(16, dtype=torch.uint8, device=dev)
    st = mx.lib().mxfp8_gemm(pad.data_ptr(), 16, pad.data_ptr(), 1, pad.data_ptr(), 16, pad.data_ptr(), 1,
                             5, 3, 0, out.data_ptr(), 3, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert (out == 0).all()
    del a, sa, b, sb


def test_gemm_16384x8192x5120_sampled(oracle_mod):
    """The bench size: sampled rows and columns against the oracle."""
    dev = _dev()
    M, N, K = 16384, 8192, 5120
    print(f"case: gemm {M}x{N}x{K}, sampled", flush=True)
    x = synth.normal_bf16((M, K), 1.0, seed=60, device=dev)
    w = synth.normal_bf16((N, K), 0.02, seed=61, device=dev)
    qa, _, sa, _ = mx.mxfp8_quant_2d(x, rowwise=True)
    qb, _, sb, _ = mx.mxfp8_quant_2d(w, rowwise=True)
    del x, w
    c = mx.mxfp8_gemm(qa, sa, qb, sb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 14)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 30)]))
    ridx = torch.from_numpy(rows).to(dev)
    cidx = torch.from_numpy(cols).to(dev)
    got = c[ridx][:, cidx].cpu().numpy()
    _check(oracle_mod, "bench_size", qa[ridx].cpu().numpy(), sa[ridx].cpu().numpy(), qb[cidx].cpu().numpy(),
           sb[cidx].cpu().numpy(), got)
    del qa, qb, sa, sb, c
    torch.cuda.empty_cache()


@pytest.mark.parametrize("scales", ["packed", "padded"])
def test_gemm_ragged_16000x8000x5216_sampled(oracle_mod, scales):
    """Full-size ragged shape: partial 256-row and 256-column tiles, a last
    K stage of 96 columns, and 163 scale blocks per row (a partial last
    scale group).  Packed scale rows (163 bytes apart) take the byte-wise
    scale path; rows padded to 176 bytes take the 16-byte path for the full
    groups and the byte-wise one for the last."""
    dev = _dev()
    M, N, K = 16000, 8000, 5216
    print(f"case: gemm {M}x{N}x{K}, {scales} scales, sampled", flush=True)
    x = synth.normal_bf16((M, K), 1.0, seed=62, device=dev)
    w = synth.normal_bf16((N, K), 0.02, seed=63, device=dev)
    qa, _, sa, _ = mx.mxfp8_quant_2d(x, rowwise=True)
    qb, _, sb, _ = mx.mxfp8_quant_2d(w, rowwise=True)
    del x, w
    if scales == "padded":
        pa = torch.zeros((M, 176), dtype=torch.uint8, device=dev)
        pb = torch.zeros((N, 176), dtype=torch.uint8, device=dev)
        pa[:, :K // 32] = sa
        pb[:, :K // 32] = sb
        sa_in, sb_in = pa[:, :K // 32], pb[:, :K // 32]
    else:
        sa_in, sb_in = sa, sb
    c = mx.mxfp8_gemm(qa, sa_in, qb, sb_in)
    torch.cuda.synchronize()
    rng = np.random.default_rng(10)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.integers(0, M, 12)]))
    cols = np.unique(np.concatenate([[0, 255, 256, N - 1], rng.integers(0, N, 28)]))
    ridx = torch.from_numpy(rows).to(dev)
    cidx = torch.from_numpy(cols).to(dev)
    got = c[ridx][:, cidx].cpu().numpy()
    _check(oracle_mod, f"ragged_{scales}", qa[ridx].cpu().numpy(), sa[ridx].cpu().numpy(), qb[cidx].cpu().numpy(),
           sb[cidx].cpu().numpy(), got)
    del qa, qb, sa, sb, c
    torch.cuda.empty_cache()


def test_gemm_single_products_exact_and_truncation_threshold():
    """The two facts the bound rests on.  With one nonzero per row (K = 32),
    C[m][n] is one product: exact for all 65536 code pairs, NaN exactly
    where a code is NaN.  Adding a 1.0 * 1.0 term beside it keeps a product
    of 2^-13 and drops one just below (the 13-bit truncation)."""
    dev = _dev()
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    codes = np.arange(256, dtype=np.uint8)
    a = np.zeros((256, 32), np.uint8)
    a[:, 0] = codes
    s = np.full((256, 1), 127, np.uint8)
    c = mx.mxfp8_gemm(t(a), t(s), t(a), t(s)).cpu().numpy().astype(np.float64)
    dec = _values(codes.reshape(256, 1).repeat(32, 1), s)[:, 0]
    want = np.outer(dec, dec)
    fin = np.isfinite(want)
    assert np.array_equal(np.isnan(c), ~fin)
    assert np.array_equal(c[fin], want[fin])
    # two terms: 1.0 plus a small product p in the same MFMA step
    a2 = a.copy()
    a2[:, 5] = 0x38
    c2 = mx.mxfp8_gemm(t(a2), t(s), t(a2), t(s)).cpu().numpy().astype(np.float64)
    small = fin & (np.abs(want) < 1) & (want > 0)
    kept = c2[small] - 1.0
    assert np.all(kept[want[small] >= 2.0 ** -13] == np.trunc(want[small][want[small] >= 2.0 ** -13] * 2 ** 13) / 2 ** 13)
    assert np.all(kept[want[small] < 2.0 ** -13] == 0)


# ------------------------------------------------------------ grouped form
def _check_grouped(oracle_mod, name, a, sa, b, sb, offs, got, sentinel):
    want, mag = oracle_mod.mx_grouped_gemm(a, sa, b, sb, offs)
    got = np.asarray(got, np.float64)
    covered = ~np.isnan(mag[:, 0]) if mag.shape[1] else np.zeros(a.shape[0], bool)
    assert np.all(got[~covered] == sentinel), f"{name}: rows outside every group were written"
    start = 0
    for g in range(b.shape[0]):
        end = int(min(max(int(offs[g]), start), a.shape[0]))
        if end > start:
            bound = 64 * 2.0 ** -13 * _step_max_sum(a[start:end], sa[start:end], b[g], sb[g]) \
                + (a.shape[1] / 64 + 1) * 2.0 ** -24 * mag[start:end]
            err = np.abs(got[start:end] - want[start:end])
            assert np.all(err <= bound), f"{name}: group {g} beyond the bound"
        start = end


@pytest.mark.parametrize("K", [160, 1120])
@pytest.mark.parametrize("offs", [[0, 300, 345, 602], [25, 10, 1000, 1000], [640, 640, 640, 640]])
def test_grouped_gemm_random(oracle_mod, offs, K):
    dev = _dev()
    print(f"case: grouped gemm offsets {offs} K={K}", flush=True)
    rng = np.random.default_rng(sum(offs) + K)
    M, N, G = 640, 200, 4
    a, sa = _rand_operands(rng, M, K)
    bs = [_rand_operands(rng, N, K) for _ in range(G)]
    b, sb = np.stack([x[0] for x in bs]), np.stack([x[1] for x in bs])
    offs = np.array(offs, np.int32)
    out = torch.full((M, N), -7.0, dtype=torch.float32, device=dev)
    mx.mxfp8_grouped_gemm(_to_dev(a, dev), _to_dev(sa, dev), _to_dev(b, dev), _to_dev(sb, dev),
                          torch.from_numpy(offs).to(dev), out=out)
    _check_grouped(oracle_mod, f"grouped{offs.tolist()}", a, sa, b, sb, offs, out.cpu().numpy(), -7.0)


def test_grouped_gemm_one_group_is_the_plain_gemm():
    dev = _dev()
    rng = np.random.default_rng(11)
    a, sa = _rand_operands(rng, 300, 256)
    b, sb = _rand_operands(rng, 170, 256)
    ta, tsa, tb, tsb = (_to_dev(x, dev) for x in (a, sa, b, sb))
    plain = mx.mxfp8_gemm(ta, tsa, tb, tsb)
    grouped = mx.mxfp8_grouped_gemm(ta, tsa, tb[None], tsb[None], torch.tensor([300], dtype=torch.int32, device=dev))
    assert torch.equal(plain, grouped)


def test_grouped_gemm_partial_rows_in_full_rounds(oracle_mod):
    """The M-grouped form runs every group's whole 256-row tiles before the
    groups' partial last rows.  Five groups over 4500 rows (1000 rows each,
    then 500) against 4096 columns: 13 whole tile rows and 5 partial ones,
    288 tiles, so on 256 CUs partial tiles run both in the full round and in
    a last round of quarter tiles.  Every group's rows must equal, bit for
    bit, the plain GEMM of those rows with that group's expert, and sampled
    rows (most in partial tiles) match the oracle."""
    dev = _dev()
    M, N, K, G = 4500, 4096, 256, 5
    ends = [1000, 2000, 3000, 4000, 4500]
    print(f"case: grouped gemm partial rows in full rounds {M}x{N}x{K} G={G}", flush=True)
    rng = np.random.default_rng(31)
    a, sa = _rand_operands(rng, M, K)
    b, sb = _rand_operands(rng, G * N, K)
    A, SA = _to_dev(a, dev), _to_dev(sa, dev)
    B, SB = _to_dev(b, dev).view(G, N, K), _to_dev(sb, dev).view(G, N, K // 32)
    got = mx.mxfp8_grouped_gemm(A, SA, B, SB, torch.tensor(ends, dtype=torch.int32, device=dev))
    start = 0
    for g, end in enumerate(ends):
        plain = mx.mxfp8_gemm(A[start:end], SA[start:end], B[g], SB[g])
        torch.cuda.synchronize()
        assert torch.equal(got[start:end], plain), f"group {g}"
        start = end
    rows = np.array([768, 999, 1768, 3999, 4000, 4255, 4256, 4499])  # partial rows; 4000 and 4255 in a whole tile
    cols = np.unique(np.concatenate([[0, 63, 64, N - 1], rng.integers(0, N, 12)]))
    host = got.cpu().numpy()
    for r in rows:
        g = int(np.searchsorted(ends, r, side="right"))
        bg, sbg = b[g * N:(g + 1) * N], sb[g * N:(g + 1) * N]
        _check(oracle_mod, f"grouped_partial_row{r}", a[[r]], sa[[r]], bg[cols], sbg[cols], host[[r]][:, cols])


def test_grouped_gemm_16640x8192x5120_g4_sampled(oracle_mod):
    """The pages' grouped shape (16640 tokens, 4 experts of 8192 x 5120),
    operands from the casts, uneven groups; sampled rows of every group."""
    dev = _dev()
    M, N, K, G = 16640, 8192, 5120, 4
    print(f"case: grouped gemm {M}x{N}x{K} G={G}, sampled", flush=True)
    x = synth.normal_bf16((M, K), 1.0, seed=80, device=dev)
    qa, _, sa, _ = mx.mxfp8_quant_2d(x, rowwise=True)
    del x
    w = synth.normal_bf16((G * N, K), 0.02, seed=81, device=dev)
    qb, _, sb, _ = mx.mxfp8_quant_2d(w, rowwise=True)
    del w
    qb, sb = qb.view(G, N, K), sb.view(G, N, K // 32)
    offs = np.array([3000, 7100, 12000, 16640], np.int32)
    c = mx.mxfp8_grouped_gemm(qa, sa, qb, sb, torch.from_numpy(offs).to(dev))
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 14)]))
    cidx = torch.from_numpy(cols).to(dev)
    start = 0
    for g in range(G):
        end = int(offs[g])
        rows = np.unique(np.concatenate([[start, end - 1], rng.integers(start, end, 6)]))
        ridx = torch.from_numpy(rows).to(dev)
        _check(oracle_mod, f"g{g}", qa[ridx].cpu().numpy(), sa[ridx].cpu().numpy(), qb[g][cidx].cpu().numpy(),
               sb[g][cidx].cpu().numpy(), c[ridx][:, cidx].cpu().numpy())
        start = end
    del qa, qb, sa, sb, c
    torch.cuda.empty_cache()
