"""GPU parity of the fp4 decode GEMV on bf16 x (fairy2i_gemv with x_dtype BF16 and MFMA_F4 or
AUTO): every workgroup builds its digit records on chip (fp4).  Where the records use one exponent
per row (launches of one wave per tile) the outputs must equal the two-call form
(fairy2i_x_digits_f6, then the GEMV on the digit form) bit for bit -- same digits, same MFMA inputs,
same order.  Small launches (batch 1-2) build per-wave records at one exponent per 256-column chunk:
their fp32 outputs are held within 1e-6 of the two-call form, and every form matches the oracle
within the fp32 tolerance.  Cases cover every launch form: small launches (a tile's chunks split
over 2, 4 or 8 waves), one wave per tile, the mixed-granularity large launch (four tiles per
workgroup sharing the records, then the split tail), batch 1 and 2, T = 1..4, ragged rows and the
longest rows the records allow."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL_F32, announce, check_bf16, device, down, rel_l2, up, x_to_dev

import widely_linear_gemv_amd as f2

pytestmark = pytest.mark.gpu


def layer(n, m, T, seed):
    return workloads.random_codes(T, n, m, seed=seed), workloads.random_scales(n, T, seed=seed + 1)


def bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


TOL_LOCAL = 1e-6     # fp32 summation across chunks, relative L2


def local_form(n_tiles, m, B):
    """Whether a call on bf16 x takes the per-wave records with per-chunk exponents: batch 1-2,
    below 1536 tiles, and at least two 256-column chunks (so a tile's chunks split over waves)."""
    return B <= 2 and n_tiles < 1536 and m > 256


def assert_two_call(got, two, local, ydt, label, want):
    """The fused form against the two-call form: bit for bit; or, with per-chunk exponents (each
    chunk's X keeps at least the bits it keeps at one exponent per row), fp32 outputs no further
    from the oracle's than the two-call form's plus TOL_LOCAL; the local form's bf16 outputs are
    checked against the oracle by the caller."""
    if not local:
        assert np.array_equal(bits(got), bits(two)), label
    elif ydt == torch.float32:
        assert rel_l2(got, want) <= rel_l2(two, want) + TOL_LOCAL, (label, rel_l2(got, want), rel_l2(two, want))


@pytest.mark.parametrize("n,m,T,B", [(5, 64, 1, 1), (17, 320, 2, 2), (40, 2048, 2, 1), (33, 1088, 3, 2),
                                     (100, 5504, 2, 1), (9, 8192, 2, 1), (21, 4096, 4, 2), (300, 2048, 2, 2),
                                     (1030, 5504, 2, 1), (1040, 4096, 3, 2)])
def test_fused_matches_two_call_and_oracle(n, m, T, B):
    dev = device()
    codes, scales = layer(n, m, T, seed=n * 7 + m + T)
    act = workloads.activations(B, 2 * m, seed=800 + B + m)
    packed, s = up(oracle.pack(codes), dev), up(scales, dev)
    x = x_to_dev(act, dev)
    local = local_form((n + 15) // 16, m, B)
    want = oracle.gemv_ref(codes, scales, act.values)
    for ydt in (torch.float32, torch.bfloat16):
        announce("gemv fp4 fused", n, m, T, B, ydt)
        got = down(f2.fairy2i_gemv(packed, s, x, algo=f2.GEMV_MFMA_F4, y_dtype=ydt))
        two = down(f2.fairy2i_gemv(packed, s, f2.fairy2i_x_digits_f6(x), algo=f2.GEMV_MFMA_F4, y_dtype=ydt))
        assert_two_call(got, two, local, ydt, (n, m, T, B, ydt), want)
    assert rel_l2(down(f2.fairy2i_gemv(packed, s, x, algo=f2.GEMV_MFMA_F4)), want) <= TOL_F32
    check_bf16(down(f2.fairy2i_gemv(packed, s, x, algo=f2.GEMV_MFMA_F4, y_dtype=torch.bfloat16)), want, "fused")


@pytest.mark.parametrize("B,m,T", [(1, 1088, 2), (2, 320, 3), (2, 2048, 1)])
def test_fused_rounding_matches_two_call(B, m, T):
    """x over 2^-20 .. 2^6 with zeros, and a quarter of its entries exactly half-way for
    X = x 2^S (odd multiples of 2^-(S+1) beside a maximum of 1, S = 21, or of 3, S = 20): the
    records built on chip round to nearest even exactly as the digit form does, whose X the
    digit-form test holds to np.rint, so the outputs are bit-identical to the two-call form.  (At
    batch 1 the launch takes per-chunk exponents; there the ties hold only in the chunks that
    contain the maximum, and the outputs are held to TOL_LOCAL and the oracle.)"""
    dev = device()
    n = 48
    rng = np.random.default_rng(90 + B + m + T)
    v = rng.standard_normal((B, 2 * m)).astype(np.float32)
    v *= np.float32(2.0) ** rng.integers(-20, 6, size=v.shape).astype(np.float32)
    v[rng.random(v.shape) < 0.05] = 0.0
    for b, amax, S in ((0, 1.0, 21), (1, 3.0, 20)):
        if b >= B:
            break
        v[b] *= np.float32(amax) / np.abs(v[b]).max()
        v[b, int(np.argmax(np.abs(v[b])))] = amax
        ties = rng.random(2 * m) < 0.25
        odd = (2 * rng.integers(0, 128, size=2 * m) + 1).astype(np.float32)
        sign = np.where(rng.random(2 * m) < 0.5, -1.0, 1.0).astype(np.float32)
        v[b] = np.where(ties, sign * odd * np.float32(2.0) ** -(S + 1), v[b])
        v[b, int(np.argmax(np.abs(v[b])))] = amax          # the maximum survives the ties
    bits_ = workloads.f32_to_bf16_bits(v)
    act = workloads.Activations(values=workloads.bf16_bits_to_f32(bits_), dtype="bf16", bf16_bits=bits_)
    codes, scales = layer(n, m, T, seed=700 + m)
    packed, s = up(oracle.pack(codes), dev), up(scales, dev)
    x = x_to_dev(act, dev)
    announce("gemv fp4 fused rounding", n, m, T, B)
    local = local_form(3, m, B)
    want = oracle.gemv_ref(codes, scales, act.values)
    for ydt in (torch.float32, torch.bfloat16):
        got = down(f2.fairy2i_gemv(packed, s, x, algo=f2.GEMV_MFMA_F4, y_dtype=ydt))
        two = down(f2.fairy2i_gemv(packed, s, f2.fairy2i_x_digits_f6(x), algo=f2.GEMV_MFMA_F4, y_dtype=ydt))
        assert_two_call(got, two, local, ydt, (m, T, B, ydt), want)
    assert rel_l2(down(f2.fairy2i_gemv(packed, s, x, algo=f2.GEMV_MFMA_F4)), want) <= TOL_F32


@pytest.mark.parametrize("B,T,batch,n", [(1, 2, 128, 256), (1, 3, 48, 256), (2, 2, 100, 256), (1, 1, 200, 256),
                                         (2, 2, 513, 40), (1, 4, 97, 256), (1, 2, 800, 256), (1, 3, 800, 250)])
def test_fused_large_strided_launch(B, T, batch, n):
    """The strided batch (one launch over many layers sharing x) in the large-launch forms: four
    tiles per workgroup sharing one set of records (the last workgroup partly empty when the tile
    count is not a multiple of four), and from 12288 tiles at batch 1 and T <= 3 the
    mixed-granularity form (then the last 1536 tiles split over four waves); below 1536 tiles at
    batch 1, the per-chunk-exponent form.  Distinct layers; every output against the two-call
    form, sampled layers against the oracle."""
    dev = device()
    m = 2048
    g = torch.Generator(device=dev)
    g.manual_seed(batch + T)
    nb = f2.fairy2i_packed_bytes(n, m, T)
    pool = torch.randint(0, 256, (batch, nb), dtype=torch.uint8, device=dev, generator=g)
    spool = (torch.rand((batch, n, T, 2, 2), device=dev, generator=g) * 0.02).contiguous()
    act = workloads.activations(B, 2 * m, seed=900 + B)
    x = x_to_dev(act, dev)
    y1 = torch.empty((batch, B, 2 * n), device=dev)
    y2 = torch.empty_like(y1)
    announce("gemv fp4 fused strided", batch, n, m, T, B)
    f2.fairy2i_gemv_strided(pool, spool, x, y1, algo=f2.GEMV_MFMA_F4)
    f2.fairy2i_gemv_strided(pool, spool, f2.fairy2i_x_digits_f6(x), y2, algo=f2.GEMV_MFMA_F4)
    a, b = down(y1), down(y2)
    local = local_form(batch * ((n + 15) // 16), m, B)
    if not local:
        assert np.array_equal(bits(a), bits(b))
    if batch * ((n + 15) // 16) >= 1536:           # AUTO takes the fp4 kernel on bf16 x for large launches
        y3 = torch.empty_like(y1)
        f2.fairy2i_gemv_strided(pool, spool, x, y3)
        assert np.array_equal(bits(down(y3)), bits(a))
    # the pool's packed bytes are arbitrary: recover codes through the oracle's unpacking
    for k in (0, batch // 2, batch - 1):
        codes = oracle.unpack(down(pool[k]), n, m, T)
        want = oracle.gemv_ref(codes, down(spool[k]), act.values)
        assert rel_l2(a[k], want) <= TOL_F32, k
        if local:
            assert_two_call(a[k], b[k], local, torch.float32, k, want)


@pytest.mark.parametrize("B,m,tiles,fused", [(1, 2048, 24, True), (1, 5504, 8, True), (1, 8192, 16, True),
                                              (1, 8192, 260, True), (1, 1024, 40, False), (1, 1024, 130, True),
                                              (1, 960, 300, False), (2, 2048, 24, False)])
def test_auto_on_bf16_x_small_launches(B, m, tiles, fused):
    """AUTO on bf16 x below 1536 tiles: the fp4 kernel with on-chip digits at batch 1 for
    2048 <= m <= 8192, and for 1024 <= m < 2048 in launches of at least 128 tiles; the bf16
    kernel otherwise.  Checked bit for bit against the kernel that should run, and against the
    oracle."""
    dev = device()
    n, T = 16 * tiles, 2
    codes, scales = layer(n, m, T, seed=40 + m + tiles)
    act = workloads.activations(B, 2 * m, seed=60 + B + m)
    packed, s = up(oracle.pack(codes), dev), up(scales, dev)
    x = x_to_dev(act, dev)
    announce("gemv auto bf16 x", n, m, T, B, fused)
    got = down(f2.fairy2i_gemv(packed, s, x))
    want_algo = f2.GEMV_MFMA_F4 if fused else f2.GEMV_MFMA_BF16
    assert np.array_equal(bits(got), bits(down(f2.fairy2i_gemv(packed, s, x, algo=want_algo)))), (B, m, tiles)
    assert rel_l2(got, oracle.gemv_ref(codes, scales, act.values)) <= TOL_F32


@pytest.mark.parametrize("m,T,NW_tiles", [(2048, 2, 24), (1088, 3, 5), (5504, 2, 80), (512, 1, 8), (8192, 2, 2)])
def test_fused_local_chunk_exponents(m, T, NW_tiles):
    """Small launches on bf16 x (here batch 1): every chunk of 256 columns is digitized at its own
    exponent, which enters the MFMAs as a block scale.  x puts chunks at very different scales --
    2^-100 (exponent 121: the scale split over both operands), 2^100 (exponent -79), all zeros,
    N(0, 1) -- and ragged rows end on a partial chunk.  Each case alone (x nonzero in one chunk,
    so the output has that chunk's scale) and all together, against the oracle at the fp32
    tolerance; 2 to 8 waves per tile (one to four passes of two chunks per wave)."""
    dev = device()
    n = 16 * NW_tiles
    codes, scales = layer(n, m, T, seed=1100 + m + T)
    packed, s = up(oracle.pack(codes), dev), up(scales, dev)
    nchunk = (m + 255) // 256
    rng = np.random.default_rng(1200 + m)
    base = rng.standard_normal((1, 2 * m)).astype(np.float32)
    col_chunk = np.concatenate([np.arange(m) // 256] * 2)          # chunk of every real column
    factor = np.ones(nchunk, dtype=np.float32)
    factor[0 % nchunk] = np.float32(2.0) ** -100
    factor[1 % nchunk] = np.float32(2.0) ** 100
    factor[2 % nchunk] = 0.0
    cases = {"all": factor[col_chunk]}
    for c in range(min(nchunk, 3)):
        f = np.zeros(nchunk, dtype=np.float32)
        f[c] = factor[c] if factor[c] != 0 else 1.0
        cases[f"chunk{c}"] = f[col_chunk]
    cases["last"] = (col_chunk == nchunk - 1).astype(np.float32)    # the ragged chunk alone
    for label, f in cases.items():
        bits_ = workloads.f32_to_bf16_bits(base * f)
        act = workloads.Activations(values=workloads.bf16_bits_to_f32(bits_), dtype="bf16", bf16_bits=bits_)
        x = x_to_dev(act, dev)
        announce("gemv fp4 local exponents", m, T, n, label)
        got = down(f2.fairy2i_gemv(packed, s, x, algo=f2.GEMV_MFMA_F4))
        want = oracle.gemv_ref(codes, scales, act.values)
        assert np.all(np.isfinite(got)), label
        assert rel_l2(got, want) <= TOL_F32, (label, rel_l2(got, want))


def test_fused_grouped_and_zero_column():
    """Grouped call (items of different n sharing x) on bf16 x; an all-zero batch column (S = 0,
    every digit 0) next to a normal one."""
    dev = device()
    m, T, B = 1024, 2, 2
    act = workloads.activations(B, 2 * m, seed=950)
    vals = act.values.copy()
    bits16 = act.bf16_bits.copy()
    bits16[1] = 0
    vals[1] = 0.0
    x = torch.from_numpy(bits16.view(np.int16)).to(dev).view(torch.bfloat16)
    items, refs = [], []
    for k, n in enumerate((16, 33, 300)):
        codes, scales = layer(n, m, T, seed=960 + k)
        items.append((up(oracle.pack(codes), dev), up(scales, dev), x, torch.empty((B, 2 * n), device=dev)))
        refs.append(oracle.gemv_ref(codes, scales, vals))
    announce("gemv fp4 fused grouped")
    ys = f2.fairy2i_gemv_grouped(items, algo=f2.GEMV_MFMA_F4)
    xd = f2.fairy2i_x_digits_f6(x)
    ys2 = f2.fairy2i_gemv_grouped([(p, s, xd, torch.empty_like(y)) for (p, s, _, y) in items], algo=f2.GEMV_MFMA_F4)
    for y, y2, want in zip(ys, ys2, refs):       # 23 tiles at m = 1024: per-chunk exponents
        assert_two_call(down(y)[0], down(y2)[0], True, torch.float32, "grouped", want[0])
        assert np.all(down(y)[1] == 0.0)
        assert rel_l2(down(y)[0], want[0]) <= TOL_F32


@pytest.mark.parametrize("B,m,T", [(1, 8192, 2), (2, 4096, 2), (2, 64, 1), (1, 5504, 3), (2, 2048, 4)])
def test_fused_persistent_row_lengths(B, m, T):
    """The resident-workgroup form (launches of at least 1536 tiles) up to the longest rows whose
    records fit: batch 2 builds its records from x in global memory (no staged copy), batch 1 from
    the copy in LDS.  One-tile layers, so the launch's tile count is the layer count; every output
    against the two-call form bit for bit, sampled layers against the oracle."""
    dev = device()
    n, batch = 16, 1540
    g = torch.Generator(device=dev)
    g.manual_seed(m + 10 * B + T)
    nb = f2.fairy2i_packed_bytes(n, m, T)
    pool = torch.randint(0, 256, (batch, nb), dtype=torch.uint8, device=dev, generator=g)
    spool = (torch.rand((batch, n, T, 2, 2), device=dev, generator=g) * 0.02).contiguous()
    act = workloads.activations(B, 2 * m, seed=970 + B + m)
    x = x_to_dev(act, dev)
    y1 = torch.empty((batch, B, 2 * n), device=dev)
    y2 = torch.empty_like(y1)
    announce("gemv fp4 fused persistent", B, m, T)
    f2.fairy2i_gemv_strided(pool, spool, x, y1, algo=f2.GEMV_MFMA_F4)
    f2.fairy2i_gemv_strided(pool, spool, f2.fairy2i_x_digits_f6(x), y2, algo=f2.GEMV_MFMA_F4)
    a = down(y1)
    assert np.array_equal(bits(a), bits(down(y2)))
    for k in (0, batch - 1):
        codes = oracle.unpack(down(pool[k]), n, m, T)
        assert rel_l2(a[k], oracle.gemv_ref(codes, down(spool[k]), act.values)) <= TOL_F32, k


_LDS_ORDER = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
import widely_linear_gemv_amd as f2
dev = torch.device("cuda:0")
g = torch.Generator(device=dev)
g.manual_seed(5)
for n, batch in ((40, 1), (16, 1540)):          # small launches, then the resident-workgroup form
    for m in (4160, 8192):                       # 67 KB of LDS first, then 128 KB
        nb = f2.fairy2i_packed_bytes(n, m, 2)
        pool = torch.randint(0, 256, (batch, nb), dtype=torch.uint8, device=dev, generator=g)
        sc = (torch.rand((batch, n, 2, 2, 2), device=dev, generator=g) * 0.02).contiguous()
        x = torch.randn((1, 2 * m), device=dev, generator=g).to(torch.bfloat16)
        y1 = torch.empty((batch, 1, 2 * n), device=dev)
        y2 = torch.empty_like(y1)
        f2.fairy2i_gemv_strided(pool, sc, x, y1, algo=f2.GEMV_MFMA_F4)
        f2.fairy2i_gemv_strided(pool, sc, f2.fairy2i_x_digits_f6(x), y2, algo=f2.GEMV_MFMA_F4)
        torch.cuda.synchronize()
        if batch == 1:                           # per-chunk exponents: close to the two-call form
            err = ((y1 - y2).norm() / y2.norm()).item()
            assert err <= 1e-5, (n, batch, m, err)
        else:
            assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), (n, batch, m)
print("lds order ok")
"""


def test_fused_lds_limit_grows_within_a_process():
    """A fresh process whose first launches on bf16 x need just over 64 KB of LDS and whose later
    ones need 128 KB: the kernels' LDS limit is set for the largest launch the API accepts, so
    the later launches run too (they used to fail with the limit of the first)."""
    import os
    import subprocess
    device()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    announce("gemv fp4 fused LDS limit in a fresh process")
    res = subprocess.run([sys.executable, "-c", _LDS_ORDER, root], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0 and "lds order ok" in res.stdout, res.stdout[-2000:] + res.stderr[-2000:]
