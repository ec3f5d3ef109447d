"""GPU parity: fairy2i_gemv (VALU and MFMA kernels) against the oracle GEMV.

fp32 output: relative L2 <= 1e-5 against the fp64 oracle; bf16 output: <= 2e-3.  Inputs are
oracle-quantized layers (tiny, attention) or seeded random codes and scales (MLP shapes),
packed by the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL_F32, announce, check_bf16, device, down, rel_l2, up, x_to_dev

import widely_linear_gemv_amd as f2

pytestmark = pytest.mark.gpu

ALGOS = {"valu": f2.GEMV_VALU, "mfma": f2.GEMV_MFMA, "bf16": f2.GEMV_MFMA_BF16, "i8": f2.GEMV_MFMA_I8,
         "f4": f2.GEMV_MFMA_F4}
DIGITS = {"i8": f2.fairy2i_x_digits, "f4": f2.fairy2i_x_digits_f6}     # kernels that take a digit form


def run(dev, codes, scales, act, algo, y_dtype):
    packed = up(oracle.pack(codes), dev)
    s = up(scales.astype(np.float32), dev)
    x = x_to_dev(act, dev)
    if algo == f2.GEMV_MFMA_I8:
        x = f2.fairy2i_x_digits(x)
    elif algo == f2.GEMV_MFMA_F4:
        x = f2.fairy2i_x_digits_f6(x)
    y = f2.fairy2i_gemv(packed, s, x, algo=algo, y_dtype=y_dtype)
    return down(y)


def check(dev, codes, scales, act, algo, label):
    want = oracle.gemv_ref(codes, scales.astype(np.float32), act.values)
    announce("gemv", label, algo, "f32 out")
    got = run(dev, codes, scales, act, ALGOS[algo], torch.float32)
    err = rel_l2(got, want)
    assert err <= TOL_F32, (label, algo, "f32", err)
    announce("gemv", label, algo, "bf16 out")
    check_bf16(run(dev, codes, scales, act, ALGOS[algo], torch.bfloat16), want, (label, algo))


_ATTN = {}


def attention_layer():
    if not _ATTN:
        codes, s32, _, _ = oracle.quantize(workloads.ATTN.weight(), 2)
        _ATTN["v"] = (codes, s32)
    return _ATTN["v"]


def test_tiny_fp32_x():
    dev = device()
    codes, s32, _, _ = oracle.quantize(workloads.TINY.weight(), 2)
    act = workloads.activations(1, 256, workloads.TINY_X_SEED, "f32")
    check(dev, codes, s32, act, "valu", "tiny")


@pytest.mark.parametrize("B,algo", [(1, "valu"), (4, "valu"), (16, "valu"), (1, "bf16"), (4, "bf16"),
                                    (16, "bf16"), (1, "i8"), (1, "f4"), (1, "mfma"), (4, "mfma"), (16, "mfma")])
def test_attention(B, algo):
    dev = device()
    codes, s32 = attention_layer()
    act = workloads.activations(B, 4096, workloads.ATTN_X_SEEDS[B])
    check(dev, codes, s32, act, algo, f"attention B={B}")


@pytest.mark.parametrize("shape", ["gate_up", "down"])
@pytest.mark.parametrize("T", [2, 3])
@pytest.mark.parametrize("B", [1, 8])
def test_mlp_shapes(shape, T, B):
    dev = device()
    layer = workloads.MLP_GATE_UP if shape == "gate_up" else workloads.MLP_DOWN
    n, m = layer.n, layer.m
    codes = workloads.random_codes(T, n, m, seed=layer.seed + T)
    scales = workloads.random_scales(n, T, seed=layer.seed + 10 * T)
    act = workloads.activations(B, 2 * m, workloads.MLP_X_SEEDS[shape] + B)
    for algo in ("mfma", "valu", "bf16") + (("i8", "f4") if B <= 2 else ()):
        check(dev, codes, scales, act, algo, f"{shape} T={T} B={B}")


@pytest.mark.parametrize("n,m,T,B", [(1, 64, 1, 1), (17, 192, 2, 3), (33, 128, 4, 5), (5, 320, 3, 16),
                                     (16, 64, 2, 2), (100, 1024, 2, 7), (19, 5504, 3, 2), (40, 6208, 2, 1)])
@pytest.mark.parametrize("algo", ["valu", "bf16", "i8", "f4"])
def test_ragged_and_small(n, m, T, B, algo):
    if algo in DIGITS and B > 2:
        pytest.skip("the digit-form kernels take B <= 2")
    """Ragged row tiles, m not a multiple of 128 (half-empty last MFMA step), every T, odd B."""
    dev = device()
    codes = workloads.random_codes(T, n, m, seed=n + m + T + B)
    scales = workloads.random_scales(n, T, seed=n * 3 + B)
    act = workloads.activations(B, 2 * m, seed=m + B)
    check(dev, codes, scales, act, algo, f"n={n} m={m} T={T} B={B}")


@pytest.mark.parametrize("algo,B", [("valu", 4), ("bf16", 4), ("i8", 2), ("f4", 2), ("f4", 1)])
def test_zero_and_wide_range_x(algo, B):
    """x with exact zeros and magnitudes spread over 2^-6 .. 2^8 inside each 32-column block."""
    dev = device()
    n, m, T = 64, 512, 2
    rng = np.random.default_rng(3)
    v = rng.standard_normal((B, 2 * m)).astype(np.float32)
    v *= np.float32(2.0) ** rng.integers(-6, 8, size=v.shape).astype(np.float32)
    v[rng.random(v.shape) < 0.1] = 0.0
    bits = workloads.f32_to_bf16_bits(v)
    act = workloads.Activations(values=workloads.bf16_bits_to_f32(bits), dtype="bf16", bf16_bits=bits)
    codes = workloads.random_codes(T, n, m, seed=4)
    scales = workloads.random_scales(n, T, seed=5)
    check(dev, codes, scales, act, algo, "wide-range x")


def test_stage_independence_on_gpu():
    """The T stage terms are independent and summed: the T-stage result equals the sum of the
    single-stage results (each computed by the GPU from the same codes)."""
    dev = device()
    codes, s32 = attention_layer()
    act = workloads.activations(4, 4096, 203)
    announce("gemv stage independence")
    full = run(dev, codes, s32, act, f2.GEMV_MFMA, torch.float32)
    parts = sum(run(dev, codes[t:t + 1], np.ascontiguousarray(s32[:, t:t + 1]), act, f2.GEMV_MFMA,
                    torch.float32) for t in range(2))
    assert rel_l2(full, parts) <= TOL_F32


def test_graph_replay_matches_eager():
    """A captured sequence of GEMV launches replays to the eager result, every time, with eager
    work and synchronizations between replays."""
    dev = device()
    codes, s32 = attention_layer()
    packed = up(oracle.pack(codes), dev)
    s = up(s32, dev)
    outs = {}
    for B in (1, 4, 16):
        act = workloads.activations(B, 4096, workloads.ATTN_X_SEEDS[B])
        x = x_to_dev(act, dev)
        announce("graph replay B =", B)
        eager = f2.fairy2i_gemv(packed, s, x, algo=f2.GEMV_MFMA)
        eager_valu = f2.fairy2i_gemv(packed, s, x, algo=f2.GEMV_VALU)
        eager_i8 = f2.fairy2i_gemv(packed, s, f2.fairy2i_x_digits(x), algo=f2.GEMV_MFMA_I8) if B <= 2 else None
        eager_f4 = f2.fairy2i_gemv(packed, s, f2.fairy2i_x_digits_f6(x), algo=f2.GEMV_MFMA_F4) if B <= 2 else None
        torch.cuda.synchronize()
        y = torch.empty_like(eager)
        yv = torch.empty_like(eager)
        yi = torch.empty_like(eager)
        yf = torch.empty_like(eager)
        xd = f2.XDigits(torch.empty((f2.fairy2i_x_digits_bytes(2048, B),), dtype=torch.uint8, device=dev), B, 2048)
        xf = f2.XDigits(torch.empty((f2.fairy2i_x_digits_f6_bytes(2048, B),), dtype=torch.uint8, device=dev), B,
                        2048, f2.X_DIGITS_F6)
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cap):
            f2.fairy2i_gemv(packed, s, x, y=y, algo=f2.GEMV_MFMA)
            f2.fairy2i_gemv(packed, s, x, y=yv, algo=f2.GEMV_VALU)
            if B <= 2:
                f2.fairy2i_x_digits(x, out=xd)
                f2.fairy2i_gemv(packed, s, xd, y=yi, algo=f2.GEMV_MFMA_I8)
                f2.fairy2i_x_digits_f6(x, out=xf)
                f2.fairy2i_gemv(packed, s, xf, y=yf, algo=f2.GEMV_MFMA_F4)
        for rep in range(3):
            y.fill_(float("nan"))
            yv.fill_(float("nan"))
            yi.fill_(float("nan"))
            yf.fill_(float("nan"))
            xd.buf.fill_(0x55)
            xf.buf.fill_(0x55)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, eager), (B, rep)
            assert torch.equal(yv, eager_valu), (B, rep)
            if B <= 2:
                assert torch.equal(yi, eager_i8), (B, rep)
                assert torch.equal(yf, eager_f4), (B, rep)
            f2.fairy2i_gemv(packed, s, x, algo=f2.GEMV_VALU)     # eager work between replays
            torch.cuda.synchronize()
        outs[B] = eager


@pytest.mark.parametrize("algo", ["mfma", "valu", "i8", "f4"])
def test_grouped_matches_single_and_oracle(algo):
    """A grouped call over items of different n (and more items than one launch holds) gives,
    item by item, exactly the single-call result, within tolerance of the oracle."""
    dev = device()
    m, T, B = 512, 2, (2 if algo in DIGITS else 3)
    ns = [16, 33, 1, 200, 64] * 11              # 55 items -> two launches of the grouped kernel
    act = workloads.activations(B, 2 * m, seed=21)
    x = x_to_dev(act, dev)
    if algo in DIGITS:
        x = DIGITS[algo](x)
    items, singles, refs = [], [], []
    for k, n in enumerate(ns):
        codes = workloads.random_codes(T, n, m, seed=1000 + k)
        scales = workloads.random_scales(n, T, seed=2000 + k)
        packed = up(oracle.pack(codes), dev)
        s = up(scales, dev)
        y = torch.full((B, 2 * n), float("nan"), dtype=torch.float32, device=dev)
        items.append((packed, s, x, y))
        singles.append(f2.fairy2i_gemv(packed, s, x, algo=ALGOS[algo]))
        if k < 10:
            refs.append(oracle.gemv_ref(codes, scales, act.values))
    announce("grouped gemv", algo, len(items), "items")
    f2.fairy2i_gemv_grouped(items, algo=ALGOS[algo])
    torch.cuda.synchronize()
    for k, it in enumerate(items):
        assert torch.equal(it[3], singles[k]), k
        if k < 10:
            assert rel_l2(down(it[3]), refs[k]) <= TOL_F32, k


@pytest.mark.parametrize("B,dtype", [(1, "bf16"), (2, "bf16"), (1, "f32"), (2, "f32")])
def test_x_digits_represent_x(B, dtype):
    """The digit form holds, per batch column, S with max|x| 2^S in [2^21, 2^22) and digits whose
    value d0 + 2^8 d1 + 2^16 d2 equals round_half_even(x 2^S); for bf16 x that is x 2^S exactly
    whenever |x| is within 2^14 of the column maximum.  Slot 3 is zero."""
    dev = device()
    m = 1024
    rng = np.random.default_rng(40 + B)
    v = rng.standard_normal((B, 2 * m)).astype(np.float32)
    v *= np.float32(2.0) ** rng.integers(-20, 6, size=v.shape).astype(np.float32)
    v[rng.random(v.shape) < 0.05] = 0.0
    if B == 2:
        v[1] = 0.0                                   # an all-zero column: S = 0, all digits 0
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(v)
        v = workloads.bf16_bits_to_f32(bits)
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        x = torch.from_numpy(v).to(dev)
    announce("x digits", B, dtype)
    blob = down(f2.fairy2i_x_digits(x).buf)
    hdr = blob[:64].view(np.int32)
    assert hdr[0] == B and hdr[1] == m
    dg = blob[64:].view(np.int8).reshape(B, 2, 4, m).astype(np.int64)
    for b in range(B):
        amax = float(np.abs(v[b]).max())
        S = int(hdr[2 + b])
        if amax == 0.0:
            assert S == 0 and not dg[b].any()
            continue
        assert 2.0 ** 21 <= amax * 2.0 ** S < 2.0 ** 22
        X = dg[b, :, 0] + 256 * dg[b, :, 1] + 65536 * dg[b, :, 2]
        assert not dg[b, :, 3].any()
        want = np.rint(v[b].reshape(2, m).astype(np.float64) * 2.0 ** S)
        assert np.array_equal(X, want.astype(np.int64))
        if dtype == "bf16":
            near = np.abs(v[b].reshape(2, m)) >= amax * 2.0 ** -14
            assert np.array_equal(X[near] * 2.0 ** -S, v[b].reshape(2, m)[near].astype(np.float64))


def f6_value(bits):
    """fp6 e2m3 (sign, 2 exponent bits, 3 mantissa bits; bias 1) -> float."""
    sgn = -1.0 if bits & 0x20 else 1.0
    e, mant = (bits >> 3) & 3, bits & 7
    return sgn * (mant / 8.0 if e == 0 else (1.0 + mant / 8.0) * 2.0 ** (e - 1))


def f6_record_columns(g, s):
    """Columns (within a 256-column chunk) of the 32 digits of a record of lane group g, half s: the
    order in which the fp4 planes of the packed words list their codes.  Element q comes from word
    2s + q // 16 of the lane's 64 columns; within the word from nibble j = q % 8, its lower code
    (bits 0-1) for (q // 8) % 2 == 0, else its upper code; code p of a word sits at bits
    8 (p % 4) + 2 (p // 4)."""
    cols = []
    for q in range(32):
        word, upper, j = 2 * s + q // 16, (q // 8) % 2, q % 8
        bit = 4 * j + 2 * upper
        p = 4 * ((bit % 8) // 2) + bit // 8
        cols.append(64 * g + 16 * word + p)
    return cols


@pytest.mark.parametrize("B,dtype,m", [(1, "bf16", 1088), (2, "f32", 1024), (1, "f32", 64)])
def test_x_digits_f6_represent_x(B, dtype, m):
    """The fp6 digit form holds the same S as the int8 form, and in every record 32 fp6 digits in
    [-4, 3] whose value sum_l 8^l d_l over the eight digit records of a column equals
    round_half_even(x 2^S); bytes 24..31 of each record and the records of absent 64-column groups
    are zero."""
    dev = device()
    rng = np.random.default_rng(50 + B + m)
    v = rng.standard_normal((B, 2 * m)).astype(np.float32)
    v *= np.float32(2.0) ** rng.integers(-20, 6, size=v.shape).astype(np.float32)
    v[rng.random(v.shape) < 0.05] = 0.0
    if B == 2:
        v[1] = 0.0
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(v)
        v = workloads.bf16_bits_to_f32(bits)
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        x = torch.from_numpy(v).to(dev)
    announce("x digits f6", B, dtype, m)
    xf = f2.fairy2i_x_digits_f6(x)
    blob = down(xf.buf)
    assert blob.size == f2.fairy2i_x_digits_f6_bytes(m, B)
    hdr = blob[:64].view(np.int32)
    assert hdr[0] == B and hdr[1] == m
    S_i8 = down(f2.fairy2i_x_digits(x).buf)[:64].view(np.int32)[2:2 + B]
    nchunk = -(-m // 256)
    rec = blob[64:].reshape(nchunk, 2, B, 64, 32)
    assert not rec[..., 24:].any()
    for b in range(B):
        S = int(hdr[2 + b])
        assert S == S_i8[b]
        want = np.rint(v[b].reshape(2, m).astype(np.float64) * 2.0 ** S).astype(np.int64)
        X = np.zeros((2, m), dtype=np.int64)
        seen = np.zeros((2, m), dtype=bool)
        for c in range(nchunk):
            for s in range(2):
                for g in range(4):
                    present = 256 * c + 64 * g < m
                    cols = f6_record_columns(g, s)
                    for comp in range(2):
                        for l in range(8):
                            r = rec[c, s, b, 16 * g + 8 * comp + l]
                            word = int.from_bytes(r[:24].tobytes(), "little")
                            for q in range(32):
                                d = f6_value((word >> (6 * q)) & 0x3F)
                                if not present:
                                    assert d == 0.0
                                    continue
                                assert d == int(d) and -4 <= d <= 3
                                X[comp, 256 * c + cols[q]] += int(d) * 8 ** l
                                seen[comp, 256 * c + cols[q]] = True
        assert seen.all()
        assert np.array_equal(X, want)


@pytest.mark.parametrize("B,m,T", [(3, 320, 2), (4, 2048, 2), (9, 320, 1), (16, 320, 3), (16, 2048, 2)])
def test_grouped_large_batch_shared_x(B, m, T):
    """Grouped launches of at least 1536 row tiles at B >= 3 run the shared-x bf16 kernel (x
    staged per chunk in LDS for 8 tiles of one item).  Items of 2048 rows plus ragged ones (37,
    1, 200 rows: workgroups with absent tiles), a partial last chunk (m = 320), odd B and both
    column groups; every item (or a sample at m = 2048) against the oracle."""
    dev = device()
    ns = [2048] * 12 + [37, 1, 200]
    act = workloads.activations(B, 2 * m, seed=70 + B + m)
    x = x_to_dev(act, dev)
    items, host = [], []
    for k, n in enumerate(ns):
        codes = workloads.random_codes(T, n, m, seed=3000 + 17 * k + B)
        scales = workloads.random_scales(n, T, seed=4000 + k)
        y = torch.full((B, 2 * n), float("nan"), dtype=torch.float32, device=dev)
        items.append((up(oracle.pack(codes), dev), up(scales, dev), x, y))
        host.append((codes, scales))
    assert sum((n + 15) // 16 for n in ns) >= 1536
    announce("grouped large batch", B, m, T)
    f2.fairy2i_gemv_grouped(items, algo=f2.GEMV_MFMA_BF16)
    torch.cuda.synchronize()
    check_items = range(len(ns)) if m <= 320 else (0, 11, 12, 13, 14)
    for k in check_items:
        codes, scales = host[k]
        want = oracle.gemv_ref(codes, scales, act.values)
        assert rel_l2(down(items[k][3]), want) <= TOL_F32, (k, ns[k])


@pytest.mark.parametrize("algo,B,n,m,T,batch,ydt", [
    ("f4", 1, 2048, 2048, 2, 13, "f32"),     # 1664 tiles: one wave per tile
    ("f4", 2, 37, 320, 3, 5, "bf16"),        # ragged n and m; a small launch (several waves per tile)
    ("i8", 1, 200, 512, 2, 9, "f32"),
    ("i8", 2, 2048, 2048, 1, 13, "f32"),
    ("bf16", 1, 2048, 2048, 2, 13, "f32"),
    ("bf16", 4, 2048, 320, 2, 13, "f32"),    # >= 1536 tiles at B >= 3: the shared-x kernel
    ("bf16", 9, 37, 320, 2, 7, "bf16"),
    ("valu", 2, 33, 128, 2, 3, "f32"),
])
def test_strided_batch_matches_grouped_and_oracle(algo, B, n, m, T, batch, ydt):
    """A strided batch (matrices back to back in one buffer; scales and outputs at strides, the
    output rows padded to 16 bytes) gives the grouped call's result on the same matrices bit for
    bit (same launch shape and order), and the first and last matrix are within tolerance of the
    oracle.  The first case also checks shared scales (stride 0)."""
    dev = device()
    act = workloads.activations(B, 2 * m, seed=90 + B + n)
    x = x_to_dev(act, dev)
    if algo in DIGITS:
        x = DIGITS[algo](x)
    pb = f2.fairy2i_packed_bytes(n, m, T)
    packed = torch.empty((batch, pb), dtype=torch.uint8, device=dev)
    scales = torch.empty((batch, n, T, 2, 2), dtype=torch.float32, device=dev)
    host = []
    for k in range(batch):
        codes = workloads.random_codes(T, n, m, seed=5000 + 31 * k + n)
        sc = workloads.random_scales(n, T, seed=6000 + k)
        packed[k] = up(oracle.pack(codes), dev)
        scales[k] = up(sc, dev)
        host.append((codes, sc))
    ydtype = torch.float32 if ydt == "f32" else torch.bfloat16
    elem = 4 if ydt == "f32" else 2
    ystride = -(-(B * 2 * n * elem) // 16) * 16 // elem
    ybuf = torch.full((batch, ystride), float("nan"), dtype=ydtype, device=dev)
    y = ybuf[:, :B * 2 * n].unflatten(1, (B, 2 * n))
    announce("strided gemv", algo, B, n, m, T, batch, ydt)
    f2.fairy2i_gemv_strided(packed, scales, x, y, algo=ALGOS[algo])
    ygbuf = torch.full_like(ybuf, float("nan"))
    yg = ygbuf[:, :B * 2 * n].unflatten(1, (B, 2 * n))
    f2.fairy2i_gemv_grouped([(packed[k], scales[k], x, yg[k]) for k in range(batch)], algo=ALGOS[algo])
    torch.cuda.synchronize()
    assert torch.equal(y, yg)
    for k in (0, batch - 1):
        codes, sc = host[k]
        want = oracle.gemv_ref(codes, sc, act.values)
        if ydt == "f32":
            assert rel_l2(down(y[k]), want) <= TOL_F32, k
        else:
            check_bf16(down(y[k]), want, (algo, k))
    if algo == "f4" and n == 2048:                      # scales shared by every matrix
        ys = torch.full_like(y, float("nan"))
        f2.fairy2i_gemv_strided(packed, scales[0], x, ys, algo=ALGOS[algo])
        torch.cuda.synchronize()
        want = oracle.gemv_ref(host[batch - 1][0], host[0][1], act.values)
        assert rel_l2(down(ys[batch - 1]), want) <= TOL_F32


@pytest.mark.parametrize("algo,B", [("f4", 1), ("i8", 1), ("bf16", 4)])
def test_strided_pool_full_size(algo, B):
    """The benchmark's own launch: the quantized 4096 x 4096 attention layer repeated 256 times back
    to back (1 GiB, 32768 tiles in one strided launch; at batch 1 the fp4 launch splits its last
    tiles over four waves each); every copy's output equals the oracle's for that layer within
    tolerance, and all copies are bit-identical."""
    dev = device()
    codes, s32 = attention_layer()
    P = 256
    act = workloads.activations(B, 4096, workloads.ATTN_X_SEEDS[B])
    want = oracle.gemv_ref(codes, s32, act.values)
    layer = up(oracle.pack(codes), dev)
    pool = layer.unsqueeze(0).repeat(P, 1).contiguous()
    spool = up(s32, dev).unsqueeze(0).repeat(P, 1, 1, 1, 1).contiguous()
    x = x_to_dev(act, dev)
    if algo in DIGITS:
        x = DIGITS[algo](x)
    y = torch.full((P, B, 4096), float("nan"), dtype=torch.float32, device=dev)
    announce("strided pool", algo, B, P)
    f2.fairy2i_gemv_strided(pool, spool, x, y, algo=ALGOS[algo])
    torch.cuda.synchronize()
    assert torch.equal(y, y[0:1].expand_as(y))
    assert rel_l2(down(y[P - 1]), want) <= TOL_F32
    del pool, spool, y
    torch.cuda.empty_cache()


@pytest.mark.gpu
@pytest.mark.parametrize("algo,n,m,T,ydt", [
    ("f4", 1000, 192, 2, "f32"),      # one chunk per tile: the split tiles' extra waves stream nothing
    ("f4", 1000, 192, 1, "bf16"),
    ("f4", 1000, 2112, 2, "f32"),     # nine chunks, the last one of a single 64-column group
    ("f4", 1000, 2112, 3, "bf16"),
    ("i8", 1000, 192, 2, "f32"),
    ("i8", 1000, 2112, 4, "f32"),
])
def test_large_digit_launch_matches_single_launches(algo, n, m, T, ydt):
    """Batch-1 fp4 and int8 launches of 12600 ragged tiles (200 matrices of 63 tiles).  The fp4
    launch takes its first tiles one wave each and the last 1536 split over four waves whose exact
    integer sums meet before the epilogue; the int8 launch takes one wave per tile throughout.
    Both halves of the batch launched on their own (6300 tiles: one wave per tile) give the same
    outputs bit for bit; every matrix is within 1e-6 relative L2 (fp32 outputs) of its
    single-matrix launch, whose waves split the chunks and add fp32 partial outputs in another
    order (bit for bit where that launch also has one wave per tile, a single chunk; bf16 outputs
    within their own tolerance); the first and last are within tolerance of the oracle."""
    dev = device()
    batch = 200
    act = workloads.activations(1, 2 * m, seed=4242 + m)
    x = DIGITS[algo](x_to_dev(act, dev))
    pb = f2.fairy2i_packed_bytes(n, m, T)
    packed = torch.empty((batch, pb), dtype=torch.uint8, device=dev)
    scales = torch.empty((batch, n, T, 2, 2), dtype=torch.float32, device=dev)
    host = {}
    for k in range(batch):
        codes = workloads.random_codes(T, n, m, seed=7000 + 13 * k + m)
        sc = workloads.random_scales(n, T, seed=8000 + k)
        packed[k] = up(oracle.pack(codes), dev)
        scales[k] = up(sc, dev)
        if k in (0, batch - 1):
            host[k] = (codes, sc)
    ydtype = torch.float32 if ydt == "f32" else torch.bfloat16
    y = torch.full((batch, 1, 2 * n), float("nan"), dtype=ydtype, device=dev)
    announce("large launch", algo, n, m, T, batch, ydt)
    f2.fairy2i_gemv_strided(packed, scales, x, y, algo=ALGOS[algo])
    yh = torch.full_like(y, float("nan"))
    h = batch // 2
    f2.fairy2i_gemv_strided(packed[:h], scales[:h], x, yh[:h], algo=ALGOS[algo])
    f2.fairy2i_gemv_strided(packed[h:], scales[h:], x, yh[h:], algo=ALGOS[algo])
    ys = torch.full_like(y, float("nan"))
    for k in range(batch):
        f2.fairy2i_gemv(packed[k], scales[k], x, y=ys[k], algo=ALGOS[algo])
    torch.cuda.synchronize()
    assert torch.equal(y, yh)
    if m <= 256:
        assert torch.equal(y, ys)
    else:
        tol = 1e-6 if ydt == "f32" else 2e-3
        for k in range(batch):
            assert rel_l2(down(y[k].float()), down(ys[k].float())) <= tol, k
    for k, (codes, sc) in host.items():
        want = oracle.gemv_ref(codes, sc, act.values)
        if ydt == "f32":
            assert rel_l2(down(y[k]), want) <= TOL_F32, k
        else:
            check_bf16(down(y[k]), want, ("large launch", k))


@pytest.mark.parametrize("algo,B", [("i8", 1), ("i8", 2), ("f4", 1), ("f4", 2)])
def test_digit_form_fp32_outlier_bound(algo, B):
    """fp32 x with one large outlier per batch column (1e4 and -3e4 among N(0, 1) values): the digit
    forms hold X_b = round_half_even(x_b 2^S_b) with max|x_b| 2^S_b in [2^21, 2^22), so each element
    moves by at most 2^-22 max|x_b|.  The GEMV must equal the oracle on that rounded x within the
    fp32 tolerance, and stay within the propagated bound 2^-22 max|x_b| sum_j |R^_ij| of the oracle
    on the exact x (R^ the layer's real form).  Here the rounding is visible: relative L2 against
    the exact x is of order 1e-5 (8e-6 for these outliers), which is why fp32 x with wide dynamic range is better served by the
    bf16 kernel or by bf16 x (every bf16 value within 2^14 of the column maximum is held exactly)."""
    dev = device()
    n, m, T = 256, 5504, 2
    codes = workloads.random_codes(T, n, m, seed=71)
    scales = workloads.random_scales(n, T, seed=72).astype(np.float32)
    rng = np.random.default_rng(73 + B)
    v = rng.standard_normal((B, 2 * m)).astype(np.float32)
    v[0, 1234] = 1.0e4
    if B == 2:
        v[1, 2 * m - 7] = -3.0e4
    rounded = np.empty_like(v, dtype=np.float64)
    delta = np.empty(B)
    for b in range(B):
        amax = float(np.abs(v[b]).max())
        S = 22 - np.frexp(amax)[1]                   # amax 2^S in [2^21, 2^22)
        rounded[b] = np.rint(v[b].astype(np.float64) * 2.0 ** S) * 2.0 ** -S
        delta[b] = 2.0 ** -22 * amax
    announce("gemv digit form fp32 outlier", algo, B)
    packed, s = up(oracle.pack(codes), dev), up(scales, dev)
    xd = DIGITS[algo](up(v, dev))
    got = down(f2.fairy2i_gemv(packed, s, xd, algo=ALGOS[algo]))
    assert rel_l2(got, oracle.gemv_ref(codes, scales, rounded)) <= TOL_F32
    exact = oracle.gemv_ref(codes, scales, v)
    row_abs = np.abs(oracle.dequantize_real(codes, scales)).sum(axis=1)       # [2n]
    for b in range(B):
        bound = delta[b] * row_abs + 1e-6 * np.abs(exact[b]).max()
        assert np.all(np.abs(got[b] - exact[b]) <= bound), b
    assert rel_l2(got, exact) <= 1e-4
