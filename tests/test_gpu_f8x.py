"""GPU parity of the batch 3-16 decode GEMV on the scaled matrix cores (fairy2i_gemv with bf16 x,
MFMA_F4 and B > 2): fp4 code planes times x split into two fp8 e4m3 parts under one E8M0 scale per
32-column block.  Against the oracle at the fp32 tolerance, on single, grouped (items with
different x) and strided calls; ragged rows and tiles (workgroups of 4 or 8 tiles partly empty);
T = 1..4; B = 3..16 (one, two and four column groups); bf16 outputs; chunks at 2^+-100, all-zero
chunks and batch columns; and, where x has entries far below their chunk's maximum, the stated
bound of the split (each entry off by at most 2^-17 of the maximum of the 32 values that share its
block scale, so at most 2^-17 of its 256-column chunk's maximum)."""
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


def bf16_act(v):
    bits = workloads.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))
    return workloads.Activations(values=workloads.bf16_bits_to_f32(bits), dtype="bf16", bf16_bits=bits)


@pytest.mark.parametrize("n,m,T,B", [(40, 2048, 2, 4), (17, 320, 1, 3), (130, 1088, 3, 5), (256, 4096, 2, 8),
                                     (33, 5504, 2, 9), (300, 2048, 2, 16), (21, 64, 4, 12), (129, 8192, 2, 6),
                                     (64, 2048, 4, 16), (100, 1024, 3, 16), (7, 512, 1, 16)])
def test_f8x_matches_oracle(n, m, T, B):
    dev = device()
    codes, scales = layer(n, m, T, seed=3000 + n + m + T)
    act = workloads.activations(B, 2 * m, seed=3100 + B + m)
    packed, s = up(oracle.pack(codes), dev), up(scales, dev)
    x = x_to_dev(act, dev)
    want = oracle.gemv_ref(codes, scales, act.values)
    announce("gemv fp4 x fp8", n, m, T, B)
    got = down(f2.fairy2i_gemv(packed, s, x, algo=f2.GEMV_MFMA_F4))
    assert got.shape == (B, 2 * n)
    assert rel_l2(got, want) <= TOL_F32, rel_l2(got, want)
    check_bf16(down(f2.fairy2i_gemv(packed, s, x, algo=f2.GEMV_MFMA_F4, y_dtype=torch.bfloat16)), want, "f8x")


def test_f8x_grouped_distinct_x_and_strided():
    """A grouped call whose items read different x (each workgroup takes its item's x), and a
    strided batch of distinct layers sharing one x, against the oracle item by item."""
    dev = device()
    m, T, B = 2048, 2, 8
    items, refs = [], []
    for k, n in enumerate((16, 200, 33)):
        codes, scales = layer(n, m, T, seed=3200 + k)
        act = workloads.activations(B, 2 * m, seed=3300 + k)
        items.append((up(oracle.pack(codes), dev), up(scales, dev), x_to_dev(act, dev),
                      torch.empty((B, 2 * n), device=dev)))
        refs.append(oracle.gemv_ref(codes, scales, act.values))
    announce("gemv fp4 x fp8 grouped")
    ys = f2.fairy2i_gemv_grouped(items, algo=f2.GEMV_MFMA_F4)
    for y, want in zip(ys, refs):
        assert rel_l2(down(y), want) <= TOL_F32
    batch, n = 24, 250
    g = torch.Generator(device=dev)
    g.manual_seed(33)
    nb = f2.fairy2i_packed_bytes(n, m, T)
    pool = torch.randint(0, 256, (batch, nb), dtype=torch.uint8, device=dev, generator=g)
    spool = (torch.rand((batch, n, T, 2, 2), device=dev, generator=g) * 0.02).contiguous()
    act = workloads.activations(B, 2 * m, seed=3400)
    yb = torch.empty((batch, B, 2 * n), device=dev)
    f2.fairy2i_gemv_strided(pool, spool, x_to_dev(act, dev), yb, algo=f2.GEMV_MFMA_F4)
    a = down(yb)
    for k in (0, 11, batch - 1):
        codes = oracle.unpack(down(pool[k]), n, m, T)
        assert rel_l2(a[k], oracle.gemv_ref(codes, down(spool[k]), act.values)) <= TOL_F32, k


@pytest.mark.parametrize("B", [4, 16])
def test_f8x_block_scales(B):
    """Chunks of 256 columns (every block scale covers values of one chunk) at very different
    scales (2^-100, 2^100, zero) and an all-zero batch column, every entry within 2^9 of its chunk's
    maximum (so the split is exact): each case alone (only that chunk nonzero, so the output has
    its scale) and all together, against the oracle."""
    dev = device()
    n, m, T = 48, 1024, 2
    codes, scales = layer(n, m, T, seed=3500 + B)
    packed, s = up(oracle.pack(codes), dev), up(scales, dev)
    rng = np.random.default_rng(3600 + B)
    mag = 2.0 ** rng.uniform(-9, 0, size=(B, 2 * m))             # within 2^9 of a chunk maximum of 1
    base = (np.where(rng.random((B, 2 * m)) < 0.5, -1.0, 1.0) * mag).astype(np.float32)
    blk = (np.arange(2 * m) % m) // 256                          # chunk index of every real column
    scale = np.ones(2 * m, dtype=np.float32)
    scale[blk == 1] = 2.0 ** -100
    scale[blk == 2] = 2.0 ** 100
    scale[blk == 3] = 0.0
    cases = {"all": base * scale}
    cases["all"][1] = 0.0                                          # an all-zero batch column
    for label, sel in (("tiny", 1), ("huge", 2)):
        v = np.zeros_like(base)
        v[:, blk == sel] = (base * scale)[:, blk == sel]
        cases[label] = v
    for label, v in cases.items():
        act = bf16_act(v)
        announce("gemv fp4 x fp8 block scales", B, label)
        got = down(f2.fairy2i_gemv(packed, s, x_to_dev(act, dev), algo=f2.GEMV_MFMA_F4))
        want = oracle.gemv_ref(codes, scales, act.values)
        assert np.all(np.isfinite(got)), label
        nz = np.linalg.norm(want, axis=1) > 0
        assert np.all(got[~nz] == 0.0), label
        assert rel_l2(got[nz], want[nz]) <= TOL_F32, (label, rel_l2(got[nz], want[nz]))


def test_f8x_split_bound():
    """Entries far below their chunk's maximum (2^-12 .. 2^-24 of it), where the low fp8 part
    rounds: each output within the bound the split states (every x entry off by at most 2^-17 of
    its chunk's max |x|, times the sum of the row's |scales| over the codes that read it), plus the
    fp32 tolerance."""
    dev = device()
    n, m, T, B = 64, 2048, 2, 4
    codes, scales = layer(n, m, T, seed=3700)
    packed, s = up(oracle.pack(codes), dev), up(scales, dev)
    rng = np.random.default_rng(3800)
    v = (rng.standard_normal((B, 2 * m)) * 2.0 ** rng.uniform(-24, -12, size=(B, 2 * m))).astype(np.float32)
    v[:, np.arange(2 * m) % 32 == 5] = 1.0                        # a maximum in every 32 columns
    act = bf16_act(v)
    got = down(f2.fairy2i_gemv(packed, s, x_to_dev(act, dev), algo=f2.GEMV_MFMA_F4)).astype(np.float64)
    want = oracle.gemv_ref(codes, scales, act.values)
    cmax = np.abs(act.values).reshape(B, -1, 256).max(axis=2)     # [B][chunks of each component]
    err_x = np.repeat(cmax * 2.0 ** -17, 256, axis=1)             # per entry bound, [B][2m]
    # |y_i error| <= sum over stages, matrices and both components of |scale| * |x error|: every
    # code reads x_j (Re, Im) with weights of magnitude at most s_re + s_im of its row and stage
    wsum = np.abs(scales).sum(axis=(1, 2, 3))                     # [n]
    e_col = err_x[:, :m] + err_x[:, m:]                           # [B][m], both components
    bound = wsum[None, :] * e_col.sum(axis=1)[:, None]            # [B][n], loose
    bound = np.concatenate([bound, bound], axis=1) + 1e-5 * np.abs(want).max()
    announce("gemv fp4 x fp8 split bound")
    assert np.all(np.abs(got - want) <= bound)
    assert rel_l2(got, want) <= 1e-3


@pytest.mark.parametrize("B,batch,fp8", [(4, 100, True), (3, 97, True), (4, 20, False), (8, 100, False)])
def test_auto_batch_3_to_4(B, batch, fp8):
    """AUTO on bf16 x at batch 3-4 takes this kernel for launches of at least 1536 tiles (here a
    strided batch of 16-tile layers) and the bf16 kernel below that and at batch 5 and up: bit for
    bit the output of the kernel that should run, and the oracle on sampled layers."""
    dev = device()
    n, m, T = 256, 2048, 2
    g = torch.Generator(device=dev)
    g.manual_seed(4000 + B + batch)
    nb = f2.fairy2i_packed_bytes(n, m, T)
    pool = torch.randint(0, 256, (batch, nb), dtype=torch.uint8, device=dev, generator=g)
    spool = (torch.rand((batch, n, T, 2, 2), device=dev, generator=g) * 0.02).contiguous()
    act = workloads.activations(B, 2 * m, seed=4100 + B)
    x = x_to_dev(act, dev)
    y_auto, y_want = (torch.empty((batch, B, 2 * n), device=dev) for _ in range(2))
    announce("gemv auto batch 3-4", B, batch, fp8)
    f2.fairy2i_gemv_strided(pool, spool, x, y_auto)
    f2.fairy2i_gemv_strided(pool, spool, x, y_want, algo=f2.GEMV_MFMA_F4 if fp8 else f2.GEMV_MFMA_BF16)
    assert torch.equal(y_auto.view(torch.int32), y_want.view(torch.int32))
    a = down(y_auto)
    for k in (0, batch - 1):
        codes = oracle.unpack(down(pool[k]), n, m, T)
        assert rel_l2(a[k], oracle.gemv_ref(codes, down(spool[k]), act.values)) <= TOL_F32, k
