"""Oracle pins: 2-bit packing and the storage budget (2 bits per real parameter at T=2)."""
import oracle
import pins


def test_pack_golden_bytes():
    pins.check_pack_golden(oracle.pack_words)


def test_pack_tile_order():
    pins.check_pack_tile_order(oracle.pack, oracle.unpack)


def test_pack_roundtrip_and_size():
    pins.check_pack_roundtrip(oracle.pack, oracle.unpack, oracle.packed_nbytes)


def test_storage_bits_per_real_parameter():
    pins.check_storage_bits(oracle.pack)


def test_llama2_7b_stack_bytes():
    """The 224 linear layers of LLaMA-2 7B at T = 2: codes in bytes, plus fp32 scales."""
    import workloads
    codes = scales = 0
    for layer in range(workloads.STACK_LAYERS):
        for p in range(7):
            L = workloads.stack_layer(layer, p)
            codes += oracle.packed_nbytes(L.n, L.m, 2)
            scales += L.n * 2 * 2 * 2 * 4
    assert codes == 1_619_001_344
    assert scales == 21_757_952
