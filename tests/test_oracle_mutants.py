"""Each pin must catch a plausible mistake planted in a copy of the oracle (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle.phase_quant as pq
import pins


def fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_split_sign_error_caught():
    def bad(R):
        U, W = oracle.split(R)
        return np.conj(U), W                 # Im U = (R12 - R21)/2
    fails(pins.check_split_identity, bad)
    fails(pins.check_split_hand, bad)


def test_split_swapped_blocks_caught():
    def bad(R):
        n, m = R.shape[0] // 2, R.shape[1] // 2
        R2 = np.array(R, copy=True)
        R2[:n, m:], R2[n:, :m] = R[n:, :m], R[:n, m:]     # R12 <-> R21
        return oracle.split(R2)
    fails(pins.check_split_identity, bad)


def test_split_conj_on_wrong_matrix_caught():
    def bad(R):
        U, W = oracle.split(R)
        return U, np.conj(W)
    fails(pins.check_split_identity, bad)


def test_projection_last_tie_caught():
    def bad(a, b):
        s = np.stack([a, b, -a, -b], axis=0)[::-1]
        return (3 - np.argmax(s, axis=0)).astype(np.uint8)     # last maximum wins
    fails(pins.check_project_bruteforce, bad)
    fails(pins.check_project_golden, bad)


def test_projection_sign_error_caught():
    def bad(a, b):
        return np.argmax(np.stack([a, -b, -a, b], axis=0), axis=0).astype(np.uint8)  # i <-> -i
    fails(pins.check_project_bruteforce, bad)
    fails(pins.check_project_angle, bad)


def test_sequential_sum_order_caught():
    def bad(v):
        out = np.zeros(v.shape[0])
        for j in range(v.shape[1]):
            out = out + v[:, j]
        return out
    fails(pins.check_ordered_sum_golden, bad)


def test_scale_mean_over_all_entries_caught(monkeypatch):
    real_stage = pq._stage

    def bad_stage(r_re, r_im, per_tensor=False):
        k, s_re, s_im, _, _ = real_stage(r_re, r_im)
        m = r_re.shape[1]
        on_re = (k == 0) | (k == 2)
        s_re = pq.ordered_row_sum(np.where(on_re, np.abs(r_re), 0.0)) / m
        s_im = pq.ordered_row_sum(np.where(~on_re, np.abs(r_im), 0.0)) / m
        new_re = np.where(k == 0, r_re - s_re[:, None], np.where(k == 2, r_re + s_re[:, None], r_re))
        new_im = np.where(k == 1, r_im - s_im[:, None], np.where(k == 3, r_im + s_im[:, None], r_im))
        return k, s_re, s_im, new_re, new_im

    monkeypatch.setattr(pq, "_stage", bad_stage)
    fails(pins.check_ls_identity, oracle.quantize, oracle.split, oracle.dequantize)
    fails(pins.check_quantize_hand, oracle.quantize, oracle.unsplit)


def test_residual_sign_error_caught(monkeypatch):
    real_stage = pq._stage

    def bad_stage(r_re, r_im, per_tensor=False):
        k, s_re, s_im, _, _ = real_stage(r_re, r_im)
        new_re = np.where(k == 0, r_re + s_re[:, None], np.where(k == 2, r_re - s_re[:, None], r_re))
        new_im = np.where(k == 1, r_im - s_im[:, None], np.where(k == 3, r_im + s_im[:, None], r_im))
        return k, s_re, s_im, new_re, new_im

    monkeypatch.setattr(pq, "_stage", bad_stage)
    fails(pins.check_norm_nonincreasing, oracle.quantize)
    fails(pins.check_quantize_hand, oracle.quantize, oracle.unsplit)


def test_scale_wrong_component_caught(monkeypatch):
    real_stage = pq._stage

    def bad_stage(r_re, r_im, per_tensor=False):
        k, s_re, s_im, _, _ = real_stage(r_re, r_im)
        on_re = (k == 0) | (k == 2)
        n_re = np.maximum(on_re.sum(axis=1), 1)
        s_re = pq.ordered_row_sum(np.where(on_re, np.abs(r_im), 0.0)) / n_re   # |Im| on the real axis
        new_re = np.where(k == 0, r_re - s_re[:, None], np.where(k == 2, r_re + s_re[:, None], r_re))
        new_im = np.where(k == 1, r_im - s_im[:, None], np.where(k == 3, r_im + s_im[:, None], r_im))
        return k, s_re, s_im, new_re, new_im

    monkeypatch.setattr(pq, "_stage", bad_stage)
    fails(pins.check_ls_identity, oracle.quantize, oracle.split, oracle.dequantize)


def test_pack_consecutive_codes_per_byte_caught():
    def bad_words(codes):
        T, _, n, m = codes.shape
        c = codes.astype(np.uint32).reshape(T, 2, n, m // 16, 4, 4)    # [word][byte][pair]: 4 in a row
        byte = c[..., 0] | c[..., 1] << 2 | c[..., 2] << 4 | c[..., 3] << 6
        return byte[..., 0] | byte[..., 1] << 8 | byte[..., 2] << 16 | byte[..., 3] << 24
    fails(pins.check_pack_golden, bad_words)


def test_pack_msb_first_caught():
    def bad_words(codes):
        w = oracle.pack_words(codes)
        b = np.stack([(w >> (8 * k)) & 255 for k in range(4)], axis=-1)
        rev = ((b & 3) << 6) | ((b & 12) << 2) | ((b & 48) >> 2) | ((b & 192) >> 6)
        return rev[..., 0] | rev[..., 1] << 8 | rev[..., 2] << 16 | rev[..., 3] << 24
    fails(pins.check_pack_golden, bad_words)


def test_pack_row_major_order_caught():
    """The plain row-major order [row][plane][words] is caught by the word-order fixture."""
    def bad_pack(codes):
        T, _, n, m = codes.shape
        w = oracle.pack_words(codes)                                    # [T][2][n][m/16]
        w = np.concatenate([w, np.zeros((T, 2, (-n) % 16, m // 16), dtype=w.dtype)], axis=2)
        return np.ascontiguousarray(w.transpose(2, 0, 1, 3)).astype("<u4").view(np.uint8).reshape(-1)
    fails(pins.check_pack_tile_order, bad_pack, oracle.unpack)


def test_pack_groups_before_planes_caught():
    """Swapping the plane and group levels inside a chunk is caught."""
    def bad_pack(codes):
        T, _, n, m = codes.shape
        w = oracle.pack_words(codes)
        nt = -(-n // 16)
        w = np.concatenate([w, np.zeros((T, 2, 16 * nt - n, m // 16), dtype=w.dtype)], axis=2)
        out = []
        for tile in range(nt):
            for c in range(-(-m // 256)):
                G = min(256, m - 256 * c) // 64
                for g in range(G):
                    for P in range(2 * T):
                        w0 = (256 * c + 64 * g) // 16
                        out.append(w[P // 2, P % 2, 16 * tile:16 * tile + 16, w0:w0 + 4].reshape(-1))
        return np.concatenate(out).astype("<u4").view(np.uint8)
    fails(pins.check_pack_tile_order, bad_pack, oracle.unpack)


def test_gemv_conj_on_u_caught():
    def bad(codes, scales, x, stages=None):
        m = codes.shape[3]
        x = np.asarray(x, dtype=np.float64).copy()
        x[:, m:] = -x[:, m:]                 # conj(x) fed to both U and W
        y = oracle.gemv_ref(codes, scales, x, stages)
        return y
    fails(pins.check_gemv_hand, bad)
    fails(pins.check_gemv_routes, bad, oracle.gemv_ref_real)


def test_gemv_dropped_stage_caught():
    def bad(codes, scales, x, stages=None):
        return oracle.gemv_ref(codes[:1], scales[:, :1], x, None if stages is None else [0])
    fails(pins.check_gemv_hand, bad)


def test_act_quant_half_away_caught():
    def bad(x):
        q, d = oracle.act_quant_ref(x)
        x = np.asarray(x, dtype=np.float64)
        for t in range(x.shape[0]):
            if d[t] != 0:
                r = (x[t] / float(d[t])).astype(np.float32).astype(np.float64)
                q[t] = np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -127, 127).astype(np.int8)
        return q, d
    fails(pins.check_act_quant_golden, bad)


def test_gemm_epilogue_sign_error_caught():
    def bad(P, scales, delta):
        P = np.array(P, copy=True)
        P[:, 1, 1, 1] = -P[:, 1, 1, 1]       # W imaginary-axis b term with the wrong sign
        return oracle.gemm_epilogue_ref(P, scales, delta)
    fails(pins.check_gemm_epilogue, oracle.gemm_int_ref, bad, oracle.gemv_ref)


def test_gemm_transposed_plane_caught():
    def bad(codes, q):
        P = oracle.gemm_int_ref(codes, q)
        return P[:, :, ::-1]                   # B_re and B_im swapped
    fails(pins.check_gemm_routes, bad, oracle.gemm_int_ref_loops)


def test_dequantize_real_swapped_blocks_caught():
    """R12 and R21 exchanged (the transpose-like slip) fails the route and hand checks."""
    def bad(codes, scales):
        R = oracle.dequantize_real(codes, scales)
        n, m = R.shape[0] // 2, R.shape[1] // 2
        out = R.copy()
        out[:n, m:], out[n:, :m] = R[n:, :m], R[:n, m:]
        return out
    fails(pins.check_dequantize_real, bad, oracle.gemv_ref)


def test_per_tensor_mean_of_row_means_caught():
    """Averaging the per-row means (instead of the tensor-wide mean) fails the pins."""
    def bad(R, T, per_tensor=False):
        codes, s32, s64, norms = oracle.quantize(R, T)
        if per_tensor:
            s64 = np.broadcast_to(s64.mean(axis=0, keepdims=True), s64.shape).copy()
            s32 = s64.astype(np.float32)
        return codes, s32, s64, norms
    fails(pins.check_per_tensor_scales, bad, oracle.split)


def test_per_tensor_plain_row_sum_caught(monkeypatch):
    """Combining the row sums with np.sum (numpy's own order) instead of the pinned order fails
    the hand-worked order cases."""
    def bad_mean(row_sums, row_counts):
        count = int(np.sum(row_counts))
        return float(np.sum(np.asarray(row_sums, dtype=np.float64))) / count if count > 0 else 0.0
    monkeypatch.setattr(pq, "_tensor_mean", bad_mean)
    fails(pins.check_per_tensor_order, oracle.quantize)


def test_per_tensor_sequential_row_sum_caught(monkeypatch):
    """Rows added left to right fail the hand-worked order cases as well."""
    def bad_mean(row_sums, row_counts):
        total = 0.0
        for v in np.asarray(row_sums, dtype=np.float64):
            total = total + float(v)
        count = int(np.sum(row_counts))
        return total / count if count > 0 else 0.0
    monkeypatch.setattr(pq, "_tensor_mean", bad_mean)
    fails(pins.check_per_tensor_order, oracle.quantize)

