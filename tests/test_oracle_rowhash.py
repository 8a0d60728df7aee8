"""Pins of the P~ row checksum (a verification aid, not part of the method):
the splitmix64 reference outputs, odd weights, order independence, and that
any single changed code changes the sum."""
import numpy as np
import pytest

import oracle

# splitmix64 from seed 0, first three outputs (the generator's published
# reference values)
SPLITMIX64_SEED0 = (0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F)


def test_splitmix64_reference_outputs():
    assert tuple(oracle.splitmix64(0, 3)) == SPLITMIX64_SEED0


def test_weights_odd_and_distinct():
    w = oracle.key_weights(4096)
    assert (w & np.uint64(1)).all()
    assert len(np.unique(w)) == w.size
    assert int(w[0]) == SPLITMIX64_SEED0[0] | 1 and int(w[1]) == SPLITMIX64_SEED0[1] | 1


def test_unit_rows_give_the_weights():
    n = 300
    p = np.eye(n, dtype=np.uint8)
    assert np.array_equal(oracle.row_hash(p), oracle.key_weights(n))


def test_linear_and_independent_of_visit_order():
    rng = np.random.default_rng(3)
    a = rng.integers(0, 128, (5, 700), dtype=np.uint8)
    b = rng.integers(0, 127, (5, 700), dtype=np.uint8)
    with np.errstate(over="ignore"):
        assert np.array_equal(oracle.row_hash(a + b), oracle.row_hash(a) + oracle.row_hash(b))
    # summing block by block in any order gives the same value
    w = oracle.key_weights(700)
    parts = [(a[:, j0:j0 + 128].astype(np.uint64) * w[j0:j0 + 128]).sum(-1, dtype=np.uint64)
             for j0 in range(0, 700, 128)]
    acc = np.zeros(5, np.uint64)
    with np.errstate(over="ignore"):
        for part in reversed(parts):
            acc += part
    assert np.array_equal(acc, oracle.row_hash(a))


def test_every_single_code_change_detected():
    rng = np.random.default_rng(4)
    row = rng.integers(0, 127, 512, dtype=np.uint8)
    h0 = oracle.row_hash(row)
    for j in range(0, 512, 7):
        for new in (0x00, 0x01, 0x38, 0x7E, 0x80, 0xFE):
            if new == row[j]:
                continue
            r = row.copy()
            r[j] = new
            assert oracle.row_hash(r) != h0


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("causal", [True, False])
def test_checksum_only_path_matches_the_dump(orc, order, causal):
    """attention_fp8_rowhash (no output accumulation, checksum and zero count
    in C) gives the checksums of the full loop's P~ dump and its counts."""
    import synth
    w = synth.qwen_like(1, 4, 2, 64, seed=5, N=333, texts=1)
    op = orc.prepare(w.q, w.k, w.v, signs=w.signs, rotate=True, center=True)
    for bn in (64, 128):
        full = orc.attention_fp8(op, p_scale=256.0, kv_order=order, block_n=bn, causal=causal, want_p=True, k_sink=4)
        h, z = orc.attention_fp8_rowhash(op, p_scale=256.0, kv_order=order, block_n=bn, causal=causal, k_sink=4)
        assert np.array_equal(h, orc.row_hash(full.p))
        assert np.array_equal(z, full.row_zeros)
        rows = np.array([0, 5, 332, 128], np.int32)
        hs, zs = orc.attention_fp8_rowhash(op, p_scale=256.0, kv_order=order, block_n=bn, causal=causal, rows=rows,
                                           k_sink=4)
        assert np.array_equal(hs, h[:, :, rows]) and np.array_equal(zs, z[:, :, rows])
