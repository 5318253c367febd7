"""The seeded workloads: determinism and the shapes the five cases promise."""
import numpy as np

import synth


def test_generators_are_deterministic_and_blockwise():
    w = synth.case2()
    k1, v1 = w.kv_rows(0, 3, 1000, 3100)
    k2, v2 = w.kv_rows(0, 3, 1000, 3100)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    # any sub-range regenerates the same rows
    k3, v3 = w.kv_rows(0, 3, 2047, 2049)
    assert np.array_equal(k3, k1[1047:1049]) and np.array_equal(v3, v1[1047:1049])
    # different sequences and slots draw different rows
    k4, _ = w.kv_rows(0, 4, 1000, 3100)
    assert not np.array_equal(k1, k4)


def test_case_shapes():
    c0 = synth.case0()
    assert c0.context_lens.tolist() == [100, 37] and c0.head_dim == 64
    assert c0.num_q_heads == 8 and c0.q_dtype == "f32" and c0.attended_keys() == 137
    c1 = synth.case1()
    assert c1.batch == 64 and c1.layer_window.tolist() == [1024]
    assert c1.attended_keys() == 64 * 1024
    assert c1.block_table[0, 5, :3].tolist() == [5 * 256, 5 * 256 + 1, 5 * 256 + 2]
    c2 = synth.case2()
    assert c2.context_lens.min() >= 8192 and c2.context_lens.max() <= 32768
    assert c2.outlier_channels.size == 6 and c2.num_pages == 40001
    c3 = synth.case3()
    assert c3.num_layers == 3 and set(c3.layer_slot.tolist()) == {0}
    assert c3.attended_keys() == 32 * 16384
    c4 = synth.case4()
    assert c4.num_layers == 12 and c4.num_slots == 11
    assert c4.layer_slot.tolist() == [0, 1, 2, 3, 4, 10, 5, 6, 7, 8, 9, 10]
    assert c4.layer_window.tolist() == [1024] * 5 + [0] + [1024] * 5 + [0]
    prefix = c4.context_lens - 64
    assert prefix.min() >= 512 and prefix.max() <= 32768
    assert 4500 < np.median(prefix) < 7500


def test_page_tables_are_injective_and_poison_elsewhere():
    for w in (synth.case2(), synth.case3(), synth.case4(batch=32)):
        used = []
        for s in range(w.num_slots):
            for b in range(w.batch):
                first, ctx = w.stored_range(s, b)
                p0, p1 = first // 16, synth.pages_for(ctx)
                row = w.block_table[s, b]
                used.append(row[p0:p1])
                assert np.all(row[:p0] == w.poison_page)
                assert np.all(row[p1:] == w.poison_page)
        used = np.concatenate(used)
        assert used.size == np.unique(used).size
        assert used.max() < w.poison_page < w.num_pages


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, 1.0078125 + 2 ** -20, -3.0],
                 dtype=np.float32)
    # 1 + 2^-8 is a tie -> 1.0 (even); 1 + 3*2^-8 is a tie -> 1 + 2^-6 (even)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    assert got.tolist() == [1.0, 1.0, 1.015625, 1.0078125, -3.0]
    q = synth.case1().q_f32()
    assert np.array_equal(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(q)), q)
