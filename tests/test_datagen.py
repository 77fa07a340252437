"""The seeded generator: deterministic, thread-count independent, consistent state."""
import numpy as np
import torch

import datagen


def test_normal_deterministic_and_chunk_independent():
    a = datagen.normal(1, 2, (3, datagen.CHUNK + 5))
    b = datagen.normal(1, 2, (3, datagen.CHUNK + 5))
    np.testing.assert_array_equal(a, b)
    c = datagen.normal(1, 3, (4,))
    assert not np.array_equal(a.ravel()[:4], c)
    # chunk k of a long draw equals the same chunk drawn alone
    first = datagen.normal(1, 2, (datagen.CHUNK,))
    np.testing.assert_array_equal(a.ravel()[:datagen.CHUNK], first)


def test_bf16_storage_rounding():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    t = datagen.to_storage(x, "bf16")
    assert t.dtype == torch.bfloat16
    assert t.float().tolist() == [1.0, 1.0 + 2.0 ** -6]


def test_lognormal_norms():
    r = datagen.lognormal_rows(3, 7, (2000, 64), 0.5)
    ln = np.log(np.linalg.norm(r, axis=1))
    assert abs(ln.mean()) < 0.05 and abs(ln.std() - 0.5) < 0.05


def test_decode_state_is_consistent():
    spec = datagen.CaseSpec(11, "decode", B=4, L=1000, m=4, H_I=8, d_I=16, H=4, D=32, K=8, W=8,
                            w_cap=16, ragged=True)
    c = datagen.make_case(spec)
    for b in range(4):
        t = int(c["pos"][b])
        slot = t % 4
        for j in range(slot):          # tail rows are the ring's raw rows
            p = t - slot + j
            assert torch.equal(c["x_tail"][b, j], c["rings"][0][b, p % 16])
        assert torch.all(c["x_tail"][b, slot] == 0)
        assert torch.all(c["rings"][0][b, t % 16] == 0)
    assert c["kv"].shape == (4, 250, 32) and c["k_idx"].shape == (4, 250, 16)
    assert c["w"].dtype == torch.float32


def test_config_table():
    assert datagen.CONFIGS[4].entries == 262144 and datagen.CONFIGS[4].B == 4
    assert datagen.CONFIGS[5].entries == 262144 and datagen.CONFIGS[5].n_attn == 3
    assert datagen.CONFIGS[3].chunk == 4096 and datagen.CONFIGS[3].entries == 32768
    assert datagen.CONFIGS[2].entries == 16384 and datagen.CONFIGS[2].B == 8
    assert datagen.CONFIGS[1].dtype == "f32" and datagen.CONFIGS[1].entries == 512


def test_prefill_indexer_inputs_equal_the_full_prefill_case():
    spec = datagen.CaseSpec(931, "prefill", B=1, L=4096, m=4, w_cap=512, chunk=256, H_I=8,
                            d_I=32, H=2, D=64)
    full = datagen.make_prefill(spec)
    part = datagen.make_prefill_indexer(spec)
    for k in ("k_idx", "xi_chunk", "zi_chunk", "bias_i", "q_pos", "e_count", "q_idx", "w"):
        assert torch.equal(part[k], full[k]), k
