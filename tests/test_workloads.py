"""Host-side checks of the seeded input generator (no attention arithmetic involved)."""
import numpy as np

from mla_decode_context_amd import workloads as WL


def test_tiny_dcp_layout():
    wl = WL.make_workload("tiny_dcp")
    assert list(wl.seq_lens) == [6, 37, 128, 255]
    assert list(wl.query_start_loc) == [0, 4, 8, 12, 16]
    assert wl.q_nope.shape == (16, 16, 512) and wl.q_pe.shape == (16, 16, 64)
    assert abs(wl.scale - 192 ** -0.5) < 1e-15
    for r, sh in enumerate(wl.shards):
        used = set()
        for b in range(wl.B):
            g = wl.global_kv(b)
            n = int(sh.token_counts[b])
            assert n == len(range(r, int(wl.seq_lens[b]), wl.W))
            nb = -(-n // wl.P)
            assert np.all(sh.block_table[b, nb:] == -1)
            for j in range(n):
                blk = sh.block_table[b, j // wl.P]
                assert np.array_equal(sh.cache[blk, j % wl.P], g[j * wl.W + r])
            if n % wl.P:
                assert np.all(sh.cache[sh.block_table[b, nb - 1], n % wl.P:] == WL.BF16_NAN)
            used.update(int(x) for x in sh.block_table[b, :nb])
        spare = [i for i in range(sh.cache.shape[0]) if i not in used]
        assert spare, "pool must hold spare blocks"
        assert np.all(sh.cache[spare] == WL.BF16_NAN)
        # physical ids follow a random permutation, not the logical order
        logical = [int(x) for x in sh.block_table.ravel() if x >= 0]
        assert logical != sorted(logical)


def test_deterministic_across_threads():
    a = WL.make_workload("tiny_dcp", threads=1)
    b = WL.make_workload("tiny_dcp", threads=8)
    assert np.array_equal(a.q_nope, b.q_nope) and np.array_equal(a.q_pe, b.q_pe)
    for sa, sb in zip(a.shards, b.shards):
        assert np.array_equal(sa.cache, sb.cache)
        assert np.array_equal(sa.block_table, sb.block_table)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    bits = WL.f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6... i.e. 1.015625)
    assert list(back) == [1.0, 1.0, 1.015625, -2.5, 1.0]


def test_mixed_lengths():
    S, Q = WL._draw_lengths(WL.CONFIGS["mixed_wuv"], 4)
    assert len(S) == 98 and set(Q[:96]) <= {1, 2, 4} and list(Q[96:]) == [512, 512]
    assert S.min() >= 512 and S.max() <= 16384
    S4, Q4 = WL._draw_lengths(WL.CONFIGS["long_dcp8"], 3)
    assert [S4[0], S4[64], S4[128], S4[192]] == [2, 3, 5, 7] and np.all(Q4 == 2)


def test_run_layout_places_runs_of_tokens():
    # Runs of I tokens dealt to the shards in turn: shard r's local token j is the
    # global token at position ((j div I) * W + r) * I + j mod I (written out
    # here on its own; the GPU parity tests hold the kernels to the same layout).
    for I, P in ((5, 16), (16, 16), (1, 7)):
        wl = WL.make_custom("runs", [6, 37, 128, 255], [4, 4, 4, 4], H=16, W=3, P=P, seed=0, I=I)
        assert wl.I == I
        for r, sh in enumerate(wl.shards):
            for b in range(wl.B):
                g = wl.global_kv(b)
                S = int(wl.seq_lens[b])
                n = int(sh.token_counts[b])
                pos = [((j // I) * wl.W + r) * I + j % I for j in range(n)]
                assert all(p < S for p in pos) and (n == 0 or ((n // I) * wl.W + r) * I + n % I >= S)
                for j, p in enumerate(pos):
                    assert np.array_equal(sh.cache[sh.block_table[b, j // P], j % P], g[p])
        assert sum(int(sh.token_counts[b]) for sh in wl.shards for b in range(wl.B)) == int(wl.seq_lens.sum())
