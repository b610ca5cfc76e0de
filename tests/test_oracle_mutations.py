"""Plants plausible mistakes in the oracle (CPU only) and checks that the pins
catch each one: a pin that cannot fail proves nothing."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import kv_bytes as KB

from . import test_oracle_attention as T
from . import test_oracle_kv_bytes as TB


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _sdpa_cases():
    return [(4, 2, 64, 4, [38, 101]), (2, 2, 16, 8, [1, 16, 17]), (8, 1, 32, 8, [33, 5])]


def test_interleaved_head_map_is_caught(monkeypatch):
    def decode_interleaved(q, k_pages, v_pages, block_table, seq_lens, n_q_heads, n_kv_heads, block_size, scale):
        q = np.asarray(q, dtype=np.float64)
        out = np.zeros(q.shape)
        for b in range(q.shape[0]):
            K, V = A.gather(k_pages, v_pages, block_table[b], int(seq_lens[b]), block_size)
            for hq in range(n_q_heads):
                h = hq % n_kv_heads                     # planted: interleaved groups
                out[b, hq] = A.attend(q[b, hq], K[:, h], V[:, h], scale)
        return out
    monkeypatch.setattr(A, "decode", decode_interleaved)
    assert _fails(T.test_gqa_equals_mha_with_repeated_kv_heads)
    assert any(_fails(T.test_matches_torch_sdpa_float64, *c) for c in _sdpa_cases())


def test_missing_scale_is_caught(monkeypatch):
    orig = A.attend
    monkeypatch.setattr(A, "attend", lambda q, K, V, scale: orig(q, K, V, 1.0))
    assert any(_fails(T.test_matches_torch_sdpa_float64, *c) for c in _sdpa_cases())
    assert _fails(T.test_brute_force_python_loops)


def test_dropped_last_token_is_caught(monkeypatch):
    orig = A.gather
    monkeypatch.setattr(A, "gather", lambda k, v, row, n, bs: orig(k, v, row, max(n - 1, 0), bs))
    assert any(_fails(T.test_matches_torch_sdpa_float64, *c) for c in _sdpa_cases())
    assert _fails(T.test_single_token_returns_its_value)


def test_untransposed_value_tile_is_caught(monkeypatch):
    def gather_bad_v(k_pages, v_pages, block_table_row, n_tokens, block_size):
        K, _ = A_gather(k_pages, v_pages, block_table_row, n_tokens, block_size)
        n_blocks = (n_tokens + block_size - 1) // block_size
        pages = np.asarray(block_table_row[:n_blocks], dtype=np.int64)
        vp = np.asarray(v_pages[pages])              # [blk][Hkv][D][bs] read as if [blk][bs][Hkv][D]
        V = vp.reshape(n_blocks * block_size, k_pages.shape[1], -1)[:n_tokens]
        return K, np.asarray(V, dtype=np.float64)
    A_gather = A.gather
    monkeypatch.setattr(A, "gather", gather_bad_v)
    assert _fails(T.test_single_token_returns_its_value) or \
        any(_fails(T.test_matches_torch_sdpa_float64, *c) for c in _sdpa_cases())


def test_wrong_key_chunk_order_is_caught(monkeypatch):
    def key_tile_swapped(k_pages, page, head):
        chunks, bs, x = k_pages.shape[2], k_pages.shape[3], k_pages.shape[4]
        return k_pages[page, head].transpose(1, 2, 0).reshape(bs, chunks * x)   # planted: x-major
    def gather_swapped(k_pages, v_pages, row, n, bs):
        n_blocks = (n + bs - 1) // bs
        K = np.concatenate([key_tile_swapped(k_pages, int(p), h)[None] for p in row[:n_blocks]
                            for h in range(k_pages.shape[1])]) if n_blocks else np.zeros((0, bs, 1))
        K = K.reshape(n_blocks, k_pages.shape[1], bs, -1).transpose(0, 2, 1, 3).reshape(n_blocks * bs,
                                                                                         k_pages.shape[1], -1)[:n]
        _, V = A_gather(k_pages, v_pages, row, n, bs)
        return np.asarray(K, dtype=np.float64), V
    A_gather = A.gather
    monkeypatch.setattr(A, "gather", gather_swapped)
    assert any(_fails(T.test_matches_torch_sdpa_float64, *c) for c in _sdpa_cases())


def test_lse_without_max_is_caught(monkeypatch):
    def partial_bad(q, K, V, scale):
        o, lse = orig(q, K, V, scale)
        if not math.isfinite(lse):
            return o, lse
        s = scale * (np.asarray(K, dtype=np.float64) @ np.asarray(q, dtype=np.float64))
        return o, float(lse - s.max())                  # planted: forgot to add the max back
    orig = A.partial
    monkeypatch.setattr(A, "partial", partial_bad)
    assert _fails(T.test_partial_lse_closed_form) or _fails(T.test_partials_combine_to_full_attention)


def test_combine_without_reweighting_is_caught(monkeypatch):
    def combine_plain(outs, lses):
        outs = [np.asarray(o, dtype=np.float64) for o in outs if True]
        lses = np.asarray(lses, dtype=np.float64)
        keep = [o for o, l in zip(outs, lses) if np.isfinite(l)]
        return np.mean(keep, axis=0) if keep else np.zeros_like(outs[0])   # planted: plain average
    monkeypatch.setattr(A, "lse_combine", combine_plain)
    assert _fails(T.test_partials_combine_to_full_attention)


def test_append_slot_index_mistake_is_caught(monkeypatch):
    def append_bad(k_pages, v_pages, block_table, positions, k_new, v_new, block_size):
        k_out = np.array(k_pages, copy=True)
        v_out = np.array(v_pages, copy=True)
        x = k_pages.shape[4]
        for b in range(k_new.shape[0]):
            pos = int(positions[b])
            page = int(block_table[b][pos // block_size])
            slot = (pos + 1) % block_size                 # planted: off by one slot
            for h in range(k_new.shape[1]):
                for i in range(k_new.shape[2]):
                    k_out[page, h, i // x, slot, i % x] = k_new[b, h, i]
                    v_out[page, h, i, slot] = v_new[b, h, i]
        return k_out, v_out
    monkeypatch.setattr(A, "append", append_bad)
    assert _fails(T.test_append_writes_exactly_the_slot_bits)


def test_kv_formula_without_factor_two_is_caught(monkeypatch):
    monkeypatch.setattr(KB, "kv_cache_bytes", lambda L, n_kv, d, s, b, p: L * n_kv * d * s * b * p)
    assert any(_fails(TB.test_per_token_matches_pages, c) for c in TB.GOLDEN["per_token"])


def test_kv_formula_with_query_heads_is_caught():
    # Using n_q_heads (32 for Llama-3-8B) where n_kv_heads belongs gives 512 KiB, not the printed 128 KiB.
    case = [c for c in TB.GOLDEN["per_token"] if c["model"] == "Llama-3-8B"][0]
    assert KB.kv_bytes_per_token(case["n_layers"], 32, case["head_dim"], case["bytes_per_elem"]) != case["bytes"]


# ------------------------------------------------------------ 8-bit KV cache
from oracle import kv_quant as KQ  # noqa: E402

from . import test_oracle_kv_quant as TQ  # noqa: E402


def test_quant_zero_point_sign_is_caught(monkeypatch):
    monkeypatch.setattr(KQ, "dequantize_vector",
                        lambda u, s, z: np.float64(s) * (np.asarray(u, dtype=np.float64) + np.float64(z)))
    assert _fails(TQ.test_hand_worked_vector_with_exact_scale)
    assert _fails(TQ.test_grid_points_round_trip_exactly)


def test_quant_floor_instead_of_rint_is_caught(monkeypatch):
    orig_rint = np.rint

    class _NP:
        def __getattr__(self, name):
            return np.floor if name == "rint" else getattr(np, name)
    monkeypatch.setattr(KQ, "np", _NP())
    assert _fails(TQ.test_hand_worked_vector_with_exact_scale)
    assert orig_rint is np.rint


def test_quant_meta_slot_off_by_one_is_caught(monkeypatch):
    orig = KQ.dequantize_vector

    def tiles_shifted(k_codes, v_codes, meta, page, head):
        ku = k_codes[page, head].transpose(1, 0, 2).reshape(k_codes.shape[3], -1)
        vu = v_codes[page, head].T
        m = np.roll(meta[page, head], 1, axis=1)          # planted: scale of the previous slot
        return orig(ku, m[0][:, None], m[1][:, None]), orig(vu, m[2][:, None], m[3][:, None])
    monkeypatch.setattr(KQ, "dequantized_tiles", tiles_shifted)
    assert any(_fails(TQ.test_decode_equals_decode_of_dequantized_pools, *c)
               for c in [(8, 2, 64, [40, 5, 17]), (4, 4, 32, [33])])
    assert _fails(TQ.test_decode_brute_force_tiny)


def test_quant_key_chunk_order_is_caught(monkeypatch):
    orig = KQ.dequantize_vector

    def tiles_swapped(k_codes, v_codes, meta, page, head):
        ku = k_codes[page, head].transpose(1, 2, 0).reshape(k_codes.shape[3], -1)   # planted: x-major
        vu = v_codes[page, head].T
        m = meta[page, head]
        return orig(ku, m[0][:, None], m[1][:, None]), orig(vu, m[2][:, None], m[3][:, None])
    monkeypatch.setattr(KQ, "dequantized_tiles", tiles_swapped)
    # needs more than one 16-feature chunk: the D = 64 and D = 32 pins
    assert any(_fails(TQ.test_decode_equals_decode_of_dequantized_pools, *c)
               for c in [(8, 2, 64, [40, 5, 17]), (4, 4, 32, [33])])


# ------------------------------------------------------- multi-token queries
from . import test_oracle_multi as TM  # noqa: E402

_SELF = [(4, 2, 32, 37, 0), (4, 2, 32, 45, 7)]


def test_multi_causal_bound_excluding_self_is_caught(monkeypatch):
    def range_no_self(seq_len, q_len, i, window):
        hi = seq_len - q_len + i               # planted: the query's own key left out
        return (max(0, hi - window) if window > 0 else 0), hi
    monkeypatch.setattr(A, "query_range", range_no_self)
    assert any(_fails(TM.test_all_tokens_as_queries_is_causal_self_attention, *c) for c in _SELF)
    assert _fails(TM.test_brute_force_tiny_window)


def test_multi_window_off_by_one_is_caught(monkeypatch):
    orig = A.query_range
    monkeypatch.setattr(A, "query_range",
                        lambda n, T, i, w: (orig(n, T, i, w)[0] + (1 if w > 0 else 0), orig(n, T, i, w)[1]))
    assert _fails(TM.test_all_tokens_as_queries_is_causal_self_attention, 4, 2, 32, 45, 7)
    assert _fails(TM.test_keys_outside_the_range_do_not_matter)


def test_multi_query_order_reversed_is_caught(monkeypatch):
    orig = A.query_range
    monkeypatch.setattr(A, "query_range", lambda n, T, i, w: orig(n, T, T - 1 - i, w))   # planted
    assert any(_fails(TM.test_all_tokens_as_queries_is_causal_self_attention, *c) for c in _SELF)


# ----------------------------------------------- byte accounting, copies, pool
from collections import deque  # noqa: E402

from oracle import page_pool as PP  # noqa: E402

from . import test_oracle_page_pool as TP  # noqa: E402


def test_gqa_ratio_inverted_is_caught(monkeypatch):
    orig = KB.mha_to_gqa_ratio
    monkeypatch.setattr(KB, "mha_to_gqa_ratio", lambda hq, hkv: 1.0 / orig(hq, hkv))   # planted
    assert any(_fails(TB.test_mha_gqa_ratio_matches_pages, c) for c in TB.GOLDEN["ratios"])


def test_attended_bytes_per_cached_token_is_caught(monkeypatch):
    monkeypatch.setattr(KB, "attended_kv_bytes",
                        lambda lens, hkv, d, p: sum(max(int(n) - 1, 0) for n in lens) * 2 * hkv * d * p)   # planted
    assert _fails(TB.test_one_llama2_layer_of_the_32gb_example_is_one_gib)


def test_copy_blocks_wrong_direction_is_caught(monkeypatch):
    orig = A.copy_blocks
    monkeypatch.setattr(A, "copy_blocks", lambda k, v, s, d: orig(k, v, d, s))   # planted: dst -> src
    assert _fails(T.test_copy_blocks_then_fork_decode_equals_unshared_cache)


def test_pool_takes_from_the_back_is_caught(monkeypatch):
    orig = PP.PagePool.reserve

    def reserve_back(self, seq_id, n_tokens, block_size=16):
        self.free = deque(reversed(self.free))       # planted: pops the end of the free list
        try:
            return orig(self, seq_id, n_tokens, block_size)
        finally:
            self.free = deque(reversed(self.free))
    monkeypatch.setattr(PP.PagePool, "reserve", reserve_back)
    assert _fails(TP.test_hand_worked_sequence_of_operations)
    assert _fails(TP.test_tiny_workload_layout)


def test_pool_release_to_the_front_is_caught(monkeypatch):
    def release_front(self, seq_id):
        for p in self.seqs.pop(seq_id):
            self.refs[p] -= 1
            if self.refs[p] == 0:
                self.free.appendleft(p)              # planted
    monkeypatch.setattr(PP.PagePool, "release", release_front)
    assert _fails(TP.test_hand_worked_sequence_of_operations)


def test_fork_without_reference_count_is_caught(monkeypatch):
    def fork_norefs(self, parent, child):
        self.seqs[child] = list(self.seqs[parent])   # planted: shared pages not counted
    monkeypatch.setattr(PP.PagePool, "fork", fork_norefs)
    assert _fails(TP.test_fork_and_copy_on_write)


def test_write_into_shared_block_without_copy_is_caught(monkeypatch):
    def rfw_nocopy(self, seq_id, position, block_size=16):
        self.reserve(seq_id, position + 1, block_size)
        return None                                  # planted: never copies
    monkeypatch.setattr(PP.PagePool, "reserve_for_write", rfw_nocopy)
    assert _fails(TP.test_fork_and_copy_on_write)


def test_block_table_zero_padding_is_caught(monkeypatch):
    orig = PP.PagePool.block_table
    monkeypatch.setattr(PP.PagePool, "block_table",
                        lambda self, ids, mb: np.maximum(orig(self, ids, mb), 0))   # planted: pads with page 0
    assert _fails(TP.test_hand_worked_sequence_of_operations)


def test_quant_decode_interleaved_head_map_is_caught(monkeypatch):
    def decode_interleaved(q, k_codes, v_codes, meta, block_table, seq_lens, n_q_heads, n_kv_heads,
                           block_size, scale):
        q = np.asarray(q, dtype=np.float64)
        out = np.zeros(q.shape)
        for b in range(q.shape[0]):
            n = int(seq_lens[b])
            if n == 0:
                continue
            K, V = KQ.gather(k_codes, v_codes, meta, block_table[b], n, block_size)
            for hq in range(n_q_heads):
                h = hq % n_kv_heads                  # planted: interleaved instead of contiguous groups
                out[b, hq] = A.attend(q[b, hq], K[:, h], V[:, h], scale)
        return out
    monkeypatch.setattr(KQ, "decode", decode_interleaved)
    assert _fails(TQ.test_decode_equals_decode_of_dequantized_pools, 8, 2, 64, [40, 5, 17])


def test_quant_gather_dropped_last_token_is_caught(monkeypatch):
    orig = KQ.gather
    monkeypatch.setattr(KQ, "gather", lambda kc, vc, m, row, n, bs: tuple(
        x[: max(n - 1, 0)] for x in orig(kc, vc, m, row, n, bs)))   # planted
    assert _fails(TQ.test_decode_brute_force_tiny)


def test_quant_append_slot_off_by_one_is_caught(monkeypatch):
    orig_append = KQ.append

    def append_next_slot(kc, vc, meta, bt, positions, kn, vn, bs):
        return orig_append(kc, vc, meta, bt, [int(p) + 1 for p in positions], kn, vn, bs)   # planted: off by one
    monkeypatch.setattr(KQ, "append", append_next_slot)
    assert _fails(TQ.test_append_writes_exactly_the_slot)
