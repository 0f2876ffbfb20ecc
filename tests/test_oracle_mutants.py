"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them.  The planted copy is built from the oracle's
own source text with one edit, run through the pin tests, and discarded."""
import inspect
import types

import pytest

from oracle import attention as O
from tests import test_oracle_chunk_pins as PC
from tests import test_oracle_fp8_prefill_pins as P8
from tests import test_oracle_fp8kv_chunk_pins as PQ
from tests import test_oracle_pins as P
from tests import test_oracle_rope_fp8_pins as PR

SRC = inspect.getsource(O)


def _mutant(old: str, new: str) -> types.ModuleType:
    assert old in SRC, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _bf(): return P.test_decode_matches_bruteforce_on_unpaged_tensors(8, 4)
def _bf62(): return P.test_decode_matches_bruteforce_on_unpaged_tensors(6, 2)


MUTANTS = {
    "interleaved_head_map": ("heads = slice(g * r, (g + 1) * r)", "heads = slice(g, Hq, Hk)",
                             [P.test_decode_head_mapping_matches_page_diagram, P.test_prefill_gqa_matches_sdpa]),
    "block_order_reversed": ("phys = np.asarray(block_table[b, :nb], dtype=np.int64)",
                             "phys = np.asarray(block_table[b, :nb][::-1], dtype=np.int64)",
                             [_bf, P.test_gather_follows_page_token_block_mapping]),
    "rope_term_dropped": ("s = s + Qc[:, Dn:] @ KR[c0:c0 + nk, 0, :].T", "s = s",
                          [P.test_prefill_mla_matches_sdpa_with_concatenated_rope_key,
                           P.test_prefill_matches_bruteforce_with_rope]),
    "causal_key_range_short": ("nk = int(i.max()) + 1", "nk = int(i.max())",
                               [P.test_prefill_gqa_matches_sdpa, P.test_prefill_first_row_returns_its_own_value_row]),
    "causal_strict": ("vis = j[None, :] <= i[:, None]", "vis = j[None, :] < i[:, None]",
                      [P.test_prefill_gqa_matches_sdpa, P.test_prefill_first_row_returns_its_own_value_row]),
    "block_mask_transposed": ("block_mask[b][(i // BLOCK)[:, None], (j // BLOCK)[None, :]]",
                              "block_mask[b][(j // BLOCK)[None, :], (i // BLOCK)[:, None]]",
                              [P.test_prefill_block_mask_matches_sdpa_element_mask,
                               P.test_prefill_matches_bruteforce_with_block_mask]),
    "k_scale_dropped": ("kv_dtype) * k_scale", "kv_dtype)",
                        [P.test_decode_fp8_matches_sdpa_on_torch_dequantised_cache]),
    "v_scale_dropped": ("kv_dtype) * v_scale", "kv_dtype)",
                        [P.test_decode_fp8_matches_sdpa_on_torch_dequantised_cache]),
    "decode_scale_dropped": ("s = scale * (qb[heads] @ K.T)", "s = (qb[heads] @ K.T)",
                             [P.test_decode_matches_torch_sdpa]),
    "decode_reads_k_for_v": ("V = widen(gather_kv_rows(v_pool,", "V = widen(gather_kv_rows(k_pool,",
                             [_bf62]),
    "prefill_scale_dropped": ("s = scale * s", "s = s", [P.test_prefill_gqa_matches_sdpa]),
    "e4m3_bias_8": ("2.0 ** (e - 7)", "2.0 ** (e - 8)", [P.test_e4m3fn_table_matches_torch_all_codes]),
    "e4m3_subnormal_scale": ("m * 2.0 ** -9", "m * 2.0 ** -10", [P.test_e4m3fn_closed_form_points]),
    "e4m3_no_nan": ("if e == 0xF and m == 0x7:", "if False:", [P.test_e4m3fn_closed_form_points]),
    "bf16_wrong_shift": ("<< np.uint32(16)", "<< np.uint32(15)", [P.test_bf16_widen_matches_torch]),
    "lse_sign": ("m_safe + np.log(", "m_safe - np.log(", [P.test_decode_matches_torch_sdpa]),
    "gqa_ratio_inverted_prefill": ("Qc = Q[gi, heads, :]", "Qc = Q[gi, g:g + r, :]",
                                   [P.test_prefill_gqa_matches_sdpa]),
    "fp8_q_scale_dropped": ('q = widen(q_nope, "e4m3fn") * (qs[..., None] if qs.ndim else qs)',
                            'q = widen(q_nope, "e4m3fn")',
                            [P8.test_fp8_prefill_matches_bruteforce_on_torch_decoded_codes]),
    "fp8_k_scale_dropped": ('kk = widen(k, "e4m3fn") * (ks[..., None] if ks.ndim else ks)',
                            'kk = widen(k, "e4m3fn")',
                            [P8.test_fp8_prefill_gqa_without_rope_matches_sdpa]),
    "fp8_scale_on_rope": ('np.concatenate([q, widen(q_rope, "bf16")], axis=2)',
                          'np.concatenate([q, widen(q_rope, "bf16") * float(q_scale)], axis=2)',
                          [P8.test_fp8_prefill_scales_leave_the_rope_part_alone]),
    "fp8_blockwise_key_scale_mean": ("(ks[..., None] if ks.ndim else ks)", "(ks.mean() if ks.ndim else ks)",
                                     [P8.test_fp8_blockwise_matches_bruteforce_on_torch_decoded_codes]),
    "fp8_blockwise_query_scale_flipped": ("(qs[..., None] if qs.ndim else qs)",
                                          "(qs[::-1, :, None] if qs.ndim else qs)",
                                          [P8.test_fp8_blockwise_matches_bruteforce_on_torch_decoded_codes]),
    "quantizer_ties_to_odd": ("((d_lo == d_hi) & (lo % 2 == 0))", "((d_lo == d_hi) & (lo % 2 == 1))",
                              [PQ.test_quantizer_closed_form_points]),
    "quantizer_top_code_missing": ("pos = _E4M3FN[:0x7F]", "pos = _E4M3FN[:0x7E]",
                                   [PQ.test_quantizer_closed_form_points]),
    "quantizer_rounds_down": ("pick_lo = (d_lo < d_hi)", "pick_lo = (d_lo <= 1e30)",
                              [lambda: PQ.test_quantizer_matches_torch_cast_on_every_bf16_value(1.0)]),
    "fp8kv_v_scale_dropped": ("V = widen(gather_kv_rows(v_pool, block_table, b, g, Lk), kvd) * float(v_scale)",
                              "V = widen(gather_kv_rows(v_pool, block_table, b, g, Lk), kvd)",
                              [PQ.test_fp8_chunk_prefill_matches_bruteforce_on_torch_decoded_pages]),
    "chunk_key_range_short": ("off + int(i.max()) + 1))", "off + int(i.max())))",
                              [PC.test_chunk_prefill_matches_sdpa_with_offset_mask,
                               PC.test_chunk_first_query_of_a_new_sequence_returns_its_value_row]),
    "rope_fp8_scale_on_the_nope_keys": ("kr = widen(k_rope, \"e4m3fn\") * ks[:, None, None]\n    return ragged_prefill(widen(q, \"bf16\"), widen(k, \"bf16\")",
                                        "kr = widen(k_rope, \"e4m3fn\")\n    return ragged_prefill(widen(q, \"bf16\"), widen(k, \"bf16\") * ks[:, None, None]",
                                        [PR.test_rope_fp8_scales_touch_only_the_rope_term,
                                         PR.test_rope_fp8_prefill_matches_bruteforce_on_torch_decoded_codes]),
    "rope_fp8_scale_rows_reversed": ("kr = widen(k_rope, \"e4m3fn\") * ks[:, None, None]",
                                     "kr = widen(k_rope, \"e4m3fn\") * ks[::-1, None, None]",
                                     [PR.test_rope_fp8_zero_scale_acts_as_zero_codes_row_by_row]),
    "rope_fp8_scale_dropped": ("kr = widen(k_rope, \"e4m3fn\") * ks[:, None, None]",
                               "kr = widen(k_rope, \"e4m3fn\")",
                               [PR.test_rope_fp8_with_power_of_two_scales_is_a_bf16_rope_key]),
    "fp8_rope_dropped": ('np.concatenate([q, widen(q_rope, "bf16")], axis=2)',
                         'np.concatenate([q, 0 * widen(q_rope, "bf16")], axis=2)',
                         [P8.test_fp8_prefill_matches_sdpa_with_concatenated_rope_key]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    old, new, catchers = MUTANTS[name]
    mutant = _mutant(old, new)
    monkeypatch.setattr(P, "O", mutant)
    monkeypatch.setattr(P8, "O", mutant)
    monkeypatch.setattr(PQ, "O", mutant)
    monkeypatch.setattr(PC, "O", mutant)
    monkeypatch.setattr(PR, "O", mutant)
    caught = []
    for fn in catchers:
        try:
            fn()
        except Exception:        # an assertion, or the mutant breaking outright
            caught.append(fn.__name__)
    assert caught, f"mutant {name} passed every pin it was aimed at"
