"""Planted mistakes in the oracle (CPU only): the oracle's pins must catch them.

Each mutant below is a copy of one oracle function with one plausible mistake written into its
source (a dropped square root, a flipped rotation sign, a 1-based frequency index, ...). The
mutant replaces the function for the duration of one test, in the oracle module (so the other
oracle functions call it) and in the package namespace (so the pins see it). Every pin of
tests/test_oracle.py then runs against the mutated oracle, and the test asserts that the pin
named for that mistake fails. A mistake that no pin catches would leave a part of the oracle
unpinned.
"""
import inspect
import itertools
import textwrap

import pytest

import oracle
import oracle.attention as A
import test_oracle as pins
from conftest import read_golden_rows

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")  # mutants may overflow on purpose

# (oracle function, source text, mutated text, the pin that must fail)
MUTANTS = {
    "dropped_sqrt_in_scale": ("prefill_rows", "scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D",
                              "test_single_head_d4_t3_constructed_case"),
    "rotation_sign": ("rope_rotate", "rr[..., :h] = a * c - b * s", "rr[..., :h] = a * c + b * s",
                      "test_rope_two_dims_is_plane_rotation"),
    "one_based_frequency": ("rope_inv_freq", "i = np.arange(head_dim // 2, dtype=np.float64)",
                            "i = np.arange(1, head_dim // 2 + 1, dtype=np.float64)",
                            "test_rope_wavelength_count_matches_printed"),
    "mask_on_the_diagonal": ("causal_mask", "j[None, :] > np.asarray(q_positions)[:, None]",
                             "j[None, :] >= np.asarray(q_positions)[:, None]", "test_mask_matches_printed_matrix"),
    "gqa_mapping_interleaved": ("kv_head_of", "return h // (n_heads // n_kv_heads)", "return h % n_kv_heads",
                                "test_gqa_equals_mha_with_repeated_kv"),
    "softmax_over_queries": ("softmax_rows", "m = np.max(s, axis=-1, keepdims=True)",
                             "m = np.max(s, axis=0, keepdims=True)", "test_equal_keys_give_prefix_means"),
    "softmax_sum_over_queries": ("softmax_rows", "return e / np.sum(e, axis=-1, keepdims=True)",
                                 "return e / np.sum(e, axis=0, keepdims=True)",
                                 "test_rows_sum_to_one_and_masked_weights_are_zero"),
    "decode_position": ("decode", "qh = rope_rotate(qh, [c - 1], rope_theta)\n",
                        "qh = rope_rotate(qh, [c], rope_theta)\n", "test_decode_equals_prefill_row_by_row"),
    "mla_rope_on_latent_dims": ("decode", "rot_dims=Dqk - Dv, rot_offset=Dv", "rot_dims=Dqk - Dv, rot_offset=0",
                                "test_mla_decoupled_rope_absorbed_equals_per_head"),
    "pairing_swap": ("rope_rotate", "    if interleaved:", "    if not interleaved:",
                     "test_rope_pair_index_and_frequency"),
    "missing_max_shift": ("softmax_rows", "e = np.exp(s - m)", "e = np.exp(s)",
                          "test_softmax_survives_large_scores"),
    "transposed_scores": ("attention_weights", "s = np.float64(scale) * (_f64(q) @ _f64(k).T)",
                          "s = np.float64(scale) * (_f64(k) @ _f64(q).T)",
                          "test_single_head_d4_t3_constructed_case"),
    "decode_context_off_by_one": ("decode", "kcache[b, :c, g, :], vcache[b, :c, g, :]",
                                  "kcache[b, :c - 1, g, :], vcache[b, :c - 1, g, :]",
                                  "test_decode_equals_prefill_row_by_row"),
    "chunk_positions_not_offset": ("prefill_chunk", "pos = int(q_start[b]) + np.arange(S)", "pos = np.arange(S)",
                                   "test_prefill_chunk_equals_rows_of_the_full_prefill"),
    "window_drops_own_key": ("window_mask", "(j < p - window + 1)", "(j < p - window + 2)",
                             "test_window_sink_visibility_matches_hand_table"),
    "v_from_rotated_keys": ("prefill_rows", "v[b, :, g, :], scale, mask)", "kh[0, :, 0, :v.shape[3]], scale, mask)",
                            "test_row0_attends_only_to_itself"),
}


def _mutated(fn_name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(A, fn_name)))
    assert src.count(old) == 1, (fn_name, old)
    ns = dict(vars(A))
    exec(compile(src.replace(old, new), f"<mutant of {fn_name}>", "exec"), ns)  # noqa: S102
    return ns[fn_name]


def _calls(fn):
    """Every argument set pytest would call a pin with: its parametrizations, and the golden reader."""
    grids = []
    for mark in getattr(fn, "pytestmark", []):
        if mark.name != "parametrize":
            continue
        names = mark.args[0].split(",") if isinstance(mark.args[0], str) else list(mark.args[0])
        names = [n.strip() for n in names]
        grids.append([dict(zip(names, v if len(names) > 1 else (v,))) for v in mark.args[1]])
    wants_golden = "golden" in inspect.signature(fn).parameters
    for combo in itertools.product(*grids) if grids else [()]:
        kw = {}
        for part in combo:
            kw.update(part)
        if wants_golden:
            kw["golden"] = read_golden_rows
        yield kw


def failing_pins():
    failed = set()
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        for kw in _calls(fn):
            try:
                fn(**kw)
            except Exception:  # noqa: BLE001 (an assertion, or the mutant breaking a shape)
                failed.add(name)
                break
    return failed


def test_unmutated_oracle_passes_every_pin():
    assert failing_pins() == set()


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, monkeypatch):
    fn_name, old, new, pin = MUTANTS[mutant]
    bad = _mutated(fn_name, old, new)
    monkeypatch.setattr(A, fn_name, bad)
    if hasattr(oracle, fn_name):
        monkeypatch.setattr(oracle, fn_name, bad)
    failed = failing_pins()
    assert pin in failed, (mutant, sorted(failed))
