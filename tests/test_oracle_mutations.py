"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check each trips a pin.

Each mutation is a textual edit of the oracle's source (an anchor that must occur exactly
once, or the stated number of times, all of them replaced), executed as a fresh module; the
real oracle is untouched.  A mutation that no pin catches would mean the pins leave that
part of the oracle unchecked.
"""
import importlib.util
import os

import pytest

import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "dsv4_oracle.py")

MUTATIONS = {
    "rope_sign": [("x[..., C - r::2] = a * c - b * s", "x[..., C - r::2] = a * c + b * s"),
                  ("x[..., C - r + 1::2] = a * s + b * c", "x[..., C - r + 1::2] = -a * s + b * c")],
    "rope_frequency": [("np.power(float(base), -2.0 * i / r)", "np.power(float(base), -1.0 * i / r)")],
    "rope_split_halves": [("a = x[..., C - r::2].copy()", "a = x[..., C - r:C - r // 2].copy()"),
                          ("b = x[..., C - r + 1::2].copy()", "b = x[..., C - r // 2:].copy()"),
                          ("x[..., C - r::2] = a * c - b * s", "x[..., C - r:C - r // 2] = a * c - b * s"),
                          ("x[..., C - r + 1::2] = a * s + b * c", "x[..., C - r // 2:] = a * s + b * c")],
    "csa_window_shift": [("lo = (w - 1) * m if overlap else w * m", "lo = w * m if overlap else w * m")],
    "hca_window_shift": [("lo = (w - 1) * m if overlap else w * m", "lo = (w - 1) * m if overlap else w * m + 1")],
    "bias_dropped": [("a += np.asarray(bias, dtype=np.float64)[slots]", "a += 0.0")],
    "bias_slot_reversed": [("a += np.asarray(bias, dtype=np.float64)[slots]",
                            "a += np.asarray(bias, dtype=np.float64)[::-1][slots]")],
    "entry_rope_position": [("pos = (np.arange(entry_begin, entry_end) + 1) * m - 1 + pos_offset",
                             "pos = np.arange(entry_begin, entry_end) * m + pos_offset")],
    "visibility_off_by_one": [("v = (t + 1) // m", "v = t // m")],
    "window_one_too_many": [("return range(max(0, t - window + 1), t + 1)",
                             "return range(max(0, t - window), t + 1)")],
    "window_excludes_self": [("return range(max(0, t - window + 1), t + 1)",
                              "return range(max(0, t - window + 1), t)")],
    "relu_dropped": [("(wv[:, None] * np.maximum(dots, 0.0)).sum(axis=0)", "(wv[:, None] * dots).sum(axis=0)")],
    "head_weight_dropped": [("(wv[:, None] * np.maximum(dots, 0.0)).sum(axis=0)",
                             "np.maximum(dots, 0.0).sum(axis=0)")],
    "topk_tie_high_index": [("key=lambda w: (-s[w], w)", "key=lambda w: (-s[w], -w)")],
    "topk_smallest": [("key=lambda w: (-s[w], w)", "key=lambda w: (s[w], w)")],
    "sink_dropped": [("denom = np.exp(s - M) + e.sum(axis=1)", "denom = e.sum(axis=1)")],
    "sink_sign": [("denom = np.exp(s - M) + e.sum(axis=1)", "denom = np.exp(-s - M) + e.sum(axis=1)")],
    "scale_dropped": [("z = (qr @ K.T) * scale", "z = (qr @ K.T)")],
    "no_counter_rotation": [("return rope(o, -p_t, rope_dim, base)", "return o")],
    "counter_rotation_sign": [("return rope(o, -p_t, rope_dim, base)", "return rope(o, p_t, rope_dim, base)")],
    "query_not_rotated": [("qr = rope(q, p_t, rope_dim, base)", "qr = q")],
    "window_not_rotated": [("out[b] = rope(kv[b], pos, rope_dim, base)", "out[b] = kv[b]")],
    "sentinel_not_masked": [("sel = sel[sel >= 0]", "sel = sel")],
    "signed_zero_not_canonical": [("s = np.asarray(scores, dtype=np.float64) + 0.0",
                                   "s = np.asarray(scores, dtype=np.float64)"),
                                  ("key=lambda w: (-s[w], w)",
                                   "key=lambda w: (-s[w], 0 if np.signbit(s[w]) else -1, w)")],
    "split_halves_swapped": [("early = np.array([s_ < m for s_ in slots])",
                              "early = np.array([s_ >= m for s_ in slots])")],
    "oproj_heads_interleaved": [("mid[:, g * rank:(g + 1) * rank] = a[:, g * kg:(g + 1) * kg] @ w_a[g].T",
                                 "mid[:, g * rank:(g + 1) * rank] = "
                                 "np.asarray(attn, dtype=np.float64)[:, g::groups].reshape(T, -1) @ w_a[g].T")],
    "oproj_group_order_reversed": [("mid[:, g * rank:(g + 1) * rank] = a[:, g * kg:(g + 1) * kg] @ w_a[g].T",
                                    "mid[:, g * rank:(g + 1) * rank] = a[:, g * kg:(g + 1) * kg] @ w_a[groups - 1 - g].T")],
    "oproj_second_product_dropped": [("return mid @ w_b.T, mid", "return mid[:, :w_b.shape[0]], mid")],
    "inproj_gate_reads_kv_weight": [('out["c_q" if name == "q_a" else name] = x @ W[name].T',
                                     'out["c_q" if name == "q_a" else name] = x @ W["kv" if name == "gate" else name].T')],
    "inproj_latent_always_rounded": [('lat = round_bf16(out["c_q"]) if round_latent else out["c_q"]',
                                      'lat = round_bf16(out["c_q"])')],
    "inproj_indexer_query_from_query": [("out[name] = lat @ W[name].T",
                                         "out[name] = lat @ W[name].T if name == \"q\" else out[\"q\"][:, :W[name].shape[0]]")],
    # window buffer origin and clipping (decode rings, chunk halos)
    "window_start_clip_dropped": [("r0 = max(lo - kv_pos0_b, 0)", "r0 = lo - kv_pos0_b")],
    "window_end_clip_off_by_one": [("r1 = min(qpos + 1 - kv_pos0_b, kv_win_b.shape[0])",
                                    "r1 = min(qpos + 1 - kv_pos0_b, kv_win_b.shape[0] - 1)")],
    "window_buffer_origin_ignored": [("r0 = max(lo - kv_pos0_b, 0)", "r0 = max(lo, 0)"),
                                     ("r1 = min(qpos + 1 - kv_pos0_b, kv_win_b.shape[0])",
                                      "r1 = min(qpos + 1, kv_win_b.shape[0])")],
    # query start positions and pool capacities
    "index_q_pos0_ignored": [("V = n_visible(int(q_pos0[b]) + t, m, int(n_pool[b]))",
                              "V = n_visible(t, m, int(n_pool[b]))")],
    "index_n_pool_cap_dropped": [("V = n_visible(int(q_pos0[b]) + t, m, int(n_pool[b]))",
                                  "V = n_visible(int(q_pos0[b]) + t, m)")],
    "swa_new_pos0_ignored": [("pos = new_pos0[b] + np.arange(S_new) + pos_offset",
                              "pos = np.arange(S_new) + pos_offset")],
    "hca_n_pool_cap_dropped": [("V = n_visible(qpos, m_hca, npb)", "V = n_visible(qpos, m_hca)")],
    "attend_q_pos0_ignored": [("qpos = int(q_pos0[b]) + t", "qpos = t", 2)],
    "hca_q_pos0_off_by_one": [("V = n_visible(qpos, m_hca, npb)", "V = n_visible(qpos - 1, m_hca, npb)")],
    "compress_entry_range_ignored": [("for w in range(entry_begin, entry_end):",
                                      "for w in range(0, entry_end - entry_begin):")],
}


def _mutant(edits):
    with open(SRC) as f:
        text = f.read()
    for edit in edits:
        old, new = edit[:2]
        n = edit[2] if len(edit) > 2 else 1  # occurrences the edit must find (all replaced)
        assert text.count(old) == n, f"mutation anchor found {text.count(old)} times, not {n}: {old!r}"
        text = text.replace(old, new)
    spec = importlib.util.spec_from_loader("oracle_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(text, SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _mutant(MUTATIONS[name])
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutation {name} passed every pin"
