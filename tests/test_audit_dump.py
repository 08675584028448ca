"""attention_mask_dump (host code in the library): the visibility grid, the SVG and the
per-query index lists, checked against the oracle's visibility rules and against the
pages' 16-token worked example ("Attention mask layout": sliding window 8, CSA m=4 with
top-2, HCA m'=8).  No GPU needed."""
from __future__ import annotations

import json
import os
import re
import xml.etree.ElementTree as ET

import numpy as np
import pytest

import oracle
import workloads as W
from long_context_sparse_09_amd import DSV4Error, attention_mask_dump

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example_16tok.json")))
CHAR = {"#": 1, "@": 2, ":": 3, ".": 0, "!": 4}


def parse(text):
    """Text grid -> (positions, window cells [rows, P], entry cells [rows, E])."""
    pos, win, ent = [], [], []
    for line in text.splitlines()[2:]:
        m = re.match(r"\s*(\d+) (\S+)(?: \|(\S*))?$", line)
        assert m, line
        pos.append(int(m.group(1)))
        win.append([CHAR[c] for c in m.group(2)])
        ent.append([CHAR[c] for c in (m.group(3) or "")])
    return pos, np.array(win), np.array(ent)


def oracle_window(rows, P, window, q_pos0=0):
    g = np.zeros((rows, P), dtype=int)
    for t in range(rows):
        for j in oracle.window_rows(q_pos0 + t, window):
            g[t, j] = 1
    return g


def test_sliding_matches_window_rule_and_worked_example():
    S, Wn = GOLDEN["S"], GOLDEN["sliding_window"]
    pos, win, ent = parse(attention_mask_dump("sliding", S, Wn))
    assert pos == list(range(S)) and ent.size == 0
    assert np.array_equal(win, oracle_window(S, S, Wn))
    first_cut = min(t for t in range(S) if win[t, 0] == 0)
    assert first_cut == GOLDEN["stated"]["sliding_lower_left_cut_from_query"]


def test_hca_entry_visibility_matches_worked_example():
    S, Wn, m = GOLDEN["S"], GOLDEN["sliding_window"], GOLDEN["hca_m"]
    E = S // m
    pos, win, ent = parse(attention_mask_dump("hca", S, Wn, m=m, n_entries=E))
    assert np.array_equal(win, oracle_window(S, S, Wn))
    for t in range(S):
        vis = oracle.n_visible(t, m, E)
        assert list(ent[t]) == [2] * vis + [0] * (E - vis)
    first = {str(w): min(t for t in range(S) if ent[t, w] == 2) for w in range(E)}
    assert first == {k: v for k, v in GOLDEN["stated"]["hca_entry_first_visible_query"].items()}


def _tiny_csa_lists(S=16, m=4, k=2, seed=3):
    """The oracle's own top-k lists for random indexer inputs of the worked-example size."""
    nI, cI = 4, 8
    q = W.normal_rows(seed, 0, "aq", (nI, cI), slice(0, S), S).astype(np.float64)[None]
    w = W.normal_rows(seed, 0, "aw", (nI,), slice(0, S), S).astype(np.float64)[None]
    kp = W.normal_rows(seed, 0, "ak", (cI,), slice(0, S // m), S // m).astype(np.float64)[None]
    idx, _ = oracle.csa_index_topk(q, w, kp, [0], [S // m], m, k)
    return idx[0].astype(np.int32)


def test_csa_selected_entries_match_the_lists_and_warmup_sentinels():
    S, Wn, m, k = GOLDEN["S"], GOLDEN["sliding_window"], GOLDEN["csa_m"], GOLDEN["index_topk"]
    E = S // m
    lists = _tiny_csa_lists(S, m, k)
    pos, win, ent = parse(attention_mask_dump("csa", S, Wn, m=m, topk_idx=lists, n_entries=E))
    assert np.array_equal(win, oracle_window(S, S, Wn))
    for t in range(S):
        vis = oracle.n_visible(t, m, E)
        sel = set(int(e) for e in lists[t] if e >= 0)
        want = [2 if w in sel else (3 if w < vis else 0) for w in range(E)]
        assert list(ent[t]) == want, t
    empty = [t for t in range(S) if not (ent[t] == 2).any()]
    assert empty == GOLDEN["stated"]["csa_queries_with_no_entry"]
    # the index-list dump shows every slot, -1 sentinels included, and counts them
    dump = attention_mask_dump("csa", S, Wn, m=m, topk_idx=lists, n_entries=E, fmt="lists")
    lines = dump.splitlines()[1:]
    assert len(lines) == S
    for t, line in enumerate(lines):
        nums = [int(x) for x in re.findall(r"-?\d+", line.split(":", 1)[1].split("[")[0])]
        assert nums == [int(e) for e in lists[t]]
        n_empty = int((lists[t] < 0).sum())
        assert (f"[{n_empty} empty slot" in line) == (n_empty > 0)


def test_csa_flags_an_entry_that_is_not_visible():
    lists = -np.ones((6, 2), dtype=np.int32)
    lists[2, 0] = 1  # query 2 sees no entry yet (m = 4)
    _, _, ent = parse(attention_mask_dump("csa", 6, 8, m=4, topk_idx=lists, n_entries=2))
    assert ent[2, 1] == 4 and (ent[np.arange(6) != 2] != 4).all()


def test_offset_queries_and_ansi_and_svg_agree_with_text():
    lists = np.array([[3, -1], [0, 24]], dtype=np.int32)
    kw = dict(m=4, topk_idx=lists, n_entries=26, q_pos0=100)
    pos, win, ent = parse(attention_mask_dump("csa", 2, 8, **kw))
    assert pos == [100, 101]
    assert np.array_equal(win, oracle_window(2, 102, 8, q_pos0=100))
    # query 101 sees entries 0..24 (102 // 4 = 25): 0 and 24 selected, 23 a candidate, 25 masked
    assert ent[0, 3] == 2 and ent[1, 0] == 2 and ent[1, 24] == 2 and ent[1, 23] == 3 and ent[1, 25] == 0
    ansi = attention_mask_dump("csa", 2, 8, fmt="ansi", **kw)
    plain = re.sub(r"\x1b\[\d+m", "", ansi)
    assert "\x1b[" in ansi
    assert [l.replace("#", "?") for l in plain.splitlines()[2:]] == \
        [l.replace("#", "?").replace("@", "?") for l in attention_mask_dump("csa", 2, 8, **kw).splitlines()[2:]]
    root = ET.fromstring(attention_mask_dump("csa", 2, 8, fmt="svg", **kw))
    rects = [r for r in root.iter() if r.tag.endswith("rect")]
    assert len(rects) == 2 * (102 + 26)
    state = {(int(r.get("data-q")), int(r.get("data-c"))): int(r.get("data-state")) for r in rects}
    for t in range(2):
        for c in range(102):
            assert state[(t, c)] == win[t, c]
        for c in range(26):
            assert state[(t, 102 + c)] == ent[t, c]


def test_argument_errors():
    with pytest.raises(KeyError):
        attention_mask_dump("mla", 4, 8)
    with pytest.raises(DSV4Error, match="index lists"):
        attention_mask_dump("csa", 4, 8, m=4, n_entries=1)
    with pytest.raises(DSV4Error, match="window"):
        attention_mask_dump("sliding", 4, 0)
    with pytest.raises(DSV4Error, match="cells"):
        attention_mask_dump("sliding", 5000, 8)
    assert attention_mask_dump("sliding", 0, 8).count("\n") == 2  # header and legend only


@pytest.mark.gpu
def test_dump_of_gpu_topk_lists_matches_oracle_selection():
    """The dump of the GPU indexer's lists for the worked-example size shows the oracle's picks."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sparse_09_amd as L
    from gpu_util import check_topk_row

    S, Wn, m, k, nI, cI, seed = 16, 8, 4, 2, 4, 8, 3
    q = W.normal_rows(seed, 0, "aq", (nI, cI), slice(0, S), S).astype(np.float32)[None]
    w = W.normal_rows(seed, 0, "aw", (nI,), slice(0, S), S).astype(np.float32)[None]
    kp = W.normal_rows(seed, 0, "ak", (cI,), slice(0, S // m), S // m).astype(np.float32)[None]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    idx = torch.empty(1, S, k, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(L.csa_index_topk_workspace_size(1, S, S // m, k), 16), dtype=torch.uint8, device="cuda")
    zeros = torch.zeros(1, dtype=torch.int32, device="cuda")
    n_pool = torch.full((1,), S // m, dtype=torch.int32, device="cuda")
    L.csa_index_topk(dev(q), dev(w), dev(kp), zeros, n_pool, idx, None, m, ws)
    gpu = idx.cpu().numpy()[0]
    ref = _tiny_csa_lists(S, m, k, seed)
    for t in range(S):
        V = oracle.n_visible(t, m, S // m)
        s = oracle.index_scores(q[0, t].astype(np.float64), w[0, t].astype(np.float64), kp[0, :V].astype(np.float64))
        check_topk_row(gpu[t], s, k, f"t={t}")
    got = attention_mask_dump("csa", S, Wn, m=m, topk_idx=gpu, n_entries=S // m)
    want = attention_mask_dump("csa", S, Wn, m=m, topk_idx=ref, n_entries=S // m)
    assert parse(got)[2].tolist() == parse(want)[2].tolist()
