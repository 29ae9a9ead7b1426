"""Host logic of the per-layer P~V precision choice (no GPU needed).

"SageAttention ..." detail page, §2 Q2 item 3: a layer keeps the faster
kernel when its cosine similarity to full precision is above 99.8%.
"""
import json

import pytest

from quantized_attention_qk_amd.adaptive import (DEFAULT_THRESHOLD, choose_mode, load_modes,
                                                 sample_rows, save_modes)


def test_threshold_is_the_pages_value():
    consts = json.load(open(__file__.replace("test_adaptive.py", "golden/pages_constants.json")))
    assert DEFAULT_THRESHOLD == consts["adaptive_cos_threshold"]["value"]


@pytest.mark.parametrize("cos,mode", [(0.9999, "fp8"), (0.998, "fp8"), (0.99799, "fp16"),
                                      (0.5, "fp16"), (float("nan"), "fp16")])
def test_choose_mode(cos, mode):
    assert choose_mode(cos) == mode


def test_choose_mode_candidates():
    # the page's own pair (all-INT8 kernel or FP16) and the ordered 3-way choice
    assert choose_mode(0.9985, candidates=("int8",)) == "int8"
    assert choose_mode(0.9975, candidates=("int8",)) == "fp16"
    cos = {"fp8": 0.9990, "int8": 0.9970}
    assert choose_mode(cos, candidates=("fp8", "int8")) == "fp8"
    assert choose_mode(cos, candidates=("int8", "fp8")) == "fp8"
    assert choose_mode({"fp8": 0.99, "int8": 0.999}, candidates=("fp8", "int8")) == "int8"
    assert choose_mode({"fp8": 0.99, "int8": 0.99}, candidates=("fp8", "int8")) == "fp16"
    with pytest.raises(ValueError):
        choose_mode(0.999, candidates=("fp16",))


def test_sample_rows_seeded_and_bounded():
    a = sample_rows(1000, 64, seed=3)
    b = sample_rows(1000, 64, seed=3)
    assert a.tolist() == b.tolist()
    assert 0 in a.tolist() and 999 in a.tolist()
    assert len(set(a.tolist())) == a.numel() and 0 < a.numel() <= 64
    assert int(a.min()) >= 0 and int(a.max()) < 1000
    assert sample_rows(5, 64, seed=0).tolist() == [0, 1, 2, 3, 4]
    assert sample_rows(1, 8, seed=0).tolist() == [0]


def test_modes_round_trip(tmp_path):
    t = {"blocks.0.attn": {"pv_mode": "fp8", "cos_fp8": 0.9991},
         "blocks.1.attn": {"pv_mode": "fp16", "cos_fp8": 0.9962}}
    p = tmp_path / "modes.json"
    save_modes(t, str(p))
    assert load_modes(str(p)) == t
    t2 = {"a": {"pv_mode": "int8", "cos_int8": 0.999}}
    save_modes(t2, str(p))
    assert load_modes(str(p)) == t2
    p.write_text(json.dumps({"x": {"pv_mode": "int4"}}))
    with pytest.raises(ValueError):
        load_modes(str(p))
