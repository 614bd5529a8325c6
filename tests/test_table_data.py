"""The installed dispatch table is regenerable from the data it carries: every
entry keeps each candidate variant's measured time, and applying the promotion
rule to those times gives the entry's choice (no GPU)."""
import json

import gemv_skinny_gemm_02_amd as skg
from gemv_skinny_gemm_02_amd import tuner


def test_promotion_rule():
    # the default stays unless something is at least 2 % faster
    assert tuner.choose("a", {"a": 10.0, "b": 9.9}) == "a"
    assert tuner.choose("a", {"a": 10.0, "b": 9.79}) == "b"
    assert tuner.choose("a", {"a": 10.0, "b": 9.8}) == "b"              # exactly 2 %
    # a default that was not measured gives way to the fastest; ties go to the first name
    assert tuner.choose("z", {"b": 5.0, "a": 5.0}) == "a"
    assert tuner.choose("a", {"a": 5.0}) == "a"


def test_installed_table_follows_from_its_candidates():
    path = skg.default_table_path()
    assert tuner.check(path) == []
    t = json.load(open(path))
    assert len(t["entries"]) > 100
    for e in t["entries"]:
        assert e["default"] in e["candidates"] or e["choice"] == min(e["candidates"], key=lambda v: e["candidates"][v]["us"])
