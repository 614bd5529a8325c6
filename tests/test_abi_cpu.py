"""The C ABI library without a GPU: it loads, exports every declared symbol,
and its table logic (identity header, refusals, lookup, defaults) behaves."""
import json
import os
import re
import subprocess
import sys

import pytest

import gemv_skinny_gemm_02_amd as skg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="session", autouse=True)
def _lib():
    if not os.path.exists(skg.lib_path()):
        from gemv_skinny_gemm_02_amd import build
        build.build()
    skg.load()


def _declared():
    txt = open(os.path.join(ROOT, "include", "skinny_gemm.h")).read()
    return sorted(set(re.findall(r"\b(skinny_gemm_\w+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 14
    out = subprocess.run(["nm", "-D", "--defined-only", skg.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (skinny_gemm_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = skg.load()
    for n in names:
        assert hasattr(lib, n)


def _identity(**kw):
    d = dict(arch="gfx950", hip="70226015", cc="deadbeef", space="cafe0001")
    d.update(kw)
    return ";".join(f"{k}={v}" for k, v in d.items())


def _write(tmp_path, ident, entries, name="t.json", drop=()):
    idd = dict(x.split("=") for x in ident.split(";"))
    for k in drop:
        idd.pop(k)
    path = tmp_path / name
    path.write_text(json.dumps({"format": "skinny_gemm_table", "identity": idd, "entries": entries}))
    return str(path)


E1 = [{"op": "bf16", "rows": 8, "N": 4096, "K": 4096, "choice": "gemv_r1_k4_p2",
       "candidates": {"gemv_r1_k4_p2": {"us": 5.0}, "gemv_r4_k4_p1": {"us": 6.0}}},
      {"op": "gated", "rows": 16, "N": 12288, "K": 4096, "choice": "tile_f2_k4_p4"}]


def test_variants_and_buckets():
    names = skg.variants("bf16")
    assert names == skg.variants("a8w8_block") and len(names) == skg.skinny_gemm_num_variants(0)
    assert any(n.startswith("gemv_") for n in names) and any(n.startswith("tile_") for n in names)
    # every op has a variant for every M in 1..600
    for op in skg.OPS:
        for M in range(1, 601):
            assert any(skg.skinny_gemm_variant_supports(op, i, M) for i in range(len(names))), (op, M)
    # GEMV variants never claim rows above 16; the packed-weight stream serves
    # only the packed bf16 and gated forms, up to 8 rows; the bf16 tile
    # variants serve every bucket from one row
    for i, n in enumerate(names):
        if n.startswith("gemv_"):
            assert not skg.skinny_gemm_variant_supports("bf16", i, 17)
        elif n.startswith("pg_"):
            assert not skg.skinny_gemm_variant_supports("bf16", i, 1)
            assert skg.skinny_gemm_variant_supports("bf16_packed", i, 8)
            assert skg.skinny_gemm_variant_supports("gated_packed", i, 1)
            assert not skg.skinny_gemm_variant_supports("bf16_packed", i, 9)
            assert not skg.skinny_gemm_variant_supports("a8w8_block_packed", i, 1)
        else:
            assert skg.skinny_gemm_variant_supports("bf16", i, 1)


def test_table_engaged_lookup_and_buckets(tmp_path):
    ident = _identity()
    p = _write(tmp_path, ident, E1)
    skg.skinny_gemm_load_table_as(p, ident)
    engaged, status = skg.skinny_gemm_table_status()
    assert engaged and status.startswith("engaged 2 shapes")
    # M in (6, 8] rounds up to the rows-8 bucket; no nearest fallback outside it
    for M in (7, 8):
        assert skg.skinny_gemm_query("bf16", M, 4096, 4096) == ("gemv_r1_k4_p2", "table")
    for M in (6, 9, 12):
        assert skg.skinny_gemm_query("bf16", M, 4096, 4096)[1] == "default"
    assert skg.skinny_gemm_query("bf16", 8, 4096, 4095)[1] == "default"
    assert skg.skinny_gemm_query("gated", 13, 12288, 4096) == ("tile_f2_k4_p4", "table")
    assert skg.skinny_gemm_query("fp8_tensor", 8, 4096, 4096)[1] == "default"


def test_mid_m_buckets(tmp_path):
    """The binding's bucket list is the library's: a table entry at every
    bucket engages, rows between buckets are refused, and M above 128 rounds
    up to its mid-M bucket (steps of 16 to 256, of 32 to 512: the grid the
    decode page tunes its verify and drafter rows at, Decode optimization
    round 3, "Retained change 3")."""
    assert skg.BUCKETS[:13] == (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 64, 96, 128)
    assert skg.BUCKETS[13:] == tuple(range(144, 257, 16)) + tuple(range(288, 513, 32))
    ident = _identity()
    tile = "tlds_f1_s1_p4"
    entries = [{"op": "bf16", "rows": b, "N": 4096, "K": 4096, "choice": tile} for b in skg.BUCKETS if b >= 16]
    p = _write(tmp_path, ident, entries)
    skg.skinny_gemm_load_table_as(p, ident)
    assert skg.skinny_gemm_table_status()[1].startswith(f"engaged {len(entries)} shapes")
    for M in (129, 144, 145, 200, 256, 257, 300, 511, 512):
        assert skg.skinny_gemm_query("bf16", M, 4096, 4096) == (tile, "table"), M
    assert skg.skinny_gemm_query("bf16", 513, 4096, 4096)[1] == "default"
    for rows in (130, 250, 260, 500, 600):
        bad = entries + [{"op": "bf16", "rows": rows, "N": 4096, "K": 4096, "choice": tile}]
        code = f"""
import gemv_skinny_gemm_02_amd as skg
skg.skinny_gemm_load_table_as({_write(tmp_path, ident, bad, name=f"b{rows}.json")!r}, {ident!r})
assert not skg.skinny_gemm_table_status()[0]
"""
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
        assert r.returncode == 0 and "is not a rows bucket" in r.stderr, (rows, r.stderr)


@pytest.mark.parametrize("case,needle", [
    ("stale", "has no selection-space token"),
    ("space", "selection-space token"),
    ("arch", "made for gfx942"),
    ("hip", "tuned on HIP runtime"),
    ("cc", "built by compiler"),
    ("variant", "does not compile"),
    ("bucket", "is not a rows bucket"),
    ("unsupported", "is not compiled for"),
])
def test_table_refusals(tmp_path, case, needle):
    ident = _identity()
    entries = json.loads(json.dumps(E1))
    drop = ()
    table_ident = ident
    if case == "stale":
        drop = ("space",)
    elif case == "space":
        table_ident = _identity(space="00000099")
    elif case == "arch":
        table_ident = _identity(arch="gfx942")
    elif case == "hip":
        table_ident = _identity(hip="60000000")
    elif case == "cc":
        table_ident = _identity(cc="01234567")
    elif case == "variant":
        entries[0]["choice"] = "gemv_r3_k9_u9"
    elif case == "bucket":
        entries[0]["rows"] = 5
    elif case == "unsupported":
        entries[1]["choice"] = "gemv_r8_k4_p1"
    p = _write(tmp_path, table_ident, entries, drop=drop)
    code = f"""
import gemv_skinny_gemm_02_amd as skg
skg.skinny_gemm_load_table_as({p!r}, {ident!r})
e, s = skg.skinny_gemm_table_status()
assert not e, s
assert skg.skinny_gemm_query('bf16', 8, 4096, 4096)[1] == 'default'
print(s)
"""
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("skinny_gemm:")]
    assert len(lines) == 1 and "refused" in lines[0] and needle in lines[0], r.stderr


def test_force_knob_refuses_table(tmp_path):
    ident = _identity()
    p = _write(tmp_path, ident, E1)
    code = f"""
import gemv_skinny_gemm_02_amd as skg
skg.skinny_gemm_load_table_as({p!r}, {ident!r})
assert not skg.skinny_gemm_table_status()[0]
assert skg.skinny_gemm_query('bf16', 3, 4096, 4096) == ('gemv_r4_k1_p2', 'force')
# a forced variant that cannot run the rows falls back to the default
assert skg.skinny_gemm_query('bf16', 40, 4096, 4096)[1] == 'default'
"""
    env = dict(os.environ, SKINNY_GEMM_FORCE="gemv_r4_k1_p2")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, env=env)
    assert r.returncode == 0, r.stderr
    assert "SKINNY_GEMM_FORCE=gemv_r4_k1_p2 reroutes the dispatch" in r.stderr


def test_malformed_and_missing(tmp_path):
    ident = _identity()
    bad = tmp_path / "bad.json"
    bad.write_text('{"identity": {"arch": "gfx950", ')
    with pytest.raises(skg.SkinnyGemmError) as e:
        skg.skinny_gemm_load_table_as(str(bad), ident)
    assert e.value.status == 4
    assert not skg.skinny_gemm_table_status()[0]
    with pytest.raises(skg.SkinnyGemmError):
        skg.skinny_gemm_load_table_as(str(tmp_path / "nope.json"), ident)
    with pytest.raises(skg.SkinnyGemmError):
        skg.skinny_gemm_load_table_as(None, "arch=gfx950")
    skg.skinny_gemm_load_table_as(None, ident)         # explicit no table
    assert skg.skinny_gemm_query("bf16", 1, 4096, 4096)[1] == "default"


def test_defaults_follow_the_rows_rule():
    """The untuned rule: VALU weight stream for few rows (up to 8 for small
    weights), the LDS tile with the K split inside the workgroup for small
    weights and for 6..16 rows on evenly tiling shapes, the LDS tile with a K
    split across workgroups sized by N otherwise."""
    skg.skinny_gemm_load_table_as(None, _identity())
    q = lambda op, M, N, K: skg.skinny_gemm_query(op, M, N, K)[0]
    for op in skg.OPS:
        for M in (1, 2, 3):
            if op == "a8w8_quant_packed":
                assert q(op, M, 4096, 4096).startswith("tlds_f1_s"), (op, M)
            elif op.endswith("_packed"):  # packed weight, few rows: direct x
                assert q(op, M, 4096, 4096).startswith("tlds_d_"), (op, M)
            elif op not in ("a8w8_quant", "a8w8_block"):   # A8W8: the LDS tile from one row
                assert q(op, M, 4096, 4096).startswith("gemv_"), (op, M)
            else:
                assert q(op, M, 4096, 4096).startswith("tlds_"), (op, M)
        for M in (16, 24, 32, 64, 96, 128, 129, 1000):
            assert q(op, M, 4096, 4096).startswith("tlds_"), (op, M)
    for M in (64, 96, 128):     # packed weight, many rows: x through LDS
        assert not q("bf16_packed", M, 4096, 4096).startswith("tlds_d_"), M
    for M in (1, 2, 3, 4, 8, 16, 64, 128, 300):
        assert q("a8w8_quant", M, 8192, 4096).startswith("tlds_"), M
        assert q("a8w8_quant", M, 32768, 1024).startswith("tlds_"), M
    assert q("bf16", 4, 2048, 2048).startswith("gemv_")
    assert q("fp8_tensor", 4, 248320, 4096).startswith("tlds_")
    assert q("a8w8_block", 4, 8192, 4096).startswith("tlds_")
    for M in (4, 6):            # small weights stay on the VALU stream up to 6 rows
        assert q("bf16", M, 1024, 1024).startswith("gemv_"), M
        assert q("bf16", M, 2048, 2048).startswith("gemv_"), M
    for M in (8, 12, 16, 32, 64):   # then direct x with K split over the waves
        assert q("bf16", M, 1024, 1024) == "tlds_d_k4_f1_s1_p4_m1", M
    assert q("bf16", 128, 1024, 1024).startswith("tlds_k4_")
    for M in (4, 6):            # large rows: direct x over eight waves
        assert q("bf16", M, 4096, 4096) == "tlds_d_w8_k8_f1_s1_p4_m2", M
        assert q("bf16", M, 4096, 12288) == "tlds_d_w8_k8_f1_s1_p4_m2", M
    assert q("bf16", 128, 2048, 2048) == "tlds_w8_k4_f1_s1_p4_m2"
    # GEMV shape: two rows per wave for one x row, eight for a vocabulary N,
    # one wave per row (no K split) for rows under 2 KiB
    assert q("bf16", 1, 4096, 4096) == "gemv_r2_k4_p1"
    assert q("bf16", 3, 4096, 4096) == "gemv_r4_k4_p1"
    assert q("fp8_tensor", 2, 248320, 4096) == "gemv_r8_k4_p1"
    assert q("a8w8_block", 1, 32768, 1024) == "tlds_f1_s1_p4_m2"
    assert q("a8w8_block", 1, 8192, 4096) == "tlds_d_w8_k8_f1_s1_p4_m2"
    # in-workgroup K split where the 16-row tiles come in multiples of 256
    assert q("bf16", 8, 4096, 4096) == "tlds_k4_f1_s1_p4_m2"
    assert q("gated", 16, 12288, 4096) == "tlds_k4_f1_s1_p4_m2"
    assert q("a8w8_block", 8, 8192, 4096) == "tlds_w8_k4_f1_s1_p4_m2"
    assert q("bf16", 8, 6144, 4096) == "tlds_f1_s4_p4"            # 384 tiles: split across workgroups
    assert q("a8w8_block", 8, 32768, 1024) == "tlds_f1_s1_p4_m2"  # 1 KiB rows
    # K split across workgroups: 4 up to 8192 weight rows, 2 up to 16384, else 1
    assert q("bf16", 32, 4096, 12288) == "tlds_f1_s4_p4"
    assert q("bf16", 64, 4096, 12288) == "tlds_f1_s4_p4_m4"
    assert q("bf16", 128, 4096, 12288) == "tlds_w8_f1_s4_p4_m4"
    assert q("bf16", 32, 12288, 4096) == "tlds_f1_s2_p4"
    assert q("gated", 32, 12288, 4096) == "tlds_f1_s1_p4"

def test_selection_token_names_the_buckets():
    """The text the selection-space token hashes lists exactly the rows
    buckets dispatch uses (a table tuned for another bucket list is refused)."""
    src = open(os.path.join(ROOT, "gemv_skinny_gemm_02_amd", "csrc", "variants.hpp")).read()
    arr = re.search(r"kBuckets\[\]\s*=\s*\{([^}]*)\}", src).group(1)
    buckets = tuple(int(v) for v in arr.replace("\n", " ").split(",") if v.strip())
    text = re.search(r'"buckets=([0-9,]+);', src).group(1)
    assert tuple(int(v) for v in text.split(",")) == buckets == skg.BUCKETS


def test_default_split_falls_back_when_tiles_do_not_fit():
    """The built-in default splits K across workgroups for mid-sized weights;
    at M far beyond the skinny range its output tiles would outgrow the
    split-K tile state (20480 tiles), and the default then takes the rule's
    no-split choice instead of one the launch would refuse."""
    for op in ("bf16", "bf16_packed", "gated", "a8w8_block"):
        assert skg.skinny_gemm_workspace_bytes(op, 1024, 8192, 4096) > 0, op      # splits K
        assert skg.skinny_gemm_workspace_bytes(op, 65536, 8192, 4096) == 0, op    # too many tiles to split


def test_two_operand_tile_heights():
    """The two-operand tile serves bf16 and A8W8 (both layouts) at every tile
    height of whole 16-row fragments, 96-row tiles included (the A8W8 x
    scales sit in LDS in blocks of 64 rows); the other forms never get it."""
    names = skg.variants("bf16")
    heights = set()
    for i, n in enumerate(names):
        m = re.fullmatch(r"mt_m(\d+)_f(\d+)_a(\d+)_b(\d+)_s(\d+)_p(\d+)", n)
        if not m:
            continue
        fm, fn, wm, wn = (int(v) for v in m.groups()[:4])
        heights.add(16 * fm * wm)
        for op in ("bf16", "bf16_packed", "a8w8_block", "a8w8_block_packed"):
            assert skg.skinny_gemm_variant_supports(op, i, 144), (op, n)
        for op in ("gated", "gated_packed", "fp8_tensor", "fp8_tensor_packed", "a8w8_quant", "a8w8_quant_packed"):
            assert not skg.skinny_gemm_variant_supports(op, i, 144), (op, n)
    assert 96 in heights and 384 in heights and 128 in heights, sorted(heights)
