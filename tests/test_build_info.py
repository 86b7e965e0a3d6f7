"""The build stamp and source hash that bench.py reports with every line
(which sources the loaded library was built from)."""
import os

from outer_product_gemm_amd import build as B


def test_code_only_ignores_comments_and_spacing():
    a = "int x = 1; // note\n/* block\n comment */ float  y=2;\n"
    b = "int x = 1;\nfloat  y=2;   // other note\n"
    assert B._code_only(a) == B._code_only(b) == "int x = 1; float y=2;"
    assert B._code_only("int x = 2;") != B._code_only("int x = 1;")


def test_source_hash_covers_every_source_by_default():
    names = sorted(n for n in os.listdir(B.CSRC) if n.endswith((".hip", ".h", ".cpp")))
    assert B.source_hash() == B.source_hash(names)
    assert B.source_hash(names[:1]) != B.source_hash(names)
    assert len(B.source_hash()) == 16


def test_stamp_round_trip(tmp_path, monkeypatch):
    monkeypatch.setattr(B, "STAMP", str(tmp_path / "stamp.json"))
    assert B.read_stamp() is None
    s = B.write_stamp()
    assert B.read_stamp() == s
    assert s["source_hash"] == B.source_hash()
