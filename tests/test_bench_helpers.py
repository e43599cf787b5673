"""Host-side helpers of bench.py (no GPU): the kernel-source digest that ties a
committed rocprofv3 traffic record to the code it was measured on."""
from __future__ import annotations

import bench


def _digest_of(tmp_path, monkeypatch, text: str) -> str:
    f = tmp_path / "k.hip"
    f.write_text(text)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "sgemm", ["k.hip"])
    return bench.source_digest("sgemm")


def test_digest_ignores_comments_and_layout(tmp_path, monkeypatch):
    base = _digest_of(tmp_path, monkeypatch, "int f(int x) { return x + 1; }\n")
    commented = _digest_of(tmp_path, monkeypatch,
                           "// a note\nint f(int x)  /* inline */ {\n    return x + 1;   // why\n}\n")
    assert base == commented


def test_digest_changes_with_code(tmp_path, monkeypatch):
    a = _digest_of(tmp_path, monkeypatch, "int f(int x) { return x + 1; }\n")
    b = _digest_of(tmp_path, monkeypatch, "int f(int x) { return x + 2; }\n")
    assert a != b


def test_digest_covers_included_headers():
    for kind, files in bench.KERNEL_SOURCES.items():
        assert any(f.endswith("epilogue.h") for f in files), kind
        assert any(f.endswith(f"{kind}_mfma.hip") for f in files), kind
