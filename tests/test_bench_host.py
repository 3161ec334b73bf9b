"""Host logic of the benchmark (no GPU): which committed counter figures a
bench line may quote.  A traffic figure in profiles/ holds for the kernel code
and the path thresholds it was measured with, so it is reported only while
both still match; comments in the kernel sources do not count as code."""
import bench


def _profile(tmp_path, lines):
    d = tmp_path / "profiles"
    d.mkdir(exist_ok=True)
    (d / "t.md").write_text("# a summary\n\nsome prose: with a colon\n\n" + "\n".join(lines) + "\n")


def test_traffic_reported_only_for_matching_code_and_thresholds(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha256", lambda: "abc")
    _profile(tmp_path, ["traffic_bytes_per_launch: 123", "source_sha256: abc", "path_rows: 3 24"])
    assert bench.measured_traffic("t.md", (3, 24)) == 123
    assert bench.measured_traffic("t.md", [3, 24]) == 123
    assert bench.measured_traffic("t.md", (3, 32)) is None      # other wide threshold
    assert bench.measured_traffic("t.md", (4, 24)) is None      # other streaming threshold
    monkeypatch.setattr(bench, "source_sha256", lambda: "abd")
    assert bench.measured_traffic("t.md", (3, 24)) is None      # kernels changed
    assert bench.measured_traffic("missing.md", (3, 24)) is None


def test_traffic_without_thresholds_is_not_reported(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha256", lambda: "abc")
    _profile(tmp_path, ["traffic_bytes_per_launch: 123", "source_sha256: abc"])
    assert bench.measured_traffic("t.md", (3, 24)) is None
    _profile(tmp_path, ["traffic_bytes_per_launch: many", "source_sha256: abc", "path_rows: 3 24"])
    assert bench.measured_traffic("t.md", (3, 24)) is None


def test_code_only_ignores_comments_and_keeps_literals():
    a = 'int a = 1;  // one\n/* block\n   comment */\nconst char* s = "//kept /* too */";\nchar c = \'"\';\n'
    b = 'int a = 1;\n\n\nconst char* s = "//kept /* too */";   // another\nchar c = \'"\'; /**/\n'
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) == 'int a = 1;\nconst char* s = "//kept /* too */";\nchar c = \'"\';'
    assert bench._code_only(a) != bench._code_only(a.replace("1;", "2;"))
    assert bench._code_only('s = "a\\"//b";') == 's = "a\\"//b";'   # escaped quote inside a string
