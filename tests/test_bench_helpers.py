"""Host-side helpers of bench.py (CPU only)."""

import bench


def test_strip_comments_keeps_code_and_strings():
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "a//b /* c */";\nfloat f;'
    assert bench.strip_comments(src) == 'int a = 1; const char* s = "a//b /* c */"; float f;'


def test_comment_edits_do_not_change_the_code_hash(tmp_path, monkeypatch):
    """A counter record stays valid across comment edits and goes stale on a code edit."""
    csrc = tmp_path / "equivariant_gnn_message_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("// kernel\n__global__ void k(float* p) { p[0] = 1.0f; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (csrc / "k.hip").write_text("// kernel, reworded\n__global__ void k(float* p) {\n  p[0] = 1.0f;  /* one */\n}\n")
    assert bench.kernel_source_hash() == h0
    (csrc / "k.hip").write_text("__global__ void k(float* p) { p[0] = 2.0f; }\n")
    assert bench.kernel_source_hash() != h0
