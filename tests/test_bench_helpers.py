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


def test_forward_flops_count_single_scalar_path():
    """1x0e (x) SH l=0 -> 1x0e: one CG term, one K entry, one s product."""
    from equivariant_gnn_message_amd import e3conv as E
    plan = E.Plan("1x0e", 0, "1x0e", 1.0)
    assert bench._conv_counts(plan) == (1, 1, 1)
    assert bench.forward_flops_per_edge(plan) == 2 * 1 + 2 * 1 * (1 + 1)
    assert bench.jvp_flops_per_edge(plan) == 4 * 1 + 6 * 1 * (1 + 1)


def test_forward_flops_count_large_layout():
    """64x(0e+1o+2e) (x) SH lmax 3 -> 64x(0e+1o+2e+3o): 17 paths; the scalar s
    costs min(2 l1 + 1, 2 l3 + 1) products per path (4 + 16 + 27 = 47)."""
    from equivariant_gnn_message_amd import e3conv as E
    plan = E.Plan("64x0e+64x1o+64x2e", 3, "64x0e+64x1o+64x2e+64x3o", 32.0)
    nnz, nnz_k, smul = bench._conv_counts(plan)
    assert len(plan.paths()) == 17 and smul == 47
    assert nnz_k <= sum((2 * q["l1"] + 1) * (2 * q["l3"] + 1) for q in plan.paths())
    assert bench.forward_flops_per_edge(plan) == 2 * nnz + 2 * 64 * (nnz_k + smul)


def test_roofline_picks_the_longer_roof():
    ms = 1.0
    below = bench.roofline("k", ms, nbytes=8e12 * 1e-3, flops=1e9)     # 1 ms of bytes, 0.013 ms of flops
    assert below["bound"] == "hbm" and abs(below["frac"] - 1.0) < 1e-12
    above = bench.roofline("k", ms, nbytes=1e9, flops=78.6e12 * 1e-3)  # 1 ms of flops, 0.125 ms of bytes
    assert above["bound"] == "alu" and above["unit"] == "TFLOP/s" and abs(above["frac"] - 1.0) < 1e-12
    assert abs(above["hbm_frac"] - 0.125) < 1e-12
    assert bench.roofline("k", ms, nbytes=1e9)["bound"] == "hbm"
