"""Host-side logic of bench.py (no GPU): the check that keeps the committed
HBM-traffic figure tied to the code it was measured on."""
import os
import shutil

import bench


SRC = ["diffusion_transformer_dit_amd/csrc/gemm.hip", "diffusion_transformer_dit_amd/csrc/common.h"]


def _copy_tree(tmp_path):
    for f in SRC:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, f), dst)


def test_code_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.code_digest(SRC)
    gemm = tmp_path / SRC[0]
    text = gemm.read_text()
    # comment-only edits and re-indentation keep the digest
    gemm.write_text("// a new leading comment\n/* and a block\n   comment */\n" + text.replace("\n", "\n  ", 50))
    assert bench.code_digest(SRC) == base
    # a changed token of code changes it
    gemm.write_text(text.replace("constexpr int kGroupM = 4;", "constexpr int kGroupM = 8;"))
    assert "constexpr int kGroupM = 4;" in text
    assert bench.code_digest(SRC) != base

