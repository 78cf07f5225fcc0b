"""Host-side logic of bench.py that needs no GPU: the source hash that
decides whether the stored HBM counters still describe the kernels."""
import os
import shutil

import bench


def _copy_sources(tmp_path):
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "combine_ll_moe_amd", "csrc")
    dst = tmp_path / "csrc"
    dst.mkdir()
    for name in bench.PATH_SOURCES:
        shutil.copy(os.path.join(root, name), dst / name)
    return root, dst


def test_source_hash_ignores_comments_and_spacing(tmp_path):
    root, dst = _copy_sources(tmp_path)
    assert bench.kernel_source_hash(str(dst)) == bench.kernel_source_hash(root)
    f = dst / "combine.hip"
    text = f.read_text()
    f.write_text("// a new comment line\n/* and a\n   block */\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_source_hash(str(dst)) == bench.kernel_source_hash(root)


def test_source_hash_sees_code_changes(tmp_path):
    root, dst = _copy_sources(tmp_path)
    f = dst / "api.hip"
    text = f.read_text()
    assert "constexpr int kTargetBlocks = 512;" in text
    f.write_text(text.replace("constexpr int kTargetBlocks = 512;", "constexpr int kTargetBlocks = 513;"))
    assert bench.kernel_source_hash(str(dst)) != bench.kernel_source_hash(root)



def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr
