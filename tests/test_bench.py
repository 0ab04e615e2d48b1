"""bench.py host logic (no GPU): the one-GPU contract and the lookup of the
measured HBM traffic in the committed profile summaries."""
import os
import subprocess
import sys

import bench

HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(HERE, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _tree(tmp_path, csrc_text, profile_lines):
    (tmp_path / "linear_attention_fwd_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "linear_attention_fwd_amd" / "csrc" / "k.hip").write_text(csrc_text)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "p.md").write_text("\n".join(profile_lines) + "\n")
    return str(tmp_path)


def test_measured_traffic_follows_the_source_digest(tmp_path):
    import hashlib
    digest = hashlib.sha256(b"kernel v1").hexdigest()[:16]
    root = _tree(tmp_path, "kernel v1", [
        "# summary",
        f"traffic: kda_chunk_rec_kernel bytes_per_launch=1189377751 csrc_sha256={digest}",
        "traffic: kda_chunk_prep_kernel bytes_per_launch=5 csrc_sha256=0000000000000000",
    ])
    assert bench.measured_traffic(root, "kda_chunk_rec_kernel") == 1189377751
    # a summary taken from other sources, and a kernel with none, give no figure
    assert bench.measured_traffic(root, "kda_chunk_prep_kernel") is None
    assert bench.measured_traffic(root, "kda_decode_kernel") is None
    # once the kernel sources change, the old figure no longer applies
    (tmp_path / "linear_attention_fwd_amd" / "csrc" / "k.hip").write_text("kernel v2")
    assert bench.measured_traffic(root, "kda_chunk_rec_kernel") is None


def test_decode_byte_counts():
    """State bytes: the fp32 state read and written per (sequence, head); total
    adds 8D + 2 input bytes per replayed or window token and 2D output bytes per
    output, per head."""
    D = 128
    assert bench.decode_state_bytes(512, 96) == 512 * 96 * D * D * 4 * 2
    acc = [0, 4, 2]
    tokens = (0 + 1) + (4 + 1) + (2 + 1)
    H = 5
    assert bench.decode_total_bytes(acc, H) == \
        bench.decode_state_bytes(3, H) + H * tokens * (8 * D + 2) + 3 * H * 2 * D
    # a window of W2 drafts adds their inputs and outputs
    assert bench.decode_total_bytes(acc, H, W2=4) - bench.decode_total_bytes(acc, H) == \
        3 * 4 * H * (8 * D + 2) + 3 * 4 * H * 2 * D
