"""Host-side checks of bench.py: the algorithmic byte and flop counts its
roofline fractions divide by, the traffic lookup in the counter summaries,
and the one-GPU guard. No GPU is touched."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_decode_bytes_per_request_by_hand():
    # state tile in and out: 2 x 32 heads x 128 x 128 x 4 B; q and k: 2 x 16 x 128 x 2 B;
    # v and o: 2 x 32 x 128 x 2 B; g and beta: 2 x 32 x 4 B; two slot indices: 8 B
    want = 2 * 32 * 128 * 128 * 4 + 2 * 16 * 128 * 2 + 2 * 32 * 128 * 2 + 2 * 32 * 4 + 8
    assert want == 4_219_144
    assert bench.decode_bytes_per_request(16, 32, 128, 128, 2) == want
    assert 64 * want == 270_025_216


def test_verify_bytes_per_request_by_hand():
    # the source tile read once, 4 draft states written, 4 tokens of inputs and
    # outputs, 1 source and 4 destination indices
    per_token = 2 * 16 * 128 * 2 + 2 * 32 * 128 * 2 + 2 * 32 * 4
    want = 32 * 128 * 128 * 4 * 5 + 4 * per_token + 4 * 5
    assert bench.verify_bytes_per_request(4, 16, 32, 128, 128, 2) == want
    assert 64 * want == 677_446_912


def test_prefill_flops_and_bytes_per_token_by_hand():
    # per value head: W 2 C dk, U' and the intra output 4 C dv, U, the inter
    # output and the state advance 6 dk dv, the two Gram matrices shared by
    # G = 2 value heads 4 C dk / G
    per_head = 2 * 64 * 128 + 4 * 64 * 128 + 6 * 128 * 128 + 4 * 64 * 128 // 2
    assert per_head == 163_840
    assert bench.prefill_flops_per_token(32, 128, 128) == 32 * per_head
    assert abs(8192 * bench.prefill_flops_per_token(32, 128, 128) / 1e9 - 42.95) < 0.005
    assert bench.prefill_bytes_per_token(16, 32, 128, 128) == 24_832


def test_prefill_f32_flops_per_token_by_hand():
    # per token and value head at 128 x 128, C = 64, G = 2: K H, Q H and the
    # state advance 3 x 2 x 128 x 128; T R and P U over the lower triangle
    # including the diagonal, (64 + 1) / 2 tokens on average, 2 x 2 x 32.5 x 128;
    # K K^T and Q K^T over their lower triangles, 64 x 128 per token per key
    # head, halved over the two value heads; the solve 64^3 / 3 per chunk
    want = 3 * 2 * 128 * 128 + 2 * 2 * 32.5 * 128 + 2 * 64 * 128 / 2 + 64 ** 3 / 3 / 64
    assert bench.prefill_f32_flops_per_token_head(128, 128) == pytest.approx(want)
    assert want == pytest.approx(124_501.33, abs=0.01)


def test_traffic_lookup_follows_the_kernel_source(tmp_path, monkeypatch):
    csrc = tmp_path / "hybrid_linear_attention_02_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (csrc / "k.hip").write_text("kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench._src_hash("k.hip")
    (tmp_path / "profiles" / "p.txt").write_text(
        f"# summary\nkernel_source_sha256_16: {sha}\nhbm_bytes_per_launch: 12345\n")
    assert bench._traffic("p.txt", ["k.hip"], "hbm_bytes_per_launch") == 12345.0
    assert bench._traffic("missing.txt", ["k.hip"], "hbm_bytes_per_launch") is None
    assert bench._traffic("p.txt", ["k.hip"], "no_such_key") is None
    (csrc / "k.hip").write_text("kernel v2\n")            # the kernel changed since the counters
    assert bench._traffic("p.txt", ["k.hip"], "hbm_bytes_per_launch") is None


def test_committed_counter_summaries_carry_their_keys():
    for name, key in (("decode_counters_batched_b64_h32_128x128.txt", "hbm_bytes_per_launch"),
                      ("prefill_t8192_counters.md", "hbm_bytes_per_call"),
                      ("prefill_f32_t8192_counters.md", "hbm_bytes_per_call")):
        path = os.path.join(ROOT, "profiles", name)
        text = open(path).read()
        assert "kernel_source_sha256_16:" in text
        vals = dict(line.split(":", 1) for line in text.splitlines() if line.startswith(key))
        assert float(vals[key]) > 0


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True,
                       text=True, env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
