"""Host-side checks of bench.py: the single-GPU guard and the algorithmic byte counts its
roofline divides by (recomputed here from the tensor shapes, element by element)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr or "multi-GPU" in r.stderr
    assert r.stdout.strip() == ""


def _prefill_tensors(T, H, dk, dv, N, h0, gate, o_bytes=2):
    """Bytes of every tensor one chunk call reads or writes once (bf16 activations)."""
    b = 2 * T * H * dk * 2          # q, k (bf16)
    b += T * H * dv * 2             # v (bf16)
    b += T * H * 4                  # beta (fp32)
    b += T * H * dv * o_bytes       # o (bf16 in the roofline's accounting; fp32 as written)
    b += N * H * dk * dv * 4        # final state (fp32)
    if h0:
        b += N * H * dk * dv * 4    # initial state
    if gate == "g":
        b += T * H * dk * 4         # g [T, H, dk] fp32
    elif gate == "z":
        b += T * H * dk * 2 + H * 4 + H * dk * 4   # z (bf16), A_log [H], dt_bias [H, dk]
    elif gate == "head":
        b += T * H * 4              # g [T, H] fp32
    return b


@pytest.mark.parametrize("T,H,dk,dv,N,h0", [(4096, 96, 128, 128, 1, False),
                                             (32768, 96, 128, 128, 8, True),
                                             (64, 1, 16, 16, 1, False)])
def test_prefill_byte_counts(T, H, dk, dv, N, h0):
    for ob in (2, 4):
        assert bench.prefill_step_bytes(T, H, dk, dv, N, h0, ob) == \
            _prefill_tensors(T, H, dk, dv, N, h0, "g", ob)
        assert bench.gdn_step_bytes(T, H, dk, dv, N, h0, ob) == \
            _prefill_tensors(T, H, dk, dv, N, h0, "head", ob)
        got = bench.gated_step_bytes(T, H, dk, dv, N, h0, ob)
        want = _prefill_tensors(T, H, dk, dv, N, h0, "z", ob)
        # A_log and dt_bias are a few KB per call; the count may leave them out
        assert abs(got - want) <= H * 4 + H * dk * 4


def test_headline_prefill_bytes():
    # 1540 B per (token, head) with o counted as bf16 (the roofline's accounting), 1796 B
    # with the fp32 o the call writes; plus 64 KiB of final state per head
    assert bench.prefill_step_bytes(4096, 96, 128, 128, 1, False) == 4096 * 96 * 1540 + 96 * 65536
    assert bench.prefill_step_bytes(4096, 96, 128, 128, 1, False) == 611844096
    assert bench.prefill_step_bytes(4096, 96, 128, 128, 1, False, 4) == 4096 * 96 * 1796 + 96 * 65536
    # the packed and long workloads: 4.945 GB (h0 and hT of 8 sequences) and 19.38 GB
    assert round(bench.prefill_step_bytes(32768, 96, 128, 128, 8, True) / 1e9, 3) == 4.945
    assert round(bench.prefill_step_bytes(131072, 96, 128, 128, 1, False) / 1e9, 2) == 19.38


def test_useful_flops():
    # 2 [3 dk dv + (C/2)(3 dk + 2 dv)] = 139264 per (token, head) at d = 128, C = 64
    assert bench.prefill_useful_flops(1, 1, 128, 128, 64) == 139264
    assert round(bench.prefill_useful_flops(4096, 96, 128, 128, 64) / 1e9, 2) == 54.76


def test_decode_byte_counts():
    B, H, dk, dv = 64, 96, 128, 128
    want = B * H * (2 * dk * dv * 4        # state read and written (fp32)
                    + 2 * dk * 2 + dv * 2  # q, k, v (bf16)
                    + dk * 4 + 4           # g [dk] and beta (fp32)
                    + dv * 4)              # o (fp32)
    assert bench.decode_step_bytes(B, H, dk, dv) == want
    C = 2 * dk + dv
    conv = B * H * 3 * C * 2 * 2 + H * C * 4 * 2   # raw rows, caches read + written, weights
    assert bench.decode_conv_step_bytes(B, H, dk, dv) == want + conv


def test_epilogue_bytes():
    T, H, dv = 4096, 96, 128
    assert bench.epilogue_bytes(T, H, dv) == T * H * dv * (4 + 2 + 2)   # o fp32, gate, y bf16


def test_stale_traffic_summary_is_ignored(tmp_path, monkeypatch):
    """A counter summary taken on another kernel source gives no traffic figure."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "chunk_prefill_traffic.md").write_text(
        "source_digest: 0000000000000000\nhbm_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "channel_gated_delta_amd").symlink_to(os.path.join(ROOT, "channel_gated_delta_amd"))
    assert bench.measured_traffic("chunk", "prefill") is None
    digest = bench.kernel_source_digest("chunk")
    (prof / "chunk_prefill_traffic.md").write_text(
        "source_digest: %s\nhbm_bytes_per_launch: 123\n" % digest)
    assert bench.measured_traffic("chunk", "prefill") == 123.0
