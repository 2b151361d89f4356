"""bench.py's host-side contract: the single-GPU refusal and the algorithmic byte, flop and
source-digest bookkeeping behind its roofline figures (no GPU needed)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_prefill_bytes_headline_workload():
    # B4 T2048 H16 d128, bf16 q/k/v/o, fp32 beta, no decay, final state written, none read:
    # per token and head 4 x 128 x 2 bytes (q, k, v, o) + 4 (beta); per (sequence, head)
    # one 128 x 128 fp32 state
    tok, heads, d = 4 * 2048, 16, 128
    want = tok * heads * (4 * d * 2 + 4) + 4 * heads * d * d * 4
    assert bench.prefill_bytes(4, 2048, 16, 16, 128, gated=False, N=4, init=False) == want == 138_936_320


def test_prefill_bytes_counts_gates_initial_state_and_shared_qk():
    base = bench.prefill_bytes(2, 64, 2, 4, 16, gated=False, N=2, init=False)
    # g adds one fp32 per token and value head; an initial state adds one more state read
    assert bench.prefill_bytes(2, 64, 2, 4, 16, gated=True, N=2, init=False) == base + 2 * 64 * 4 * 4
    assert bench.prefill_bytes(2, 64, 2, 4, 16, gated=False, N=2, init=True) == base + 2 * 4 * 16 * 16 * 4
    # q and k are read per key head: doubling the value heads adds v, o, beta and states only
    wide = bench.prefill_bytes(2, 64, 2, 8, 16, gated=False, N=2, init=False)
    assert wide - base == 2 * 64 * 4 * (2 * 16 * 2 + 4) + 2 * 4 * 16 * 16 * 4


def test_prefill_flops_headline_workload():
    # algorithmic count, triangles exploited: per token and value head 6 d_k d_v against the
    # state plus C ((1 + 2/r) d_k + 2 d_v) for the masked Gram products (shared by the r
    # value heads of a q/k head) and T R, P Delta; 139,264 flop at r = 1, 131,072 at r = 2
    assert bench.prefill_flops(1, 1, 1, 128, 64) == 139_264
    assert bench.prefill_flops(1, 1, 2, 128, 64) == 2 * 131_072
    assert bench.prefill_flops(4 * 2048, 16, 16, 128, 64) == 18_253_611_008     # 18.25 GFLOP
    assert bench.prefill_flops(2 * 8192, 16, 32, 128, 64) == 68_719_476_736     # 68.72 GFLOP
    assert bench.prefill_flops(32768, 32, 32, 128, 64) == 146_028_888_064       # 146.03 GFLOP


def test_prefill_dense_tile_flops():
    # per chunk and value head: [K;Q] M (2 x 2C x D x D), T R and P Delta (2 x C x C x D each),
    # K^T Delta (2 x C x D x D); per chunk and key head K K^T and Q K^T (2 x 2 x C x C x D)
    C, D, chunks, hv, hqk = 64, 128, 4 * 2048 // 64, 16, 16
    per_v = 2 * 2 * C * D * D + 2 * 2 * C * C * D + 2 * C * D * D
    per_qk = 2 * 2 * C * C * D
    assert bench.prefill_flops_dense(4 * 2048, 16, 16, 128, 64) == chunks * (hv * per_v + hqk * per_qk)
    assert bench.prefill_flops_dense(4 * 2048, 16, 16, 128, 64) == 21_474_836_480
    assert bench.prefill_flops(4 * 2048, 16, 16, 128, 64) < bench.prefill_flops_dense(4 * 2048, 16, 16, 128, 64)


def test_decode_bytes():
    # per (sequence, head): the fp32 state read and written; per sequence q, k (key heads),
    # v, o (value heads) in bf16, beta and g in fp32
    n, h, d = 256, 32, 128
    want = n * h * d * d * 4 * 2 + n * (2 * h * d * 2 + 2 * h * d * 2 + 2 * h * 4)
    assert bench.decode_bytes(n, h, h, d) == want == 1_082_195_968


def test_traffic_is_used_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    digest = bench.source_digest()
    assert len(digest) == 16
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: digest)
    (prof / "traffic.json").write_text(json.dumps(
        {"source_digest": "0" * 16, "prefill_config2": {"bytes_per_call": 1},
         "decode_bytes_per_call": 2}))
    assert bench.load_traffic("prefill_config2") is None
    assert bench.load_traffic("decode_bytes_per_call") is None
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 16)
    assert bench.load_traffic("prefill_config2") == {"bytes_per_call": 1}
    assert bench.load_traffic("decode_bytes_per_call") == 2
    assert bench.load_traffic("no_such_entry") is None
    # the roofline block takes the counted bytes only from a matching digest
    blk = bench.prefill_roofline("prefill_config2", "k", 50.0, 138_936_320, 8192, 16, 16, 128)
    assert blk["roofline"]["traffic"] == 1
    assert abs(blk["roofline"]["frac"] - 138_936_320 / 50e-6 / 1e9 / 8000) < 1e-12
    assert blk["mfma"]["algorithmic_flops"] == 18_253_611_008


def test_counter_digest_ignores_comments_only():
    """The digest that keys the counters covers the code: comments and blank lines may change,
    a changed token may not."""
    src = "// a kernel\n__global__ void k(int* p) {  // one store\n\n    p[0] = 1; /* the\n  value */\n}\n"
    same = "/* reworded\n   header */\n__global__ void k(int* p) {\n    p[0] = 1;   // stores one\n}\n"
    other = "__global__ void k(int* p) {\n    p[0] = 2;\n}\n"
    assert bench.code_text(src) == bench.code_text(same)
    assert bench.code_text(src) != bench.code_text(other)
    assert "one store" not in bench.code_text(src) and "p[0] = 1;" in bench.code_text(src)


def test_chunk_bwd_bytes_and_flops():
    """The reverse pass's algorithmic bytes and flops, written out per term for the gated
    B1 H16 T2048 d128 shape: bf16 q, k, v, dL/do in; fp32 beta, g in; fp32 dq, dk, dv,
    dbeta, dg out; 401,408 flop per token-head."""
    tok, h, d = 2048, 16, 128
    reads = tok * h * d * 2 * 4 + tok * h * 4 * 2
    writes = tok * h * d * 4 * 3 + tok * h * 4 * 2
    assert bench.chunk_bwd_bytes(tok, h, h, d, gated=True, N=1, init=False, dfinal=False) == reads + writes
    assert bench.chunk_bwd_bytes(tok, h, h, d, gated=True, N=1, init=True, dfinal=True) == \
        reads + writes + 3 * h * d * d * 4
    assert bench.chunk_bwd_bytes(tok, h, h, d, gated=False, N=1, init=False, dfinal=False) == \
        reads + writes - 2 * tok * h * 4
    assert bench.chunk_bwd_flops(1, 1, 128, 64) == 401_408
    assert bench.chunk_bwd_flops(tok, h, d, 64) == tok * h * 401_408
