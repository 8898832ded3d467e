"""Host logic of the benchmark: the byte counts behind its roofline fractions,
against totals written out here from the workload definitions (d = 128; one
token-head moves q, k, v and o in bf16 and g, beta in fp32: 3*256 + 256 + 8 =
1032 bytes; a state is 128 x 128 fp32 = 65536 bytes)."""
import bench

TOKEN_HEAD = 3 * 128 * 2 + 128 * 2 + 8
STATE = 128 * 128 * 4


def test_token_head_and_state_sizes():
    assert TOKEN_HEAD == 1032 and STATE == 65536


def test_decode_bytes():
    # 64 sequences x 32 heads: every state read and written, plus one token
    assert bench.DEC_STATE_BYTES == 2 * 64 * 32 * STATE == 268_435_456
    assert bench.DEC_ALG_BYTES == 64 * 32 * (2 * STATE + TOKEN_HEAD) == 270_548_992


def test_prefill_bytes():
    # 4 x 4096 tokens, 16 heads, initial and final states
    assert bench.PRE_IO_BYTES == 16384 * 16 * TOKEN_HEAD + 2 * 4 * 16 * STATE == 278_921_216
    assert bench.io_min_bytes(2) == bench.PRE_IO_BYTES
    # the chunk-parallel form adds L and M written and read, fixed written and
    # read: 6 states per chunk-head, 4096 chunk-heads
    assert bench.PRE_CHUNK_HEADS == 4 * 64 * 16 == 4096
    assert bench.PRE_CP_BYTES == bench.PRE_IO_BYTES + 4096 * 6 * STATE == 1_889_533_952


def test_other_prefill_workloads():
    # varlen: 32768 tokens, 32 heads, 8 sequences with initial and final states
    assert bench.io_min_bytes(3) == 32768 * 32 * TOKEN_HEAD + 2 * 8 * 32 * STATE == 1_115_684_864
    # long: 131072 tokens, 4 heads, one sequence without an initial state
    assert bench.io_min_bytes(4) == 131072 * 4 * TOKEN_HEAD + 4 * STATE == 541_327_360


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_cp_form_bytes():
    # the chunk-parallel form adds 6 states per chunk-head: prefill 4096 chunk-heads,
    # long 2048 chunks x 4 heads
    assert bench.cp_form_bytes(2) == bench.PRE_CP_BYTES
    assert bench.cp_form_bytes(4) == bench.io_min_bytes(4) + 8192 * 6 * STATE == 3_762_552_832
    # one fixup step per (chunk, head): M_c and L_c read, fixed[c] written
    assert bench.FIX_STEP_BYTES == 3 * STATE
    # L and M returned by the scan schedule: written once, plus the factors
    # (13,312 B written, read back with 32 KiB of q and k rows) per chunk-head
    assert bench.lm_request_bytes(2) == bench.PRE_IO_BYTES + 4096 * (2 * STATE + 13312 + 13312 + 32768)


def test_records_are_used_only_on_their_sources(tmp_path, monkeypatch):
    import json
    src = tmp_path / "k.hip"
    src.write_text("kernel v1")
    (tmp_path / "profiles").mkdir()
    rec = {"sources": {"k.hip": bench._sha256(str(src))}, "hbm_bytes_per_launch": 7}
    (tmp_path / "profiles" / "r.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_record("r.json")["hbm_bytes_per_launch"] == 7
    src.write_text("kernel v2")
    assert bench.load_record("r.json") is None
    assert bench.load_record("missing.json") is None


def test_only_choices():
    assert bench.parse(["--only", "fixup_long"]).only == "fixup_long"
    assert bench.parse([]).only is None and bench.parse([]).steps >= 20
