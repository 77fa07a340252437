"""Host-side contract of bench.py (no GPU): one GPU only, option validation, and the byte
accounting of the FP8 main cache ("What the cache costs, checked four ways": 64 bf16 rotary
dims + 448 FP8 dims = 576 bytes per entry)."""
import json
import os
import subprocess
import sys

from sparse_long_context_csa_amd import accounting as acc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_unknown_cache_format_is_refused():
    r = _bench("--kv-format", "fp6")
    assert r.returncode == 2 and "invalid choice" in r.stderr


def test_fp8_entry_bytes():
    assert acc.FP8_ENTRY_BYTES == 576
    kw = dict(B=4, n_vis=262144, m=4, D=512, H=64, H_I=64, d_I=128, K=512, W=128)
    bf = acc.decode_step_bytes(**kw)
    f8 = acc.decode_step_bytes(**kw, entry_bytes=acc.FP8_ENTRY_BYTES)
    # the selected entries shrink from 1,024 to 576 bytes; the window rows stay bf16; the
    # stored new entry too
    assert bf.gather - f8.gather == 4 * 512 * (1024 - 576)
    assert bf.compress - f8.compress == 4 * (1024 - 576)
    assert bf.keys == f8.keys


def test_fp4_entry_bytes():
    # "DeepSeek-V4.1-Flash's KV-Cache Compression, Checked Down to the Byte", section 4: 288 B
    assert acc.FP4_ENTRY_BYTES == 288
    kw = dict(B=4, n_vis=262144, m=4, D=512, H=64, H_I=64, d_I=128, K=512, W=128)
    bf = acc.decode_step_bytes(**kw)
    f4 = acc.decode_step_bytes(**kw, entry_bytes=acc.FP4_ENTRY_BYTES)
    assert bf.gather - f4.gather == 4 * 512 * (1024 - 288)
    assert bf.compress - f4.compress == 4 * (1024 - 288)
