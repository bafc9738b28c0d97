"""The measurement probes behind the decode kernel's secondary ceilings (tests/probes/).

lds_rates prints the wave-instruction rates of the LDS gathers and atomics the decode
kernel streams through; stream_rate the read rate of a plain kernel over the same code
tiles.  These runs check that both complete and print rates in the physically possible
range; the figures themselves are read from their output.
"""
import os
import re
import subprocess

import pytest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes")


def _run(name: str) -> str:
    exe = os.path.join(HERE, name)
    if not os.path.exists(exe):
        pytest.skip(f"{name} not built (tests/probes/build_probes.py)")
    print(f"[probe] {name}", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.gpu
def test_lds_rates_probe():
    out = _run("lds_rates")
    clk = {m.group(1): float(m.group(2)) for m in re.finditer(r"^(ds_\w+)\s.*\(\s*([\d.]+) clk", out, re.M)}
    assert set(clk) == {"ds_read_b32", "ds_read_b64", "ds_add_u32", "ds_add_u64", "ds_add_f32"}
    # one wave instruction moves at most 64 x 8 bytes; no LDS serves that in under a clock
    assert all(v > 1.0 for v in clk.values()), clk
    # the fp32 LDS add is the slow form the histogram's fixed point avoids
    assert clk["ds_add_f32"] > 4 * clk["ds_add_u32"], clk


@pytest.mark.gpu
def test_stream_rate_probe():
    out = _run("stream_rate")
    gbs = float(re.search(r"([\d.]+) GB/s", out).group(1))
    assert 500.0 < gbs < 8000.0, out
    # one CU streams faster when most others are idle than its share of the full grid's rate
    per = {int(g): float(r) for g, r in re.findall(r"(\d+) work-groups: .*?([\d.]+) GB/s per work-group", out)}
    assert set(per) == {256, 128, 32, 8}, out
    assert per[8] > per[256], out


@pytest.mark.gpu
@pytest.mark.parametrize("shape,groups", [("32k", 256), ("gqa", 256), ("ragged", 512)])
def test_decode_timeline_probe(shape, groups):
    """The per-phase and per-step timeline of one decode call (libpqkv_timeline.so, stamps at
    the phase boundaries and at every step of every wave), and the XCD of every work-group."""
    import sys

    script = os.path.join(HERE, "decode_timeline.py")
    if not os.path.exists(os.path.join(HERE, "libpqkv_timeline.so")):
        pytest.skip("libpqkv_timeline.so not built (tests/probes/build_probes.py)")
    print(f"[probe] decode_timeline --shape {shape}", flush=True)
    r = subprocess.run([sys.executable, script, "--shape", shape], capture_output=True, text=True, timeout=300)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    m = re.search(r"XCC_ID == work-group id mod 8: (\d+) of (\d+)", r.stdout)
    assert m and int(m.group(2)) == groups, r.stdout
    # the XCD-aware mapping assumes the hardware deals work-groups out round-robin
    assert int(m.group(1)) == int(m.group(2)), r.stdout
