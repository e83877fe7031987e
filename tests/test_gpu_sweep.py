"""GPU check of the offline sweep (the ahead-of-time search of "Helion in
vLLM: A Unified Route to Tunable Linear Kernels", "What the integration
changes" and "The costs behind the gains"): it sweeps one small FP8 shape,
writes a table keyed by this device's signature that the loader accepts,
and a second run given the same log resumes -- nothing measured again, the
same table -- also after the log lost its last records to a kill.
"""
import os

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def qll():
    import quantized_linear_layer_scaled_amd as q
    q.load_library()
    return q


def test_sweep_table_loads_and_resumes(qll, tmp_path):
    from quantized_linear_layer_scaled_amd import sweep
    out, log = tmp_path / "t.tsv", tmp_path / "t.log.jsonl"
    args = ["--ops", "fp8", "--shapes", "512x256", "--m", "1,64", "--reps", "2",
            "--out", str(out), "--log", str(log)]
    try:
        r = sweep.main(args)
        assert r["timed"] > 0 and r["entries"] == 2, r
        sig = qll.device_signature()
        assert qll.table_signature(str(out)) == sig
        assert qll.table_validate(str(out), sig) == (0, "")
        assert qll.init(str(out)) == 0 and qll.table_entries() == 2
        first = out.read_text().splitlines()
        for M in (1, 64):
            name, splits = qll.select("fp8", M, 512, 256)
            assert f"fp8 512 256 {M} {name} {splits}" in "\n".join(first)
        # resume from a complete log: nothing is measured again
        r2 = sweep.main(args)
        assert r2["timed"] == 0, r2
        assert out.read_text().splitlines()[3:] == first[3:]
        # a log cut short by a kill: the last records are measured again
        lines = log.read_text().splitlines()
        log.write_text("\n".join(lines[:-3]) + "\n" + lines[-3][:10])
        r3 = sweep.main(args)
        assert r3["timed"] == 3, r3
        assert qll.table_validate(str(out), sig) == (0, "")
    finally:
        qll.init()  # back to the shipped table
