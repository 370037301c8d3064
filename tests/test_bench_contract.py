"""bench.py on a host without a GPU: more than one GPU is refused with a
message (the benchmark measures one GPU) before anything touches a device,
and the byte counts behind its bandwidth figures."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_lift_byte_counts_at_the_headline_shape():
    # Per residue at H=8, D=Dv=16, P=4, Q=8, Cz=64, R=2 in 16-bit: inputs
    # q,k,v 768 + points 768 + frames 24 + zl,zr 512 + mask 1 = 2073 B; the
    # method's rows per head: query and key rows of d_qk = 16+12+2+128 = 158
    # columns, a value row of d_v = 16+24+128 = 168, i.e. 8 x 484 x 2 = 7744 B.
    sys.path.insert(0, ROOT)
    import bench
    from rna_structure_amd.synth import make_config
    sh = make_config("sweep_16384")["shape"]
    assert bench.lift_method_bytes(sh, False) == sh.N * (2073 + 7744)
    assert bench.lift_method_bytes(sh, True) == sh.N * (2073 + 7744) + sh.N * sh.N
    # the lift's own rows share the pair factors among the heads: fewer bytes
    assert bench.lift_bytes(sh, False) < bench.lift_method_bytes(sh, False)
