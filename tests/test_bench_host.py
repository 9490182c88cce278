"""Host-side pieces of bench.py: the comment-blind source hash that ties the
committed counter summary to the kernel sources it was taken on."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_text_drops_comments_and_blank_space_only():
    src = ('int a = 1;   // trailing\n/* block\n   comment */\tfloat b;\n'
           'const char* s = "not // a comment /* either */"; char q = \'"\'; char e = \'\\\'\';\n')
    assert bench.code_text(src) == ('int a = 1; float b; const char* s = "not // a comment /* either */"; '
                                    'char q = \'"\'; char e = \'\\\'\';')


def test_code_hash_ignores_comment_edits_but_not_code(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("// v1\n__global__ void k(float* x) { x[0] = 1.0f; }\n")
    b.write_text("/* v2, reworded */\n__global__ void k(float* x)\n{\n    x[0] = 1.0f;  // store\n}\n")
    c.write_text("__global__ void k(float* x) { x[0] = 2.0f; }\n")
    assert bench.code_hash(str(a)) == bench.code_hash(str(b)) != bench.code_hash(str(c))


def test_measured_traffic_only_for_the_profiled_shard():
    assert bench.measured_traffic("fused", 12345, "gpt2") is None
    assert bench.measured_traffic(None, 97_350_700, "gpt2") is None
    assert bench.measured_traffic("fused", 97_350_700, "no-such-workload") is None


def test_more_than_one_gpu_is_refused_before_any_device_work():
    """bench.py measures one rank's shard on one GPU; asked for more (by flag or
    by a distributed launcher's WORLD_SIZE) it exits with status 2 and says so,
    before importing torch or touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args], capture_output=True, text=True,
                           timeout=120, env=dict(os.environ, **env))
        assert r.returncode == 2, (args, env, r.returncode, r.stderr[-500:])
        assert "one GPU" in r.stderr and r.stdout == "", r.stderr[-500:]
