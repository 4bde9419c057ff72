"""bench.py's command-line contract on the host: more than one GPU is refused
with exit status 2 and a message, before anything touches a GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True, timeout=120,
                       cwd=ROOT, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _profile_bench_commands():
    """Every bench.py invocation quoted in the profile summaries, as argument lists."""
    import glob
    import re
    import shlex

    found = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*"))):
        for line in open(path, encoding="utf-8"):
            m = re.search(r"bench\.py((?: +[^ `|>]+)*)", line)
            if m and "rocprofv3" in line:
                found.append((os.path.basename(path), shlex.split(m.group(1))))
    return found


def test_profile_commands_parse():
    """The summaries under profiles/ name the command that made them: each must
    still be a valid bench.py command line (no option renamed or removed)."""
    sys.path.insert(0, ROOT)
    try:
        import bench
    finally:
        sys.path.remove(ROOT)
    cmds = _profile_bench_commands()
    names = {name for name, _ in cmds}
    assert {"sdpa_decode_wg8_llama_128k.md", "sdpa_prefill_llama_int4.md", "sdpa_partial_valu_llama_128k.md"} <= names
    for name, args in cmds:
        try:
            bench.build_parser().parse_args(args)
        except SystemExit:
            raise AssertionError("%s: bench.py %s no longer parses" % (name, " ".join(args)))
