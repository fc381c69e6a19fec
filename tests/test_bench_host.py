"""bench.py on the host: the one-GPU guard, and the committed rocprofv3 records it reads are
those of the current kernel sources (bench.py reports HBM traffic only from counters taken on
the sources it runs). Every record under profiles/ names the kind of kernel it covers and the
fingerprint (bench.source_fingerprint) of that kernel's source, the shared device header and the
C ABI header."""
import glob
import json
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_fingerprint_covers_the_shared_headers(tmp_path, monkeypatch):
    for kind in bench.SOURCES:
        fp = bench.source_fingerprint(kind)
        assert re.fullmatch(r"[0-9a-f]{64}", fp)
    assert bench.source_fingerprint("fwd") != bench.source_fingerprint("bwd")
    csrc = tmp_path / "csrc"
    inc = tmp_path / "include"
    csrc.mkdir()
    inc.mkdir()
    for name in ("attn_fwd.hip", "attn_common.h"):
        (csrc / name).write_bytes(open(os.path.join(bench.CSRC, name), "rb").read())
    (inc / "attn.h").write_bytes(open(os.path.join(ROOT, "include", "attn.h"), "rb").read())
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.source_fingerprint("fwd")
    for path in (csrc / "attn_fwd.hip", csrc / "attn_common.h", inc / "attn.h"):
        old = path.read_bytes()
        # a code change in any of the three files changes it ...
        path.write_bytes(old + b"\nstatic const int fingerprint_probe = 1;\n")
        assert bench.source_fingerprint("fwd") != base, path
        # ... an edit of comments or blank space does not
        path.write_bytes(b"/* a comment\n   on two lines */\n" + old.replace(b"\n", b"\n\n") +
                         b"\n// another\n")
        assert bench.source_fingerprint("fwd") == base, path
        path.write_bytes(old)
    assert bench.source_fingerprint("fwd") == base


def test_code_only_strips_comments_and_layout():
    src = b"int a; /* x\n y */ int  b;  // z\n\tint c;\n"
    assert bench.code_only(src) == b"int a; int b; int c;"


def test_traffic_records_match_the_kernel_sources():
    assert bench.traffic_for("long_gqa") is not None
    assert bench.traffic_for("long_gqa", backward=True) is not None


def test_every_profile_names_the_current_sources():
    files = sorted(glob.glob(os.path.join(PROFILES, "*")))
    assert files
    for path in files:
        text = open(path).read()
        if path.endswith(".json"):
            fps = [json.loads(text)["source_fingerprint"]]
            fps = [(f["kind"], f["sha256"]) for f in fps]
        else:
            fps = re.findall(r"fingerprint \((\w+)\)\s+([0-9a-f]{64})", text)
        assert fps, path
        for kind, sha in fps:
            assert sha == bench.source_fingerprint(kind), (path, kind)
