"""Build (--build) or run (NAME [args]) one of the probes in this directory."""

import os
import subprocess
import sys

from exact_tiled_attention_flash_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


def exe_path(name):
    return os.path.join(B.BUILD, "probe_" + name)


def build_all():
    os.makedirs(B.BUILD, exist_ok=True)
    for f in sorted(os.listdir(HERE)):
        if f.endswith(".hip"):
            name = f[:-4]
            cmd = [B.hipcc()] + B.HIPFLAGS + [os.path.join(HERE, f), "-o", exe_path(name)]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (f, r.stderr))
            print("built", exe_path(name))


def main(argv):
    if not argv or argv[0] == "--build":
        build_all()
        return 0
    exe = exe_path(argv[0])
    if not os.path.exists(exe):
        raise SystemExit("%s is not built: run python -m exact_tiled_attention_flash_amd.probes --build" % exe)
    return subprocess.run([exe] + argv[1:]).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
