"""GPU: PKV_DEBUG=1 mode (device-data preconditions checked on the host).

The flag is read once per process, so the calls run in a child process
started with it set (tests/pkv_debug_child.py): valid writes, decode,
shared-prefix decode and multi-query attention match the oracle, and a
write with a slot used twice or a shared-prefix group whose member differs
from its first member is rejected with nothing launched.
"""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_debug_mode_checks_and_parity():
    env = dict(os.environ, PKV_DEBUG="1")
    env["PYTHONPATH"] = os.pathsep.join([os.path.dirname(HERE), env.get("PYTHONPATH", "")])
    print("child: tests/pkv_debug_child.py with PKV_DEBUG=1", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "pkv_debug_child.py")], env=env,
                       capture_output=True, text=True, timeout=150)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, r.stderr[-3000:]
    assert "PKV_DEBUG child: all passed" in r.stdout
