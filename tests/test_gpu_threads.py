"""The library called from several host threads at once: a fresh process
(its per-device launch-size cache empty) in which four threads step their
own shards on their own streams together must get, bit for bit, what the
same steps give taken one after another (tests/threads_child.py)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_four_threads_from_a_cold_start():
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "threads_child.py")], stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=110)
    print(r.stdout[-2000:], flush=True)
    assert r.returncode == 0 and "threads ok" in r.stdout, r.stdout[-2000:]
