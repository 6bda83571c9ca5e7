"""The bf16 kernel variants selected by environment variables (read once per process by the
library), each in a child process of its own against the oracle: the cross-tile prefetch
switched off, the ping-pong kernel with K step 64 and two stages, the plain schedule in both
of its stage layouts, and n-fastest tile order."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))

VARIANTS = [
    {"MOE_FFN_PF": "0"},
    {"MOE_FFN_PIPE": "pp"},
    {"MOE_FFN_PIPE": "64x2"},
    {"MOE_FFN_PIPE": "32x4"},
    {"MOE_FFN_ORDER": "n"},
]


@pytest.mark.parametrize("env", VARIANTS, ids=lambda e: ",".join(f"{k}={v}" for k, v in e.items()))
def test_bf16_kernel_variant(env):
    print(f"\n[case] bf16 variant {env}", flush=True)
    child_env = dict(os.environ)
    for k in ("MOE_FFN_PF", "MOE_FFN_PIPE", "MOE_FFN_ORDER"):
        child_env.pop(k, None)
    child_env.update(env)
    p = subprocess.run([sys.executable, "-u", os.path.join(HERE, "_variant_child.py")], env=child_env,
                       capture_output=True, text=True, timeout=240)
    print(p.stdout[-3000:], p.stderr[-2000:] if p.returncode else "", flush=True)
    assert p.returncode == 0
