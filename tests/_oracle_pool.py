"""Worker of the process pool that evaluates the oracle's expert FFN on selected rows of
MXFP4 experts (decoding an MXFP4 expert is the slow part of a full-size check; the workers
run it in parallel). Imports only numpy and the oracle, so spawned workers start quickly
and never touch the GPU."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import moe_oracle as O  # noqa: E402


def mxfp4_expert_rows(job):
    """job = (e, xr [n, H] float64, (gate, up, down packed bytes), (their e8m0 scales),
    fp8_requant) -> (e, h [n, Hp], y [n, H], h block scales [n, Hp/128] or None) from the
    oracle's decoders and expert FFN; with fp8_requant, h is the requantised value."""
    e, xr, packed, scales, fp8 = job
    wg, wu, wd = (O.decode_mxfp4(p, s) for p, s in zip(packed, scales))
    h, y = O.expert_ffn(xr, wg, wu, wd, fp8_requant=fp8)
    hs = None
    if fp8:
        h, hs = O.requant_fp8_1x128(h)
    return e, h, y, hs
