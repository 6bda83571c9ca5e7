"""Seeded synthetic inputs for the five MoE-layer workloads.

Recipe (all draws seeded; every tensor is reproducible on its own):

* Small host-side draws (activations, router logits, router matrix, skew permutation,
  Dirichlet combine weights) use numpy PCG64 seeded by
  ``SeedSequence([seed, config_id, tensor_id, expert_id])``, so they are identical on
  every machine.
* Stacked expert weights use one torch generator per tensor on the target device and are
  drawn in chunks of experts (at most 2^28 values per draw), so a 34 GB weight set takes a
  few dozen launches and well under a second in HBM. The host never needs the whole set: a
  check that wants expert ``e`` copies back exactly the bits the GPU holds.
* Values are rounded once, here, to the storage format the library consumes
  (fp32, bf16 round-to-nearest-even, OCP e4m3fn with power-of-two 1x128 block scales,
  OCP MXFP4 = e2m1 codes with an e8m0 scale per 32 reduction elements). Both the HIP
  path and the oracle read the same bits; rounding inputs is data preparation, not
  part of the layer.

tensor_id: 0 x, 1 logits / router matrix, 2 W_gate, 3 W_up, 4 W_down,
5 skew permutation, 6 Dirichlet combine weights, 7/8/9 shared-expert W_gate/W_up/W_down.

Storage layouts (row-major, dense):

* ``x``: [T, H] fp32 | bf16 | e4m3fn codes (uint8) with ``x_sf`` [T, H/128] fp32.
* ``logits``: [T, E] fp32, or a given routing ``topk_idx`` [T, K] int32 +
  ``topk_w`` [T, K] fp32.
* fp32 / bf16 weights: ``w_gate``, ``w_up`` [E, H, Hp] and ``w_down`` [E, Hp, H]:
  logical W[e][k][n] with the reduction index k first (g = x.Wg, y = h.Wd).
* MXFP4 weights are stored reduction-contiguous: gate/up bytes [E, Hp, H/2] with
  scales [E, H/32, Hp]; down bytes [E, H, Hp/2] with scales [E, Hp/32, H]. Byte j of
  row n holds logical k = 2j in its low nibble and k = 2j+1 in its high nibble; scale
  [b][n] covers k in [32b, 32b+32) of column n and means 2^(byte-127).
"""
from __future__ import annotations

import dataclasses
import json
import math
import os
from typing import Optional

import numpy as np
import torch

CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5")
SKEW_TARGETS = (0.2, 1.0, 10.0, 20.0)

_CONFIG_ID = {"c1": 0, "c2": 1, "c3": 2, "c4": 3, "c5": 4}
_BIAS_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "skew_bias.json")

# Full-size workload shapes.
_SHAPES = {
    # tiny fp32 layer, logits = x . Wr
    "c1": dict(T=64, H=128, Hp=64, E=8, K=2, act="f32", wgt="f32", out="f32", routing="xwr"),
    # bf16 layer, uniform routing
    "c2": dict(T=4096, H=2048, Hp=1024, E=64, K=6, act="bf16", wgt="bf16", out="bf16",
               routing="normal"),
    # one expert-parallel rank's balanced share: 48 local experts + 4 redundant slots
    "c3": dict(T=8192, H=7168, Hp=2048, E=52, K=8, act="bf16", wgt="bf16", out="bf16",
               routing="balanced"),
    # whole 384-expert layer on one GPU under skewed routing
    "c4": dict(T=8192, H=7168, Hp=2048, E=384, K=8, act="bf16", wgt="bf16", out="bf16",
               routing="skew"),
    # low-precision variant of c4 at maxvio 1
    "c5": dict(T=8192, H=7168, Hp=2048, E=384, K=8, act="fp8", wgt="mxfp4", out="bf16",
               routing="skew"),
}


@dataclasses.dataclass
class Workload:
    name: str
    T: int
    H: int
    Hp: int
    E: int
    K: int
    act: str
    wgt: str
    out: str
    x: torch.Tensor
    x_sf: Optional[torch.Tensor]
    logits: Optional[torch.Tensor]
    topk_idx: Optional[torch.Tensor]
    topk_w: Optional[torch.Tensor]
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    sf_gate: Optional[torch.Tensor]
    sf_up: Optional[torch.Tensor]
    sf_down: Optional[torch.Tensor]
    meta: dict
    # optional shared expert: bf16 (fp32 in an fp32 layer) weights [H, Hs], [H, Hs], [Hs, H]
    # and, for an fp8 layer, the bf16 activations it reads (the same draw as x, before fp8)
    ws_gate: Optional[torch.Tensor] = None
    ws_up: Optional[torch.Tensor] = None
    ws_down: Optional[torch.Tensor] = None
    x_shared: Optional[torch.Tensor] = None

    @property
    def Hs(self) -> int:
        return 0 if self.ws_gate is None else int(self.ws_gate.shape[1])

    @property
    def M(self) -> int:
        return self.T * self.K


# ----------------------------------------------------------------------------- seeding
def _seq(seed: int, cid: int, tid: int, eid: int = 0) -> np.random.SeedSequence:
    return np.random.SeedSequence([seed, cid, tid, eid])


def _np_rng(seed, cid, tid, eid=0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_seq(seed, cid, tid, eid)))


def _torch_gen(device, seed, cid, tid, eid=0) -> torch.Generator:
    state = int(_seq(seed, cid, tid, eid).generate_state(1, np.uint64)[0]) & ((1 << 63) - 1)
    g = torch.Generator(device=device)
    g.manual_seed(state)
    return g


# ----------------------------------------------------------------------------- formats
def _to_e4m3_blocked(x32: torch.Tensor):
    """fp32 [R, C] -> (e4m3fn codes uint8 [R, C], fp32 power-of-two scales [R, C/128]).

    Scale s = 2^ceil(log2(amax/448)) per 1x128 block, at least 2^-127 (the smallest e8m0
    value; amax = 0 -> s = 1), codes are x/s rounded to nearest even by torch's e4m3fn cast
    (|x/s| <= 448 by construction).
    """
    R, C = x32.shape
    blocks = x32.reshape(R, C // 128, 128)
    amax = blocks.abs().amax(dim=2)
    # amax = mant * 2^expo, mant in [0.5, 1), and 448 = 0.875 * 2^9: the smallest power of two
    # s with 448 s >= amax is 2^(expo - 9) when mant <= 0.875, else 2^(expo - 8)
    mant, expo = torch.frexp(amax)
    ce = (expo - 9 + (mant > 0.875).to(expo.dtype)).clamp_min(-127)
    scale = torch.where(amax > 0, torch.ldexp(torch.ones_like(amax), ce), torch.ones_like(amax))
    q = (blocks / scale.unsqueeze(2)).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(R, C), scale.to(torch.float32)


def _to_mxfp4(w_kn: torch.Tensor):
    """Logical fp32 W [..., Kred, N] -> (packed bytes [..., N, Kred/2], e8m0 scales
    [..., Kred/32, N]); leading dimensions (a chunk of experts) are carried through.

    OCP MX: per 32 reduction elements X = 2^(floor(log2 amax) - 2); element codes are
    e2m1 round-to-nearest-even of w/X, saturating at 6; amax = 0 -> scale byte 0.
    """
    *lead, Kred, N = w_kn.shape
    w = w_kn.transpose(-1, -2).reshape(*lead, N, Kred // 32, 32)
    amax = w.abs().amax(dim=-1)
    _, expo = torch.frexp(amax)                 # amax = m * 2^expo, m in [0.5, 1)
    shared = expo.to(torch.int32) - 1 - 2       # floor(log2 amax) - emax(e2m1)
    sbyte = torch.where(amax > 0, shared + 127, torch.zeros_like(shared)).clamp(0, 254)
    X = torch.ldexp(torch.ones_like(amax), sbyte.to(torch.int32) - 127)
    v = w / X.unsqueeze(-1)
    del w
    a = v.abs()
    # e2m1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; ">=" where a tie rounds up to the even code
    mag = (a > 0.25).to(torch.uint8)
    for bound, ge in ((0.75, True), (1.25, False), (1.75, True), (2.5, False), (3.5, True), (5.0, False)):
        mag += (a >= bound) if ge else (a > bound)
    del a
    code = mag | ((v < 0).to(torch.uint8) << 3)
    code = code.reshape(*lead, N, Kred // 2, 2)
    packed = code[..., 0] | (code[..., 1] << 4)
    return packed.contiguous(), sbyte.to(torch.uint8).transpose(-1, -2).contiguous()


# ----------------------------------------------------------------------------- routing inputs
def skew_beta(T: int, E: int, K: int, maxvio: float, lowp: bool = False) -> float:
    """Calibrated skew strength for a full-size shape (written by calibrate_skew.py)."""
    with open(_BIAS_FILE) as f:
        table = json.load(f)
    key = f"T{T}_E{E}_K{K}_maxvio{maxvio:g}" + ("_lowp" if lowp else "")
    if key not in table:
        raise KeyError(f"no calibrated skew for {key}; run workloads/calibrate_skew.py")
    return float(table[key]["beta"])


def skew_logits(T: int, E: int, beta: float, seed: int = 0, cid: int = 3) -> np.ndarray:
    """Router logits N(0,1) + a per-expert Zipf-shaped bias -beta*ln(1+rank(e)), fp32."""
    base = _np_rng(seed, cid, 1).standard_normal((T, E), dtype=np.float64).astype(np.float32)
    rank = _np_rng(seed, cid, 5).permutation(E)
    bias = (-beta * np.log1p(rank.astype(np.float64))).astype(np.float32)
    return (base + bias[None, :]).astype(np.float32)


# ----------------------------------------------------------------------------- weights
_CHUNK_VALUES = 1 << 28   # fp32 values drawn per launch (1 GiB)


def _weight_chunks(device, seed, cid, E, H, Hp):
    """(tensor index, first expert, fp32 chunk [n, rows, cols]) for gate, up and down, drawn
    N(0, 1/fan_in) from one generator per tensor, experts in order, a chunk of experts per
    draw (fan_in = H for gate/up, Hp for down)."""
    per = max(1, _CHUNK_VALUES // (H * Hp))
    for i, (tid, shp, std) in enumerate(((2, (H, Hp), 1.0 / math.sqrt(H)),
                                         (3, (H, Hp), 1.0 / math.sqrt(H)),
                                         (4, (Hp, H), 1.0 / math.sqrt(Hp)))):
        g = _torch_gen(device, seed, cid, tid)
        for e0 in range(0, E, per):
            n = min(per, E - e0)
            yield i, e0, torch.randn((n, *shp), generator=g, device=device).mul_(std)


def _draw_weights(device, seed, cid, E, H, Hp, wgt):
    """Stacked gate/up [E,H,Hp] and down [E,Hp,H] weights, N(0, 1/fan_in)."""
    if wgt in ("f32", "bf16"):
        dt = torch.float32 if wgt == "f32" else torch.bfloat16
        out = (torch.empty((E, H, Hp), dtype=dt, device=device),
               torch.empty((E, H, Hp), dtype=dt, device=device),
               torch.empty((E, Hp, H), dtype=dt, device=device))
        for i, e0, chunk in _weight_chunks(device, seed, cid, E, H, Hp):
            out[i][e0:e0 + chunk.shape[0]].copy_(chunk)      # bf16: round to nearest even
            del chunk
        return (*out, None, None, None)
    if wgt == "mxfp4":
        packed = (torch.empty((E, Hp, H // 2), dtype=torch.uint8, device=device),
                  torch.empty((E, Hp, H // 2), dtype=torch.uint8, device=device),
                  torch.empty((E, H, Hp // 2), dtype=torch.uint8, device=device))
        scales = (torch.empty((E, H // 32, Hp), dtype=torch.uint8, device=device),
                  torch.empty((E, H // 32, Hp), dtype=torch.uint8, device=device),
                  torch.empty((E, Hp // 32, H), dtype=torch.uint8, device=device))
        for i, e0, chunk in _weight_chunks(device, seed, cid, E, H, Hp):
            p, sc = _to_mxfp4(chunk)
            del chunk
            packed[i][e0:e0 + p.shape[0]].copy_(p)
            scales[i][e0:e0 + p.shape[0]].copy_(sc)
            del p, sc
        return (*packed, *scales)
    raise ValueError(wgt)


# ----------------------------------------------------------------------------- public
def make(*, T, H, Hp, E, K, act="bf16", wgt="bf16", out="bf16", routing="normal",
         beta=0.0, maxvio=None, seed=0, cid=99, device="cpu", name=None, shared_hs=0) -> Workload:
    """Draw one workload. ``routing`` is one of:

    * ``"xwr"``: logits = x . Wr computed once in fp64 and rounded to fp32, Wr N(0, 1/H);
    * ``"normal"``: logits N(0, 1);
    * ``"skew"``: logits N(0, 1) + Zipf-shaped per-expert bias of strength ``beta``;
    * ``"balanced"``: given routing topk_idx[t,k] = (K*t + k) mod E with Dirichlet(1)
      combine weights per token.
    """
    if act == "fp8" and H % 128:
        raise ValueError("fp8 activations need H % 128 == 0")
    x64 = _np_rng(seed, cid, 0).standard_normal((T, H), dtype=np.float64)
    x32 = torch.from_numpy(x64.astype(np.float32))
    x_sf = None
    if act == "f32":
        x = x32.to(device)
    elif act == "bf16":
        x = x32.to(torch.bfloat16).to(device)
    elif act == "fp8":
        q, s = _to_e4m3_blocked(x32)
        x, x_sf = q.to(device), s.to(device)
    else:
        raise ValueError(act)

    logits = topk_idx = topk_w = None
    if routing == "xwr":
        wr = _np_rng(seed, cid, 1).standard_normal((H, E), dtype=np.float64) / math.sqrt(H)
        xin = x32.to(torch.float64).numpy() if act == "f32" else None
        if xin is None:
            raise ValueError("xwr routing is defined for fp32 activations")
        logits = torch.from_numpy((xin @ wr).astype(np.float32)).to(device)
    elif routing == "normal":
        logits = torch.from_numpy(
            _np_rng(seed, cid, 1).standard_normal((T, E), dtype=np.float64).astype(np.float32)
        ).to(device)
    elif routing == "skew":
        logits = torch.from_numpy(skew_logits(T, E, beta, seed, cid)).to(device)
    elif routing == "balanced":
        t = np.arange(T, dtype=np.int64)[:, None]
        k = np.arange(K, dtype=np.int64)[None, :]
        topk_idx = torch.from_numpy(((K * t + k) % E).astype(np.int32)).to(device)
        gam = _np_rng(seed, cid, 6).standard_gamma(1.0, size=(T, K))
        topk_w = torch.from_numpy((gam / gam.sum(axis=1, keepdims=True)).astype(np.float32)).to(device)
    else:
        raise ValueError(routing)

    wg, wu, wd, sg, su, sd = _draw_weights(device, seed, cid, E, H, Hp, wgt)
    shared = {}
    if shared_hs:
        sdt = torch.float32 if act == "f32" else torch.bfloat16
        for key, tid, shp, std in (("ws_gate", 7, (H, shared_hs), 1.0 / math.sqrt(H)),
                                   ("ws_up", 8, (H, shared_hs), 1.0 / math.sqrt(H)),
                                   ("ws_down", 9, (shared_hs, H), 1.0 / math.sqrt(shared_hs))):
            g = _torch_gen(device, seed, cid, tid, 0)
            shared[key] = (torch.randn(shp, generator=g, device=device) * std).to(sdt)
        if act == "fp8":
            shared["x_shared"] = x32.to(torch.bfloat16).to(device)
    return Workload(name=name or f"custom_T{T}_H{H}_Hp{Hp}_E{E}_K{K}_{act}_{wgt}",
                    T=T, H=H, Hp=Hp, E=E, K=K, act=act, wgt=wgt, out=out,
                    x=x, x_sf=x_sf, logits=logits, topk_idx=topk_idx, topk_w=topk_w,
                    w_gate=wg, w_up=wu, w_down=wd, sf_gate=sg, sf_up=su, sf_down=sd,
                    meta=dict(routing=routing, beta=beta, maxvio_target=maxvio, seed=seed, cid=cid),
                    **shared)


def config(name: str, device="cpu", maxvio: Optional[float] = None, seed: int = 0,
           shared_hs: int = 0, act: Optional[str] = None) -> Workload:
    """One of the five named workloads at full size (c4 takes a maxvio target; c5 uses 1).
    ``shared_hs`` > 0 adds a shared expert of that intermediate size; ``act`` overrides the
    activation format (e.g. bf16 activations for the MXFP4 workload, quantised by the layer)."""
    s = dict(_SHAPES[name])
    if act is not None:
        s["act"] = act
    routing = s.pop("routing")
    beta = 0.0
    if routing == "skew":
        if name == "c5":
            maxvio = 1.0
        if maxvio is None:
            raise ValueError("c4 needs maxvio in %s" % (SKEW_TARGETS,))
        beta = skew_beta(s["T"], s["E"], s["K"], maxvio, lowp=(name == "c5"))
    label = name if maxvio is None or name == "c5" else f"{name}_maxvio{maxvio:g}"
    return make(**s, routing=routing, beta=beta, maxvio=maxvio, seed=seed,
                cid=_CONFIG_ID[name], device=device, name=label, shared_hs=shared_hs)


def with_maxvio(w: Workload, maxvio: float) -> Workload:
    """The skewed workload ``w`` (c4 shape) with the routing logits of another maxvio target:
    same activations and weights, logits N(0,1) + the bias calibrated for ``maxvio``."""
    if w.meta.get("routing") != "skew":
        raise ValueError("with_maxvio needs a skew-routed workload")
    beta = skew_beta(w.T, w.E, w.K, maxvio, lowp=(w.act == "fp8"))
    seed, cid = w.meta["seed"], w.meta["cid"]
    logits = torch.from_numpy(skew_logits(w.T, w.E, beta, seed, cid)).to(w.x.device)
    meta = dict(w.meta, beta=beta, maxvio_target=maxvio)
    return dataclasses.replace(w, logits=logits, meta=meta,
                               name=w.name.split("_maxvio")[0] + f"_maxvio{maxvio:g}")


def to_numpy_bits(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Host copy of a tensor's exact bits: bf16 -> uint16, fp32 -> float32, bytes -> uint8."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
