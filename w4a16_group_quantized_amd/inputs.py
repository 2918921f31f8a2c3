"""Seeded synthetic inputs for the routed-expert W4A16 group-32 MoE layer.

This module draws random numbers and packs nothing by arithmetic: every packed
int32 word is drawn directly as a uniform 32-bit integer, so each of its eight
4-bit fields is an independent uniform value in [0, 15].  It holds none of the
layer's arithmetic and is the only code shared by the CPU oracle side and the
HIP side (both receive the arrays it returns).

Workload shapes follow the 512-expert, top-10, hidden-2560, moe-intermediate-640
geometry of "[Model][SM70] Adapt Qwen3.8 Flash Next NVFP4" (section
"Implemented route") and the TP4 per-rank shard with local intermediate 160 and
2-8 decode tokens of "[Perf][SM70] Narrow Qwen3.8 AWQ active grouped decode"
(section "Purpose"); the weight format is AWQ-style W4A16 with group size 32
along K ("[Model][SM70] Support Qwen3.8 Flash Next with PLE offload", section
"SM70 QSA prefill tuning").

Tensor layouts (N = output rows, K = reduction dim, G = K / 32):
  logits   float32 [T, E]
  x        float16 [T, H]
  w13_q    int32   [E, 2I, H/8]   w13 rows [0, I) are gate, [I, 2I) are up
  w13_s    float16 [E, 2I, H/32]
  w13_z    int32   [E, 2I/8, H/32]
  w2_q     int32   [E, H, I/8]
  w2_s     float16 [E, H, I/32]
  w2_z     int32   [E, H/8, I/32]
Weight nibble j of a word is bits [4j, 4j+4) and holds k = 8*word + j; zero
nibble j of a word holds row n = 8*word + j of that group.

Draw order: ``SeedSequence(seed).spawn(9)`` gives one PCG64 stream per tensor,
in the order logits, x, w13_q, w13_z, w13_s, w2_q, w2_z, w2_s, gate_w.  Every
tensor is filled row-major, so a smaller T is a row prefix of a larger T at the
same seed, and the weights of E + 1 experts are those of E experts followed by
one more.

The MoE block around the routed layer adds two inputs: the router's gate
projection gate_w float16 [E, H], drawn N(0, 1/H) so that the logits it makes
from N(0, 1) activations have unit variance like the logits drawn directly;
and a shared expert, stored as expert E of weight arrays of E + 1 experts.
"""

from __future__ import annotations

import dataclasses

import numpy as np

GROUP_SIZE = 32

_STREAMS = ("logits", "x", "w13_q", "w13_z", "w13_s", "w2_q", "w2_z", "w2_s", "gate_w")


@dataclasses.dataclass(frozen=True)
class MoEShape:
    """Geometry of one MoE layer call."""

    E: int
    top_k: int
    H: int
    I: int
    T: int
    zipf_s: float | None = None  # per-expert logit bias log(Zipf rank weight)

    def validate(self) -> None:
        if self.E < 1 or not 1 <= self.top_k <= self.E:
            raise ValueError(f"bad E/top_k: {self}")
        if self.H % GROUP_SIZE or self.I % GROUP_SIZE:
            raise ValueError(f"H and I must be multiples of {GROUP_SIZE}: {self}")
        if self.T < 0:
            raise ValueError(f"T must be >= 0: {self}")


# Named workloads (sizes only; the recipe is the same for all of them).
WORKLOADS: dict[str, MoEShape] = {
    "tiny_e8_k2_h256_i128_t4": MoEShape(E=8, top_k=2, H=256, I=128, T=4),
    "decode_e512_k10_h2560_i640_t8": MoEShape(E=512, top_k=10, H=2560, I=640, T=8),
    "decode_shard_e512_k10_h2560_i160_t8": MoEShape(E=512, top_k=10, H=2560, I=160, T=8),
    "prefill_e512_k10_h2560_i640_t1024": MoEShape(E=512, top_k=10, H=2560, I=640, T=1024),
    "prefill_zipf_e512_k10_h2560_i640_t4096": MoEShape(
        E=512, top_k=10, H=2560, I=640, T=4096, zipf_s=1.1
    ),
}


def _rngs(seed: int) -> dict[str, np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(_STREAMS, children)}


def zipf_logit_bias(E: int, s: float) -> np.ndarray:
    """log of the normalised Zipf(s) weight of rank e+1, for expert e (fp64)."""
    ranks = np.arange(1, E + 1, dtype=np.float64)
    w = ranks ** (-s)
    return np.log(w / w.sum())


def _words(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint32).view(np.int32)


def _scales(rng: np.random.Generator, shape) -> np.ndarray:
    u = rng.random(size=shape, dtype=np.float32)
    return (np.float32(0.002) + np.float32(0.018) * u).astype(np.float16)


def make_activations(shape: MoEShape, seed: int = 0) -> dict[str, np.ndarray]:
    """Router logits [T,E] fp32 and activations x [T,H] fp16."""
    shape.validate()
    r = _rngs(seed)
    logits = r["logits"].standard_normal((shape.T, shape.E), dtype=np.float32)
    if shape.zipf_s is not None:
        bias = zipf_logit_bias(shape.E, shape.zipf_s).astype(np.float32)
        logits = (logits + bias[None, :]).astype(np.float32)
    x = r["x"].standard_normal((shape.T, shape.H), dtype=np.float32).astype(np.float16)
    return {"logits": np.ascontiguousarray(logits), "x": np.ascontiguousarray(x)}


def make_weights(shape: MoEShape, seed: int = 0) -> dict[str, np.ndarray]:
    """Packed W4 weights, packed zeros and fp16 scales for w13 and w2."""
    shape.validate()
    E, H, I, g = shape.E, shape.H, shape.I, GROUP_SIZE
    r = _rngs(seed)
    return {
        "w13_q": _words(r["w13_q"], (E, 2 * I, H // 8)),
        "w13_z": _words(r["w13_z"], (E, 2 * I // 8, H // g)),
        "w13_s": _scales(r["w13_s"], (E, 2 * I, H // g)),
        "w2_q": _words(r["w2_q"], (E, H, I // 8)),
        "w2_z": _words(r["w2_z"], (E, H // 8, I // g)),
        "w2_s": _scales(r["w2_s"], (E, H, I // g)),
    }


def make_inputs(shape: MoEShape, seed: int = 0) -> dict[str, np.ndarray]:
    """All inputs of one layer call: activations plus weights."""
    out = make_activations(shape, seed)
    out.update(make_weights(shape, seed))
    return out


def make_gate_weight(shape: MoEShape, seed: int = 0) -> np.ndarray:
    """Router gate projection [E, H] fp16, N(0, 1/H)."""
    shape.validate()
    r = _rngs(seed)["gate_w"]
    w = r.standard_normal((shape.E, shape.H), dtype=np.float32) * np.float32(1.0 / np.sqrt(shape.H))
    return np.ascontiguousarray(w.astype(np.float16))


def make_block_inputs(shape: MoEShape, seed: int = 0, shared: bool = True) -> dict[str, np.ndarray]:
    """Inputs of the MoE block: x, the gate projection and the weights of the E
    routed experts, followed by the shared expert's (index E) when ``shared``.
    The drawn logits are kept too, for calls that take logits directly."""
    out = make_activations(shape, seed)
    out.update(make_weights(dataclasses.replace(shape, E=shape.E + int(shared)), seed))
    out["gate_w"] = make_gate_weight(shape, seed)
    return out
