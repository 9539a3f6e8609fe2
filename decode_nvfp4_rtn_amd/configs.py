"""Workload definitions: synthetic layer shapes of the five measured configurations.

Shapes follow the model families the pages name (Qwen3-8B and Gemma3-12B in
the Disaggregated Quantization speed comparison; a 27B model in its
time-to-first-token measurement).  Y = X W^T with X [M, K] and W [N, K].
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Layer:
    name: str
    n: int
    k: int


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    kind: str              # "prefill" (NVFP4 W4A4), "w4a16" or "lut2"
    layers: tuple
    ms: tuple              # token counts / batch sizes
    act: str = "bf16"      # activation dtype
    outliers: str = None   # None, "channels", "elements"
    out: str = "bf16"      # timed output dtype
    notes: str = ""


QWEN3_LAYERS = (
    Layer("qkv", 6144, 4096),
    Layer("o_proj", 4096, 4096),
    Layer("gate_up", 24576, 4096),
    Layer("down", 4096, 12288),
)

BIG27_LAYERS = (
    Layer("qkv", 7168, 5120),
    Layer("o_proj", 5120, 5120),
    Layer("gate_up", 34816, 5120),
    Layer("down", 5120, 17408),
)

GEMMA3_LAYERS = (
    Layer("3840x3840", 3840, 3840),
    Layer("30720x3840", 30720, 3840),
    Layer("3840x15360", 3840, 15360),
)

TINY_PREFILL = Config(1, "tiny-prefill", "prefill", (Layer("tiny", 256, 512),), (64,),
                      act="f32", outliers="channels", out="f32")
TINY_DECODE = Config(1, "tiny-decode", "w4a16", (Layer("tiny", 256, 512),), (1,),
                     act="bf16", out="f32")
QWEN3_PREFILL = Config(2, "qwen3-8b-prefill", "prefill", QWEN3_LAYERS, (8192,),
                       outliers="channels")
QWEN3_DECODE = Config(3, "qwen3-8b-decode-w4a16", "w4a16", QWEN3_LAYERS, (1, 4, 8, 16, 32))
BIG27_PREFILL = Config(4, "27b-prefill", "prefill", BIG27_LAYERS, (4096, 16384, 32768),
                       outliers="elements")
GEMMA3_LUT2 = Config(5, "gemma3-12b-decode-lut2", "lut2", GEMMA3_LAYERS, (1, 8, 16))

ALL = (TINY_PREFILL, TINY_DECODE, QWEN3_PREFILL, QWEN3_DECODE, BIG27_PREFILL, GEMMA3_LUT2)
