"""The five synthetic PFA workloads: shapes, dtypes, keep schedules, shifts, seeds.

Pure data. Both the HIP path and the fp64 oracle read these definitions; the
method's arithmetic lives in neither this file nor ``inputs.py``.

Sources for the numbers (Progressive Focused Transformer paper notes, CVPR 2025):
  * window 32x32 ("Framework" section);
  * keep schedule [1024, 256, 128, 64, 32, 16] ("Progressive focused resource
    allocation" section), read here as per attention layer within one chain;
  * SwinIR-like shifted windows on alternate layers ("Loss / training strategy"
    section), read as: first layer unshifted, then every second layer shifted by
    half a window.
The global individualized-attention workload follows "From Local Windows to
Adaptive Candidates via Individualized Exploratory" (individualized attention
paragraph: an index matrix I of N x k global candidates per token; the Fig. 7
description: a dense local plus sparse global region centred on each token).
"""

from dataclasses import dataclass, field
from typing import List

PFT_SCHEDULE = [1024, 256, 128, 64, 32, 16]
PFT_SHIFTS = [0, 16, 0, 16, 0, 16]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    H: int
    W: int
    d: int
    win: int                 # window side w (N = w*w); 0 = global mode (N = H*W)
    dtype: str               # "f32" or "bf16" for Q/K/V; I is int32, A and O fp32
    scale: float             # multiply N(0,1) draws by this before rounding to dtype
    seed_base: int
    blocks: int = 1          # independent chains (each with its own Q/K/V per layer)
    K: List[int] = field(default_factory=list)       # kept count per layer
    shifts: List[int] = field(default_factory=list)  # cyclic shift per layer
    k_global: int = 0        # global mode: candidates per token
    dilation: int = 0        # global mode: dilation of the 8x8 initial neighbourhood

    @property
    def N(self) -> int:
        return self.win * self.win if self.win else self.H * self.W

    @property
    def n_windows(self) -> int:
        return (self.H // self.win) * (self.W // self.win) if self.win else 1

    @property
    def n_wh(self) -> int:
        """Window-heads per layer call."""
        return self.B * self.heads * self.n_windows

    @property
    def layers(self) -> int:
        return len(self.K) if self.win else 1

    def pairs(self, layer: int) -> int:
        """Candidate pairs (i, j in I^{l-1}(i)) evaluated by one layer call."""
        if not self.win:
            return self.B * self.heads * self.N * self.k_global
        k_prev = self.N if layer == 0 else self.K[layer - 1]
        return self.n_wh * self.N * k_prev

    def qkv_seed(self, block: int, layer: int, which: str) -> int:
        return self.seed_base + 100 * block + 10 * layer + {"q": 0, "k": 1, "v": 2}[which]

    @property
    def index_seed(self) -> int:
        return self.seed_base + 9


TINY = Workload("tiny_16x16_d16_f32", B=1, heads=1, H=16, W=16, d=16, win=16, dtype="f32",
                scale=1.0, seed_base=1000, K=[256, 64, 32], shifts=[0, 0, 0])
MAP256 = Workload("map256x256_h6_d32_f32", B=1, heads=6, H=256, W=256, d=32, win=32, dtype="f32",
                  scale=1.0, seed_base=2000, K=list(PFT_SCHEDULE), shifts=list(PFT_SHIFTS))
PATCH64 = Workload("patch64x64_b32_h6_d32_bf16", B=32, heads=6, H=64, W=64, d=32, win=32,
                   dtype="bf16", scale=32 ** -0.5, seed_base=3000, K=list(PFT_SCHEDULE),
                   shifts=list(PFT_SHIFTS))
MAP640 = Workload("map640x384_h6_d32_bf16_6blocks", B=1, heads=6, H=384, W=640, d=32, win=32,
                  dtype="bf16", scale=1.0, seed_base=4000, blocks=6, K=list(PFT_SCHEDULE),
                  shifts=list(PFT_SHIFTS))
GLOBAL64 = Workload("global64x64_h6_d32_k64_bf16", B=1, heads=6, H=64, W=64, d=32, win=0,
                    dtype="bf16", scale=1.0, seed_base=5000, k_global=64, dilation=4)

ALL = [TINY, MAP256, PATCH64, MAP640, GLOBAL64]
BY_NAME = {w.name: w for w in ALL}
