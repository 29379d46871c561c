"""The five benchmark workloads of the LoopVQ hot path, as plain data.

Geometry symbols follow the LoopVQ review (arXiv 2611.05304), section 3.1:
D head dim, T loop steps, T_c steps per block, G joint-vector length,
K = 2^b codebook entries, c = G / T_c channels per step per code.
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class LoopConfig:
    index: int                 # 1..5
    name: str
    layers: int
    B: int
    H_kv: int
    H_q: int
    D: int
    T: int
    T_c: int
    G: int
    K: int
    N: int                     # quantized context tokens (after the sinks)
    n_s: int                   # bf16 sink tokens
    rho_k: Tuple[float, ...]   # AR(1) coefficient per step transition (len T-1)
    rho_v: Tuple[float, ...]
    chunk_corr: float = 0.0    # equicorrelation inside each chunk of c channels
    tasq: bool = False         # channel pre-transform on keys
    decode_steps: int = 0      # decode calls after prefill (page encode every 8)
    page: int = 8
    theta: float = 1.0e4
    n_calib: int = 4096        # calibration joint vectors per codebook
    kmeans_iters: int = 50

    @property
    def c(self) -> int:
        return self.G // self.T_c

    @property
    def n_blk(self) -> int:
        return self.T // self.T_c

    @property
    def chunks(self) -> int:
        return self.D // self.c

    @property
    def gqa(self) -> int:
        return self.H_q // self.H_kv

    @property
    def bits(self) -> float:
        return (self.K.bit_length() - 1) / self.G

    def codes_per_layer(self) -> int:
        """Index bytes written by one layer's encode, K and V summed."""
        return 2 * self.B * self.H_kv * self.n_blk * self.N * self.chunks

    def units_per_layer(self) -> int:
        """(batch, kv-head, token, block) index rows read by one decode call per layer."""
        return self.B * self.H_kv * self.N * self.n_blk


def _ramp(a: float, b: float, n: int) -> Tuple[float, ...]:
    if n == 1:
        return (a,)
    return tuple(a + (b - a) * i / (n - 1) for i in range(n))


CONFIGS = (
    LoopConfig(1, "tiny single head", 1, 1, 1, 1, 128, 4, 4, 16, 256, 512, 4,
               (0.85,) * 3, (0.9,) * 3),
    LoopConfig(2, "0.5-bit looped slice", 1, 32, 16, 16, 128, 4, 4, 16, 256, 8192, 4,
               (0.85,) * 3, (0.9,) * 3),
    LoopConfig(3, "0.25-bit GQA", 1, 64, 8, 32, 128, 4, 4, 32, 256, 32768, 4,
               _ramp(0.69, 0.94, 3), _ramp(0.69, 0.94, 3), chunk_corr=0.16),
    LoopConfig(4, "deep loop", 1, 16, 16, 16, 128, 32, 4, 16, 256, 16384, 4,
               (0.85,) * 31, (0.9,) * 31),
    LoopConfig(5, "full stack with pre-transform", 24, 8, 16, 16, 128, 4, 4, 16, 256, 65536, 4,
               (0.85,) * 3, (0.9,) * 3, tasq=True, decode_steps=256),
)


def config_by_index(i: int) -> LoopConfig:
    return CONFIGS[i - 1]
