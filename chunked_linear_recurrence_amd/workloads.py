"""The synthetic workloads the library is tested and measured on.

Each entry fixes a problem shape, the storage dtype of the activations, the input value
distributions and the seed.  The shapes follow the page
"分块推理：解锁循环模型并行计算，实现长序列高效处理": chunk length Q = 256 for Mamba-2
(§4.1), and a vertical-segment length V with V >= Q for the layer stack (§3.2, §4.2).
The value distributions are the usual Mamba-2 ones (dt a softplus-clamped step, A a
negative per-head rate) and stand in for a trained model's activations.
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str                 # "f32" or "bf16": storage of x, dt, B, C, y
    dt_min: float = 1e-3
    dt_max: float = 0.1
    init: str = "zero"         # "zero" or "normal" (std init_std)
    init_std: float = 0.1
    layers: int = 1            # > 1: a stack of layers with a residual between them
    segment: int = 0           # vertical segment length V (stack only)
    residual: bool = False
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def nchunks(self) -> int:
        return (self.seqlen + self.chunk - 1) // self.chunk

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    @property
    def act_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32_L256", batch=1, seqlen=256, nheads=2, headdim=16, dstate=16,
                 ngroups=1, chunk=64, dtype="f32",
                 notes="tiny fp32 layer; the oracle finishes it instantly"),
        Workload("mamba2_130m_layer_b2_L2048", batch=2, seqlen=2048, nheads=24, headdim=64,
                 dstate=128, ngroups=1, chunk=256, dtype="bf16",
                 notes="one Mamba-2-130M-shaped layer (d_model 768, expand 2)"),
        Workload("throughput_b8_L4096_h32", batch=8, seqlen=4096, nheads=32, headdim=64,
                 dstate=128, ngroups=1, chunk=256, dtype="bf16", init="normal",
                 notes="batched throughput layer with a random initial state"),
        Workload("long_context_b1_L131072_h48", batch=1, seqlen=131072, nheads=48, headdim=64,
                 dstate=128, ngroups=1, chunk=256, dtype="bf16", dt_max=1e-2,
                 notes="one 128K-token sequence, 512 chunks in the state pass"),
        Workload("vertical_stack_24x_L32768_V2048", batch=1, seqlen=32768, nheads=24,
                 headdim=64, dstate=128, ngroups=1, chunk=256, dtype="bf16", layers=24,
                 segment=2048, residual=True,
                 notes="24-layer stack run as 2048-token vertical segments"),
    ]
}

# The order in which the workloads are listed (small parity case first).
ORDER = list(WORKLOADS)

# The workload the benchmark line is measured on: the 128K-token single sequence.
BENCH_WORKLOAD = "long_context_b1_L131072_h48"

