"""Model shapes and decoding settings of the synthetic workloads.

Pure data: no arithmetic of the method lives here.  The five named workloads follow
the model families on the LoopSpec page (arXiv:2609.17184, section 3.1: Ouro with a
full loop depth of 4, Raven/Huginn with 32) and the CopyLoop page (copy-suffix
proposals with shallow screening).  Shapes beyond what the pages state (layer
internals, MLP width of the Huginn-shaped model, tied head) are readings listed in
the design notes; the smaller `mini-*` shapes keep the same head dimensions so the
same kernels are exercised at sizes a CPU reference finishes in seconds.
"""

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class ModelCfg:
    name: str
    V: int                 # vocabulary
    d: int                 # model width
    n_heads: int
    head_dim: int
    F: int                 # SwiGLU hidden width
    L: int                 # layers in the shared loop block B
    R: int                 # full loop depth
    dtype: str             # "f32" or "bf16": storage precision of weights, GEMM inputs and KV
    readout_depths: Tuple[int, ...]   # D: depths at which C is evaluated (always contains R)
    L_pre: int = 0         # extra layers in the prelude P (Huginn/Raven family)
    L_coda: int = 0        # extra layers in the coda C (Huginn/Raven family)
    rope_theta: float = 10000.0
    norm_eps: float = 1e-6
    init_std: float = 0.02

    def __post_init__(self):
        assert self.n_heads * self.head_dim == self.d
        assert self.head_dim % 2 == 0
        assert self.R in self.readout_depths
        assert all(1 <= r <= self.R for r in self.readout_depths)
        assert tuple(sorted(self.readout_depths)) == tuple(self.readout_depths)


@dataclass(frozen=True)
class DecodeCfg:
    greedy: bool
    T: float = 1.0
    top_p: float = 1.0
    d1: int = 2
    d2: Optional[int] = None          # second (residual) proposal depth; None = single proposal
    gate: bool = True
    residual: bool = True             # False: Table 3's non-residual second proposal (p_d2, x1 masked)
    max_branches: int = 8
    prompt_len: int = 32
    new_tokens: int = 64
    seed_w: int = 0                   # weight seed (PCG64)
    seed_p: int = 1                   # prompt seed (PCG64)
    seed_s: int = 2                   # sampling key (Philox4x32-10)
    copy: bool = False                # copy-suffix proposals with shallow screening (CopyLoop)
    screen_depth: int = 4
    tau: float = 0.1
    copy_max_cands: int = 16
    copy_max_len: int = 8
    prompt_kind: str = "uniform"      # "uniform" or "segments" (repeated 64-token segments + noise)


@dataclass(frozen=True)
class Workload:
    key: str
    model: ModelCfg
    decode: DecodeCfg
    description: str = ""


TINY = ModelCfg("tiny-fp32", V=512, d=128, n_heads=4, head_dim=32, F=512, L=2, R=4, dtype="f32",
                readout_depths=(2, 4))
OURO_14 = ModelCfg("ouro-1.4b-shaped", V=49152, d=2048, n_heads=16, head_dim=128, F=5632, L=24, R=4,
                   dtype="bf16", readout_depths=(2, 3, 4))
OURO_26 = replace(OURO_14, name="ouro-2.6b-shaped", L=48)
HUGINN = ModelCfg("huginn-3.5b-shaped", V=65536, d=5280, n_heads=55, head_dim=96, F=17920, L=4, R=32,
                  dtype="bf16", readout_depths=(8, 16, 32), L_pre=2, L_coda=2)
HUGINN_COPY = replace(HUGINN, name="huginn-3.5b-shaped-copy", readout_depths=(4, 32))

WORKLOADS = {
    "C1": Workload("C1", TINY, DecodeCfg(greedy=True, d1=2, d2=None, max_branches=4, prompt_len=32, new_tokens=64),
                   "tiny looped decoder, fp32, greedy, single proposal at depth 2"),
    "C2": Workload("C2", OURO_14, DecodeCfg(greedy=False, T=1.0, top_p=0.9, d1=2, d2=3, max_branches=8,
                                            prompt_len=512, new_tokens=256),
                   "Ouro-1.4B-shaped, bf16, T=1.0 top-p 0.9, proposals at depths 2 and 3"),
    "C3": Workload("C3", OURO_26, DecodeCfg(greedy=True, d1=2, d2=3, max_branches=8, prompt_len=1024, new_tokens=512),
                   "Ouro-2.6B-shaped, bf16, greedy, proposals at depths 2 and 3"),
    "C3s": Workload("C3s", OURO_26, DecodeCfg(greedy=False, T=0.7, top_p=0.9, d1=2, d2=3, max_branches=8,
                                              prompt_len=1024, new_tokens=512),
                    "Ouro-2.6B-shaped, bf16, T=0.7 top-p 0.9, proposals at depths 2 and 3"),
    "C4": Workload("C4", HUGINN, DecodeCfg(greedy=True, d1=8, d2=16, max_branches=16, prompt_len=2048, new_tokens=512),
                   "Huginn-3.5B-shaped, bf16, greedy, proposals at depths 8 and 16"),
    "C5": Workload("C5", HUGINN_COPY, DecodeCfg(greedy=False, T=1.0, top_p=0.95, d1=4, d2=None, max_branches=16,
                                                prompt_len=8192, new_tokens=512, copy=True, screen_depth=4,
                                                tau=0.1, prompt_kind="segments"),
                   "Huginn-shaped stress: 8192-token repetitive context, copy-suffix proposals screened at depth 4"),
}

# Small shapes with the real head dimensions, used where a CPU reference must finish quickly.
MINI_OURO = ModelCfg("mini-ouro", V=1024, d=256, n_heads=2, head_dim=128, F=704, L=2, R=4, dtype="bf16",
                     readout_depths=(2, 3, 4))
MINI_HUGINN = ModelCfg("mini-huginn", V=1024, d=192, n_heads=2, head_dim=96, F=640, L=2, R=8, dtype="bf16",
                       readout_depths=(2, 4, 8), L_pre=2, L_coda=2)
TINY_V8 = replace(TINY, name="tiny-v8", V=8)

SMALL = {
    "tiny": Workload("tiny", TINY, DecodeCfg(greedy=True, d1=2, max_branches=4, prompt_len=16, new_tokens=24)),
    "tiny-sample": Workload("tiny-sample", replace(TINY, readout_depths=(2, 3, 4)),
                            DecodeCfg(greedy=False, T=1.0, top_p=0.9, d1=2, d2=3,
                                                           max_branches=8, prompt_len=16, new_tokens=24)),
    "mini-ouro": Workload("mini-ouro", MINI_OURO, DecodeCfg(greedy=False, T=1.0, top_p=0.9, d1=2, d2=3,
                                                            max_branches=8, prompt_len=24, new_tokens=24)),
    "mini-ouro-greedy": Workload("mini-ouro-greedy", MINI_OURO, DecodeCfg(greedy=True, d1=2, d2=3, max_branches=8,
                                                                          prompt_len=24, new_tokens=24)),
    "mini-huginn": Workload("mini-huginn", MINI_HUGINN, DecodeCfg(greedy=True, d1=2, d2=4, max_branches=16,
                                                                  prompt_len=20, new_tokens=16)),
    "mini-huginn-sample": Workload("mini-huginn-sample", MINI_HUGINN,
                                   DecodeCfg(greedy=False, T=1.0, top_p=0.9, d1=2, d2=4, max_branches=16,
                                             prompt_len=20, new_tokens=16)),
    "mini-huginn-copy": Workload("mini-huginn-copy", replace(MINI_HUGINN, readout_depths=(2, 8)),
                                 DecodeCfg(greedy=False, T=1.0, top_p=0.95, d1=2, max_branches=16, prompt_len=96,
                                           new_tokens=24, copy=True, screen_depth=2, tau=0.0,
                                           prompt_kind="segments")),
}


def get(key: str) -> Workload:
    if key in WORKLOADS:
        return WORKLOADS[key]
    return SMALL[key]
