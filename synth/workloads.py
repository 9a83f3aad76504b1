"""Named synthetic workloads: method settings plus the generator recipe for each.

tiny     B=1,   V=1024 fp32,   R=60,  D=8,  K=W=8,  m=1, T=1, draft = 4 n, target = draft + 0.5 n'
b8       B=8,   V=32000 bf16,  R=60,  D=8,  K=W=10, m=1, T=1, Zipf a=1.1 + n, target + 0.7 n', 64 steps
headline B=32,  V=128256 bf16, R=60,  D=8,  K=W=10, m=1, T in {0.6, 1.0}, as b8, 128 steps
smart    B=64,  V=151936 bf16, SMART keep rule, top-k 8, budget 128, D<=10, alpha=1,
         C_draft = 0.02|T| ms, C_verify = 0.01 (exp(0.004 |T|^1.3) - 1) ms, m=1, T=1
stress   B=256, V=128256 bf16, R=128, D=10, K=W=12, m in {0,1,3}, T=1; trees b < 128 Zipf
         a=1.5 (peaked), b >= 128 a=0.8 (flat); target + 0.7 n'
n, n' are the generator's unit-variance Irwin-Hall jitters (see synth.hip).
"""
import dataclasses

from . import BF16, F32, Params, tables

TOPR, SMART = 0, 1


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    V: int
    dtype: int
    R: int = 60
    D: int = 8
    K: int = 10
    W: int = 0
    m: int = 1
    probe: int = 1
    T: float = 1.0
    trunc: int = 128
    mode: int = TOPR
    budget: int = 128
    alpha: float = 1.0
    lam: float = 0.0
    gamma: float = 0.0
    delta: float = 0.0
    rho: float = 1.0
    eps_m0: float = 1e-6
    steps: int = 1
    zipf: tuple = ()
    split: int = 0
    draft_scale: float = 1.0
    sigma: float = 0.7
    gen_seed: int = 0x5EED
    order: int = 0  # 0: the probe first (RheoSampling), 1: the probe last (RRSw baseline)

    def params(self):
        return Params(self.V, self.dtype, len(self.zipf), self.split if self.split else self.B,
                      self.draft_scale, self.sigma, self.gen_seed)

    def tables(self):
        return tables(self.V, list(self.zipf))

    @property
    def width(self):
        return self.W if self.W > 0 else self.K

    @property
    def maxpar(self):
        return self.budget if self.mode == SMART else self.width

    @property
    def n_nodes(self):
        """Rows of the emitted tree, root included."""
        return (self.budget if self.mode == SMART else self.R) + 1

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", B=1, V=1024, dtype=F32, R=60, D=8, K=8, W=8, m=1, T=1.0, steps=1,
                     zipf=(), draft_scale=4.0, sigma=0.5),
    "b8": Workload("b8", B=8, V=32000, dtype=BF16, R=60, D=8, K=10, m=1, T=1.0, steps=64,
                   zipf=(1.1,), sigma=0.7),
    "headline": Workload("headline", B=32, V=128256, dtype=BF16, R=60, D=8, K=10, m=1, T=1.0,
                         steps=128, zipf=(1.1,), sigma=0.7),
    "smart": Workload("smart", B=64, V=151936, dtype=BF16, mode=SMART, K=8, budget=128, D=10,
                      alpha=1.0, lam=0.02, gamma=0.01, delta=0.004, rho=1.3, m=1, T=1.0,
                      zipf=(1.1,), sigma=0.7),
    "headline_fp32": Workload("headline_fp32", B=32, V=128256, dtype=F32, R=60, D=8, K=10, m=1,
                              T=1.0, steps=128, zipf=(1.1,), sigma=0.7),
    "stress": Workload("stress", B=256, V=128256, dtype=BF16, R=128, D=10, K=12, m=1, T=1.0,
                       zipf=(1.5, 0.8), split=128, sigma=0.7),
}


def get(name, **kw):
    w = WORKLOADS[name]
    return w.replace(**kw) if kw else w
