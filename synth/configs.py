"""Layer shapes of the five synthetic workloads.

The shapes follow the architecture table of "Kolibri Pre-Training from
Scratch: UniBPE, Hybrid Attention and Exact Quantile Balancing" (§2, "Kolibri
at a Glance": Kolibri width 2560, 384 routed experts, top-6, routed hidden
512, one shared expert; Kolibri Origin width 2048, 128 experts, top-8, hidden
768) and the toy layer of its running example (§6.1: 4 tokens, 4 experts,
top-2).  The German guide "Kolibri 1 im Detail" (section on routing and
SwiGLU experts) fixes the 2560 -> 512 -> 2560 expert shape for the shared
expert as well.

This module holds shapes and distribution parameters only; no arithmetic of
the method lives here.
"""
from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class LayerConfig:
    name: str            # short workload name
    seed: int            # root of the SeedSequence tree for this workload
    N: int               # tokens in the batch (T on the pages)
    d: int               # model width
    E: int               # routed experts
    K: int               # experts chosen per token
    h: int               # routed expert hidden width
    h_shared: int        # shared expert hidden width
    n_shared: int        # number of always-on shared experts (0 or 1)
    recompute_bias: bool  # run one EQB update on the batch and re-route with it
    beta_std: float      # std of the incoming correction bias (0 -> all zeros)
    offset: Optional[str]  # per-expert logit offset: None, "toy_collapse", "zipf1.2"
    x_std: float = 1.0
    w_std: float = 0.02
    dtype: str = "bf16"  # storage type of x and all weights

    @property
    def r(self) -> int:
        """Per-expert fair share used by the expert quantile, floor(N*K/E)."""
        return (self.N * self.K) // self.E

    def describe(self) -> dict:
        return {"workload": self.name, "N": self.N, "d": self.d, "E": self.E,
                "K": self.K, "h": self.h, "h_shared": self.h_shared,
                "n_shared": self.n_shared, "eqb_recompute": self.recompute_bias,
                "offset": self.offset}


CONFIGS = {
    # Toy layer of the running example: routing collapsed onto experts 0 and 1.
    "toy": LayerConfig("toy", 1001, N=4, d=64, E=4, K=2, h=32, h_shared=32,
                       n_shared=1, recompute_bias=True, beta_std=0.0,
                       offset="toy_collapse", dtype="fp32"),
    # Kolibri-Origin-shaped layer, uniform expert popularity, bias given.
    "origin": LayerConfig("origin", 1002, N=4096, d=2048, E=128, K=8, h=768,
                          h_shared=768, n_shared=1, recompute_bias=False,
                          beta_std=0.1, offset=None),
    # Kolibri-shaped prefill batch with one EQB update over the batch.
    "prefill": LayerConfig("prefill", 1003, N=16384, d=2560, E=384, K=6, h=512,
                           h_shared=512, n_shared=1, recompute_bias=True,
                           beta_std=0.1, offset=None),
    # Kolibri-shaped decode-sized batch: bound by expert weight reads.
    "decode": LayerConfig("decode", 1004, N=64, d=2560, E=384, K=6, h=512,
                          h_shared=512, n_shared=1, recompute_bias=False,
                          beta_std=0.1, offset=None),
    # Kolibri-shaped large batch with Zipf(1.2) expert popularity, EQB update.
    "skewed": LayerConfig("skewed", 1005, N=65536, d=2560, E=384, K=6, h=512,
                          h_shared=512, n_shared=1, recompute_bias=True,
                          beta_std=0.1, offset="zipf1.2"),
}

ORDER = ["toy", "origin", "prefill", "decode", "skewed"]


def scaled(cfg: LayerConfig, N: int, name: Optional[str] = None) -> LayerConfig:
    """Same layer with a different token count (for small parity cases)."""
    from dataclasses import replace
    return replace(cfg, N=N, name=name or f"{cfg.name}_N{N}")
