"""The five MoE-layer workloads as seeded synthetic recipes.

Each workload fixes the layer shape (T tokens, hidden H, expert intermediate
I, E experts, top-k) and the input recipe:
  x      ~ N(0, 1) rounded to bf16            (stream X, tokens t0..t0+T-1)
  W_r    ~ N(0, 0.02) rounded to bf16, [H][E] (stream WR)
  W_e,m  ~ N(0, 0.02) fp32, then NVFP4        (stream 16 + 3e + m)
  bias   = Zipf-style popularity bias on the router logits,
           b[e] = -beta * 1.1 * ln(1 + pi(e)), pi a seeded permutation;
           beta is set per workload so the routing statistic the workload
           states comes out (measured with these generators, seed 0):
             concurrent decode T=64:   ~600 distinct experts (beta 0.10: 601)
             speculative verify T=256: per-expert counts 0..~40 (0.29: max 39)
             prefill chunk T=8192:     up to ~4x the mean count (0.17: 4.00x)
           The tiny and single-user cases carry no bias.
The latent workloads are K3's LatentMoE block (lightseek.org, "Kimi K3
optimization on GB300", part I): tokens of the hidden width H_model = 7168,
experts in the 3584-wide routed latent with I = 3072 ([p2] "The model, as
the serving system sees it"), and the two projections
  P_down [H_model][H], P_up [H][H_model] ~ N(0, 0.02) rounded to bf16
                                          (streams PROJ_DOWN, PROJ_UP);
the router reads the hidden state, so W_r is [H_model][E].
The normal variate is the Irwin-Hall sum of twelve uniforms (synth_def.h).
"""
from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int = 896
    k: int = 16
    beta: Optional[float] = None  # Zipf bias strength; None = no bias
    seed: int = 0
    zipf_s: float = 1.1
    H_model: Optional[int] = None  # latent block: hidden width (the experts run at H)

    @property
    def P(self):
        return self.T * self.k


WORKLOADS = {
    "tiny": Workload("tiny", T=8, H=512, I=256),
    "decode_1": Workload("decode_1", T=1, H=7168, I=2048),
    "decode_64": Workload("decode_64", T=64, H=7168, I=2048, beta=0.10),
    "verify_256": Workload("verify_256", T=256, H=7168, I=2048, beta=0.29),
    "prefill_8192": Workload("prefill_8192", T=8192, H=7168, I=2048, beta=0.17),
    # the latent block at K3's shapes (NEXT: the pages' actual model)
    "latent_tiny": Workload("latent_tiny", T=8, H=512, I=256, H_model=1024),
    "latent_decode_1": Workload("latent_decode_1", T=1, H=3584, I=3072, H_model=7168),
    "latent_decode_64": Workload("latent_decode_64", T=64, H=3584, I=3072, beta=0.10, H_model=7168),
    "latent_prefill_8192": Workload("latent_prefill_8192", T=8192, H=3584, I=3072, beta=0.17, H_model=7168),
}


def bias_for(w: Workload):
    import synth
    if w.beta is None:
        return None
    return synth.zipf_bias(w.seed, w.E, w.beta, w.zipf_s)
