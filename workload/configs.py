"""The five workload shapes.

Shapes follow the pages' benchmark setup: block size 8 (seven drafts per
verification; myaiexp.com "DFlash 2", § コツ; latenode.com FAQ), 16 kept
candidates per position (tamsi.dev, § "L'idée, sans le papier"), concurrency
1 / 8 / 32 (latenode.com, § "El desacuerdo empieza…"), sampling at
temperature 1.0 (latenode.com FAQ), a five-layer drafter (tamsi.dev,
§ "L'idée…") and the context-copy regime with long accepts
(postsingularityinstitute.com, § Résumé).
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    B: int            # requests
    T: int            # block slots (slot 0 = last verified token)
    D: int            # hidden size
    V: int            # vocabulary
    r: int            # selector rank
    verify: str       # "greedy" | "sample" | "mixed" (first half greedy)
    logits: str       # "draft_plus_noise" | "context_copy"
    noise_sd: float = 1.0     # target = draft logits + N(0, noise_sd^2)
    plant_alpha: float = 0.0  # margin planted toward a random token per draft row
    agree_frac: float = 0.8   # context copy: fraction of slots where target argmax = draft top-1
    temperature: float = 1.0
    top_k: int = 0            # sampled rows: 0 = full softmax, else top-k then top-p filtering
    top_p: float = 1.0
    anchored: bool = False    # selector anchored on each block's slot-0 token
    sampled_path: bool = False  # sampled rows: the draft path is drawn (proposal q), verified against q
    fused_target_head: bool = False  # verified from target hidden states through the LM head (no target logits)
    fused_tap_proj: bool = False  # conv taps projected from x inside the conv call (never written)
    K: int = 16
    L: int = 5        # conv layer calls per cycle
    seed: int = 0
    w_sd: float = 0.02

    @property
    def P(self):
        return self.T - 1

    @property
    def M(self):
        return self.B * self.P


# plant_alpha = 9.75 gives ~0.85 per-slot agreement of target argmax with the
# draft's top-1 at V = 151936, D = 5120, i.e. a mean n_emit near 4.8 at block 8.
CONFIGS = {
    "c1_tiny": Config("c1_tiny", B=1, T=8, D=256, V=4096, r=32, verify="greedy",
                      logits="draft_plus_noise", noise_sd=0.5),
    "c2_b1": Config("c2_b1", B=1, T=8, D=5120, V=151936, r=192, verify="greedy",
                    logits="draft_plus_noise", noise_sd=1.0, plant_alpha=9.75),
    "c3_b8": Config("c3_b8", B=8, T=8, D=5120, V=151936, r=192, verify="sample",
                    logits="draft_plus_noise", noise_sd=1.0, plant_alpha=9.75),
    "c4_b32": Config("c4_b32", B=32, T=8, D=5120, V=151936, r=192, verify="mixed",
                     logits="draft_plus_noise", noise_sd=1.0, plant_alpha=9.75),
    "c5_stress": Config("c5_stress", B=32, T=16, D=5120, V=262144, r=192, verify="greedy",
                        logits="context_copy", plant_alpha=12.0, agree_frac=0.8),
}


def get_config(config_name, **overrides):
    """A named configuration, optionally with fields replaced (e.g. a rename
    so that a reshaped variant draws its own random streams)."""
    import dataclasses
    cfg = CONFIGS[config_name]
    return dataclasses.replace(cfg, **overrides) if overrides else cfg
