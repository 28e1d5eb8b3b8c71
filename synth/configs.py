"""The five workload shapes of the substitute-draft step.

Shapes follow the model families the SubSpec pages evaluate (Qwen2.5 7B / 32B and
Llama 3.1 8B, Review "SubSpec: Using the Target Model's Own Low-Bit Shadow as Its
Draft Model" §3.2 and §3.5), with random-init weights in place of trained ones.
The pages fix the deep-narrow tree (depth 48, Review §6.3 and §3.7) and the
2048-token static KV cache (Review §5.2, Critique 8).
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    H: int                 # hidden size (GEMM K for qkv / gate_up)
    I: int                 # MLP intermediate size (0: no MLP, single linear)
    nq: int                # query heads
    nkv: int               # key/value heads
    hd: int                # head dim
    L: int                 # layers
    V: int                 # vocab (0: no LM head)
    T: int                 # tree tokens per step
    C: int                 # committed KV length shared with the target
    tree: str              # "R" random recursive, "CB" chain+branches, "RB" random branching
    rope_theta: float = 1e6
    eps: float = 1e-6
    depth_cap: int = 48
    steps: int = 1          # draft expansion steps per decode cycle
    temps: Tuple[float, ...] = field(default_factory=tuple)
    w_std: float = 0.02
    lm_head: bool = False
    verify: bool = False


CONFIGS = {
    # A single 512x512 substitute linear layer plus one-head, dim-64 tree attention.
    1: Config(1, "linear512-attn1x64", H=512, I=0, nq=1, nkv=1, hd=64, L=1, V=0,
              T=16, C=128, tree="R"),
    # One Qwen2.5-7B-shaped decoder layer.
    2: Config(2, "qwen2.5-7b-layer", H=3584, I=18944, nq=28, nkv=4, hd=128, L=1, V=0,
              T=48, C=1024, tree="CB"),
    # The full 28-layer Qwen2.5-7B-shaped stack with a bf16 LM head and a verify pass.
    3: Config(3, "qwen2.5-7b-stack", H=3584, I=18944, nq=28, nkv=4, hd=128, L=28,
              V=152064, T=64, C=2048, tree="CB", steps=48, lm_head=True, verify=True),
    # The 64-layer Qwen2.5-32B-shaped stack with a 256-token random-branching tree.
    4: Config(4, "qwen2.5-32b-stack", H=5120, I=27648, nq=40, nkv=8, hd=128, L=64, V=0,
              T=256, C=4096, tree="RB"),
    # The 32-layer Llama-3.1-8B-shaped long-context stack.
    5: Config(5, "llama3.1-8b-longctx", H=4096, I=14336, nq=32, nkv=8, hd=128, L=32,
              V=128256, T=48, C=16384, tree="CB", rope_theta=5e5, eps=1e-5,
              temps=(0.2, 0.6), lm_head=True),
}


def get_config(cid: int, **overrides) -> Config:
    """Return config `cid`, optionally with fields replaced (for reduced test sizes)."""
    import dataclasses
    c = CONFIGS[cid]
    return dataclasses.replace(c, **overrides) if overrides else c


def layer_shapes(c: Config):
    """(name, N, K) of the four fused linear layers of one decoder layer."""
    qkv = (c.nq + 2 * c.nkv) * c.hd
    return [("qkv", qkv, c.H), ("o", c.H, c.nq * c.hd),
            ("gate_up", 2 * c.I, c.H), ("down", c.H, c.I)]
