"""Synthetic parameter lists shaped like the models the pages train.

Holds shapes and workload recipes only; none of the optimizer's arithmetic.

The pages train GPT-2 (350M) and GPT-Neo (2.7B, 6.7B) with BF16+SR
("Stochastic Rounding for LLM Training: Theory and Practice", Figures 4-6)
and a 1.5B-parameter language model with 8-bit Adam ("8-bit Optimizers via
Block-wise Quantization", evaluation).  No weights or data are used: the
lists below reproduce the tensor shapes of a GPT-2 style decoder (fused qkv
with bias, tied output head), in this order:

  wte [V, d], wpe [ctx, d],
  per layer: ln1.w, ln1.b [d]; qkv.w [d, 3d]; qkv.b [3d]; proj.w [d, d];
             proj.b [d]; ln2.w, ln2.b [d]; fc.w [d, ffn]; fc.b [ffn];
             mlp_proj.w [ffn, d]; mlp_proj.b [d],
  ln_f.w, ln_f.b [d].

The position of a tensor in its list is its tensor id (the RNG stream id of
its stochastic rounding).
"""

from dataclasses import dataclass, field
from typing import List, Tuple


@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: Tuple[int, ...]
    kind: str          # "embedding" | "weight" | "bias" | "ln_weight" | "ln_bias"
    fan_in: int

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


@dataclass(frozen=True)
class Workload:
    name: str
    tensors: Tuple[TensorSpec, ...]
    steps: int
    lr: float
    weight_decay: float
    seed: int
    grad_recipe: str           # key into workloads.gen recipes
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    state_mode: str = "auto"   # "auto" (fp32 under 4096 elements, else 8-bit) | "bf16"

    @property
    def numel(self) -> int:
        return sum(t.numel for t in self.tensors)


def gpt_tensors(layers: int, d: int, ffn: int, vocab: int, ctx: int) -> List[TensorSpec]:
    t = [TensorSpec("wte", (vocab, d), "embedding", d),
         TensorSpec("wpe", (ctx, d), "embedding", d)]
    for i in range(layers):
        p = f"h{i}."
        t += [
            TensorSpec(p + "ln1.w", (d,), "ln_weight", 1),
            TensorSpec(p + "ln1.b", (d,), "ln_bias", 1),
            TensorSpec(p + "qkv.w", (d, 3 * d), "weight", d),
            TensorSpec(p + "qkv.b", (3 * d,), "bias", 1),
            TensorSpec(p + "proj.w", (d, d), "weight", d),
            TensorSpec(p + "proj.b", (d,), "bias", 1),
            TensorSpec(p + "ln2.w", (d,), "ln_weight", 1),
            TensorSpec(p + "ln2.b", (d,), "ln_bias", 1),
            TensorSpec(p + "fc.w", (d, ffn), "weight", d),
            TensorSpec(p + "fc.b", (ffn,), "bias", 1),
            TensorSpec(p + "mlp_proj.w", (ffn, d), "weight", ffn),
            TensorSpec(p + "mlp_proj.b", (d,), "bias", 1),
        ]
    t += [TensorSpec("ln_f.w", (d,), "ln_weight", 1),
          TensorSpec("ln_f.b", (d,), "ln_bias", 1)]
    return t


def single_tensor() -> Workload:
    """One 1,048,576-element tensor (512 blocks), ten steps from zero state."""
    return Workload(
        name="single-1M",
        tensors=(TensorSpec("w", (1024, 1024), "single", 1024),),
        steps=10, lr=1e-3, weight_decay=0.01, seed=0, grad_recipe="single")


def gpt2_350m() -> Workload:
    return Workload(
        name="gpt2-350m", tensors=tuple(gpt_tensors(24, 1024, 4096, 50257, 1024)),
        steps=3, lr=6e-4, weight_decay=0.1, seed=0, grad_recipe="fan_in")


def lm_1p5b() -> Workload:
    return Workload(
        name="lm-1.5b", tensors=tuple(gpt_tensors(48, 1600, 6400, 50257, 1024)),
        steps=3, lr=1.5e-4, weight_decay=0.01, seed=0, grad_recipe="nonuniform")


def gptneo_2p7b(state_mode: str = "auto") -> Workload:
    return Workload(
        name="gptneo-2.7b" + ("-bf16" if state_mode == "bf16" else ""),
        tensors=tuple(gpt_tensors(32, 2560, 10240, 50257, 2048)),
        steps=3, lr=3.2e-4, weight_decay=0.1, seed=0, grad_recipe="plain",
        state_mode=state_mode)


def gptneo_6p7b() -> Workload:
    return Workload(
        name="gptneo-6.7b", tensors=tuple(gpt_tensors(32, 4096, 16384, 50257, 2048)),
        steps=5, lr=1.2e-4, weight_decay=0.1, seed=1234, grad_recipe="outliers100")


def many_small(numel: int, count: int = 30000) -> Workload:
    """`count` equal tensors of `numel` elements (a stress case for the multi-tensor schedule:
    each wave's stride over the blocks crosses many tensors)."""
    return Workload(
        name=f"many-{numel}",
        tensors=tuple(TensorSpec(f"t{i}", (numel,), "weight", numel) for i in range(count)),
        steps=3, lr=1e-3, weight_decay=0.01, seed=0, grad_recipe="plain")


WORKLOADS = {
    "single-1M": single_tensor,
    "gpt2-350m": gpt2_350m,
    "lm-1.5b": lm_1p5b,
    "gptneo-2.7b": gptneo_2p7b,
    "gptneo-2.7b-bf16": lambda: gptneo_2p7b("bf16"),
    "gptneo-6.7b": gptneo_6p7b,
    "many-4096": lambda: many_small(4096),
    "many-6151": lambda: many_small(6151),
    "many-2000": lambda: many_small(2000),    # every tensor under 4096 elements: fp32 state
    "many-2048": lambda: many_small(2048),    # fp32 state, one whole block per tensor
}


def get(name: str) -> Workload:
    """The workload of that name (case-insensitive); ValueError naming the known ones."""
    by_lower = {k.lower(): k for k in WORKLOADS}
    key = by_lower.get(name.lower())
    if key is None:
        raise ValueError(f"unknown workload {name!r}; known: {', '.join(WORKLOADS)}")
    return WORKLOADS[key]()


def subset_for_sampling(w: Workload) -> List[int]:
    """Tensor ids of a fixed subset: embeddings, first and last layer, final LN."""
    names = [t.name for t in w.tensors]
    last = max((int(n[1:].split(".")[0]) for n in names if n.startswith("h")), default=-1)
    keep = []
    for i, n in enumerate(names):
        if n in ("wte", "wpe", "ln_f.w", "ln_f.b", "w") or n.startswith("h0.") \
                or (last >= 0 and n.startswith(f"h{last}.")):
            keep.append(i)
    return keep
