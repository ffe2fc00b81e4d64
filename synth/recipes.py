"""Synthetic workloads: tensor lists, value distributions and hyperparameters.

These are inputs, not arithmetic.  Shapes follow the workloads named for the
method (a GPT-2 1.5B-shaped model, a 7.5B model, ZeRO-1 at N_d = 64, a local
reduce of N_d = 8 gradient buffers) and the optimizer values of the DeepSpeed
JSON example on the "DeepSpeed ZeRO" page (配置说明: Adam lr 3e-5, betas
0.9/0.999, eps 1e-8, weight_decay 3e-7; fp16 initial_scale_power 16).
"""
from dataclasses import dataclass, field
from typing import List, Optional

F16, BF16 = 1, 2

# DeepSpeed JSON example of the "DeepSpeed ZeRO" page
PAGE_ADAM = dict(lr=3e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=3e-7)


def gpt2_tensors(layers=48, d=1600, vocab=50257):
    t = [("wte", vocab * d)]
    for i in range(layers):
        t += [(f"h{i}.ln1.g", d), (f"h{i}.ln1.b", d), (f"h{i}.qkv", d * 3 * d), (f"h{i}.proj", d * d),
              (f"h{i}.ln2.g", d), (f"h{i}.ln2.b", d), (f"h{i}.fc", d * 4 * d), (f"h{i}.fc2", 4 * d * d)]
    return t


def llama_tensors(layers=32, d=4096, mlp=11008, vocab=32000, total=None):
    t = [("embed", vocab * d)]
    for i in range(layers):
        t += [(f"l{i}.attn_norm", d), (f"l{i}.wq", d * d), (f"l{i}.wk", d * d), (f"l{i}.wv", d * d),
              (f"l{i}.wo", d * d), (f"l{i}.ffn_norm", d), (f"l{i}.w_gate", mlp * d), (f"l{i}.w_up", mlp * d),
              (f"l{i}.w_down", d * mlp)]
    t += [("final_norm", d), ("lm_head", vocab * d)]
    if total is not None:
        s = sum(n for _, n in t)
        assert total >= s
        if total > s:
            t.append(("extra", total - s))
    return t


@dataclass
class Workload:
    name: str
    cid: int                      # seed = 0x5EED0000 + cid
    tensors: List[tuple]          # (name, numel) in flatten order
    nd: int
    ranks: List[int]              # ranks exercised
    dtype: int
    grad_mode: str                # "reduce" (N_d rank buffers), "flat" (one reduced buffer), "ragged" (per tensor)
    param_mode: str               # "flat" or "ragged"
    grad_sigma: float             # std of the (scaled) 16-bit gradient values
    loss_scale: float
    master_sigma: float = 0.02
    master_given: bool = True     # fp32 master drawn directly (else upcast of the 16-bit params)
    zero_mod: int = 0             # 1/zero_mod of gradient positions are exact +0 in every buffer
    max_norm: float = 1.0
    hp: dict = field(default_factory=lambda: dict(PAGE_ADAM))
    steps: int = 1

    @property
    def seed(self):
        return 0x5EED0000 + self.cid

    @property
    def psi(self):
        return sum(n for _, n in self.tensors)

    @property
    def numel(self):
        return [n for _, n in self.tensors]


def tiny():
    return Workload("tiny", 1, [("flat", 1 << 20)], nd=4, ranks=[0, 1, 2, 3], dtype=F16, grad_mode="reduce",
                    param_mode="flat", grad_sigma=1e-3 * 1024, loss_scale=1024.0,
                    hp=dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01), steps=5)


def gpt2_shard():
    return Workload("gpt2_1p5b_nd8", 2, gpt2_tensors(), nd=8, ranks=[7, 3], dtype=BF16, grad_mode="flat",
                    param_mode="flat", grad_sigma=1e-4, loss_scale=1.0)


def zero1_7p5b():
    return Workload("zero1_7p5b_nd64", 3, [("flat", 7_500_000_000)], nd=64, ranks=[0, 63], dtype=F16,
                    grad_mode="flat", param_mode="flat", grad_sigma=1e-3 * 65536, loss_scale=65536.0)


def reduce8():
    return Workload("reduce_1p5b_nd8", 4, [("flat", 1_500_000_000)], nd=8, ranks=[7, 0], dtype=F16,
                    grad_mode="reduce", param_mode="flat", grad_sigma=1e-3, loss_scale=1.0, zero_mod=1000)


def full7p5b():
    return Workload("full_7p5b_nd1", 5, llama_tensors(total=7_500_000_000), nd=1, ranks=[0], dtype=BF16,
                    grad_mode="ragged", param_mode="ragged", grad_sigma=1e-4, loss_scale=1.0,
                    hp=dict(PAGE_ADAM, weight_decay=0.1))


def ragged_mini(nd=3):
    return Workload(f"ragged_mini_nd{nd}", 6, llama_tensors(layers=4, d=256, mlp=688, vocab=2000), nd=nd,
                    ranks=list(range(nd)), dtype=BF16, grad_mode="ragged", param_mode="ragged",
                    grad_sigma=1e-4, loss_scale=1.0, hp=dict(PAGE_ADAM, weight_decay=0.1), steps=3)


def big_tensor():
    """A parity case: one tensor of more than 2^31 elements between two small ones, at
    N_d = 1, so element offsets inside a tensor pass the 32-bit range; fp16 with a loss
    scale, the master taken from the 16-bit parameters, and a gradient norm well above
    max_norm (clipping active)."""
    return Workload("big_tensor_nd1", 7, [("head", 4099), ("big", (1 << 31) + 12345), ("tail", 77)], nd=1,
                    ranks=[0], dtype=F16, grad_mode="ragged", param_mode="ragged", grad_sigma=1e-3 * 1024,
                    loss_scale=1024.0, master_given=False, hp=dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                                                                   weight_decay=0.01))


ALL = {"tiny": tiny, "gpt2": gpt2_shard, "zero1_7p5b": zero1_7p5b, "reduce8": reduce8, "full7p5b": full7p5b}
