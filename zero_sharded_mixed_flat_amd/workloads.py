"""The workloads: sizes, layouts, value distributions and hyperparameters.

Pure data.  Both the parity tests (which feed the oracle) and the benchmark
read these definitions; nothing here computes any part of the step.

Shapes follow the pages' examples:
* ``tiny_nd4_z2``: 2**20 parameters on 4 emulated ranks under ZeRO-2; every
  rank's share runs, three steps.
* ``llama3_8b_nd8_z2``: an 8.03e9-parameter flat vector (LLaMA-3 8B sized,
  CMU 11-868 Lecture 18 notes §1.2) on 8 ranks under ZeRO-2; one rank's share.
* ``paper_7p5b_nd64_z3``: the paper's 7.5B-parameter, 64-way example (Lecture
  18 notes §2.1; ZeRO reading notes 026 §四) under ZeRO-3, as 48 equal layer
  units, with the per-layer gather of the 16-bit parameters.
* ``gpt2_1p5b_nd16_z1``: GPT-2 1.5B (48 layers, h = 1600, 4h MLP, vocab 50257;
  Lecture 18 notes §1.3; ZeRO paper notes 0x03) as a ragged per-tensor flat
  bucket on 16 ranks under ZeRO-1, fp16 with a loss scale of 65536.
* ``gpt3_175b_nd16_z1``: a 175e9-parameter vector (GPT-3 175B sized, Lecture 18
  notes §1.2) on 16 ranks; the rank's owner update on a pre-reduced gradient.
* ``llama3_8b_nd8_z2_offload``: the LLaMA-3-8B-sized ZeRO-2 share with
  ZeRO-Offload (Lecture 18 notes §4.4): master, m and v live in host memory
  and the host AdamW updates them; the reduced gradient goes to the host and
  the 16-bit parameters come back.
* ``llama3_8b_nd8_z2_offload_delayed``: the same with ZeRO-Offload's
  one-step-delayed update (Lecture 18 notes §4.4): the host AdamW of step t
  runs while the GPU reduces step t+1's gradient and takes its norm.
* ``paper_7p5b_nd64_z3_qwz8`` / ``_qwz4``: the ZeRO-3 workload with the
  ZeRO++ quantised-weight gather (Lecture 18 notes §4.5): the rank quantises
  its updated 16-bit shard to INT8 / INT4 codes with one scale per 256
  elements, and every unit is gathered from all ranks' codes, dequantised
  into the 16-bit full buffer.  Slices are aligned to 256 so a block never
  straddles two owners.

Pages cited by short name:
  ZeRO paper notes  "ZeRO:" paper notes (puzhiyuan.github.io)
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    psi: int
    nd: int
    stage: int
    units: tuple                  # unit sizes: one flat unit, or one per layer (stage 3)
    grad_dtype: str               # "f16" or "bf16"
    param_dtype: str
    grad_std: float               # per-rank gradient contributions ~ N(0, grad_std)
    master_std: float
    m_std: float                  # 0 means m starts at zero
    v_std: float                  # v = |N(0, v_std)|; 0 means zero
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    max_norm: float
    loss_scale: float = 1.0       # gradients are stored multiplied by this
    outlier_frac: float = 0.0     # fraction of gradient elements multiplied by outlier_mult
    outlier_mult: float = 1.0
    rank: int = 0                 # the rank whose share runs (when not all ranks are emulated)
    all_ranks: bool = False       # every rank's share runs in one step
    pre_reduced: bool = False     # the gradient arrives already averaged (owner update only)
    gather_per_unit: bool = False # the 16-bit shards of every rank are gathered unit by unit
    gather_shard_std: float = 0.0 # other ranks' 16-bit parameter shards ~ N(0, this)
    gather_bits: int = 16         # 16: plain gather; 8 or 4: block-quantised codes
    offload: bool = False         # fp32 state in host memory, AdamW on the CPU (ZeRO-Offload)
    offload_delay: bool = False   # ... with the one-step-delayed update (the host AdamW of step t
                                  # overlaps the GPU's reduce and norm of step t+1)
    steps: int = 1
    align: int = 8
    tensors: tuple = field(default=None, repr=False)   # ragged tensor sizes, if any

    @property
    def inv_loss_scale(self):
        return 1.0 / self.loss_scale


def gpt2_tensor_sizes(layers=48, h=1600, vocab=50257, ctx=1024):
    """Parameter tensors of GPT-2 in storage order (tied output embedding)."""
    sizes = [vocab * h, ctx * h]
    for _ in range(layers):
        sizes += [h, h,                    # ln_1 weight, bias
                  h * 3 * h, 3 * h,        # attention qkv weight, bias
                  h * h, h,                # attention output projection weight, bias
                  h, h,                    # ln_2 weight, bias
                  h * 4 * h, 4 * h,        # MLP up weight, bias
                  4 * h * h, h]            # MLP down weight, bias
    sizes += [h, h]                        # final layer norm weight, bias
    return tuple(sizes)


_GPT2 = gpt2_tensor_sizes()

WORKLOADS = {
    w.name: w for w in [
        Workload(
            name="tiny_nd4_z2", psi=1 << 20, nd=4, stage=2, units=(1 << 20,),
            grad_dtype="f16", param_dtype="f16", grad_std=1e-3,
            master_std=0.02, m_std=0.0, v_std=0.0,
            lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_norm=1.0,
            all_ranks=True, steps=3),
        Workload(
            name="llama3_8b_nd8_z2", psi=8_030_000_000, nd=8, stage=2, units=(8_030_000_000,),
            grad_dtype="bf16", param_dtype="bf16", grad_std=1e-4,
            master_std=0.02, m_std=1e-5, v_std=1e-8,
            lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0,
            rank=7),
        Workload(
            name="llama3_8b_nd8_z2_offload", psi=8_030_000_000, nd=8, stage=2, units=(8_030_000_000,),
            grad_dtype="bf16", param_dtype="bf16", grad_std=1e-4,
            master_std=0.02, m_std=1e-5, v_std=1e-8,
            lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0,
            rank=7, offload=True),
        Workload(
            name="llama3_8b_nd8_z2_offload_delayed", psi=8_030_000_000, nd=8, stage=2, units=(8_030_000_000,),
            grad_dtype="bf16", param_dtype="bf16", grad_std=1e-4,
            master_std=0.02, m_std=1e-5, v_std=1e-8,
            lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0,
            rank=7, offload=True, offload_delay=True),
        Workload(
            name="paper_7p5b_nd64_z3", psi=7_500_000_000, nd=64, stage=3,
            units=(156_250_000,) * 48,
            grad_dtype="f16", param_dtype="f16", grad_std=1e-3,
            outlier_frac=0.01, outlier_mult=100.0,
            master_std=0.02, m_std=0.0, v_std=0.0,
            lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_norm=1.0,
            rank=0, gather_per_unit=True, gather_shard_std=0.02),
        *[Workload(
            name=f"paper_7p5b_nd64_z3_qwz{bits}", psi=7_500_000_000, nd=64, stage=3,
            units=(156_250_000,) * 48,
            grad_dtype="f16", param_dtype="f16", grad_std=1e-3,
            outlier_frac=0.01, outlier_mult=100.0,
            master_std=0.02, m_std=0.0, v_std=0.0,
            lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_norm=1.0,
            rank=0, gather_per_unit=True, gather_shard_std=0.02, gather_bits=bits, align=256)
          for bits in (8, 4)],
        Workload(
            name="gpt2_1p5b_nd16_z1", psi=sum(_GPT2), nd=16, stage=1, units=(sum(_GPT2),),
            grad_dtype="f16", param_dtype="f16", grad_std=1e-3, loss_scale=65536.0,
            master_std=0.02, m_std=1e-5, v_std=1e-8,
            lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0,
            rank=5, tensors=_GPT2),
        Workload(
            name="gpt3_175b_nd16_z1", psi=175_000_000_000, nd=16, stage=1,
            units=(175_000_000_000,),
            grad_dtype="bf16", param_dtype="bf16", grad_std=1e-4,
            master_std=0.02, m_std=1e-5, v_std=1e-8,
            lr=6e-5, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0,
            rank=0, pre_reduced=True),
    ]
}

# The largest configuration that fits one GPU: the 175e9-parameter, 16-rank
# owner update (10.94e9 owned elements, about 175 GB resident in HBM).
BENCH_DEFAULT = "gpt3_175b_nd16_z1"


def get(name):
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None
