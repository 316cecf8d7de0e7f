"""CPU oracle for one data-parallel rank's share of a ZeRO mixed-precision Adam step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or helper
with the HIP library; both sides receive the same seeded inputs and nothing else.

What it computes, and where the pages fix it
--------------------------------------------
ZeRO changes who stores and updates each parameter, not the arithmetic: in a
fixed-rank-order emulation the sharded run is bit-identical to plain data
parallelism (CMU 11-868 Lecture 18 notes, §2.5 and §7 pitfall 2; ZeRO reading
notes 026, §三).  So the oracle is the plain, unsharded mixed-precision
Adam(W) step -- rank-order gradient averaging, global-norm clipping, fp32
master/m/v update, cast to the 16-bit parameter -- restricted to one rank's
owned slice of the flat parameter vector:

* ``partition``  -- flat-bucket ownership (Lecture 18 notes §3.2 and
  exercise 6; Illustrated distributed training (8) ZeRO §8.4), and restoring
  sharded state under another partition (ZeRO reading notes 026 §五).
  Integers only.
* ``accounting`` -- per-rank model-state bytes 16Ψ, 4Ψ+KΨ/Nd, 2Ψ+(2+K)Ψ/Nd,
  (4+K)Ψ/Nd and communication volume 2Ψ / 3Ψ × (Nd−1)/Nd (Lecture 18 notes
  §2.1, §3.1; L3.2 Memory optimisation and ZeRO §2.3).
* ``rounding``   -- fp32 → bf16 / fp16 round-to-nearest-even.
* ``quant``      -- block-quantised 16-bit parameters for the gather (ZeRO++
  quantised weights; Lecture 18 notes §4.5): absmax INT8/INT4 per 256.
* ``step``       -- the averaged reduce-scatter slice (Lecture 18 notes §2.2
  step 3), the exact global L2 norm and clip coefficient (Lecture 18 notes
  §1.4; L3.2 §4.2 ``gradient_clipping``), the Adam(W) update of the owned
  fp32 state followed by the copy to 16-bit (Lecture 18 notes §2.2 step 4),
  and the gather of 16-bit slices (§2.2 step 5; Illustrated ZeRO §8.4).

Readings where the pages are silent (each one is listed with its reason in the
repository's design notes): the mean is an fp32 rank-order sum divided by Nd;
the reduced gradient is stored in the gradient's 16-bit dtype with the loss
scale kept; the norm is taken over the stored, unscaled reduced gradient;
clip coefficient = min(1, max_norm / (norm + 1e-6)); Adam is Kingma & Ba with
bias correction and decoupled (AdamW) weight decay; a non-finite gradient
skips the whole step.

Parity-unpinned items: the pages fix neither the Adam variant nor the clip
epsilon nor where the loss scale is removed.  They are pinned here only to the
published formulas they restate, through library routines
(``torch.optim.AdamW``, ``torch.nn.utils.clip_grad_norm_``) and closed forms.

16-bit data is carried as ``numpy.uint16`` bit patterns with a dtype tag
``"f16"`` or ``"bf16"``; fp32 state is ``numpy.float32``.

Pages cited by short name:
  L3.2              "L3.2 显存优化与 ZeRO" (yulong.wang)
  Illustrated ZeRO  "图解分布式训练（八）—— ZeRO 学习" (llm.jiangnianmeng.cn)
"""

from . import accounting, partition, quant, rounding, step  # noqa: F401
from .accounting import comm_volume, max_params, model_state_bytes  # noqa: F401
from .partition import Plan, make_plan, merge, reshard, reshard_segments, segments, shard_of  # noqa: F401
from .rounding import narrow, widen  # noqa: F401
from .step import (  # noqa: F401
    AdamHparams,
    adam_update,
    clip_coef,
    gather,
    norm_from_sumsq,
    reduce_shard,
    step_sharded,
    step_unsharded,
    sumsq_exact,
)
