"""Model-state and communication accounting per data-parallel rank.

Test infrastructure: see the package docstring.

Pages:
* Mixed-precision Adam keeps a 2-byte parameter, a 2-byte gradient and K bytes
  of optimizer state per parameter (K = 12: fp32 master, momentum, variance),
  16 bytes in all (CMU 11-868 Lecture 18 notes §1.2; L3.2 Memory optimisation
  and ZeRO §2.1; ZeRO reading notes 026 §二).  The slides count a resident fp32
  gradient as optimizer state too, K = 16, 20 bytes in all (Lecture 18 notes §1.2).
* Per-rank bytes: plain DP (4+K)Ψ; stage 1 4Ψ + KΨ/Nd; stage 2 2Ψ + (2+K)Ψ/Nd;
  stage 3 (4+K)Ψ/Nd (Lecture 18 notes §2.1 and summary; L3.2 §2.3 table).
* Elements each rank sends per step: DP, stage 1 and stage 2 move 2Ψ, stage 3
  moves 3Ψ, each times (Nd-1)/Nd for ring collectives (Lecture 18 notes §3.1;
  L3.2 §2.3; ZeRO paper notes 0x07).

Pages cited by short name:
  L3.2              "L3.2 显存优化与 ZeRO" (yulong.wang)
  ZeRO paper notes  "ZeRO:" paper notes (puzhiyuan.github.io)
"""


def bytes_per_param(nd, stage, k=12):
    """Model-state bytes one rank holds per parameter of the whole model."""
    if stage == 0:
        return 4.0 + k
    if stage == 1:
        return 4.0 + k / nd
    if stage == 2:
        return 2.0 + (2.0 + k) / nd
    if stage == 3:
        return (4.0 + k) / nd
    raise ValueError("stage must be 0, 1, 2 or 3")


def model_state_bytes(psi, nd, stage, k=12):
    """Per-rank model-state bytes for ``psi`` parameters over ``nd`` ranks."""
    if nd < 1:
        raise ValueError("nd must be >= 1")
    return psi * bytes_per_param(nd, stage, k)


def max_params(mem_bytes, nd, stage, k=12):
    """Largest parameter count whose model states fit in ``mem_bytes`` per rank.

    ``nd=float('inf')`` gives the limit as the rank count grows.
    """
    if nd == float("inf"):
        limit = {0: 4.0 + k, 1: 4.0, 2: 2.0}.get(stage)
        if limit is None:
            return float("inf")
        return mem_bytes / limit
    return mem_bytes / bytes_per_param(nd, stage, k)


def comm_volume(psi, nd, stage):
    """Elements one rank sends per step (reduce-scatter + all-gather rings)."""
    if nd < 1:
        raise ValueError("nd must be >= 1")
    passes = 3.0 if stage == 3 else 2.0
    return passes * psi * (nd - 1) / nd
