"""Model-state memory of mixed-precision Adam under ZeRO (test infrastructure).

The pages count, per parameter, 2 bytes of fp16/bf16 parameter, 2 bytes of
fp16/bf16 gradient and K = 12 bytes of fp32 master, momentum and variance, so
plain data parallelism holds (2 + 2 + K) * psi bytes on every GPU
("ZeRO 技术原理" section 3; "DeepSpeed ZeRO" 表格计算).  Stage 1 partitions
the K part, stage 2 also the gradient, stage 3 also the parameter
("ZeRO 技术原理" 3.1; the memory formula tables of the answer.freetools.me page
and of "DeepSpeed ZeRO" ZeRO Stage 1/2/3).
"""


def model_state_bytes(stage: int, psi: float, nd: int, k: int = 12) -> float:
    if stage == 0:
        return (2 + 2 + k) * psi
    if stage == 1:
        return (2 + 2) * psi + k * psi / nd
    if stage == 2:
        return 2 * psi + (2 + k) * psi / nd
    if stage == 3:
        return (2 + 2 + k) * psi / nd
    raise ValueError("stage must be 0..3")
