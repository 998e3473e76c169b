"""Seeded synthetic workloads (shape lists, hyperparameters, input draws).

Shared by the HIP path's tests/benchmark and by the oracle's tests; it holds
no step of the optimizer itself."""
from .configs import (Dist, Workload, WORKLOADS, ALIASES, get, numel, real_total,  # noqa: F401
                      TINY, GPT2_SMALL, LLAMA_7B, GPT_100B_RANK, GPT_1T_LAST_RANK, opt_hparams)
from .gen import (CHUNK, fill, shard_inputs, grad_for_step, inf_positions,  # noqa: F401
                  sample_indices, to_bits16, POS_INF_BITS)
