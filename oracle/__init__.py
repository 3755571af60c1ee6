"""CPU oracle of the score-centering correction (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It shares no code with the HIP library.
"""
from .sc_oracle import (BATCH_KEYS, CLAMP, DEV_BAD_ID, IS_MIS, IS_NONE, IS_TIS,
                        is_weight, DEV_BAD_RESP, DEV_BAD_SAMPLED,
                        DEV_DUP_ID, DEV_NONFINITE, MODE_CORRECTION,
                        MODE_DLOGITS, MODE_SCORE, batch_sums, bf16_rne,
                        group_norm, lmhead_backward, lmhead_logits, masked_row,
                        record_topk,
                        sc_row, trainer_log_softmax)
