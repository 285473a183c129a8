"""fp64 CPU oracle for the KDA core -- test infrastructure only (see kda_oracle)."""
from .kda_oracle import *  # noqa: F401,F403
from .kda_oracle import (G_MIN, logistic, gate_log_decay, beta_of, recurrence,  # noqa: F401
                         recurrence_dplr, recurrence_matrix, chunkwise, packed, decode_step)
