"""CPU oracle of the gated delta rule (fp64, token by token).

TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and the CPU
baseline of bench.py. The GPU product path never imports this package.
"""
from .oracle import ERR_ARG, ERR_DOMAIN, MISMATCH, OK, backward, build, load, ref_check, run, snapshot_count  # noqa: F401
