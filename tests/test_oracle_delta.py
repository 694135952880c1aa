"""The Chipmunk column-sum and sparse-delta oracles against their pins (CPU)."""
import oracle
import oracle_pins as pins


def test_colsum():
    pins.check_colsum(oracle.colsum_scores_ref, oracle.colsum_mask_ref, oracle.row_lse_ref)


def test_delta():
    pins.check_delta(oracle.delta_fresh_ref, oracle.delta_forward_ref)
