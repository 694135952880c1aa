"""The 4-bit QK^T oracle (E2M1, MXFP4 blocks) against its pins (CPU)."""
import oracle
import oracle_pins as pins


def test_e2m1():
    pins.check_e2m1(oracle.e2m1_decode_table, oracle.e2m1_encode)


def test_mx4():
    pins.check_mx4(oracle.mx4_quantize_ref, oracle.mx4_dequantize_ref, oracle.e2m1_decode_table)


def test_fp4_attention():
    pins.check_fp4_attention(oracle.mx4_quantize_ref, oracle.fp4_attention_ref, oracle.fp8_attention_ref,
                             oracle.vsmooth_quantize_ref, oracle.e2m1_decode_table)
