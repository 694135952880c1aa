"""The FP8 value-path oracle (E4M3, V-Smooth, ExpCast, FP8 attention) against its pins (CPU)."""
import oracle
import oracle_pins as pins


def test_e4m3():
    pins.check_e4m3(oracle.e4m3_decode_table, oracle.e4m3_encode)


def test_expcast():
    pins.check_expcast(oracle.expcast_byte, oracle.e4m3_decode_table)


def test_vsmooth():
    pins.check_vsmooth(oracle.vsmooth_quantize_ref, oracle.e4m3_decode_table)


def test_fp8_attention():
    pins.check_fp8_attention(oracle.vsmooth_quantize_ref, oracle.fp8_attention_ref, oracle.e4m3_decode_table,
                             oracle.dequantize_ref)


def test_fp8_reference_point():
    pins.check_fp8_reference_point(oracle.vsmooth_quantize_ref, oracle.fp8_attention_ref, oracle.e4m3_decode_table,
                                   oracle.dequantize_ref)
