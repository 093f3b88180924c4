"""MI355X (gfx950) RTN weight quantization and fused-dequantization GEMV.

The compute path is the HIP library ``libqgemv.so`` (C ABI in
``include/qgemv.h``); ``dequant_gemv_rtn_amd.binding`` marshals torch tensors
into it.  Importing this package does not load the library: the first call
into ``binding`` does, and fails loudly if it is missing.
"""

FORMATS = {
    "int4_asym": 1,
    "fp4_e2m1": 2,
    "fp4_razer": 3,
    "fp4_afpq": 4,
    "bfp6": 5,
    "bfp4": 6,
    "int8": 7,
    "fp3_razer": 8,
    "fp3_afpq": 9,
}
