"""ctypes binding of libmxq_measure.so (include/mxq_measure.h): the byte-pattern
references the benchmark times beside the MXNorm forward.  Argument
marshalling only; the patterns run in the library's HIP kernels."""
import ctypes as C
import os

ONE_WAVE_CHUNK8 = 0
TWO_WAVES_CHUNK8 = 1
ONE_WAVE_LANE16 = 2
ONE_WAVE_LANE16X = 3
TWO_WAVES_LANE16 = 4
TWO_WAVES_LANE16X = 5
LAYOUTS = {ONE_WAVE_CHUNK8: "one_wave_chunk8", TWO_WAVES_CHUNK8: "two_waves_chunk8",
           ONE_WAVE_LANE16: "one_wave_lane16", ONE_WAVE_LANE16X: "one_wave_lane16x",
           TWO_WAVES_LANE16: "two_waves_lane16", TWO_WAVES_LANE16X: "two_waves_lane16x"}

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmxq_measure.so")
_lib = None


def library_path():
    return _PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError("libmxq_measure.so not built: run __graft_entry__.build() "
                               "(looked for %s)" % _PATH)
        import torch  # noqa: F401  (load torch's HIP runtime first, as for libmxnorm.so)
        L = C.CDLL(_PATH)
        L.mxq_pattern_supported.restype = C.c_int
        L.mxq_pattern_supported.argtypes = [C.c_int, C.c_int64]
        L.mxq_measure_pattern.restype = C.c_int
        L.mxq_measure_pattern.argtypes = [C.c_int, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p,
                                          C.c_void_p, C.c_void_p, C.c_void_p]
        L.mxq_bwd_pattern_supported.restype = C.c_int
        L.mxq_bwd_pattern_supported.argtypes = [C.c_int, C.c_int64]
        L.mxq_measure_bwd_pattern.restype = C.c_int
        L.mxq_measure_bwd_pattern.argtypes = [C.c_int, C.c_void_p, C.c_void_p, C.c_int64,
                                              C.c_int64, C.c_void_p, C.c_void_p]
        _lib = L
    return _lib
