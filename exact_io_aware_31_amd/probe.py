"""Python binding of libfa_probe (include/fa_probe.h): the chip's measured ceilings.

Argument marshalling and timing only; the two kernels are in fa_probe.hip.
    mfma_bf16_rate(torch)   -> dict: dense bf16 matrix TFLOP/s and the shader clock under that load
    stream_read_rate(torch) -> dict: streaming HBM read GB/s
Both time their launches with HIP events on torch's current stream, which is
the stream the launches are enqueued on.
"""
import ctypes
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "_lib", "libfa_probe.so")
THREADS = 256          # FA_PROBE_THREADS
READ_CHUNK = 65536     # FA_PROBE_READ_CHUNK
MFMA_FLOP = 2 * 32 * 32 * 16  # one v_mfma_f32_32x32x16_bf16

_lib = None


def load_library(path: str = LIB_PATH):
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m exact_io_aware_31_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.fa_probe_mfma_bf16.argtypes = [vp, vp, i, i, vp]
    lib.fa_probe_mfma_bf16.restype = i
    lib.fa_probe_stream_read.argtypes = [vp, ctypes.c_size_t, vp, i, vp]
    lib.fa_probe_stream_read.restype = i
    if path == LIB_PATH:
        _lib = lib
    return lib


def _stream(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _timed(torch, launch, reps: int):
    """Per-launch milliseconds (HIP events around each launch on the current stream)."""
    launch()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        launch()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def mfma_bf16_rate(torch, iters: int = 40000, reps: int = 3, waves_per_simd=(1, 2, 3)):
    """Best dense bf16 rate over workgroup counts giving 1, 2 and 3 waves per SIMD, with the
    shader clock measured during that launch (s_memtime against the 100 MHz s_memrealtime)."""
    lib = load_library()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    best = None
    for w in waves_per_simd:
        blocks = cus * w
        out = torch.empty(blocks * THREADS, dtype=torch.float32, device="cuda")
        stamps = torch.zeros(4, dtype=torch.int64, device="cuda")

        def launch():
            rc = lib.fa_probe_mfma_bf16(ctypes.c_void_p(out.data_ptr()),
                                        ctypes.c_void_p(stamps.data_ptr()), blocks, iters,
                                        _stream(torch))
            if rc != 0:
                raise RuntimeError(f"fa_probe_mfma_bf16 returned {rc}")

        ms = _timed(torch, launch, reps)
        t0, r0, t1, r1 = (int(x) for x in stamps.cpu())
        flops = blocks * 4 * iters * 4 * MFMA_FLOP
        tf = flops / (min(ms) * 1e-3) / 1e12
        real_s = (r1 - r0) / 100e6
        clock = (t1 - t0) / real_s / 1e9 if real_s > 0 else None
        rec = {"tflops": round(tf, 1), "waves_per_simd": w, "blocks": blocks,
               "ms": round(min(ms), 4), "clock_ghz": round(clock, 3) if clock else None,
               "wave0_ms_by_realtime": round(real_s * 1e3, 4)}
        if best is None or rec["tflops"] > best["tflops"]:
            best = rec
        del out, stamps
    best["what"] = ("dense bf16 v_mfma_f32_32x32x16 rate, four register-operand chains per wave, "
                    "pseudo-random full-mantissa operands in [-1, 1), "
                    f"best of {list(waves_per_simd)} waves per SIMD on {cus} CUs")
    return best


def stream_read_rate(torch, nbytes: int = 8 << 30, reps: int = 5,
                     blocks=(2048, 4096, 8192, 16384, 32768, 65536)):
    """Best streaming-read rate (16-byte non-temporal loads) over a few grid sizes; median of
    reps per grid size."""
    lib = load_library()
    nbytes -= nbytes % READ_CHUNK
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    best = None
    for nb in blocks:
        out = torch.empty(nb * THREADS, dtype=torch.int32, device="cuda")

        def launch():
            rc = lib.fa_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                          ctypes.c_void_p(out.data_ptr()), nb, _stream(torch))
            if rc != 0:
                raise RuntimeError(f"fa_probe_stream_read returned {rc}")

        ms = statistics.median(_timed(torch, launch, reps))
        gbs = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "blocks": nb, "ms": round(ms, 4)}
        del out
    del buf
    torch.cuda.empty_cache()
    best["what"] = (f"streaming read of {nbytes >> 20} MiB, 16-byte non-temporal loads, sixteen in "
                    f"flight per lane, a contiguous run per workgroup, best of grids {list(blocks)} "
                    f"(median of {reps})")
    return best
