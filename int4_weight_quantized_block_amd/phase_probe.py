"""Per-wave phase timing of the large-M GEMM (a measurement tool, not part of the layer).

    python -m int4_weight_quantized_block_amd.phase_probe build   # on the build machine
    python -m int4_weight_quantized_block_amd.phase_probe run     # on the GPU

``build`` writes a copy of csrc/gemm.hip in which the plain bf16 single-linear kernel (W4A8 or
W4A4, symmetric, K % 128 == 0) reads the GPU's constant 100 MHz real-time counter at five
points of every wave -- kernel entry, after the prologue's wait for the first stage, after the
main loop, after the epilogue has issued its stores, after the stores have drained -- and
stores the stamps of the first 256 workgroups to a device array; it links that copy with the
other objects of ``build.py`` into ``_phase/libw4phase.so`` (beside this file), which also
exports ``w4_phase_stamps`` to copy the array out.  The instrumentation is inserted at fixed
anchor strings of the kernel source, each checked, so a source change that moves one fails
the build instead of timing the wrong place.

``run`` loads that library in place of libw4.so, runs the attention projection 4096 x 3072 ->
3072 (W4A8, g = 256; 256 tiles = one per compute unit, so every workgroup is stamped) once
after an idle pause and then as the last of 60 back-to-back launches, and prints the median,
10th and 90th percentile of each phase over the 1024 waves.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

from . import build as _b

PHASE_DIR = os.path.join(_b.PKG, "_phase")
PHASE_SRC = os.path.join(PHASE_DIR, "gemm_phase.hip")
PHASE_LIB = os.path.join(PHASE_DIR, "libw4phase.so")
N_WG = 256  # stamped workgroups (one per tile of the probed shape)

# (anchor, replacement) pairs applied in order; each anchor must occur exactly once
_EDITS = [
    ("namespace w4 {\n",
     "namespace w4 {\n__device__ unsigned long long g_phase_ts[%d * 4 * 8];\n" % N_WG),
    ("""    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using L = Lay<ABITS>;
    const int tid = threadIdx.x;""",
     """    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using L = Lay<ABITS>;
    constexpr bool STAMP = EPI == kEpiBf16 && !PAIR && !KTAIL && !ASYM;
    unsigned long long pts[5] = {0, 0, 0, 0, 0};
    if constexpr (STAMP) pts[0] = __builtin_amdgcn_s_memrealtime();
    const int tid = threadIdx.x;"""),
    ("""    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
""",
     """    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (STAMP) pts[1] = __builtin_amdgcn_s_memrealtime();
"""),
    ("""    if constexpr (EPI == kEpiPartial) {
        // raw accumulators""",
     """    if constexpr (STAMP) {
        asm volatile("" :: "v"(acc[0][0][0]), "v"(acc[FN - 1][FM - 1][15]));
        pts[2] = __builtin_amdgcn_s_memrealtime();
    }
    if constexpr (EPI == kEpiPartial) {
        // raw accumulators"""),
    ("""        store_block(mrow0);
    }
}""",
     """        store_block(mrow0);
    }
    if constexpr (STAMP) {
        pts[3] = __builtin_amdgcn_s_memrealtime();
        wait_vmcnt<0>();
        pts[4] = __builtin_amdgcn_s_memrealtime();
        if (lane == 0 && blockIdx.x < %d) {
            unsigned long long *o = g_phase_ts + ((int64_t)blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * 8;
            for (int q = 0; q < 5; ++q) o[q] = pts[q];
        }
    }
}""" % N_WG),
]

_EXPORT = """
extern "C" int w4_phase_stamps(unsigned long long *host) {
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(w4::g_phase_ts), sizeof(unsigned long long) * %d * 4 * 8, 0,
                                    hipMemcpyDeviceToHost);
}
""" % N_WG


def build(verbose: bool = False) -> str:
    """Write the stamped copy of gemm.hip and link libw4phase.so with the other objects."""
    src = open(os.path.join(_b.CSRC, "gemm.hip")).read()
    for anchor, repl in _EDITS:
        n = src.count(anchor)
        if n != 1:
            raise RuntimeError("phase probe: anchor found %d times in gemm.hip:\n%s" % (n, anchor))
        src = src.replace(anchor, repl)
    os.makedirs(PHASE_DIR, exist_ok=True)
    with open(PHASE_SRC, "w") as f:
        f.write(src + _EXPORT)
    _b.build(verbose)  # the other objects, current with their sources
    obj = os.path.join(PHASE_DIR, "gemm_phase.o")
    cmd = [_b._hipcc()] + _b.FLAGS + ["-x", "hip", "-c", PHASE_SRC, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode:
        raise RuntimeError("hipcc failed on the phase copy:\n" + r.stdout)
    objs = [os.path.join(_b.OBJDIR, os.path.splitext(s)[0] + ".o") for s in _b.SOURCES if s != "gemm.hip"]
    _b._link([obj] + objs, PHASE_LIB, verbose)
    return PHASE_LIB


def run() -> None:
    import numpy as np
    import torch

    import int4_weight_quantized_block_amd as w4
    import synth

    if not os.path.exists(PHASE_LIB):
        raise ImportError("%s is not built; run `python -m int4_weight_quantized_block_amd.phase_probe build`"
                          % PHASE_LIB)
    w4.library_path = lambda: PHASE_LIB  # the binding loads the stamped library instead of libw4.so
    lib = w4.load_library()
    get = lib.w4_phase_stamps
    get.argtypes, get.restype = [ctypes.c_void_p], ctypes.c_int
    dev = "cuda:0"
    d = synth.attn_proj(device=dev)
    packed, sw, _ = w4.w4_pack_weights(d["W"], 256, False)
    q, sx, rs = w4.w4_rotate_quant_act(d["X"], 256, 8)
    Y = torch.empty((d["X"].shape[0], d["W"].shape[0]), dtype=torch.bfloat16, device=dev)
    if (Y.shape[0] // 256) * (Y.shape[1] // 192) != N_WG:
        raise RuntimeError("phase probe: the probed shape must have %d tiles" % N_WG)
    buf = np.zeros(N_WG * 4 * 8, dtype=np.uint64)

    def launch(n):
        for _ in range(n):
            w4.w4_linear_cached_rot(q, sx, rs, 8, packed, sw, bias=d["bias"], out=Y)

    def report(tag):
        if get(buf.ctypes.data) != 0:
            raise RuntimeError("w4_phase_stamps failed")
        t = buf.reshape(N_WG * 4, 8)[:, :5].astype(np.int64) * 0.01  # 100 MHz ticks -> us
        ph = np.diff(t, axis=1)
        print("%s: kernel span %.2f us (first stamp to last), start spread %.2f us" % (
            tag, t[:, 4].max() - t[:, 0].min(), t[:, 0].max() - t[:, 0].min()), flush=True)
        for i, name in enumerate(["prologue (to the first stage's data)", "main loop",
                                  "epilogue (to the last store issued)", "store drain"]):
            v = ph[:, i]
            print("  %-38s median %6.2f  p10 %6.2f  p90 %6.2f us" % (
                name, np.median(v), np.percentile(v, 10), np.percentile(v, 90)), flush=True)

    import time
    launch(2)
    torch.cuda.synchronize()
    time.sleep(0.2)
    launch(1)
    torch.cuda.synchronize()
    report("one launch after idle")
    launch(60)
    torch.cuda.synchronize()
    report("last of 60 back to back")


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "build":
        print(build(verbose="-v" in sys.argv))
    elif len(sys.argv) > 1 and sys.argv[1] == "run":
        run()
    else:
        print(__doc__)
