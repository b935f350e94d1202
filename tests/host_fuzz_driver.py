"""Seeded random calls of every host-only entry point (configuration choice with and without an
override, the two-part cut, the tile schedule, the pipeline protocol, the swizzle), printing each
call's arguments before it runs; run in its own process by tests/test_host_fuzz.py, so that a crash
ends only this process and its last line names the arguments. Exits 2 if a call took over 0.5 s."""
import ctypes
import os
import random
import sys
import time

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import software_pipelined_tiled_amd as spt  # noqa: E402

INT = [-(1 << 31), -5, -1, 0, 1, 2, 3, 4, 5, 7, 8, 9, 16, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000,
       4096, 65536, (1 << 31) - 1]
SIZES = [0, 1, 7, 8, 9, 31, 32, 33, 64, 100, 255, 256, 257, 1023, 4093, 4096, 5119, 8192, 28672, 1 << 20, (1 << 31) - 1]


def main(seed: int, n: int) -> int:
    rng = random.Random(seed)
    pick = rng.choice
    L = spt.lib()
    for it in range(n):
        M, N, K = pick(SIZES), pick(SIZES), pick(SIZES)
        lda = max(K, 1) + pick([0, 0, 1, 8, 64])
        ldb = max(K, 1) + pick([0, 0, 1, 8])
        ldc = max(N, 1) + pick([0, 0, 3, 8])
        dt, odt = pick([0, 1]), pick([0, 1, 2])
        base = dict(bm=pick([32, 64, 128, 256]), bn=pick([32, 64, 128, 256]), bk=pick([32, 64, 128]),
                    stages=pick([1, 2, 3, 4, 5, 8]), waves=pick([2, 4, 8]), mfma=pick([0, 16, 32]),
                    persistent=pick([0, 1, 2]), group_m=pick([0, 1, 8]), load_path=pick([0, 1, 2, 3]),
                    grid=pick([0, 1, 3, 256]), lds_bytes=pick([0, 65536]), splits=pick([0, 1, 2, 3, 16]),
                    stream=pick([0, 1, 2]))
        cfg = {k: pick(INT) if rng.random() < 0.3 else v for k, v in base.items()}
        cu, lds = pick([(256, 160 * 1024), (1, 1024), (0, 0), (-1, 65536), (304, 65536), (8, 160 * 1024)])
        sched = [pick(INT) for _ in range(7)]
        proto = [pick(INT) for _ in range(5)] + [pick([0, 1, 8, 32, -1])]
        swz = [pick(INT) for _ in range(4)]
        print(it, M, N, K, lda, ldb, ldc, dt, odt, cu, lds, cfg, sched, proto, swz, flush=True)
        t0 = time.perf_counter()
        spt.gemm_select_config_status(M, N, K, dt, dt, odt, lda, ldb, ldc, cu, lds)
        spt.gemm_select_config_status(M, N, K, dt, dt, odt, lda, ldb, ldc, cu, lds, config=cfg)
        try:
            spt.gemm_select_parts(M, N, K, dt, dt, odt, lda, ldb, ldc, cu, lds)
        except spt.GemmError:
            pass
        o1, o2, o3 = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int()
        L.gemm_schedule_tile(*sched, ctypes.byref(o1), ctypes.byref(o2), ctypes.byref(o3))
        buf = (ctypes.c_int * 32)()
        L.gemm_pipeline_protocol(*proto[:5], buf, min(proto[5], 32))
        L.gemm_lds_chunk_offset(*swz)
        if time.perf_counter() - t0 > 0.5:
            print("slow", it, flush=True)
            return 2
    print("done", n, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(int(sys.argv[1]), int(sys.argv[2])))
