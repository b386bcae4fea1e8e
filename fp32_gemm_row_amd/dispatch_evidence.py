"""Measure the evidence behind each constant of the library's kernel choice.

    python -m fp32_gemm_row_amd.dispatch_evidence [--out profiles/dispatch_rules.md]

For every rule of the host dispatch (``choose()`` and the split-plan
estimates in ``csrc/solve.hip``), times the plan the library picks for a few
shapes on either side of the rule's constant against the alternative the
constant rules out, and writes a markdown table with the command that made it.
Alternatives are forced through ``fgr_solve_path`` (path and tile) or through
``fgr_set_workspace_limit(0)`` (the plan's form without a workspace: no split
of the reduction across workgroups). Time: median of per-launch HIP events
over 30 launches after 10 warm-ups, on torch's current stream; inputs uniform
in [0, 1) (the values do not change the time). Needs a GPU.
"""

from __future__ import annotations

import argparse
import os
import statistics
import sys

import fp32_gemm_row_amd as fgr

AUTO = (fgr.PATH_AUTO, fgr.TILE_AUTO, -1)
NOSPLIT = (fgr.PATH_AUTO, fgr.TILE_AUTO, 0)


def forced(path, tile=fgr.TILE_AUTO):
    return (path, tile, -1)


# (rule, constants and where, what the rule does, [(shape, [(label, alternative), ...]), ...])
RULES = [
    ("Direct-copy tail", "tail_tiles(cus) = 11 cus / 16 (choose)",
     "256x256 tiles: a last partial wave of at most 176 tiles is cut into split-kernel tiles (MFMA_DMA_TAIL)",
     [((4096, 4096, 6656), [("auto (160 left over)", AUTO), ("MFMA_DMA", forced(fgr.PATH_MFMA_DMA, 256))]),
      ((4096, 4096, 7168), [("auto (192 left over)", AUTO), ("MFMA_DMA_TAIL", forced(fgr.PATH_MFMA_DMA_TAIL, 256))])]),
    ("k-split tail", "ksplit_tail_tiles(cus) = cus / 2 (choose, launch_ksplit_tail)",
     "k-split tiles: a last partial wave of at most 128 tiles goes to the tail form",
     [((3584, 3584, 3584), [("auto (128x128, 16 left over)", AUTO),
                            ("MFMA_KSPLIT 128", forced(fgr.PATH_MFMA_KSPLIT, 128))]),
      ((3001, 3001, 3001), [("auto (64x64, 161 left over)", AUTO),
                            ("MFMA_KSPLIT_TAIL 64", forced(fgr.PATH_MFMA_KSPLIT_TAIL, 64))])]),
    ("128x128 or 64x64 k-split tiles",
     "t128 == 0 mod cus, t128 >= 3 cus or a last wave > 3 cus / 4 (choose)",
     "128x128 tiles in whole waves, from three waves on or with a last wave more than 3/4 full; else 64x64",
     [((2047, 2047, 2047), [("auto (128x128, one wave)", AUTO),
                            ("MFMA_KSPLIT 64", forced(fgr.PATH_MFMA_KSPLIT, 64))]),
      ((2816, 2816, 2816), [("auto (128x128, 484 tiles)", AUTO),
                            ("MFMA_KSPLIT 64", forced(fgr.PATH_MFMA_KSPLIT, 64))]),
      ((2304, 2304, 2304), [("auto (64x64; 324 of 128)", AUTO),
                            ("MFMA_KSPLIT_TAIL 128", forced(fgr.PATH_MFMA_KSPLIT_TAIL, 128))]),
      ((2560, 2560, 2560), [("auto (64x64; 400 of 128)", AUTO),
                            ("MFMA_KSPLIT 128", forced(fgr.PATH_MFMA_KSPLIT, 128))]),
      ((3072, 3072, 3072), [("auto (aligned, 64x64; 576 of 128)", AUTO),
                            ("MFMA_KSPLIT_TAIL 128", forced(fgr.PATH_MFMA_KSPLIT_TAIL, 128))]),
      ((2048, 4096, 4096), [("auto (aligned, 128x128, two whole waves)", AUTO),
                            ("MFMA_KSPLIT 64", forced(fgr.PATH_MFMA_KSPLIT, 64))]),
      ((3001, 3001, 3001), [("auto (64x64; 576 of 128)", AUTO),
                            ("MFMA_KSPLIT_TAIL 128", forced(fgr.PATH_MFMA_KSPLIT_TAIL, 128))])]),
    ("Short reductions", "kShortReduction = 104, kShortReductionWholeWaves = 72 (choose)",
     "N < 104 (N < 72 with every row aligned and whole waves of 256x256 tiles) with a 64x64 tile per CU: "
     "register-staged 64x64 tiles instead of the direct-copy kernel",
     [((8192, 64, 8192), [("auto", AUTO), ("MFMA_DMA", forced(fgr.PATH_MFMA_DMA, 256))]),
      ((8192, 80, 8192), [("auto (whole waves)", AUTO), ("MFMA_VEC 64", forced(fgr.PATH_MFMA_VEC, 64))]),
      ((8192, 96, 8192), [("auto (whole waves)", AUTO), ("MFMA_VEC 64", forced(fgr.PATH_MFMA_VEC, 64))]),
      ((6144, 80, 6144), [("auto (partial wave)", AUTO), ("MFMA_DMA_TAIL", forced(fgr.PATH_MFMA_DMA_TAIL, 256))]),
      ((65792, 96, 256), [("auto", AUTO), ("MFMA_DMA_TAIL", forced(fgr.PATH_MFMA_DMA_TAIL, 256))]),
      ((4096, 96, 4096), [("auto (whole waves)", AUTO), ("MFMA_VEC 64", forced(fgr.PATH_MFMA_VEC, 64))]),
      ((8192, 112, 8192), [("auto", AUTO), ("MFMA_VEC 64", forced(fgr.PATH_MFMA_VEC, 64))])]),
    ("Short reductions, unaligned B", "kShortReduction = 104, kShortReductionNarrowB = 384 (choose)",
     "unaligned rows: 32-bit register-staged tiles up to N = 104, and up to N = 384 where the direct-copy "
     "kernel would copy B 4 bytes at a time",
     [((8191, 65, 8191), [("auto", AUTO), ("MFMA_DMA", forced(fgr.PATH_MFMA_DMA, 256))]),
      ((8191, 255, 8191), [("auto", AUTO), ("MFMA_DMA", forced(fgr.PATH_MFMA_DMA, 256))]),
      ((8191, 128, 8191), [("auto (A aligned)", AUTO), ("MFMA_DMA", forced(fgr.PATH_MFMA_DMA, 256))]),
      ((8191, 511, 8191), [("auto", AUTO), ("MFMA_SCALAR 128", forced(fgr.PATH_MFMA_SCALAR, 128))]),
      ((8192, 129, 8192), [("auto (B aligned)", AUTO), ("MFMA_SCALAR 128", forced(fgr.PATH_MFMA_SCALAR, 128))])]),
    ("Matrix-vector rows", "kSkinnyMinM = 5, kGemvMaxRows = 8 (choose)",
     "M <= 4: the matrix-vector kernel; 5 <= M <= 8 with N >= 64 and K >= 128: the k-split / split plans",
     [((4, 8192, 8192), [("auto", AUTO), ("MFMA_SPLITK 32x128", forced(fgr.PATH_MFMA_SPLITK, fgr.TILE_32X128))]),
      ((5, 4096, 1024), [("auto", AUTO), ("GEMV_VEC", forced(fgr.PATH_GEMV_VEC))]),
      ((8, 2048, 2048), [("auto", AUTO), ("GEMV_VEC", forced(fgr.PATH_GEMV_VEC))])]),
    ("Skinny tiles", "kSkinnyMinB = 16 Mi, kSkinnyWideB = 32 Mi, kSkinnyMaxM = 64 (skinny_b, choose)",
     "5 <= M <= 64 with a large B: 32x128 tiles streaming B once",
     [((16, 4096, 2048), [("auto (B 8 Mi)", AUTO), ("MFMA_SPLITK 32x128", forced(fgr.PATH_MFMA_SPLITK, fgr.TILE_32X128))]),
      ((16, 8192, 8192), [("auto (B 64 Mi)", AUTO), ("MFMA_SPLITK 32", forced(fgr.PATH_MFMA_SPLITK, 32))]),
      ((64, 8192, 8192), [("auto (two rows of tiles)", AUTO), ("MFMA_SPLITK 64", forced(fgr.PATH_MFMA_SPLITK, 64))])]),
    ("Matrix-vector split", "gemv_time, kGemvMinPart = 1024 (gemv_plan)",
     "few 32-column blocks: rows of B split over workgroups when the time estimate says so",
     [((1, 16384, 1024), [("auto", AUTO), ("no split", NOSPLIT)]),
      ((4, 8192, 1024), [("auto", AUTO), ("no split", NOSPLIT)]),
      ((1, 8192, 8192), [("auto", AUTO), ("no split", NOSPLIT)])]),
    ("Split reduction", "splitk_time, kSplitkMinPart = 256 (splitk_plan)",
     "fewer 64x64 tiles than CUs and a long N: each tile's reduction split into P parts",
     [((128, 262144, 128), [("auto", AUTO), ("no split", NOSPLIT), ("MFMA_SPLITK 32", forced(fgr.PATH_MFMA_SPLITK, 32))]),
      ((512, 8192, 512), [("auto", AUTO), ("no split", NOSPLIT)]),
      ((96, 8192, 4096), [("auto", AUTO), ("no split", NOSPLIT), ("MFMA_SPLITK 64", forced(fgr.PATH_MFMA_SPLITK, 64))])]),
    ("Split reduction, 128x128 tiles", "kSplitk128MinPart = 2048 (choose)",
     "split plans take 128x128 tiles when their parts are at least 2048 long and they pad no more",
     [((128, 2097152, 128), [("auto", AUTO), ("MFMA_SPLITK 64", forced(fgr.PATH_MFMA_SPLITK, 64))]),
      ((128, 262144, 128), [("auto", AUTO), ("MFMA_SPLITK 128", forced(fgr.PATH_MFMA_SPLITK, 128))]),
      ((512, 65536, 512), [("auto", AUTO), ("MFMA_SPLITK 64", forced(fgr.PATH_MFMA_SPLITK, 64))])]),
    ("k-split tail split", "kMixedTailMinN = 1024, kTailSplitMinN = 4096 (launch_ksplit_tail)",
     "a partial last wave of 64x64 tiles with N >= 1024 splits its tiles' reduction in the whole tiles' grid",
     [((1023, 4097, 1039), [("auto", AUTO), ("no split (split-kernel tail)", NOSPLIT)]),
      ((1536, 4096, 1536), [("auto", AUTO), ("no split (split-kernel tail)", NOSPLIT)])]),
    ("Unaligned whole-device shapes", "kKsplitUnalignedMinN = 768, t256 mod cus (choose)",
     "neither operand's rows aligned, enough 256x256 tiles: direct copies in whole waves of 256x256 tiles "
     "or below N = 768, else 128x128 k-split tiles",
     [((8191, 6143, 4095), [("auto (two whole waves)", AUTO), ("MFMA_KSPLIT 128", forced(fgr.PATH_MFMA_KSPLIT, 128))]),
      ((8191, 1023, 8191), [("auto (four whole waves)", AUTO), ("MFMA_KSPLIT 128", forced(fgr.PATH_MFMA_KSPLIT, 128))]),
      ((4095, 4097, 4099), [("auto (272 tiles)", AUTO), ("MFMA_DMA_TAIL", forced(fgr.PATH_MFMA_DMA_TAIL, 256))]),
      ((6143, 4095, 6143), [("auto (576 tiles)", AUTO), ("MFMA_DMA_TAIL", forced(fgr.PATH_MFMA_DMA_TAIL, 256))]),
      ((8191, 511, 8191), [("auto", AUTO), ("MFMA_KSPLIT 128", forced(fgr.PATH_MFMA_KSPLIT, 128))]),
      ((4096, 4096, 4095), [("auto (A aligned)", AUTO), ("MFMA_KSPLIT 128", forced(fgr.PATH_MFMA_KSPLIT, 128))])]),
    ("Column strip", "kStripMax = 8 (strip_plan_ok)",
     "K = 64 q + w, w <= 8: tiles on the q column blocks, the w columns on the vector ALUs, one launch",
     [((1023, 1025, 1027), [("auto", AUTO), ("MFMA_KSPLIT_TAIL 64", forced(fgr.PATH_MFMA_KSPLIT_TAIL, 64))]),
      ((1023, 1025, 1032), [("auto", AUTO), ("MFMA_KSPLIT_TAIL 64", forced(fgr.PATH_MFMA_KSPLIT_TAIL, 64))])]),
]


def time_call(fn, steps=30, warmup=10):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s, e in ev:
        s.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    return statistics.median(s.elapsed_time(e) for s, e in ev) * 1e3  # us


def measure(M, N, K, alt):
    import torch

    path, tile, limit = alt
    A = torch.rand(M * N, device="cuda")
    B = torch.rand(N * K, device="cuda")
    C = torch.empty(M * K, device="cuda")
    prev = fgr.set_workspace_limit(limit)
    try:
        if path == fgr.PATH_AUTO and tile == fgr.TILE_AUTO:
            us = time_call(lambda: fgr.solve(A, B, C, M, N, K))
        else:
            us = time_call(lambda: fgr.solve_path(A, B, C, M, N, K, path, tile))
    finally:
        fgr.set_workspace_limit(prev)
    return us


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    ap.add_argument("--out", default=os.path.join(root, "profiles", "dispatch_rules.md"))
    args = ap.parse_args()
    import torch

    if not torch.cuda.is_available():
        print("dispatch_evidence needs a GPU", file=sys.stderr)
        return 2
    fgr.load_library()
    lines = [
        "# Dispatch rules: the measurements behind each constant",
        "",
        "Command: `python -m fp32_gemm_row_amd.dispatch_evidence` (run from the repository root on one MI355X).",
        "Median of 30 per-launch HIP events after 10 warm-ups, microseconds per call (host launch cost included",
        "where it exceeds the GPU time). 'auto' is the plan `solve()` picks; 'no split' is that plan with",
        "`fgr_set_workspace_limit(0)` (its form without a workspace). **Bold**: the faster of the plans timed.",
        "",
    ]
    total = agree = 0
    for name, const, what, cases in RULES:
        lines += [f"## {name}", "", f"- Constant: `{const}`", f"- Rule: {what}", "",
                  "| M x N x K | plan picked | " + " | ".join(f"alt {i + 1}" for i in range(3)) + " |",
                  "|---|---|---|---|---|"]
        for (M, N, K), alts in cases:
            picked = fgr.PATH_NAMES.get(fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K))
            ptile = fgr.select_tile(1 << 40, 2 << 40, 3 << 40, M, N, K)
            res = []
            for label, alt in alts:
                us = measure(M, N, K, alt)
                res.append((label, us))
                print(f"{name}: {M}x{N}x{K} {label}: {us:.1f} us", flush=True)
            best = min(us for _, us in res)
            cells = [f"**{lab}: {us:.1f}**" if us == best else f"{lab}: {us:.1f}" for lab, us in res]
            cells += [""] * (3 - len(cells))
            lines.append(f"| {M}x{N}x{K} | {picked} {ptile} | " + " | ".join(cells) + " |")
            total += 1
            agree += res[0][1] <= best * 1.03
        lines.append("")
    lines += [
        f"The automatic plan is the fastest timed (or within 3% of it) on {agree} of {total} shapes.",
        "",
        "Constants not reachable through the boundary: `kTileGroup = 4` (tile-rows per group of the workgroup",
        "order; a compile-time constant), and the host-side workspace constants `kPoolKeepBytes`,",
        "`kCachedStreams`, `kCachedMaxBytes` (they change host time per call, not the kernels).",
        "",
    ]
    with open(args.out, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines))
    print(args.out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
