"""Per-stage timing of the 2-layer d=64 h=256 MFMA kernel from clock stamps.

    python -m test_learned_neural_amd.stage_stamps --build   # compile the instrumented library (CPU)
    python -m test_learned_neural_amd.stage_stamps           # run it on the GPU and print the table
    python -m test_learned_neural_amd.stage_stamps --isa     # instruction mix per stage (CPU, static)

The instrumented build (-DTM_STAGE_STAMPS=1, a separate library beside the
product one) makes the eight waves of the first key-side workgroup record the
shader clock at every stage boundary of 64 chunks of its first stream.  With
--retrieval (build and run) the stamps come from the first retrieval
workgroup of a few-stream launch instead (-DTM_STAMP_R=1, a library of its
own).  The table gives, per stage, the median over those chunks of each
wave's cycles, as the minimum, median and maximum over the waves (the
maximum across waves is what the barrier that follows waits for).
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
STAMPS_LIB = os.path.join(PKG, "libtitans_mem_stamps.so")
STAMPS_R_LIB = os.path.join(PKG, "libtitans_mem_stamps_r.so")
STAGES = 24
WAVES = 8
CHUNKS = 64

STAGE_NAMES = [
    "chunk inputs from the staging area into LDS",
    "barrier; next chunk's prefetch issued",
    "(empty)",
    "state fragments and W2/S2 copies; Z1 = K W1^T, SiLU, SiLU'; A1 copy",
    "barrier",
    "(empty)",
    "(empty)",
    "O over the workgroup's units; partials published",
    "V loads; coefficients; raw scores Q K^T and Q W1^T, Q S1^T",
    "wait for the partner's O (every thread its own words)",
    "O sum, Delta2, last chunk's y finished",
    "barrier",
    "Delta2 copies, masked scores SC1, update weights",
    "barrier",
    "Delta1 = (Delta2 W2) * SiLU'",
    "Zq1, H1 = SiLU",
    "layer-1 fold into W1, S1",
    "barrier; H1 copy",
    "barrier",
    "masked scores D o (H1 A1^T)",
    "layer-2 fold into W2, S2",
    "barrier; y tiles, kept or sent",
    "barrier (end of chunk)",
]

STAGE_NAMES_R = [
    "chunk inputs into LDS",
    "barrier; next chunk's prefetch; copies' words requested",
    "coefficients",
    "raw scores Q K^T",
    "barrier",
    "masked scores SC1; remaining words requested",
    "wait: W2, S2 copies and A1",
    "wait: Delta2 and the query products",
    "wait: Delta1; receipt",
    "copies into LDS; last chunk's y finished",
    "barrier",
    "Zq1, H1 = SiLU",
    "barrier",
    "H1 copy",
    "barrier",
    "masked scores D o (H1 A1^T)",
    "barrier",
    "y tiles, kept or sent",
    "barrier (end of chunk)",
    "(empty)",
    "(empty)",
    "(empty)",
    "(empty)",
]


def build(retrieval: bool = False):
    sys.path.insert(0, ROOT)
    from test_learned_neural_amd import build as b
    if retrieval:
        b.build(verbose=True, extra=["-DTM_STAGE_STAMPS=1", "-DTM_STAMP_R=1"], out=STAMPS_R_LIB,
                build_dir=os.path.join(ROOT, "_build", "stamps_r"))
    else:
        b.build(verbose=True, extra=["-DTM_STAGE_STAMPS=1"], out=STAMPS_LIB,
                build_dir=os.path.join(ROOT, "_build", "stamps"))


def isa():
    """Static instruction counts of the instrumented build between consecutive
    stage stamps (s_memtime) of the read-after-write instance, from its gfx950
    assembly.  Straight-line counts: each branch's blocks count once, loops
    once per body, and the compiler may move work across a stamp."""
    import re
    import subprocess
    import tempfile
    sys.path.insert(0, ROOT)
    from test_learned_neural_amd import build as b
    src = os.path.join(b.CSRC, "tm_mlp2_group.hip")
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "k.s")
        subprocess.check_call([b.hipcc()] + b.COMMON + ["-DTM_STAGE_STAMPS=1", "-x", "hip"] + b.DEVICE +
                              b.PER_FILE["tm_mlp2_group.hip"] + ["--cuda-device-only", "-S", src, "-o", out],
                              stderr=subprocess.DEVNULL)
        lines = open(out).read().split("\n")
    start = next(i for i, l in enumerate(lines) if re.match(r"^_Z\S*mlp2_group_kernelILb1ELi8ELb0ELb0E\S*:", l))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    body = lines[start:end]
    stamps = [i for i, l in enumerate(body) if "s_memtime" in l]
    classes = ["valu", "trans", "lane", "mfma", "lds", "vmem", "salu"]

    def cls(op):
        if op.startswith("v_mfma"):
            return "mfma"
        if op.startswith(("v_readlane", "v_readfirstlane", "v_writelane")):
            return "lane"
        if op.startswith(("v_exp", "v_rcp", "v_log", "v_sqrt", "v_rsq")):
            return "trans"
        if op.startswith("v_"):
            return "valu"
        if op.startswith("ds_"):
            return "lds"
        if op.startswith(("global_", "buffer_", "flat_", "scratch_")):
            return "vmem"
        if op.startswith("s_") and not op.startswith(("s_waitcnt", "s_barrier", "s_nop")):
            return "salu"
        return None

    print("static instructions per stage (read-after-write instance; 'valu' excludes transcendental and lane ops)")
    print(f"  {'stage':<62s}" + "".join(f"{c:>7s}" for c in classes))
    tot = dict.fromkeys(classes, 0)
    for k, (a, z) in enumerate(zip(stamps, stamps[1:])):
        cnt = dict.fromkeys(classes, 0)
        for l in body[a + 1:z]:
            t = l.strip().split()
            if not t or t[0].startswith((";", ".")) or t[0].endswith(":"):
                continue
            c = cls(t[0])
            if c:
                cnt[c] += 1
        for c in classes:
            tot[c] += cnt[c]
        name = STAGE_NAMES[k] if k < len(STAGE_NAMES) else f"stage {k + 1}"
        print(f"  {k + 1:2d} {name[:59]:<59s}" + "".join(f"{cnt[c]:7d}" for c in classes))
    print(f"  {'total':<62s}" + "".join(f"{tot[c]:7d}" for c in classes))


def run(steps: int = 2, per_wave: bool = False, workload: str = "headline", retrieval: bool = False):
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    from test_learned_neural_amd import titans_mem as tmm
    from test_learned_neural_amd import workloads as wl
    lib_path = STAMPS_R_LIB if retrieval else STAMPS_LIB
    names = STAGE_NAMES_R if retrieval else STAGE_NAMES
    if not os.path.exists(lib_path):
        raise SystemExit(f"{lib_path} is missing: run with --build first")
    tmm.LIB_PATH = lib_path
    lib = tmm.load()
    cfg = wl.WORKLOADS[workload]
    inp = wl.make_inputs(cfg, workers=16)
    B, H, N, d, P = cfg.B, cfg.H, cfg.N, cfg.d, cfg.param_count
    tok = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).reshape(B, H, N, d).cuda()
    per = lambda a, n: torch.from_numpy(a).reshape(B, H, n).cuda()
    args = (tok(inp["k"]), tok(inp["v"]), tok(inp["q"]), per(inp["alpha"], N), per(inp["eta"], N),
            per(inp["theta"], N), per(inp["W0"], P), per(inp["S0"], P), cfg.chunk)
    for _ in range(steps):
        tmm.forward(*args, hidden=cfg.hidden, n_layers=cfg.n_layers)
    torch.cuda.synchronize()
    n = CHUNKS * WAVES * STAGES
    buf = (ctypes.c_ulonglong * n)()
    fn = lib.titans_mem_stage_stamps
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    assert fn(ctypes.addressof(buf), n) == 0
    st = np.frombuffer(buf, dtype=np.uint64).astype(np.int64).reshape(CHUNKS, WAVES, STAGES)
    d = np.diff(st, axis=2)                      # [chunk, wave, stage]
    med = np.median(d, axis=0)                   # [wave, stage]
    total = np.median(st[:, :, -1] - st[:, :, 0], axis=0)
    print(f"{cfg.name}: cycles per stage (median over {CHUNKS} chunks; min / median / max over {WAVES} waves)")
    for k in range(STAGES - 1):
        row = med[:, k]
        print(f"  {k + 1:2d} {names[k]:<58s} {row.min():7.0f} {np.median(row):7.0f} {row.max():7.0f}")
    if per_wave:
        print("  per wave (median over chunks), waves 0..%d:" % (WAVES - 1))
        for k in range(STAGES - 1):
            print(f"  {k + 1:2d} " + " ".join(f"{v:6.0f}" for v in med[:, k]))
    nxt = np.median(st[1:, :, 0] - st[:-1, :, 0], axis=0)
    print(f"  chunk (stamp 0 to stamp 23): {np.median(total):.0f} cycles; chunk to chunk: {np.median(nxt):.0f} cycles")


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--build", action="store_true")
    ap.add_argument("--isa", action="store_true")
    ap.add_argument("--per-wave", action="store_true", help="also print every wave's median per stage")
    ap.add_argument("--workload", default="headline", help="a 2-layer d=64 h=256 workload of workloads.py")
    ap.add_argument("--retrieval", action="store_true",
                    help="stamps of the first retrieval workgroup (few-stream workloads only)")
    a = ap.parse_args()
    if a.build:
        build(a.retrieval)
    elif a.isa:
        isa()
    else:
        run(per_wave=a.per_wave, workload=a.workload, retrieval=a.retrieval)
