"""Per-phase timeline of the persistent B = 1 block kernel (GR00T_FLAG_PERSIST).

A diagnostic build of the library (GR00T_PHASE_TRACE: every workgroup pair (XCD 0, ticket 0)
and (XCD 7, ticket 31) records s_memrealtime at the 16 phase boundaries of each block) runs
get_action at B = 1 on the 32-block bf16 model with 300 VL tokens (256 image + 44 text), then
the timestamps of the last Euler step are read back and averaged per phase over both
workgroups and all blocks. The product library is not touched.

usage:
  python -m flow_matching_dit_amd.phase_trace --build          # compile the diagnostic library (no GPU)
  python -m flow_matching_dit_amd.phase_trace [--calls N]      # run it on the GPU, print a markdown table
"""
import argparse
import ctypes
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TRACE_LIB = os.path.join(HERE, "lib_trace", "libgr00t_head_trace.so")
PHASES = ["adaLN", "q / q,k,v", "XCD wait", "attention", "XCD wait", "o projection", "device wait",
          "residual", "XCD wait", "LayerNorm", "MLP up + GELU", "XCD wait", "MLP down", "device wait",
          "residual + XCD wait"]
WORDS = 2 * 64 * 16  # persist_trace_words()


def build():
    from flow_matching_dit_amd import build as B
    return B.build(verbose=True, lib=TRACE_LIB, build_dir=os.path.join(HERE, "_build_trace"),
                   defines=("GR00T_PHASE_TRACE",))


def run(calls: int):
    import torch
    from flow_matching_dit_amd import head as H
    from flow_matching_dit_amd import synth
    lib = H.load_library(TRACE_LIB)
    lib.gr00t_persist_phase_trace.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint64), ctypes.c_int32]
    lib.gr00t_persist_phase_trace.restype = ctypes.c_int
    w = synth.WORKLOADS["dit32_bf16_b1"]
    wt, inp, nz = synth.make_weights(w), synth.make_inputs(w), synth.make_noise(w)
    h = H.Gr00tHead(w.cfg, 1, w.vl_len, H.FLAG_PERSIST)
    h.load_weights(wt).finalize()
    d = H.device_inputs(inp, nz, h.act_torch_dtype)
    out = torch.empty((1, w.cfg.action_horizon, w.cfg.action_dim), dtype=torch.float32, device="cuda:0")
    nl = w.cfg.num_layers
    per_phase = [[] for _ in PHASES]
    block_us, step_us = [], []
    buf = (ctypes.c_uint64 * WORDS)()
    for _ in range(calls):
        h.get_action(**d, out=out)
        torch.cuda.synchronize()
        rc = lib.gr00t_persist_phase_trace(h.h, buf, WORDS)
        if rc != 0:
            sys.exit(f"gr00t_persist_phase_trace failed ({rc})")
        ts = list(buf)
        for wg in range(2):
            for l in range(nl):
                row = ts[(wg * 64 + l) * 16:(wg * 64 + l) * 16 + 16]
                for p in range(1, 16):
                    per_phase[p - 1].append((row[p] - row[p - 1]) * 0.01)
                block_us.append((row[15] - row[0]) * 0.01)
        step_us.append((ts[(nl - 1) * 16 + 13] - ts[0]) * 0.01)
    h.close()
    means = [statistics.fmean(v) for v in per_phase]
    print(f"B = 1, {nl} blocks, {calls} calls (the last Euler step of each), two workgroups per block:")
    print(f"mean block {statistics.fmean(block_us):.2f} us, step (block 0 start to the last block's "
          f"final device wait) {statistics.median(step_us):.1f} us\n")
    print("| " + " | ".join(PHASES) + " |")
    print("|" + "---|" * len(PHASES))
    print("| " + " | ".join(f"{m:.2f}" for m in means) + " |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--build", action="store_true")
    ap.add_argument("--calls", type=int, default=10)
    args = ap.parse_args()
    if args.build:
        build()
    else:
        run(args.calls)


if __name__ == "__main__":
    main()
