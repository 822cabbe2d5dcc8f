"""Benchmark: bs=1 block-diffusion decode of the Qwen3-4B-shaped random-init model on one GPU.

The workload is the generation of 4096 new tokens after a 256-token prompt: 128 blocks of 32,
block b decoded at prefix 256 + 32 b (256 .. 4320, mean 2288).  A step is one block:
ceil(32 / k) denoising rounds (self-conditioning input, 36 layers, fused head statistics,
commit) plus the commit pass that writes a block's K/V, as one replay of the library's
captured graph.  By default blocks are pipelined: each block's round 0 also carries the
pending commit pass of the block before it (dlm_decode_block_pipelined, one 64-row forward),
so a block streams the weights ceil(32 / k) times; --separate-commit runs every block with its
own commit pass instead (dlm_decode_block).

The timed region runs exactly --steps blocks, spread evenly over the 128 blocks of the
generation (step i decodes block floor((i + 1/2) 128 / steps) at that block's prefix; with
--steps 128 every block once), so the time per block, the tokens/s and the roofline fraction
are those of the whole 4096-token generation whatever --steps is; the prefix is set on the
device before each block and the block's token readback is queued after it.  A second leg
decodes the 128 blocks in order, as one generation (full_generation).  Prefill is timed on its
own.  The headline k runs on every seed of --seeds (a new model and prompt each; the value is
the median), the other k values and legs on --seed.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
METRIC = "bs=1 block-decode tokens/s at fixed k commits/round; rounds/s; % HBM roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(shape, L, head_rows=32, kv_elem_bytes=2):
    """HBM bytes one round must move at prefix length L: every weight once, the
    embedding once for the head, the adapter, the prefix + block K/V of every layer
    (kv_elem_bytes per cached element: 2 for bf16, 1 for an FP8 cache)."""
    s = shape
    D = s.head_dim
    per_layer = 2 * ((s.hq + 2 * s.hkv) * D * s.d + s.d * s.hq * D + 3 * s.ffn * s.d)
    w = s.n_layers * per_layer + 2 * s.d * s.d          # layers + W_sc
    head = 2 * s.vocab * s.d
    kv = s.n_layers * 2 * kv_elem_bytes * s.hkv * D * (L + s.block)
    return w + head + kv


FP8_CACHE_SCALES = (0.0625, 0.0625)     # k, v: |k|, |v| up to 28 before saturation


COUNTERS = os.path.join(ROOT, "profiles", "gate_up_swiglu_qwen4b_counters.txt")
KERNEL_SOURCES = ["block_diffusion_decoding_denoise_amd/csrc/gemm.hip", "block_diffusion_decoding_denoise_amd/csrc/gemm.h",
                  "block_diffusion_decoding_denoise_amd/csrc/common.h"]


def counter_traffic():
    """HBM bytes per launch of the gate/up kernel from the committed FETCH_SIZE / WRITE_SIZE
    counter runs, or None when the kernel sources changed since those runs."""
    import hashlib
    try:
        fields = {}
        for line in open(COUNTERS):
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.split()[0] if v.split() else ""
        h = hashlib.sha256()
        for f in KERNEL_SOURCES:
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        if fields.get("kernel_source_sha256") != h.hexdigest():
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def commit_pass_bytes(shape, L):
    s = shape
    D = s.head_dim
    per_layer = 2 * ((s.hq + 2 * s.hkv) * D * s.d + s.d * s.hq * D + 3 * s.ffn * s.d)
    last = 2 * (s.hq + 2 * s.hkv) * D * s.d
    kv = (s.n_layers - 1) * 2 * 2 * s.hkv * D * (L + s.block)
    return (s.n_layers - 1) * per_layer + last + kv


def moe_dense_pass_bytes(s, L, with_head):
    """Bytes of one forward of the MoE model apart from the routed experts: attention weights,
    router, KV, and (rounds) the head and the adapter."""
    D = s.head_dim
    attn_w = 2 * ((s.hq + 2 * s.hkv) * D * s.d + s.d * s.hq * D)
    per_layer = attn_w + 2 * s.n_experts * s.d + 2 * 2 * s.hkv * D * (L + s.block)
    if with_head:
        return s.n_layers * per_layer + 2 * s.vocab * s.d + 2 * s.d * s.d
    last = 2 * (s.hq + 2 * s.hkv) * D * s.d
    return (s.n_layers - 1) * per_layer + last


def moe_expert_bytes(s):
    F, d = s.expert_ffn, s.d
    return 2 * F * d // 2 + 2 * F * d // 32 + d * F // 2 + d * F // 32


def run_ops(torch, dlm, emb, seed):
    """The head and attention ops alone at their workload sizes (the head with 32 / 24 / 16 / 0
    open rows of 32 over the 151,936 x 2560 embedding; attention with 32 / 8 heads of 128, a
    32-query block, prefix 512 / 4096 / 32768, over a bf16 and over an FP8 e4m3 cache), each
    call replayed from a captured graph and timed with HIP events; bytes are the algorithmic
    ones (every embedding or K/V byte once)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    V, d = emb.shape
    out = {"head": [], "attention": []}
    # ---- head: rows N(0, 1) normalised to unit RMS, in bf16; committed rows by a seeded permutation
    h = torch.randn(32, d, device="cuda", generator=g)
    h = (h / h.pow(2).mean(dim=1, keepdim=True).sqrt()).to(torch.bfloat16)
    perm = torch.randperm(32, device="cuda", generator=g)
    ws = torch.empty(128 << 20, dtype=torch.uint8, device="cuda")
    for n_committed in (0, 8, 16, 32):
        committed = torch.zeros(32, dtype=torch.uint8, device="cuda")
        committed[perm[:n_committed]] = 1
        dlm.head_rowstats(h, emb, committed, ws=ws)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(4):
                dlm.head_rowstats(h, emb, committed, ws=ws)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3 / 20
        m = 32 - n_committed
        nbytes = V * d * 2 + m * d * 2 + 32 * (4 * 4 + d * 4) if m else 0
        out["head"].append({"open_rows": m, "us": round(t * 1e6, 2),
                            "GB_s": round(nbytes / t / 1e9, 1), "frac": round(nbytes / t / HBM_PEAK, 4)})
    del ws
    # ---- attention: K/V copies rotated so that at least 512 MiB is cycled (short prefixes would
    # otherwise sit in the 256 MB memory-side cache)
    hq, hkv, D, B = 32, 8, 128, 32
    out["attention_fp8_cache"] = []
    for kv in ("bf16", "fp8"):
        es = 2 if kv == "bf16" else 1
        for L in (512, 4096, 32768):
            cap = (L + B + 31) // 32 * 32
            per = 2 * hkv * cap * D * es
            n = max(2, -(-(512 << 20) // per))
            if kv == "bf16":
                kc = torch.randn(n, hkv, cap, D, device="cuda", generator=g).to(torch.bfloat16)
                vc = torch.randn(n, hkv, cap // 32, D, 32, device="cuda", generator=g).to(torch.bfloat16)
                scales = None
            else:
                # e4m3 codes of magnitude <= 7.5 with random signs (no NaN codes)
                def codes(*shape):
                    mag = torch.randint(0, 0x50, shape, device="cuda", generator=g, dtype=torch.int32)
                    sgn = torch.randint(0, 2, shape, device="cuda", generator=g, dtype=torch.int32) << 7
                    return (mag | sgn).to(torch.uint8)
                kc = codes(n, hkv, cap, D)
                vc = codes(n, hkv, cap // 32, D, 32)
                scales = (0.125, 0.2)
            q = torch.randn(B, hq, D, device="cuda", generator=g).to(torch.bfloat16)
            o = torch.empty_like(q)
            aws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
            dlm.block_attn(q, kc[0], vc[0], L, out=o, ws=aws, kv_scales=scales)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(n):
                    dlm.block_attn(q, kc[i], vc[i], L, out=o, ws=aws, kv_scales=scales)
            graph.replay()
            torch.cuda.synchronize()
            reps = max(1, 200 // n)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / 1e3 / (reps * n)
            nbytes = (L + B) * hkv * D * es * 2 + 2 * B * hq * D * 2
            out["attention" if kv == "bf16" else "attention_fp8_cache"].append(
                {"L": L, "us": round(t * 1e6, 2), "GB_s": round(nbytes / t / 1e9, 1),
                 "frac": round(nbytes / t / HBM_PEAK, 4), "rotated_copies": n})
            del kc, vc, aws, graph
            torch.cuda.empty_cache()
    log("ops: head " + ", ".join(f"{r['open_rows']} open {r['us']:.0f} us" for r in out["head"]) +
        "; attention " + ", ".join(f"L={r['L']} {r['us']:.1f} us {r['GB_s']:.0f} GB/s" for r in out["attention"]) +
        "; FP8 cache " + ", ".join(f"L={r['L']} {r['us']:.1f} us {r['GB_s']:.0f} GB/s" for r in out["attention_fp8_cache"]))
    return out


def run_moe(args, torch, dlm, synth, np):
    """The MoE configuration: bf16 attention and head, MXFP4 experts (codes drawn on the device
    from a seeded generator: expert values do not change the work), k commits per round."""
    s = synth.MOE16B
    t0 = time.time()
    w = synth.Weights(s, args.seed, cache=False)
    dev = {}
    for n in w.names_dense():
        a = w[n]
        dev[n] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(args.seed)
    ET, F, d = s.n_experts + s.n_shared, s.expert_ffn, s.d
    for i in range(s.n_layers):
        for name, shp in (("x_w13", (ET, 2 * F, d // 2)), ("x_w2", (ET, d, F // 2))):
            dev[f"l{i}.{name}"] = torch.randint(0, 256, shp, dtype=torch.uint8, device="cuda", generator=gen)
            sshp = shp[:-1] + (shp[-1] * 2 // 32,)
            dev[f"l{i}.{name}_scale"] = torch.randint(119, 122, sshp, dtype=torch.uint8, device="cuda", generator=gen)
    B = s.block
    cap = args.prompt + (args.moe_blocks + 4) * B
    model = dlm.Model(s, dev, cap=cap)
    for i in range(s.n_layers):          # decode reads only the packed copies
        for name in ("x_w13", "x_w13_scale", "x_w2", "x_w2_scale"):
            dev.pop(f"l{i}.{name}")
    torch.cuda.empty_cache()
    log(f"moe model built in {time.time() - t0:.1f}s")
    prompt = torch.from_numpy(synth.prompt_ids(s, args.prompt, args.seed))
    rule = dlm.CommitRule.fixed_k(args.k)
    pipelined = not args.separate_commit
    bufs = [torch.zeros(B, dtype=torch.int32, device="cuda") for _ in range(2)]
    model.set_len(0)
    model.prefill(prompt)
    prev = None
    if pipelined:
        # as in the dense leg: three warm-up blocks capture every graph the timed loop replays,
        # and the pending commit pass of the last one lands at [prompt - B, prompt)
        for i in range(3):
            model.decode_block_pipelined(rule, prev, bufs[i % 2])
            prev = bufs[i % 2]
        torch.cuda.synchronize()
        model.set_len(args.prompt - B)
    else:
        model.decode_block(rule)
        torch.cuda.synchronize()
        model.set_len(args.prompt)
    hits = model.view("moe_hits", (s.n_layers,), torch.int32)
    torch.cuda.synchronize()
    hits_before = int(hits.sum().item())     # prefill and warm-up forwards (the workspace starts zeroed)
    hits.zero_()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    host_tok = torch.empty(args.moe_blocks, B, dtype=torch.int32).pin_memory()
    ev0.record()
    for i in range(args.moe_blocks):
        if pipelined:
            cur = bufs[1] if prev is bufs[0] else bufs[0]
            model.decode_block_pipelined(rule, prev, cur)
            host_tok[i].copy_(cur, non_blocking=True)
            prev = cur
        else:
            model.decode_block(rule)
            host_tok[i].copy_(model.tokens, non_blocking=True)
    ev1.record()
    torch.cuda.synchronize()
    sec = ev0.elapsed_time(ev1) / 1e3
    R = math.ceil(B / args.k)
    total_hits = int(hits.sum().item())
    if pipelined:
        # round 0 of a block carries the previous block's commit rows with the same weights; its
        # expert count is that of the 64-row forward
        dense = sum(R * moe_dense_pass_bytes(s, args.prompt + B * i, True) for i in range(args.moe_blocks))
        forwards_per_block = R * s.n_layers
    else:
        dense = sum(R * moe_dense_pass_bytes(s, args.prompt + B * i, True) +
                    moe_dense_pass_bytes(s, args.prompt + B * i, False) for i in range(args.moe_blocks))
        forwards_per_block = R * s.n_layers + (s.n_layers - 1)
    total = dense + total_hits * moe_expert_bytes(s)
    out = {"workload": f"MoE 16B-A1B-shaped (20 layers, d 2048, 256 experts of 512 top-8 + 1 shared, MXFP4 "
                       f"experts, MXFP8 activations), bs=1, block 32, fixed k={args.k}, prompt {args.prompt}, "
                       f"{args.moe_blocks * B} new tokens",
           "commit_pass": "pipelined into the next block's round 0" if pipelined else "separate",
           "tok_s": args.moe_blocks * B / sec, "rounds_s": args.moe_blocks * R / sec,
           "ms_per_block": 1e3 * sec / args.moe_blocks, "hbm_frac": total / sec / HBM_PEAK,
           "mean_experts_hit_per_layer_forward": total_hits / (args.moe_blocks * forwards_per_block),
           "bytes_per_block": total / args.moe_blocks,
           # every forward of the leg (prefill, warm-up, timed): each distinct expert's weights
           # and scales once per forward -- the algorithmic bytes of all its expert launches
           "expert_bytes_all_forwards": (hits_before + total_hits) * moe_expert_bytes(s)}
    log(f"moe k={args.k}: {out['tok_s']:.0f} tok/s, {out['ms_per_block']:.2f} ms/block, "
        f"{100 * out['hbm_frac']:.1f}% of 8 TB/s, {out['mean_experts_hit_per_layer_forward']:.1f} experts/layer")
    model.close()
    del model, dev
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128,
                    help="timed blocks, spread evenly over the 128 blocks of the 4096-token generation")
    ap.add_argument("--new-tokens", type=int, default=4096, help="tokens of the generation the steps sample")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--k", type=int, default=6, help="commits per round of the headline number")
    ap.add_argument("--k-list", default="1,2,6,11", help="other k values also timed (empty to skip)")
    ap.add_argument("--prompt", type=int, default=256)
    ap.add_argument("--seed", type=int, default=1234, help="seed of the model and prompt of every leg")
    ap.add_argument("--no-ops", action="store_true", help="skip the head and attention op leg")
    ap.add_argument("--no-fp8-cache", action="store_true", help="skip the headline k with an FP8 KV cache")
    ap.add_argument("--seeds", default="1234,1235,1236",
                    help="seeds of the headline k: the first is --seed's run, each further seed draws a new "
                         "model and prompt; the reported value is the median (empty: --seed only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rounds", type=int, default=1)
    ap.add_argument("--moe-blocks", type=int, default=64,
                    help="blocks of the MoE model decoded at k = --k (0 skips the MoE leg)")
    ap.add_argument("--separate-commit", action="store_true",
                    help="decode every block with its own commit pass instead of pipelining it")
    ap.add_argument("--counter-legs", action="store_true",
                    help="only the legs the HBM byte-counter runs read: head and attention ops, the "
                         "gate/up launches, a 2-block MoE leg and the reference copy")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the dominant-kernel leg plus a 256 MiB device copy (for counter runs)")
    ap.add_argument("--attn-out", action="store_true",
                    help="per-op kernels with the attention-output projection inside the attention launch "
                         "(DLM_LAYERS_ATTN_OUT)")
    ap.add_argument("--fused-layers", action="store_true",
                    help="decode with the fused layer kernels (one launch per sublayer)")
    ap.add_argument("--no-full", action="store_true", help="skip the in-order 128-block generation leg")
    ap.add_argument("--no-tiny", action="store_true", help="skip the tiny fp32 model leg")
    ap.add_argument("--no-threshold", action="store_true",
                    help="skip the threshold-block leg (whose later rounds' kernels only read the continue flag)")
    args = ap.parse_args()
    layer_path = 2 if args.attn_out else None        # DLM_LAYERS_ATTN_OUT

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU sharding is a design "
                                   "note, not implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import block_diffusion_decoding_denoise_amd as dlm

    dlm.lib()
    shape = synth.QWEN4B
    B = shape.block
    NB = args.new_tokens // B                    # blocks of the generation
    n_new = args.steps * B                       # tokens decoded in the timed region
    # step i decodes block blocks[i] (evenly spread over the generation; all of them in order
    # when --steps equals the block count)
    blocks = [min(NB - 1, int((i + 0.5) * NB / args.steps)) if args.steps < NB else i % NB
              for i in range(args.steps)]
    cap = args.prompt + (NB + 2) * B
    t0 = time.time()
    w = synth.Weights(shape, args.seed)
    names = w.names_dense()
    dev_w = {}
    for n in names:
        a = w[n]
        dev_w[n] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    log(f"weights drawn and uploaded in {time.time() - t0:.1f}s")
    model = dlm.Model(shape, dev_w, cap=cap, fused_layers=args.fused_layers, layer_path=layer_path)
    prompt = torch.from_numpy(synth.prompt_ids(shape, args.prompt, args.seed))
    host_tok = torch.empty(max(args.steps, NB), B, dtype=torch.int32).pin_memory()
    # device-side prefix of each timed block: the pending commit pass of the block before it
    # (pipelined) lands at [L - B, L), so the pipelined decode of block b starts at L_b - B
    L_of = [args.prompt + B * b for b in blocks]
    len_seq = torch.tensor([L - B if not args.separate_commit else L for L in L_of], dtype=torch.int32,
                           device="cuda")

    pipelined = not args.separate_commit
    bufs = [torch.zeros(B, dtype=torch.int32, device="cuda") for _ in range(2)]

    def run(k, steps, warmup, in_order=False):
        """Time `steps` blocks at fixed k: the sampled blocks of the generation (each at its own
        prefix), or (in_order) the generation's first `steps` blocks one after the other."""
        rule = dlm.CommitRule.fixed_k(k)
        model.set_len(0)
        model.prefill(prompt)
        torch.cuda.synchronize()
        prev = None
        if pipelined:
            # at least three warmup blocks: every graph the timed loop replays (first block,
            # and both alternations of the two token buffers) is captured before timing
            for i in range(max(warmup, 3)):
                cur = bufs[i % 2]
                model.decode_block_pipelined(rule, prev, cur)
                prev = cur
            torch.cuda.synchronize()
            # the pending warmup block's commit pass lands at [prompt - B, prompt), so timed
            # block i decodes at prefix prompt + B i, as without pipelining
            model.set_len(args.prompt - B)
        else:
            for _ in range(warmup):
                model.decode_block(rule)
            torch.cuda.synchronize()
            model.set_len(args.prompt)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t_host = time.perf_counter()
        ev0.record()
        for i in range(steps):
            if not in_order:
                model.len_dev.copy_(len_seq[i:i + 1])          # this block's prefix (device copy)
            if pipelined:
                cur = bufs[1] if prev is bufs[0] else bufs[0]
                model.decode_block_pipelined(rule, prev, cur)
                host_tok[i].copy_(cur, non_blocking=True)
                prev = cur
            else:
                model.decode_block(rule)
                host_tok[i].copy_(model.tokens, non_blocking=True)
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_host
        ms = ev0.elapsed_time(ev1)
        st = dlm.state_dict(model.state)
        R = math.ceil(B / k)
        assert st["round"] == R, st
        return ms / 1000.0, wall, R

    results = {}
    ks = [args.k] + [int(x) for x in args.k_list.split(",") if x and int(x) != args.k]
    if args.roofline_only or args.counter_legs:
        ks = []
    def block_bytes(L, R, kv_elem_bytes=2):
        if pipelined:
            # R weight streams per block: round 0 moves the previous block's commit rows with
            # the same weights (its keys reach prefix + 2 B, as the rounds' do)
            return algorithmic_bytes(shape, L, kv_elem_bytes=kv_elem_bytes) * R
        return algorithmic_bytes(shape, L) * R + commit_pass_bytes(shape, L)

    for k in ks:
        sec, wall, R = run(k, args.steps, args.warmup)
        L_mean = sum(L_of) / len(L_of)
        rb = sum(block_bytes(L, R) for L in L_of)
        results[k] = {"tok_s": n_new / sec, "rounds_s": args.steps * R / sec, "ms_per_block": 1e3 * sec / args.steps,
                      "hbm_frac": rb / sec / HBM_PEAK, "rounds_per_block": R, "tpf": B / R, "wall_s": wall,
                      "bytes_per_block": rb / args.steps, "mean_prefix": L_mean}
        log(f"k={k}: {results[k]['tok_s']:.0f} tok/s, {results[k]['rounds_s']:.0f} rounds/s, "
            f"{results[k]['ms_per_block']:.2f} ms/block, {100 * results[k]['hbm_frac']:.1f}% of 8 TB/s")

    # ---- the headline k over the whole generation in order (128 blocks, each at its prefix)
    full = None
    if ks and not args.no_full:
        sec, wall, R = run(args.k, NB, args.warmup, in_order=True)
        rb = sum(block_bytes(args.prompt + B * b, R) for b in range(NB))
        full = {"k": args.k, "blocks": NB, "new_tokens": NB * B, "tok_s": round(NB * B / sec, 1),
                "rounds_s": round(NB * R / sec, 1), "ms_per_block": round(1e3 * sec / NB, 3),
                "hbm_frac": round(rb / sec / HBM_PEAK, 4), "mean_prefix": args.prompt + B * (NB - 1) / 2,
                "wall_s": round(wall, 3)}
        log(f"k={args.k} full {NB}-block generation: {full['tok_s']:.0f} tok/s, {full['ms_per_block']:.2f} ms/block")

    # ---- the headline k with an FP8 e4m3 KV cache (same weights, prompt and rule)
    fp8_cache = None
    if ks and pipelined and not args.no_fp8_cache:
        bf16_model = model
        model = dlm.Model(shape, dev_w, cap=cap, kv_scales=FP8_CACHE_SCALES, fused_layers=args.fused_layers,
                          layer_path=layer_path)
        sec, wall, R = run(args.k, args.steps, args.warmup)
        rb = sum(block_bytes(L, R, kv_elem_bytes=1) for L in L_of)
        fp8_cache = {"k": args.k, "kv_scales": list(FP8_CACHE_SCALES), "tok_s": round(n_new / sec, 1),
                     "ms_per_block": round(1e3 * sec / args.steps, 3), "hbm_frac": round(rb / sec / HBM_PEAK, 4),
                     "bytes_per_block": rb / args.steps}
        log(f"k={args.k} with an FP8 KV cache: {fp8_cache['tok_s']:.0f} tok/s, {fp8_cache['ms_per_block']:.2f} ms/block")
        model.close()
        del model
        model = bf16_model
        torch.cuda.empty_cache()

    # ---- prefill of the prompt: the wide forwards of dlm_prefill (up to 256 rows each) against
    # 64- and 32-row forwards (dlm_prefill_rows), warm calls, median of 3, HIP events
    def time_prefill(max_rows):
        ts = []
        for _ in range(4):
            model.set_len(0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            model.prefill(prompt, max_rows=max_rows)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts[1:])[1]
    D = shape.head_dim
    per_layer = (shape.hq + 2 * shape.hkv) * D * shape.d + shape.d * shape.hq * D + 3 * shape.ffn * shape.d
    qkv_last = (shape.hq + 2 * shape.hkv) * D * shape.d
    prefill_gemm_flop = 2 * args.prompt * ((shape.n_layers - 1) * per_layer + qkv_last)
    counters_only = args.roofline_only or args.counter_legs
    pf = {r: time_prefill(r) if not counters_only else float("nan") for r in (256, 64, 32)}
    prefill = {"tokens": args.prompt, "ms": round(pf[256], 3), "tok_s": round(args.prompt / (pf[256] / 1e3), 1),
               "gemm_tflop_s": round(prefill_gemm_flop / (pf[256] / 1e3) / 1e12, 1),
               "ms_64_rows": round(pf[64], 3), "ms_32_rows": round(pf[32], 3),
               "how": "dlm_prefill (forwards of up to 256 rows), warm, median of 3; also 64- and 32-row "
                      "forwards (dlm_prefill_rows); gemm_tflop_s counts the projections' 2 x params x tokens"}
    if not counters_only:
        log(f"prefill {args.prompt} tokens: {pf[256]:.2f} ms wide ({prefill['gemm_tflop_s']} TFLOP/s in the "
            f"projections), {pf[64]:.2f} ms in 64-row forwards, {pf[32]:.2f} ms in 32-row forwards")

    # ---- dominant kernel: the FFN gate/up projection + SwiGLU, the round's largest weight
    # stream, launched alone exactly as inside the round (dlm_ffn_gate_up: same kernel, plan
    # and packed weights), cycling through the 36 layers so no launch finds its weights in a
    # cache, timed with HIP events on the stream the launches go to.
    s = shape
    x = dlm.pack_activations((torch.randn(32, s.d, device="cuda") * 0.1).to(torch.bfloat16))
    act = torch.empty(32, s.ffn, dtype=torch.bfloat16, device="cuda")
    gws = torch.zeros(max(dlm.lib().dlm_ffn_gate_up_ws_bytes(model.handle), 256), dtype=torch.uint8, device="cuda")
    for l in range(s.n_layers):
        model.ffn_gate_up(l, x, act=act, ws=gws)
    torch.cuda.synchronize()
    # the 36 launches are replayed as one graph, as the round's kernels are
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l in range(s.n_layers):
            model.ffn_gate_up(l, x, act=act, ws=gws)
    graph.replay()
    torch.cuda.synchronize()
    n_cycles = 5
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(n_cycles):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    n_launch = n_cycles * s.n_layers
    t_launch = ev0.elapsed_time(ev1) / 1e3 / n_launch
    gemm_bytes = 2 * (2 * s.ffn * s.d) + 2 * 32 * s.d + 2 * 32 * s.ffn
    roofline = {"bound": "hbm", "achieved": gemm_bytes / t_launch / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": gemm_bytes / t_launch / HBM_PEAK, "traffic": counter_traffic(),
                "kernel": "gemm_owned_kernel<3, 8, 1> (FFN gate/up + SwiGLU, N=19456, K=2560, M=32)",
                "bytes_per_launch": gemm_bytes, "us_per_launch": t_launch * 1e6, "launches": n_launch}
    log(f"gate/up + SwiGLU: {t_launch * 1e6:.1f} us/launch, {roofline['achieved']:.0f} GB/s")

    if args.roofline_only or args.counter_legs:
        extra = {}
        if args.counter_legs:
            extra["ops"] = run_ops(torch, dlm, dev_w["emb"], args.seed)
        # a plain device copy of known size, the reference for scaling the HBM byte counters
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        model.close()
        if args.counter_legs:
            del model
            dev_w.clear()
            torch.cuda.empty_cache()
            args.moe_blocks = 2
            extra["moe"] = run_moe(args, torch, dlm, synth, np)
        print(json.dumps({"roofline": roofline, "copy_bytes_per_launch": 256 << 20, "copy_launches": 4, **extra}),
              flush=True)
        return

    # ---- threshold blocks: the rounds after a block is done.  tau = 0 commits every row in round
    # 0, so a 32-round budget leaves 31 rounds whose kernels only read the continue flag:
    # dlm_decode_block (one graph of all 32) against dlm_decode_block_gated (round segments,
    # the host checking the flag between them), and one fixed-k round as the floor
    def time_threshold(fn, n=6):
        for _ in range(2):
            model.set_len(args.prompt)
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            model.set_len(args.prompt)
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n
    threshold = None
    if not args.no_threshold:
        thr_rule = dlm.CommitRule.threshold(0.0, True, 32)
        one_round = dlm.CommitRule.fixed_k(32)
        threshold = {
            "workload": "threshold rule tau=0 with forced top-1 and max_rounds=32 (the block is done in round 0), "
                        "prompt 256, one block, separate commit pass",
            "ms_block_graph": round(time_threshold(lambda: model.decode_block(thr_rule)), 3),
            "ms_gated_seg1": round(time_threshold(lambda: model.decode_block_gated(thr_rule, seg_rounds=1)), 3),
            "ms_gated_seg4": round(time_threshold(lambda: model.decode_block_gated(thr_rule, seg_rounds=4)), 3),
            "ms_one_round_floor": round(time_threshold(lambda: model.decode_block(one_round)), 3)}
        log(f"threshold block done in round 0 of 32: {threshold['ms_block_graph']:.2f} ms (all rounds enqueued), "
            f"{threshold['ms_gated_seg1']:.2f} ms gated (segments of 1), one round alone "
            f"{threshold['ms_one_round_floor']:.2f} ms")

    # ---- the head and attention ops alone (uses the model's embedding)
    ops = run_ops(torch, dlm, dev_w["emb"], args.seed) if not args.no_ops else None

    # ---- measured streaming rate of this GPU: a 1 GiB device-to-device copy (read + write bytes)
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(5):
        b.copy_(a)
    ev1.record()
    torch.cuda.synchronize()
    stream = {"kind": "device-to-device copy of 1 GiB, read + write bytes", "unit": "GB/s",
              "value": 5 * 2 * a.numel() / (ev0.elapsed_time(ev1) / 1e3) / 1e9}
    del a, b
    log(f"measured stream: {stream['value']:.0f} GB/s")

    # ---- the headline k on the further seeds: a new model and prompt each; value = median
    seeds = [int(x) for x in args.seeds.split(",") if x] if args.seeds else []
    per_seed = {str(args.seed): results[args.k]["tok_s"]}
    for sd in seeds:
        if str(sd) in per_seed:
            continue
        model.close()
        del model
        dev_w.clear()
        torch.cuda.empty_cache()
        ws = synth.Weights(shape, sd)
        for n in names:
            dev_w[n] = torch.from_numpy(ws[n].view(np.int16)).view(torch.bfloat16).to("cuda")
        del ws
        model = dlm.Model(shape, dev_w, cap=cap, fused_layers=args.fused_layers, layer_path=layer_path)
        prompt = torch.from_numpy(synth.prompt_ids(shape, args.prompt, sd))
        sec, _, _ = run(args.k, args.steps, args.warmup)
        per_seed[str(sd)] = n_new / sec
        log(f"seed {sd}: k={args.k}: {per_seed[str(sd)]:.0f} tok/s")
    value = float(np.median(list(per_seed.values())))

    moe = None
    if args.moe_blocks > 0:
        model.close()
        del model
        dev_w.clear()
        torch.cuda.empty_cache()
        moe = run_moe(args, torch, dlm, synth, np)
        model = None

    # ---- CPU baseline: the oracle in float32 on a bounded sample (one round + one commit pass)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from oracle import OracleModel, KVCache, Prec, CommitRule as OCR
        try:
            from threadpoolctl import threadpool_info
            cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
        except Exception:
            cores = os.cpu_count()
        prec = Prec("bf16", np.float32)
        om = OracleModel(shape, w, prec, cache_layers=False)
        kv = KVCache.empty(shape, args.prompt + 2 * B, np.float32)
        kv.length = args.prompt
        toks = np.zeros(B, np.int32)
        committed = np.zeros(B, np.uint8)
        t0 = time.perf_counter()
        res = oracle.denoise_round(om, kv, toks, committed, None, 0, OCR(1, 0.9, args.k, False, 32), prec)
        t_round = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.commit_pass(om, kv, toks, prec)
        t_cp = time.perf_counter() - t0
        R = math.ceil(B / args.k)
        cpu_tok_s = B / (R * t_round + t_cp)
        cpu = {"value": cpu_tok_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "sample": f"one denoising round and one commit pass of the same model at prefix {args.prompt} "
                         f"(numpy float32 mode), extrapolated to a {R}-round block: "
                         f"{t_round:.1f} s/round, {t_cp:.1f} s/commit pass"}
        log(f"cpu oracle: {cpu_tok_s:.3f} tok/s ({t_round:.1f} s/round)")
        del res
        # the host, and the oracle's head and attention ops alone (float32 mode, same threads):
        # the head at 32 open rows over the model's own embedding, the attention at the op leg's
        # shapes (32 / 8 heads of 128, a 32-query block) on N(0, 1) inputs
        model_name = ""
        try:
            for line_ in open("/proc/cpuinfo"):
                if line_.startswith("model name"):
                    model_name = line_.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        cpu["host"] = {"cpu_model": model_name, "cpu_count": os.cpu_count()}
        rng = np.random.default_rng(args.seed)
        hq_ = rng.standard_normal((32, shape.d)).astype(np.float32)
        hq_ /= np.sqrt((hq_ * hq_).mean(axis=1, keepdims=True))
        hb_ = oracle.bf16_round(hq_).astype(np.float32)
        t0 = time.perf_counter()
        oracle.head_rowstats(hb_, w["emb"], np.zeros(32, np.uint8), prec)
        t_head = time.perf_counter() - t0
        t_attn = {}
        for L_ in (512, 4096, 32768):
            q_ = rng.standard_normal((B, 32, 128)).astype(np.float32)
            k_ = rng.standard_normal((8, L_ + B, 128)).astype(np.float32)
            v_ = rng.standard_normal((8, L_ + B, 128)).astype(np.float32)
            t0 = time.perf_counter()
            oracle.attention(q_, k_, v_, 1.0 / math.sqrt(128))
            t_attn[L_] = time.perf_counter() - t0
        cpu["ops"] = {"head_32_open_rows_s": round(t_head, 3),
                      "attention_s": {str(L_): round(t, 4) for L_, t in t_attn.items()}}
        log(f"cpu oracle ops: head (32 open rows) {t_head:.2f} s; attention " +
            ", ".join(f"L={L_} {t:.3f} s" for L_, t in t_attn.items()))

    # ---- the tiny fp32 model: prompt 64, 4 blocks, threshold 0.9 with forced top-1, 32 rounds at
    # most (random weights: every round commits its top-1 only, so 32 rounds per block)
    tiny = None
    if not args.no_tiny:
        ts = synth.TINY
        tw = synth.Weights(ts, args.seed)
        tdev = {n: torch.from_numpy(np.ascontiguousarray(tw[n])).cuda() for n in tw.names_dense()}
        tm = dlm.Model(ts, tdev, cap=64 + 5 * 32)
        tprompt = torch.from_numpy(synth.prompt_ids(ts, 64, args.seed))
        trule = dlm.CommitRule.threshold(0.9, True, 32)
        tm.generate(tprompt, 4, trule)                 # captures the graph
        torch.cuda.synchronize()
        tm.set_len(0)
        tm.prefill(tprompt)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(4):
            tm.decode_block(trule)
        e1.record()
        torch.cuda.synchronize()
        tsec = e0.elapsed_time(e1) / 1e3
        rounds = 4 * 32
        tiny = {"workload": "tiny fp32 (2 layers, d 256, vocab 4096), prompt 64, 4 blocks of 32, threshold 0.9 "
                            "with forced top-1, max 32 rounds", "rounds_s": round(rounds / tsec, 1),
                "tok_s": round(4 * 32 / tsec, 1), "ms_per_block": round(1e3 * tsec / 4, 3),
                "rounds_per_block": dlm.state_dict(tm.state)["round"]}
        tm.close()
        log(f"tiny fp32: {tiny['rounds_s']:.0f} rounds/s, {tiny['ms_per_block']:.2f} ms/block")

    # ---- the CPU oracle on one core: one round of a 1-layer and of a 2-layer cut of the same
    # model at prefix 256 (numpy float32), extrapolated to the 36-layer round
    cpu1 = None
    if not args.no_cpu_baseline:
        try:
            from threadpoolctl import threadpool_limits
            import oracle
            from oracle import OracleModel, KVCache, Prec, CommitRule as OCR
            prec = Prec("bf16", np.float32)
            t = {}
            with threadpool_limits(limits=1):
                for nl in (1, 2):
                    sh = synth.small_shape(shape, n_layers=nl)
                    om = OracleModel(sh, w, prec, cache_layers=False)
                    kv = KVCache.empty(sh, args.prompt + 2 * B, np.float32)
                    kv.length = args.prompt
                    t0 = time.perf_counter()
                    oracle.denoise_round(om, kv, np.zeros(B, np.int32), np.zeros(B, np.uint8), None, 0,
                                         OCR(1, 0.9, args.k, False, 32), prec)
                    t[nl] = time.perf_counter() - t0
            per_layer = t[2] - t[1]
            t_round = t[1] + (shape.n_layers - 1) * per_layer
            R = math.ceil(B / args.k)
            cpu1 = {"value": round(B / (R * t_round * (1 + 0.9 / R)), 4), "unit": "tokens/s", "cores": 1,
                    "kind": "oracle",
                    "sample": f"one round of a 1-layer and of a 2-layer cut of the model at prefix {args.prompt} on "
                              f"one core ({t[1]:.2f} s and {t[2]:.2f} s), extrapolated to 36 layers "
                              f"({t_round:.1f} s/round) and to a {R}-round block plus a commit pass of 0.9 round"}
            log(f"cpu oracle, 1 core: {cpu1['value']:.4f} tok/s ({t_round:.1f} s/round)")
        except Exception as ex:        # noqa: BLE001 -- the baseline leg must not sink the line
            log(f"cpu oracle 1-core leg skipped: {ex}")

    h = results[args.k]
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": h["ms_per_block"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"qwen3-4b-shaped random-init block decode, bs=1, block 32, fixed k={args.k}, "
                               f"prompt {args.prompt}, {NB * B} new tokens (blocks at prefixes {args.prompt}.."
                               f"{args.prompt + B * NB}, mean {args.prompt + B * (NB - 1) / 2:.0f}); "
                               f"{args.steps} timed blocks spread evenly over them (mean prefix "
                               f"{h['mean_prefix']:.0f})",
                   "k": args.k, "block": B, "prompt": args.prompt, "new_tokens": NB * B, "timed_blocks": args.steps,
                   "mean_prefix": h["mean_prefix"], "layers": s.n_layers,
                   "layer_kernels": "fused (one launch per sublayer)" if args.fused_layers else
                   "per op, attention output projection inside the attention launch" if args.attn_out else
                   "per op",
                   "commit_pass": "pipelined into the next block's round 0" if pipelined else "separate",
                   "d": s.d, "ffn": s.ffn, "vocab": s.vocab},
        "rounds_per_s": h["rounds_s"], "hbm_frac_step": h["hbm_frac"], "tpf": h["tpf"],
        "value_per_seed": {k: round(v, 2) for k, v in per_seed.items()},
        "prefill": prefill,
        "hbm_stream_measured": stream, "ops": ops, "fp8_cache": fp8_cache,
        "per_k": {str(k): {kk: round(v, 4) if isinstance(v, float) else v for kk, v in r.items()}
                  for k, r in results.items()},
        "roofline": roofline, "cpu_baseline": cpu, "cpu_baseline_1core": cpu1, "moe": moe,
        "full_generation": full, "tiny_fp32": tiny, "threshold_dead_rounds": threshold,
    }
    print(json.dumps(line), flush=True)
    if model is not None:
        model.close()


if __name__ == "__main__":
    main()
