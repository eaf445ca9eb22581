#!/usr/bin/env python3
"""Benchmark of the DSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload: prefill of one causal sequence of L = 131072 tokens with
the full-size shapes (indexer 64 heads x 128 FP8, top-k 2048, 128 bf16 query
heads over a 576-d latent).  One step is the whole hot path on that input:
per-token E4M3 quantisation of the indexer q/k, the fused indexer + top-k
(no L x L score matrix) and sparse MLA over the selected rows.  ``value`` is
prefill tokens/s = L * K / wall time of K steps (inputs resident in HBM).

Also reported (one JSON line): per-kernel HIP-event times and their roofline
fractions, decode tokens/s for B = 64 sequences at context 32768 and for the
ragged paged batch (B = 128, context 4096..131072, shuffled 64-token pages),
short prefill (L = 4096) through the masked-MHA mode next to the same
selection through sparse MLA, the indexer's KL-alignment loss forward on the
headline selection (the step beside the path in sparse training), the
L = 16384 prefill and the backward of its sparse-training step, the measured
MFMA/HBM peaks, and the fp64 CPU oracle timed on a bounded sample of the
headline workload.

Inputs are synthetic (synth), drawn on the GPU with the same counter-based
generator the oracle side uses.
"""
from __future__ import annotations

import argparse
import json
import math
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
METRIC = "DSA prefill tokens/s at L=128K + decode tokens/s; % FP8 MFMA / HBM peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--decode-steps", type=int, default=100, help="decode steps timed (median reported)")
    ap.add_argument("--decode-warmup", type=int, default=5)
    ap.add_argument("--no-prefill16k", action="store_true", help="skip the L=16384 prefill entry")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak microbenchmarks")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward section")
    ap.add_argument("--backward-steps", type=int, default=3)
    ap.add_argument("--cpu-rows-1t", type=int, default=16, help="query rows in the single-thread oracle sample")
    ap.add_argument("--no-decode", action="store_true", help="prefill only")
    ap.add_argument("--no-paged", action="store_true", help="skip the ragged paged decode batch")
    ap.add_argument("--no-short", action="store_true", help="skip the short-prefill (masked MHA) section")
    ap.add_argument("--no-kl", action="store_true", help="skip the indexer KL-loss section")
    ap.add_argument("--kl-steps", type=int, default=3)
    ap.add_argument("--short-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=256, help="query rows in the oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run plain 1 GiB device copies (to scale HBM counters)")
    ap.add_argument("--L", type=int, default=None, help="override the prefill length (testing only)")
    return ap.parse_args()


class Stages:
    """HIP events between the launches of one step, on the launching stream."""

    def __init__(self, torch, names):
        self.torch = torch
        self.names = names
        self.acc = {n: 0.0 for n in names}
        self.count = 0

    def new(self):
        return [self.torch.cuda.Event(enable_timing=True) for _ in range(len(self.names) + 1)]

    def add(self, evs):
        for i, n in enumerate(self.names):
            self.acc[n] += evs[i].elapsed_time(evs[i + 1])
        self.count += 1

    def avg_ms(self):
        return {n: self.acc[n] / max(self.count, 1) for n in self.names}


class StageSamples(Stages):
    """Per-step stage times kept whole, for medians."""

    def __init__(self, torch, names):
        super().__init__(torch, names)
        self.samples = {n: [] for n in names}

    def add(self, evs):
        super().add(evs)
        for i, n in enumerate(self.names):
            self.samples[n].append(evs[i].elapsed_time(evs[i + 1]))
        tot = evs[0].elapsed_time(evs[-1])
        self.samples.setdefault("_step", []).append(tot)

    def median_ms(self):
        import statistics
        return {n: statistics.median(v) for n, v in self.samples.items() if v}


# --------------------------------------------------------------------------- prefill
def setup_prefill(torch, dsa, synth, cfg, dev):
    L = cfg.L
    t = {}
    t["qi"], t["ki"], t["w"] = synth.prefill_indexer_inputs(cfg, device=dev)
    t["q"] = synth.prefill_attn_q(cfg, device=dev)
    t["kv"] = synth.prefill_latent(cfg, device=dev)
    t["q8"] = torch.empty((L, cfg.H_I, cfg.D_I), dtype=torch.uint8, device=dev)
    t["qs"] = torch.empty(L, dtype=torch.float32, device=dev)
    t["k8"] = torch.empty((L, cfg.D_I), dtype=torch.uint8, device=dev)
    t["ks"] = torch.empty(L, dtype=torch.float32, device=dev)
    t["idx"] = torch.empty((L, cfg.k), dtype=torch.int32, device=dev)
    t["out"] = torch.empty((L, cfg.H, 512), dtype=torch.bfloat16, device=dev)
    t["lse"] = torch.empty((L, cfg.H), dtype=torch.float32, device=dev)
    t["args"] = dsa.make_prefill_args(L, cfg.H_I, cfg.D_I, cfg.H, cfg.k, dsa.DSA_E4M3, t["q8"], t["qs"], t["k8"],
                                      t["ks"], t["w"], dsa.DSA_BF16, t["q"], t["kv"], cfg.sm_scale, t["idx"],
                                      t["out"], t["lse"])
    t["ws"] = torch.empty(max(1, dsa.dsa_prefill_workspace_bytes(t["args"])), dtype=torch.uint8, device=dev)
    return t


def prefill_step(dsa, cfg, t, evs, stream):
    L = cfg.L
    evs[0].record(stream)
    dsa.dsa_quantize_e4m3_per_token(t["qi"], t["q8"], t["qs"], rows=L, cols=cfg.H_I * cfg.D_I, stream=stream)
    dsa.dsa_quantize_e4m3_per_token(t["ki"], t["k8"], t["ks"], rows=L, cols=cfg.D_I, stream=stream)
    evs[1].record(stream)
    dsa.dsa_prefill_select(t["args"], workspace=t["ws"], stream=stream)
    evs[2].record(stream)
    dsa.dsa_sparse_mla_fwd(t["q"], t["kv"], t["idx"], cfg.sm_scale, t["out"], t["lse"], stream=stream)
    evs[3].record(stream)


def prefill_work(cfg):
    L, k = cfg.L, cfg.k
    pairs = L * (L + 1) // 2
    selected = sum(min(k, t + 1) for t in range(min(L, k))) + max(0, L - k) * k
    return {
        "quantize_bytes": L * cfg.H_I * cfg.D_I * 5 + L * cfg.D_I * 5 + 2 * L * 4,
        "indexer_flop": 2 * cfg.H_I * cfg.D_I * pairs,
        "causal_pairs": pairs,
        "mla_flop": 2 * cfg.H * (576 + 512) * selected,
        "selected_pairs": selected,
    }


# --------------------------------------------------------------------------- decode
def setup_decode(torch, dsa, synth, cfg, dev):
    ctx = synth.decode_ctx(cfg)
    bt, nb = synth.decode_block_table(cfg, ctx)
    t = {"ctx_cpu": ctx, "nb": nb}
    t["k8p"], t["ksp"], t["kvp"] = synth.build_decode_pools(cfg, ctx, bt, nb, device=dev)
    t["q8"], t["qs"], t["w"], t["q"] = [x.to(dev) for x in synth.decode_queries(cfg, device=dev)]
    t["ctx"] = ctx.to(torch.int32).to(dev)
    t["bt"] = bt.to(dev)
    max_ctx = int(ctx.max())
    t["max_ctx"] = max_ctx
    t["ld"] = (max_ctx + 63) // 64 * 64
    t["scores"] = torch.empty((cfg.B, t["ld"]), dtype=torch.float32, device=dev)
    t["idx"] = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device=dev)
    t["out"] = torch.empty((cfg.B, cfg.H, 512), dtype=torch.bfloat16, device=dev)
    t["lse"] = torch.empty((cfg.B, cfg.H), dtype=torch.float32, device=dev)
    nws = dsa.dsa_sparse_mla_workspace_bytes(cfg.B, cfg.H, cfg.k)
    t["ws"] = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    # rows are at most ld long: a short batch may split its top-k rows over more CUs
    ntw = dsa.dsa_topk_workspace_bytes(cfg.B, t["ld"], cfg.k)
    t["topk_ws"] = torch.empty(ntw, dtype=torch.uint8, device=dev) if ntw > 0 else None
    t["args"] = dsa.make_decode_args(cfg.B, cfg.H_I, cfg.D_I, cfg.H, cfg.k, t["q8"], t["qs"], t["w"], t["q"],
                                     t["k8p"], t["ksp"], t["kvp"], nb * 64, t["bt"], bt.shape[1], t["ctx"],
                                     max_ctx, cfg.sm_scale, t["out"], t["lse"], t["idx"])
    # the token appended each step: the cached token at position ctx-1 (same bytes)
    pos = (ctx - 1).to(torch.int32)
    rows = torch.stack([bt[b, int(pos[b]) // 64].long() * 64 + int(pos[b]) % 64 for b in range(cfg.B)])
    rows = rows.to(dev)
    t["app_pos"] = pos.to(dev)
    t["app_lat"] = t["kvp"].view(-1, 576)[rows].clone()
    t["app_k8"] = t["k8p"].view(-1, cfg.D_I)[rows].clone()
    t["app_ks"] = t["ksp"].view(-1)[rows].clone()
    return t


def decode_step(dsa, cfg, t, evs, stream):
    evs[0].record(stream)
    dsa.dsa_paged_cache_append(t["app_lat"], t["app_k8"], t["app_ks"], t["app_pos"], t["bt"], t["kvp"], t["k8p"],
                               t["ksp"], n_pool_rows=t["nb"] * 64, stream=stream)
    evs[1].record(stream)
    dsa.dsa_decode_indexer_scores(t["args"], t["scores"], stream=stream)
    evs[2].record(stream)
    dsa.dsa_topk_select(t["scores"], t["ctx"], cfg.k, t["idx"], workspace=t["topk_ws"], stream=stream)
    evs[3].record(stream)
    dsa.dsa_sparse_mla_paged_fwd(t["q"], t["kvp"], t["bt"], t["idx"], cfg.sm_scale, t["out"], t["lse"],
                                 workspace=t["ws"], n_pool_rows=t["nb"] * 64, stream=stream)
    evs[4].record(stream)


def decode_work(cfg, ctx):
    ctx = [int(c) for c in ctx]
    sel = sum(min(cfg.k, c) for c in ctx)
    B = cfg.B
    return {
        "append_bytes": B * (576 * 2 + cfg.D_I + 4) * 2,
        "indexer_bytes": sum(ctx) * (cfg.D_I + 4) + B * (cfg.H_I * cfg.D_I + cfg.H_I * 4 + 4) + sum(ctx) * 4,
        "topk_bytes": sum(ctx) * 4 + B * cfg.k * 4,
        "mla_bytes": sel * 1152 + B * (cfg.H * 576 * 2 + cfg.H * 512 * 2 + cfg.k * 4 + cfg.H * 4),
        "mla_flop": 2 * cfg.H * (576 + 512) * sel,
        "context_tokens": sum(ctx),
        "selected_pairs": sel,
    }


def run_decode(torch, dsa, synth, cfg, dev, steps, warmup, flush):
    t = setup_decode(torch, dsa, synth, cfg, dev)
    stream = torch.cuda.current_stream()
    names = ["cache_append", "decode_indexer", "topk", "sparse_mla"]
    st = StageSamples(torch, names)
    for i in range(warmup + steps):
        # evict the 256 MB MALL and the L2s by reading 512 MB (a read leaves no dirty
        # lines behind to be written back during the step): each step reads its inputs from HBM
        flush.view(torch.int64).sum()
        evs = st.new()
        decode_step(dsa, cfg, t, evs, stream)
        torch.cuda.synchronize()
        if i >= warmup:
            st.add(evs)
    med = st.median_ms()
    ms = {n: med[n] for n in names}
    # the step as a caller runs it: the append, then the fused entry (indexer, top-k and attention in one call)
    ws = torch.empty(max(dsa.dsa_decode_workspace_bytes(t["args"]), 256), dtype=torch.uint8, device=dev)
    fused = []
    for i in range(warmup + steps):
        flush.view(torch.int64).sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dsa.dsa_paged_cache_append(t["app_lat"], t["app_k8"], t["app_ks"], t["app_pos"], t["bt"], t["kvp"], t["k8p"],
                                   t["ksp"], n_pool_rows=t["nb"] * 64, stream=stream)
        dsa.dsa_decode(t["args"], ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= warmup:
            fused.append(e0.elapsed_time(e1))
    del ws
    work = decode_work(cfg, t["ctx_cpu"])
    step_ms = statistics.median(fused)
    res = {
        "workload": cfg.name, "B": cfg.B, "ctx_min": int(t["ctx_cpu"].min()), "ctx_max": int(t["ctx_cpu"].max()),
        "ctx_mean": float(t["ctx_cpu"].float().mean()), "k": cfg.k, "H": cfg.H,
        "paged_shuffled": cfg.shuffled, "steps": steps, "warmup": warmup,
        "timing": f"median over {steps} steps after {warmup} warm-up steps, each step after a 512 MB cache-evicting read",
        "ms_per_step": step_ms,
        "step": "dsa_paged_cache_append + dsa_decode (the fused entry); stages_ms time the per-stage entries in a "
                "separate loop of the same length",
        "ms_per_step_staged": med["_step"],
        "tokens_per_s": cfg.B / (step_ms / 1e3),
        "unit": "tokens/s",
        "cold_cache": True,
        "stages_ms": ms,
        "roofline": {
            "decode_indexer": _rl("hbm", work["indexer_bytes"] / (ms["decode_indexer"] / 1e3) / 1e9, PEAK_HBM_GBS,
                                  "GB/s"),
            "topk": _rl("hbm", work["topk_bytes"] / (ms["topk"] / 1e3) / 1e9, PEAK_HBM_GBS, "GB/s"),
            "sparse_mla": _rl("hbm", work["mla_bytes"] / (ms["sparse_mla"] / 1e3) / 1e9, PEAK_HBM_GBS, "GB/s"),
            "sparse_mla_mfma": _rl("mfma", work["mla_flop"] / (ms["sparse_mla"] / 1e3) / 1e12, PEAK_BF16_TFLOPS,
                                   "TFLOP/s"),
        },
        "work": work,
    }
    del t
    torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------------------- KL loss
def run_kl(torch, dsa, cfg, t, dev, steps):
    """The indexer KL-alignment loss forward on the headline step's own outputs:
    index scores at the selected positions, then the per-token loss against
    the head-averaged attention (each head against the sparse-MLA lse)."""
    L, k = cfg.L, cfg.k
    sc = torch.empty((L, k), dtype=torch.float32, device=dev)
    kl = torch.empty(L, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    st = Stages(torch, ["scores_at", "kl"])
    for i in range(steps + 1):
        evs = st.new()
        evs[0].record(stream)
        dsa.dsa_indexer_scores_at(t["q8"], t["qs"], t["k8"], t["ks"], t["w"], t["idx"], sc, stream=stream)
        evs[1].record(stream)
        dsa.dsa_indexer_kl_fwd(t["q"], t["kv"], t["idx"], sc, t["lse"], cfg.sm_scale, kl, stream=stream)
        evs[2].record(stream)
        torch.cuda.synchronize()
        if i > 0:
            st.add(evs)
    ms = st.avg_ms()
    selected = prefill_work(cfg)["selected_pairs"]
    sa_flop = 2 * cfg.H_I * cfg.D_I * selected
    kl_flop = 2 * cfg.H * 576 * selected
    res = {
        "workload": cfg.name, "L": L, "H": cfg.H, "k": k, "steps": steps,
        "stages_ms": {n: round(v, 3) for n, v in ms.items()},
        "tokens_per_s": round(L / ((ms["scores_at"] + ms["kl"]) / 1e3), 1),
        "mean_kl": float(kl.double().mean()),
        "roofline": {
            "scores_at": _rl("mfma", sa_flop / (ms["scores_at"] / 1e3) / 1e12, PEAK_FP8_TFLOPS, "TFLOP/s"),
            "kl": _rl("mfma", kl_flop / (ms["kl"] / 1e3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"),
        },
        "work": {"scores_at_flop": sa_flop, "kl_flop": kl_flop, "selected_pairs": selected},
    }
    del sc, kl
    return res


# --------------------------------------------------------------------------- backward
def run_backward(torch, dsa, cfg, t, dev, steps):
    """One sparse-training step's backward on a prefill's own outputs (its
    selection, attention output and lse): the index scores at the selection,
    then the sparse-MLA backward with a synthetic upstream gradient, which
    also returns the score gradient of the mean per-token KL from the same
    attention probabilities (one pass over the logits for both losses), then
    the indexer's dw, dq, dk."""
    import synth
    L, H, k = cfg.L, cfg.H, cfg.k
    dout = synth.normal(cfg.seed, 91, (L, H, 512), device=dev, std=0.01).to(torch.bfloat16)
    dq = torch.empty((L, H, 576), dtype=torch.float32, device=dev)
    dkv = torch.empty((L, 576), dtype=torch.float32, device=dev)
    mws = torch.empty(dsa.dsa_sparse_mla_bwd_workspace_bytes(L, H, L, k), dtype=torch.uint8, device=dev)
    sc = torch.empty((L, k), dtype=torch.float32, device=dev)
    dkl = torch.full((L,), 1.0 / L, dtype=torch.float32, device=dev)
    grad = torch.empty((L, k), dtype=torch.float32, device=dev)
    dw = torch.empty((L, cfg.H_I), dtype=torch.float32, device=dev)
    dqi = torch.empty((L, cfg.H_I, cfg.D_I), dtype=torch.float32, device=dev)
    dki = torch.empty((L, cfg.D_I), dtype=torch.float32, device=dev)
    iws = torch.empty(dsa.dsa_indexer_bwd_workspace_bytes(L, L, k), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    st = StageSamples(torch, ["scores_at", "sparse_mla_bwd_kl", "indexer_bwd"])
    for i in range(steps + 1):
        evs = st.new()
        evs[0].record(stream)
        dsa.dsa_indexer_scores_at(t["q8"], t["qs"], t["k8"], t["ks"], t["w"], t["idx"], sc, stream=stream)
        evs[1].record(stream)
        dsa.dsa_sparse_mla_bwd_kl(t["q"], t["kv"], t["idx"], t["out"], t["lse"], dout, sc, dkl, cfg.sm_scale, dq, dkv,
                                  grad, mws, stream=stream)
        evs[2].record(stream)
        dsa.dsa_indexer_bwd(t["q8"], t["qs"], t["k8"], t["ks"], t["w"], t["idx"], grad, dw, dqi, dki, iws,
                            stream=stream)
        evs[3].record(stream)
        torch.cuda.synchronize()
        if i > 0:
            st.add(evs)
    ms = {n: v for n, v in st.median_ms().items() if n != "_step"}
    pairs = prefill_work(cfg)["selected_pairs"]
    # the four products of the attention backward (dP, dq, dkv's logit and value parts):
    # 2 H (512 + 576 + 576 + 512) FLOP per selected pair; the logits' recompute is not counted
    mla_flop = 2 * H * (512 + 576 + 576 + 512) * pairs
    # the indexer backward: the dot products again (FP8 MFMA), then dq and each pair's dk share (bf16 MFMA,
    # the fp32 coefficient as two bf16 terms: the hardware does twice this count for those two products)
    idx_flop = 3 * 2 * cfg.H_I * cfg.D_I * pairs
    res = {
        "workload": cfg.name, "L": L, "H": H, "k": k, "steps": steps,
        "stages_ms": {n: round(v, 3) for n, v in ms.items()},
        "tokens_per_s": round(L / (sum(ms.values()) / 1e3), 1),
        "roofline": {
            # the attention backward's stage also forms the KL score gradient (a per-token pass over [T, k])
            "sparse_mla_bwd": _rl("mfma", mla_flop / (ms["sparse_mla_bwd_kl"] / 1e3) / 1e12, PEAK_BF16_TFLOPS,
                                  "TFLOP/s"),
            "indexer_bwd": _rl("mfma", idx_flop / (ms["indexer_bwd"] / 1e3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"),
        },
        "work": {"selected_pairs": pairs, "sparse_mla_bwd_flop": mla_flop, "indexer_bwd_flop": idx_flop},
        "data": "synthetic upstream gradient dout ~ N(0, 0.01^2) bf16; dkl = 1/L (mean of the per-token loss)",
    }
    del dout, dq, dkv, mws, sc, grad, dw, dqi, dki, iws
    return res


# --------------------------------------------------------------------------- short prefill
def run_short_prefill(torch, dsa, synth, cfg, dev, steps, warmup):
    """One causal sequence of cfg.L tokens: quantise + fused indexer/top-k, then
    attention over the selection either through the masked-MHA mode (per-head
    K/V up-projected from the latent, dense causal tiles under the top-k mask)
    or through sparse MLA in MQA mode (absorbed queries over the 576-d latent)."""
    L, H = cfg.L, cfg.H
    q_i, k_i, w = synth.prefill_indexer_inputs(cfg, device=dev)
    t = {"qi": q_i.view(L, -1), "ki": k_i, "w": w}
    t["q8"] = torch.empty((L, cfg.H_I, cfg.D_I), dtype=torch.uint8, device=dev)
    t["qs"] = torch.empty(L, dtype=torch.float32, device=dev)
    t["k8"] = torch.empty((L, cfg.D_I), dtype=torch.uint8, device=dev)
    t["ks"] = torch.empty(L, dtype=torch.float32, device=dev)
    t["idx"] = torch.empty((L, cfg.k), dtype=torch.int32, device=dev)
    args = dsa.make_prefill_args(L, cfg.H_I, cfg.D_I, H, cfg.k, dsa.DSA_E4M3, t["q8"], t["qs"], t["k8"], t["ks"],
                                 t["w"], dsa.DSA_BF16, None, None, cfg.sm_scale, t["idx"], None, None)
    t["sel_ws"] = torch.empty(dsa.dsa_prefill_workspace_bytes(args), dtype=torch.uint8, device=dev)
    t["q"] = synth.mha_query(cfg, device=dev)
    t["kv"] = synth.prefill_latent(cfg, device=dev)
    t["w_uk"], t["w_uv"] = synth.mha_up_weights(cfg, device=dev)
    t["out"] = torch.empty((L, H, synth.MHA_DV), dtype=torch.bfloat16, device=dev)
    t["lse"] = torch.empty((L, H), dtype=torch.float32, device=dev)
    t["mha_ws"] = torch.empty(dsa.dsa_masked_mha_workspace_bytes(L, H), dtype=torch.uint8, device=dev)
    t["q_mqa"] = synth.prefill_attn_q(cfg, device=dev)
    t["out_mqa"] = torch.empty((L, H, 512), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(evs, mode):
        evs[0].record(stream)
        dsa.dsa_quantize_e4m3_per_token(t["qi"], t["q8"], t["qs"], rows=L, cols=cfg.H_I * cfg.D_I, stream=stream)
        dsa.dsa_quantize_e4m3_per_token(t["ki"], t["k8"], t["ks"], rows=L, cols=cfg.D_I, stream=stream)
        evs[1].record(stream)
        dsa.dsa_prefill_select(args, t["sel_ws"], stream=stream)
        evs[2].record(stream)
        if mode == "mha":
            dsa.dsa_masked_mha_prefill(t["q"], t["kv"], t["w_uk"], t["w_uv"], t["idx"], cfg.sm_scale, t["out"],
                                       t["mha_ws"], t["lse"], stream=stream)
        else:
            dsa.dsa_sparse_mla_fwd(t["q_mqa"], t["kv"], t["idx"], cfg.sm_scale, t["out_mqa"], t["lse"],
                                   stream=stream)
        evs[3].record(stream)

    res = {}
    for mode in ("mha", "mqa"):
        st = Stages(torch, ["quantize", "indexer_topk", "attention"])
        for _ in range(warmup):
            step(st.new(), mode)
        torch.cuda.synchronize()
        all_evs = [st.new() for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            step(all_evs[i], mode)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for e in all_evs:
            st.add(e)
        ms = st.avg_ms()
        res[mode] = {"tokens_per_s": round(L * steps / wall, 1), "ms_per_step": round(wall / steps * 1e3, 3),
                     "stages_ms": {k: round(v, 4) for k, v in ms.items()}}
    # algorithmic work of the masked-MHA mode: per-head K/V up-projection, then
    # dense causal attention (logits over 192 dims, values over 128) under the mask
    causal = L * (L + 1) // 2
    up_flop = 2 * L * H * (synth.MHA_DN + synth.MHA_DV) * synth.MHA_DC
    att_flop = 2 * causal * H * (synth.MHA_DN + synth.MHA_DR + synth.MHA_DV)
    mha_ms = res["mha"]["stages_ms"]["attention"]
    tf = (up_flop + att_flop) / (mha_ms / 1e3) / 1e12
    res["mha"]["roofline"] = dict(_rl("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s"),
                                  kernel="masked_mha (up-projection + mask + attention)")
    sel = sum(min(i + 1, cfg.k) for i in range(L))
    mqa_ms = res["mqa"]["stages_ms"]["attention"]
    res["mqa"]["roofline"] = dict(_rl("mfma", 2 * sel * H * (576 + 512) / (mqa_ms / 1e3) / 1e12, PEAK_BF16_TFLOPS,
                                      "TFLOP/s"), kernel="sparse_mla_bf16")
    res.update({"workload": cfg.name, "L": L, "H": H, "k": cfg.k, "steps": steps,
                "work": {"mha_upproj_flop": up_flop, "mha_attention_flop": att_flop,
                         "mqa_flop": 2 * sel * H * (576 + 512)},
                "attention_speedup_mha_vs_mqa": round(mqa_ms / mha_ms, 3)})
    del t
    torch.cuda.empty_cache()
    return res


INDEXER_TRAFFIC = os.path.join(ROOT, "profiles", "prefill_indexer_topk_L131072_traffic.json")
MLA_TRAFFIC = os.path.join(ROOT, "profiles", "sparse_mla_bf16_L131072_traffic.json")


def kernel_source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(record, L):
    """HBM bytes per launch of a kernel from its committed rocprofv3
    FETCH_SIZE/WRITE_SIZE record, if it was taken on these kernel sources at
    this L; otherwise None."""
    try:
        with open(record) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("L") != L or rec.get("source_sha256") != kernel_source_hash(rec.get("sources", [])):
        return None
    return rec.get("bytes_per_launch")


def _rl(bound, achieved, peak, unit, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


# --------------------------------------------------------------------------- measured peaks
def measure_peaks(torch, dev, reps=5):
    """The chip's rates measured by plain microbenchmarks (libdsa_peaks.so):
    dense FP8 and bf16 MFMA loops, and a streaming HBM read and write of 8 GiB.
    Best of `reps` runs each."""
    import ctypes
    from sparse_attention_gemm_amd import build
    lib = ctypes.CDLL(build.PEAKS_LIB)
    lib.dsa_peak_fp8_flop_per_wave_iter.restype = ctypes.c_int64
    lib.dsa_peak_bf16_flop_per_wave_iter.restype = ctypes.c_int64
    lib.dsa_peak_fp8_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.dsa_peak_bf16_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.dsa_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.dsa_peak_hbm_write.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = n_cu * 8
    sink = torch.zeros(blocks, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def best(launch):
        ts = []
        for _ in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            assert launch() == 0
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return min(ts[1:])

    iters = 4000
    waves = blocks * 4
    fp8_ms = best(lambda: lib.dsa_peak_fp8_mfma(blocks, iters, sink.data_ptr(), stream.cuda_stream))
    bf16_ms = best(lambda: lib.dsa_peak_bf16_mfma(blocks, iters, sink.data_ptr(), stream.cuda_stream))
    fp8 = waves * iters * lib.dsa_peak_fp8_flop_per_wave_iter() / (fp8_ms / 1e3) / 1e12
    bf16 = waves * iters * lib.dsa_peak_bf16_flop_per_wave_iter() / (bf16_ms / 1e3) / 1e12
    buf = torch.empty(8 << 30, dtype=torch.uint8, device=dev)
    hbm_ms = best(lambda: lib.dsa_peak_hbm_read(buf.data_ptr(), buf.numel(), n_cu * 16, sink.data_ptr(),
                                                 stream.cuda_stream))
    hbm = buf.numel() / (hbm_ms / 1e3) / 1e9
    wr = {}
    for nt in (0, 1):
        ms = best(lambda: lib.dsa_peak_hbm_write(buf.data_ptr(), buf.numel(), n_cu * 16, nt, stream.cuda_stream))
        wr[nt] = buf.numel() / (ms / 1e3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return {"fp8_mfma_tflops": round(fp8, 1), "bf16_mfma_tflops": round(bf16, 1), "hbm_read_gbs": round(hbm, 1),
            "hbm_write_gbs": round(max(wr.values()), 1),
            "hbm_write_gbs_by_policy": {"default": round(wr[0], 1), "streaming": round(wr[1], 1)},
            "method": f"best of {reps}: {blocks} workgroups x 4 waves x {iters} iterations of 4 independent "
                      "32x32x64 E4M3 / 32x32x16 bf16 MFMAs; an 8 GiB streaming read with 16-byte loads; the "
                      "same 8 GiB written with 16-byte stores",
            "datasheet": {"fp8_mfma_tflops": PEAK_FP8_TFLOPS, "bf16_mfma_tflops": PEAK_BF16_TFLOPS,
                          "hbm_gbs": PEAK_HBM_GBS}}


def _with_measured(rl, measured):
    """Add the fraction of the measured peak to a roofline entry."""
    if measured:
        rl = dict(rl)
        rl["measured_peak"] = measured
        rl["frac_of_measured"] = round(rl["achieved"] / measured, 4)
    return rl


# --------------------------------------------------------------------------- prefill runs
def run_prefill(torch, dsa, synth, cfg, dev, steps, warmup, log):
    """Time `steps` whole prefill steps (after `warmup`) on resident inputs.
    Returns (wall seconds, per-stage median ms, inputs)."""
    log(f"drawing prefill inputs L={cfg.L}")
    t = setup_prefill(torch, dsa, synth, cfg, dev)
    stream = torch.cuda.current_stream()
    st = StageSamples(torch, ["quantize", "indexer_topk", "sparse_mla"])
    for i in range(warmup):
        prefill_step(dsa, cfg, t, st.new(), stream)
        torch.cuda.synchronize()
        log(f"warmup step {i} done")
    all_evs = [st.new() for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        prefill_step(dsa, cfg, t, all_evs[i], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for e in all_evs:
        st.add(e)
    log(f"{steps} prefill steps at L={cfg.L} in {wall:.3f} s")
    return wall, st.median_ms(), t


def prefill_rooflines(cfg, ms, peaks, traffic=True):
    work = prefill_work(cfg)
    idx_tflops = work["indexer_flop"] / (ms["indexer_topk"] / 1e3) / 1e12
    mla_tflops = work["mla_flop"] / (ms["sparse_mla"] / 1e3) / 1e12
    q_gbs = work["quantize_bytes"] / (ms["quantize"] / 1e3) / 1e9
    mp = peaks or {}
    kernels = {
        "prefill_indexer_topk": _with_measured(
            dict(_rl("mfma", idx_tflops, PEAK_FP8_TFLOPS, "TFLOP/s",
                     recorded_traffic(INDEXER_TRAFFIC, cfg.L) if traffic else None),
                 kernel="prefill_indexer_topk", ms=round(ms["indexer_topk"], 3)), mp.get("fp8_mfma_tflops")),
        "sparse_mla_bf16": _with_measured(
            dict(_rl("mfma", mla_tflops, PEAK_BF16_TFLOPS, "TFLOP/s",
                     recorded_traffic(MLA_TRAFFIC, cfg.L) if traffic else None),
                 kernel="sparse_mla_bf16", ms=round(ms["sparse_mla"], 3)), mp.get("bf16_mfma_tflops")),
    }
    stages = {
        "quantize": _with_measured(dict(ms=round(ms["quantize"], 3), **_rl("hbm", q_gbs, PEAK_HBM_GBS, "GB/s")),
                                   mp.get("hbm_read_gbs")),
        "indexer_topk": kernels["prefill_indexer_topk"],
        "sparse_mla": kernels["sparse_mla_bf16"],
    }
    # the headline roofline is the kernel that takes longest in the step
    dominant = max(kernels.values(), key=lambda r: r["ms"])
    return dominant, kernels, stages, work


# --------------------------------------------------------------------------- CPU baseline
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _omp():
    """The OpenMP runtime the oracle runs on (libgomp, loaded with it)."""
    import ctypes
    try:
        g = ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None
    g.omp_get_max_threads.restype = ctypes.c_int
    g.omp_set_num_threads.argtypes = [ctypes.c_int]
    return g


def _oracle_sample(torch, synth, cfg, rows):
    """Inputs of the given query rows (drawn with the same generator as the GPU's)."""
    k_i = synth.prefill_indexer_keys(cfg)
    kv = synth.prefill_latent(cfg)
    q_rows, w_rows, qa_rows = [], [], []
    for r in rows:
        qi, w = synth.prefill_indexer_query(cfg, rows=(int(r), int(r) + 1))
        q_rows.append(qi)
        w_rows.append(w)
        qa_rows.append(synth.prefill_attn_q(cfg, rows=(int(r), int(r) + 1)))
    return torch.cat(q_rows), k_i, torch.cat(w_rows), torch.cat(qa_rows), kv


def _oracle_path(oracle, cfg, rows, qi, k_i, w, qa, kv):
    """The whole path for the sampled rows: quantise, indexer over s <= t,
    top-k, sparse MLA.  Returns seconds."""
    import numpy as np
    n = len(rows)
    t0 = time.perf_counter()
    q8, qsc = oracle.quantize_rows(qi.view(n, -1).numpy())
    k8, ksc = oracle.quantize_rows(k_i.numpy())
    pos = rows.astype(np.int32)
    sc = oracle.indexer_rows(q8.reshape(n, cfg.H_I, cfg.D_I), k8, w.numpy(), pos, q_scale=qsc, k_scale=ksc)
    idx, _ = oracle.topk_rows(sc, pos.astype(np.int64) + 1, cfg.k)
    oracle.sparse_mla_rows(qa, kv, idx, cfg.sm_scale)
    return time.perf_counter() - t0


def cpu_baseline(torch, synth, cfg, nrows, nrows_1t):
    """The fp64 oracle on `nrows` query rows evenly spaced over the sequence
    (an unbiased sample of the per-row cost, since the rows cover every
    context length in proportion), on every host thread; then on `nrows_1t`
    rows on one thread.  Rates are tokens/s of the whole path; the full-length
    run time is extrapolated from them (the whole oracle run is not made)."""
    import numpy as np
    import oracle
    oracle.build()
    L = cfg.L
    rows = np.unique(((np.arange(nrows) + 0.5) * L / nrows).astype(np.int64))
    ins = _oracle_sample(torch, synth, cfg, rows)
    omp = _omp()
    threads = omp.omp_get_max_threads() if omp else int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    dt = _oracle_path(oracle, cfg, rows, *ins)
    value = len(rows) / dt
    res = {"value": round(value, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "cpu_model": _cpu_model(), "host_threads": os.cpu_count(),
           "sample": f"{len(rows)} query rows evenly spaced over L={L} (quantise, fp64 indexer over all s<=t, "
                     f"top-{cfg.k}, fp64 sparse MLA over {cfg.H} heads); {dt:.1f} s wall on {threads} threads",
           "extrapolated_full_run_hours": round(L / value / 3600, 2),
           "extrapolation": f"the full L={L} oracle run is not made; its time is L / value, from the sampled "
                            "rows' rate (evenly spaced rows cover every context length in proportion)"}
    if omp and nrows_1t > 0:
        rows1 = np.unique(((np.arange(nrows_1t) + 0.5) * L / nrows_1t).astype(np.int64))
        ins1 = _oracle_sample(torch, synth, cfg, rows1)
        omp.omp_set_num_threads(1)
        try:
            dt1 = _oracle_path(oracle, cfg, rows1, *ins1)
        finally:
            omp.omp_set_num_threads(threads)
        res["single_thread"] = {"value": round(len(rows1) / dt1, 3), "unit": "tokens/s", "cores": 1,
                                "sample": f"{len(rows1)} evenly spaced rows, {dt1:.1f} s wall"}
    return res


# --------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported by this build "
              f"(the multi-GPU sharding of the path is described in the design notes, not built).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    from sparse_attention_gemm_amd import dsa
    dsa.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    peaks = None
    if not args.no_peaks:
        log("measured peaks (FP8 / bf16 MFMA loops, HBM read stream)")
        peaks = measure_peaks(torch, dev)
    cfg = synth.CONFIGS["prefill128k"]
    if args.L:
        cfg = synth.scaled_down(cfg, L=args.L)
    wall, ms, t = run_prefill(torch, dsa, synth, cfg, dev, args.steps, args.warmup, log)
    dominant, kernels, stages, work = prefill_rooflines(cfg, ms, peaks)
    value = cfg.L * args.steps / wall
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3+bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "L": cfg.L, "H_I": cfg.H_I, "D_I": cfg.D_I, "H": cfg.H, "k": cfg.k,
                   "seed": cfg.seed, "parallelism": "single GPU"},
        "roofline": dominant,
        "rooflines": kernels,
        "stages": stages,
        "stage_timing": f"median over the {args.steps} timed steps (HIP events on the launching stream)",
        "measured_peaks": peaks,
        "work": work,
    }
    if not args.no_kl:
        log("indexer KL loss on the headline selection")
        line["kl_loss"] = run_kl(torch, dsa, cfg, t, dev, args.kl_steps)
    if args.calibrate_copy:
        # plain copies of known size for scaling HBM counters: the runtime's
        # device copy, then an elementwise kernel (vector loads and stores)
        a = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        line["copy_calibration"] = {"bytes_read": a.numel() * 4, "bytes_written": b.numel() * 4,
                                    "launches": "3 runtime copies, then 3 elementwise copies"}
        del a, b
    del t
    torch.cuda.empty_cache()
    if not args.no_prefill16k and not args.L:
        c16 = synth.CONFIGS["prefill16k"]
        w16, ms16, t16 = run_prefill(torch, dsa, synth, c16, dev, max(args.steps, 5), 1, log)
        d16, k16, s16, work16 = prefill_rooflines(c16, ms16, peaks, traffic=False)
        line["prefill16k"] = {"workload": c16.name, "L": c16.L, "tokens_per_s": round(c16.L * max(args.steps, 5) / w16, 1),
                              "ms_per_step": round(w16 / max(args.steps, 5) * 1e3, 3), "stages": s16, "work": work16}
        if not args.no_backward:
            log("backward of the L=16384 step (sparse MLA, indexer KL)")
            line["backward"] = run_backward(torch, dsa, c16, t16, dev, args.backward_steps)
        del t16
        torch.cuda.empty_cache()
    if not args.no_decode:
        flush = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
        dcfg = synth.CONFIGS["decode"]
        log("decode B=64 ctx=32768")
        line["decode"] = run_decode(torch, dsa, synth, dcfg, dev, args.decode_steps, args.decode_warmup, flush)
        if not args.no_paged:
            log("paged decode B=128")
            line["paged_decode"] = run_decode(torch, dsa, synth, synth.CONFIGS["paged"], dev, args.decode_steps,
                                              args.decode_warmup, flush)
        for key in ("decode", "paged_decode"):
            if key in line and peaks:
                rl = line[key]["roofline"]
                for name in ("decode_indexer", "topk", "sparse_mla"):
                    rl[name] = _with_measured(rl[name], peaks["hbm_read_gbs"])
                rl["sparse_mla_mfma"] = _with_measured(rl["sparse_mla_mfma"], peaks["bf16_mfma_tflops"])
        del flush
    if not args.no_short:
        log("short prefill L=4096 (masked MHA and sparse MLA)")
        line["short_prefill"] = run_short_prefill(torch, dsa, synth, synth.CONFIGS["mha4k"], dev, args.short_steps, 3)
    if not args.no_cpu_baseline:
        log(f"oracle on {args.cpu_rows} sampled rows, then {args.cpu_rows_1t} on one thread")
        line["cpu_baseline"] = cpu_baseline(torch, synth, cfg, args.cpu_rows, args.cpu_rows_1t)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
