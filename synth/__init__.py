"""Seeded synthetic inputs for the DSA hot path (indexer -> top-k -> sparse MLA).

This module only *draws* inputs.  It holds none of the method's arithmetic: no
indexer score, no selection, no attention and no per-token quantisation.  It is
the one piece of code that both the GPU path (tests, bench) and the CPU oracle
side use, so that both sides see bit-identical inputs.

Generator
---------
Every element of every tensor is a pure function of ``(seed, tensor_id,
flat_index)``: a splitmix64 hash (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) of a counter.  Any slice of any
tensor can therefore be drawn on its own, on the CPU or on the GPU, and comes out
the same bits either way.  All steps are integer arithmetic plus one correctly
rounded fp32 multiply (and, for uniforms, one fp32 multiply-add done as two
correctly rounded ops), so torch on the CPU and torch on the GPU agree bit for
bit.

"Gaussian" values are the sum of eight independent 16-bit uniform integers,
centred and scaled to unit variance (Irwin-Hall with n = 8: excess kurtosis
-0.15, support +-4.9 sigma).  This is the stand-in for N(0, 1) throughout.

Workloads
---------
The configurations follow the DeepSeek-V3.2 write-ups: top-k = 2048 selected
positions per query and a 128K (131072-token) context (mizuki-eaf.pages.dev,
section "DeepSeek Sparse Attention" and the "DSA key parameters" table;
m.36881.com.cn, "Fine-grained Token Selection").  Head counts, dims,
distributions and seeds are the workload recipe the library is measured on.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

MASK64 = (1 << 64) - 1


def _s64(v: int) -> int:
    """Python int -> the int64 with the same low 64 bits."""
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


_GOLDEN = _s64(0x9E3779B97F4A7C15)
_M1 = _s64(0xBF58476D1CE4E5B9)
_M2 = _s64(0x94D049BB133111EB)
_TID = _s64(0xD1B54A32D192ED03)
_SEED = _s64(0xA0761D6478BD642F)


def _srl(x: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 tensors (torch's >> is arithmetic)."""
    return (x >> k) & ((1 << (64 - k)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _srl(z, 30)) * _M1
    z = (z ^ _srl(z, 27)) * _M2
    return z ^ _srl(z, 31)


def hash64(seed: int, tid: int, idx: torch.Tensor, lane: int = 0) -> torch.Tensor:
    """splitmix64 of the counter (seed, tid, lane, idx); int64 bits."""
    base = _s64(seed * _SEED + tid * _TID + lane * 0x632BE59BD9B4E019 + 0x1234567)
    return _mix(idx * _GOLDEN + base)


def _counter(start: int, numel: int, device) -> torch.Tensor:
    return torch.arange(start, start + numel, dtype=torch.int64, device=device)


_IH_MEAN = 8 * 32767.5
_IH_STD = math.sqrt(8 * (65536.0 ** 2 - 1) / 12.0)
_IH_SCALE = torch.tensor(1.0 / _IH_STD, dtype=torch.float32).item()


def normal(seed, tid, shape, start=0, device="cpu", std=1.0, chunk=1 << 27):
    """Gaussian stand-in (Irwin-Hall n=8), fp32, flat elements start..start+numel.

    ``std`` is applied as one correctly rounded fp32 multiply after the
    unit-variance draw (std=1 skips it).
    """
    numel = 1
    for s in shape:
        numel *= s
    out = torch.empty(numel, dtype=torch.float32, device=device)
    c_std = torch.tensor(std, dtype=torch.float32).item()
    for off in range(0, numel, chunk):
        n = min(chunk, numel - off)
        idx = _counter(start + off, n, device)
        acc = torch.zeros(n, dtype=torch.int64, device=device)
        for lane in (0, 1):
            h = hash64(seed, tid, idx, lane)
            for sh in (0, 16, 32, 48):
                acc += _srl(h, sh) & 0xFFFF
        del idx
        acc -= int(2 * _IH_MEAN) // 2  # 262140, exact
        v = acc.to(torch.float32) * _IH_SCALE
        if std != 1.0:
            v = v * c_std
        out[off:off + n] = v
    return out.view(*shape)


def uniform(seed, tid, shape, start=0, device="cpu", lo=0.0, hi=1.0):
    """U[lo, hi) in fp32: 24-bit grid, then lo + (hi-lo)*u as two rounded ops."""
    numel = 1
    for s in shape:
        numel *= s
    h = hash64(seed, tid, _counter(start, numel, device))
    u = (_srl(h, 40)).to(torch.float32) * (2.0 ** -24)
    if (lo, hi) != (0.0, 1.0):
        u = u * torch.tensor(hi - lo, dtype=torch.float32).item()
        u = u + torch.tensor(lo, dtype=torch.float32).item()
    return u.view(*shape)


def randint(seed, tid, shape, lo, hi, start=0, device="cpu"):
    """Integers in [lo, hi] (inclusive), from the top 53 bits modulo the range."""
    numel = 1
    for s in shape:
        numel *= s
    h = hash64(seed, tid, _counter(start, numel, device))
    return (_srl(h, 11) % (hi - lo + 1) + lo).view(*shape)


def permutation(seed, tid, n, device="cpu"):
    """A seeded random permutation of range(n): argsort of n hash keys."""
    keys = hash64(seed, tid, _counter(0, n, device))
    return torch.sort(keys, stable=True).indices


def to_e4m3_bits(x: torch.Tensor) -> torch.Tensor:
    """Round fp32 to OCP E4M3FN bytes with torch's own cast (RNE).

    Used only to draw FP8 *payloads* that are inputs of the decode workloads
    ("FP8 e4m3 q/k with per-token scales"), never for the per-token quantiser.
    """
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


# tensor ids (part of the counter; fixed forever so that drawn data is stable)
T_QI, T_KI, T_W, T_Q, T_KV, T_QS, T_KS, T_CTX, T_PERM = range(1, 10)
T_NEW_KV, T_NEW_K8, T_NEW_KS = 10, 11, 12
T_MHA_Q, T_WUK, T_WUV = 13, 14, 15

# Logical per-sequence row stride of decode tensors: every position of every
# sequence has a fixed counter, independent of paging.
DECODE_MAXCTX = 131072
PAGE = 64
D_QK, D_V = 576, 512
# masked-MHA mode: per-head no-rope key, rope and value dims; compressed latent dims
MHA_DN, MHA_DR, MHA_DV, MHA_DC = 128, 64, 128, 512


@dataclass
class PrefillConfig:
    """One causal sequence of L tokens (query t sits at position t)."""
    name: str
    L: int
    H_I: int
    D_I: int
    H: int
    k: int
    seed: int
    attn_dtype: str        # "f32" or "bf16"
    fp8_indexer: bool      # True: q_I/k_I go through per-token e4m3 quantisation
    w_std: float = 0.5
    q_std: float = 1.0     # attention q; 40 gives a sharp softmax
    sm_scale: float = 1.0 / math.sqrt(192.0)


@dataclass
class DecodeConfig:
    """B sequences, one query each at position ctx_b - 1, paged 64-token cache."""
    name: str
    B: int
    ctx_lo: int
    ctx_hi: int            # ctx_b ~ U{ctx_lo..ctx_hi}; equal -> fixed
    H_I: int
    D_I: int
    H: int
    k: int
    seed: int
    shuffled: bool
    w_std: float = 0.125
    sm_scale: float = 1.0 / math.sqrt(192.0)


CONFIGS = {
    # tiny fp32 prefill: parity only
    "tiny": PrefillConfig("tiny_fp32_L2048", 2048, 4, 64, 8, 256, 0, "f32", False),
    # the same with the indexer operands quantised per token to e4m3 (4 heads of 64 dims)
    "tiny_fp8": PrefillConfig("tiny_fp8_L2048", 2048, 4, 64, 8, 256, 0, "f32", True),
    "decode": DecodeConfig("decode_B64_ctx32768", 64, 32768, 32768, 64, 128, 128, 2048, 0, False),
    "prefill16k": PrefillConfig("prefill_L16384", 16384, 64, 128, 128, 2048, 1, "bf16", True),
    "prefill128k": PrefillConfig("prefill_L131072", 131072, 64, 128, 128, 2048, 1, "bf16", True),
    # short prefill through the masked-MHA mode (dense multi-head attention under the top-k mask)
    "mha4k": PrefillConfig("masked_mha_prefill_L4096", 4096, 64, 128, 128, 2048, 3, "bf16", True),
    "paged": DecodeConfig("paged_decode_B128_ctx4096-131072", 128, 4096, 131072, 64, 128, 128, 2048, 2,
                          True),
}


def scaled_down(cfg, **kw):
    """Same recipe, other sizes (for parity at sizes the oracle finishes)."""
    d = dict(cfg.__dict__)
    d.update(kw)
    return type(cfg)(**d)


# ----------------------------------------------------------------- prefill draws
def prefill_indexer_query(cfg: PrefillConfig, rows=None, device="cpu"):
    """q_I [T, H_I, D_I] fp32 and w [T, H_I] fp32 for rows [r0, r1) (default all)."""
    r0, r1 = (0, cfg.L) if rows is None else rows
    n = r1 - r0
    hd = cfg.H_I * cfg.D_I
    q = normal(cfg.seed, T_QI, (n, cfg.H_I, cfg.D_I), start=r0 * hd, device=device)
    w = normal(cfg.seed, T_W, (n, cfg.H_I), start=r0 * cfg.H_I, device=device, std=cfg.w_std)
    return q, w


def prefill_indexer_keys(cfg: PrefillConfig, device="cpu"):
    """k_I [L, D_I] fp32."""
    return normal(cfg.seed, T_KI, (cfg.L, cfg.D_I), device=device)


def prefill_indexer_inputs(cfg: PrefillConfig, rows=None, device="cpu"):
    """q_I [T, H_I, D_I] fp32 for the given rows (default all), k_I [L, D_I] fp32,
    w [T, H_I] fp32."""
    q, w = prefill_indexer_query(cfg, rows, device)
    return q, prefill_indexer_keys(cfg, device), w


def prefill_attn_q(cfg: PrefillConfig, rows=None, device="cpu"):
    """Attention q [T, H, 576] in the attention dtype (bf16 via RNE cast)."""
    r0, r1 = (0, cfg.L) if rows is None else rows
    per = cfg.H * D_QK
    q = normal(cfg.seed, T_Q, (r1 - r0, cfg.H, D_QK), start=r0 * per, device=device, std=cfg.q_std)
    return q if cfg.attn_dtype == "f32" else q.to(torch.bfloat16)


def prefill_latent(cfg: PrefillConfig, device="cpu"):
    """Latent cache [L, 576] ~ N(0,1)/24 in the attention dtype."""
    kv = normal(cfg.seed, T_KV, (cfg.L, D_QK), device=device, std=1.0 / 24.0)
    return kv if cfg.attn_dtype == "f32" else kv.to(torch.bfloat16)


def mha_query(cfg: PrefillConfig, rows=None, device="cpu"):
    """Masked-MHA query [T, H, 192] bf16 (128 no-rope dims, then 64 rope dims),
    N(0, q_std^2) before the RNE cast."""
    r0, r1 = (0, cfg.L) if rows is None else rows
    per = cfg.H * (MHA_DN + MHA_DR)
    q = normal(cfg.seed, T_MHA_Q, (r1 - r0, cfg.H, MHA_DN + MHA_DR), start=r0 * per, device=device,
               std=cfg.q_std)
    return q.to(torch.bfloat16)


def mha_up_weights(cfg: PrefillConfig, device="cpu"):
    """Up-projections w_uk [H, 128, 512] and w_uv [H, 128, 512] bf16 with std
    24/sqrt(512): applied to the latent (std 1/24) they give per-head keys and
    values of about unit scale."""
    std = 24.0 / math.sqrt(MHA_DC)
    w_uk = normal(cfg.seed, T_WUK, (cfg.H, MHA_DN, MHA_DC), device=device, std=std)
    w_uv = normal(cfg.seed, T_WUV, (cfg.H, MHA_DV, MHA_DC), device=device, std=std)
    return w_uk.to(torch.bfloat16), w_uv.to(torch.bfloat16)


# ------------------------------------------------------------------ decode draws
def decode_ctx(cfg: DecodeConfig):
    """Context lengths [B] int64 (CPU)."""
    if cfg.ctx_lo == cfg.ctx_hi:
        return torch.full((cfg.B,), cfg.ctx_lo, dtype=torch.int64)
    return randint(cfg.seed, T_CTX, (cfg.B,), cfg.ctx_lo, cfg.ctx_hi)


def decode_seq_keys(cfg: DecodeConfig, b: int, ctx: int, device="cpu"):
    """Logical FP8 index keys of sequence b: payload [ctx, D_I] u8, scale [ctx] f32."""
    base = b * DECODE_MAXCTX
    x = normal(cfg.seed, T_KI, (ctx, cfg.D_I), start=base * cfg.D_I, device=device)
    ks = uniform(cfg.seed, T_KS, (ctx,), start=base, device=device, lo=0.5, hi=2.0)
    return to_e4m3_bits(x), ks


def decode_seq_latent(cfg: DecodeConfig, b: int, ctx: int, device="cpu"):
    """Logical bf16 latent rows of sequence b: [ctx, 576]."""
    base = b * DECODE_MAXCTX * D_QK
    return normal(cfg.seed, T_KV, (ctx, D_QK), start=base, device=device, std=1.0 / 24.0).to(torch.bfloat16)


def decode_queries(cfg: DecodeConfig, bs=None, device="cpu"):
    """Per-sequence query side for sequences bs (default all):
    q8 [n, H_I, D_I] u8, qs [n] f32, w [n, H_I] f32, q [n, H, 576] bf16."""
    bs = list(range(cfg.B)) if bs is None else list(bs)
    q8, qs, w, q = [], [], [], []
    for b in bs:
        q8.append(to_e4m3_bits(normal(cfg.seed, T_QI, (cfg.H_I, cfg.D_I), start=b * cfg.H_I * cfg.D_I,
                                      device=device)))
        qs.append(uniform(cfg.seed, T_QS, (1,), start=b, device=device, lo=0.5, hi=2.0))
        w.append(normal(cfg.seed, T_W, (cfg.H_I,), start=b * cfg.H_I, device=device, std=cfg.w_std))
        q.append(normal(cfg.seed, T_Q, (cfg.H, D_QK), start=b * cfg.H * D_QK, device=device).to(torch.bfloat16))
    return torch.stack(q8), torch.cat(qs), torch.stack(w), torch.stack(q)


def decode_block_table(cfg: DecodeConfig, ctx: torch.Tensor):
    """Block table [B, max_blocks] int32 (-1 past the end) and the block count.

    Sequence b owns ceil(ctx_b / 64) logical pages.  Without shuffling, the
    physical pages are laid out sequence after sequence (an identity table);
    with shuffling they are a seeded permutation of all pages.
    """
    nb = [(int(c) + PAGE - 1) // PAGE for c in ctx]
    total = sum(nb)
    maxb = max(nb)
    phys = torch.arange(total, dtype=torch.int64)
    if cfg.shuffled:
        phys = permutation(cfg.seed, T_PERM, total)
    bt = torch.full((cfg.B, maxb), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(nb):
        bt[b, :n] = phys[off:off + n].to(torch.int32)
        off += n
    return bt, total


POISON_LATENT = 1.0e4   # latent value in page-tail slots (positions >= ctx)
POISON_KEY = 0x7E       # e4m3 +448 in page-tail key slots
POISON_SCALE = 2.0


def build_decode_pools(cfg: DecodeConfig, ctx, bt, nblocks, seqs=None, device="cpu"):
    """Scatter the logical per-sequence data into physical page pools.

    Returns k8 [nblocks, 64, D_I] u8, ks [nblocks, 64] f32, kv [nblocks, 64, 576]
    bf16.  Slots past each sequence's end are filled with poison.  ``seqs``
    restricts which sequences are materialised (other pages stay poison).
    """
    k8 = torch.full((nblocks, PAGE, cfg.D_I), POISON_KEY, dtype=torch.uint8, device=device)
    ks = torch.full((nblocks, PAGE), POISON_SCALE, dtype=torch.float32, device=device)
    kv = torch.full((nblocks, PAGE, D_QK), POISON_LATENT, dtype=torch.bfloat16, device=device)
    seqs = range(cfg.B) if seqs is None else seqs
    for b in seqs:
        c = int(ctx[b])
        n = (c + PAGE - 1) // PAGE
        pages = bt[b, :n].to(torch.int64).to(device)
        kb, sb = decode_seq_keys(cfg, b, c, device=device)
        lat = decode_seq_latent(cfg, b, c, device=device)
        pad = n * PAGE - c
        if pad:
            kb = torch.cat([kb, torch.full((pad, cfg.D_I), POISON_KEY, dtype=torch.uint8, device=device)])
            sb = torch.cat([sb, torch.full((pad,), POISON_SCALE, dtype=torch.float32, device=device)])
            lat = torch.cat([lat, torch.full((pad, D_QK), POISON_LATENT, dtype=torch.bfloat16, device=device)])
        k8[pages] = kb.view(n, PAGE, cfg.D_I)
        ks[pages] = sb.view(n, PAGE)
        kv[pages] = lat.view(n, PAGE, D_QK)
    return k8, ks, kv


def new_token_rows(cfg: DecodeConfig, step: int, device="cpu"):
    """One new token per sequence for a cache append: latent [B,576] bf16,
    key payload [B, D_I] u8, key scale [B] f32."""
    lat = normal(cfg.seed + 1000 * (step + 1), T_NEW_KV, (cfg.B, D_QK), device=device,
                 std=1.0 / 24.0).to(torch.bfloat16)
    k8 = to_e4m3_bits(normal(cfg.seed + 1000 * (step + 1), T_NEW_K8, (cfg.B, cfg.D_I), device=device))
    ks = uniform(cfg.seed + 1000 * (step + 1), T_NEW_KS, (cfg.B,), device=device, lo=0.5, hi=2.0)
    return lat, k8, ks
