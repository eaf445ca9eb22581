"""dsa_decode_noalloc (workspace in the library's static device scratch)
against dsa_decode (caller workspace), through the C ABI: the same kernels,
so every output must be bit-identical.  Two calls in a row, the second with a
smaller batch, shorter contexts, fewer heads and a smaller k, so the scratch
holds the first call's contents when the second starts; then the first
request again.  (The refusal of a request larger than the static scratch is
checked on the host, in test_capi_cpu.py.)"""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_gemm_amd import dsa as d
    d.load()
    return d


def _request(dsa, cfg):
    ctx = synth.decode_ctx(cfg)
    bt, nb = synth.decode_block_table(cfg, ctx)
    pools = [p.to(DEV) for p in synth.build_decode_pools(cfg, ctx, bt, nb)]
    qside = [x.to(DEV) for x in synth.decode_queries(cfg)]
    ctxd, btd = ctx.to(torch.int32).to(DEV), bt.to(DEV)

    def outputs():
        return (torch.full((cfg.B, cfg.H, 512), 7.0, dtype=torch.bfloat16, device=DEV),
                torch.full((cfg.B, cfg.H), 7.0, dtype=torch.float32, device=DEV),
                torch.full((cfg.B, cfg.k), 7, dtype=torch.int32, device=DEV))

    def args(out, lse, idx):
        return dsa.make_decode_args(cfg.B, cfg.H_I, cfg.D_I, cfg.H, cfg.k, *qside, *pools, nb * 64, btd,
                                    bt.shape[1], ctxd, int(ctx.max()), cfg.sm_scale, out, lse, idx)
    keep = (pools, qside, ctxd, btd)
    return args, outputs, keep


def _same(a, b):
    return all(torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y) for x, y in zip(a, b))


def test_noalloc_decode_matches_decode_twice(dsa):
    big = synth.DecodeConfig("t", 6, 4096, 9000, 64, 128, 128, 2048, 31, True)
    small = synth.DecodeConfig("t", 3, 100, 3000, 64, 128, 32, 256, 32, True)
    reqs = []
    for cfg in (big, small):
        print(f"[case] noalloc decode B={cfg.B} ctx=[{cfg.ctx_lo},{cfg.ctx_hi}] H={cfg.H} k={cfg.k}", flush=True)
        args, outputs, keep = _request(dsa, cfg)
        ref = outputs()
        a = args(*ref)
        ws = torch.empty(dsa.dsa_decode_workspace_bytes(a), dtype=torch.uint8, device=DEV)
        assert ws.numel() <= dsa.dsa_decode_static_scratch_bytes()
        dsa.dsa_decode(a, ws)
        got = outputs()
        dsa.dsa_decode_noalloc(args(*got))
        torch.cuda.synchronize()
        assert _same(ref, got), f"noalloc differs from dsa_decode (B={cfg.B})"
        assert not torch.equal(got[2], torch.full_like(got[2], 7)), "nothing written"
        reqs.append((args, outputs, keep, ref))
    # the first request again, after the smaller one left its contents in the scratch
    args, outputs, keep, ref = reqs[0]
    again = outputs()
    dsa.dsa_decode_noalloc(args(*again))
    torch.cuda.synchronize()
    assert _same(ref, again)
