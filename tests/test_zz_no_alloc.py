"""The no-allocation decode step (still_hybrid_attn_decode_step_noalloc)
against the plain decode step it mirrors: same inputs, same caches, two calls
in a row with the second on a smaller batch, on the bf16 d = 128 kernels and
on the general kernels.  Both use the same kernels, so outputs and caches
must agree bit for bit (stronger than the parity bar)."""
import numpy as np
import pytest
import torch

import workloads
from parity import make_case, prepare, say, torch_dtype

pytestmark = pytest.mark.gpu


def prefilled_pair(gpu_lib, cfg, seed, n0, general):
    """Two identical caches after a prefill of n0 tokens, plus the inputs."""
    raw = workloads.make_prefill(cfg, seed)
    dt = torch_dtype(cfg["dtype"])
    dev, _ = prepare(raw, dt)
    B, Hkv, d = cfg["batch"], cfg["n_kv_heads"], cfg["head_dim"]
    W, C, lam = cfg["window"], cfg["chunk"], cfg["topk"]
    cap = min(lam, C) * (-(-cfg["seqlen"] // C)) + 1
    caches = []
    for _ in range(2):
        gc = gpu_lib.DecodeCache(batch=B, n_kv_heads=Hkv, head_dim=d, window=W, chunk=C, topk=lam,
                                 sel_cap=cap, dtype=dt, pos=n0)
        gpu_lib.fwd(dev["q"][:, :n0].contiguous(), dev["k"][:, :n0].contiguous(),
                    dev["v"][:, :n0].contiguous(), dev["wphi_q"], dev["wphi_k"], window=W, chunk=C,
                    topk=lam, cache=gc, general=general)
        caches.append(gc)
    return dev, caches


def step_both(gpu_lib, dev, caches, t, general):
    q = dev["q"][:, t:t + 1].contiguous()
    k = dev["k"][:, t:t + 1].contiguous()
    v = dev["v"][:, t:t + 1].contiguous()
    a = gpu_lib.decode_step(q, k, v, dev["wphi_q"], dev["wphi_k"], caches[0], general=general)
    b = gpu_lib.decode_step_noalloc(q, k, v, dev["wphi_q"], dev["wphi_k"], caches[1], general=general)
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("general", [False, True], ids=["picked", "general"])
def test_noalloc_decode_equals_plain_decode(gpu_lib, general):
    dtype = "f32" if general else "bf16"
    d = 64 if general else 128
    # first call: 4 sequences; second call: 2 sequences (a smaller input)
    for B, seed in ((4, 71), (2, 72)):
        cfg = make_case("n", B, 130 + 70, 8, 2, d, 64, 64, 16, dtype=dtype, outlier_frac=0.02,
                        heavy_scale=6.0)
        say(f"[noalloc] general={general} shape={workloads.shape_of(cfg)} seed={seed}")
        dev, caches = prefilled_pair(gpu_lib, cfg, seed, 130, general)
        for t in (130, 131):
            a, b = step_both(gpu_lib, dev, caches, t, general)
            assert caches[0].pos == caches[1].pos == t + 1
            assert torch.isfinite(b.float()).all()
            assert torch.equal(a, b), f"B={B} t={t}: max |diff| {float((a.float() - b.float()).abs().max()):.3g}"
        for key, x in caches[0].tensors().items():
            assert torch.equal(x, getattr(caches[1], key)), key
        say(f"  B={B}: two steps equal the plain decode step bit for bit; caches equal")
