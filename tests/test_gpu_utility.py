"""GPU parity of the future-KV-utility diagnostic (full text App. A.7.4,
Table 12) against the float64 oracle: the utility of every key, element by
element, and the overlap between each routing criterion's selection and the
top keys by utility.  Bar: utilities within 1e-5 relative L2 and 1e-4 of
the largest value elementwise (fp32 exp and sums of at most N G terms from
the same rounded inputs); overlap counts equal, except where the keys at
the cut have utilities within 1e-5 relative of each other."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from parity import make_case, prepare, rel_l2, say, torch_dtype

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_G4_ragged": (make_case("u", 1, 520, 8, 2, 128, 64, 64, 16, outlier_frac=0.02, heavy_scale=6.0), 41),
    "f32_d64_G1_W32": (make_case("v", 2, 200, 2, 2, 64, 32, 32, 8, dtype="f32"), 42),
    "bf16_no_window": (make_case("w", 1, 150, 4, 1, 128, 0, 64, 0), 43),
}


def gpu_and_oracle(gpu_lib, cfg, seed):
    raw = workloads.make_prefill(cfg, seed)
    dev, ref = prepare(raw, torch_dtype(cfg["dtype"]))
    u = gpu_lib.future_kv_utility(dev["q"], dev["k"], window=cfg["window"], chunk=cfg["chunk"])
    torch.cuda.synchronize()
    p = O.Params(window=cfg["window"], chunk=cfg["chunk"], topk=cfg["topk"])
    return dev, ref, u.double().cpu().numpy(), O.future_kv_utility(ref["q"], ref["k"], p, cfg["n_kv_heads"])


@pytest.mark.parametrize("name", list(CASES))
def test_utility_matches_oracle(gpu_lib, name):
    cfg, seed = CASES[name]
    say(f"[util] case={name} shape={workloads.shape_of(cfg)} seed={seed}")
    _, _, u, uo = gpu_and_oracle(gpu_lib, cfg, seed)
    err, mx = rel_l2(u, uo), float(np.abs(u - uo).max() / max(np.abs(uo).max(), 1e-30))
    say(f"  rel-L2 {err:.2e}, max err / max {mx:.2e}")
    assert np.isfinite(u).all() and err <= 1e-5 and mx <= 1e-4
    W, N = cfg["window"], cfg["seqlen"]
    if W > 0:
        assert np.all(u[:, :, max(0, N - W):] == 0)


def near_tie_slack(u, sel, N, W):
    """Keys whose utility lies within 1e-5 relative of the m-th eligible
    value, per (b, g): the most an fp32-vs-fp64 reordering can move."""
    B, Hkv = u.shape[:2]
    slack = np.zeros((B, Hkv), np.int64)
    for b in range(B):
        for g in range(Hkv):
            m = int(O.kv_utility_overlap(sel[b:b + 1, g:g + 1], u[b:b + 1, g:g + 1], N, W)[0, 0, 0])
            if m == 0:
                continue
            vals = np.sort(u[b, g, : N - W])[::-1]
            cut = vals[m - 1]
            slack[b, g] = int(np.sum(np.abs(vals - cut) <= 1e-5 * max(abs(cut), 1e-30))) - 1
    return slack


@pytest.mark.parametrize("route", ["saliency", "diagonal", "keynorm", "random"])
def test_overlap_with_selection(gpu_lib, route):
    cfg, seed = CASES["bf16_G4_ragged"]
    dev, ref, u, uo = gpu_and_oracle(gpu_lib, cfg, seed)
    W, C, lam, N = cfg["window"], cfg["chunk"], cfg["topk"], cfg["seqlen"]
    sel = gpu_lib.fwd(dev["q"], dev["k"], dev["v"], dev["wphi_q"], dev["wphi_k"], window=W, chunk=C,
                      topk=lam, return_sel=True, route=route)["sel_idx"].cpu().numpy()
    a = O.kv_utility_overlap(sel, u, N, W)
    b = O.kv_utility_overlap(sel, uo, N, W)
    slack = np.maximum(near_tie_slack(u, sel, N, W), near_tie_slack(uo, sel, N, W))
    frac = a[..., 1].sum() / max(1, a[..., 0].sum())
    say(f"  [{route}] overlap {a[..., 1].ravel().tolist()} of {a[..., 0].ravel().tolist()} ({frac:.1%})")
    assert np.array_equal(a[..., 0], b[..., 0])
    assert np.all(np.abs(a[..., 1] - b[..., 1]) <= slack)
