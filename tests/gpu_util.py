"""Helpers for the GPU parity tests: error metrics against the fp64 oracle
and row sampling for shapes too large to evaluate in full."""
import numpy as np
import torch

BF16_MAX_ABS = 2e-2      # max |O_gpu - O_ref| over all elements, bf16 inputs
BF16_MEAN_ABS = 2e-3     # mean |O_gpu - O_ref|, bf16 inputs
F32_REL = 1e-5           # max |O_gpu - O_ref| / max |O_ref|, fp32 inputs


def to64(t):
    return t.detach().float().cpu().double().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)


def errors(gpu, ref):
    d = np.abs(to64(gpu) - np.asarray(ref, np.float64))
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def assert_close(gpu, ref, dtype, what):
    """The stated parity bar for the dtype the path computes in."""
    g = to64(gpu)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    mx, mean = errors(g, ref)
    if dtype == torch.float32:
        scale = max(float(np.abs(ref).max()), 1e-30) if ref.size else 1.0
        rel = mx / scale
        # diagnostic only (an elementwise relative bound is unbounded near 0):
        # the share of elements outside allclose(rtol=1e-5, atol=1e-6)
        off = float(np.mean(~np.isclose(g, ref, rtol=1e-5, atol=1e-6))) if ref.size else 0.0
        print(f"{what}: fp32 norm-wise rel err {rel:.2e}; elementwise allclose(1e-5, 1e-6) "
              f"misses {off:.2%} of elements", flush=True)
        assert rel <= F32_REL, f"{what}: fp32 norm-wise rel err {rel:.2e} > {F32_REL:.0e}"
        return rel
    assert mx <= BF16_MAX_ABS, f"{what}: max abs err {mx:.3e} > {BF16_MAX_ABS:.0e}"
    assert mean <= BF16_MEAN_ABS, f"{what}: mean abs err {mean:.3e} > {BF16_MEAN_ABS:.0e}"
    return mx, mean


def sample_rows(B, H, S, n, seed=0, extra=()):
    """n random (b, h, i) rows plus the given extra rows (deduplicated)."""
    g = np.random.default_rng(seed)
    rows = {(int(g.integers(B)), int(g.integers(H)), int(g.integers(S))) for _ in range(n)}
    rows.update((int(b), int(h), int(i)) for b, h, i in extra)
    return sorted(rows)


def convex_bound_ok(o, v, Hq):
    """Every output is a convex combination of value rows, so each feature of
    O lies within [min_j v_jc, max_j v_jc] of its KV head (over the whole
    sequence, a superset of the visible keys).  Checked on the device."""
    G = Hq // v.shape[1]
    vmax = v.float().amax(dim=2).repeat_interleave(G, dim=1)[:, :, None, :]
    vmin = v.float().amin(dim=2).repeat_interleave(G, dim=1)[:, :, None, :]
    of = o.float()
    slack = 1e-2 * (vmax - vmin).abs() + 1e-6
    ok = (of <= vmax + slack) & (of >= vmin - slack)
    return bool(ok.all().item()), bool(torch.isfinite(of).all().item())
