"""Shared helpers for the GPU tests: moving seeded cases to the device,
calling the library through its binding, and the parity bars."""
from __future__ import annotations

import numpy as np
import torch

# Parity bars.  bf16: max-abs <= 1e-2 and relative RMS <= 5e-3 over the whole
# output; fp32: max-abs <= 2e-5 and relative RMS <= 1e-5; lse: 1e-3 (bf16
# inputs) or 1e-5 (fp32) absolute.
BF16_MAX_ABS, BF16_REL_RMS, BF16_LSE = 1e-2, 5e-3, 1e-3
F32_MAX_ABS, F32_REL_RMS, F32_LSE = 2e-5, 1e-5, 1e-5


_CONFIG_CACHE = {}


def config_case(name, with_logits=False):
    """Seeded full-size workload, generated once per test session."""
    import synthetic
    key = (name, with_logits)
    if key not in _CONFIG_CACHE:
        _CONFIG_CACHE.clear() if len(_CONFIG_CACHE) > 2 else None
        _CONFIG_CACHE[key] = synthetic.make_config_case(name, with_logits=with_logits)
    return _CONFIG_CACHE[key]


def lib():
    """Import the binding (fails loudly when libtreeattn.so is missing)."""
    import tree_masked_attention_forward_amd as ta
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return ta


class DevCase:
    def __init__(self, case, device="cuda"):
        self.case = case
        d = torch.device(device)
        self.parents = torch.from_numpy(case.parents).to(d)
        self.node_offsets = torch.from_numpy(case.node_offsets).to(d)
        self.prefix_offsets = torch.from_numpy(case.prefix_offsets).to(d)
        self.q = case.q.to(d)
        self.k_tree = case.k_tree.to(d)
        self.v_tree = case.v_tree.to(d)
        self.k_prefix = case.k_prefix.to(d)
        self.v_prefix = case.v_prefix.to(d)
        self.logits = None if case.logits is None else case.logits.to(d)
        self.draft = None if case.draft is None else torch.from_numpy(case.draft).to(d)
        self.max_nodes = max(case.max_nodes, 1)
        self.max_prefix = case.max_prefix


def gpu_mask(ta, dc):
    mask, depth, status = ta.build_mask(dc.parents, dc.node_offsets, dc.max_nodes)
    return mask, depth, status


def gpu_forward(ta, dc, mask, **kw):
    c = dc.case
    return ta.forward(dc.q, dc.k_tree, dc.v_tree, dc.k_prefix, dc.v_prefix, dc.prefix_offsets,
                      dc.node_offsets, mask, dc.max_nodes, dc.max_prefix, c.scale,
                      return_lse=True, **kw)


def rel_rms(a, b):
    den = np.sqrt(np.mean(b.astype(np.float64) ** 2))
    return float(np.sqrt(np.mean((a.astype(np.float64) - b) ** 2)) / max(den, 1e-300))


def check_attention(out, lse, ref_out, ref_lse, fp32: bool, what: str = ""):
    """Element-by-element comparison against the oracle at the parity bar."""
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.float().cpu().numpy().astype(np.float64)
    assert o.shape == ref_out.shape, (o.shape, ref_out.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    max_abs = float(np.abs(o - ref_out).max()) if o.size else 0.0
    rr = rel_rms(o, ref_out) if o.size else 0.0
    lse_err = float(np.abs(l - ref_lse).max()) if l.size else 0.0
    bars = (F32_MAX_ABS, F32_REL_RMS, F32_LSE) if fp32 else (BF16_MAX_ABS, BF16_REL_RMS, BF16_LSE)
    msg = f"{what}: max_abs={max_abs:.3e} rel_rms={rr:.3e} lse_err={lse_err:.3e} bars={bars}"
    print(msg, flush=True)
    assert max_abs <= bars[0] and rr <= bars[1] and lse_err <= bars[2], msg
    return max_abs, rr, lse_err
